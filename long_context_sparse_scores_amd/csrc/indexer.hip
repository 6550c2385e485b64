// Indexer scoring on gfx950.
//
// [TEARDOWN, 刀一 DSA] (clawlihai.cn GLM-5.2 1M architecture teardown): an
// indexer with index_n_heads 32 and index_head_dim 128 scores every cached
// token before attention; [CTXFR, "Attention sparse IndexShare"]
// (glmmodel.cn/fr context-window page): the scoring is made of dot products.
//   score[b,t,s] = sum_h w[b,t,h] * max(0, q[b,t,h,:] . k[b,s,:])   (s <= p; -inf beyond)
//
// The work is an HBM stream of the index-key cache (256 bytes per key) with
// 8192 flops per key.  That is 32 flop/byte, more than the vector ALUs can
// sustain at full HBM bandwidth, so the 32 heads of a query form the M side
// of a dense 32x128 by 128xN contraction on the matrix cores:
// v_mfma_f32_16x16x32_bf16, two 16-head blocks sharing each 16-key B operand.
//
// Keys reach the matrix cores through LDS: each wave streams its keys with
// direct-to-LDS loads, every instruction reading four whole keys (1 KiB
// contiguous), into a private four-stage ring; the 16-byte chunks of key k are
// stored XOR-swizzled by k so the MFMA operand reads (16 keys, one chunk
// each) hit distinct banks.  A wave only reads what it loaded itself, so it
// waits on its own load counter and never on a workgroup barrier.  Scores
// are kept in registers and stored after the loads have drained.
#include "common.h"

namespace dsa {
namespace {

constexpr int kH = 32;
constexpr int kD = 128;
constexpr int kWaves = 8;                     // two waves per SIMD
constexpr int kTile = 16;                     // keys per MFMA tile = keys per stage
constexpr int kStages = 4;
constexpr int kTilesPerWave = 16;             // per block
constexpr int kKeysPerBlock = kWaves * kTile * kTilesPerWave;  // 2048
constexpr int kTileBytes = kTile * kD * 2;    // 4 KiB
constexpr int kLoadsPerTile = kTileBytes / (kWave * 16);       // 4 direct-to-LDS loads

__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds_byte_addr) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds_byte_addr) : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmem() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Load tile `key0 .. key0+15` of this wave into its LDS stage at byte address `dst`.
// Slot (key k, chunk s) receives logical chunk s ^ k of key k.
__device__ __forceinline__ void load_tile(const uint16_t* __restrict__ kb, int64_t key0, int L, uint32_t dst, int lane) {
#pragma unroll
    for (int i = 0; i < kLoadsPerTile; ++i) {
        const int slot = 64 * i + lane;
        const int k = slot >> 4;
        const int chunk = (slot & 15) ^ k;
        int64_t key = key0 + k;
        key = key < L ? key : (int64_t)L - 1;  // ragged tail: a valid row, never stored
        lds_dma16(kb + key * kD + 8 * chunk, dst + 1024u * i);
    }
}

__global__ __launch_bounds__(kWaves * kWave) void indexer_decode_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w, const uint16_t* __restrict__ k_idx,
    int64_t k_bstride, const int32_t* __restrict__ q_pos, int T, int L, int nblk, float* __restrict__ scores) {
    __shared__ __attribute__((aligned(16))) uint16_t ring[kWaves * kStages * kTileBytes / 2];
    const int row = blockIdx.x / nblk;  // b*T + t
    const int blk = blockIdx.x % nblk;
    const int b = row / T;
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const int c = lane & 15;  // key within tile (B/C column)
    const int g = lane >> 4;  // lane group: 8-dim slice of each 32-dim step; head row block in C
    const int64_t p = q_pos[row];

    // A operands: q rows (heads) 16*ht + c, dims 32*kk + 8*g .. +7.
    bf16x8_t qa[2][4];
    const uint16_t* qrow = q_idx + (int64_t)row * kH * kD;
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            qa[ht][kk] = *reinterpret_cast<const bf16x8_t*>(qrow + (16 * ht + c) * kD + 32 * kk + 8 * g);
    // Head weights for the C rows this lane holds: heads 16*ht + 4*g + r.
    float wv[2][4];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
#pragma unroll
        for (int r = 0; r < 4; ++r) wv[ht][r] = w[(int64_t)row * kH + 16 * ht + 4 * g + r];
    // The compiler's waits for these loads must not land inside the stream loop.
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) asm volatile("" ::"v"(qa[ht][kk]));
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
#pragma unroll
        for (int r = 0; r < 4; ++r) asm volatile("" ::"v"(wv[ht][r]));

    const uint16_t* kb = k_idx + (int64_t)b * k_bstride;
    const int64_t block_start = (int64_t)blk * kKeysPerBlock;
    // Tile j of this wave covers keys block_start + (kWaves*j + wave)*16 .. +15: at any step the
    // block's waves read 128 consecutive keys.
    auto tile_key0 = [&](int j) { return block_start + (int64_t)(kWaves * j + wave) * kTile; };
    int ntiles = 0;
    while (ntiles < kTilesPerWave && tile_key0(ntiles) < L) ++ntiles;
    const uint32_t my_ring = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint16_t*)ring) + wave * kStages * kTileBytes);
    const uint16_t* my_ring_ptr = ring + wave * kStages * kTileBytes / 2;

    for (int j = 0; j < kStages - 1 && j < ntiles; ++j) load_tile(kb, tile_key0(j), L, my_ring + j * kTileBytes, lane);

    float sc[kTilesPerWave];
#pragma unroll
    for (int j = 0; j < kTilesPerWave; ++j) {
        if (j >= ntiles) break;
        if (j + kStages - 1 < ntiles) {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the stage being refilled has been read
            load_tile(kb, tile_key0(j + kStages - 1), L, my_ring + ((j + kStages - 1) % kStages) * kTileBytes, lane);
        }
        const int later = ntiles - 1 - j;  // tiles issued after tile j, at most kStages - 1
        if (later >= 3) wait_vmem<3 * kLoadsPerTile>();
        else if (later == 2) wait_vmem<2 * kLoadsPerTile>();
        else if (later == 1) wait_vmem<kLoadsPerTile>();
        else wait_vmem<0>();
        const uint16_t* st = my_ring_ptr + (j % kStages) * kTileBytes / 2;
        f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const bf16x8_t kv = *reinterpret_cast<const bf16x8_t*>(st + 8 * (16 * c + ((4 * kk + g) ^ c)));
            a0 = mfma16x16x32(qa[0][kk], kv, a0);
            a1 = mfma16x16x32(qa[1][kk], kv, a1);
        }
        float part = 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            part = fmaf(wv[0][r], a0[r] > 0.0f ? a0[r] : 0.0f, part);
            part = fmaf(wv[1][r], a1[r] > 0.0f ? a1[r] : 0.0f, part);
        }
        part += __shfl_xor(part, 16, kWave);
        part += __shfl_xor(part, 32, kWave);
        sc[j] = part;
    }
    float* out = scores + (int64_t)row * L;
    if (g == 0) {
#pragma unroll
        for (int j = 0; j < kTilesPerWave; ++j) {
            if (j >= ntiles) break;
            const int64_t key = tile_key0(j) + c;
            if (key < L) out[key] = key <= p ? sc[j] : -INFINITY;
        }
    }
}

}  // namespace

hipError_t launch_indexer(const uint16_t* q_idx, const float* w, const uint16_t* k_idx, int64_t k_bstride,
                          const int32_t* q_pos, int B, int T, int L, float* scores, hipStream_t stream) {
    const int nblk = (L + kKeysPerBlock - 1) / kKeysPerBlock;
    dim3 grid((unsigned)((int64_t)nblk * B * T));
    hipLaunchKernelGGL(indexer_decode_kernel, grid, dim3(kWaves * kWave), 0, stream, q_idx, w, k_idx, k_bstride,
                       q_pos, T, L, nblk, scores);
    return hipGetLastError();
}

}  // namespace dsa
