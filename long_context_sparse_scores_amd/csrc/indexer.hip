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
// Keys are read with plain 16-byte loads in which every instruction covers
// four whole keys (1 KiB contiguous); a rolling window of five 16-key tiles
// is in flight per wave.  Each tile is then turned into the MFMA operand
// layout through a small wave-private LDS slot: lane l writes chunk l%16 of
// key 4i + l/16, and reads back chunk 4kk + l/16 of key l%16.  Chunk s of key k
// is stored at position 16k + (s ^ k), which makes both the writes and the
// reads bank-conflict free.  Scores are kept in registers and stored after the
// stream, so the loop contains only loads.
#include "common.h"

namespace dsa {
namespace {

constexpr int kH = 32;
constexpr int kD = 128;
constexpr int kTile = 16;                      // keys per MFMA tile
constexpr int kTileBytes = kTile * kD * 2;     // 4 KiB
constexpr int kLoads = kTileBytes / (kWave * 16);  // 4 loads of 1 KiB per tile
#ifndef INDEXER_AHEAD
#define INDEXER_AHEAD 4
#endif
constexpr int kAhead = INDEXER_AHEAD;          // tiles loaded ahead of the one computed

// Measured best on MI355X for 128K and 1M rows: 4 waves x 16 tiles, 4 tiles ahead.
#ifndef INDEXER_WAVES
#define INDEXER_WAVES 4
#define INDEXER_TILES 16
#endif

template <int kWaves, int kTilesPerWave>
__global__ __launch_bounds__(kWaves * kWave) void indexer_decode_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w, const uint16_t* __restrict__ k_idx,
    int64_t k_bstride, const int32_t* __restrict__ q_pos, int T, int L, int nblk, float* __restrict__ scores,
    ZeroRange zero) {
    constexpr int kKeysPerBlock = kWaves * kTile * kTilesPerWave;
    __shared__ __attribute__((aligned(16))) uint16_t stage[kWaves * 2 * kTileBytes / 2];
    const int row = blockIdx.x / nblk;  // b*T + t
    const int blk = blockIdx.x % nblk;
    const int b = row / T;
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const int c = lane & 15;  // key within tile (B/C column)
    const int g = lane >> 4;  // lane group: 8-dim slice of each 32-dim step; head row block in C
    const int64_t p = q_pos[row];
    if (zero.base && blk == 0)
        for (int i = threadIdx.x; i < zero.count; i += kWaves * kWave) zero.base[row * zero.stride + i] = 0u;

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

    const uint16_t* kb = k_idx + (int64_t)b * k_bstride;
    // Tile j of this wave covers keys tile_key0(j) .. +15; at each step the block's
    // waves read kWaves*16 consecutive keys.
    const int64_t block_start = (int64_t)blk * kKeysPerBlock;
    auto tile_key0 = [&](int j) { return block_start + (int64_t)(kWaves * j + wave) * kTile; };
    uint16_t* my_stage = stage + wave * kTileBytes;  // two 4 KiB slots per wave

    u32x4_t buf[kAhead + 1][kLoads];
    auto load_tile = [&](int j, u32x4_t (&dst)[kLoads]) {
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            int64_t key = tile_key0(j) + 4 * i + (lane >> 4);
            key = key < L ? key : (int64_t)L - 1;  // ragged tail: a valid row, never stored
            dst[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kb + key * kD + 8 * (lane & 15)));
        }
    };
#pragma unroll
    for (int j = 0; j < kAhead; ++j) load_tile(j, buf[j]);

    float sc[kTilesPerWave];
#pragma unroll
    for (int j = 0; j < kTilesPerWave; ++j) {
        if (j + kAhead < kTilesPerWave) load_tile(j + kAhead, buf[(j + kAhead) % (kAhead + 1)]);
        // registers -> LDS (swizzled) -> MFMA operand layout
        uint16_t* slot = my_stage + (j & 1) * (kTileBytes / 2);
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            const int k = 4 * i + (lane >> 4);
            *reinterpret_cast<u32x4_t*>(slot + 8 * (16 * k + ((lane & 15) ^ k))) = buf[j % (kAhead + 1)][i];
        }
        f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const bf16x8_t kv = *reinterpret_cast<const bf16x8_t*>(slot + 8 * (16 * c + ((4 * kk + g) ^ c)));
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
            const int64_t key = tile_key0(j) + c;
            if (key < L) out[key] = key <= p ? sc[j] : -INFINITY;
        }
    }
}

}  // namespace

template <int W, int N>
hipError_t launch_indexer_cfg(const uint16_t* q_idx, const float* w, const uint16_t* k_idx, int64_t k_bstride,
                              const int32_t* q_pos, int B, int T, int L, float* scores, hipStream_t stream,
                              ZeroRange zero) {
    constexpr int keys_per_block = W * kTile * N;
    const int nblk = (L + keys_per_block - 1) / keys_per_block;
    dim3 grid((unsigned)((int64_t)nblk * B * T));
    hipLaunchKernelGGL((indexer_decode_kernel<W, N>), grid, dim3(W * kWave), 0, stream, q_idx, w, k_idx, k_bstride,
                       q_pos, T, L, nblk, scores, zero);
    return hipGetLastError();
}

hipError_t launch_indexer(const uint16_t* q_idx, const float* w, const uint16_t* k_idx, int64_t k_bstride,
                          const int32_t* q_pos, int B, int T, int L, float* scores, hipStream_t stream,
                          ZeroRange zero) {
    return launch_indexer_cfg<INDEXER_WAVES, INDEXER_TILES>(q_idx, w, k_idx, k_bstride, q_pos, B, T, L, scores,
                                                            stream, zero);
}

}  // namespace dsa
