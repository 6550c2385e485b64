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
// Lane l streams 16 bytes per instruction from key (l%16), dims 32*kk+8*(l/16),
// so each instruction reads 16 keys x 64 contiguous bytes.
#include "common.h"

namespace dsa {
namespace {

constexpr int kH = 32;
constexpr int kD = 128;
constexpr int kWaves = 4;
constexpr int kTile = 16;                                  // keys per MFMA tile
constexpr int kTilesPerStep = 4;                           // tiles per wave per pipeline step
constexpr int kKeysPerStep = kWaves * kTile * kTilesPerStep;  // 256 keys per block step
constexpr int kStepsPerBlock = 8;                          // 2048 keys per block

struct KeyRegs {
    bf16x8_t v[kTilesPerStep][4];
};

__device__ __forceinline__ void load_keys(KeyRegs& r, const uint16_t* __restrict__ kb, int64_t base, int L,
                                          int c, int g) {
#pragma unroll
    for (int t = 0; t < kTilesPerStep; ++t) {
        int64_t key = base + t * kTile + c;
        key = key < L ? key : (int64_t)L - 1;  // ragged tail: read a valid row, never store it
        const bf16x8_t* p = reinterpret_cast<const bf16x8_t*>(kb + key * kD + 8 * g);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) r.v[t][kk] = __builtin_nontemporal_load(p + 4 * kk);
    }
}

__global__ __launch_bounds__(kWaves * kWave) void indexer_decode_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w, const uint16_t* __restrict__ k_idx,
    int64_t k_bstride, const int32_t* __restrict__ q_pos, int T, int L, int nblk, float* __restrict__ scores) {
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

    const uint16_t* kb = k_idx + (int64_t)b * k_bstride;
    float* out = scores + (int64_t)row * L;
    const int64_t block_start = (int64_t)blk * kKeysPerStep * kStepsPerBlock;
    const int64_t wave_off = (int64_t)wave * kTile * kTilesPerStep;

    KeyRegs cur, nxt;
    int64_t base = block_start + wave_off;
    if (base >= L) return;
    load_keys(cur, kb, base, L, c, g);
    for (int step = 0; step < kStepsPerBlock; ++step) {
        const int64_t nbase = base + kKeysPerStep;
        const bool more = (step + 1 < kStepsPerBlock) && (nbase < L);
        if (more) load_keys(nxt, kb, nbase, L, c, g);
#pragma unroll
        for (int t = 0; t < kTilesPerStep; ++t) {
            f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                a0 = mfma16x16x32(qa[0][kk], cur.v[t][kk], a0);
                a1 = mfma16x16x32(qa[1][kk], cur.v[t][kk], a1);
            }
            float part = 0.0f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                part = fmaf(wv[0][r], a0[r] > 0.0f ? a0[r] : 0.0f, part);
                part = fmaf(wv[1][r], a1[r] > 0.0f ? a1[r] : 0.0f, part);
            }
            part += __shfl_xor(part, 16, kWave);
            part += __shfl_xor(part, 32, kWave);
            const int64_t key = base + t * kTile + c;
            if (g == 0 && key < L) out[key] = key <= p ? part : -INFINITY;
        }
        if (!more) break;
        cur = nxt;
        base = nbase;
    }
}

}  // namespace

hipError_t launch_indexer(const uint16_t* q_idx, const float* w, const uint16_t* k_idx, int64_t k_bstride,
                          const int32_t* q_pos, int B, int T, int L, float* scores, hipStream_t stream) {
    const int64_t keys_per_block = (int64_t)kKeysPerStep * kStepsPerBlock;
    const int nblk = (int)((L + keys_per_block - 1) / keys_per_block);
    dim3 grid((unsigned)((int64_t)nblk * B * T));
    hipLaunchKernelGGL(indexer_decode_kernel, grid, dim3(kWaves * kWave), 0, stream, q_idx, w, k_idx, k_bstride,
                       q_pos, T, L, nblk, scores);
    return hipGetLastError();
}

}  // namespace dsa
