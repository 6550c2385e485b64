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
// Measured best on MI355X for 128K and 1M rows: 4 waves x 16 tiles, 4 tiles ahead.
constexpr int kAhead = 4;                      // tiles loaded ahead of the one computed
constexpr int kDecodeWaves = 4;
constexpr int kDecodeTiles = 16;               // tiles per wave

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

// ------------------------------------------------------------------ FP8 (E4M3) index keys
// The same scan over an index-key cache stored as OCP E4M3 codes ([CTXFR,
// "Entraînement par renforcement de l'agent intelligent"] names an FP8 KV
// cache), with the index queries in E4M3 too: 128 bytes per key, half the HBM
// stream.  v_mfma_f32_16x16x32_fp8_fp8 takes the same operand layout as the
// bf16 instruction with one byte per element (lane l: A[l%16][8*(l/16) .. +7],
// B[8*(l/16) .. +7][l%16]) and accumulates exactly in fp32 for the values the
// products and sums here produce.
//
// A wave's tile is 32 keys (4 KiB): each 16-byte load instruction covers eight
// whole keys (1 KiB contiguous).  Lane l brings 16-byte chunk l%8 of key
// 8i + l/8; in the wave's LDS slot chunk s of key k sits at 16-byte position
// 8k + (s ^ ((k >> 1) & 7)), so each 16-lane write phase fills 256 contiguous
// bytes and each 32-lane read phase of the 8-byte B operands (key 16*kb + l%16,
// chunk 2*kk + (l/16)/2, half (l/16)%2) touches every bank once.
constexpr int kTile8 = 32;                      // keys per tile (two MFMA column blocks)
constexpr int kD8 = 128;                        // bytes per key
constexpr int kTile8Bytes = kTile8 * kD8;       // 4 KiB
constexpr int kLoads8 = kTile8Bytes / (kWave * 16);  // 4 loads of 1 KiB per tile

// Measured best on MI355X for 128K x 32 and 1M x 4: 4 waves x 16 tiles of 32 keys, 6 tiles ahead.
constexpr int kDecode8Waves = 4;
constexpr int kDecode8Tiles = 16;
constexpr int kDecode8Ahead = 6;

__device__ __forceinline__ f32x4_t mfma16x16x32_fp8(long a, long b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, c, 0, 0, 0);
}

template <int kWaves, int kTilesPerWave, int kAhead8>
__global__ __launch_bounds__(kWaves * kWave) void indexer_decode_fp8_kernel(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ w, const uint8_t* __restrict__ k_idx,
    int64_t k_bstride, const int32_t* __restrict__ q_pos, int T, int L, int nblk, float* __restrict__ scores,
    ZeroRange zero) {
    constexpr int kKeysPerBlock = kWaves * kTile8 * kTilesPerWave;
    __shared__ __attribute__((aligned(16))) uint8_t stage[kWaves * 2 * kTile8Bytes];
    const int row = blockIdx.x / nblk;  // b*T + t
    const int blk = blockIdx.x % nblk;
    const int b = row / T;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int c = lane & 15;
    const int g = lane >> 4;
    const int64_t p = q_pos[row];
    if (zero.base && blk == 0)
        for (int i = threadIdx.x; i < zero.count; i += kWaves * kWave) zero.base[row * zero.stride + i] = 0u;

    // A operands: head 16*ht + c, dims 32*kk + 8*g .. +7 (8 codes).
    long qa[2][4];
    const uint8_t* qrow = q_idx + (int64_t)row * kH * kD8;
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            qa[ht][kk] = *reinterpret_cast<const long*>(qrow + (16 * ht + c) * kD8 + 32 * kk + 8 * g);
    float wv[2][4];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
#pragma unroll
        for (int r = 0; r < 4; ++r) wv[ht][r] = w[(int64_t)row * kH + 16 * ht + 4 * g + r];

    const uint8_t* kb = k_idx + (int64_t)b * k_bstride;
    const int64_t block_start = (int64_t)blk * kKeysPerBlock;
    auto tile_key0 = [&](int j) { return block_start + (int64_t)(kWaves * j + wave) * kTile8; };
    uint8_t* my_stage = stage + wave * 2 * kTile8Bytes;

    u32x4_t buf[kAhead8 + 1][kLoads8];
    auto load_tile = [&](int j, u32x4_t (&dst)[kLoads8]) {
#pragma unroll
        for (int i = 0; i < kLoads8; ++i) {
            int64_t key = tile_key0(j) + 8 * i + (lane >> 3);
            key = key < L ? key : (int64_t)L - 1;  // ragged tail: a valid row, never stored
            dst[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kb + key * kD8 + 16 * (lane & 7)));
        }
    };
#pragma unroll
    for (int j = 0; j < kAhead8; ++j) load_tile(j, buf[j]);

    float sc[kTilesPerWave];
#pragma unroll
    for (int j = 0; j < kTilesPerWave; ++j) {
        if (j + kAhead8 < kTilesPerWave) load_tile(j + kAhead8, buf[(j + kAhead8) % (kAhead8 + 1)]);
        uint8_t* slot = my_stage + (j & 1) * kTile8Bytes;
#pragma unroll
        for (int i = 0; i < kLoads8; ++i) {
            const int k = 8 * i + (lane >> 3);
            *reinterpret_cast<u32x4_t*>(slot + 16 * (8 * k + ((lane & 7) ^ ((k >> 1) & 7)))) =
                buf[j % (kAhead8 + 1)][i];
        }
        float part[2];
#pragma unroll
        for (int kbk = 0; kbk < 2; ++kbk) {
            const int k = 16 * kbk + c;
            f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int s = 2 * kk + (g >> 1);
                const long kv = *reinterpret_cast<const long*>(slot + 16 * (8 * k + (s ^ ((k >> 1) & 7))) + 8 * (g & 1));
                a0 = mfma16x16x32_fp8(qa[0][kk], kv, a0);
                a1 = mfma16x16x32_fp8(qa[1][kk], kv, a1);
            }
            float v = 0.0f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                v = fmaf(wv[0][r], a0[r] > 0.0f ? a0[r] : 0.0f, v);
                v = fmaf(wv[1][r], a1[r] > 0.0f ? a1[r] : 0.0f, v);
            }
            v += __shfl_xor(v, 16, kWave);
            v += __shfl_xor(v, 32, kWave);
            part[kbk] = v;
        }
        // every lane of column c now holds both sums; lane group g < 2 keeps key 16*g + c
        sc[j] = (g & 1) ? part[1] : part[0];
    }
    float* out = scores + (int64_t)row * L;
    if (g < 2) {
#pragma unroll
        for (int j = 0; j < kTilesPerWave; ++j) {
            const int64_t key = tile_key0(j) + 16 * g + c;
            if (key < L) out[key] = key <= p ? sc[j] : -INFINITY;
        }
    }
}

// ------------------------------------------------------------------ multi-query (prefill) chunks
// A chunk of T >= 8 queries of one sequence is a dense contraction: 32*T query
// heads against every key, 2*32*128 flops per (query, key).  One 256-thread
// workgroup takes 16 queries of one sequence and a range of keys; wave w holds
// queries 4w..4w+3 (32 heads x 128 dims each) as MFMA A operands in registers.
// Key tiles of 64 keys go through a double-buffered, swizzled LDS stage and
// every B operand read from it feeds 8 MFMAs (4 queries x 2 head blocks).  The
// ReLU, the head weights and the sum over heads are folded into the epilogue;
// a 3-shuffle transpose-reduce leaves query 4w+g's score in lane group g, so
// one store covers a 16-key sub-tile for the wave's 4 queries.
constexpr int kPfQueries = 16;                 // queries per workgroup
constexpr int kPfQPerWave = 4;
constexpr int kPfTileKeys = 64;                // keys per LDS tile
constexpr int kPfTileBytes = kPfTileKeys * kD * 2;   // 16 KiB
constexpr int kPfKeysPerBlock = 2048;          // keys per workgroup
constexpr int kPrefillMinQueries = 8;          // chunks of at least this many queries per sequence

__global__ __launch_bounds__(256) void indexer_prefill_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w, const uint16_t* __restrict__ k_idx,
    int64_t k_bstride, const int32_t* __restrict__ q_pos, int T, int L, int nqg, int nkb,
    float* __restrict__ scores, ZeroRange zero) {
    __shared__ __attribute__((aligned(16))) uint16_t stage[2 * kPfTileBytes / 2];
    const int kb_i = blockIdx.x % nkb;           // key block
    const int qg = (blockIdx.x / nkb) % nqg;     // query group within the sequence
    const int b = blockIdx.x / (nkb * nqg);
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const int c = lane & 15;
    const int g = lane >> 4;
    const int t0 = qg * kPfQueries + kPfQPerWave * wave;  // this wave's first query

    if (zero.base && kb_i == 0)  // rows of this group, once
        for (int i = threadIdx.x; i < kPfQueries * zero.count; i += 256) {
            const int t = qg * kPfQueries + i / zero.count;
            if (t < T) zero.base[((int64_t)b * T + t) * zero.stride + i % zero.count] = 0u;
        }

    // A operands and head weights of the wave's 4 queries (past the end: the last query, never stored)
    bf16x8_t qa[kPfQPerWave][2][4];
    float wv[kPfQPerWave][2][4];
    int64_t prow[kPfQPerWave];
#pragma unroll
    for (int i = 0; i < kPfQPerWave; ++i) {
        const int t = min(t0 + i, T - 1);
        const int64_t row = (int64_t)b * T + t;
        const uint16_t* qrow = q_idx + row * kH * kD;
#pragma unroll
        for (int ht = 0; ht < 2; ++ht)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                qa[i][ht][kk] = *reinterpret_cast<const bf16x8_t*>(qrow + (16 * ht + c) * kD + 32 * kk + 8 * g);
#pragma unroll
        for (int ht = 0; ht < 2; ++ht)
#pragma unroll
            for (int r = 0; r < 4; ++r) wv[i][ht][r] = w[row * kH + 16 * ht + 4 * g + r];
        prow[i] = row;
    }
    // this lane stores query 4w+g
    const int my_t = t0 + g;
    const int64_t my_row = (int64_t)b * T + min(my_t, T - 1);
    const int64_t my_p = q_pos[my_row];
    float* my_out = scores + my_row * L;

    const uint16_t* kb = k_idx + (int64_t)b * k_bstride;
    const int64_t key0 = (int64_t)kb_i * kPfKeysPerBlock;
    const int ntiles = (int)((min((int64_t)L, key0 + kPfKeysPerBlock) - key0 + kPfTileKeys - 1) / kPfTileKeys);
    // tile loads: thread (wave st, lane) brings chunk lane%16 of keys 16*st + 4i + lane/16, i < 4
    u32x4_t ld[4];
    auto load_tile = [&](int j) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int64_t key = key0 + (int64_t)j * kPfTileKeys + 16 * wave + 4 * i + (lane >> 4);
            key = key < L ? key : (int64_t)L - 1;  // ragged tail: a valid row, never stored
            ld[i] = *reinterpret_cast<const u32x4_t*>(kb + key * kD + 8 * (lane & 15));
        }
    };
    auto store_tile = [&](int j) {  // chunk s of key k (within a 16-key sub-tile) at 16k + (s ^ k)
        uint16_t* sub = stage + (j & 1) * (kPfTileBytes / 2) + wave * (16 * kD);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k = 4 * i + (lane >> 4);
            *reinterpret_cast<u32x4_t*>(sub + 8 * (16 * k + ((lane & 15) ^ k))) = ld[i];
        }
    };
    load_tile(0);
    store_tile(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    for (int j = 0; j < ntiles; ++j) {
        if (j + 1 < ntiles) load_tile(j + 1);  // in flight while tile j is computed
        const uint16_t* tile = stage + (j & 1) * (kPfTileBytes / 2);
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const uint16_t* sub = tile + st * (16 * kD);
            bf16x8_t kv[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                kv[kk] = *reinterpret_cast<const bf16x8_t*>(sub + 8 * (16 * c + ((4 * kk + g) ^ c)));
            float part[kPfQPerWave];
#pragma unroll
            for (int i = 0; i < kPfQPerWave; ++i) {
                f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    a0 = mfma16x16x32(qa[i][0][kk], kv[kk], a0);
                    a1 = mfma16x16x32(qa[i][1][kk], kv[kk], a1);
                }
                float v = 0.0f;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    v = fmaf(wv[i][0][r], a0[r] > 0.0f ? a0[r] : 0.0f, v);
                    v = fmaf(wv[i][1][r], a1[r] > 0.0f ? a1[r] : 0.0f, v);
                }
                part[i] = v;
            }
            // transpose-reduce over the 4 lane groups: group g ends with query g's total
            const bool hi = (g & 2) != 0, lo = (g & 1) != 0;
            const float r0 = __shfl_xor(hi ? part[0] : part[2], 32, kWave);
            const float r1 = __shfl_xor(hi ? part[1] : part[3], 32, kWave);
            const float k0 = (hi ? part[2] : part[0]) + r0;
            const float k1 = (hi ? part[3] : part[1]) + r1;
            const float rr = __shfl_xor(lo ? k0 : k1, 16, kWave);
            const float score = (lo ? k1 : k0) + rr;
            const int64_t key = key0 + (int64_t)j * kPfTileKeys + 16 * st + c;
            if (my_t < T && key < L) my_out[key] = key <= my_p ? score : -INFINITY;
        }
        if (j + 1 < ntiles) store_tile(j + 1);
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    (void)prow;
}


// ------------------------------------------------------------------ E4M3 multi-query (prefill) chunks
// The prefill tile kernel for E4M3 index queries and keys.  gfx950's
// v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3 x E4M3, unit scales) contracts a
// whole 128-byte key in one instruction at twice the bf16 rate: lane (c, g)
// supplies bytes 32g .. 32g+31 of A row c and of B column c (a probe on the box
// confirmed that A and B bytes pair by position).  Work split as in the bf16
// kernel: 16 queries per workgroup, 4 per wave held as A operands (2 head
// blocks x 32 bytes each), 64-key tiles through a double-buffered LDS stage
// (16-byte chunk s of key k at 8k + (s ^ ((k >> 1) & 7)): conflict-free), and
// every B operand read feeds 8 instructions.
constexpr int kPf8TileKeys = 64;
constexpr int kPf8TileBytes = kPf8TileKeys * kD8;  // 8 KiB

typedef int i32x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4_t mfma16x16x128_fp8(i32x8_t a, i32x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);  // E4M3, scales 2^0
}

__global__ __launch_bounds__(256) void indexer_prefill_fp8_kernel(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ w, const uint8_t* __restrict__ k_idx,
    int64_t k_bstride, const int32_t* __restrict__ q_pos, int T, int L, int nqg, int nkb, float* __restrict__ scores,
    ZeroRange zero) {
    __shared__ __attribute__((aligned(16))) uint8_t stage[2 * kPf8TileBytes];
    const int kb_i = blockIdx.x % nkb;
    const int qg = (blockIdx.x / nkb) % nqg;
    const int b = blockIdx.x / (nkb * nqg);
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int c = lane & 15;
    const int g = lane >> 4;
    const int t0 = qg * kPfQueries + kPfQPerWave * wave;

    if (zero.base && kb_i == 0)
        for (int i = threadIdx.x; i < kPfQueries * zero.count; i += 256) {
            const int t = qg * kPfQueries + i / zero.count;
            if (t < T) zero.base[((int64_t)b * T + t) * zero.stride + i % zero.count] = 0u;
        }

    // A operands: head 16*ht + c of the wave's 4 queries, bytes 32g .. 32g+31
    i32x8_t qa[kPfQPerWave][2];
    float wv[kPfQPerWave][2][4];
#pragma unroll
    for (int i = 0; i < kPfQPerWave; ++i) {
        const int t = min(t0 + i, T - 1);  // past the end: the last query, never stored
        const int64_t row = (int64_t)b * T + t;
        const uint8_t* qrow = q_idx + row * kH * kD8;
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) qa[i][ht] = *reinterpret_cast<const i32x8_t*>(qrow + (16 * ht + c) * kD8 + 32 * g);
#pragma unroll
        for (int ht = 0; ht < 2; ++ht)
#pragma unroll
            for (int r = 0; r < 4; ++r) wv[i][ht][r] = w[row * kH + 16 * ht + 4 * g + r];
    }
    const int my_t = t0 + g;
    const int64_t my_row = (int64_t)b * T + min(my_t, T - 1);
    const int64_t my_p = q_pos[my_row];
    float* my_out = scores + my_row * L;

    const uint8_t* kb = k_idx + (int64_t)b * k_bstride;
    const int64_t key0 = (int64_t)kb_i * kPfKeysPerBlock;
    const int ntiles = (int)((min((int64_t)L, key0 + kPfKeysPerBlock) - key0 + kPf8TileKeys - 1) / kPf8TileKeys);
    // tile loads: thread i brings 16-byte chunks i and i + 256 (key = chunk / 8, s = chunk % 8)
    u32x4_t ld[2];
    auto load_tile = [&](int j) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int chunk = (int)threadIdx.x + 256 * h;
            int64_t key = key0 + (int64_t)j * kPf8TileKeys + (chunk >> 3);
            key = key < L ? key : (int64_t)L - 1;  // ragged tail: a valid row, never stored
            ld[h] = *reinterpret_cast<const u32x4_t*>(kb + key * kD8 + 16 * (chunk & 7));
        }
    };
    auto store_tile = [&](int j) {
        uint8_t* tile = stage + (j & 1) * kPf8TileBytes;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int chunk = (int)threadIdx.x + 256 * h;
            const int k = chunk >> 3, sc = chunk & 7;
            *reinterpret_cast<u32x4_t*>(tile + 16 * (8 * k + (sc ^ ((k >> 1) & 7)))) = ld[h];
        }
    };
    load_tile(0);
    store_tile(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    for (int j = 0; j < ntiles; ++j) {
        if (j + 1 < ntiles) load_tile(j + 1);  // in flight while tile j is computed
        const uint8_t* tile = stage + (j & 1) * kPf8TileBytes;
#pragma unroll
        for (int st = 0; st < kPf8TileKeys / 16; ++st) {
            const int k = 16 * st + c;  // key of this lane's B column
            const int f = (k >> 1) & 7;
            const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(tile + 16 * (8 * k + ((2 * g) ^ f)));
            const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(tile + 16 * (8 * k + ((2 * g + 1) ^ f)));
            const i32x8_t kv = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            float part[kPfQPerWave];
#pragma unroll
            for (int i = 0; i < kPfQPerWave; ++i) {
                const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
                const f32x4_t a0 = mfma16x16x128_fp8(qa[i][0], kv, zero4);
                const f32x4_t a1 = mfma16x16x128_fp8(qa[i][1], kv, zero4);
                float v = 0.0f;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    v = fmaf(wv[i][0][r], a0[r] > 0.0f ? a0[r] : 0.0f, v);
                    v = fmaf(wv[i][1][r], a1[r] > 0.0f ? a1[r] : 0.0f, v);
                }
                part[i] = v;
            }
            // transpose-reduce over the 4 lane groups: group g ends with query g's total
            const bool hi_g = (g & 2) != 0, lo_g = (g & 1) != 0;
            const float r0 = __shfl_xor(hi_g ? part[0] : part[2], 32, kWave);
            const float r1 = __shfl_xor(hi_g ? part[1] : part[3], 32, kWave);
            const float k0 = (hi_g ? part[2] : part[0]) + r0;
            const float k1 = (hi_g ? part[3] : part[1]) + r1;
            const float rr = __shfl_xor(lo_g ? k0 : k1, 16, kWave);
            const float score = (lo_g ? k1 : k0) + rr;
            const int64_t key = key0 + (int64_t)j * kPf8TileKeys + 16 * st + c;
            if (my_t < T && key < L) my_out[key] = key <= my_p ? score : -INFINITY;
        }
        if (j + 1 < ntiles) store_tile(j + 1);
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
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

template <int W, int N, int A>
hipError_t launch_indexer_fp8_cfg(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, int64_t k_bstride,
                                  const int32_t* q_pos, int B, int T, int L, float* scores, hipStream_t stream,
                                  ZeroRange zero) {
    constexpr int keys_per_block = W * kTile8 * N;
    const int nblk = (L + keys_per_block - 1) / keys_per_block;
    dim3 grid((unsigned)((int64_t)nblk * B * T));
    hipLaunchKernelGGL((indexer_decode_fp8_kernel<W, N, A>), grid, dim3(W * kWave), 0, stream, q_idx, w, k_idx,
                       k_bstride, q_pos, T, L, nblk, scores, zero);
    return hipGetLastError();
}

hipError_t launch_indexer_fp8(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, int64_t k_bstride,
                              const int32_t* q_pos, int B, int T, int L, float* scores, hipStream_t stream,
                              ZeroRange zero) {
    if (T >= kPrefillMinQueries) {
        const int nqg = (T + kPfQueries - 1) / kPfQueries;
        const int nkb = (L + kPfKeysPerBlock - 1) / kPfKeysPerBlock;
        hipLaunchKernelGGL(indexer_prefill_fp8_kernel, dim3((unsigned)((int64_t)B * nqg * nkb)), dim3(256), 0, stream,
                           q_idx, w, k_idx, k_bstride, q_pos, T, L, nqg, nkb, scores, zero);
        return hipGetLastError();
    }
    return launch_indexer_fp8_cfg<kDecode8Waves, kDecode8Tiles, kDecode8Ahead>(q_idx, w, k_idx, k_bstride, q_pos, B,
                                                                               T, L, scores, stream, zero);
}

hipError_t launch_indexer(const uint16_t* q_idx, const float* w, const uint16_t* k_idx, int64_t k_bstride,
                          const int32_t* q_pos, int B, int T, int L, float* scores, hipStream_t stream,
                          ZeroRange zero) {
    if (T >= kPrefillMinQueries) {
        const int nqg = (T + kPfQueries - 1) / kPfQueries;
        const int nkb = (L + kPfKeysPerBlock - 1) / kPfKeysPerBlock;
        hipLaunchKernelGGL(indexer_prefill_kernel, dim3((unsigned)((int64_t)B * nqg * nkb)), dim3(256), 0, stream,
                           q_idx, w, k_idx, k_bstride, q_pos, T, L, nqg, nkb, scores, zero);
        return hipGetLastError();
    }
    return launch_indexer_cfg<kDecodeWaves, kDecodeTiles>(q_idx, w, k_idx, k_bstride, q_pos, B, T, L, scores, stream,
                                                          zero);
}

}  // namespace dsa
