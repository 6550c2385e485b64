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
// Keys are read with 16-byte loads through a raw buffer of the sequence's L
// rows (rows past L read as zeros, so the ragged end needs no clamp), every
// instruction covering four whole keys (1 KiB contiguous), and the sum over
// the MFMA lane groups uses permlane swaps.  One 16-key tile per wave is in
// flight at a time: with two workgroups of four waves per CU that is about
// 8 MiB in flight over the chip, which streams at the chip's measured read
// rate (7.0 TB/s at 128K x 32; one or three tiles ahead per wave measured 2%
// and 7% slower).  Each tile is
// then turned into the MFMA operand layout through a small wave-private LDS
// slot: lane l writes chunk l%16 of key 4i + l/16, and reads back chunk
// 4kk + l/16 of key l%16.  Chunk s of key k is stored at position 16k + (s ^ k),
// which makes both the writes and the reads bank-conflict free.  Scores wait
// in LDS and are stored after the stream, so the loop contains only loads.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "common.h"

namespace dsa {
namespace {

// ReLU as one v_max_f32: this file is compiled with -fno-honor-nans, so max(x, 0)
// needs no extra instruction to quiet a signalling NaN first; scores of finite
// inputs are unchanged.
__device__ __forceinline__ float relu(float x) { return fmaxf(x, 0.0f); }

constexpr int kH = 32;
constexpr int kD = 128;
constexpr int kTile = 16;                      // keys per MFMA tile
constexpr int kTileBytes = kTile * kD * 2;     // 4 KiB
constexpr int kLoads = kTileBytes / (kWave * 16);  // 4 loads of 1 KiB per tile
// 4 waves x 16 tiles of 16 keys per block (1024 keys), no tile loaded ahead.
constexpr int kAhead = 0;                      // tiles loaded ahead of the one computed
constexpr int kDecodeWaves = 4;
constexpr int kDecodeTiles = 16;               // tiles per wave and block
constexpr int kDecodeMaxPer = 8;               // blocks per workgroup (their scores wait in LDS)

// Top-k preparation (TopkPrep) by a decode launch: the first key block of each
// row clears the row's counters; with `hist`, every block counts the top 11-bit
// digit of each visible score in LDS as it is computed and, at the end, adds
// the non-zero bins to the row's histogram.
__device__ __forceinline__ void prep_start(const TopkPrep& prep, int row, int blk, uint32_t* hist_lds, int nthreads) {
    if (prep.base && blk == 0)
        for (int i = threadIdx.x; i < prep.zero_count; i += nthreads)
            prep.base[row * prep.stride + prep.zero_off + i] = 0u;
    if (prep.hist) {
        for (int i = threadIdx.x; i < kTopBins; i += nthreads) hist_lds[i] = 0u;
        __syncthreads();  // before the first key is counted (and before any key load is in flight)
    }
}

// Sum over the four 16-lane groups of a wave, every lane ending with the total
// (the MFMA C layout spreads a key's 32 heads over the groups).
// v_permlane16_swap(x, x) pairs each row with its neighbour, v_permlane32_swap
// each half with the other; the two swapped copies add up to the pair's sum.
__device__ __forceinline__ float sum_all_groups(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(h[0]) + __uint_as_float(h[1]);
}

// Histogram bin of a score, or the spare bin kTopBins (never flushed) for a
// key the selection does not see: one LDS add with no branch.
__device__ __forceinline__ int hist_bin(float score, bool counted) {
    return counted ? (int)(score_key(score) >> 21) : kTopBins;
}

__device__ __forceinline__ void prep_flush(const TopkPrep& prep, int row, const uint32_t* hist_lds, int nthreads) {
    __syncthreads();  // every wave's counts are in
    uint32_t* gh = prep.base + row * prep.stride;
    for (int i = threadIdx.x; i < kTopBins; i += nthreads) {
        const uint32_t v = hist_lds[i];
        if (v) atomicAdd(&gh[i], v);
    }
}

// A workgroup's range of scores, waiting in LDS (sst[0, nkeys)), to the row
// at keys key0 .. key0 + nkeys - 1: 16-byte stores when rows start 16-byte aligned.
__device__ __forceinline__ void store_scores(float* row_out, const float* sst, int64_t key0, int nkeys, int L,
                                             int nthreads) {
    const __amdgpu_buffer_rsrc_t out = wt_rsrc(row_out);
    const bool vec = (L & 3) == 0;
    for (int i = 4 * (int)threadIdx.x; i < nkeys; i += 4 * nthreads) {
        if (vec && i + 4 <= nkeys) {
            store_wt16(out, 4u * (uint32_t)(key0 + i), *reinterpret_cast<const u32x4_t*>(&sst[i]));
        } else {
            for (int e = i; e < nkeys && e < i + 4; ++e) store_wt4(out, 4u * (uint32_t)(key0 + e), sst[e]);
        }
    }
}

// Workgroups run through `per` (at most kDecodeMaxPer) consecutive key blocks
// of one row (about two resident workgroups per CU over all rows), so the
// query and its weights are loaded once, the histogram is flushed once, and
// the rolling window of tiles runs on across block boundaries instead of each
// block starting cold (a workgroup per block left about an eighth of the
// chip's slots idle between one workgroup's end and the next one's first
// load).  The scores wait in LDS and are stored once the range is done: a
// store in flight among the loads would make the compiler wait for every
// outstanding load at the next use (it cannot order loads after stores).
template <int kWaves, int kAheadT>
__global__ __launch_bounds__(kWaves * kWave) void indexer_decode_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w, const uint16_t* __restrict__ k_idx,
    int64_t k_bstride, const int32_t* __restrict__ q_pos, int T, int L, int nblk, int wpr, int per,
    float* __restrict__ scores, TopkPrep prep) {
    constexpr int kTilesPerWave = kDecodeTiles;
    constexpr int kKeysPerBlock = kWaves * kTile * kTilesPerWave;
    constexpr int kBufs = kAheadT + 1;
    static_assert(kTilesPerWave % 4 == 0, "the four lane groups take whole tiles each");
    static_assert(kTilesPerWave % kBufs == 0, "tile j of every block sits in buffer j % kBufs");
    __shared__ __attribute__((aligned(16))) uint16_t stage[kWaves * 2 * kTileBytes / 2];
    __shared__ uint32_t hist_lds[kTopBins + 1];  // + the spare bin of keys not counted
    __shared__ __attribute__((aligned(16))) float sst[kDecodeMaxPer * kKeysPerBlock];  // scores of the range
    const int row = blockIdx.x / wpr;  // b*T + t
    const int blk0 = (blockIdx.x % wpr) * per;
    const int blk1 = min(blk0 + per, nblk);
    if (blk0 >= blk1) return;
    const int b = row / T;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int c = lane & 15;  // key within tile (B/C column)
    const int g = lane >> 4;  // lane group: 8-dim slice of each 32-dim step; head row block in C
    const int64_t p = q_pos[row];
    const int last_seen = (int)min(p, (int64_t)L - 1);  // keys the selection counts: 0 .. last_seen
    prep_start(prep, row, blk0, hist_lds, kWaves * kWave);

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

    // The sequence's keys as a buffer of L rows: rows past L (the ragged tail,
    // the last block's look-ahead) read as zeros and their scores are never used.
    const __amdgpu_buffer_rsrc_t krs = sized_rsrc(k_idx + (int64_t)b * k_bstride, (uint32_t)L * (kD * 2));
    // Tile j of block blk for this wave covers keys blk*kKeysPerBlock + (kWaves*j + wave)*16 .. +15;
    // at each step the block's waves read kWaves*16 consecutive keys.
    auto tile_key0 = [&](int blk, int j) { return blk * kKeysPerBlock + (kWaves * j + wave) * kTile; };
    uint16_t* my_stage = stage + wave * kTileBytes;  // two 4 KiB slots per wave
    const uint32_t ld_lane = (uint32_t)(lane >> 4) * (kD * 2) + 16u * (lane & 15);

    u32x4_t buf[kBufs][kLoads];
    auto load_tile = [&](int blk, int j, u32x4_t (&dst)[kLoads]) {
#pragma unroll
        for (int i = 0; i < kLoads; ++i)  // keys tile_key0 + 4i + lane/16, 16-byte chunk lane%16
            dst[i] = load_nt16(krs, (uint32_t)tile_key0(blk, j) * (kD * 2) + ld_lane + i * (4 * kD * 2));
    };
    // In tile order (no reordering by the scheduler): the loop's first wait,
    // for tile 0, then counts only the loads issued after it, on entry as on
    // every later block.
#pragma unroll
    for (int j = 0; j < kAheadT; ++j) {
        load_tile(blk0, j, buf[j]);
        __builtin_amdgcn_sched_barrier(0);
    }

    for (int blk = blk0; blk < blk1; ++blk) {
        float sc[kTilesPerWave];
#pragma unroll
        for (int j = 0; j < kTilesPerWave; ++j) {
            // the window runs on into the next block (loaded every time, so the wait counts stay fixed)
            if (j + kAheadT < kTilesPerWave) load_tile(blk, j + kAheadT, buf[(j + kAheadT) % kBufs]);
            else load_tile(blk + 1, j + kAheadT - kTilesPerWave, buf[(j + kAheadT) % kBufs]);
            // registers -> LDS (swizzled) -> MFMA operand layout
            uint16_t* slot = my_stage + (j & 1) * (kTileBytes / 2);
#pragma unroll
            for (int i = 0; i < kLoads; ++i) {
                const int k = 4 * i + (lane >> 4);
                *reinterpret_cast<u32x4_t*>(slot + 8 * (16 * k + ((lane & 15) ^ k))) = buf[j % kBufs][i];
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
                part = fmaf(wv[0][r], relu(a0[r]), part);
                part = fmaf(wv[1][r], relu(a1[r]), part);
            }
            part = sum_all_groups(part);
            sc[j] = part;
            if (prep.hist && g == (j & 3))  // lane group g counts the tiles j = g (mod 4)
                atomicAdd(&hist_lds[hist_bin(part, tile_key0(blk, j) + c <= last_seen)], 1u);
        }
        if (g == 0) {  // lane group 0 keeps the scores (the others hold the same sums)
#pragma unroll
            for (int j = 0; j < kTilesPerWave; ++j) {
                const int64_t key = tile_key0(blk, j) + c;
                sst[(blk - blk0) * kKeysPerBlock + (kWaves * j + wave) * kTile + c] = key <= p ? sc[j] : -INFINITY;
            }
        }
    }
    __syncthreads();  // every wave's scores (and histogram counts) are in LDS
    store_scores(scores + (int64_t)row * L, sst, (int64_t)blk0 * kKeysPerBlock,
                 (int)min((int64_t)(blk1 - blk0) * kKeysPerBlock, (int64_t)L - (int64_t)blk0 * kKeysPerBlock), L,
                 kWaves * kWave);
    if (prep.hist) prep_flush(prep, row, hist_lds, kWaves * kWave);
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

// 4 waves x 16 tiles of 32 keys per block (2048 keys), no tile loaded ahead
// (with the buffer loads, measured at 128K x 32: 79.5 us against 80.8 with one
// and 84.5 with three; at 1M x 4: 79.4 against 81.4 with one).
constexpr int kDecode8Waves = 4;
constexpr int kDecode8Tiles = 16;
constexpr int kDecode8Ahead = 0;
constexpr int kDecode8MaxPer = 4;  // blocks per workgroup (their scores wait in LDS)

__device__ __forceinline__ f32x4_t mfma16x16x32_fp8(long a, long b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, c, 0, 0, 0);
}

// Like the bf16 scan, each workgroup runs through `per` (at most
// kDecode8MaxPer) consecutive blocks of one row, the scores waiting in LDS.
template <int kWaves, int kAhead8>
__global__ __launch_bounds__(kWaves * kWave) void indexer_decode_fp8_kernel(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ w, const uint8_t* __restrict__ k_idx,
    int64_t k_bstride, const int32_t* __restrict__ q_pos, int T, int L, int nblk, int wpr, int per,
    float* __restrict__ scores, TopkPrep prep) {
    constexpr int kTilesPerWave = kDecode8Tiles;
    constexpr int kKeysPerBlock = kWaves * kTile8 * kTilesPerWave;
    constexpr int kBufs = kAhead8 + 1;
    static_assert(kTilesPerWave % 2 == 0, "lane groups 2, 3 take the odd tiles");
    static_assert(kTilesPerWave % kBufs == 0, "tile j of every block sits in buffer j % kBufs");
    __shared__ __attribute__((aligned(16))) uint8_t stage[kWaves * 2 * kTile8Bytes];
    __shared__ uint32_t hist_lds[kTopBins + 1];  // + the spare bin of keys not counted
    __shared__ __attribute__((aligned(16))) float sst[kDecode8MaxPer * kKeysPerBlock];  // scores of the range
    const int row = blockIdx.x / wpr;  // b*T + t
    const int blk0 = (blockIdx.x % wpr) * per;
    const int blk1 = min(blk0 + per, nblk);
    if (blk0 >= blk1) return;
    const int b = row / T;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int c = lane & 15;
    const int g = lane >> 4;
    const int64_t p = q_pos[row];
    const int last_seen = (int)min(p, (int64_t)L - 1);  // keys the selection counts: 0 .. last_seen
    prep_start(prep, row, blk0, hist_lds, kWaves * kWave);

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

    // keys past L (the ragged tail, the last block's look-ahead) read as zeros, their scores never used
    const __amdgpu_buffer_rsrc_t krs = sized_rsrc(k_idx + (int64_t)b * k_bstride, (uint32_t)L * kD8);
    auto tile_key0 = [&](int blk, int j) { return blk * kKeysPerBlock + (kWaves * j + wave) * kTile8; };
    uint8_t* my_stage = stage + wave * 2 * kTile8Bytes;

    u32x4_t buf[kBufs][kLoads8];
    auto load_tile = [&](int blk, int j, u32x4_t (&dst)[kLoads8]) {
#pragma unroll
        for (int i = 0; i < kLoads8; ++i)  // keys tile_key0 + 8i + lane/8, 16-byte chunk lane%8: 1 KiB contiguous
            dst[i] = load_nt16(krs, (uint32_t)tile_key0(blk, j) * kD8 + 16u * lane + i * 1024);
    };
#pragma unroll
    for (int j = 0; j < kAhead8; ++j) {  // in tile order (see the bf16 scan)
        load_tile(blk0, j, buf[j]);
        __builtin_amdgcn_sched_barrier(0);
    }

    for (int blk = blk0; blk < blk1; ++blk) {
        float sc[kTilesPerWave];
#pragma unroll
        for (int j = 0; j < kTilesPerWave; ++j) {
            if (j + kAhead8 < kTilesPerWave) load_tile(blk, j + kAhead8, buf[(j + kAhead8) % kBufs]);
            else load_tile(blk + 1, j + kAhead8 - kTilesPerWave, buf[(j + kAhead8) % kBufs]);
            uint8_t* slot = my_stage + (j & 1) * kTile8Bytes;
#pragma unroll
            for (int i = 0; i < kLoads8; ++i) {
                const int k = 8 * i + (lane >> 3);
                *reinterpret_cast<u32x4_t*>(slot + 16 * (8 * k + ((lane & 7) ^ ((k >> 1) & 7)))) = buf[j % kBufs][i];
            }
            float part[2];
#pragma unroll
            for (int kbk = 0; kbk < 2; ++kbk) {
                const int k = 16 * kbk + c;
                f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const int s = 2 * kk + (g >> 1);
                    const long kv =
                        *reinterpret_cast<const long*>(slot + 16 * (8 * k + (s ^ ((k >> 1) & 7))) + 8 * (g & 1));
                    a0 = mfma16x16x32_fp8(qa[0][kk], kv, a0);
                    a1 = mfma16x16x32_fp8(qa[1][kk], kv, a1);
                }
                float v = 0.0f;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    v = fmaf(wv[0][r], relu(a0[r]), v);
                    v = fmaf(wv[1][r], relu(a1[r]), v);
                }
                part[kbk] = sum_all_groups(v);
            }
            // every lane of column c now holds both sums; lane group g keeps key 16*(g & 1) + c
            sc[j] = (g & 1) ? part[1] : part[0];
            if (prep.hist && (g >> 1) == (j & 1))  // groups 0, 1 count the even tiles, groups 2, 3 the odd ones
                atomicAdd(&hist_lds[hist_bin(sc[j], tile_key0(blk, j) + 16 * (g & 1) + c <= last_seen)], 1u);
        }
        if (g < 2) {  // lane groups 0 and 1 keep the tile's two 16-key halves
#pragma unroll
            for (int j = 0; j < kTilesPerWave; ++j) {
                const int64_t key = tile_key0(blk, j) + 16 * g + c;
                sst[(blk - blk0) * kKeysPerBlock + (kWaves * j + wave) * kTile8 + 16 * g + c] =
                    key <= p ? sc[j] : -INFINITY;
            }
        }
    }
    __syncthreads();  // every wave's scores (and histogram counts) are in LDS
    store_scores(scores + (int64_t)row * L, sst, (int64_t)blk0 * kKeysPerBlock,
                 (int)min((int64_t)(blk1 - blk0) * kKeysPerBlock, (int64_t)L - (int64_t)blk0 * kKeysPerBlock), L,
                 kWaves * kWave);
    if (prep.hist) prep_flush(prep, row, hist_lds, kWaves * kWave);
}

// ------------------------------------------------------------------ multi-query (prefill) chunks
// A chunk of T >= 8 queries of one sequence is a dense contraction: 32*T query
// heads against every key, 2*32*128 flops per (query, key).  One 256-thread
// workgroup takes 16 queries of one sequence and a range of keys; wave w holds
// queries 4w..4w+3 (32 heads x 128 dims each) as MFMA A operands in registers.
// Key tiles of 64 keys go through a double-buffered, swizzled LDS stage and
// every B operand read from it feeds 8 MFMAs (4 queries x 2 head blocks).  The
// ReLU, the head weights and the sum over heads are folded into the epilogue;
// a sum over the four lane groups by permlane swaps leaves query 4w+g's score
// in lane group g, so one store covers a 16-key sub-tile for the wave's 4
// queries.
constexpr int kPfQueries = 16;                 // queries per workgroup
constexpr int kPfQPerWave = 4;
constexpr int kPfTileKeys = 64;                // keys per LDS tile
constexpr int kPfTileBytes = kPfTileKeys * kD * 2;   // 16 KiB
constexpr int kPfKeysPerBlock = 2048;          // keys per workgroup
constexpr int kPrefillMinQueries = 8;          // chunks of at least this many queries per sequence

// Causal skip for a multi-query workgroup: keys past the largest position of
// its queries are visible to none of them, so whole tiles past it are neither
// loaded nor computed; their scores are written as -inf (fill_masked).
__device__ __forceinline__ int64_t group_max_pos(const int32_t* __restrict__ q_pos, int b, int T, int qg) {
    int64_t m = -1;
#pragma unroll
    for (int i = 0; i < kPfQueries; ++i) {
        const int t = min(qg * kPfQueries + i, T - 1);
        m = max(m, (int64_t)q_pos[(int64_t)b * T + t]);
    }
    return m;
}

// Smallest position among a multi-query workgroup's queries: key tiles below
// it are visible to every query of the group.
__device__ __forceinline__ int64_t group_min_pos(const int32_t* __restrict__ q_pos, int b, int T, int qg) {
    int64_t m = INT64_MAX;
#pragma unroll
    for (int i = 0; i < kPfQueries; ++i) {
        const int t = min(qg * kPfQueries + i, T - 1);
        m = min(m, (int64_t)q_pos[(int64_t)b * T + t]);
    }
    return m;
}

// Tile loop of a multi-query workgroup: tile(j, masked, parity) for j < ntiles,
// the first nfull tiles (every key below L and visible to every query) without
// masking, in pairs so that each tile's LDS buffer (j & 1) is a compile-time
// constant; a tile past nfull may still be fully visible, and masking it
// changes nothing.
template <typename Tile>
__device__ __forceinline__ void pf_tile_runs(int ntiles, int nfull, Tile&& tile) {
    using F = std::false_type;
    using M = std::true_type;
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    int j = 0;
    for (; j + 2 <= nfull; j += 2) {
        tile(j, F(), P0());
        tile(j + 1, F(), P1());
    }
    for (; j < ntiles; j += 2) {
        tile(j, M(), P0());
        if (j + 1 < ntiles) tile(j + 1, M(), P1());
    }
}

// -inf for keys [k0, k1) of the group's score rows (queries below T).
__device__ __forceinline__ void fill_masked(__amdgpu_buffer_rsrc_t grp_out, int qg, int T, int L, int64_t k0,
                                            int64_t k1) {
    const int nk = (int)(k1 - k0);
    if (nk <= 0) return;
    const int nq = min(kPfQueries, T - qg * kPfQueries);
    for (int i = threadIdx.x; i < nq * nk; i += 256)
        store_wt4(grp_out, 4u * (uint32_t)((int64_t)(i / nk) * L + k0 + i % nk), -INFINITY);
}

// The wave's 4 per-query partial scores summed over its 4 lane groups: lane
// group g returns query g's total.  v_permlane32_swap trades the upper 32
// lanes of its first operand for the lower 32 of its second, and
// v_permlane16_swap the odd 16-lane rows of its first operand for the even
// rows of its second; after each swap the two registers add up to one query's
// sum over twice as many lane groups.  No LDS round trip, no lane selects.
__device__ __forceinline__ float sum_lane_groups(const float (&part)[4]) {
    const auto s02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]), __float_as_uint(part[2]), false, false);
    const auto s13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[1]), __float_as_uint(part[3]), false, false);
    const float x = __uint_as_float(s02[0]) + __uint_as_float(s02[1]);  // lanes 0-31: query 0, 32-63: query 2
    const float y = __uint_as_float(s13[0]) + __uint_as_float(s13[1]);  // lanes 0-31: query 1, 32-63: query 3
    const auto sxy = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    return __uint_as_float(sxy[0]) + __uint_as_float(sxy[1]);
}

// Per-lane constants of a multi-query workgroup's score stores: lane group g
// writes row 4*wave + g of the group's score rows, key column c of each
// 16-key sub-tile.  The row buffer ends after the group's last query below T,
// so rows past it drop their stores; keys past L get an offset past the end.
struct PfOut {
    __amdgpu_buffer_rsrc_t rs;
    uint32_t off;  // bytes: (row * L + key0 + c) * 4
    int nk;        // keys of the block below L, minus c
    int vis;       // last key of the block this lane's query sees, minus c (may be < 0)
};
__device__ __forceinline__ PfOut pf_out(float* scores, const int32_t* __restrict__ q_pos, int b, int T, int L, int qg,
                                        int wave, int g, int c, int64_t key0) {
    PfOut o;
    const int nq = min(kPfQueries, T - qg * kPfQueries);
    o.rs = sized_rsrc(scores + ((int64_t)b * T + qg * kPfQueries) * L, 4u * (uint32_t)nq * (uint32_t)L);
    const int row = kPfQPerWave * wave + g;
    o.off = 4u * ((uint32_t)row * (uint32_t)L + (uint32_t)key0 + (uint32_t)c);
    o.nk = (int)min((int64_t)L - key0, (int64_t)kPfKeysPerBlock) - c;
    const int64_t p = q_pos[(int64_t)b * T + min(qg * kPfQueries + row, T - 1)];
    o.vis = (int)max(min(p - key0, (int64_t)kPfKeysPerBlock), (int64_t)-1) - c;
    return o;
}
// Score of key key0 + kbase + c (kbase: the sub-tile's first key in the
// block, wave-uniform): -inf past the query's position; dropped for keys past
// L and rows past the last query.  Unmasked (a tile below L that every query
// sees): the wave-uniform key offset goes in the scalar offset; rows past the
// last query still fall outside the buffer by their own offset.
template <bool kMasked>
__device__ __forceinline__ void pf_store(const PfOut& o, int kbase, float score) {
    if constexpr (kMasked) {
        const uint32_t off = kbase < o.nk ? o.off + 4u * (uint32_t)kbase : kOutOfRange;
        store_wt4(o.rs, off, kbase <= o.vis ? score : -INFINITY);
    } else {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(score), o.rs, (int)o.off, (int)(4u * (uint32_t)kbase), 16);
    }
}

__global__ __launch_bounds__(256) void indexer_prefill_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w, const uint16_t* __restrict__ k_idx,
    int64_t k_bstride, const int32_t* __restrict__ q_pos, int T, int L, int nqg, int nkb,
    float* __restrict__ scores, TopkPrep prep) {
    __shared__ __attribute__((aligned(16))) uint16_t stage[2 * kPfTileBytes / 2];
    const int kb_i = blockIdx.x % nkb;           // key block
    const int qg = (blockIdx.x / nkb) % nqg;     // query group within the sequence
    const int b = blockIdx.x / (nkb * nqg);
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int c = lane & 15;
    const int g = lane >> 4;
    const int t0 = qg * kPfQueries + kPfQPerWave * wave;  // this wave's first query

    if (prep.base && kb_i == 0)  // rows of this group, once
        for (int i = threadIdx.x; i < kPfQueries * prep.zero_count; i += 256) {
            const int t = qg * kPfQueries + i / prep.zero_count;
            if (t < T) prep.base[((int64_t)b * T + t) * prep.stride + prep.zero_off + i % prep.zero_count] = 0u;
        }

    // A operands and head weights of the wave's 4 queries (past the end: the last query, never stored)
    bf16x8_t qa[kPfQPerWave][2][4];
    float wv[kPfQPerWave][2][4];
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
    }
    const int64_t key0 = (int64_t)kb_i * kPfKeysPerBlock;
    const PfOut out = pf_out(scores, q_pos, b, T, L, qg, wave, g, c, key0);

    const int64_t kblk_end = min((int64_t)L, key0 + kPfKeysPerBlock);
    const int64_t kvis_end = min(kblk_end, max(key0, group_max_pos(q_pos, b, T, qg) + 1));
    const int ntiles = (int)((kvis_end - key0 + kPfTileKeys - 1) / kPfTileKeys);
    const int64_t kall_end = min(kblk_end, max(key0, group_min_pos(q_pos, b, T, qg) + 1));  // seen by all
    const int nfull = (int)((kall_end - key0) / kPfTileKeys);
    fill_masked(wt_rsrc(scores + ((int64_t)b * T + qg * kPfQueries) * L), qg, T, L,
                key0 + (int64_t)ntiles * kPfTileKeys, kblk_end);
    if (ntiles == 0) return;
    // tile loads: thread (wave st, lane) brings chunk lane%16 of keys 16*st + 4i + lane/16, i < 4;
    // keys past L read zeros (their scores are never stored), so the tile after the last is safe
    const __amdgpu_buffer_rsrc_t krs = sized_rsrc(k_idx + (int64_t)b * k_bstride, (uint32_t)L * (kD * 2));
    const uint32_t ld_off = (uint32_t)key0 * (kD * 2) + (16 * wave + (lane >> 4)) * (kD * 2) + 16 * (lane & 15);
    u32x4_t ld[4];
    auto load_tile = [&](int j) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            ld[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                    krs, (int)(ld_off + (uint32_t)j * kPfTileBytes + i * 4 * kD * 2), 0, 0));
    };
    auto store_tile = [&](int parity) {  // chunk s of key k (within a 16-key sub-tile) at 16k + (s ^ k)
        uint16_t* sub = stage + parity * (kPfTileBytes / 2) + wave * (16 * kD);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k = 4 * i + (lane >> 4);
            *reinterpret_cast<u32x4_t*>(sub + 8 * (16 * k + ((lane & 15) ^ k))) = ld[i];
        }
    };
    load_tile(0);
    store_tile(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    pf_tile_runs(ntiles, nfull, [&](int j, auto masked, auto parity) {
        constexpr int kP = decltype(parity)::value;
        load_tile(j + 1);  // in flight while tile j is computed
        const uint16_t* tile = stage + kP * (kPfTileBytes / 2);
        // B operands of sub-tile st + 1 are read while sub-tile st is computed
        bf16x8_t kv[2][4];
        auto read_sub = [&](int st) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                kv[st & 1][kk] =
                    *reinterpret_cast<const bf16x8_t*>(tile + st * (16 * kD) + 8 * (16 * c + ((4 * kk + g) ^ c)));
        };
        // The tile's (sub-tile, query) pairs p = 4 st + i as a pipeline: each
        // of pair p's 8 MFMAs issues beside one ReLU and weighted add of pair
        // p - 1, in the plain sum's order (head row r, then head block), so two
        // VALU instructions sit behind every MFMA instead of a VALU-only
        // epilogue after each query; sched_barrier keeps that order.
        const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
        f32x4_t acc[2][2];  // [pair parity][head block]
        float part[kPfQPerWave];
        float v = 0.0f;
        read_sub(0);
#pragma unroll
        for (int pp = 0; pp <= 4 * kPfQPerWave; ++pp) {
            const int st = pp / kPfQPerWave, i = pp % kPfQPerWave;                 // pair pp (pp < 16)
            const int pst = (pp - 1) / kPfQPerWave, pi = (pp - 1) % kPfQPerWave;   // pair pp - 1 (pp > 0)
            if (pp < 4 * kPfQPerWave && i == 0 && st + 1 < 4) read_sub(st + 1);
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const int ht = s & 1, r = s >> 1;  // MFMA k-step r of head block ht; epilogue head row r
                if (pp < 4 * kPfQPerWave)
                    acc[pp & 1][ht] = mfma16x16x32(qa[i][ht][r], kv[st & 1][r], r == 0 ? zero4 : acc[pp & 1][ht]);
                if (pp > 0) v = fmaf(wv[pi][ht][r], relu(acc[(pp - 1) & 1][ht][r]), s == 0 ? 0.0f : v);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (pp > 0) {
                part[pi] = v;
                if (pi == kPfQPerWave - 1)
                    pf_store<decltype(masked)::value>(out, j * kPfTileKeys + 16 * pst, sum_lane_groups(part));
            }
        }
        store_tile(kP ^ 1);
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    });
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
    TopkPrep prep) {
    __shared__ __attribute__((aligned(16))) uint8_t stage[2 * kPf8TileBytes];
    const int kb_i = blockIdx.x % nkb;
    const int qg = (blockIdx.x / nkb) % nqg;
    const int b = blockIdx.x / (nkb * nqg);
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int c = lane & 15;
    const int g = lane >> 4;
    const int t0 = qg * kPfQueries + kPfQPerWave * wave;

    if (prep.base && kb_i == 0)
        for (int i = threadIdx.x; i < kPfQueries * prep.zero_count; i += 256) {
            const int t = qg * kPfQueries + i / prep.zero_count;
            if (t < T) prep.base[((int64_t)b * T + t) * prep.stride + prep.zero_off + i % prep.zero_count] = 0u;
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
    const int64_t key0 = (int64_t)kb_i * kPfKeysPerBlock;
    const PfOut out = pf_out(scores, q_pos, b, T, L, qg, wave, g, c, key0);

    const int64_t kblk_end = min((int64_t)L, key0 + kPfKeysPerBlock);
    const int64_t kvis_end = min(kblk_end, max(key0, group_max_pos(q_pos, b, T, qg) + 1));
    const int ntiles = (int)((kvis_end - key0 + kPf8TileKeys - 1) / kPf8TileKeys);
    const int64_t kall_end = min(kblk_end, max(key0, group_min_pos(q_pos, b, T, qg) + 1));  // seen by all
    const int nfull = (int)((kall_end - key0) / kPf8TileKeys);
    fill_masked(wt_rsrc(scores + ((int64_t)b * T + qg * kPfQueries) * L), qg, T, L,
                key0 + (int64_t)ntiles * kPf8TileKeys, kblk_end);
    if (ntiles == 0) return;
    // tile loads: thread i brings 16-byte chunks i and i + 256 (key = chunk / 8, s = chunk % 8);
    // keys past L read zeros (their scores are never stored), so the tile after the last is safe
    const __amdgpu_buffer_rsrc_t krs = sized_rsrc(k_idx + (int64_t)b * k_bstride, (uint32_t)L * kD8);
    const uint32_t ld_off = (uint32_t)key0 * kD8 + 16u * threadIdx.x;
    u32x4_t ld[2];
    auto load_tile = [&](int j) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
            ld[h] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                    krs, (int)(ld_off + (uint32_t)j * kPf8TileBytes + h * 4096), 0, 0));
    };
    auto store_tile = [&](int parity) {
        uint8_t* tile = stage + parity * kPf8TileBytes;
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
    pf_tile_runs(ntiles, nfull, [&](int j, auto masked, auto parity) {
        constexpr int kP = decltype(parity)::value;
        load_tile(j + 1);  // in flight while tile j is computed
        const uint8_t* tile = stage + kP * kPf8TileBytes;
        i32x8_t kv[2];  // B operands of sub-tile st + 1 are read while sub-tile st is computed
        auto read_sub = [&](int st) {
            const int k = 16 * st + c;  // key of this lane's B column
            const int f = (k >> 1) & 7;
            const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(tile + 16 * (8 * k + ((2 * g) ^ f)));
            const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(tile + 16 * (8 * k + ((2 * g + 1) ^ f)));
            kv[st & 1] = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        // (sub-tile, query) pairs as a pipeline, as in the bf16 kernel: pair
        // p's two MFMAs issue among the 16 epilogue instructions of pair p - 1.
        const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
        f32x4_t acc[2][2];  // [pair parity][head block]
        float part[kPfQPerWave];
        float v = 0.0f;
        read_sub(0);
#pragma unroll
        for (int pp = 0; pp <= 4 * kPfQPerWave; ++pp) {
            const int st = pp / kPfQPerWave, i = pp % kPfQPerWave;                 // pair pp (pp < 16)
            const int pst = (pp - 1) / kPfQPerWave, pi = (pp - 1) % kPfQPerWave;   // pair pp - 1 (pp > 0)
            if (pp < 4 * kPfQPerWave && i == 0 && st + 1 < 4) read_sub(st + 1);
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const int ht = s & 1, r = s >> 1;  // epilogue head row r of head block ht
                if (pp < 4 * kPfQPerWave && (s & 3) == 0)
                    acc[pp & 1][s >> 2] = mfma16x16x128_fp8(qa[i][s >> 2], kv[st & 1], zero4);
                if (pp > 0) v = fmaf(wv[pi][ht][r], relu(acc[(pp - 1) & 1][ht][r]), s == 0 ? 0.0f : v);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (pp > 0) {
                part[pi] = v;
                if (pi == kPfQPerWave - 1)
                    pf_store<decltype(masked)::value>(out, j * kPf8TileKeys + 16 * pst, sum_lane_groups(part));
            }
        }
        store_tile(kP ^ 1);
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    });
}
}  // namespace

bool indexer_counts_histogram(int T) { return T < kPrefillMinQueries; }

int64_t indexer_grid_blocks(int B, int T, int L, bool fp8) {
    if (T >= kPrefillMinQueries)
        return (int64_t)B * ((T + kPfQueries - 1) / kPfQueries) * ((L + kPfKeysPerBlock - 1) / kPfKeysPerBlock);
    const int keys_per_block = fp8 ? kDecode8Waves * kTile8 * kDecode8Tiles : kDecodeWaves * kTile * kDecodeTiles;
    return (int64_t)B * T * ((L + keys_per_block - 1) / keys_per_block);
}

// Resident workgroups per CU of a kernel at this block size (looked up once per device and kernel).
template <typename K>
int resident_per_cu(K kernel, int threads, std::atomic<int>* cache) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess || n < 1) n = 1;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

int device_cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Workgroups per row and blocks per workgroup: all of the rows' workgroups
// resident at once when there are few rows (at most max_per blocks each), one
// block each when there are many.
struct DecodeGrid {
    int wpr, per;
};
DecodeGrid decode_grid(int rows, int nblk, int64_t slots, int max_per) {
    int wpr = nblk;
    if (slots > 0 && 2 * (int64_t)rows <= slots) wpr = (int)std::min<int64_t>(nblk, slots / rows);
    wpr = std::max(wpr, (nblk + max_per - 1) / max_per);
    const int per = (nblk + wpr - 1) / wpr;
    return DecodeGrid{(nblk + per - 1) / per, per};
}

hipError_t launch_indexer_decode(const uint16_t* q_idx, const float* w, const uint16_t* k_idx, int64_t k_bstride,
                                 const int32_t* q_pos, int B, int T, int L, float* scores, hipStream_t stream,
                                 TopkPrep prep) {
    constexpr int W = kDecodeWaves;
    constexpr int keys_per_block = W * kTile * kDecodeTiles;
    static std::atomic<int> occ[64];
    const auto kernel = indexer_decode_kernel<W, kAhead>;
    const int rows = B * T;
    const int nblk = (L + keys_per_block - 1) / keys_per_block;
    const int64_t slots = (int64_t)resident_per_cu(kernel, W * kWave, occ) * device_cu_count();
    const DecodeGrid dg = decode_grid(rows, nblk, slots, kDecodeMaxPer);
    hipLaunchKernelGGL(kernel, dim3((unsigned)((int64_t)rows * dg.wpr)), dim3(W * kWave), 0, stream, q_idx, w, k_idx,
                       k_bstride, q_pos, T, L, nblk, dg.wpr, dg.per, scores, prep);
    return hipGetLastError();
}

hipError_t launch_indexer_decode_fp8(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, int64_t k_bstride,
                                     const int32_t* q_pos, int B, int T, int L, float* scores, hipStream_t stream,
                                     TopkPrep prep) {
    constexpr int W = kDecode8Waves;
    constexpr int keys_per_block = W * kTile8 * kDecode8Tiles;
    static std::atomic<int> occ[64];
    const auto kernel = indexer_decode_fp8_kernel<W, kDecode8Ahead>;
    const int rows = B * T;
    const int nblk = (L + keys_per_block - 1) / keys_per_block;
    const int64_t slots = (int64_t)resident_per_cu(kernel, W * kWave, occ) * device_cu_count();
    const DecodeGrid dg = decode_grid(rows, nblk, slots, kDecode8MaxPer);
    hipLaunchKernelGGL(kernel, dim3((unsigned)((int64_t)rows * dg.wpr)), dim3(W * kWave), 0, stream, q_idx, w, k_idx,
                       k_bstride, q_pos, T, L, nblk, dg.wpr, dg.per, scores, prep);
    return hipGetLastError();
}

hipError_t launch_indexer_fp8(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, int64_t k_bstride,
                              const int32_t* q_pos, int B, int T, int L, float* scores, hipStream_t stream,
                              TopkPrep prep) {
    if (T >= kPrefillMinQueries) {
        const int nqg = (T + kPfQueries - 1) / kPfQueries;
        const int nkb = (L + kPfKeysPerBlock - 1) / kPfKeysPerBlock;
        hipLaunchKernelGGL(indexer_prefill_fp8_kernel, dim3((unsigned)((int64_t)B * nqg * nkb)), dim3(256), 0, stream,
                           q_idx, w, k_idx, k_bstride, q_pos, T, L, nqg, nkb, scores, prep);
        return hipGetLastError();
    }
    return launch_indexer_decode_fp8(q_idx, w, k_idx, k_bstride, q_pos, B, T, L, scores, stream, prep);
}

hipError_t launch_indexer(const uint16_t* q_idx, const float* w, const uint16_t* k_idx, int64_t k_bstride,
                          const int32_t* q_pos, int B, int T, int L, float* scores, hipStream_t stream,
                          TopkPrep prep) {
    if (T >= kPrefillMinQueries) {
        const int nqg = (T + kPfQueries - 1) / kPfQueries;
        const int nkb = (L + kPfKeysPerBlock - 1) / kPfKeysPerBlock;
        hipLaunchKernelGGL(indexer_prefill_kernel, dim3((unsigned)((int64_t)B * nqg * nkb)), dim3(256), 0, stream,
                           q_idx, w, k_idx, k_bstride, q_pos, T, L, nqg, nkb, scores, prep);
        return hipGetLastError();
    }
    return launch_indexer_decode(q_idx, w, k_idx, k_bstride, q_pos, B, T, L, scores, stream, prep);
}

}  // namespace dsa
