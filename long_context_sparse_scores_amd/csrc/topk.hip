// Exact top-k selection on gfx950: radix select over order-preserving keys.
//
// [TEARDOWN, 刀一 DSA] (clawlihai.cn GLM-5.2 1M architecture teardown):
// index_topk 2048 — each query keeps the 2048 best-scoring visible tokens.
// Candidates are s in [0, p]; ties at the threshold go to the lower
// position; the kept positions are written in ascending order, -1 padded.
//
// Scores become uint32 keys whose unsigned order is the float order.  The
// k-th largest key K* is found digit by digit (11 + 11 + 10 bits, most
// significant first).  Each row is cut into slices (a few hundred workgroups
// over all rows, so a few long rows still fill the chip); a slice is cut
// into one contiguous range per wave.  Five launches:
//   init    zero the row's two global histograms and counters;
//   hist    histogram of the top digit (LDS per slice, non-zero bins added
//           to the row's histogram);
//   filter  every slice finds the threshold digit T from that histogram,
//           counts per wave the keys whose top digit is above T, and appends
//           the keys whose top digit equals T to the row's candidate list,
//           histogramming their middle digit;
//   resolve one workgroup per row: the low digits of K* and the number of
//           keys equal to K* still to take, from the candidates; counts per
//           wave of the candidates above / equal to K*;
//   write   each wave turns the counts of the waves before it into an output
//           offset and writes its selected positions in order (ballot ranks):
//           every key above K*, and keys equal to K* while their rank in
//           position order is below the number still to take.
// The score rows are re-read from L2 / the last-level cache by each pass.
// When a row's candidate list overflows its capacity (heavily tied scores),
// resolve reads the whole row instead; the result is the same.
#include "common.h"

namespace dsa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kBins = 2048;
constexpr int kTargetBlocks = 512;   // slices over all rows
constexpr int kMinSlice = 4096;
constexpr int kMaxUnits = 2048;      // waves (slice x 4) per row
constexpr int kStage = 256;          // per-wave LDS staging of candidates
constexpr int kBatch = 16;           // loads in flight per lane in the streaming passes

// Per-row workspace (32-bit words).
enum : int { kCtrCand = 0, kStKey = 2, kStTakeEq = 3, kCtrWords = 8 };

struct Layout {
    int slice;    // elements per slice (multiple of 256)
    int nslice;   // slices per row
    int cap;      // candidate capacity per row
    __host__ __device__ int units() const { return nslice * kWaves; }
    __host__ __device__ int wave_len() const { return slice / kWaves; }
    __host__ __device__ size_t row_words() const { return 2 * kBins + kCtrWords + 3 * (size_t)units() + 2 * (size_t)cap; }
};

struct RowWs {
    uint32_t* hist1;   // [kBins] top digit
    uint32_t* hist2;   // [kBins] middle digit of the candidates
    uint32_t* ctr;     // [kCtrWords]
    uint32_t* gt_hi;   // [units] keys with top digit > T, per wave
    uint32_t* gt_c;    // [units] candidates > K*, per wave
    uint32_t* eq_c;    // [units] candidates == K*, per wave
    uint32_t* cpos;    // [cap] candidate positions
    uint32_t* ckey;    // [cap] candidate keys
};

__device__ __forceinline__ RowWs row_ws(void* ws, int row, const Layout& lo) {
    uint32_t* b = reinterpret_cast<uint32_t*>(ws) + (size_t)row * lo.row_words();
    RowWs r;
    r.hist1 = b;
    r.hist2 = b + kBins;
    r.ctr = b + 2 * kBins;
    r.gt_hi = r.ctr + kCtrWords;
    r.gt_c = r.gt_hi + lo.units();
    r.eq_c = r.gt_c + lo.units();
    r.cpos = r.eq_c + lo.units();
    r.ckey = r.cpos + lo.cap;
    return r;
}

__device__ __forceinline__ int64_t n_visible(const int32_t* q_pos, int row, int L) {
    int64_t p = q_pos[row];
    if (p < 0) return 0;
    return (p < L - 1 ? p : (int64_t)L - 1) + 1;
}

// Rank of this lane among the set lanes of `mask` below it.
__device__ __forceinline__ uint32_t lane_rank(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Find the bin holding the `need`-th largest element of a histogram of `nbins`
// (<= 2048) bins, 1 <= need <= total.  Returns the bin and the count of
// elements in higher bins.  All threads of the block must call it.
struct BinPick {
    uint32_t bin, above;
};

__device__ BinPick pick_bin(const uint32_t* hist, int nbins, uint32_t need, uint32_t* scan_scratch,
                            BinPick* result) {
    constexpr int per = kBins / kThreads;  // 8 bins per thread, upper bins first (suffix scan)
    const int t = threadIdx.x;
    uint32_t h[per];
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < per; ++i) {
        const int bin = nbins - 1 - (per * t + i);
        h[i] = bin >= 0 ? hist[bin] : 0u;
        s += h[i];
    }
    if (t == 0) *result = BinPick{0u, 0u};
    uint32_t total;
    const uint32_t above = block_excl_scan<kWaves>(s, scan_scratch, &total);
    if (above < need && need <= above + s) {
        uint32_t acc = above;
#pragma unroll
        for (int i = 0; i < per; ++i) {
            if (acc + h[i] >= need) {
                result->bin = (uint32_t)(nbins - 1 - (per * t + i));
                result->above = acc;
                break;
            }
            acc += h[i];
        }
    }
    __syncthreads();
    const BinPick r = *result;
    __syncthreads();
    return r;
}

__global__ __launch_bounds__(kThreads) void topk_init_kernel(void* ws, Layout lo) {
    RowWs rw = row_ws(ws, blockIdx.x, lo);
    for (int i = threadIdx.x; i < 2 * kBins + kCtrWords; i += kThreads) rw.hist1[i] = 0u;  // hist1, hist2, ctr
}

__global__ __launch_bounds__(kThreads) void topk_hist_kernel(const float* __restrict__ scores,
                                                             const int32_t* __restrict__ q_pos, int L, int k,
                                                             Layout lo, void* ws) {
    const int row = blockIdx.x / lo.nslice;
    const int slice = blockIdx.x % lo.nslice;
    const int64_t n = n_visible(q_pos, row, L);
    const int64_t start = (int64_t)slice * lo.slice;
    if (n <= k || start >= n) return;
    __shared__ uint32_t h[kBins];
    for (int i = threadIdx.x; i < kBins; i += kThreads) h[i] = 0u;
    __syncthreads();
    const float* src = scores + (int64_t)row * L + start;
    const int m = (int)((n - start) < lo.slice ? (n - start) : lo.slice);
    for (int i0 = 0; i0 < m; i0 += kBatch * kThreads) {
        float v[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int i = i0 + j * kThreads + threadIdx.x;
            v[j] = i < m ? src[i] : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j)
            if (i0 + j * kThreads + (int)threadIdx.x < m) atomicAdd(&h[score_key(v[j]) >> 21], 1u);
    }
    __syncthreads();
    uint32_t* g = row_ws(ws, row, lo).hist1;
    for (int i = threadIdx.x; i < kBins; i += kThreads)
        if (h[i]) atomicAdd(&g[i], h[i]);
}

// Resolve K* from the candidates (or, after an overflow, the whole row) and
// count per wave the candidates above / equal to it.
__device__ void resolve_row(const float* __restrict__ row_scores, int64_t n, int k, const Layout& lo, RowWs rw,
                            uint32_t T, uint32_t above_T, int units_used, uint32_t* h3, uint32_t* gtc,
                            uint32_t* eqc, uint32_t* scratch, BinPick* pick) {
    const uint32_t ncand = rw.ctr[kCtrCand];
    const bool from_list = ncand <= (uint32_t)lo.cap;
    const uint32_t need = (uint32_t)k - above_T;
    const BinPick b1 = pick_bin(rw.hist2, kBins, need, scratch, pick);
    const uint32_t need1 = need - b1.above;
    const uint32_t prefix = (T << 11) | b1.bin;  // top 22 bits of K*
    for (int i = threadIdx.x; i < 1024; i += kThreads) h3[i] = 0u;
    for (int i = threadIdx.x; i < kMaxUnits; i += kThreads) gtc[i] = eqc[i] = 0u;
    __syncthreads();
    // visit every key of the row whose top digit is T: f(key, position)
    auto for_candidates = [&](auto&& f) {
        constexpr int kB = 8;  // loads in flight per thread
        if (from_list) {
            for (uint32_t i0 = 0; i0 < ncand; i0 += kB * kThreads) {
                uint32_t kk[kB], pp[kB];
#pragma unroll
                for (int j = 0; j < kB; ++j) {
                    const uint32_t i = i0 + j * kThreads + threadIdx.x;
                    kk[j] = i < ncand ? rw.ckey[i] : 0u;
                    pp[j] = i < ncand ? rw.cpos[i] : 0u;
                }
#pragma unroll
                for (int j = 0; j < kB; ++j)
                    if (i0 + j * kThreads + threadIdx.x < ncand) f(kk[j], pp[j]);
            }
        } else {
            for (int64_t i0 = 0; i0 < n; i0 += kB * kThreads) {
                float v[kB];
#pragma unroll
                for (int j = 0; j < kB; ++j) {
                    const int64_t i = i0 + j * kThreads + threadIdx.x;
                    v[j] = i < n ? row_scores[i] : 0.0f;
                }
#pragma unroll
                for (int j = 0; j < kB; ++j) {
                    const int64_t i = i0 + j * kThreads + threadIdx.x;
                    const uint32_t key = score_key(v[j]);
                    if (i < n && (key >> 21) == T) f(key, (uint32_t)i);
                }
            }
        }
    };
    for_candidates([&](uint32_t key, uint32_t) {
        if ((key >> 10) == prefix) atomicAdd(&h3[key & 0x3FFu], 1u);
    });
    __syncthreads();
    const BinPick b2 = pick_bin(h3, 1024, need1, scratch, pick);
    const uint32_t kstar = (prefix << 10) | b2.bin;
    const uint32_t take_eq = need1 - b2.above;
    const uint32_t wl = (uint32_t)lo.wave_len();
    for_candidates([&](uint32_t key, uint32_t pos) {
        if (key > kstar) atomicAdd(&gtc[pos / wl], 1u);
        else if (key == kstar) atomicAdd(&eqc[pos / wl], 1u);
    });
    __syncthreads();
    for (int u = threadIdx.x; u < units_used; u += kThreads) {
        rw.gt_c[u] = gtc[u];
        rw.eq_c[u] = eqc[u];
    }
    if (threadIdx.x == 0) {
        rw.ctr[kStKey] = kstar;
        rw.ctr[kStTakeEq] = take_eq;
    }
}

__global__ __launch_bounds__(kThreads) void topk_filter_kernel(const float* __restrict__ scores,
                                                               const int32_t* __restrict__ q_pos, int L, int k,
                                                               Layout lo, void* ws) {
    const int row = blockIdx.x / lo.nslice;
    const int slice = blockIdx.x % lo.nslice;
    const int64_t n = n_visible(q_pos, row, L);
    const int64_t start = (int64_t)slice * lo.slice;
    if (n <= k || start >= n) return;
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    RowWs rw = row_ws(ws, row, lo);

    __shared__ uint32_t h2[kBins];
    __shared__ uint32_t stage_pos[kWaves][kStage], stage_key[kWaves][kStage];
    __shared__ uint32_t scratch[kWaves];
    __shared__ BinPick pick;

    const BinPick b0 = pick_bin(rw.hist1, kBins, (uint32_t)k, scratch, &pick);
    const uint32_t T = b0.bin;
    for (int i = threadIdx.x; i < kBins; i += kThreads) h2[i] = 0u;
    __syncthreads();

    // this wave's range of the slice
    const int64_t w0 = start + (int64_t)wave * lo.wave_len();
    const int64_t w1 = min(w0 + lo.wave_len(), n);
    const float* row_scores = scores + (int64_t)row * L;
    uint32_t gt = 0;
    // Candidates are staged per wave in LDS and appended to the row's list in
    // batches: one global atomic per batch rather than per 64 keys.
    uint32_t staged = 0;  // wave-uniform
    uint32_t* sp = stage_pos[wave];
    uint32_t* sk = stage_key[wave];
    auto flush = [&]() {
        __builtin_amdgcn_wave_barrier();
        uint32_t base = 0;
        if (lane == 0) base = atomicAdd(&rw.ctr[kCtrCand], staged);
        base = __shfl(base, 0, kWave);
        for (uint32_t j = lane; j < staged; j += kWave) {
            const uint32_t slot = base + j;
            if (slot < (uint32_t)lo.cap) {
                rw.cpos[slot] = sp[j];
                rw.ckey[slot] = sk[j];
            }
        }
        __builtin_amdgcn_wave_barrier();
        staged = 0;
    };
    for (int64_t i0 = w0; i0 < w1; i0 += kBatch * kWave) {
        float v[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int64_t i = i0 + j * kWave + lane;
            v[j] = i < w1 ? row_scores[i] : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int64_t i = i0 + j * kWave + lane;
            const bool valid = i < w1;
            const uint32_t key = score_key(v[j]);
            const uint32_t top = key >> 21;
            gt += (valid && top > T) ? 1u : 0u;
            const bool cand = valid && top == T;
            const uint64_t m = __ballot(cand);
            if (m) {
                const uint32_t c = (uint32_t)__popcll(m);
                if (staged + c > (uint32_t)kStage) flush();
                if (cand) {
                    atomicAdd(&h2[(key >> 10) & 0x7FFu], 1u);
                    const uint32_t slot = staged + lane_rank(m);
                    sp[slot] = (uint32_t)i;
                    sk[slot] = key;
                }
                staged += c;
            }
        }
    }
    if (staged) flush();
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) gt += __shfl_xor(gt, off, kWave);
    if (lane == 0) rw.gt_hi[slice * kWaves + wave] = gt;
    __syncthreads();
    for (int i = threadIdx.x; i < kBins; i += kThreads)
        if (h2[i]) atomicAdd(&rw.hist2[i], h2[i]);
}

// One workgroup per row: the exact threshold key from the candidates.
__global__ __launch_bounds__(kThreads) void topk_resolve_kernel(const float* __restrict__ scores,
                                                                const int32_t* __restrict__ q_pos, int L, int k,
                                                                Layout lo, void* ws) {
    const int row = blockIdx.x;
    const int64_t n = n_visible(q_pos, row, L);
    if (n <= k) return;
    const int slices_used = (int)((n + lo.slice - 1) / lo.slice);
    RowWs rw = row_ws(ws, row, lo);
    __shared__ uint32_t h3[1024];
    __shared__ uint32_t gtc[kMaxUnits], eqc[kMaxUnits];
    __shared__ uint32_t scratch[kWaves];
    __shared__ BinPick pick;
    const BinPick b0 = pick_bin(rw.hist1, kBins, (uint32_t)k, scratch, &pick);
    resolve_row(scores + (int64_t)row * L, n, k, lo, rw, b0.bin, b0.above, slices_used * kWaves, h3, gtc, eqc,
                scratch, &pick);
}

__global__ __launch_bounds__(kThreads) void topk_write_kernel(const float* __restrict__ scores,
                                                              const int32_t* __restrict__ q_pos, int L, int k,
                                                              Layout lo, void* ws, int32_t* __restrict__ idx) {
    const int row = blockIdx.x / lo.nslice;
    const int slice = blockIdx.x % lo.nslice;
    const int64_t n = n_visible(q_pos, row, L);
    int32_t* out = idx + (int64_t)row * k;
    if (n <= k) {  // every visible position, in order, then -1
        if (slice == 0)
            for (int j = threadIdx.x; j < k; j += kThreads) out[j] = j < n ? j : -1;
        return;
    }
    const int64_t start = (int64_t)slice * lo.slice;
    if (start >= n) return;
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    RowWs rw = row_ws(ws, row, lo);
    const uint32_t kstar = rw.ctr[kStKey];
    const uint32_t take_eq = rw.ctr[kStTakeEq];
    // selected keys and equal keys in the waves before this one
    const int u = slice * kWaves + wave;
    uint32_t gt_b = 0, eq_b = 0;
    for (int v = lane; v < u; v += kWave) {
        gt_b += rw.gt_hi[v] + rw.gt_c[v];
        eq_b += rw.eq_c[v];
    }
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) {
        gt_b += __shfl_xor(gt_b, off, kWave);
        eq_b += __shfl_xor(eq_b, off, kWave);
    }
    uint32_t pos = gt_b + (eq_b < take_eq ? eq_b : take_eq);
    uint32_t eq_seen = eq_b;
    const int64_t w0 = start + (int64_t)wave * lo.wave_len();
    const int64_t w1 = min(w0 + lo.wave_len(), n);
    const float* row_scores = scores + (int64_t)row * L;
    for (int64_t i0 = w0; i0 < w1; i0 += kBatch * kWave) {
        float v[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int64_t i = i0 + j * kWave + lane;
            v[j] = i < w1 ? row_scores[i] : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int64_t i = i0 + j * kWave + lane;
            const bool valid = i < w1;
            const uint32_t key = score_key(v[j]);
            const bool eq = valid && key == kstar;
            const uint64_t meq = __ballot(eq);
            const bool sel = valid && (key > kstar || (eq && eq_seen + lane_rank(meq) < take_eq));
            const uint64_t msel = __ballot(sel);
            if (sel) {
                const uint32_t o = pos + lane_rank(msel);
                if (o < (uint32_t)k) out[o] = (int32_t)i;
            }
            pos += (uint32_t)__popcll(msel);
            eq_seen += (uint32_t)__popcll(meq);
        }
    }
}

Layout make_layout(int rows, int L) {
    const int max_slices = (L + kMinSlice - 1) / kMinSlice;
    int ns = (kTargetBlocks + rows - 1) / rows;
    if (ns > max_slices) ns = max_slices;
    if (ns > kMaxUnits / kWaves) ns = kMaxUnits / kWaves;
    if (ns < 1) ns = 1;
    int64_t slice = ((int64_t)L + ns - 1) / ns;
    slice = (slice + 255) / 256 * 256;
    Layout lo;
    lo.slice = (int)slice;
    lo.nslice = (int)(((int64_t)L + slice - 1) / slice);
    int64_t cap = (int64_t)L / 8;
    if (cap < 4096) cap = 4096;
    lo.cap = (int)((cap + 63) / 64 * 64);
    return lo;
}

}  // namespace

size_t topk_ws_bytes(int rows, int L, int k) {
    (void)k;
    return align_up((size_t)rows * make_layout(rows, L).row_words() * sizeof(uint32_t), 256);
}

hipError_t launch_topk(const float* scores, const int32_t* q_pos, int rows, int L, int k, int32_t* idx, void* ws,
                       hipStream_t stream) {
    const Layout lo = make_layout(rows, L);
    const unsigned grid = (unsigned)((int64_t)rows * lo.nslice);
    hipLaunchKernelGGL(topk_init_kernel, dim3(rows), dim3(kThreads), 0, stream, ws, lo);
    hipLaunchKernelGGL(topk_hist_kernel, dim3(grid), dim3(kThreads), 0, stream, scores, q_pos, L, k, lo, ws);
    hipLaunchKernelGGL(topk_filter_kernel, dim3(grid), dim3(kThreads), 0, stream, scores, q_pos, L, k, lo, ws);
    hipLaunchKernelGGL(topk_resolve_kernel, dim3(rows), dim3(kThreads), 0, stream, scores, q_pos, L, k, lo, ws);
    hipLaunchKernelGGL(topk_write_kernel, dim3(grid), dim3(kThreads), 0, stream, scores, q_pos, L, k, lo, ws, idx);
    return hipGetLastError();
}

}  // namespace dsa
