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
//   init    zero the row's global histogram and counters;
//   hist    histogram of the top digit (LDS per slice, non-zero bins added
//           to the row's histogram);
//   filter  every slice finds the threshold digit T from that histogram,
//           counts per wave the keys whose top digit is above T, and appends
//           the keys whose top digit equals T to the row's candidate list;
//   resolve one workgroup per row: the middle and low digits of K* and the
//           number of keys equal to K* still to take, from the candidates
//           (LDS histograms); per wave, the
//           number of selected keys and of keys equal to K* before it;
//   write   each wave writes its selected positions in order (ballot ranks)
//           from its output offset: every key above K*, and keys equal to K*
//           while their rank in position order is below the number to take.
// Each pass issues its score loads before it reads the row's histograms and
// counters, and synchronises through LDS only, so the two latencies overlap.
// The score rows are re-read from L2 / the last-level cache by each pass.
// When a row's candidate list overflows its capacity (heavily tied scores),
// resolve reads the whole row instead; the result is the same.
#include "common.h"

namespace dsa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kResolveThreads = 1024;
constexpr int kBins = 2048;
constexpr int kTargetBlocks = 512;   // slices over all rows
constexpr int kMinSlice = 4096;
constexpr int kMaxUnits = 2048;      // waves (slice x 4) per row
constexpr int kStage = 256;          // per-wave LDS staging of candidates
constexpr int kBatch = 32;           // loads in flight per lane in the streaming passes
constexpr int kCandRegs = 8;         // candidates per resolve thread kept in registers

// Per-row workspace (32-bit words).
enum : int { kCtrCand = 0, kStKey = 2, kStTakeEq = 3, kCtrWords = 8 };

struct Layout {
    int slice;    // elements per slice (multiple of 256)
    int nslice;   // slices per row
    int cap;      // candidate capacity per row
    __host__ __device__ int units() const { return nslice * kWaves; }
    __host__ __device__ int wave_len() const { return slice / kWaves; }
    __host__ __device__ size_t row_words() const { return kBins + kCtrWords + 3 * (size_t)units() + 2 * (size_t)cap; }
};

struct RowWs {
    uint32_t* hist1;   // [kBins] top digit
    uint32_t* ctr;     // [kCtrWords]
    uint32_t* gt_hi;   // [units] keys with top digit > T, per wave
    uint32_t* sel_b;   // [units] selected keys in the waves before (written by resolve)
    uint32_t* eq_b;    // [units] keys == K* in the waves before (written by resolve)
    uint32_t* cpos;    // [cap] candidate positions
    uint32_t* ckey;    // [cap] candidate keys
};

__device__ __forceinline__ RowWs row_ws(void* ws, int row, const Layout& lo) {
    uint32_t* b = reinterpret_cast<uint32_t*>(ws) + (size_t)row * lo.row_words();
    RowWs r;
    r.hist1 = b;
    r.ctr = b + kBins;
    r.gt_hi = r.ctr + kCtrWords;
    r.sel_b = r.gt_hi + lo.units();
    r.eq_b = r.sel_b + lo.units();
    r.cpos = r.eq_b + lo.units();
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

// Workgroup barrier for LDS hand-offs that leaves outstanding global loads in
// flight (__syncthreads would wait for them as well).
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Exclusive prefix sum over a workgroup of NT threads; `scratch` holds NT/64 words of LDS.
template <int NT>
__device__ __forceinline__ uint32_t excl_scan(uint32_t x, uint32_t* scratch, uint32_t* total) {
    constexpr int NW = NT / kWave;
    const int w = threadIdx.x / kWave;
    const uint32_t inc = wave_incl_scan(x);
    if (lane_id() == kWave - 1) scratch[w] = inc;
    lds_sync();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const uint32_t v = scratch[i];
        before += (i < w) ? v : 0u;
        tot += v;
    }
    lds_sync();
    *total = tot;
    return before + inc - x;
}

// This thread's bins of a histogram of `nbins` (<= 2048) bins, highest first:
// thread t holds bins nbins-1 - (per*t + i).
template <int NT>
struct HistPart {
    uint32_t h[kBins / NT];
};

template <int NT>
__device__ __forceinline__ HistPart<NT> load_hist(const uint32_t* hist, int nbins) {
    constexpr int per = kBins / NT;
    HistPart<NT> hp;
#pragma unroll
    for (int i = 0; i < per; ++i) {
        const int bin = nbins - 1 - (per * (int)threadIdx.x + i);
        hp.h[i] = bin >= 0 ? hist[bin] : 0u;
    }
    return hp;
}

// The bin holding the `need`-th largest element (1 <= need <= total) and the
// count of elements in higher bins.  All NT threads call it.
struct BinPick {
    uint32_t bin, above;
};

template <int NT>
__device__ BinPick pick_bin(const HistPart<NT>& hp, int nbins, uint32_t need, uint32_t* scratch, BinPick* result) {
    constexpr int per = kBins / NT;
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < per; ++i) s += hp.h[i];
    if (threadIdx.x == 0) *result = BinPick{0u, 0u};
    uint32_t total;
    const uint32_t above = excl_scan<NT>(s, scratch, &total);  // count in higher bins (also orders the reset)
    if (above < need && need <= above + s) {
        uint32_t acc = above;
#pragma unroll
        for (int i = 0; i < per; ++i) {
            if (acc + hp.h[i] >= need) {
                result->bin = (uint32_t)(nbins - 1 - (per * (int)threadIdx.x + i));
                result->above = acc;
                break;
            }
            acc += hp.h[i];
        }
    }
    lds_sync();
    const BinPick r = *result;
    lds_sync();
    return r;
}

__global__ __launch_bounds__(kThreads) void topk_init_kernel(void* ws, Layout lo) {
    RowWs rw = row_ws(ws, blockIdx.x, lo);
    for (int i = threadIdx.x; i < kBins + kCtrWords; i += kThreads) rw.hist1[i] = 0u;  // hist1, ctr
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
    const float* src = scores + (int64_t)row * L + start;
    const int m = (int)((n - start) < lo.slice ? (n - start) : lo.slice);
    lds_sync();
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
    lds_sync();
    uint32_t* g = row_ws(ws, row, lo).hist1;
    for (int i = threadIdx.x; i < kBins; i += kThreads)
        if (h[i]) atomicAdd(&g[i], h[i]);
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

    __shared__ uint32_t stage_pos[kWaves][kStage], stage_key[kWaves][kStage];
    __shared__ uint32_t scratch[kWaves];
    __shared__ BinPick pick;

    // the row's top-digit histogram, then this wave's first batch of scores
    const HistPart<kThreads> hp = load_hist<kThreads>(rw.hist1, kBins);
    const int64_t w0 = start + (int64_t)wave * lo.wave_len();
    const int64_t w1 = min(w0 + lo.wave_len(), n);
    const float* row_scores = scores + (int64_t)row * L;
    float v[kBatch];
    auto load_batch = [&](int64_t i0) {
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int64_t i = i0 + j * kWave + lane;
            v[j] = i < w1 ? row_scores[i] : 0.0f;
        }
    };
    load_batch(w0);
    const BinPick b0 = pick_bin<kThreads>(hp, kBins, (uint32_t)k, scratch, &pick);
    const uint32_t T = b0.bin;

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
        if (i0 != w0) load_batch(i0);
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
}

// One 1024-thread workgroup per row: K* from the candidates (or, after an
// overflow, from the whole row), then per wave of the filter/write passes the
// number of selected keys and of keys equal to K* in the waves before it.
__global__ __launch_bounds__(kResolveThreads) void topk_resolve_kernel(const float* __restrict__ scores,
                                                                       const int32_t* __restrict__ q_pos, int L,
                                                                       int k, Layout lo, void* ws) {
    constexpr int NT = kResolveThreads;
    const int row = blockIdx.x;
    const int64_t n = n_visible(q_pos, row, L);
    if (n <= k) return;
    const int units_used = (int)((n + lo.slice - 1) / lo.slice) * kWaves;
    RowWs rw = row_ws(ws, row, lo);
    const float* row_scores = scores + (int64_t)row * L;
    __shared__ uint32_t h2[kBins];
    __shared__ uint32_t h3[1024];
    __shared__ uint32_t gtc[kMaxUnits], eqc[kMaxUnits];
    __shared__ uint32_t scratch[NT / kWave];
    __shared__ BinPick pick;

    // everything this kernel reads, issued together
    const HistPart<NT> hp1 = load_hist<NT>(rw.hist1, kBins);
    const uint32_t ncand = rw.ctr[kCtrCand];
    uint32_t kk[kCandRegs], pp[kCandRegs];
    const uint32_t reg_cap = (uint32_t)min(lo.cap, kCandRegs * NT);
#pragma unroll
    for (int j = 0; j < kCandRegs; ++j) {
        const uint32_t i = j * NT + threadIdx.x;
        kk[j] = i < reg_cap ? rw.ckey[i] : 0u;
        pp[j] = i < reg_cap ? rw.cpos[i] : 0u;
    }
    uint32_t gh[kMaxUnits / NT];
#pragma unroll
    for (int j = 0; j < kMaxUnits / NT; ++j) {
        const int u = (kMaxUnits / NT) * threadIdx.x + j;
        gh[j] = u < units_used ? rw.gt_hi[u] : 0u;
    }
    for (int i = threadIdx.x; i < kBins; i += NT) h2[i] = 0u;
    for (int i = threadIdx.x; i < 1024; i += NT) h3[i] = 0u;
    for (int i = threadIdx.x; i < kMaxUnits; i += NT) gtc[i] = eqc[i] = 0u;

    const BinPick b0 = pick_bin<NT>(hp1, kBins, (uint32_t)k, scratch, &pick);  // also orders the resets
    const uint32_t T = b0.bin;
    const uint32_t need = (uint32_t)k - b0.above;
    const bool in_regs = ncand <= reg_cap;
    const bool from_list = ncand <= (uint32_t)lo.cap;
    // visit every key of the row whose top digit is T: f(key, position)
    auto for_candidates = [&](auto&& f) {
        if (in_regs) {
#pragma unroll
            for (int j = 0; j < kCandRegs; ++j)
                if (j * NT + threadIdx.x < ncand) f(kk[j], pp[j]);
        } else if (from_list) {
            for (uint32_t i0 = 0; i0 < ncand; i0 += kCandRegs * NT) {
                uint32_t ck[kCandRegs], cp[kCandRegs];
#pragma unroll
                for (int j = 0; j < kCandRegs; ++j) {
                    const uint32_t i = i0 + j * NT + threadIdx.x;
                    ck[j] = i < ncand ? rw.ckey[i] : 0u;
                    cp[j] = i < ncand ? rw.cpos[i] : 0u;
                }
#pragma unroll
                for (int j = 0; j < kCandRegs; ++j)
                    if (i0 + j * NT + threadIdx.x < ncand) f(ck[j], cp[j]);
            }
        } else {
            for (int64_t i0 = 0; i0 < n; i0 += kCandRegs * NT) {
                float sv[kCandRegs];
#pragma unroll
                for (int j = 0; j < kCandRegs; ++j) {
                    const int64_t i = i0 + j * NT + threadIdx.x;
                    sv[j] = i < n ? row_scores[i] : 0.0f;
                }
#pragma unroll
                for (int j = 0; j < kCandRegs; ++j) {
                    const int64_t i = i0 + j * NT + threadIdx.x;
                    const uint32_t key = score_key(sv[j]);
                    if (i < n && (key >> 21) == T) f(key, (uint32_t)i);
                }
            }
        }
    };
    for_candidates([&](uint32_t key, uint32_t) { atomicAdd(&h2[(key >> 10) & 0x7FFu], 1u); });
    lds_sync();
    const HistPart<NT> hp2 = load_hist<NT>(h2, kBins);
    const BinPick b1 = pick_bin<NT>(hp2, kBins, need, scratch, &pick);
    const uint32_t need1 = need - b1.above;
    const uint32_t prefix = (T << 11) | b1.bin;  // top 22 bits of K*
    for_candidates([&](uint32_t key, uint32_t) {
        if ((key >> 10) == prefix) atomicAdd(&h3[key & 0x3FFu], 1u);
    });
    lds_sync();
    const HistPart<NT> hp3 = load_hist<NT>(h3, 1024);
    const BinPick b2 = pick_bin<NT>(hp3, 1024, need1, scratch, &pick);
    const uint32_t kstar = (prefix << 10) | b2.bin;
    const uint32_t take_eq = need1 - b2.above;
    const uint32_t wl = (uint32_t)lo.wave_len();
    for_candidates([&](uint32_t key, uint32_t pos) {
        if (key > kstar) atomicAdd(&gtc[pos / wl], 1u);
        else if (key == kstar) atomicAdd(&eqc[pos / wl], 1u);
    });
    lds_sync();
    // per wave (unit): selected keys and keys equal to K* in the units before it
    constexpr int kPer = kMaxUnits / NT;
    uint32_t sel[kPer], eq[kPer], ssum = 0, esum = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int u = kPer * threadIdx.x + j;
        sel[j] = u < units_used ? gh[j] + gtc[u] : 0u;
        eq[j] = u < units_used ? eqc[u] : 0u;
        ssum += sel[j];
        esum += eq[j];
    }
    uint32_t tot;
    uint32_t sb = excl_scan<NT>(ssum, scratch, &tot);
    uint32_t eb = excl_scan<NT>(esum, scratch, &tot);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int u = kPer * threadIdx.x + j;
        if (u < units_used) {
            rw.sel_b[u] = sb;
            rw.eq_b[u] = eb;
        }
        sb += sel[j];
        eb += eq[j];
    }
    if (threadIdx.x == 0) {
        rw.ctr[kStKey] = kstar;
        rw.ctr[kStTakeEq] = take_eq;
    }
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
    const int u = slice * kWaves + wave;
    const uint32_t kstar = rw.ctr[kStKey];
    const uint32_t take_eq = rw.ctr[kStTakeEq];
    const uint32_t sel_b = rw.sel_b[u];
    const uint32_t eq_b = rw.eq_b[u];
    const int64_t w0 = start + (int64_t)wave * lo.wave_len();
    const int64_t w1 = min(w0 + lo.wave_len(), n);
    const float* row_scores = scores + (int64_t)row * L;
    uint32_t pos = sel_b + (eq_b < take_eq ? eq_b : take_eq);
    uint32_t eq_seen = eq_b;
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

ZeroRange topk_state_range(void* ws, int rows, int L) {
    (void)rows;
    const Layout lo = make_layout(rows, L);
    ZeroRange z;
    z.base = reinterpret_cast<uint32_t*>(ws);  // each row's words start with hist1, then the counters
    z.stride = (int64_t)lo.row_words();
    z.count = kBins + kCtrWords;
    return z;
}

hipError_t launch_topk(const float* scores, const int32_t* q_pos, int rows, int L, int k, int32_t* idx, void* ws,
                       hipStream_t stream, bool state_zeroed) {
    const Layout lo = make_layout(rows, L);
    const unsigned grid = (unsigned)((int64_t)rows * lo.nslice);
    if (!state_zeroed) hipLaunchKernelGGL(topk_init_kernel, dim3(rows), dim3(kThreads), 0, stream, ws, lo);
    hipLaunchKernelGGL(topk_hist_kernel, dim3(grid), dim3(kThreads), 0, stream, scores, q_pos, L, k, lo, ws);
    hipLaunchKernelGGL(topk_filter_kernel, dim3(grid), dim3(kThreads), 0, stream, scores, q_pos, L, k, lo, ws);
    hipLaunchKernelGGL(topk_resolve_kernel, dim3(rows), dim3(kResolveThreads), 0, stream, scores, q_pos, L, k, lo,
                       ws);
    hipLaunchKernelGGL(topk_write_kernel, dim3(grid), dim3(kThreads), 0, stream, scores, q_pos, L, k, lo, ws, idx);
    return hipGetLastError();
}

}  // namespace dsa
