// Exact top-k selection on gfx950: radix select over order-preserving keys.
//
// [TEARDOWN, 刀一 DSA] (clawlihai.cn GLM-5.2 1M architecture teardown):
// index_topk 2048 — each query keeps the 2048 best-scoring visible tokens.
// Candidates are s in [0, p]; ties at the threshold go to the lower
// position; the kept positions are written in ascending order, -1 padded.
//
// Every row is split into 4096-element chunks, one workgroup each, so a few
// long rows still fill the chip.  Scores become uint32 keys whose unsigned
// order is the float order; three histogram passes (digits of 11, 11 and 10
// bits, most significant first) narrow the k-th largest key K* exactly:
//   pass 0: histogram of bits 31..21 over all candidates
//   pass 1: histogram of bits 20..10 over candidates whose top digit is the
//           threshold digit of pass 0
//   pass 2: histogram of bits 9..0 for the 22-bit threshold prefix
// Each pass accumulates an LDS histogram per chunk and adds its non-zero bins
// to the row's global histogram.  Every later kernel re-derives the
// threshold digits from those histograms (a suffix scan over 2048 bins), so
// no extra launch is needed to publish them.  Then a count pass stores, per
// chunk, how many keys are > K* and == K*; the write pass turns the counts
// before its chunk into an output offset and writes the chunk's selected
// positions in order: all keys > K*, plus keys == K* while the running count
// of equal keys (in position order) is below the number still needed.
#include "common.h"

namespace dsa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kChunk = 4096;
constexpr int kBins = 2048;

struct RowWs {
    uint32_t* hist;   // [3][kBins]
    uint32_t* cnt;    // [nchunk][2]: (#key > K*, #key == K*)
    uint32_t* state;  // [4]: K*, equal keys to take
};

__host__ __device__ inline size_t row_ws_words(int nchunk) { return 3 * kBins + 2 * (size_t)nchunk + 4; }

__device__ __forceinline__ RowWs row_ws(void* ws, int row, int nchunk) {
    uint32_t* base = reinterpret_cast<uint32_t*>(ws) + (size_t)row * row_ws_words(nchunk);
    return RowWs{base, base + 3 * kBins, base + 3 * kBins + 2 * (size_t)nchunk};
}

__device__ __forceinline__ int64_t n_visible(const int32_t* q_pos, int row, int L) {
    int64_t p = q_pos[row];
    if (p < 0) return 0;
    return (p < L - 1 ? p : (int64_t)L - 1) + 1;
}

// Find the bin holding the `need`-th largest element of a histogram of `nbins`
// bins (1 <= need <= total).  Returns the bin and the count of elements in
// higher bins.  All threads of the block must call it.
struct BinPick {
    uint32_t bin, above;
};

__device__ BinPick pick_bin(const uint32_t* __restrict__ hist, int nbins, uint32_t need, uint32_t* scan_scratch,
                            BinPick* result) {
    const int per = kBins / kThreads;  // 8 bins per thread (upper bins first for a suffix scan)
    const int t = threadIdx.x;
    // thread t owns bins [nbins - per*(t+1), nbins - per*t) when nbins == 2048; for 1024 bins
    // threads 128.. own nothing.
    uint32_t h[per];
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < per; ++i) {
        int bin = nbins - 1 - (per * t + i);  // descending
        h[i] = bin >= 0 ? hist[bin] : 0u;
        s += h[i];
    }
    if (t == 0) *result = BinPick{0u, 0u};
    uint32_t total;
    uint32_t above = block_excl_scan<kWaves>(s, scan_scratch, &total);  // count in higher bins
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
    BinPick r = *result;
    __syncthreads();
    return r;
}

__global__ __launch_bounds__(kThreads) void topk_zero_kernel(uint32_t* ws, int rows, int nchunk) {
    const size_t words = row_ws_words(nchunk);
    const size_t per_row = 3 * kBins;
    const size_t total = (size_t)rows * per_row;
    for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < total; i += (size_t)gridDim.x * kThreads) {
        size_t r = i / per_row, j = i % per_row;
        ws[r * words + j] = 0u;
    }
}

// Passes 0..2: histogram of the pass's digit over the keys matching the prefix found so far.
template <int PASS>
__global__ __launch_bounds__(kThreads) void topk_hist_kernel(const float* __restrict__ scores,
                                                             const int32_t* __restrict__ q_pos, int L, int k,
                                                             int nchunk, void* ws) {
    const int row = blockIdx.x / nchunk;
    const int chunk = blockIdx.x % nchunk;
    const int64_t n = n_visible(q_pos, row, L);
    if (n <= k) return;  // everything visible is kept
    const int64_t start = (int64_t)chunk * kChunk;
    if (start >= n) return;
    RowWs rw = row_ws(ws, row, nchunk);
    __shared__ uint32_t h[kBins];
    __shared__ uint32_t scratch[kWaves];
    __shared__ BinPick pick;
    for (int i = threadIdx.x; i < kBins; i += kThreads) h[i] = 0u;

    uint32_t prefix = 0;  // threshold digits found by earlier passes
    if (PASS >= 1) {
        BinPick b0 = pick_bin(rw.hist, kBins, (uint32_t)k, scratch, &pick);
        prefix = b0.bin;
        if (PASS >= 2) {
            BinPick b1 = pick_bin(rw.hist + kBins, kBins, (uint32_t)k - b0.above, scratch, &pick);
            prefix = (prefix << 11) | b1.bin;
        }
    }
    __syncthreads();
    const float* src = scores + (int64_t)row * L + start;
    const int64_t m = (n - start) < kChunk ? (n - start) : kChunk;
    for (int64_t i = threadIdx.x; i < m; i += kThreads) {
        uint32_t key = score_key(src[i]);
        if (PASS == 0) {
            atomicAdd(&h[key >> 21], 1u);
        } else if (PASS == 1) {
            if ((key >> 21) == prefix) atomicAdd(&h[(key >> 10) & 0x7FFu], 1u);
        } else {
            if ((key >> 10) == prefix) atomicAdd(&h[key & 0x3FFu], 1u);
        }
    }
    __syncthreads();
    uint32_t* gh = rw.hist + PASS * kBins;
    for (int i = threadIdx.x; i < kBins; i += kThreads)
        if (h[i]) atomicAdd(&gh[i], h[i]);
}

struct Threshold {
    uint32_t key, take_eq;
};

__device__ Threshold find_threshold(RowWs rw, int k, uint32_t* scratch, BinPick* pick) {
    BinPick b0 = pick_bin(rw.hist, kBins, (uint32_t)k, scratch, pick);
    uint32_t rem = (uint32_t)k - b0.above;
    BinPick b1 = pick_bin(rw.hist + kBins, kBins, rem, scratch, pick);
    rem -= b1.above;
    BinPick b2 = pick_bin(rw.hist + 2 * kBins, 1024, rem, scratch, pick);
    rem -= b2.above;
    return Threshold{(b0.bin << 21) | (b1.bin << 10) | b2.bin, rem};
}

__global__ __launch_bounds__(kThreads) void topk_count_kernel(const float* __restrict__ scores,
                                                              const int32_t* __restrict__ q_pos, int L, int k,
                                                              int nchunk, void* ws) {
    const int row = blockIdx.x / nchunk;
    const int chunk = blockIdx.x % nchunk;
    const int64_t n = n_visible(q_pos, row, L);
    if (n <= k) return;
    const int64_t start = (int64_t)chunk * kChunk;
    if (start >= n) return;
    RowWs rw = row_ws(ws, row, nchunk);
    __shared__ uint32_t scratch[kWaves];
    __shared__ BinPick pick;
    Threshold th = find_threshold(rw, k, scratch, &pick);
    const float* src = scores + (int64_t)row * L + start;
    const int64_t m = (n - start) < kChunk ? (n - start) : kChunk;
    uint32_t gt = 0, eq = 0;
    for (int64_t i = threadIdx.x; i < m; i += kThreads) {
        uint32_t key = score_key(src[i]);
        gt += key > th.key;
        eq += key == th.key;
    }
    uint32_t tg, te;
    block_excl_scan<kWaves>(gt, scratch, &tg);
    block_excl_scan<kWaves>(eq, scratch, &te);
    if (threadIdx.x == 0) {
        rw.cnt[2 * chunk] = tg;
        rw.cnt[2 * chunk + 1] = te;
        if (chunk == 0) {
            rw.state[0] = th.key;
            rw.state[1] = th.take_eq;
        }
    }
}

__global__ __launch_bounds__(kThreads) void topk_write_kernel(const float* __restrict__ scores,
                                                              const int32_t* __restrict__ q_pos, int L, int k,
                                                              int nchunk, void* ws, int32_t* __restrict__ idx) {
    const int row = blockIdx.x / nchunk;
    const int chunk = blockIdx.x % nchunk;
    const int64_t n = n_visible(q_pos, row, L);
    int32_t* out = idx + (int64_t)row * k;
    if (n <= k) {  // every visible position, in order, then -1
        if (chunk == 0)
            for (int j = threadIdx.x; j < k; j += kThreads) out[j] = j < n ? j : -1;
        return;
    }
    const int64_t start = (int64_t)chunk * kChunk;
    if (start >= n) return;
    RowWs rw = row_ws(ws, row, nchunk);
    __shared__ uint32_t scratch[kWaves];
    const uint32_t kstar = rw.state[0];
    const uint32_t take_eq = rw.state[1];
    // counts of the chunks before this one
    uint32_t gt_b = 0, eq_b = 0;
    for (int c = threadIdx.x; c < chunk; c += kThreads) {
        gt_b += rw.cnt[2 * c];
        eq_b += rw.cnt[2 * c + 1];
    }
    uint32_t gt_before, eq_before;
    block_excl_scan<kWaves>(gt_b, scratch, &gt_before);
    block_excl_scan<kWaves>(eq_b, scratch, &eq_before);
    uint32_t pos = gt_before + (eq_before < take_eq ? eq_before : take_eq);
    uint32_t eq_seen = eq_before;  // equal keys at lower positions in this row so far
    const float* src = scores + (int64_t)row * L + start;
    const int64_t m = (n - start) < kChunk ? (n - start) : kChunk;
    for (int64_t base = 0; base < m; base += kThreads) {
        const int64_t i = base + threadIdx.x;
        const bool valid = i < m;
        const uint32_t key = valid ? score_key(src[i]) : 0u;
        const uint32_t is_eq = valid && key == kstar;
        uint32_t eq_tot;
        const uint32_t eq_rank = eq_seen + block_excl_scan<kWaves>(is_eq, scratch, &eq_tot);
        const uint32_t sel = valid && (key > kstar || (is_eq && eq_rank < take_eq));
        uint32_t sel_tot;
        const uint32_t off = block_excl_scan<kWaves>(sel, scratch, &sel_tot);
        if (sel && pos + off < (uint32_t)k) out[pos + off] = (int32_t)(start + i);
        pos += sel_tot;
        eq_seen += eq_tot;
    }
}

}  // namespace

static int topk_nchunk(int L) { return (L + kChunk - 1) / kChunk; }

size_t topk_ws_bytes(int rows, int L, int k) {
    (void)k;
    return align_up((size_t)rows * row_ws_words(topk_nchunk(L)) * sizeof(uint32_t), 256);
}

hipError_t launch_topk(const float* scores, const int32_t* q_pos, int rows, int L, int k, int32_t* idx, void* ws,
                       hipStream_t stream) {
    const int nchunk = topk_nchunk(L);
    const unsigned grid = (unsigned)((int64_t)rows * nchunk);
    const size_t zero_words = (size_t)rows * 3 * kBins;
    unsigned zgrid = (unsigned)((zero_words + kThreads * 8 - 1) / (kThreads * 8));
    if (zgrid > 4096) zgrid = 4096;
    hipLaunchKernelGGL(topk_zero_kernel, dim3(zgrid), dim3(kThreads), 0, stream, (uint32_t*)ws, rows, nchunk);
    hipLaunchKernelGGL(topk_hist_kernel<0>, dim3(grid), dim3(kThreads), 0, stream, scores, q_pos, L, k, nchunk, ws);
    hipLaunchKernelGGL(topk_hist_kernel<1>, dim3(grid), dim3(kThreads), 0, stream, scores, q_pos, L, k, nchunk, ws);
    hipLaunchKernelGGL(topk_hist_kernel<2>, dim3(grid), dim3(kThreads), 0, stream, scores, q_pos, L, k, nchunk, ws);
    hipLaunchKernelGGL(topk_count_kernel, dim3(grid), dim3(kThreads), 0, stream, scores, q_pos, L, k, nchunk, ws);
    hipLaunchKernelGGL(topk_write_kernel, dim3(grid), dim3(kThreads), 0, stream, scores, q_pos, L, k, nchunk, ws,
                       idx);
    return hipGetLastError();
}

}  // namespace dsa
