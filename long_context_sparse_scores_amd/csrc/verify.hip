// MTP draft verification (gfx950).
//
// [MTPBLOG, "Rejection Sampling"] (4sapi.ai GLM-5.2 MTP / IndexShare write-up):
// for every vocabulary entry take the smaller of the target and draft
// probabilities and sum them; the sum is the probability that the draft is
// accepted.  [MTPBLOG, "MTP"] and [TEARDOWN, 刀四 MTP]: accepted drafts are
// kept, everything from the first rejected position on is dropped.  The rule
// with exactly that acceptance probability is standard speculative sampling:
// accept x_i iff u_i < p_i(x_i)/q_i(x_i); at the first rejection resample
// from max(p_i - q_i, 0); after S acceptances sample from p_S.
//
// Three launches, all bandwidth-bound streams over 151552-wide fp32 rows:
//   stats   per (row, 8192-wide chunk): chunk max and sum of exp(x - max)
//   minsum  per (draft step, chunk): sum_v min(p_v, q_v) using the merged row stats
//   accept  one block per sequence: merge the sums in chunk order, run the
//           accept loop, and invert the CDF of the residual (or of p_S) with
//           a block-wide ordered scan over contiguous per-thread segments.
// Exponentials are fp32; every sum is fp64 and merged in a fixed order, so
// results are deterministic run to run.
#include "common.h"

namespace dsa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kChunk = 8192;

struct RowStat {
    float m;
    double s;
};

template <typename T, typename Op>
__device__ T block_reduce(T v, T* scratch, Op op) {
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) v = op(v, __shfl_xor(v, off, kWave));
    const int w = threadIdx.x / kWave;
    if (lane_id() == 0) scratch[w] = v;
    __syncthreads();
    T r = scratch[0];
#pragma unroll
    for (int i = 1; i < kWaves; ++i) r = op(r, scratch[i]);
    __syncthreads();
    return r;
}

__device__ __forceinline__ const float* row_ptr(const float* target, const float* draft, int B, int S, int V,
                                               int row) {
    const int nt = B * (S + 1);
    return row < nt ? target + (int64_t)row * V : draft + (int64_t)(row - nt) * V;
}

__global__ __launch_bounds__(kThreads) void verify_stats_kernel(const float* __restrict__ target,
                                                                const float* __restrict__ draft, int B, int S,
                                                                int V, int nchunk, RowStat* __restrict__ stats) {
    __shared__ float fs[kWaves];
    __shared__ double ds[kWaves];
    const int row = blockIdx.x / nchunk;
    const int chunk = blockIdx.x % nchunk;
    const float* src = row_ptr(target, draft, B, S, V, row) + (int64_t)chunk * kChunk;
    const int n = min(kChunk, V - chunk * kChunk);
    float m = -INFINITY;
    for (int i = threadIdx.x; i < n; i += kThreads) m = fmaxf(m, src[i]);
    m = block_reduce(m, fs, [](float a, float b) { return fmaxf(a, b); });
    double s = 0.0;
    for (int i = threadIdx.x; i < n; i += kThreads) s += (double)__expf(src[i] - m);
    s = block_reduce(s, ds, [](double a, double b) { return a + b; });
    if (threadIdx.x == 0) stats[blockIdx.x] = RowStat{m, s};
}

// Merge a row's chunk statistics in chunk order.
__device__ RowStat merge_row(const RowStat* __restrict__ stats, int row, int nchunk) {
    const RowStat* st = stats + (int64_t)row * nchunk;
    float M = -INFINITY;
    for (int c = 0; c < nchunk; ++c) M = fmaxf(M, st[c].m);
    double s = 0.0;
    for (int c = 0; c < nchunk; ++c) s += st[c].s * (double)__expf(st[c].m - M);
    return RowStat{M, s};
}

__global__ __launch_bounds__(kThreads) void verify_minsum_kernel(const float* __restrict__ target,
                                                                 const float* __restrict__ draft, int B, int S,
                                                                 int V, int nchunk, const RowStat* __restrict__ stats,
                                                                 double* __restrict__ msum) {
    __shared__ double ds[kWaves];
    const int pair = blockIdx.x / nchunk;  // b*S + i
    const int chunk = blockIdx.x % nchunk;
    const int b = pair / S, i = pair % S;
    const int trow = b * (S + 1) + i;
    const int drow = B * (S + 1) + pair;
    const RowStat tp = merge_row(stats, trow, nchunk);
    const RowStat dp = merge_row(stats, drow, nchunk);
    const double it = 1.0 / tp.s, id = 1.0 / dp.s;
    const float* t = target + (int64_t)trow * V + (int64_t)chunk * kChunk;
    const float* d = draft + (int64_t)pair * V + (int64_t)chunk * kChunk;
    const int n = min(kChunk, V - chunk * kChunk);
    double acc = 0.0;
    for (int v = threadIdx.x; v < n; v += kThreads) {
        const double p = (double)__expf(t[v] - tp.m) * it;
        const double q = (double)__expf(d[v] - dp.m) * id;
        acc += p < q ? p : q;
    }
    acc = block_reduce(acc, ds, [](double a, double b) { return a + b; });
    if (threadIdx.x == 0) msum[blockIdx.x] = acc;
}

template <typename T>
__device__ T block_excl_scan_t(T x, T* scratch, T* total) {
    const int l = lane_id();
    T inc = x;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        T y = __shfl_up(inc, off, kWave);
        if (l >= off) inc += y;
    }
    const int w = threadIdx.x / kWave;
    if (l == kWave - 1) scratch[w] = inc;
    __syncthreads();
    T before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        before += (i < w) ? scratch[i] : (T)0;
        tot += scratch[i];
    }
    __syncthreads();
    *total = tot;
    return before + inc - x;
}

__global__ __launch_bounds__(kThreads) void verify_accept_kernel(
    const float* __restrict__ target, const float* __restrict__ draft, const int32_t* __restrict__ tokens,
    const float* __restrict__ u_acc, const float* __restrict__ u_res, int B, int S, int V, int nchunk,
    const RowStat* __restrict__ stats, const double* __restrict__ msum, float* __restrict__ min_sum,
    int32_t* __restrict__ n_acc, int32_t* __restrict__ next_tok) {
    __shared__ int rej_sh;
    __shared__ double dscr[kWaves];
    __shared__ int found;
    __shared__ int last_sh;
    const int b = blockIdx.x;
    if (threadIdx.x < S) {
        const int i = threadIdx.x;
        double a = 0.0;
        for (int c = 0; c < nchunk; ++c) a += msum[(int64_t)(b * S + i) * nchunk + c];
        min_sum[b * S + i] = (float)a;
    }
    if (threadIdx.x == 0) {
        int rej = -1;
        for (int i = 0; i < S; ++i) {
            const int x = tokens[b * S + i];
            if (x < 0 || x >= V) {  // a token outside the vocabulary has target probability 0
                rej = i;
                break;
            }
            const RowStat tp = merge_row(stats, b * (S + 1) + i, nchunk);
            const RowStat dp = merge_row(stats, B * (S + 1) + b * S + i, nchunk);
            const double p = (double)expf(target[(int64_t)(b * (S + 1) + i) * V + x] - tp.m) / tp.s;
            const double q = (double)expf(draft[(int64_t)(b * S + i) * V + x] - dp.m) / dp.s;
            if (!((double)u_acc[b * S + i] < p / q)) {
                rej = i;
                break;
            }
        }
        rej_sh = rej;
        found = V;
        last_sh = -1;
        n_acc[b] = rej < 0 ? S : rej;
    }
    __syncthreads();
    const int rej = rej_sh;
    // distribution to sample: residual max(p_i - q_i, 0) at the rejection, else p_S
    const int trow = b * (S + 1) + (rej < 0 ? S : rej);
    const RowStat tp = merge_row(stats, trow, nchunk);
    const double it = 1.0 / tp.s;
    const float* t = target + (int64_t)trow * V;
    const float* d = nullptr;
    double id = 0.0;
    float dm = 0.0f;
    if (rej >= 0) {
        const RowStat dp = merge_row(stats, B * (S + 1) + b * S + rej, nchunk);
        id = 1.0 / dp.s;
        dm = dp.m;
        d = draft + (int64_t)(b * S + rej) * V;
    }
    auto mass = [&](int v) -> double {
        const double p = (double)__expf(t[v] - tp.m) * it;
        if (rej < 0) return p;
        const double q = (double)__expf(d[v] - dm) * id;
        return p > q ? p - q : 0.0;
    };
    const int seg = (V + kThreads - 1) / kThreads;
    const int v0 = threadIdx.x * seg;
    const int v1 = min(V, v0 + seg);
    double part = 0.0;
    for (int v = v0; v < v1; ++v) part += mass(v);
    double total;
    const double before = block_excl_scan_t<double>(part, dscr, &total);
    const double thr = (double)u_res[b] * total;
    if (before <= thr && thr < before + part) {
        double cum = before;
        for (int v = v0; v < v1; ++v) {
            cum += mass(v);
            if (cum > thr) {
                atomicMin(&found, v);
                break;
            }
        }
    }
    __syncthreads();
    if (found == V) {  // thr at or above the rounded total: take the last token with mass
        int last = -1;
        for (int v = v0; v < v1; ++v)
            if (mass(v) > 0.0) last = v;
        if (last >= 0) atomicMax(&last_sh, last);
        __syncthreads();
        if (threadIdx.x == 0) next_tok[b] = last_sh;
    } else if (threadIdx.x == 0) {
        next_tok[b] = found;
    }
}

}  // namespace

static int verify_nchunk(int V) { return (V + kChunk - 1) / kChunk; }

size_t verify_ws_bytes(int B, int S, int V) {
    const int nc = verify_nchunk(V);
    const size_t rows = (size_t)B * (S + 1) + (size_t)B * S;
    return align_up(rows * nc * sizeof(RowStat), 256) + align_up((size_t)B * S * nc * sizeof(double), 256);
}

hipError_t launch_verify(const float* target, const float* draft, const int32_t* draft_tokens, const float* u_acc,
                         const float* u_res, int B, int S, int V, float* min_sum, int32_t* n_acc, int32_t* next_tok,
                         void* ws, hipStream_t stream) {
    const int nc = verify_nchunk(V);
    const int rows = B * (S + 1) + B * S;
    RowStat* stats = reinterpret_cast<RowStat*>(ws);
    double* msum = reinterpret_cast<double*>(reinterpret_cast<char*>(ws) +
                                             align_up((size_t)rows * nc * sizeof(RowStat), 256));
    hipLaunchKernelGGL(verify_stats_kernel, dim3((unsigned)(rows * nc)), dim3(kThreads), 0, stream, target, draft, B,
                       S, V, nc, stats);
    hipLaunchKernelGGL(verify_minsum_kernel, dim3((unsigned)(B * S * nc)), dim3(kThreads), 0, stream, target, draft,
                       B, S, V, nc, stats, msum);
    hipLaunchKernelGGL(verify_accept_kernel, dim3((unsigned)B), dim3(kThreads), 0, stream, target, draft,
                       draft_tokens, u_acc, u_res, B, S, V, nc, stats, msum, min_sum, n_acc, next_tok);
    return hipGetLastError();
}

}  // namespace dsa
