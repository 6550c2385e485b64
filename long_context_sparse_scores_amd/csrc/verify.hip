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
// Four launches over 151552-wide fp32 rows (8192-wide chunks):
//   stats   per (row, chunk): chunk max and sum of exp(x - max);
//   merge   per row (one wave): the row's max and softmax denominator;
//   minsum  per (draft step, chunk): sum_v min(p_v, q_v) and, for the resample
//           after a rejection there, sum_v max(p_v - q_v, 0);
//   accept  one block per sequence: the 7 acceptance tests side by side, the
//           first rejection, then the inverse CDF of the residual (or of p_S):
//           the chunk holding the threshold from the chunk sums, and inside it
//           a block-wide ordered scan over contiguous per-thread segments.
// Exponentials are fp32; every sum is fp64 and merged in a fixed order, so
// results are deterministic run to run.
#include "common.h"

namespace dsa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kChunk = 8192;
constexpr int kPer = kChunk / kThreads;  // 32 values per thread and chunk
constexpr int kMaxSteps = kThreads;      // draft steps handled by the accept block

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

// Rows: target rows b*(S+1) + i first (B*(S+1) of them), then draft rows b*S + i.
__device__ __forceinline__ const float* row_ptr(const float* target, const float* draft, int B, int S, int V,
                                               int row) {
    const int nt = B * (S + 1);
    return row < nt ? target + (int64_t)row * V : draft + (int64_t)(row - nt) * V;
}

// Thread t's values of a chunk: x[j] = src[t + 256 j] (coalesced), -inf past the end.
__device__ __forceinline__ void load_strided(const float* src, int n, float (&x)[kPer]) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int i = (int)threadIdx.x + kThreads * j;
        x[j] = i < n ? src[i] : -INFINITY;
    }
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
    float x[kPer];
    load_strided(src, n, x);
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < kPer; ++j) m = fmaxf(m, x[j]);
    m = block_reduce(m, fs, [](float a, float b) { return fmaxf(a, b); });
    double s = 0.0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) s += (double)__expf(x[j] - m);  // -inf past the end: 0
    s = block_reduce(s, ds, [](double a, double b) { return a + b; });
    if (threadIdx.x == 0) stats[blockIdx.x] = RowStat{m, s};
}

// One wave per row: max over the chunks, then the chunks' sums rescaled to it,
// accumulated per lane in chunk order and reduced by a fixed tree.
__global__ __launch_bounds__(kThreads) void verify_merge_kernel(const RowStat* __restrict__ stats, int rows,
                                                                int nchunk, RowStat* __restrict__ merged) {
    const int row = blockIdx.x * kWaves + (int)threadIdx.x / kWave;
    if (row >= rows) return;
    const int lane = lane_id();
    const RowStat* st = stats + (int64_t)row * nchunk;
    float M = -INFINITY;
    for (int c = lane; c < nchunk; c += kWave) M = fmaxf(M, st[c].m);
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, kWave));
    double s = 0.0;
    for (int c = lane; c < nchunk; c += kWave) s += st[c].s * (double)__expf(st[c].m - M);
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, kWave);
    if (lane == 0) merged[row] = RowStat{M, s};
}

__global__ __launch_bounds__(kThreads) void verify_minsum_kernel(const float* __restrict__ target,
                                                                 const float* __restrict__ draft, int B, int S,
                                                                 int V, int nchunk, const RowStat* __restrict__ merged,
                                                                 double* __restrict__ msum, double* __restrict__ rsum) {
    __shared__ double ds[kWaves];
    const int pair = blockIdx.x / nchunk;  // b*S + i
    const int chunk = blockIdx.x % nchunk;
    const int b = pair / S, i = pair % S;
    const int trow = b * (S + 1) + i;
    const float* t = target + (int64_t)trow * V + (int64_t)chunk * kChunk;
    const float* d = draft + (int64_t)pair * V + (int64_t)chunk * kChunk;
    const int n = min(kChunk, V - chunk * kChunk);
    float xt[kPer], xd[kPer];
    load_strided(t, n, xt);
    load_strided(d, n, xd);
    const RowStat tp = merged[trow];
    const RowStat dp = merged[B * (S + 1) + pair];
    const double it = 1.0 / tp.s, id = 1.0 / dp.s;
    double mn = 0.0, res = 0.0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const double p = (double)__expf(xt[j] - tp.m) * it;
        const double q = (double)__expf(xd[j] - dp.m) * id;
        mn += p < q ? p : q;
        res += p > q ? p - q : 0.0;
    }
    mn = block_reduce(mn, ds, [](double a, double b) { return a + b; });
    res = block_reduce(res, ds, [](double a, double b) { return a + b; });
    if (threadIdx.x == 0) {
        msum[blockIdx.x] = mn;
        rsum[blockIdx.x] = res;
    }
}

__global__ __launch_bounds__(kThreads) void verify_accept_kernel(
    const float* __restrict__ target, const float* __restrict__ draft, const int32_t* __restrict__ tokens,
    const float* __restrict__ u_acc, const float* __restrict__ u_res, int B, int S, int V, int nchunk,
    const RowStat* __restrict__ stats, const RowStat* __restrict__ merged, const double* __restrict__ msum,
    const double* __restrict__ rsum, float* __restrict__ min_sum, int32_t* __restrict__ n_acc,
    int32_t* __restrict__ next_tok) {
    __shared__ int accepted[kMaxSteps];
    __shared__ double dscr[kWaves];
    __shared__ int rej_sh, resid_sh, chunk_sh, found, last_sh;
    __shared__ double before_sh, thr_sh;
    const int b = blockIdx.x;
    // every draft step at once: its acceptance sum and its acceptance test
    if ((int)threadIdx.x < S) {
        const int i = threadIdx.x;
        double a = 0.0;
        for (int c = 0; c < nchunk; ++c) a += msum[(int64_t)(b * S + i) * nchunk + c];
        min_sum[b * S + i] = (float)a;
        const int x = tokens[b * S + i];
        int ok = 0;
        if (x >= 0 && x < V) {  // a token outside the vocabulary has target probability 0
            const RowStat tp = merged[b * (S + 1) + i];
            const RowStat dp = merged[B * (S + 1) + b * S + i];
            const double p = (double)expf(target[(int64_t)(b * (S + 1) + i) * V + x] - tp.m) / tp.s;
            const double q = (double)expf(draft[(int64_t)(b * S + i) * V + x] - dp.m) / dp.s;
            ok = (double)u_acc[b * S + i] < p / q;
        }
        accepted[i] = ok;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int rej = -1;
        for (int i = 0; i < S; ++i)
            if (!accepted[i]) {
                rej = i;
                break;
            }
        rej_sh = rej;
        n_acc[b] = rej < 0 ? S : rej;
        // chunk sums of the distribution to sample: the residual at the rejection, else p_S;
        // a residual without mass (p == q) falls back to p itself
        const int trow = b * (S + 1) + (rej < 0 ? S : rej);
        const RowStat tp = merged[trow];
        bool residual = rej >= 0;
        auto chunk_mass = [&](int c) -> double {
            if (residual) return rsum[(int64_t)(b * S + rej) * nchunk + c];
            const RowStat cs = stats[(int64_t)trow * nchunk + c];
            return cs.s * (double)__expf(cs.m - tp.m) / tp.s;
        };
        double total = 0.0;
        for (int c = 0; c < nchunk; ++c) total += chunk_mass(c);
        if (residual && !(total > 0.0)) {
            residual = false;
            total = 0.0;
            for (int c = 0; c < nchunk; ++c) total += chunk_mass(c);
        }
        resid_sh = residual;
        const double thr = (double)u_res[b] * total;
        int cc = -1, last_nz = -1;
        double before = 0.0, before_last = 0.0;
        for (int c = 0; c < nchunk; ++c) {
            const double m = chunk_mass(c);
            if (m > 0.0) {
                last_nz = c;
                before_last = before;
            }
            if (cc < 0 && before + m > thr) {
                cc = c;
                before_sh = before;
            }
            before += m;
        }
        if (cc < 0) {  // thr at or above the rounded total: the last chunk with mass, its last token
            cc = last_nz;
            before_sh = before_last;
            thr_sh = INFINITY;
        } else {
            thr_sh = thr;
        }
        chunk_sh = cc;
        found = V;
        last_sh = -1;
    }
    __syncthreads();
    const int rej = rej_sh;
    const bool residual = resid_sh;
    const int cc = chunk_sh;
    if (cc < 0) {  // nothing has mass (cannot happen for finite logits)
        if (threadIdx.x == 0) next_tok[b] = 0;
        return;
    }
    const int trow = b * (S + 1) + (rej < 0 ? S : rej);
    const RowStat tp = merged[trow];
    const double it = 1.0 / tp.s;
    RowStat dp = {0.0f, 1.0};
    if (residual) dp = merged[B * (S + 1) + b * S + rej];
    const double id = 1.0 / dp.s;
    // this thread's contiguous segment of the chunk
    const int base = cc * kChunk;
    const int n = min(kChunk, V - base);
    const int v0 = (int)threadIdx.x * kPer;
    const float* t = target + (int64_t)trow * V + base + v0;
    const float* d = draft + (int64_t)(b * S + (rej < 0 ? 0 : rej)) * V + base + v0;
    double mass[kPer];
    float xt[kPer], xd[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        xt[j] = v0 + j < n ? t[j] : -INFINITY;
        xd[j] = (residual && v0 + j < n) ? d[j] : -INFINITY;
    }
    double part = 0.0;
    int last = -1;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const double p = (double)__expf(xt[j] - tp.m) * it;
        double r = p;
        if (residual) {
            const double q = (double)__expf(xd[j] - dp.m) * id;
            r = p > q ? p - q : 0.0;
        }
        mass[j] = r;
        part += r;
        if (r > 0.0) last = v0 + j;
    }
    double total;
    const double before = before_sh + block_excl_scan_t<double>(part, dscr, &total);
    const double thr = thr_sh;
    if (before <= thr && thr < before + part) {
        double cum = before;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            cum += mass[j];
            if (cum > thr) {
                atomicMin(&found, base + v0 + j);
                break;
            }
        }
    }
    if (last >= 0) atomicMax(&last_sh, base + last);
    __syncthreads();
    // not found inside (threshold within rounding of the chunk's end, or past the total): its last token with mass
    if (threadIdx.x == 0) next_tok[b] = found < V ? found : last_sh;
}

}  // namespace

static int verify_nchunk(int V) { return (V + kChunk - 1) / kChunk; }

size_t verify_ws_bytes(int B, int S, int V) {
    const int nc = verify_nchunk(V);
    const size_t rows = (size_t)B * (S + 1) + (size_t)B * S;
    return align_up(rows * nc * sizeof(RowStat), 256) + align_up(rows * sizeof(RowStat), 256) +
           2 * align_up((size_t)B * S * nc * sizeof(double), 256);
}

hipError_t launch_verify(const float* target, const float* draft, const int32_t* draft_tokens, const float* u_acc,
                         const float* u_res, int B, int S, int V, float* min_sum, int32_t* n_acc, int32_t* next_tok,
                         void* ws, hipStream_t stream) {
    if (S > kMaxSteps) return hipErrorInvalidValue;
    const int nc = verify_nchunk(V);
    const int rows = B * (S + 1) + B * S;
    char* w = reinterpret_cast<char*>(ws);
    RowStat* stats = reinterpret_cast<RowStat*>(w);
    w += align_up((size_t)rows * nc * sizeof(RowStat), 256);
    RowStat* merged = reinterpret_cast<RowStat*>(w);
    w += align_up((size_t)rows * sizeof(RowStat), 256);
    double* msum = reinterpret_cast<double*>(w);
    w += align_up((size_t)B * S * nc * sizeof(double), 256);
    double* rsum = reinterpret_cast<double*>(w);
    hipLaunchKernelGGL(verify_stats_kernel, dim3((unsigned)(rows * nc)), dim3(kThreads), 0, stream, target, draft, B,
                       S, V, nc, stats);
    hipLaunchKernelGGL(verify_merge_kernel, dim3((unsigned)((rows + kWaves - 1) / kWaves)), dim3(kThreads), 0, stream,
                       stats, rows, nc, merged);
    hipLaunchKernelGGL(verify_minsum_kernel, dim3((unsigned)(B * S * nc)), dim3(kThreads), 0, stream, target, draft,
                       B, S, V, nc, merged, msum, rsum);
    hipLaunchKernelGGL(verify_accept_kernel, dim3((unsigned)B), dim3(kThreads), 0, stream, target, draft,
                       draft_tokens, u_acc, u_res, B, S, V, nc, stats, merged, msum, rsum, min_sum, n_acc, next_tok);
    return hipGetLastError();
}

}  // namespace dsa
