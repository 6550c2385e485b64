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
//   minsum  per (draft step, chunk): sum_v min(p_v, q_v), and sum_v
//           max(p_v - q_v, 0) for the resample after a rejection there; the
//           block of the chunk holding the step's draft token also makes its
//           acceptance test;
//   accept  one block per sequence: the first rejection, then the inverse CDF
//           of the residual (or of p_S): the chunk holding the threshold from
//           a wave scan of the chunk sums, and inside it a block-wide ordered
//           scan over contiguous per-thread segments.
// Exponentials are fp32; every sum is fp64 and merged in a fixed order, so
// results are deterministic run to run.
#include "common.h"

namespace dsa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kChunk = 8192;
constexpr int kPer = kChunk / kThreads;  // 32 values per thread and chunk
constexpr int kMaxSteps = kWave;         // draft steps: the accept block finds the first rejection with one ballot

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

// Thread t's values of a chunk, -inf past the end.  VEC (rows of a multiple of
// 4 values, 16-byte aligned): x[4j + e] = src[4t + 1024 j + e], one 16-byte
// load per lane and 1 KiB per wave instruction; else x[j] = src[t + 256 j].
template <bool VEC>
__device__ __forceinline__ void load_chunk(const float* src, int n, float (&x)[kPer]) {
    if constexpr (VEC) {
#pragma unroll
        for (int j = 0; j < kPer / 4; ++j) {
            const int i = 4 * (int)threadIdx.x + 4 * kThreads * j;  // n is a multiple of 4
            const float4 v = i < n ? *reinterpret_cast<const float4*>(src + i)
                                   : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
            x[4 * j] = v.x;
            x[4 * j + 1] = v.y;
            x[4 * j + 2] = v.z;
            x[4 * j + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int i = (int)threadIdx.x + kThreads * j;
            x[j] = i < n ? src[i] : -INFINITY;
        }
    }
}

// Chunk index of value j of this thread as load_chunk<VEC> places it.
template <bool VEC>
__device__ __forceinline__ int chunk_index(int j) {
    return VEC ? 4 * (int)threadIdx.x + 4 * kThreads * (j / 4) + (j % 4) : (int)threadIdx.x + kThreads * j;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

template <bool VEC>
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
    load_chunk<VEC>(src, n, x);
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
    s = wave_sum(s);
    if (lane == 0) merged[row] = RowStat{M, s};
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) void verify_minsum_kernel(const float* __restrict__ target,
                                                                 const float* __restrict__ draft, int B, int S,
                                                                 int V, int nchunk, const RowStat* __restrict__ merged,
                                                                 const int32_t* __restrict__ tokens,
                                                                 const float* __restrict__ u_acc,
                                                                 double* __restrict__ msum, double* __restrict__ rsum,
                                                                 int32_t* __restrict__ acc) {
    __shared__ double ds[kWaves];
    const int pair = blockIdx.x / nchunk;  // b*S + i
    const int chunk = blockIdx.x % nchunk;
    const int b = pair / S, i = pair % S;
    const int trow = b * (S + 1) + i;
    const float* t = target + (int64_t)trow * V + (int64_t)chunk * kChunk;
    const float* d = draft + (int64_t)pair * V + (int64_t)chunk * kChunk;
    const int n = min(kChunk, V - chunk * kChunk);
    float xt[kPer], xd[kPer];
    load_chunk<VEC>(t, n, xt);
    load_chunk<VEC>(d, n, xd);
    const RowStat tp = merged[trow];
    const RowStat dp = merged[B * (S + 1) + pair];
    // The acceptance test of draft step i, u < p(x)/q(x), made by the block of
    // the chunk holding its token x (chunk 0 for a token outside the
    // vocabulary, whose target probability is 0).
    if (threadIdx.x == 0) {
        const int x = tokens[pair];
        const bool in = x >= 0 && x < V;
        if ((in ? x / kChunk : 0) == chunk) {
            int ok = 0;
            if (in) {
                const double px = (double)expf(target[(int64_t)trow * V + x] - tp.m) / tp.s;
                const double qx = (double)expf(draft[(int64_t)pair * V + x] - dp.m) / dp.s;
                ok = (double)u_acc[pair] < px / qx;
            }
            acc[pair] = ok;
        }
    }
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

template <bool VEC>
__global__ __launch_bounds__(kThreads) void verify_accept_kernel(
    const float* __restrict__ target, const float* __restrict__ draft, const int32_t* __restrict__ acc,
    const float* __restrict__ u_res, int B, int S, int V, int nchunk, const RowStat* __restrict__ stats,
    const RowStat* __restrict__ merged, const double* __restrict__ msum, const double* __restrict__ rsum,
    float* __restrict__ min_sum, int32_t* __restrict__ n_acc, int32_t* __restrict__ next_tok) {
    __shared__ double dscr[kWaves];
    __shared__ int rej_sh, resid_sh, chunk_sh, found, last_sh;
    __shared__ double before_sh, thr_sh;
    __shared__ RowStat tp_sh, dp_sh;
    __shared__ float seg[2][kChunk + kChunk / 32];  // the chosen chunk, value i at i + i / 32
    const int b = blockIdx.x;
    const int lane = lane_id();
    const int wave = (int)threadIdx.x / kWave;
    if (wave > 0) {
        // acceptance sums: waves 1-3 take draft steps i = w - 1, w + 2, ...; lane
        // l adds the chunk min-sums l, l + 64, ... in order, then a fixed tree
        for (int i = wave - 1; i < S; i += kWaves - 1) {
            double a = 0.0;
            for (int c = lane; c < nchunk; c += kWave) a += msum[(int64_t)(b * S + i) * nchunk + c];
            a = wave_sum(a);
            if (lane == 0) min_sum[b * S + i] = (float)a;
        }
    } else {
        // wave 0: the first rejection (S <= 64: one ballot) from the tests the
        // min-sum pass made, with every row statistic it may need loaded beside
        // them: lane i holds target row i and draft row i of this sequence
        const int ok = lane < S ? acc[b * S + lane] : 1;
        const RowStat tl = lane < S ? merged[b * (S + 1) + lane] : RowStat{0.0f, 1.0};
        const RowStat dl = lane < S ? merged[B * (S + 1) + b * S + lane] : RowStat{0.0f, 1.0};
        const RowStat tlast = merged[b * (S + 1) + S];
        const double ur = (double)u_res[b];
        const uint64_t rm = __ballot(!ok);
        const int rej = rm ? __ffsll((unsigned long long)rm) - 1 : -1;
        RowStat tp = tlast, dp = {0.0f, 1.0};
        if (rej >= 0) {
            tp = RowStat{__shfl(tl.m, rej, kWave), __shfl(tl.s, rej, kWave)};
            dp = RowStat{__shfl(dl.m, rej, kWave), __shfl(dl.s, rej, kWave)};
        }
        // chunk masses of the distribution to sample: the residual at the
        // rejection, else p_S; a residual without mass (p == q) falls back to p
        // itself.  Lane l holds chunks l + 64 s; prefix sums come from a wave
        // scan per 64 chunks, carried across them in chunk order.
        const int trow = b * (S + 1) + (rej < 0 ? S : rej);
        bool residual = rej >= 0;
        auto chunk_mass = [&](int c) -> double {
            if (c >= nchunk) return 0.0;
            if (residual) return rsum[(int64_t)(b * S + rej) * nchunk + c];
            const RowStat cs = stats[(int64_t)trow * nchunk + c];
            return cs.s * (double)__expf(cs.m - tp.m) / tp.s;
        };
        // inclusive and exclusive prefix of chunk c0 + lane within its 64-chunk group
        auto scan = [&](double m, double& excl) -> double {
            double inc = m;
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) {
                const double y = __shfl_up(inc, off, kWave);
                if (lane >= off) inc += y;
            }
            const double e = __shfl_up(inc, 1, kWave);
            excl = lane == 0 ? 0.0 : e;
            return inc;
        };
        // the first 64 chunks' masses stay in a register (every chunk for V <= 2^19)
        double m_first = chunk_mass(lane);
        auto mass_of = [&](int c0) -> double { return c0 == 0 ? m_first : chunk_mass(c0 + lane); };
        auto total_mass = [&]() -> double {
            double carry = 0.0, excl;
            for (int c0 = 0; c0 < nchunk; c0 += kWave) carry += __shfl(scan(mass_of(c0), excl), kWave - 1, kWave);
            return carry;
        };
        double total = total_mass();
        if (residual && !(total > 0.0)) {
            residual = false;
            m_first = chunk_mass(lane);
            total = total_mass();
        }
        const double thr = ur * total;
        // the first chunk whose end passes thr, and the last chunk with mass
        double carry = 0.0;
        int cc = -1, last_nz = -1;
        double before = 0.0, before_last = 0.0;
        for (int c0 = 0; c0 < nchunk && cc < 0; c0 += kWave) {
            const double m = mass_of(c0);
            double excl;
            const double inc = scan(m, excl);
            const double bef = carry + excl;
            const uint64_t hit = __ballot(c0 + lane < nchunk && bef + m > thr);
            const uint64_t nz = __ballot(m > 0.0);
            if (hit) {
                const int l = __ffsll((unsigned long long)hit) - 1;
                cc = c0 + l;
                before = __shfl(bef, l, kWave);
            }
            if (nz) {
                const int l = 63 - __clzll((long long)nz);
                last_nz = c0 + l;
                before_last = __shfl(bef, l, kWave);
            }
            carry += __shfl(inc, kWave - 1, kWave);
        }
        if (lane == 0) {
            rej_sh = rej;
            n_acc[b] = rej < 0 ? S : rej;
            resid_sh = residual;
            tp_sh = tp;
            dp_sh = residual ? dp : RowStat{0.0f, 1.0};
            if (cc < 0) {  // thr at or above the rounded total: the last chunk with mass, its last token
                chunk_sh = last_nz;
                before_sh = before_last;
                thr_sh = INFINITY;
            } else {
                chunk_sh = cc;
                before_sh = before;
                thr_sh = thr;
            }
            found = V;
            last_sh = -1;
        }
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
    const RowStat tp = tp_sh, dp = dp_sh;
    const double it = 1.0 / tp.s;
    const double id = 1.0 / dp.s;
    // this thread's contiguous segment of the chunk: coalesced loads into LDS,
    // then 32 consecutive values per thread (bank-conflict free with the padding)
    const int base = cc * kChunk;
    const int n = min(kChunk, V - base);
    const int v0 = (int)threadIdx.x * kPer;
    float xt[kPer], xd[kPer];
    load_chunk<VEC>(target + (int64_t)trow * V + base, n, xt);
    if (residual) load_chunk<VEC>(draft + (int64_t)(b * S + rej) * V + base, n, xd);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int i = chunk_index<VEC>(j);
        seg[0][i + (i >> 5)] = xt[j];
        if (residual) seg[1][i + (i >> 5)] = xd[j];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        xt[j] = seg[0][v0 + j + (v0 >> 5)];
        xd[j] = residual ? seg[1][v0 + j + (v0 >> 5)] : -INFINITY;
    }
    double mass[kPer];
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
           2 * align_up((size_t)B * S * nc * sizeof(double), 256) + align_up((size_t)B * S * sizeof(int32_t), 256);
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
    w += align_up((size_t)B * S * nc * sizeof(double), 256);
    int32_t* acc = reinterpret_cast<int32_t*>(w);  // acceptance test of each draft step
    // 16-byte loads when every row starts 16-byte aligned (the logits are)
    const bool vec = V % 4 == 0;
    hipLaunchKernelGGL(vec ? verify_stats_kernel<true> : verify_stats_kernel<false>, dim3((unsigned)(rows * nc)),
                       dim3(kThreads), 0, stream, target, draft, B, S, V, nc, stats);
    hipLaunchKernelGGL(verify_merge_kernel, dim3((unsigned)((rows + kWaves - 1) / kWaves)), dim3(kThreads), 0, stream,
                       stats, rows, nc, merged);
    hipLaunchKernelGGL(vec ? verify_minsum_kernel<true> : verify_minsum_kernel<false>, dim3((unsigned)(B * S * nc)),
                       dim3(kThreads), 0, stream, target, draft, B, S, V, nc, merged, draft_tokens, u_acc, msum, rsum,
                       acc);
    hipLaunchKernelGGL(vec ? verify_accept_kernel<true> : verify_accept_kernel<false>, dim3((unsigned)B),
                       dim3(kThreads), 0, stream, target, draft, acc, u_res, B, S, V, nc, stats, merged, msum, rsum,
                       min_sum, n_acc, next_tok);
    return hipGetLastError();
}

}  // namespace dsa
