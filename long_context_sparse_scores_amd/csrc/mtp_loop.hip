// Pieces of the multi-round MTP loop around the draft path (gfx950).
//
// [MTPBLOG, "MTP"] and [TEARDOWN, 刀四 MTP] (4sapi.ai GLM-5.2 MTP / IndexShare
// write-up; clawlihai.cn architecture teardown): generation proceeds in rounds
// of draft -> verify -> keep the accepted prefix, the next round starting from
// the verified tokens.  [MTPBLOG, "KV Share"]: the draft layers read the
// backbone's cache and only new tokens get new cache rows.
//
//   target-only verification ([MTPBLOG, "Rejection Sampling"]: the rule that
//   rejection sampling replaced): a draft is kept while it is the target's
//   first choice.  Two launches: the argmax of every (row, 8192-wide chunk),
//   then one wave per sequence merges the chunks (larger value, then lower
//   index) and finds the first draft that is not the argmax.
//
//   commit: after verification, the rows of the accepted drafts and of the
//   next token are written into the index-key and latent caches and the
//   position advances, all on the device, so rounds chain without the host
//   reading n_accepted.  One block per candidate row, 16-byte copies.
#include "common.h"

namespace dsa {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 8192;
constexpr int kPer = kChunk / kThreads;   // 32 logits per thread and chunk

struct ArgMax {
    float v;
    int i;
};

// The better of two candidates: larger value, then lower index.
__device__ __forceinline__ ArgMax better(ArgMax a, ArgMax b) {
    return (b.v > a.v || (b.v == a.v && b.i < a.i)) ? b : a;
}

__device__ __forceinline__ ArgMax shfl_xor_am(ArgMax a, int off) {
    return ArgMax{__shfl_xor(a.v, off, kWave), __shfl_xor(a.i, off, kWave)};
}

// Argmax of chunk c of row r (lowest index among equal maxima): part[r * nchunk + c].
__global__ __launch_bounds__(kThreads) void argmax_chunk_kernel(const float* __restrict__ x, int V, int nchunk,
                                                                ArgMax* __restrict__ part) {
    const int r = blockIdx.x / nchunk;
    const int c = blockIdx.x % nchunk;
    const float* row = x + (int64_t)r * V;
    const int base = c * kChunk;
    // thread t reads logits base + t + 256j (coalesced); its indices increase with
    // j, so a strict comparison keeps the lowest index among its equal maxima
    float v[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int i = base + (int)threadIdx.x + kThreads * j;
        v[j] = i < V ? row[i] : -INFINITY;
    }
    ArgMax best{-INFINITY, 0x7FFFFFFF};
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int i = base + (int)threadIdx.x + kThreads * j;
        if (i < V && (v[j] > best.v || best.i == 0x7FFFFFFF)) best = ArgMax{v[j], i};
    }
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) best = better(best, shfl_xor_am(best, off));
    __shared__ ArgMax sw[kThreads / kWave];
    if (lane_id() == 0) sw[threadIdx.x / kWave] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
        ArgMax r0 = sw[0];
#pragma unroll
        for (int w = 1; w < kThreads / kWave; ++w) r0 = better(r0, sw[w]);
        part[blockIdx.x] = r0;
    }
}

// One wave per sequence: the argmax of rows 0..S, then the first draft that differs.
__global__ __launch_bounds__(kWave) void target_only_decide_kernel(const ArgMax* __restrict__ part,
                                                                   const int32_t* __restrict__ draft_tokens, int S,
                                                                   int nchunk, int32_t* __restrict__ n_acc,
                                                                   int32_t* __restrict__ next_tok) {
    const int b = blockIdx.x;
    const int lane = lane_id();
    int n = S;
    int nxt = 0;
    for (int i = 0; i <= S; ++i) {
        const ArgMax* pr = part + ((int64_t)b * (S + 1) + i) * nchunk;
        ArgMax best{-INFINITY, 0x7FFFFFFF};
        for (int c = lane; c < nchunk; c += kWave) best = better(best, pr[c]);
#pragma unroll
        for (int off = kWave / 2; off > 0; off >>= 1) best = better(best, shfl_xor_am(best, off));
        if (i == S || draft_tokens[(int64_t)b * S + i] != best.i) {
            n = i;
            nxt = best.i;
            break;
        }
    }
    if (lane == 0) {
        n_acc[b] = n;
        next_tok[b] = nxt;
    }
}

// Block (b, j): row j of the candidates goes to position q_pos_in[b] + 1 + j when
// j <= n_acc[b] and the position is inside the cache; block (b, 0) also writes
// the next position.  Rows are copied as 16-byte chunks.
__global__ __launch_bounds__(128) void mtp_commit_kernel(const int32_t* __restrict__ n_acc,
                                                         const int32_t* __restrict__ q_pos_in,
                                                         const u32x4_t* __restrict__ new_k,
                                                         const u32x4_t* __restrict__ new_kv, u32x4_t* k_cache,
                                                         int64_t k_bstride16, u32x4_t* kv_cache, int64_t kv_bstride16,
                                                         int S, int L, int k_row16, int kv_row16,
                                                         int32_t* __restrict__ q_pos_out) {
    const int b = blockIdx.x / (S + 1);
    const int j = blockIdx.x % (S + 1);
    const int n = n_acc[b];
    const int64_t p = q_pos_in[b];
    if (j == 0 && threadIdx.x == 0) {
        const int64_t np = p + n + 1;
        q_pos_out[b] = (int32_t)(np < L ? np : (int64_t)L - 1);
    }
    const int64_t pos = p + 1 + j;
    if (j > n || pos < 0 || pos >= L) return;  // (a negative q_pos_in writes nothing)
    const int64_t src = (int64_t)b * (S + 1) + j;
    for (int c = threadIdx.x; c < k_row16 + kv_row16; c += 128) {
        if (c < k_row16)
            k_cache[b * k_bstride16 + pos * k_row16 + c] = new_k[src * k_row16 + c];
        else
            kv_cache[b * kv_bstride16 + pos * kv_row16 + (c - k_row16)] = new_kv[src * kv_row16 + (c - k_row16)];
    }
}

}  // namespace

size_t target_only_ws_bytes(int B, int S, int V) {
    const int nchunk = (V + kChunk - 1) / kChunk;
    return align_up((size_t)B * (S + 1) * nchunk * sizeof(ArgMax), 256);
}

hipError_t launch_target_only(const float* target, const int32_t* draft_tokens, int B, int S, int V,
                              int32_t* n_acc, int32_t* next_tok, void* ws, hipStream_t stream) {
    const int nchunk = (V + kChunk - 1) / kChunk;
    ArgMax* part = reinterpret_cast<ArgMax*>(ws);
    hipLaunchKernelGGL(argmax_chunk_kernel, dim3((unsigned)((int64_t)B * (S + 1) * nchunk)), dim3(kThreads), 0,
                       stream, target, V, nchunk, part);
    hipLaunchKernelGGL(target_only_decide_kernel, dim3(B), dim3(kWave), 0, stream, part, draft_tokens, S, nchunk,
                       n_acc, next_tok);
    return hipGetLastError();
}

hipError_t launch_mtp_commit(const int32_t* n_acc, const int32_t* q_pos_in, const void* new_k, const void* new_kv,
                             void* k_cache, int64_t k_bstride_bytes, void* kv_cache, int64_t kv_bstride_bytes, int B,
                             int S, int L, int k_row_bytes, int kv_row_bytes, int32_t* q_pos_out,
                             hipStream_t stream) {
    hipLaunchKernelGGL(mtp_commit_kernel, dim3((unsigned)(B * (S + 1))), dim3(128), 0, stream, n_acc, q_pos_in,
                       reinterpret_cast<const u32x4_t*>(new_k), reinterpret_cast<const u32x4_t*>(new_kv),
                       reinterpret_cast<u32x4_t*>(k_cache), k_bstride_bytes / 16, reinterpret_cast<u32x4_t*>(kv_cache),
                       kv_bstride_bytes / 16, S, L, k_row_bytes / 16, kv_row_bytes / 16, q_pos_out);
    return hipGetLastError();
}

}  // namespace dsa
