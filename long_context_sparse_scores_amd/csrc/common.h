// Device helpers and internal launch interfaces shared by the libdsa kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// D(16x16 fp32) += A(16x32 bf16) * B(32x16 bf16).
// Lane l holds A[l%16][8*(l/16) .. +7], B[8*(l/16) .. +7][l%16];
// result register r of lane l is D[4*(l/16) + r][l%16].
__device__ __forceinline__ f32x4_t mfma16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// LDS transpose read of 4 bf16: within each group of 16 lanes, lane 4q+r
// receives element r of the 8-byte chunk addressed by lane 4j+q as value j.
// The result is consumed as a whole vector (concatenated with a shuffle):
// extracting its elements one by one has been seen to miscompile.
__device__ __forceinline__ bf16x4_t lds_read_tr16(const void* lds_ptr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (__attribute__((address_space(3))) bf16x4_t*)(const_cast<void*>(lds_ptr)));
}

// Order-preserving map fp32 -> uint32 (larger score -> larger key); -0 and +0 map to one key.
__device__ __forceinline__ uint32_t score_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum across one wave.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
    const int l = lane_id();
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        uint32_t y = __shfl_up(x, off, kWave);
        if (l >= off) x += y;
    }
    return x;
}

// Exclusive prefix sum across a block of NW waves; `scratch` holds NW words of LDS.
// Every thread of the block must call it.
template <int NW>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t x, uint32_t* scratch, uint32_t* total) {
    const int w = threadIdx.x / kWave;
    uint32_t inc = wave_incl_scan(x);
    if (lane_id() == kWave - 1) scratch[w] = inc;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        uint32_t v = scratch[i];
        before += (i < w) ? v : 0u;
        tot += v;
    }
    __syncthreads();
    *total = tot;
    return before + inc - x;
}

// ------------------------------------------------------------- launch interfaces
// Words [r*stride, r*stride + count) of a uint32 buffer, for every row r: a
// range some later kernel needs zeroed, which the indexer clears on the way.
struct ZeroRange {
    uint32_t* base = nullptr;
    int64_t stride = 0;
    int count = 0;
};

hipError_t launch_indexer(const uint16_t* q_idx, const float* w, const uint16_t* k_idx, int64_t k_bstride,
                          const int32_t* q_pos, int B, int T, int L, float* scores, hipStream_t stream,
                          ZeroRange zero = ZeroRange());

// The same scores from E4M3 index queries and keys (one byte per element).
hipError_t launch_indexer_fp8(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, int64_t k_bstride,
                              const int32_t* q_pos, int B, int T, int L, float* scores, hipStream_t stream,
                              ZeroRange zero = ZeroRange());

size_t topk_ws_bytes(int rows, int L, int k);
// The part of the top-k workspace that must be zero when the selection starts.
ZeroRange topk_state_range(void* ws, int rows, int L);
// state_zeroed: the caller has already cleared topk_state_range (e.g. through the indexer).
hipError_t launch_topk(const float* scores, const int32_t* q_pos, int rows, int L, int k, int32_t* idx, void* ws,
                       hipStream_t stream, bool state_zeroed = false);

int attn_num_splits(int rows, int k);
size_t attn_ws_bytes(int rows, int k);
hipError_t launch_attn(const uint16_t* q, const uint16_t* kv, int64_t kv_bstride, const int32_t* idx, int B,
                       int T, int L, int k, float sm_scale, uint16_t* out, float* lse, void* ws,
                       hipStream_t stream);

// The same attention over latent rows stored as E4M3 codes (kv_bstride in bytes).
hipError_t launch_attn_fp8(const uint16_t* q, const uint8_t* kv, int64_t kv_bstride, const int32_t* idx, int B,
                           int T, int L, int k, float sm_scale, uint16_t* out, float* lse, void* ws,
                           hipStream_t stream);

size_t verify_ws_bytes(int B, int S, int V);
hipError_t launch_verify(const float* target, const float* draft, const int32_t* draft_tokens, const float* u_acc,
                         const float* u_res, int B, int S, int V, float* min_sum, int32_t* n_acc,
                         int32_t* next_tok, void* ws, hipStream_t stream);

size_t target_only_ws_bytes(int B, int S, int V);
hipError_t launch_target_only(const float* target, const int32_t* draft_tokens, int B, int S, int V,
                              int32_t* n_acc, int32_t* next_tok, void* ws, hipStream_t stream);
hipError_t launch_mtp_commit(const int32_t* n_acc, const int32_t* q_pos_in, const void* new_k, const void* new_kv,
                             void* k_cache, int64_t k_bstride_bytes, void* kv_cache, int64_t kv_bstride_bytes, int B,
                             int S, int L, int k_row_bytes, int kv_row_bytes, int32_t* q_pos_out, hipStream_t stream);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace dsa
