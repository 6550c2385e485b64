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

// Stores written through the L2 to memory (sc1) for results a later kernel
// reads: the data leaves the L2 while the kernel runs instead of in the
// write-back that ends it (measured at decode 128K: the index scan 169 -> 166
// us, an attention layer's split-and-combine 26 -> 24.4 us).  The base must
// be wave-uniform; offsets are bytes, below 2^31.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wt_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7FFFFFFF, 0x00020000);
}
// A raw buffer of `bytes` bytes (at most 2^31 - 1): a lane whose offset plus
// access size passes the end reads zeros and its store is dropped, so a
// ragged edge needs no branch (kOutOfRange is past any such buffer).
constexpr uint32_t kOutOfRange = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t sized_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
// 16-byte streaming load (nt: the line is not kept for reuse).
__device__ __forceinline__ u32x4_t load_nt16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2));
}
__device__ __forceinline__ void store_wt16(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4_t v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 16);
}
__device__ __forceinline__ void store_wt4(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t v) {
    __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, 0, 16);
}
__device__ __forceinline__ void store_wt4(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
    store_wt4(r, off, __float_as_uint(v));
}

// Device-scope load (sc1): it misses in this XCD's L2, so it sees what
// workgroups on other XCDs wrote through to memory during the same launch.
__device__ __forceinline__ uint32_t load_dev4u(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 16);
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

// Inclusive prefix sum across one wave, in DPP moves (no LDS permutes): row
// shifts by 1, 2, 4, 8 scan each row of 16 lanes (a lane shifted in from
// outside the row adds 0), then row_bcast:15 adds the end of rows 0 and 2 to
// rows 1 and 3, and row_bcast:31 the end of row 1 to rows 2 and 3.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_add(uint32_t x) {
    return x + (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROW_MASK, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
    x = dpp_add<0x111, 0xF>(x);  // row_shr:1
    x = dpp_add<0x112, 0xF>(x);  // row_shr:2
    x = dpp_add<0x114, 0xF>(x);  // row_shr:4
    x = dpp_add<0x118, 0xF>(x);  // row_shr:8
    x = dpp_add<0x142, 0xA>(x);  // row_bcast:15 into rows 1 and 3
    x = dpp_add<0x143, 0xC>(x);  // row_bcast:31 into rows 2 and 3
    return x;
}

// ------------------------------------------------------------- launch interfaces
// Top-k state the indexer prepares for the selection that follows it (layer
// group): for every row r, the uint32 words at base + r*stride.  Words
// [zero_off, zero_off + zero_count) are cleared; when `hist` is set, the row's
// histogram of the top 11 bits of the order-preserving score keys (visible
// keys only) is added into words [0, 2048), which the previous selection on
// this workspace left zero (the filter checks that it did).
struct TopkPrep {
    uint32_t* base = nullptr;
    int64_t stride = 0;
    int zero_off = 0;
    int zero_count = 0;
    bool hist = false;
};

constexpr int kTopBins = 2048;  // bins of the top score-key digit (11 bits)

// Whether the indexer launch for chunks of T queries per sequence can add the
// top-digit histogram (TopkPrep::hist): the per-query decode kernels can, the
// multi-query tile kernels cannot.
bool indexer_counts_histogram(int T);
// Workgroups of the indexer launch for these sizes (bf16 or E4M3 keys).
int64_t indexer_grid_blocks(int B, int T, int L, bool fp8);

hipError_t launch_indexer(const uint16_t* q_idx, const float* w, const uint16_t* k_idx, int64_t k_bstride,
                          const int32_t* q_pos, int B, int T, int L, float* scores, hipStream_t stream,
                          TopkPrep prep = TopkPrep());

// The same scores from E4M3 index queries and keys (one byte per element).
hipError_t launch_indexer_fp8(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, int64_t k_bstride,
                              const int32_t* q_pos, int B, int T, int L, float* scores, hipStream_t stream,
                              TopkPrep prep = TopkPrep());

size_t topk_ws_bytes(int rows, int L, int k);
// What the indexer prepares before a selection: with `hist`, it clears the
// counters and adds the top-digit histogram onto what the last selection left
// (zero, and stamped as such); without, it clears both.
TopkPrep topk_prep(void* ws, int rows, int L, bool hist);
// How much of the selection's state is ready when launch_topk is called.
enum class TopkState {
    kNone,       // nothing: clear the state and build the histogram
    kCleared,    // the histogram and counters are zero (TopkPrep without hist)
    kHistogram,  // counters zero and the histogram complete (TopkPrep with hist)
};
hipError_t launch_topk(const float* scores, const int32_t* q_pos, int rows, int L, int k, int32_t* idx, void* ws,
                       hipStream_t stream, TopkState state = TopkState::kNone);

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
