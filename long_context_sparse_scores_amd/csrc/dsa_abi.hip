// C ABI of libdsa.so: argument validation, workspace planning and launch order.
// The operations themselves are described in include/dsa.h with the page
// passages that define them.
#include <cmath>
#include <cstddef>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/dsa.h"
#include "common.h"

// Scratch of dsa_layer_group_noalloc, one copy on each GPU the library runs on,
// held until the process ends.  Host code never uses this name as an address:
// it takes the device address from hipGetSymbolAddress (scratch_address below).
static __device__ __align__(256) unsigned char scratch[DSA_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_err[512] = "no error";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    std::snprintf(g_err, sizeof(g_err), "no error");
    return DSA_OK;
}

int hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(DSA_ERR_HIP, "%s: HIP launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kMaxBlocks = (int64_t)1 << 31;

bool group_size_ok(uint32_t n) {
    return n == sizeof(dsa_group_args) || n == DSA_GROUP_ARGS_V2_SIZE || n == DSA_GROUP_ARGS_V1_SIZE;
}

// elem_bytes: 2 for bf16 index queries/keys, 1 for E4M3.
int check_indexer(const void* q_idx, const float* w, const void* k_idx, int64_t k_bstride, const int32_t* q_pos,
                  int B, int T, int L, int H, int D, const float* scores, int elem_bytes = 2) {
    if (!q_idx || !w || !k_idx || !q_pos || !scores) return fail(DSA_ERR_NULL, "indexer: NULL pointer argument");
    if (B < 1 || T < 1 || L < 1) return fail(DSA_ERR_SHAPE, "indexer: B=%d T=%d L=%d must be >= 1", B, T, L);
    if (L > DSA_ATTN_CONTEXT_MAX) return fail(DSA_ERR_SHAPE, "indexer: L=%d above %d", L, DSA_ATTN_CONTEXT_MAX);
    if (H != DSA_INDEX_HEADS || D != DSA_INDEX_DIM)
        return fail(DSA_ERR_UNSUPPORTED, "indexer: H=%d D=%d, supported H=%d D=%d", H, D, DSA_INDEX_HEADS,
                    DSA_INDEX_DIM);
    if (B > 1 && k_bstride < (int64_t)L * D)
        return fail(DSA_ERR_SHAPE, "indexer: k_bstride %lld < L*D", (long long)k_bstride);
    if (dsa::indexer_grid_blocks(B, T, L, elem_bytes == 1) >= kMaxBlocks)
        return fail(DSA_ERR_SHAPE, "indexer: grid too large");
    if (!aligned16(q_idx) || !aligned16(w) || !aligned16(k_idx) || !aligned16(scores) ||
        ((k_bstride * elem_bytes) % 16) != 0)
        return fail(DSA_ERR_ALIGN, "indexer: pointers and the key batch stride in bytes must be 16-byte aligned");
    return DSA_OK;
}

int check_topk(const float* scores, const int32_t* q_pos, int B, int T, int L, int k, const int32_t* idx) {
    if (!scores || !q_pos || !idx) return fail(DSA_ERR_NULL, "topk: NULL pointer argument");
    if (B < 1 || T < 1 || L < 1) return fail(DSA_ERR_SHAPE, "topk: B=%d T=%d L=%d must be >= 1", B, T, L);
    if (k < 1 || k > DSA_TOPK_MAX) return fail(DSA_ERR_UNSUPPORTED, "topk: k=%d outside [1, %d]", k, DSA_TOPK_MAX);
    if ((int64_t)B * T * ((L + 4095) / 4096) >= kMaxBlocks) return fail(DSA_ERR_SHAPE, "topk: grid too large");
    if (!aligned16(scores) || !aligned16(idx)) return fail(DSA_ERR_ALIGN, "topk: pointers must be 16-byte aligned");
    return DSA_OK;
}

// elem_bytes: 2 for bf16 latent rows, 1 for E4M3.
int check_attn(const uint16_t* q, const void* kv, int64_t kv_bstride, const int32_t* idx, int B, int T, int L,
               int Hq, int Dqk, int Dv, int k, float sm_scale, const uint16_t* out, const float* lse,
               int elem_bytes = 2) {
    if (!q || !kv || !idx || !out) return fail(DSA_ERR_NULL, "attn: NULL pointer argument");
    if (B < 1 || T < 1 || L < 1) return fail(DSA_ERR_SHAPE, "attn: B=%d T=%d L=%d must be >= 1", B, T, L);
    if (L > DSA_ATTN_CONTEXT_MAX) return fail(DSA_ERR_SHAPE, "attn: L=%d above %d", L, DSA_ATTN_CONTEXT_MAX);
    if (Hq != DSA_ATTN_HEADS || Dqk != DSA_LATENT_DIM || Dv != DSA_VALUE_DIM)
        return fail(DSA_ERR_UNSUPPORTED, "attn: Hq=%d Dqk=%d Dv=%d, supported %d/%d/%d", Hq, Dqk, Dv, DSA_ATTN_HEADS,
                    DSA_LATENT_DIM, DSA_VALUE_DIM);
    if (k < 1 || k > DSA_TOPK_MAX) return fail(DSA_ERR_UNSUPPORTED, "attn: k=%d outside [1, %d]", k, DSA_TOPK_MAX);
    if (!std::isfinite(sm_scale)) return fail(DSA_ERR_SHAPE, "attn: sm_scale must be finite");
    if (B > 1 && kv_bstride < (int64_t)L * Dqk)
        return fail(DSA_ERR_SHAPE, "attn: kv_bstride %lld < L*Dqk", (long long)kv_bstride);
    if ((int64_t)B * T * 64 >= kMaxBlocks) return fail(DSA_ERR_SHAPE, "attn: grid too large");
    if (!aligned16(q) || !aligned16(kv) || !aligned16(idx) || !aligned16(out) || (lse && !aligned16(lse)) ||
        ((kv_bstride * elem_bytes) % 16) != 0)
        return fail(DSA_ERR_ALIGN, "attn: pointers and the kv batch stride in bytes must be 16-byte aligned");
    return DSA_OK;
}


// One layer's indexer inputs: bf16 (q_idx, k_idx) or E4M3 (q_idx8, k_idx8).
struct IndexerIn {
    const uint16_t* q_idx;
    const uint8_t* q_idx8;
    const float* w;
    const uint16_t* k_idx;
    const uint8_t* k_idx8;
    int32_t* idx_out;
};

IndexerIn indexer_in(const dsa_group_args& a, int l) {
    if (a.share) return IndexerIn{a.q_idx, a.q_idx_fp8, a.w, a.k_idx, a.k_idx_fp8, a.idx_out};
    return IndexerIn{a.layer_q_idx[l], a.layer_q_idx_fp8[l], a.layer_w[l], a.layer_k_idx[l], a.layer_k_idx_fp8[l],
                     a.layer_idx_out[l]};
}

size_t group_ws_bytes(int rows, int L, int k) {
    return dsa::align_up((size_t)rows * L * sizeof(float), 256) + dsa::topk_ws_bytes(rows, L, k) +
           dsa::attn_ws_bytes(rows, k);
}

// Validate a group call and copy its arguments into *full: the caller's struct
// may be an older, shorter version, whose missing fields read as NULL and
// share as 1.  Nothing is enqueued.
int check_group(const dsa_group_args* args, dsa_group_args* full) {
    if (!args) return fail(DSA_ERR_NULL, "group: NULL args");
    if (!group_size_ok(args->struct_size))
        return fail(DSA_ERR_SHAPE, "group: struct_size %u, expected %zu, %zu or %zu", args->struct_size,
                    sizeof(dsa_group_args), (size_t)DSA_GROUP_ARGS_V2_SIZE, (size_t)DSA_GROUP_ARGS_V1_SIZE);
    std::memset(full, 0, sizeof(*full));
    std::memcpy(full, args, args->struct_size);
    if (args->struct_size <= offsetof(dsa_group_args, share)) full->share = 1;
    const dsa_group_args* a = full;
    if (a->n_layers < 1 || a->n_layers > DSA_GROUP_LAYERS_MAX)
        return fail(DSA_ERR_SHAPE, "group: n_layers=%d outside [1, %d]", a->n_layers, DSA_GROUP_LAYERS_MAX);
    if (a->share != 0 && a->share != 1) return fail(DSA_ERR_SHAPE, "group: share=%d must be 0 or 1", a->share);
    const int B = a->B, T = a->T, L = a->L, k = a->k;
    const float* some_scores = reinterpret_cast<const float*>(16);  // the workspace is checked by the caller
    const int n_index = a->share ? 1 : a->n_layers;  // indexer + top-k runs
    for (int l = 0; l < n_index; ++l) {
        const IndexerIn in = indexer_in(*a, l);
        const bool fp8 = in.q_idx8 || in.k_idx8;
        if (fp8 && (!in.q_idx8 || !in.k_idx8 || in.q_idx || in.k_idx))
            return fail(DSA_ERR_SHAPE, "group: %s: set the E4M3 index queries and keys together, with the bf16 ones "
                        "NULL", a->share ? "q_idx_fp8/k_idx_fp8" : "layer_q_idx_fp8/layer_k_idx_fp8");
        int st = fp8 ? check_indexer(in.q_idx8, in.w, in.k_idx8, a->k_bstride, a->q_pos, B, T, L, DSA_INDEX_HEADS,
                                     DSA_INDEX_DIM, some_scores, 1)
                     : check_indexer(in.q_idx, in.w, in.k_idx, a->k_bstride, a->q_pos, B, T, L, DSA_INDEX_HEADS,
                                     DSA_INDEX_DIM, some_scores, 2);
        if (st != DSA_OK && !a->share) {  // name the layer whose indexer inputs are wrong
            char msg[sizeof(g_err)];
            std::snprintf(msg, sizeof(msg), "%s", g_err);
            return fail(st, "group (share = 0): layer %d: %s", l, msg);
        }
        if (st != DSA_OK) return st;
        if (!in.idx_out) return fail(DSA_ERR_NULL, "group: NULL %s", a->share ? "idx_out" : "layer_idx_out");
        st = check_topk(some_scores, a->q_pos, B, T, L, k, in.idx_out);
        if (st != DSA_OK) return st;
    }
    for (int l = 0; l < a->n_layers; ++l) {
        if (a->kv_fp8[l] && a->kv[l])
            return fail(DSA_ERR_SHAPE, "group: layer %d has both kv and kv_fp8; set one of them", l);
        const int32_t* idx = indexer_in(*a, l).idx_out;
        const int st = a->kv_fp8[l] ? check_attn(a->q[l], a->kv_fp8[l], a->kv_bstride[l], idx, B, T, L, DSA_ATTN_HEADS,
                                                 DSA_LATENT_DIM, DSA_VALUE_DIM, k, a->sm_scale, a->out[l], a->lse[l], 1)
                                    : check_attn(a->q[l], a->kv[l], a->kv_bstride[l], idx, B, T, L, DSA_ATTN_HEADS,
                                                 DSA_LATENT_DIM, DSA_VALUE_DIM, k, a->sm_scale, a->out[l], a->lse[l], 2);
        if (st != DSA_OK) return st;
    }
    return DSA_OK;
}

// Enqueue a validated group on a workspace of at least group_ws_bytes.
int launch_group(const dsa_group_args& a, void* ws, hipStream_t s) {
    const int B = a.B, T = a.T, L = a.L, k = a.k, rows = B * T;
    char* base = reinterpret_cast<char*>(ws);
    float* scores = reinterpret_cast<float*>(base);
    void* topk_ws = base + dsa::align_up((size_t)rows * L * sizeof(float), 256);
    void* attn_ws = reinterpret_cast<char*>(topk_ws) + dsa::topk_ws_bytes(rows, L, k);
    // The indexer prepares the selection: the per-query decode kernels clear its
    // counters and add the top-digit histogram of the scores (two launches
    // fewer); the multi-query tile kernels clear the state for the histogram pass.
    const bool hist = dsa::indexer_counts_histogram(T);
    const dsa::TopkPrep prep = dsa::topk_prep(topk_ws, rows, L, hist);
    for (int l = 0; l < a.n_layers; ++l) {
        const IndexerIn in = indexer_in(a, l);
        if (l == 0 || !a.share) {
            hipError_t e = in.q_idx8 ? dsa::launch_indexer_fp8(in.q_idx8, in.w, in.k_idx8, a.k_bstride, a.q_pos, B, T,
                                                               L, scores, s, prep)
                                     : dsa::launch_indexer(in.q_idx, in.w, in.k_idx, a.k_bstride, a.q_pos, B, T, L,
                                                           scores, s, prep);
            if (e != hipSuccess) return hip_status(e, "dsa_layer_group/indexer");
            e = dsa::launch_topk(scores, a.q_pos, rows, L, k, in.idx_out, topk_ws, s,
                                 hist ? dsa::TopkState::kHistogram : dsa::TopkState::kCleared);
            if (e != hipSuccess) return hip_status(e, "dsa_layer_group/topk");
        }
        const hipError_t e = a.kv_fp8[l] ? dsa::launch_attn_fp8(a.q[l], a.kv_fp8[l], a.kv_bstride[l], in.idx_out, B, T,
                                                                L, k, a.sm_scale, a.out[l], a.lse[l], attn_ws, s)
                                         : dsa::launch_attn(a.q[l], a.kv[l], a.kv_bstride[l], in.idx_out, B, T, L, k,
                                                            a.sm_scale, a.out[l], a.lse[l], attn_ws, s);
        if (e != hipSuccess) return hip_status(e, "dsa_layer_group/attention");
    }
    return ok();
}

// Device address of the current device's copy of `scratch`, looked up once per
// device (with that device current) and kept.
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(DSA_ERR_HIP, "group (no allocation): hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(DSA_ERR_UNSUPPORTED, "group (no allocation): device %d outside [0, %d)", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(DSA_ERR_HIP, "group (no allocation): hipGetSymbolAddress of the scratch on device %d: %s", dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return DSA_OK;
}

}  // namespace

extern "C" {

int dsa_abi_version(void) { return DSA_ABI_VERSION; }

const char* dsa_last_error(void) { return g_err; }

int dsa_indexer_scores(const uint16_t* q_idx, const float* w, const uint16_t* k_idx, int64_t k_bstride,
                       const int32_t* q_pos, int B, int T, int L, int H, int D, float* scores, void* stream) {
    int st = check_indexer(q_idx, w, k_idx, k_bstride, q_pos, B, T, L, H, D, scores);
    if (st != DSA_OK) return st;
    return hip_status(dsa::launch_indexer(q_idx, w, k_idx, k_bstride, q_pos, B, T, L, scores, (hipStream_t)stream),
                      "dsa_indexer_scores");
}

int dsa_indexer_scores_fp8(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, int64_t k_bstride,
                           const int32_t* q_pos, int B, int T, int L, int H, int D, float* scores, void* stream) {
    int st = check_indexer(q_idx, w, k_idx, k_bstride, q_pos, B, T, L, H, D, scores, 1);
    if (st != DSA_OK) return st;
    return hip_status(
        dsa::launch_indexer_fp8(q_idx, w, k_idx, k_bstride, q_pos, B, T, L, scores, (hipStream_t)stream),
        "dsa_indexer_scores_fp8");
}

size_t dsa_topk_workspace_size(int B, int T, int L, int k) {
    if (B < 1 || T < 1 || L < 1) return 0;
    return dsa::topk_ws_bytes(B * T, L, k);
}

int dsa_topk(const float* scores, const int32_t* q_pos, int B, int T, int L, int k, int32_t* idx, void* ws,
             size_t ws_bytes, void* stream) {
    int st = check_topk(scores, q_pos, B, T, L, k, idx);
    if (st != DSA_OK) return st;
    const size_t need = dsa::topk_ws_bytes(B * T, L, k);
    if (!ws || ws_bytes < need || !aligned16(ws))
        return fail(DSA_ERR_WORKSPACE, "topk: workspace %zu bytes given, %zu needed (16-byte aligned)", ws_bytes, need);
    return hip_status(dsa::launch_topk(scores, q_pos, B * T, L, k, idx, ws, (hipStream_t)stream), "dsa_topk");
}

size_t dsa_attn_workspace_size(int B, int T, int k) {
    if (B < 1 || T < 1 || k < 1 || k > DSA_TOPK_MAX) return 0;
    return dsa::attn_ws_bytes(B * T, k);
}

int dsa_sparse_mla_attn(const uint16_t* q, const uint16_t* kv, int64_t kv_bstride, const int32_t* idx, int B, int T,
                        int L, int Hq, int Dqk, int Dv, int k, float sm_scale, uint16_t* out, float* lse, void* ws,
                        size_t ws_bytes, void* stream) {
    int st = check_attn(q, kv, kv_bstride, idx, B, T, L, Hq, Dqk, Dv, k, sm_scale, out, lse);
    if (st != DSA_OK) return st;
    const size_t need = dsa::attn_ws_bytes(B * T, k);
    if (need > 0 && (!ws || ws_bytes < need || !aligned16(ws)))
        return fail(DSA_ERR_WORKSPACE, "attn: workspace %zu bytes given, %zu needed (16-byte aligned)", ws_bytes, need);
    return hip_status(
        dsa::launch_attn(q, kv, kv_bstride, idx, B, T, L, k, sm_scale, out, lse, ws, (hipStream_t)stream),
        "dsa_sparse_mla_attn");
}

int dsa_sparse_mla_attn_fp8kv(const uint16_t* q, const uint8_t* kv, int64_t kv_bstride, const int32_t* idx, int B,
                              int T, int L, int Hq, int Dqk, int Dv, int k, float sm_scale, uint16_t* out, float* lse,
                              void* ws, size_t ws_bytes, void* stream) {
    int st = check_attn(q, kv, kv_bstride, idx, B, T, L, Hq, Dqk, Dv, k, sm_scale, out, lse, 1);
    if (st != DSA_OK) return st;
    const size_t need = dsa::attn_ws_bytes(B * T, k);
    if (need > 0 && (!ws || ws_bytes < need || !aligned16(ws)))
        return fail(DSA_ERR_WORKSPACE, "attn: workspace %zu bytes given, %zu needed (16-byte aligned)", ws_bytes, need);
    return hip_status(
        dsa::launch_attn_fp8(q, kv, kv_bstride, idx, B, T, L, k, sm_scale, out, lse, ws, (hipStream_t)stream),
        "dsa_sparse_mla_attn_fp8kv");
}

// Workspace of a group: [scores B*T*L fp32][top-k scratch][attention scratch], each 256-byte aligned.
size_t dsa_layer_group_workspace_size(const dsa_group_args* a) {
    if (!a || !group_size_ok(a->struct_size) || a->B < 1 || a->T < 1 || a->L < 1 || a->k < 1 || a->k > DSA_TOPK_MAX)
        return 0;
    return group_ws_bytes(a->B * a->T, a->L, a->k);
}

int dsa_layer_group(const dsa_group_args* args, void* ws, size_t ws_bytes, void* stream) {
    dsa_group_args full;
    int st = check_group(args, &full);
    if (st != DSA_OK) return st;
    const size_t need = group_ws_bytes(full.B * full.T, full.L, full.k);
    if (!ws || ws_bytes < need || !aligned16(ws))
        return fail(DSA_ERR_WORKSPACE, "group: workspace %zu bytes given, %zu needed (16-byte aligned)", ws_bytes,
                    need);
    return launch_group(full, ws, (hipStream_t)stream);
}

int dsa_layer_group_noalloc(const dsa_group_args* args, void* stream) {
    dsa_group_args full;
    int st = check_group(args, &full);
    if (st != DSA_OK) return st;
    const size_t need = group_ws_bytes(full.B * full.T, full.L, full.k);
    if (need > (size_t)DSA_NOALLOC_SCRATCH_BYTES)
        return fail(DSA_ERR_WORKSPACE, "group (no allocation): needs %zu bytes of scratch, above the %zu the library "
                    "holds per GPU; use dsa_layer_group with a workspace", need, (size_t)DSA_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    st = scratch_address(&ws);
    if (st != DSA_OK) return st;
    return launch_group(full, ws, (hipStream_t)stream);
}

size_t mtp_verify_workspace_size(int B, int S, int V) {
    if (B < 1 || S < 1 || V < 1) return 0;
    return dsa::verify_ws_bytes(B, S, V);
}

int mtp_draft_verify(const float* target_logits, const float* draft_logits, const int32_t* draft_tokens,
                     const float* u_accept, const float* u_resample, int B, int S, int V, float* min_sum,
                     int32_t* n_accepted, int32_t* next_token, void* ws, size_t ws_bytes, void* stream) {
    if (!target_logits || !draft_logits || !draft_tokens || !u_accept || !u_resample || !min_sum || !n_accepted ||
        !next_token)
        return fail(DSA_ERR_NULL, "verify: NULL pointer argument");
    if (B < 1 || S < 1 || S > 64 || V < 1) return fail(DSA_ERR_SHAPE, "verify: B=%d S=%d V=%d (1 <= S <= 64)", B, S, V);
    if ((int64_t)(2 * S + 1) * B * ((V + 8191) / 8192) >= kMaxBlocks) return fail(DSA_ERR_SHAPE, "verify: too large");
    if (!aligned16(target_logits) || !aligned16(draft_logits))
        return fail(DSA_ERR_ALIGN, "verify: logits must be 16-byte aligned");
    const size_t need = dsa::verify_ws_bytes(B, S, V);
    if (!ws || ws_bytes < need || !aligned16(ws))
        return fail(DSA_ERR_WORKSPACE, "verify: workspace %zu bytes given, %zu needed (16-byte aligned)", ws_bytes,
                    need);
    return hip_status(dsa::launch_verify(target_logits, draft_logits, draft_tokens, u_accept, u_resample, B, S, V,
                                         min_sum, n_accepted, next_token, ws, (hipStream_t)stream),
                      "mtp_draft_verify");
}

size_t mtp_verify_target_only_workspace_size(int B, int S, int V) {
    if (B < 1 || S < 1 || V < 1) return 0;
    return dsa::target_only_ws_bytes(B, S, V);
}

int mtp_verify_target_only(const float* target_logits, const int32_t* draft_tokens, int B, int S, int V,
                           int32_t* n_accepted, int32_t* next_token, void* ws, size_t ws_bytes, void* stream) {
    if (!target_logits || !draft_tokens || !n_accepted || !next_token)
        return fail(DSA_ERR_NULL, "target-only verify: NULL pointer argument");
    if (B < 1 || S < 1 || S > 64 || V < 1)
        return fail(DSA_ERR_SHAPE, "target-only verify: B=%d S=%d V=%d (1 <= S <= 64)", B, S, V);
    if ((int64_t)B * (S + 1) * ((V + 8191) / 8192) >= kMaxBlocks)
        return fail(DSA_ERR_SHAPE, "target-only verify: too large");
    const size_t need = dsa::target_only_ws_bytes(B, S, V);
    if (!ws || ws_bytes < need || !aligned16(ws))
        return fail(DSA_ERR_WORKSPACE, "target-only verify: workspace %zu bytes given, %zu needed (16-byte aligned)",
                    ws_bytes, need);
    return hip_status(dsa::launch_target_only(target_logits, draft_tokens, B, S, V, n_accepted, next_token, ws,
                                              (hipStream_t)stream),
                      "mtp_verify_target_only");
}

int dsa_mtp_commit(const int32_t* n_accepted, const int32_t* q_pos_in, const void* new_k_idx, const void* new_kv,
                   void* k_idx_cache, int64_t k_bstride, int k_elem_bytes, void* kv_cache, int64_t kv_bstride,
                   int kv_elem_bytes, int B, int S, int L, int32_t* q_pos_out, void* stream) {
    if (!n_accepted || !q_pos_in || !new_k_idx || !new_kv || !k_idx_cache || !kv_cache || !q_pos_out)
        return fail(DSA_ERR_NULL, "commit: NULL pointer argument");
    if (B < 1 || S < 1 || S > 64 || L < 1) return fail(DSA_ERR_SHAPE, "commit: B=%d S=%d L=%d (1 <= S <= 64)", B, S, L);
    if ((k_elem_bytes != 1 && k_elem_bytes != 2) || (kv_elem_bytes != 1 && kv_elem_bytes != 2))
        return fail(DSA_ERR_UNSUPPORTED, "commit: element sizes %d/%d, supported 1 (E4M3) or 2 (bf16)",
                    k_elem_bytes, kv_elem_bytes);
    if (B > 1 && (k_bstride < (int64_t)L * DSA_INDEX_DIM || kv_bstride < (int64_t)L * DSA_LATENT_DIM))
        return fail(DSA_ERR_SHAPE, "commit: batch strides smaller than L rows");
    if (q_pos_out == q_pos_in) return fail(DSA_ERR_SHAPE, "commit: q_pos_out must not alias q_pos_in");
    if (!aligned16(new_k_idx) || !aligned16(new_kv) || !aligned16(k_idx_cache) || !aligned16(kv_cache) ||
        ((k_bstride * k_elem_bytes) % 16) != 0 || ((kv_bstride * kv_elem_bytes) % 16) != 0)
        return fail(DSA_ERR_ALIGN, "commit: row arrays and caches must be 16-byte aligned, strides in bytes too");
    return hip_status(dsa::launch_mtp_commit(n_accepted, q_pos_in, new_k_idx, new_kv, k_idx_cache,
                                             k_bstride * k_elem_bytes, kv_cache, kv_bstride * kv_elem_bytes, B, S, L,
                                             DSA_INDEX_DIM * k_elem_bytes, DSA_LATENT_DIM * kv_elem_bytes, q_pos_out,
                                             (hipStream_t)stream),
                      "dsa_mtp_commit");
}

}  // extern "C"
