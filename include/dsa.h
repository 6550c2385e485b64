/*
 * dsa.h — C ABI of libdsa.so: the DSA sparse-attention hot path on MI355X (gfx950).
 *
 * The method (from the pages cited below): a lightweight indexer scores every
 * cached token for each query, the 2048 best positions are kept, and absorbed
 * MLA attention runs over only those latent rows.  Under IndexShare one index
 * list serves a group of four layers; in the MTP draft path the step-1 list is
 * reused by the later steps and a rejection-sampling check computes the
 * acceptance probability sum_v min(p_v, q_v).
 *
 * Sources (web pages, cited by title and section):
 *   [TEARDOWN]  "GLM-5.2 开源：读完 1M 上下文的实现原理，你能更懂 AI"
 *               (clawlihai.cn/blog/glm-52-1m-architecture-teardown)
 *   [MTPBLOG]   GLM-5.2 MTP / IndexShare inference write-up
 *               (4sapi.ai/blog/glm-52-mtp-indexshare-inference)
 *   [CTXFR]     "Le contexte d'un million de tokens" (glmmodel.cn/fr/context-window)
 *   [SPECYUN]   "GLM-5.2 speculative decoding 实测：MTP 接受长度提升 20% 的体感"
 *               (yun88.com/news/9578)
 *
 * Conventions for every entry point
 *   Memory    Tensor pointers are DEVICE pointers owned by the caller.  The
 *             library never allocates or frees device memory; scratch comes
 *             from the caller's `ws` buffer of at least the size the matching
 *             *_workspace_size() returns (256-byte aligned).  Inner dimensions
 *             are contiguous; batch strides are given in elements.  bf16
 *             values are passed as uint16_t bit patterns.  Pointers and batch
 *             strides must be 16-byte aligned.  Outputs must not alias inputs.
 *   Streams   `stream` is a hipStream_t (NULL = the default stream).  Calls
 *             only enqueue kernels; none synchronises, allocates or memsets,
 *             so a call may be captured in a HIP graph.
 *   Errors    Each call returns DSA_OK (0) or a negative DSA_ERR_* code.  On
 *             error nothing has been enqueued, except DSA_ERR_HIP, which
 *             reports a failed launch.  dsa_last_error() returns a
 *             thread-local description of the last error.  Faults inside a
 *             kernel surface at the caller's next synchronisation.
 *   Positions q_pos[b,t] is the absolute position p of query (b,t); cached
 *             key s is visible to it iff 0 <= s <= p.  p must be < L.
 *   Thread safety  Stateless and re-entrant; concurrent calls must use
 *             distinct workspaces.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_ABI_VERSION 3

/* Shapes fixed by the GLM-5.2 config ([TEARDOWN, 刀一 DSA]: index_n_heads 32,
 * index_head_dim 128, index_topk 2048; [TEARDOWN, 刀三 MLA]: kv_lora_rank
 * 512, 64 heads; the rope width 64 completes the 576-value latent row). */
#define DSA_INDEX_HEADS 32
#define DSA_INDEX_DIM 128
#define DSA_TOPK_MAX 2048
#define DSA_ATTN_HEADS 64
#define DSA_LATENT_DIM 576
#define DSA_VALUE_DIM 512
#define DSA_GROUP_LAYERS_MAX 8
#define DSA_ATTN_CONTEXT_MAX 4194304 /* keys per sequence the indexer and attention kernels address (2^22) */

enum {
    DSA_OK = 0,
    DSA_ERR_NULL = -1,        /* a required pointer is NULL */
    DSA_ERR_SHAPE = -2,       /* a size is out of range or inconsistent */
    DSA_ERR_UNSUPPORTED = -3, /* a head count / dim other than the ones above */
    DSA_ERR_ALIGN = -4,       /* a pointer or stride is not 16-byte aligned */
    DSA_ERR_WORKSPACE = -5,   /* ws is NULL or smaller than required */
    DSA_ERR_HIP = -6          /* the HIP runtime reported a launch error */
};

int dsa_abi_version(void);
const char* dsa_last_error(void);

/* ---------------------------------------------------------------- indexer
 * [TEARDOWN, 刀一 DSA]; [CTXFR, "Attention sparse IndexShare"].
 *   scores[b,t,s] = sum_{h<H} w[b,t,h] * max(0, sum_{d<D} q_idx[b,t,h,d] * k_idx[b,s,d])
 * for s <= q_pos[b,t]; scores[b,t,s] = -inf for s > q_pos[b,t].  bf16 products,
 * fp32 accumulation (exact whenever every partial sum is representable, e.g.
 * small-integer inputs).
 *   q_idx   [B,T,H,D] bf16      w [B,T,H] fp32      q_pos [B,T] int32
 *   k_idx   row s of batch b at k_idx + b*k_bstride + s*D (bf16), s < L
 *   scores  [B,T,L] fp32 (output)
 * H must be 32 and D 128; L <= DSA_ATTN_CONTEXT_MAX.  Needs no workspace. */
int dsa_indexer_scores(const uint16_t* q_idx, const float* w, const uint16_t* k_idx, int64_t k_bstride,
                       const int32_t* q_pos, int B, int T, int L, int H, int D, float* scores, void* stream);

/* ---------------------------------------------------------------- top-k
 * [TEARDOWN, 刀一 DSA] (index_topk 2048).  For each row (b,t) the candidates
 * are s in [0, q_pos[b,t]]; they are ordered by (score descending, s
 * ascending) and the first min(k, q_pos+1) are kept.  idx[b,t,:] receives the
 * kept positions in ascending order, padded with -1 up to k.  Scores are
 * compared as IEEE values (-0 == +0); NaN scores give an unspecified choice.
 *   scores [B,T,L] fp32 (entries beyond q_pos are never read)
 *   idx    [B,T,k] int32 (output)
 * 1 <= k <= 2048. */
size_t dsa_topk_workspace_size(int B, int T, int L, int k);
int dsa_topk(const float* scores, const int32_t* q_pos, int B, int T, int L, int k, int32_t* idx, void* ws,
             size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- sparse MLA attention
 * [TEARDOWN, 刀一 DSA] (full attention over the selected tokens only) and
 * [TEARDOWN, 刀三 MLA] (one compressed latent row per token, shared by all
 * heads).  For query (b,t), head h, and every j with 0 <= idx[b,t,j] < L
 * (other entries are masked and never dereferenced):
 *   z_j = sm_scale * <q[b,t,h,:], c_j>,   c_j = kv row idx[b,t,j] of batch b (Dqk values)
 *   out[b,t,h,:] = sum_j softmax(z)_j * c_j[0:Dv]      (bf16, round-to-nearest-even)
 *   lse[b,t,h]   = ln sum_j exp(z_j)                   (fp32; -inf if no valid j)
 * A query with no valid entry outputs zeros.  bf16 operands, fp32
 * accumulation, online softmax.
 *   q    [B,T,Hq,Dqk] bf16         kv row r of batch b at kv + b*kv_bstride + r*Dqk
 *   idx  [B,T,k] int32             out [B,T,Hq,Dv] bf16      lse [B,T,Hq] fp32 or NULL
 * Hq must be 64, Dqk 576, Dv 512; 1 <= k <= 2048; L <= DSA_ATTN_CONTEXT_MAX. */
size_t dsa_attn_workspace_size(int B, int T, int k);
int dsa_sparse_mla_attn(const uint16_t* q, const uint16_t* kv, int64_t kv_bstride, const int32_t* idx, int B,
                        int T, int L, int Hq, int Dqk, int Dv, int k, float sm_scale, uint16_t* out, float* lse,
                        void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- IndexShare layer group
 * [TEARDOWN, 刀二 IndexShare] (index_topk_freq 4: the indexer sits in the
 * first of four layers and its top-k list is used by all four) and [CTXFR,
 * "Attention sparse IndexShare"].  Runs dsa_indexer_scores and dsa_topk once,
 * writes the shared list to idx_out, then runs dsa_sparse_mla_attn for each
 * layer with that same list, all on `stream`.  Layers stay separate launches:
 * in a model each layer's query depends on the previous layer's output.
 * With share = 0 (ABI version 3) the group runs without IndexShare, as
 * standard DSA does ([MTPBLOG, "Indexer Share：稀疏注意力的缓存复用"]: one
 * indexer per layer): every layer l runs its own indexer and top-k over its
 * own index queries, weights and keys, writes its own list and attends with it.
 * struct_size must be sizeof(dsa_group_args), DSA_GROUP_ARGS_V2_SIZE or
 * DSA_GROUP_ARGS_V1_SIZE; fields added later go at the end, and a shorter
 * struct leaves them NULL / 0 (share = 1).
 *
 * Workspace state: the indexer adds the top-k histogram into the workspace
 * onto what the previous call left there, which every call leaves zero and
 * marked with the shape.  So the workspace carries state from one call to the
 * next: the first call on a workspace, or the first after a call of another
 * shape, finds no mark and counts the histogram again inside the selection
 * (slower, same result); later calls of one shape skip that.  Do not modify
 * the workspace between calls of one shape. */
typedef struct {
    uint32_t struct_size;
    int n_layers;                          /* 1..DSA_GROUP_LAYERS_MAX (4 for a group) */
    int B, T, L, k;
    float sm_scale;
    /* indexer inputs (the group's first layer) */
    const uint16_t* q_idx;                 /* [B,T,32,128] */
    const float* w;                        /* [B,T,32] */
    const uint16_t* k_idx;                 /* rows as in dsa_indexer_scores */
    int64_t k_bstride;
    const int32_t* q_pos;                  /* [B,T] */
    int32_t* idx_out;                      /* [B,T,k] shared index list (output) */
    /* per layer */
    const uint16_t* q[DSA_GROUP_LAYERS_MAX];    /* [B,T,64,576] */
    const uint16_t* kv[DSA_GROUP_LAYERS_MAX];   /* rows as in dsa_sparse_mla_attn */
    int64_t kv_bstride[DSA_GROUP_LAYERS_MAX];
    uint16_t* out[DSA_GROUP_LAYERS_MAX];        /* [B,T,64,512] */
    float* lse[DSA_GROUP_LAYERS_MAX];           /* [B,T,64] or NULL */
    /* ABI version 2: FP8 (E4M3) caches, see "FP8 caches" below.  When
     * q_idx_fp8 and k_idx_fp8 are set, the indexer reads them and q_idx /
     * k_idx must be NULL (k_bstride then counts bytes).  When kv_fp8[l] is
     * set, layer l reads its latent rows there and kv[l] must be NULL
     * (kv_bstride[l] then counts bytes). */
    const uint8_t* q_idx_fp8;                   /* [B,T,32,128] E4M3 */
    const uint8_t* k_idx_fp8;                   /* rows of 128 E4M3 codes */
    const uint8_t* kv_fp8[DSA_GROUP_LAYERS_MAX];  /* rows of 576 E4M3 codes */
    /* ABI version 3: without IndexShare.  share = 1 is IndexShare (the fields
     * below are then ignored).  share = 0: layer l scores with layer_q_idx[l],
     * layer_w[l] and layer_k_idx[l] (bf16; k_bstride as above), or with
     * layer_q_idx_fp8[l] and layer_k_idx_fp8[l] (E4M3) when those are set,
     * selects its own top-k list into layer_idx_out[l] and attends with it;
     * q_idx, w, k_idx, q_idx_fp8, k_idx_fp8 and idx_out are then unused. */
    int share;
    const uint16_t* layer_q_idx[DSA_GROUP_LAYERS_MAX];      /* [B,T,32,128] per layer */
    const float* layer_w[DSA_GROUP_LAYERS_MAX];             /* [B,T,32] per layer */
    const uint16_t* layer_k_idx[DSA_GROUP_LAYERS_MAX];      /* each layer's index-key cache */
    const uint8_t* layer_q_idx_fp8[DSA_GROUP_LAYERS_MAX];
    const uint8_t* layer_k_idx_fp8[DSA_GROUP_LAYERS_MAX];
    int32_t* layer_idx_out[DSA_GROUP_LAYERS_MAX];          /* [B,T,k] per layer (output) */
} dsa_group_args;
/* Sizes of the version-1 struct (no FP8 fields) and of the version-2 struct
 * (no share fields); both are still accepted as struct_size, with the missing
 * fields taken as NULL and share as 1. */
#define DSA_GROUP_ARGS_V1_SIZE offsetof(dsa_group_args, q_idx_fp8)
#define DSA_GROUP_ARGS_V2_SIZE offsetof(dsa_group_args, share)

size_t dsa_layer_group_workspace_size(const dsa_group_args* a);
int dsa_layer_group(const dsa_group_args* a, void* ws, size_t ws_bytes, void* stream);

/* dsa_layer_group_noalloc: for callers that cannot allocate device memory or
 * pass a workspace (code under HIP graph capture that may not call hipMalloc,
 * tight serving loops, harnesses that forbid allocation).  It is
 * dsa_layer_group with the library's own scratch in place of `ws`: a static
 * device array of DSA_NOALLOC_SCRATCH_BYTES on each GPU, kept until the
 * process ends, whose address is looked up once per device on the first call
 * there (the stream must belong to the current device).  The call allocates
 * and frees nothing.  A group whose dsa_layer_group_workspace_size exceeds
 * DSA_NOALLOC_SCRATCH_BYTES is rejected with DSA_ERR_WORKSPACE before any
 * work is enqueued (48 MiB holds decode groups such as 32 queries over 128K
 * rows or 4 over 1M rows; a 4096-query prefill chunk does not fit).  Every
 * call on a GPU shares that GPU's scratch and finds the previous call's
 * contents there, as a workspace keeps them between dsa_layer_group calls
 * (see "Workspace state" above): the first call, and the first after a call
 * of another shape, recount the histogram, so the result never depends on
 * what an earlier call left.  Calls that overlap on one GPU (concurrent
 * streams or host threads) race on the scratch and must not be issued. */
#define DSA_NOALLOC_SCRATCH_BYTES (48u << 20)
int dsa_layer_group_noalloc(const dsa_group_args* a, void* stream);

/* ---------------------------------------------------------------- FP8 caches
 * [CTXFR, "Entraînement par renforcement de l'agent intelligent"] names an FP8
 * KV cache (it keeps rollout memory within budget).  These entry points take
 * OCP E4M3 codes as uint8_t, one byte per element: bit 7 sign, bits 6..3 the
 * exponent with bias 7, bits 2..0 the mantissa; exponent 0 encodes zero and
 * subnormals (M/8 * 2^-6), S.1111.111 is NaN, there are no infinities and the
 * largest finite value is 448.  The layouts, the masking rules and the
 * definitions are those of the bf16 entry points, over the decoded values;
 * strides count elements, which are bytes here, and must be multiples of 16.
 *
 * dsa_indexer_scores_fp8: q_idx and k_idx are E4M3.  The matrix cores form
 * each E4M3 x E4M3 product exactly and add the 32 products of one 32-dim block
 * aligned to the largest of them, keeping about 13 bits below it (smaller
 * contributions are truncated); block sums, heads and weights are then added
 * in fp32.  Scores are therefore exact, and equal to the bf16 entry point's on
 * the same values, whenever every product is a multiple of 2^(e-13), 2^e being
 * the leading power of two of the largest product in its block, and every
 * partial sum is representable (e.g. small-integer inputs); otherwise each
 * block may lose up to 32 * 2^-13 of its largest product. */
int dsa_indexer_scores_fp8(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, int64_t k_bstride,
                           const int32_t* q_pos, int B, int T, int L, int H, int D, float* scores, void* stream);
/* dsa_sparse_mla_attn_fp8kv: the latent rows are E4M3 (576 bytes per row,
 * kv_bstride in bytes); the query stays bf16.  Each gathered row is widened
 * exactly to bf16 (every E4M3 value is a bf16 value), so the result equals
 * dsa_sparse_mla_attn's on rows holding the same values, with the same
 * precision statement.  NaN codes propagate.  Workspace as
 * dsa_attn_workspace_size(B, T, k). */
int dsa_sparse_mla_attn_fp8kv(const uint16_t* q, const uint8_t* kv, int64_t kv_bstride, const int32_t* idx, int B,
                              int T, int L, int Hq, int Dqk, int Dv, int k, float sm_scale, uint16_t* out, float* lse,
                              void* ws, size_t ws_bytes, void* stream);
/* ---------------------------------------------------------------- MTP verification
 * [MTPBLOG, "Rejection Sampling"]: summing min(p_v, q_v) over the vocabulary
 * gives the probability that a draft token is accepted; [MTPBLOG, "MTP"] and
 * [TEARDOWN, 刀四 MTP]: accepted drafts are kept and everything from the first
 * rejection on is dropped.  The rule realising that acceptance probability is
 * standard speculative sampling:
 *   p_i = softmax(target_logits[b,i]),  q_i = softmax(draft_logits[b,i])
 *   min_sum[b,i] = sum_v min(p_i[v], q_i[v])                  (every i < S)
 *   for i = 0..S-1: accept draft_tokens[b,i] = x iff u_accept[b,i] < p_i(x)/q_i(x);
 *     at the first rejection i: next_token[b] = InvCDF(max(p_i - q_i, 0), u_resample[b]);
 *   if all S are accepted: next_token[b] = InvCDF(p_S, u_resample[b]);
 *   n_accepted[b] = number of accepted drafts (acceptance length n_accepted + 1)
 * where InvCDF(r, u) is the smallest v with sum_{v'<=v} r[v'] > u * sum_v r[v].
 * A draft token outside [0, V) has p_i(x) = 0 and is rejected; a residual
 * without mass (p_i == q_i) is replaced by p_i.
 * fp32 exponentials, fp64 sums.  Decisions whose margin is below the fp32
 * resolution of p/q, or a CDF step closer to u*sum r than that resolution,
 * may go either way.
 *   target_logits [B,S+1,V] fp32   draft_logits [B,S,V] fp32
 *   draft_tokens, u_accept [B,S]   u_resample [B]   (uniforms in (0,1))
 *   min_sum [B,S] fp32, n_accepted [B] int32, next_token [B] int32 (outputs) */
size_t mtp_verify_workspace_size(int B, int S, int V);
int mtp_draft_verify(const float* target_logits, const float* draft_logits, const int32_t* draft_tokens,
                     const float* u_accept, const float* u_resample, int B, int S, int V, float* min_sum,
                     int32_t* n_accepted, int32_t* next_token, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- multi-round MTP loop
 * [MTPBLOG, "MTP"] and [TEARDOWN, 刀四 MTP]: generation runs in rounds of
 * draft -> verify -> keep the accepted prefix, the next round starting from
 * the verified tokens.
 *
 * mtp_verify_target_only: the rule rejection sampling replaced ([MTPBLOG,
 * "Rejection Sampling"], "Target-Only"): a draft is kept while it is the
 * target model's first choice,
 *   n_accepted[b] = number of leading i with draft_tokens[b,i] == argmax_v target_logits[b,i,v]
 *   next_token[b] = argmax_v target_logits[b, n_accepted[b], v]
 * with the lowest index among equal maxima.  Logits must be finite.
 *   target_logits [B,S+1,V] fp32, draft_tokens [B,S] int32; n_accepted,
 *   next_token [B] int32 (outputs).  1 <= S <= 64. */
size_t mtp_verify_target_only_workspace_size(int B, int S, int V);
int mtp_verify_target_only(const float* target_logits, const int32_t* draft_tokens, int B, int S, int V,
                           int32_t* n_accepted, int32_t* next_token, void* ws, size_t ws_bytes, void* stream);
/* dsa_mtp_commit: [MTPBLOG, "KV Share"]: the draft layers read the
 * backbone's cache and only new tokens get new cache rows.  A round starts
 * with positions 0..q_pos_in[b] cached; the verifying pass has produced the
 * rows of positions q_pos_in[b]+1 .. q_pos_in[b]+S+1 (new_k_idx, new_kv: row j
 * for position q_pos_in[b]+1+j).  Rows j = 0..n_accepted[b] (the accepted
 * drafts and the next token) are written into the caches, the rest dropped,
 * and q_pos_out[b] = q_pos_in[b] + n_accepted[b] + 1, the position of the next
 * round's first query.  Positions >= L (the capacity) are not written and
 * q_pos_out stops at L-1.  Everything happens on the device: n_accepted is
 * read there, so rounds chain without a host round trip.  q_pos_out must not
 * alias q_pos_in (alternate two buffers).
 *   new_k_idx [B,S+1,128] and k_idx_cache rows of k_elem_bytes (2 bf16, 1 E4M3);
 *   new_kv [B,S+1,576] and kv_cache rows of kv_elem_bytes; strides in elements.
 *   0 <= n_accepted[b] <= S and 0 <= q_pos_in[b] < L are required. */
int dsa_mtp_commit(const int32_t* n_accepted, const int32_t* q_pos_in, const void* new_k_idx, const void* new_kv,
                   void* k_idx_cache, int64_t k_bstride, int k_elem_bytes, void* kv_cache, int64_t kv_bstride,
                   int kv_elem_bytes, int B, int S, int L, int32_t* q_pos_out, void* stream);
#ifdef __cplusplus
}
#endif
#endif /* DSA_H */
