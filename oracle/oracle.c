/*
 * CPU oracle for the DSA sparse-attention hot path.  TEST INFRASTRUCTURE ONLY:
 * only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this library.  It shares no code, header or constant with the HIP
 * path and is deliberately plain: scalar loops, fp64 arithmetic, library
 * qsort/exp/log, no blocking or fusion beyond what each definition states.
 *
 * Sources (web pages; cited by title and section):
 *   [TEARDOWN]  "GLM-5.2 开源：读完 1M 上下文的实现原理，你能更懂 AI",
 *               clawlihai.cn/blog/glm-52-1m-architecture-teardown
 *   [MTPBLOG]   GLM-5.2 MTP / IndexShare inference write-up,
 *               4sapi.ai/blog/glm-52-mtp-indexshare-inference
 *   [CTXFR]     "Le contexte d'un million de tokens", glmmodel.cn/fr/context-window
 *   [SPECYUN]   "GLM-5.2 speculative decoding 实测：MTP 接受长度提升 20% 的体感",
 *               yun88.com/news/9578
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - indexer score = sum_h w_h * max(0, q_h . k_s); no scale factor, one
 *     128-dim key per cached token shared by all 32 heads; key s is visible
 *     to a query at absolute position p iff s <= p;
 *   - top-k ties go to the lower position; the chosen positions are emitted
 *     in ascending order and padded with -1 when fewer than k are visible;
 *   - attention values are the first 512 of the 576 latent dims; an index
 *     outside [0, L) is masked; a query with nothing visible outputs zeros;
 *   - verification is standard speculative sampling (accept x with
 *     probability min(1, p(x)/q(x)), on rejection resample from
 *     max(p - q, 0) normalised, after S acceptances sample from the next
 *     target distribution); uniforms are inputs.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC oracle.c -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

int oracle_abi_version(void) { return 2; }

/* bf16 bit pattern -> double: the bf16 value is the top half of an fp32. */
static double bf16_to_double(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* E4M3 code -> double, from the OCP 8-bit floating point definition (the
 * FP8 cache format named in [CTXFR, "Entraînement par renforcement de l'agent
 * intelligent"]): bit 7 sign, bits 6..3 exponent E with bias 7, bits 2..0
 * mantissa M.  E = 0: (-1)^s * (M/8) * 2^-6 (zero and subnormals);
 * E = 1..15: (-1)^s * (1 + M/8) * 2^(E-7), except E = 15, M = 7, which is
 * NaN.  There are no infinities. */
static double e4m3_to_double(uint8_t c) {
    const int s = c >> 7, E = (c >> 3) & 15, M = c & 7;
    if (E == 15 && M == 7) return NAN;
    double mag = (E == 0) ? ldexp((double)M / 8.0, -6) : ldexp(1.0 + (double)M / 8.0, E - 7);
    return s ? -mag : mag;
}

void oracle_e4m3_decode(const uint8_t* codes, int64_t n, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = e4m3_to_double(codes[i]);
}

/* Element i of a cache or query array stored either as bf16 bit patterns
 * (fmt 0) or as E4M3 codes (fmt 1). */
enum { FMT_BF16 = 0, FMT_E4M3 = 1 };
static double elem(const void* base, int64_t i, int fmt) {
    return fmt == FMT_E4M3 ? e4m3_to_double(((const uint8_t*)base)[i]) : bf16_to_double(((const uint16_t*)base)[i]);
}

/* ------------------------------------------------------------------ indexer
 * [TEARDOWN, 刀一 DSA]: before attention, a small indexer with
 * index_n_heads 32 and index_head_dim 128 coarse-screens every history
 * token; [CTXFR, "Attention sparse IndexShare"]: the screen is made of dot
 * products.  For each query (b,t) at position p and each key s <= p:
 *     score[b,t,s] = sum_{h<H} w[b,t,h] * max(0, sum_{d<D} q[b,t,h,d] k[b,s,d])
 * accumulated in fp64 and rounded once to fp32.  Keys s > p get -inf.
 * Layouts: q_idx [B,T,H,D], w [B,T,H], k_idx row s of batch b at
 * k_idx + b*k_bstride + s*D, q_pos [B,T], scores [B,T,L].
 * The FP8 variant reads q_idx and k_idx as E4M3 codes; the arithmetic is the
 * same (the decoded values enter the fp64 sums).
 */
static void indexer_scores_fmt(const void* q_idx, const float* w, const void* k_idx, int64_t k_bstride,
                               const int32_t* q_pos, int B, int T, int L, int H, int D, int fmt, float* scores) {
    for (int b = 0; b < B; ++b) {
        for (int t = 0; t < T; ++t) {
            const int64_t bt = (int64_t)b * T + t;
            const int64_t p = q_pos[bt];
            double* q = (double*)malloc(sizeof(double) * (size_t)H * (size_t)D);
            for (int i = 0; i < H * D; ++i) q[i] = elem(q_idx, bt * H * D + i, fmt);
            float* row = scores + bt * (int64_t)L;
#pragma omp parallel for schedule(static)
            for (int64_t s = 0; s < L; ++s) {
                if (s > p) {
                    row[s] = -INFINITY;
                    continue;
                }
                const int64_t key = (int64_t)b * k_bstride + s * D;
                double kd[1024];
                for (int d = 0; d < D; ++d) kd[d] = elem(k_idx, key + d, fmt);
                double acc = 0.0;
                for (int h = 0; h < H; ++h) {
                    double dot = 0.0;
                    for (int d = 0; d < D; ++d) dot += q[h * D + d] * kd[d];
                    double relu = dot > 0.0 ? dot : 0.0;
                    acc += (double)w[bt * H + h] * relu;
                }
                float f = (float)acc;
                row[s] = (f == 0.0f) ? 0.0f : f; /* one zero: +0 */
            }
            free(q);
        }
    }
}

void oracle_indexer_scores(const uint16_t* q_idx, const float* w, const uint16_t* k_idx, int64_t k_bstride,
                           const int32_t* q_pos, int B, int T, int L, int H, int D, float* scores) {
    indexer_scores_fmt(q_idx, w, k_idx, k_bstride, q_pos, B, T, L, H, D, FMT_BF16, scores);
}

void oracle_indexer_scores_fp8(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, int64_t k_bstride,
                               const int32_t* q_pos, int B, int T, int L, int H, int D, float* scores) {
    indexer_scores_fmt(q_idx, w, k_idx, k_bstride, q_pos, B, T, L, H, D, FMT_E4M3, scores);
}

/* ------------------------------------------------------------------ top-k
 * [TEARDOWN, 刀一 DSA]: index_topk 2048 — keep the 2048 best-scoring
 * history tokens for each query.  Candidates are s in [0, min(p, L-1)].
 * Order them by (score descending, s ascending), keep the first
 * min(k, #candidates), and write the kept positions in ascending order,
 * padding the row with -1 up to k.
 */
typedef struct {
    float score;
    int32_t pos;
} cand_t;

static int cmp_cand(const void* a, const void* b) {
    const cand_t* x = (const cand_t*)a;
    const cand_t* y = (const cand_t*)b;
    if (x->score > y->score) return -1;
    if (x->score < y->score) return 1;
    return (x->pos > y->pos) - (x->pos < y->pos);
}

static int cmp_i32(const void* a, const void* b) {
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x > y) - (x < y);
}

void oracle_topk(const float* scores, const int32_t* q_pos, int B, int T, int L, int k, int32_t* idx) {
#pragma omp parallel for schedule(dynamic)
    for (int64_t bt = 0; bt < (int64_t)B * T; ++bt) {
        int64_t p = q_pos[bt];
        int64_t n = (p < L - 1 ? p : L - 1) + 1;
        if (n < 0) n = 0;
        cand_t* c = (cand_t*)malloc(sizeof(cand_t) * (size_t)(n > 0 ? n : 1));
        for (int64_t s = 0; s < n; ++s) {
            c[s].score = scores[bt * (int64_t)L + s];
            c[s].pos = (int32_t)s;
        }
        qsort(c, (size_t)n, sizeof(cand_t), cmp_cand);
        int64_t m = n < k ? n : k;
        int32_t* out = idx + bt * (int64_t)k;
        for (int64_t j = 0; j < m; ++j) out[j] = c[j].pos;
        qsort(out, (size_t)m, sizeof(int32_t), cmp_i32);
        for (int64_t j = m; j < k; ++j) out[j] = -1;
        free(c);
    }
}

/* ------------------------------------------------------------------ attention
 * [TEARDOWN, 刀一 DSA]: full attention only over the selected tokens;
 * [TEARDOWN, 刀三 MLA]: the cache holds one compressed latent vector per
 * token (kv_lora_rank 512, plus the 64-dim rope part: 576 values), shared by
 * the 64 heads, expanded through learned matrices that the absorbed form
 * folds into the query.  For query (b,t), head h and each valid j
 * (0 <= idx[b,t,j] < L), with c_j the cached row idx[b,t,j] of batch b:
 *     z_j = sm_scale * sum_{d<Dqk} q[b,t,h,d] c_j[d]
 *     out[b,t,h,:] = sum_j softmax(z)_j c_j[0:Dv]
 *     lse[b,t,h]   = log sum_j exp(z_j)            (-inf if no valid j)
 * in fp64.  Layouts: q [B,T,Hq,Dqk], kv row r of batch b at
 * kv + b*kv_bstride + r*Dqk, idx [B,T,k], out [B,T,Hq,Dv], lse [B,T,Hq].
 * The FP8 variant reads the cached rows as E4M3 codes (the query stays bf16).
 */
static void sparse_mla_attn_fmt(const uint16_t* q, const void* kv, int kv_fmt, int64_t kv_bstride,
                                const int32_t* idx, int B, int T, int L, int Hq, int Dqk, int Dv, int k,
                                double sm_scale, double* out, double* lse) {
#pragma omp parallel for schedule(dynamic)
    for (int64_t bt = 0; bt < (int64_t)B * T; ++bt) {
        const int64_t b = bt / T;
        const int32_t* sel = idx + bt * (int64_t)k;
        double* rows = (double*)malloc(sizeof(double) * (size_t)k * (size_t)Dqk);
        double* z = (double*)malloc(sizeof(double) * (size_t)k);
        double* qh = (double*)malloc(sizeof(double) * (size_t)Dqk);
        int nv = 0;
        for (int j = 0; j < k; ++j) {
            int32_t r = sel[j];
            if (r < 0 || r >= L) continue;
            const int64_t src = b * kv_bstride + (int64_t)r * Dqk;
            for (int d = 0; d < Dqk; ++d) rows[(int64_t)nv * Dqk + d] = elem(kv, src + d, kv_fmt);
            ++nv;
        }
        for (int h = 0; h < Hq; ++h) {
            const uint16_t* qsrc = q + (bt * Hq + h) * (int64_t)Dqk;
            for (int d = 0; d < Dqk; ++d) qh[d] = bf16_to_double(qsrc[d]);
            double* o = out + (bt * Hq + h) * (int64_t)Dv;
            if (nv == 0) {
                for (int d = 0; d < Dv; ++d) o[d] = 0.0;
                if (lse) lse[bt * Hq + h] = -INFINITY;
                continue;
            }
            double m = -INFINITY;
            for (int j = 0; j < nv; ++j) {
                double dot = 0.0;
                for (int d = 0; d < Dqk; ++d) dot += qh[d] * rows[(int64_t)j * Dqk + d];
                z[j] = sm_scale * dot;
                if (z[j] > m) m = z[j];
            }
            double den = 0.0;
            for (int j = 0; j < nv; ++j) {
                z[j] = exp(z[j] - m);
                den += z[j];
            }
            for (int d = 0; d < Dv; ++d) {
                double num = 0.0;
                for (int j = 0; j < nv; ++j) num += z[j] * rows[(int64_t)j * Dqk + d];
                o[d] = num / den;
            }
            if (lse) lse[bt * Hq + h] = m + log(den);
        }
        free(rows);
        free(z);
        free(qh);
    }
}

void oracle_sparse_mla_attn(const uint16_t* q, const uint16_t* kv, int64_t kv_bstride, const int32_t* idx,
                            int B, int T, int L, int Hq, int Dqk, int Dv, int k, double sm_scale,
                            double* out, double* lse) {
    sparse_mla_attn_fmt(q, kv, FMT_BF16, kv_bstride, idx, B, T, L, Hq, Dqk, Dv, k, sm_scale, out, lse);
}

void oracle_sparse_mla_attn_fp8kv(const uint16_t* q, const uint8_t* kv, int64_t kv_bstride, const int32_t* idx,
                                  int B, int T, int L, int Hq, int Dqk, int Dv, int k, double sm_scale,
                                  double* out, double* lse) {
    sparse_mla_attn_fmt(q, kv, FMT_E4M3, kv_bstride, idx, B, T, L, Hq, Dqk, Dv, k, sm_scale, out, lse);
}

/* ------------------------------------------------------------------ IndexShare group
 * [TEARDOWN, 刀二 IndexShare] (index_topk_freq 4) and [CTXFR, "Attention
 * sparse IndexShare"]: the indexer sits in the first layer of each group of
 * four; its top-k list is used unchanged by all four layers, so indexer and
 * top-k run once.  scores ([B,T,L]) and idx ([B,T,k]) receive the shared
 * intermediate results; layer l reads q[l], kv[l], kv_bstride[l] and writes
 * out[l], lse[l] (lse[l] may be NULL).
 * idx_fmt / kv_fmt: 0 when q_idx, k_idx / the latent rows are bf16, 1 when
 * they are E4M3 codes.
 */
void oracle_layer_group(const void* q_idx, const float* w, const void* k_idx, int64_t k_bstride,
                        const int32_t* q_pos, int B, int T, int L, int H, int D, int k, int n_layers,
                        const uint16_t* const* q, const void* const* kv, const int64_t* kv_bstride,
                        int Hq, int Dqk, int Dv, double sm_scale, int idx_fmt, int kv_fmt, float* scores,
                        int32_t* idx, double* const* out, double* const* lse) {
    indexer_scores_fmt(q_idx, w, k_idx, k_bstride, q_pos, B, T, L, H, D, idx_fmt, scores);
    oracle_topk(scores, q_pos, B, T, L, k, idx);
    for (int l = 0; l < n_layers; ++l)
        sparse_mla_attn_fmt(q[l], kv[l], kv_fmt, kv_bstride[l], idx, B, T, L, Hq, Dqk, Dv, k, sm_scale, out[l],
                            lse ? lse[l] : NULL);
}

/* ------------------------------------------------------------------ verification
 * [MTPBLOG, "Rejection Sampling"]: for every vocabulary entry take the
 * smaller of the two models' probabilities and sum; the sum is the
 * probability that the draft is accepted.  [MTPBLOG, "MTP"] and [TEARDOWN,
 * 刀四 MTP]: accepted drafts are kept and everything from the first rejected
 * position on is dropped.  The accept/resample rule that realises exactly
 * that acceptance probability is standard speculative sampling (Leviathan,
 * Kalman & Matias 2023; Chen et al. 2023):
 *   p_i = softmax(target[b,i]), q_i = softmax(draft[b,i])      (fp64)
 *   min_sum[b,i] = sum_v min(p_i[v], q_i[v])
 *   for i = 0..S-1: accept x_i = draft_tokens[b,i] iff u_acc[b,i] < p_i(x_i)/q_i(x_i);
 *     at the first rejection: next = InvCDF(max(p_i - q_i, 0), u_res[b]), stop;
 *   if all S accepted: next = InvCDF(p_S, u_res[b]);
 *   n_acc[b] = number accepted.
 * InvCDF(r, u) = the smallest v with sum_{v' <= v} r[v'] > u * sum r.
 * Layouts: target [B,S+1,V], draft [B,S,V], draft_tokens/u_acc/min_sum
 * [B,S], u_res/n_acc/next_tok [B].  ratio (may be NULL) receives
 * p_i(x_i)/q_i(x_i) for every (b,i).
 */
void oracle_softmax_row(const float* logits, int V, double* p) {
    double m = -INFINITY;
    for (int v = 0; v < V; ++v)
        if ((double)logits[v] > m) m = (double)logits[v];
    double s = 0.0;
    for (int v = 0; v < V; ++v) {
        p[v] = exp((double)logits[v] - m);
        s += p[v];
    }
    for (int v = 0; v < V; ++v) p[v] /= s;
}

static int32_t inv_cdf(const double* r, int V, double u) {
    double tot = 0.0;
    int32_t last_pos = -1;
    for (int v = 0; v < V; ++v) {
        tot += r[v];
        if (r[v] > 0.0) last_pos = v;
    }
    double thr = u * tot;
    double c = 0.0;
    for (int v = 0; v < V; ++v) {
        c += r[v];
        if (c > thr) return (int32_t)v;
    }
    return last_pos; /* u*tot rounded up to the total: the last token with mass */
}

void oracle_mtp_verify(const float* target, const float* draft, const int32_t* draft_tokens,
                       const float* u_acc, const float* u_res, int B, int S, int V, double* min_sum,
                       int32_t* n_acc, int32_t* next_tok, double* ratio) {
#pragma omp parallel for schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        double* p = (double*)malloc(sizeof(double) * (size_t)V);
        double* qd = (double*)malloc(sizeof(double) * (size_t)V);
        int rejected_at = -1;
        for (int i = 0; i < S; ++i) {
            oracle_softmax_row(target + ((int64_t)b * (S + 1) + i) * V, V, p);
            oracle_softmax_row(draft + ((int64_t)b * S + i) * V, V, qd);
            double ms = 0.0;
            for (int v = 0; v < V; ++v) ms += p[v] < qd[v] ? p[v] : qd[v];
            min_sum[(int64_t)b * S + i] = ms;
            int32_t x = draft_tokens[(int64_t)b * S + i];
            /* the target distribution has no mass outside the vocabulary: such a token has
               p(x) = 0, ratio 0, and is rejected */
            double rt = (x >= 0 && x < V) ? p[x] / qd[x] : 0.0;
            if (ratio) ratio[(int64_t)b * S + i] = rt;
            if (rejected_at < 0 && !((double)u_acc[(int64_t)b * S + i] < rt)) {
                rejected_at = i;
                for (int v = 0; v < V; ++v) p[v] = p[v] > qd[v] ? p[v] - qd[v] : 0.0;
                double tot = 0.0;
                for (int v = 0; v < V; ++v) tot += p[v];
                if (tot > 0.0) {
                    next_tok[b] = inv_cdf(p, V, (double)u_res[b]);
                } else { /* p == q in fp64: cannot reject in exact arithmetic */
                    oracle_softmax_row(target + ((int64_t)b * (S + 1) + i) * V, V, p);
                    next_tok[b] = inv_cdf(p, V, (double)u_res[b]);
                }
            }
        }
        if (rejected_at < 0) {
            n_acc[b] = S;
            oracle_softmax_row(target + ((int64_t)b * (S + 1) + S) * V, V, p);
            next_tok[b] = inv_cdf(p, V, (double)u_res[b]);
        } else {
            n_acc[b] = rejected_at;
        }
        free(p);
        free(qd);
    }
}

/* ------------------------------------------------------------------ target-only verification
 * [MTPBLOG, "Rejection Sampling"]: the rule that rejection sampling replaced
 * ("Target-Only") keeps a draft token only when it is the target model's own
 * first choice.  Reading: the first choice is the argmax of the target
 * logits (the lowest index among equal maxima); at the first draft that is
 * not, the target's first choice there becomes the next token and the rest
 * is dropped; when all S drafts are kept, the next token is the first choice
 * of the target distribution after the last draft.
 *   n_acc[b] = number of leading i with draft_tokens[b,i] == argmax target[b,i]
 *   next_tok[b] = argmax target[b, n_acc[b]]
 * Layouts: target [B,S+1,V], draft_tokens [B,S], n_acc/next_tok [B].
 */
static int32_t argmax_row(const float* x, int V) {
    int32_t best = 0;
    for (int v = 1; v < V; ++v)
        if (x[v] > x[best]) best = v;
    return best;
}

void oracle_mtp_verify_target_only(const float* target, const int32_t* draft_tokens, int B, int S, int V,
                                   int32_t* n_acc, int32_t* next_tok) {
    for (int b = 0; b < B; ++b) {
        int i = 0;
        while (i < S && draft_tokens[(int64_t)b * S + i] == argmax_row(target + ((int64_t)b * (S + 1) + i) * V, V))
            ++i;
        n_acc[b] = i;
        next_tok[b] = argmax_row(target + ((int64_t)b * (S + 1) + i) * V, V);
    }
}

/* ------------------------------------------------------------------ cache commit after verification
 * [MTPBLOG, "KV Share"]: the draft layers reuse the backbone's cache and
 * only newly produced tokens get new cache rows; [MTPBLOG, "MTP"] and
 * [TEARDOWN, 刀四 MTP]: drafts after the first rejection are dropped and the
 * next round starts from the verified tokens.  Reading: a round starts with
 * the rows of positions 0..q_pos[b] cached (q_pos[b] is the position of the
 * last verified token, whose row is cached).  The verifying pass produces the
 * rows of positions q_pos[b]+1 .. q_pos[b]+S+1 (new_k, new_kv; row j for
 * position q_pos[b]+1+j); the n_acc[b] accepted drafts and the next token are
 * kept, i.e. rows j = 0..n_acc[b], and the next round's position is
 * q_pos[b] + n_acc[b] + 1.  Rows at positions >= L (the cache capacity) are
 * not written and the position stops at L-1.
 * Layouts: new_k [B,S+1,Dk], new_kv [B,S+1,Dv] (any element type of esz
 * bytes), caches with batch strides k_bstride / kv_bstride in elements.
 */
void oracle_mtp_commit(const int32_t* n_acc, const int32_t* q_pos_in, const void* new_k, const void* new_kv,
                       void* k_cache, int64_t k_bstride, void* kv_cache, int64_t kv_bstride, int B, int S, int L,
                       int Dk, int Dv, int esz, int32_t* q_pos_out) {
    for (int b = 0; b < B; ++b) {
        const int64_t p = q_pos_in[b];
        const int n = n_acc[b];
        for (int j = 0; j <= n; ++j) {
            const int64_t pos = p + 1 + j;
            if (pos >= L) break;
            memcpy((char*)k_cache + ((int64_t)b * k_bstride + pos * Dk) * esz,
                   (const char*)new_k + (((int64_t)b * (S + 1) + j) * Dk) * esz, (size_t)Dk * esz);
            memcpy((char*)kv_cache + ((int64_t)b * kv_bstride + pos * Dv) * esz,
                   (const char*)new_kv + (((int64_t)b * (S + 1) + j) * Dv) * esz, (size_t)Dv * esz);
        }
        const int64_t np = p + n + 1;
        q_pos_out[b] = (int32_t)(np < L ? np : L - 1);
    }
}
