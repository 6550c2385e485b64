"""CPU oracle for the DSA hot path — TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``liboracle.so`` (plain C,
fp64) with numpy marshalling; it never touches the GPU and shares no code
with the HIP library.  Every function states the page passage it follows
in ``oracle.c``.

Parity status of each function (what pins it, see tests/test_oracle_*.py):
  indexer_scores  pinned: H=1/w=1 reduces to ReLU of a numpy GEMV; all dots
                  non-negative reduces to one numpy matmul; linearity in w;
                  one-hot keys/queries; causal -inf mask.
  topk            pinned: numpy stable argsort on every row (brute force);
                  closed-form special cases (ties, monotone rows, k >= p+1).
  sparse_mla_attn pinned: dense causal attention from torch's CPU
                  scaled_dot_product_attention in fp64 when k >= p+1;
                  one-hot logits; identical rows; permutation invariance.
  layer_group     pinned through its parts plus bitwise reuse of one index
                  list by every layer.
  e4m3_decode     pinned: all 256 codes against torch's float8_e4m3fn
                  dtype; OCP code points (1, 2, 3, 448, 2^-6, 2^-9, NaN, -0).
  indexer_scores (fp8) / sparse_mla_attn (fp8 latent rows)
                  pinned: equal to the bf16 functions on values that both
                  formats hold exactly, plus the bf16 pins above; the E4M3
                  decoding enters only through e4m3_decode's element reads.
  mtp_verify_target_only
                  pinned: numpy argmax brute force, closed-form cases
                  (all drafts the argmax, first-position miss, ties).
  mtp_commit      pinned: numpy slice assignment, untouched rows, capacity.
  mtp_round       composition of the pinned functions above.
  mtp_verify      pinned: sum-min identities (p=q -> 1, disjoint -> 0,
                  1 - TV distance), scipy softmax, Monte-Carlo check of the
                  speculative-sampling theorem (acceptance rate = sum-min,
                  emitted token ~ p).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(HERE, "liboracle.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        p, i32, i64, f64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        L.oracle_indexer_scores.argtypes = [p, p, p, i64, p, i32, i32, i32, i32, i32, p]
        L.oracle_topk.argtypes = [p, p, i32, i32, i32, i32, p]
        L.oracle_sparse_mla_attn.argtypes = [p, p, i64, p, i32, i32, i32, i32, i32, i32, i32, f64, p, p]
        L.oracle_layer_group.argtypes = [p, p, p, i64, p, i32, i32, i32, i32, i32, i32, i32,
                                         p, p, p, i32, i32, i32, f64, i32, i32, p, p, p, p]
        L.oracle_indexer_scores_fp8.argtypes = [p, p, p, i64, p, i32, i32, i32, i32, i32, p]
        L.oracle_sparse_mla_attn_fp8kv.argtypes = [p, p, i64, p, i32, i32, i32, i32, i32, i32, i32, f64, p, p]
        L.oracle_e4m3_decode.argtypes = [p, i64, p]
        L.oracle_mtp_verify_target_only.argtypes = [p, p, i32, i32, i32, p, p]
        L.oracle_mtp_commit.argtypes = [p, p, p, p, p, i64, p, i64, i32, i32, i32, i32, i32, i32, p]
        L.oracle_softmax_row.argtypes = [p, i32, p]
        L.oracle_mtp_verify.argtypes = [p, p, p, p, p, i32, i32, i32, p, p, p, p]
        for fn in ("oracle_indexer_scores", "oracle_topk", "oracle_sparse_mla_attn", "oracle_layer_group",
                   "oracle_softmax_row", "oracle_mtp_verify", "oracle_indexer_scores_fp8",
                   "oracle_sparse_mla_attn_fp8kv", "oracle_e4m3_decode", "oracle_mtp_verify_target_only",
                   "oracle_mtp_commit"):
            getattr(L, fn).restype = None
        _lib = L
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype)
    return a


def _p(a) -> int:
    return a.ctypes.data


def e4m3_decode(codes) -> np.ndarray:
    """OCP E4M3 codes (uint8) -> float64 values (NaN for S.1111.111)."""
    codes = _c(codes, np.uint8)
    out = np.empty(codes.shape, np.float64)
    lib().oracle_e4m3_decode(_p(codes), codes.size, _p(out))
    return out


def indexer_scores(q_idx, w, k_idx, q_pos, L=None, fp8=False) -> np.ndarray:
    """q_idx [B,T,H,D] bf16 bits (uint16), w [B,T,H] f32, k_idx [B,Lk,D] uint16,
    q_pos [B,T] int32 -> scores [B,T,L] f32 (-inf where s > p).
    fp8=True: q_idx and k_idx are E4M3 codes (uint8)."""
    et = np.uint8 if fp8 else np.uint16
    q_idx = _c(q_idx, et)
    w = _c(w, np.float32)
    k_idx = _c(k_idx, et)
    q_pos = _c(q_pos, np.int32)
    B, T, H, D = q_idx.shape
    assert D <= 1024 and k_idx.shape[0] == B and k_idx.shape[2] == D and w.shape == (B, T, H)
    Lk = k_idx.shape[1]
    L = Lk if L is None else L
    assert L <= Lk
    out = np.empty((B, T, L), np.float32)
    fn = lib().oracle_indexer_scores_fp8 if fp8 else lib().oracle_indexer_scores
    fn(_p(q_idx), _p(w), _p(k_idx), Lk * D, _p(q_pos), B, T, L, H, D, _p(out))
    return out


def topk(scores, q_pos, k) -> np.ndarray:
    """scores [B,T,L] f32, q_pos [B,T] -> idx [B,T,k] int32 (ascending, -1 padded)."""
    scores = _c(scores, np.float32)
    q_pos = _c(q_pos, np.int32)
    B, T, L = scores.shape
    out = np.empty((B, T, k), np.int32)
    lib().oracle_topk(_p(scores), _p(q_pos), B, T, L, k, _p(out))
    return out


def sparse_mla_attn(q, kv, idx, sm_scale, Dv=512, L=None, kv_fp8=False):
    """q [B,T,Hq,Dqk] uint16, kv [B,Lk,Dqk] uint16 (E4M3 codes, uint8, when
    kv_fp8), idx [B,T,k] int32 -> (out [B,T,Hq,Dv] f64, lse [B,T,Hq] f64)."""
    q = _c(q, np.uint16)
    kv = _c(kv, np.uint8 if kv_fp8 else np.uint16)
    idx = _c(idx, np.int32)
    B, T, Hq, Dqk = q.shape
    Lk = kv.shape[1]
    L = Lk if L is None else L
    k = idx.shape[2]
    assert kv.shape[0] == B and kv.shape[2] == Dqk and idx.shape[:2] == (B, T)
    out = np.empty((B, T, Hq, Dv), np.float64)
    lse = np.empty((B, T, Hq), np.float64)
    fn = lib().oracle_sparse_mla_attn_fp8kv if kv_fp8 else lib().oracle_sparse_mla_attn
    fn(_p(q), _p(kv), Lk * Dqk, _p(idx), B, T, L, Hq, Dqk, Dv, k, float(sm_scale), _p(out), _p(lse))
    return out, lse


def layer_group(q_idx, w, k_idx, q_pos, k, qs, kvs, sm_scale, Dv=512, idx_fp8=False, kv_fp8=False):
    """One IndexShare group.  qs/kvs: lists (one per layer).  idx_fp8: q_idx
    and k_idx are E4M3 codes; kv_fp8: the latent rows are E4M3 codes.
    Returns (scores, idx, [out_l], [lse_l])."""
    q_idx = _c(q_idx, np.uint8 if idx_fp8 else np.uint16)
    w = _c(w, np.float32)
    k_idx = _c(k_idx, np.uint8 if idx_fp8 else np.uint16)
    q_pos = _c(q_pos, np.int32)
    qs = [_c(q, np.uint16) for q in qs]
    kvs = [_c(kv, np.uint8 if kv_fp8 else np.uint16) for kv in kvs]
    B, T, H, D = q_idx.shape
    L = k_idx.shape[1]
    n = len(qs)
    Hq, Dqk = qs[0].shape[2], qs[0].shape[3]
    scores = np.empty((B, T, L), np.float32)
    idx = np.empty((B, T, k), np.int32)
    outs = [np.empty((B, T, Hq, Dv), np.float64) for _ in range(n)]
    lses = [np.empty((B, T, Hq), np.float64) for _ in range(n)]
    P = ctypes.c_void_p * n
    q_ptrs = P(*[_p(a) for a in qs])
    kv_ptrs = P(*[_p(a) for a in kvs])
    strides = (ctypes.c_int64 * n)(*[a.shape[1] * Dqk for a in kvs])
    out_ptrs = P(*[_p(a) for a in outs])
    lse_ptrs = P(*[_p(a) for a in lses])
    lib().oracle_layer_group(_p(q_idx), _p(w), _p(k_idx), L * D, _p(q_pos), B, T, L, H, D, k, n,
                             ctypes.cast(q_ptrs, ctypes.c_void_p), ctypes.cast(kv_ptrs, ctypes.c_void_p),
                             ctypes.cast(strides, ctypes.c_void_p), Hq, Dqk, Dv, float(sm_scale),
                             int(idx_fp8), int(kv_fp8), _p(scores), _p(idx), ctypes.cast(out_ptrs, ctypes.c_void_p),
                             ctypes.cast(lse_ptrs, ctypes.c_void_p))
    return scores, idx, outs, lses


def softmax_row(logits) -> np.ndarray:
    logits = _c(logits, np.float32)
    out = np.empty(logits.shape[-1], np.float64)
    lib().oracle_softmax_row(_p(logits), logits.shape[-1], _p(out))
    return out


def mtp_verify(target, draft, draft_tokens, u_acc, u_res):
    """target [B,S+1,V] f32, draft [B,S,V] f32, draft_tokens [B,S] int32,
    u_acc [B,S] f32, u_res [B] f32 -> dict(min_sum [B,S] f64, n_acc [B],
    next_tok [B], ratio [B,S] f64 = p(x)/q(x) at each draft token)."""
    target = _c(target, np.float32)
    draft = _c(draft, np.float32)
    draft_tokens = _c(draft_tokens, np.int32)
    u_acc = _c(u_acc, np.float32)
    u_res = _c(u_res, np.float32)
    B, S, V = draft.shape
    assert target.shape == (B, S + 1, V)
    min_sum = np.empty((B, S), np.float64)
    ratio = np.empty((B, S), np.float64)
    n_acc = np.empty(B, np.int32)
    nxt = np.empty(B, np.int32)
    lib().oracle_mtp_verify(_p(target), _p(draft), _p(draft_tokens), _p(u_acc), _p(u_res), B, S, V,
                            _p(min_sum), _p(n_acc), _p(nxt), _p(ratio))
    return {"min_sum": min_sum, "n_acc": n_acc, "next_tok": nxt, "ratio": ratio}


def mtp_verify_target_only(target, draft_tokens):
    """target [B,S+1,V] f32, draft_tokens [B,S] int32 -> (n_acc [B], next_tok [B]):
    drafts kept while each is the target's argmax (lowest index on ties)."""
    target = _c(target, np.float32)
    draft_tokens = _c(draft_tokens, np.int32)
    B, S1, V = target.shape
    S = S1 - 1
    assert draft_tokens.shape == (B, S)
    n_acc = np.empty(B, np.int32)
    nxt = np.empty(B, np.int32)
    lib().oracle_mtp_verify_target_only(_p(target), _p(draft_tokens), B, S, V, _p(n_acc), _p(nxt))
    return n_acc, nxt


def mtp_commit(n_acc, q_pos, new_k, new_kv, k_cache, kv_cache):
    """Append the kept rows in place: new_k [B,S+1,Dk], new_kv [B,S+1,Dv] (same
    element type as the caches k_cache [B,L,Dk], kv_cache [B,L,Dv]); returns
    the next round's positions [B]."""
    n_acc = _c(n_acc, np.int32)
    q_pos = _c(q_pos, np.int32)
    assert k_cache.flags["C_CONTIGUOUS"] and kv_cache.flags["C_CONTIGUOUS"]
    assert new_k.dtype == k_cache.dtype and new_kv.dtype == kv_cache.dtype == k_cache.dtype
    new_k = np.ascontiguousarray(new_k)
    new_kv = np.ascontiguousarray(new_kv)
    B, S1, Dk = new_k.shape
    Dv = new_kv.shape[2]
    L = k_cache.shape[1]
    assert kv_cache.shape[1] == L
    out = np.empty(B, np.int32)
    lib().oracle_mtp_commit(_p(n_acc), _p(q_pos), _p(new_k), _p(new_kv), _p(k_cache), L * Dk, _p(kv_cache),
                            L * Dv, B, S1 - 1, L, Dk, Dv, k_cache.itemsize, _p(out))
    return out


def mtp_round(q_idx, w, k_cache, q_pos, k, q_steps, kv_cache, sm_scale, target, draft, draft_tokens,
              u_acc, u_res, new_k, new_kv, rule="rejection", Dv=512):
    """One multi-token-prediction round, composed from the functions above in
    the order the pages give: the step-1 indexer and top-k over the cache
    (positions 0..q_pos), S draft attention steps that all reuse that list,
    verification of the S drafts (rejection sampling, or the target-only
    rule), and the commit of the kept rows.  Caches are updated in place.
    Returns dict(idx, outs, n_acc, next_tok, q_pos_next)."""
    scores = indexer_scores(q_idx, w, k_cache, q_pos)
    idx = topk(scores, q_pos, k)
    outs = [sparse_mla_attn(q, kv_cache, idx, sm_scale, Dv=Dv)[0] for q in q_steps]
    if rule == "rejection":
        r = mtp_verify(target, draft, draft_tokens, u_acc, u_res)
        n_acc, nxt = r["n_acc"], r["next_tok"]
    else:
        n_acc, nxt = mtp_verify_target_only(target, draft_tokens)
    q_next = mtp_commit(n_acc, q_pos.reshape(-1), new_k, new_kv, k_cache, kv_cache)
    return {"idx": idx, "outs": outs, "n_acc": n_acc, "next_tok": nxt, "q_pos_next": q_next}
