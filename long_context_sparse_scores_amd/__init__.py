"""Python binding of libdsa.so — the DSA sparse-attention hot path on MI355X.

Argument marshalling only: every step runs in the HIP kernels of libdsa.so.
Tensors are torch CUDA (ROCm) tensors; bf16 data may be passed as
torch.bfloat16 or as int16/uint16 bit patterns.  Calls enqueue on the
current torch stream of the tensors' device and never synchronise.  The
entry points mirror include/dsa.h one to one; see that header for the
definition of each operation and the page passage it follows.

There is no fallback: if libdsa.so is missing or a call fails, an exception
is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdsa.so")

INDEX_HEADS = 32
INDEX_DIM = 128
TOPK_MAX = 2048
ATTN_HEADS = 64
LATENT_DIM = 576
VALUE_DIM = 512
GROUP_LAYERS_MAX = 8

ERRORS = {0: "DSA_OK", -1: "DSA_ERR_NULL", -2: "DSA_ERR_SHAPE", -3: "DSA_ERR_UNSUPPORTED",
          -4: "DSA_ERR_ALIGN", -5: "DSA_ERR_WORKSPACE", -6: "DSA_ERR_HIP"}


class DsaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("%s (%d): %s" % (ERRORS.get(code, "?"), code, msg))
        self.code = code


_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_F = ctypes.c_float
_SZ = ctypes.c_size_t


class GroupArgs(ctypes.Structure):
    """Mirror of dsa_group_args in include/dsa.h."""
    _fields_ = [
        ("struct_size", ctypes.c_uint32), ("n_layers", _I), ("B", _I), ("T", _I), ("L", _I), ("k", _I),
        ("sm_scale", _F),
        ("q_idx", _P), ("w", _P), ("k_idx", _P), ("k_bstride", _I64), ("q_pos", _P), ("idx_out", _P),
        ("q", _P * GROUP_LAYERS_MAX), ("kv", _P * GROUP_LAYERS_MAX), ("kv_bstride", _I64 * GROUP_LAYERS_MAX),
        ("out", _P * GROUP_LAYERS_MAX), ("lse", _P * GROUP_LAYERS_MAX),
        ("q_idx_fp8", _P), ("k_idx_fp8", _P), ("kv_fp8", _P * GROUP_LAYERS_MAX),
        ("share", _I), ("layer_q_idx", _P * GROUP_LAYERS_MAX), ("layer_w", _P * GROUP_LAYERS_MAX),
        ("layer_k_idx", _P * GROUP_LAYERS_MAX), ("layer_q_idx_fp8", _P * GROUP_LAYERS_MAX),
        ("layer_k_idx_fp8", _P * GROUP_LAYERS_MAX), ("layer_idx_out", _P * GROUP_LAYERS_MAX),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libdsa.so (never builds it; run __graft_entry__.build() first)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libdsa.so not found at %s: build it with __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        L.dsa_abi_version.restype = _I
        L.dsa_abi_version.argtypes = []
        L.dsa_last_error.restype = ctypes.c_char_p
        L.dsa_last_error.argtypes = []
        L.dsa_indexer_scores.restype = _I
        L.dsa_indexer_scores.argtypes = [_P, _P, _P, _I64, _P, _I, _I, _I, _I, _I, _P, _P]
        L.dsa_indexer_scores_fp8.restype = _I
        L.dsa_indexer_scores_fp8.argtypes = [_P, _P, _P, _I64, _P, _I, _I, _I, _I, _I, _P, _P]
        L.dsa_topk_workspace_size.restype = _SZ
        L.dsa_topk_workspace_size.argtypes = [_I, _I, _I, _I]
        L.dsa_topk.restype = _I
        L.dsa_topk.argtypes = [_P, _P, _I, _I, _I, _I, _P, _P, _SZ, _P]
        L.dsa_attn_workspace_size.restype = _SZ
        L.dsa_attn_workspace_size.argtypes = [_I, _I, _I]
        L.dsa_sparse_mla_attn.restype = _I
        L.dsa_sparse_mla_attn.argtypes = [_P, _P, _I64, _P, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P, _SZ, _P]
        L.dsa_sparse_mla_attn_fp8kv.restype = _I
        L.dsa_sparse_mla_attn_fp8kv.argtypes = [_P, _P, _I64, _P, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P, _SZ, _P]
        L.dsa_layer_group_workspace_size.restype = _SZ
        L.dsa_layer_group_workspace_size.argtypes = [ctypes.POINTER(GroupArgs)]
        L.dsa_layer_group.restype = _I
        L.dsa_layer_group.argtypes = [ctypes.POINTER(GroupArgs), _P, _SZ, _P]
        L.dsa_layer_group_noalloc.restype = _I
        L.dsa_layer_group_noalloc.argtypes = [ctypes.POINTER(GroupArgs), _P]
        L.mtp_verify_target_only_workspace_size.restype = _SZ
        L.mtp_verify_target_only_workspace_size.argtypes = [_I, _I, _I]
        L.mtp_verify_target_only.restype = _I
        L.mtp_verify_target_only.argtypes = [_P, _P, _I, _I, _I, _P, _P, _P, _SZ, _P]
        L.dsa_mtp_commit.restype = _I
        L.dsa_mtp_commit.argtypes = [_P, _P, _P, _P, _P, _I64, _I, _P, _I64, _I, _I, _I, _I, _P, _P]
        L.mtp_verify_workspace_size.restype = _SZ
        L.mtp_verify_workspace_size.argtypes = [_I, _I, _I]
        L.mtp_draft_verify.restype = _I
        L.mtp_draft_verify.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _P, _P, _P, _P, _SZ, _P]
        _lib = L
    return _lib


def abi_version() -> int:
    return lib().dsa_abi_version()


def last_error() -> str:
    return lib().dsa_last_error().decode()


def _check(code: int):
    if code != 0:
        raise DsaError(code, last_error())


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _dev(t: torch.Tensor, name: str, dtypes, ndim: Optional[int] = None) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a CUDA tensor" % name)
    if t.dtype not in dtypes:
        raise TypeError("%s has dtype %s, expected one of %s" % (name, t.dtype, dtypes))
    if ndim is not None and t.dim() != ndim:
        raise ValueError("%s must have %d dims, has %d" % (name, ndim, t.dim()))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t.data_ptr()


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_FP8 = (torch.uint8, torch.float8_e4m3fn)   # OCP E4M3 codes


def _workspace(nbytes: int, like: torch.Tensor, ws: Optional[torch.Tensor]) -> torch.Tensor:
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError("workspace too small: %d < %d bytes" % (ws.numel() * ws.element_size(), nbytes))
        return ws
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=like.device)


# ------------------------------------------------------------------ indexer
def indexer_scores(q_idx: torch.Tensor, w: torch.Tensor, k_idx: torch.Tensor, q_pos: torch.Tensor,
                   L: Optional[int] = None, scores: Optional[torch.Tensor] = None) -> torch.Tensor:
    """q_idx [B,T,32,128] bf16, w [B,T,32] f32, k_idx [B,Lc,128] bf16, q_pos [B,T] int32
    -> scores [B,T,L] f32 (dsa_indexer_scores)."""
    B, T, H, D = q_idx.shape
    L = k_idx.shape[1] if L is None else L
    if scores is None:
        scores = torch.empty((B, T, L), dtype=torch.float32, device=q_idx.device)
    _check(lib().dsa_indexer_scores(_dev(q_idx, "q_idx", _BF16, 4), _dev(w, "w", (torch.float32,), 3),
                                    _dev(k_idx, "k_idx", _BF16, 3), k_idx.shape[1] * k_idx.shape[2],
                                    _dev(q_pos, "q_pos", (torch.int32,), 2), B, T, L, H, D,
                                    _dev(scores, "scores", (torch.float32,), 3), _stream(q_idx)))
    return scores


def indexer_scores_fp8(q_idx: torch.Tensor, w: torch.Tensor, k_idx: torch.Tensor, q_pos: torch.Tensor,
                       L: Optional[int] = None, scores: Optional[torch.Tensor] = None) -> torch.Tensor:
    """q_idx [B,T,32,128] E4M3, w [B,T,32] f32, k_idx [B,Lc,128] E4M3, q_pos [B,T] int32
    -> scores [B,T,L] f32 (dsa_indexer_scores_fp8).  E4M3 tensors are uint8 codes
    or torch.float8_e4m3fn."""
    B, T, H, D = q_idx.shape
    L = k_idx.shape[1] if L is None else L
    if scores is None:
        scores = torch.empty((B, T, L), dtype=torch.float32, device=q_idx.device)
    _check(lib().dsa_indexer_scores_fp8(_dev(q_idx, "q_idx", _FP8, 4), _dev(w, "w", (torch.float32,), 3),
                                        _dev(k_idx, "k_idx", _FP8, 3), k_idx.shape[1] * k_idx.shape[2],
                                        _dev(q_pos, "q_pos", (torch.int32,), 2), B, T, L, H, D,
                                        _dev(scores, "scores", (torch.float32,), 3), _stream(q_idx)))
    return scores


# ------------------------------------------------------------------ top-k
def topk_workspace_size(B: int, T: int, L: int, k: int) -> int:
    return lib().dsa_topk_workspace_size(B, T, L, k)


def topk(scores: torch.Tensor, q_pos: torch.Tensor, k: int, idx: Optional[torch.Tensor] = None,
         ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """scores [B,T,L] f32, q_pos [B,T] int32 -> idx [B,T,k] int32 ascending, -1 padded (dsa_topk)."""
    B, T, L = scores.shape
    if idx is None:
        idx = torch.empty((B, T, k), dtype=torch.int32, device=scores.device)
    n = topk_workspace_size(B, T, L, k)
    ws = _workspace(n, scores, ws)
    _check(lib().dsa_topk(_dev(scores, "scores", (torch.float32,), 3), _dev(q_pos, "q_pos", (torch.int32,), 2),
                          B, T, L, k, _dev(idx, "idx", (torch.int32,), 3), ws.data_ptr(),
                          ws.numel() * ws.element_size(), _stream(scores)))
    return idx


# ------------------------------------------------------------------ attention
def attn_workspace_size(B: int, T: int, k: int) -> int:
    return lib().dsa_attn_workspace_size(B, T, k)


def sparse_mla_attn(q: torch.Tensor, kv: torch.Tensor, idx: torch.Tensor, sm_scale: float,
                    L: Optional[int] = None, out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                    want_lse: bool = False, ws: Optional[torch.Tensor] = None):
    """q [B,T,64,576] bf16, kv [B,Lc,576] bf16, idx [B,T,k] int32 -> out [B,T,64,512] bf16
    (and lse [B,T,64] f32 when want_lse or lse is given) (dsa_sparse_mla_attn).
    An E4M3 kv (uint8 codes / float8_e4m3fn) goes to dsa_sparse_mla_attn_fp8kv."""
    B, T, Hq, Dqk = q.shape
    k = idx.shape[2]
    L = kv.shape[1] if L is None else L
    if out is None:
        out = torch.empty((B, T, Hq, VALUE_DIM), dtype=torch.bfloat16, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, T, Hq), dtype=torch.float32, device=q.device)
    n = attn_workspace_size(B, T, k)
    ws = _workspace(n, q, ws)
    if kv.dtype in _FP8:  # E4M3 latent rows
        _check(lib().dsa_sparse_mla_attn_fp8kv(_dev(q, "q", _BF16, 4), _dev(kv, "kv", _FP8, 3),
                                               kv.shape[1] * kv.shape[2], _dev(idx, "idx", (torch.int32,), 3), B, T, L,
                                               Hq, Dqk, VALUE_DIM, k, float(sm_scale), _dev(out, "out", _BF16, 4),
                                               None if lse is None else _dev(lse, "lse", (torch.float32,), 3),
                                               ws.data_ptr(), ws.numel() * ws.element_size(), _stream(q)))
        return (out, lse) if lse is not None else out
    _check(lib().dsa_sparse_mla_attn(_dev(q, "q", _BF16, 4), _dev(kv, "kv", _BF16, 3), kv.shape[1] * kv.shape[2],
                                     _dev(idx, "idx", (torch.int32,), 3), B, T, L, Hq, Dqk, VALUE_DIM, k,
                                     float(sm_scale), _dev(out, "out", _BF16, 4),
                                     None if lse is None else _dev(lse, "lse", (torch.float32,), 3),
                                     ws.data_ptr(), ws.numel() * ws.element_size(), _stream(q)))
    return (out, lse) if lse is not None else out


# ------------------------------------------------------------------ IndexShare group
def make_group_args(q_idx, w, k_idx, q_pos, k: int, qs: Sequence[torch.Tensor], kvs: Sequence[torch.Tensor],
                    sm_scale: float, idx_out, outs: Sequence[torch.Tensor],
                    lses: Optional[Sequence[Optional[torch.Tensor]]] = None) -> GroupArgs:
    """Fill dsa_group_args.  With IndexShare, q_idx, w, k_idx and idx_out are
    tensors; without it (share = 0), they are lists with one tensor per layer."""
    share = isinstance(q_idx, torch.Tensor)
    n = len(qs)
    if not 1 <= n <= GROUP_LAYERS_MAX or len(kvs) != n or len(outs) != n:
        raise ValueError("need 1..%d layers with matching q/kv/out lists" % GROUP_LAYERS_MAX)
    if not share and not (len(q_idx) == len(w) == len(k_idx) == len(idx_out) == n):
        raise ValueError("without IndexShare every layer needs its own q_idx, w, k_idx and idx_out")
    q0, k0 = (q_idx, k_idx) if share else (q_idx[0], k_idx[0])
    B, T, H, D = q0.shape
    L = k0.shape[1]
    a = GroupArgs()
    a.struct_size = ctypes.sizeof(GroupArgs)
    a.n_layers, a.B, a.T, a.L, a.k, a.sm_scale = n, B, T, L, k, float(sm_scale)
    a.share = 1 if share else 0
    a.k_bstride = k0.shape[1] * k0.shape[2]
    a.q_pos = _dev(q_pos, "q_pos", (torch.int32,), 2)
    if share:
        if q_idx.dtype in _FP8:  # E4M3 index queries and keys
            a.q_idx_fp8 = _dev(q_idx, "q_idx", _FP8, 4)
            a.k_idx_fp8 = _dev(k_idx, "k_idx", _FP8, 3)
        else:
            a.q_idx = _dev(q_idx, "q_idx", _BF16, 4)
            a.k_idx = _dev(k_idx, "k_idx", _BF16, 3)
        a.w = _dev(w, "w", (torch.float32,), 3)
        a.idx_out = _dev(idx_out, "idx_out", (torch.int32,), 3)
    else:
        for l in range(n):
            if tuple(k_idx[l].shape) != tuple(k0.shape):
                raise ValueError("every layer's index-key cache must have the shape of layer 0's")
            if q_idx[l].dtype in _FP8:
                a.layer_q_idx_fp8[l] = _dev(q_idx[l], "q_idx[%d]" % l, _FP8, 4)
                a.layer_k_idx_fp8[l] = _dev(k_idx[l], "k_idx[%d]" % l, _FP8, 3)
            else:
                a.layer_q_idx[l] = _dev(q_idx[l], "q_idx[%d]" % l, _BF16, 4)
                a.layer_k_idx[l] = _dev(k_idx[l], "k_idx[%d]" % l, _BF16, 3)
            a.layer_w[l] = _dev(w[l], "w[%d]" % l, (torch.float32,), 3)
            a.layer_idx_out[l] = _dev(idx_out[l], "idx_out[%d]" % l, (torch.int32,), 3)
    for l in range(n):
        a.q[l] = _dev(qs[l], "q[%d]" % l, _BF16, 4)
        if kvs[l].dtype in _FP8:
            a.kv_fp8[l] = _dev(kvs[l], "kv[%d]" % l, _FP8, 3)
        else:
            a.kv[l] = _dev(kvs[l], "kv[%d]" % l, _BF16, 3)
        if kvs[l].shape[1] < L:
            raise ValueError("kv[%d] has %d rows < L=%d" % (l, kvs[l].shape[1], L))
        a.kv_bstride[l] = kvs[l].shape[1] * kvs[l].shape[2]
        a.out[l] = _dev(outs[l], "out[%d]" % l, _BF16, 4)
        if lses is not None and lses[l] is not None:
            a.lse[l] = _dev(lses[l], "lse[%d]" % l, (torch.float32,), 3)
    return a


def layer_group_workspace_size(args: GroupArgs) -> int:
    return lib().dsa_layer_group_workspace_size(ctypes.byref(args))


def layer_group(q_idx, w, k_idx, q_pos, k: int, qs, kvs, sm_scale: float, want_lse: bool = False,
                ws: Optional[torch.Tensor] = None, idx_out=None, outs=None, lses=None):
    """One IndexShare group (dsa_layer_group): indexer and top-k once, then
    attention for every layer with that one index list.  q_idx and k_idx are
    bf16, or both E4M3 (uint8 codes / float8_e4m3fn).  A workspace `ws`
    passed to consecutive calls of one shape lets them skip a recount of the
    top-k histogram (the first call on it recounts).  Returns
    (idx, [out_l], [lse_l] or None)."""
    B, T = q_idx.shape[:2]
    if idx_out is None:
        idx_out = torch.empty((B, T, k), dtype=torch.int32, device=q_idx.device)
    return _run_group(q_idx, w, k_idx, q_pos, k, qs, kvs, sm_scale, want_lse, ws, idx_out, outs, lses)


def layer_group_unshared(q_idx: Sequence[torch.Tensor], w: Sequence[torch.Tensor], k_idx: Sequence[torch.Tensor],
                         q_pos, k: int, qs, kvs, sm_scale: float, want_lse: bool = False,
                         ws: Optional[torch.Tensor] = None, idx_out=None, outs=None, lses=None):
    """The group without IndexShare (dsa_layer_group with share = 0): every
    layer l runs its own indexer and top-k over q_idx[l], w[l], k_idx[l] and
    attends with its own list.  Returns ([idx_l], [out_l], [lse_l] or None)."""
    B, T = q_idx[0].shape[:2]
    if idx_out is None:
        idx_out = [torch.empty((B, T, k), dtype=torch.int32, device=q_idx[0].device) for _ in range(len(qs))]
    return _run_group(list(q_idx), list(w), list(k_idx), q_pos, k, qs, kvs, sm_scale, want_lse, ws, idx_out, outs,
                      lses)


NOALLOC_SCRATCH_BYTES = 48 << 20


def layer_group_noalloc(q_idx, w, k_idx, q_pos, k: int, qs, kvs, sm_scale: float, idx_out: torch.Tensor,
                        outs: Sequence[torch.Tensor], lses=None):
    """The IndexShare group on the library's own per-GPU scratch
    (dsa_layer_group_noalloc): no workspace, nothing allocated by the call.
    The caller passes every output."""
    a = make_group_args(q_idx, w, k_idx, q_pos, k, qs, kvs, sm_scale, idx_out, outs, lses)
    _check(lib().dsa_layer_group_noalloc(ctypes.byref(a), _stream(q_idx)))
    return idx_out, outs, lses


def _run_group(q_idx, w, k_idx, q_pos, k, qs, kvs, sm_scale, want_lse, ws, idx_out, outs, lses):
    q0 = q_idx if isinstance(q_idx, torch.Tensor) else q_idx[0]
    B, T = q0.shape[:2]
    dev = q0.device
    n = len(qs)
    if outs is None:
        outs = [torch.empty((B, T, ATTN_HEADS, VALUE_DIM), dtype=torch.bfloat16, device=dev) for _ in range(n)]
    if lses is None and want_lse:
        lses = [torch.empty((B, T, ATTN_HEADS), dtype=torch.float32, device=dev) for _ in range(n)]
    a = make_group_args(q_idx, w, k_idx, q_pos, k, qs, kvs, sm_scale, idx_out, outs, lses)
    need = layer_group_workspace_size(a)
    if ws is None:
        ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
    ws = _workspace(need, q0, ws)
    _check(lib().dsa_layer_group(ctypes.byref(a), ws.data_ptr(), ws.numel() * ws.element_size(), _stream(q0)))
    return idx_out, outs, lses


# ------------------------------------------------------------------ MTP verification
def verify_workspace_size(B: int, S: int, V: int) -> int:
    return lib().mtp_verify_workspace_size(B, S, V)


def mtp_draft_verify(target: torch.Tensor, draft: torch.Tensor, draft_tokens: torch.Tensor,
                     u_accept: torch.Tensor, u_resample: torch.Tensor, ws: Optional[torch.Tensor] = None):
    """target [B,S+1,V] f32, draft [B,S,V] f32, draft_tokens [B,S] int32, u_accept [B,S] f32,
    u_resample [B] f32 -> (min_sum [B,S] f32, n_accepted [B] int32, next_token [B] int32)."""
    B, S, V = draft.shape
    if tuple(target.shape) != (B, S + 1, V):
        raise ValueError("target must be [B, S+1, V]")
    dev = target.device
    min_sum = torch.empty((B, S), dtype=torch.float32, device=dev)
    n_acc = torch.empty((B,), dtype=torch.int32, device=dev)
    nxt = torch.empty((B,), dtype=torch.int32, device=dev)
    ws = _workspace(verify_workspace_size(B, S, V), target, ws)
    _check(lib().mtp_draft_verify(_dev(target, "target", (torch.float32,), 3), _dev(draft, "draft", (torch.float32,), 3),
                                  _dev(draft_tokens, "draft_tokens", (torch.int32,), 2),
                                  _dev(u_accept, "u_accept", (torch.float32,), 2),
                                  _dev(u_resample, "u_resample", (torch.float32,), 1), B, S, V, min_sum.data_ptr(),
                                  n_acc.data_ptr(), nxt.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(),
                                  _stream(target)))
    return min_sum, n_acc, nxt


# ------------------------------------------------------------------ multi-round MTP loop
def mtp_verify_target_only(target: torch.Tensor, draft_tokens: torch.Tensor, n_acc: Optional[torch.Tensor] = None,
                           next_tok: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None):
    """target [B,S+1,V] f32, draft_tokens [B,S] int32 -> (n_accepted [B], next_token [B]) int32
    (mtp_verify_target_only: drafts kept while each is the target's argmax)."""
    B, S1, V = target.shape
    S = S1 - 1
    dev = target.device
    if n_acc is None:
        n_acc = torch.empty((B,), dtype=torch.int32, device=dev)
    if next_tok is None:
        next_tok = torch.empty((B,), dtype=torch.int32, device=dev)
    ws = _workspace(lib().mtp_verify_target_only_workspace_size(B, S, V), target, ws)
    _check(lib().mtp_verify_target_only(_dev(target, "target", (torch.float32,), 3),
                                        _dev(draft_tokens, "draft_tokens", (torch.int32,), 2), B, S, V,
                                        _dev(n_acc, "n_acc", (torch.int32,), 1),
                                        _dev(next_tok, "next_tok", (torch.int32,), 1), ws.data_ptr(),
                                        ws.numel() * ws.element_size(), _stream(target)))
    return n_acc, next_tok


def _elem_bytes(t: torch.Tensor, name: str) -> int:
    if t.dtype in _FP8:
        return 1
    if t.dtype in _BF16:
        return 2
    raise TypeError("%s has dtype %s: bf16 or E4M3 expected" % (name, t.dtype))


def mtp_commit(n_acc: torch.Tensor, q_pos_in: torch.Tensor, new_k_idx: torch.Tensor, new_kv: torch.Tensor,
               k_idx_cache: torch.Tensor, kv_cache: torch.Tensor, q_pos_out: Optional[torch.Tensor] = None):
    """Keep the rows of the accepted drafts and of the next token (dsa_mtp_commit):
    new_k_idx [B,S+1,128] and new_kv [B,S+1,576] (element types of the caches
    k_idx_cache [B,L,128], kv_cache [B,L,576]) -> q_pos_out [B] int32."""
    B, S1, _ = new_k_idx.shape
    L = k_idx_cache.shape[1]
    if kv_cache.shape[1] != L:
        raise ValueError("the two caches must hold the same number of rows")
    ek, ekv = _elem_bytes(k_idx_cache, "k_idx_cache"), _elem_bytes(kv_cache, "kv_cache")
    if _elem_bytes(new_k_idx, "new_k_idx") != ek or _elem_bytes(new_kv, "new_kv") != ekv:
        raise TypeError("new rows must have the element types of their caches")
    if q_pos_out is None:
        q_pos_out = torch.empty((B,), dtype=torch.int32, device=n_acc.device)
    allt = (torch.uint8, torch.float8_e4m3fn) + _BF16
    _check(lib().dsa_mtp_commit(_dev(n_acc, "n_acc", (torch.int32,), 1), _dev(q_pos_in, "q_pos_in", (torch.int32,)),
                                _dev(new_k_idx, "new_k_idx", allt, 3), _dev(new_kv, "new_kv", allt, 3),
                                _dev(k_idx_cache, "k_idx_cache", allt, 3), L * k_idx_cache.shape[2], ek,
                                _dev(kv_cache, "kv_cache", allt, 3), L * kv_cache.shape[2], ekv, B, S1 - 1, L,
                                _dev(q_pos_out, "q_pos_out", (torch.int32,)), _stream(n_acc)))
    return q_pos_out
