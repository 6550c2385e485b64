"""Seeded synthetic inputs shaped like the DSA hot path's workloads.

Both the HIP path (through the tests and the benchmark) and the CPU oracle
take their inputs from here; nothing in this package computes any step of
the method.  Values come from the counter-based generator in ``synth.c``:
each element is a pure function of (seed, tensor id, flat index), so any
slice can be regenerated alone.

Shapes follow the GLM-5.2 config fields quoted on the architecture teardown
page (clawlihai.cn, sections "DSA" and "MLA"): indexer 32 heads x 128,
top-2048, 512-dim latent KV; the rope width 64 and the 64 attention heads
complete the absorbed-MLA row of 576 values.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass, field

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(HERE, "libsynth.so")
_lib = None

# Tensor ids: one counter stream per logical tensor.
T_Q_IDX = 1
T_W = 2
T_K_IDX = 3
T_Q_ATTN = 16       # + layer
T_KV = 32           # + layer
T_Q_STEPS = 48      # MTP step queries
T_TARGET = 64
T_DRAFT_NOISE = 65
T_DRAFT_TOKENS = 66
T_U_ACC = 67
T_U_RES = 68
T_Q_MTP_IDX = 69
T_W_MTP = 70
T_ROUND = 4096       # + 64 * round + field: per-round inputs of the multi-round loop


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        u64, i64, i32, f32 = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
        p = ctypes.c_void_p
        L.synth_int_bf16.argtypes = [u64, u64, i64, i64, i32, i32, p]
        L.synth_pow2_f32.argtypes = [u64, u64, i64, i64, i32, p]
        L.synth_normal_bf16.argtypes = [u64, u64, i64, i64, p]
        L.synth_normal_f32.argtypes = [u64, u64, i64, i64, f32, p]
        L.synth_mix_f32.argtypes = [u64, u64, i64, i64, p, f32, f32, f32, p]
        L.synth_uniform_f32.argtypes = [u64, u64, i64, i64, p]
        L.synth_raw_u64.argtypes = [u64, u64, i64, i64, p]
        L.synth_gumbel_argmax.argtypes = [u64, u64, p, i64, i64, p]
        L.synth_normal_bf16_rows.argtypes = [u64, u64, p, i64, i64, p]
        L.synth_f32_to_e4m3.argtypes = [p, i64, p]
        L.synth_int_bf16_rows.argtypes = [u64, u64, p, i64, i64, i32, i32, p]
        for fn in ("synth_int_bf16", "synth_pow2_f32", "synth_normal_bf16", "synth_normal_f32",
                   "synth_mix_f32", "synth_uniform_f32", "synth_raw_u64", "synth_gumbel_argmax",
                   "synth_normal_bf16_rows", "synth_int_bf16_rows", "synth_f32_to_e4m3"):
            getattr(L, fn).restype = None
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


# ---------------------------------------------------------------- primitives
def int_bf16(seed, tensor, shape, lo=-3, hi=3, start=0, out=None) -> np.ndarray:
    out = np.empty(shape, np.uint16) if out is None else out
    lib().synth_int_bf16(seed, tensor, start, out.size, lo, hi, _ptr(out))
    return out


def pow2_f32(seed, tensor, shape, kmax=4, start=0) -> np.ndarray:
    out = np.empty(shape, np.float32)
    lib().synth_pow2_f32(seed, tensor, start, out.size, kmax, _ptr(out))
    return out


def normal_bf16(seed, tensor, shape, start=0, out=None) -> np.ndarray:
    out = np.empty(shape, np.uint16) if out is None else out
    lib().synth_normal_bf16(seed, tensor, start, out.size, _ptr(out))
    return out


def normal_f32(seed, tensor, shape, scale=1.0, start=0) -> np.ndarray:
    out = np.empty(shape, np.float32)
    lib().synth_normal_f32(seed, tensor, start, out.size, scale, _ptr(out))
    return out


def mix_f32(seed, tensor, base: np.ndarray, a: float, b: float, scale: float, start=0) -> np.ndarray:
    base = np.ascontiguousarray(base, np.float32)
    out = np.empty(base.shape, np.float32)
    lib().synth_mix_f32(seed, tensor, start, out.size, _ptr(base), a, b, scale, _ptr(out))
    return out


def uniform_f32(seed, tensor, shape, start=0) -> np.ndarray:
    out = np.empty(shape, np.float32)
    lib().synth_uniform_f32(seed, tensor, start, out.size, _ptr(out))
    return out


def raw_u64(seed, tensor, n, start=0) -> np.ndarray:
    out = np.empty(n, np.uint64)
    lib().synth_raw_u64(seed, tensor, start, n, _ptr(out))
    return out


def gumbel_argmax(seed, tensor, logits: np.ndarray) -> np.ndarray:
    logits = np.ascontiguousarray(logits, np.float32)
    V = logits.shape[-1]
    rows = logits.size // V
    out = np.empty(logits.shape[:-1], np.int32)
    lib().synth_gumbel_argmax(seed, tensor, _ptr(logits), rows, V, _ptr(out))
    return out


def normal_bf16_rows(seed, tensor, starts: np.ndarray, rowlen: int) -> np.ndarray:
    starts = np.ascontiguousarray(starts, np.int64)
    out = np.empty((starts.size, rowlen), np.uint16)
    lib().synth_normal_bf16_rows(seed, tensor, _ptr(starts), starts.size, rowlen, _ptr(out))
    return out


def int_bf16_rows(seed, tensor, starts: np.ndarray, rowlen: int, lo=-3, hi=3) -> np.ndarray:
    starts = np.ascontiguousarray(starts, np.int64)
    out = np.empty((starts.size, rowlen), np.uint16)
    lib().synth_int_bf16_rows(seed, tensor, _ptr(starts), starts.size, rowlen, lo, hi, _ptr(out))
    return out


def to_e4m3(x: np.ndarray) -> np.ndarray:
    """fp32 values -> OCP E4M3 codes (uint8), round to nearest even, saturating."""
    x = np.ascontiguousarray(x, np.float32)
    out = np.empty(x.shape, np.uint8)
    lib().synth_f32_to_e4m3(_ptr(x), x.size, _ptr(out))
    return out


def bf16_to_f32(x: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (x.astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- workloads
@dataclass(frozen=True)
class GroupConfig:
    """One 4-layer IndexShare group: indexer + top-k once, attention per layer."""
    name: str
    seed: int
    B: int
    T: int
    L: int
    first_pos: int          # q_pos[b, t] = first_pos + t
    k: int = 2048
    n_layers: int = 4
    H: int = 32             # index_n_heads
    D: int = 128            # index_head_dim
    Hq: int = 64            # attention heads
    Dqk: int = 576          # kv_lora_rank 512 + rope 64
    Dv: int = 512
    sm_scale: float = 1.0 / 16.0   # 1/sqrt(256): 256 dims per head before absorption

    # ---- tensors (host, numpy) ----
    def q_pos(self) -> np.ndarray:
        p = self.first_pos + np.arange(self.T, dtype=np.int32)
        return np.array(np.broadcast_to(p, (self.B, self.T)), np.int32)

    def q_idx(self) -> np.ndarray:
        return int_bf16(self.seed, T_Q_IDX, (self.B, self.T, self.H, self.D))

    def w(self) -> np.ndarray:
        return pow2_f32(self.seed, T_W, (self.B, self.T, self.H))

    def k_idx(self, out=None) -> np.ndarray:
        shape = (self.B, self.L, self.D)
        if out is not None:
            assert out.shape == shape and out.dtype == np.uint16
        return int_bf16(self.seed, T_K_IDX, shape, out=out)

    def k_idx_rows(self, b: int) -> np.ndarray:
        """k_idx[b] alone, [L, D]."""
        return int_bf16(self.seed, T_K_IDX, (self.L, self.D), start=b * self.L * self.D)

    def q_idx_fp8(self) -> np.ndarray:
        """q_idx as OCP E4M3 codes (the integer values are exact in E4M3)."""
        return to_e4m3(bf16_to_f32(self.q_idx()))

    def k_idx_fp8(self) -> np.ndarray:
        return to_e4m3(bf16_to_f32(self.k_idx()))

    def k_idx_rows_fp8(self, b: int) -> np.ndarray:
        return to_e4m3(bf16_to_f32(self.k_idx_rows(b)))

    def q_attn(self, layer: int) -> np.ndarray:
        return normal_bf16(self.seed, T_Q_ATTN + layer, (self.B, self.T, self.Hq, self.Dqk))

    def kv(self, layer: int, out=None) -> np.ndarray:
        shape = (self.B, self.L, self.Dqk)
        if out is not None:
            assert out.shape == shape and out.dtype == np.uint16
        return normal_bf16(self.seed, T_KV + layer, shape, out=out)

    def kv_seq(self, layer: int, b: int) -> np.ndarray:
        """kv[layer][b] alone, [1, L, Dqk]."""
        return normal_bf16(self.seed, T_KV + layer, (1, self.L, self.Dqk), start=b * self.L * self.Dqk)

    def kv_rows(self, layer: int, b: int, rows: np.ndarray) -> np.ndarray:
        """kv[layer][b, rows, :] regenerated without building the cache."""
        rows = np.asarray(rows, np.int64)
        starts = (b * self.L + rows) * self.Dqk
        return normal_bf16_rows(self.seed, T_KV + layer, starts, self.Dqk)

    # FP8 latent cache: the same N(0,1) draws stored as E4M3 codes.
    def kv_fp8(self, layer: int) -> np.ndarray:
        return to_e4m3(bf16_to_f32(self.kv(layer)))

    def kv_seq_fp8(self, layer: int, b: int) -> np.ndarray:
        return to_e4m3(bf16_to_f32(self.kv_seq(layer, b)))

    def kv_rows_fp8(self, layer: int, b: int, rows: np.ndarray) -> np.ndarray:
        return to_e4m3(bf16_to_f32(self.kv_rows(layer, b, rows)))


@dataclass(frozen=True)
class MtpConfig:
    """MTP draft round: step-1 indexer/top-k, S attention steps, verification."""
    name: str
    seed: int
    B: int
    L: int
    S: int = 7
    V: int = 151552
    k: int = 2048
    H: int = 32
    D: int = 128
    Hq: int = 64
    Dqk: int = 576
    Dv: int = 512
    sm_scale: float = 1.0 / 16.0
    rho: float = 0.9        # draft logits = rho*target + sqrt(1-rho^2)*N(0, 2^2)
    logit_std: float = 2.0

    def q_pos(self) -> np.ndarray:
        return np.full((self.B, 1), self.L - 1, np.int32)

    def q_idx(self) -> np.ndarray:
        return int_bf16(self.seed, T_Q_MTP_IDX, (self.B, 1, self.H, self.D))

    def w(self) -> np.ndarray:
        return pow2_f32(self.seed, T_W_MTP, (self.B, 1, self.H))

    def k_idx(self, out=None) -> np.ndarray:
        return int_bf16(self.seed, T_K_IDX, (self.B, self.L, self.D), out=out)

    def k_idx_rows(self, b: int) -> np.ndarray:
        return int_bf16(self.seed, T_K_IDX, (self.L, self.D), start=b * self.L * self.D)

    def kv(self, out=None) -> np.ndarray:
        return normal_bf16(self.seed, T_KV, (self.B, self.L, self.Dqk), out=out)

    def kv_rows(self, b: int, rows: np.ndarray) -> np.ndarray:
        rows = np.asarray(rows, np.int64)
        return normal_bf16_rows(self.seed, T_KV, (b * self.L + rows) * self.Dqk, self.Dqk)

    def q_steps(self) -> np.ndarray:
        """[B, S, Hq, Dqk]: the query of draft step s is q_steps[:, s]."""
        return normal_bf16(self.seed, T_Q_STEPS, (self.B, self.S, self.Hq, self.Dqk))

    def target_logits(self) -> np.ndarray:
        return normal_f32(self.seed, T_TARGET, (self.B, self.S + 1, self.V), scale=self.logit_std)

    def draft_logits(self, target: np.ndarray) -> np.ndarray:
        a = np.float32(self.rho)
        b = np.float32(math.sqrt(max(0.0, 1.0 - self.rho * self.rho)))
        base = np.ascontiguousarray(target[:, : self.S])
        return mix_f32(self.seed, T_DRAFT_NOISE, base, float(a), float(b), self.logit_std)

    def draft_tokens(self, draft: np.ndarray) -> np.ndarray:
        return gumbel_argmax(self.seed, T_DRAFT_TOKENS, draft)

    def u_accept(self) -> np.ndarray:
        return uniform_f32(self.seed, T_U_ACC, (self.B, self.S))

    def u_resample(self) -> np.ndarray:
        return uniform_f32(self.seed, T_U_RES, (self.B,))


@dataclass(frozen=True)
class MtpRoundsConfig:
    """R rounds of draft -> verify -> commit over a cache that starts with L0
    rows per sequence (first query at position L0-1) and has room for every
    row the rounds can keep.  Target logits are N(0, 2^2) with one favoured
    token per position raised by `boost` (so that the target's first choice is
    the favoured token about 70 % of the time at this vocabulary size); draft
    logits are rho*target + sqrt(1-rho^2)*N(0, 2^2); draft tokens are drawn
    from the draft distribution."""
    name: str
    seed: int
    B: int
    L0: int
    R: int = 8
    S: int = 7
    V: int = 151552
    k: int = 2048
    H: int = 32
    D: int = 128
    Hq: int = 64
    Dqk: int = 576
    Dv: int = 512
    sm_scale: float = 1.0 / 16.0
    rho: float = 0.9
    logit_std: float = 2.0
    boost: float = 14.8

    @property
    def L(self) -> int:  # cache capacity: the initial rows plus R*(S+1), in whole 64-row blocks
        return (self.L0 + self.R * (self.S + 1) + 63) // 64 * 64

    def q_pos0(self) -> np.ndarray:
        return np.full(self.B, self.L0 - 1, np.int32)

    def k_idx(self) -> np.ndarray:
        """[B, L, 128]: the first L0 rows of each sequence generated, the rest zero."""
        out = np.zeros((self.B, self.L, self.D), np.uint16)
        for b in range(self.B):
            out[b, : self.L0] = int_bf16(self.seed, T_K_IDX, (self.L0, self.D), start=b * self.L0 * self.D)
        return out

    def kv_seq(self, b: int) -> np.ndarray:
        """[L, 576] of sequence b: L0 generated rows, then zeros."""
        out = np.zeros((self.L, self.Dqk), np.uint16)
        out[: self.L0] = normal_bf16(self.seed, T_KV, (self.L0, self.Dqk), start=b * self.L0 * self.Dqk)
        return out

    def _t(self, r: int, field: int) -> int:
        return T_ROUND + 64 * r + field

    def q_idx(self, r):
        return int_bf16(self.seed, self._t(r, 0), (self.B, 1, self.H, self.D))

    def w(self, r):
        return pow2_f32(self.seed, self._t(r, 1), (self.B, 1, self.H))

    def q_steps(self, r):
        """[B, S, Hq, Dqk]: round r's query of draft step s is q_steps(r)[:, s]."""
        return normal_bf16(self.seed, self._t(r, 2), (self.B, self.S, self.Hq, self.Dqk))

    def target_logits(self, r):
        t = normal_f32(self.seed, self._t(r, 3), (self.B, self.S + 1, self.V), scale=self.logit_std)
        fav = (raw_u64(self.seed, self._t(r, 4), self.B * (self.S + 1)) % np.uint64(self.V)).astype(np.int64)
        flat = t.reshape(-1, self.V)
        flat[np.arange(flat.shape[0]), fav] += np.float32(self.boost)
        return t

    def draft_logits(self, r, target):
        a = np.float32(self.rho)
        b = np.float32(math.sqrt(max(0.0, 1.0 - self.rho * self.rho)))
        return mix_f32(self.seed, self._t(r, 5), np.ascontiguousarray(target[:, : self.S]), float(a), float(b),
                       self.logit_std)

    def draft_tokens(self, r, draft):
        return gumbel_argmax(self.seed, self._t(r, 6), draft)

    def u_accept(self, r):
        return uniform_f32(self.seed, self._t(r, 7), (self.B, self.S))

    def u_resample(self, r):
        return uniform_f32(self.seed, self._t(r, 8), (self.B,))

    def new_k(self, r):
        """[B, S+1, 128]: index-key rows of the positions the verifying pass covers."""
        return int_bf16(self.seed, self._t(r, 9), (self.B, self.S + 1, self.D))

    def new_kv(self, r):
        return normal_bf16(self.seed, self._t(r, 10), (self.B, self.S + 1, self.Dqk))


TINY = GroupConfig("tiny_decode_8k", seed=1, B=1, T=8, L=8192, first_pos=8184)
DECODE_128K = GroupConfig("decode_128k_b32", seed=2, B=32, T=1, L=131072, first_pos=131071)
PREFILL = GroupConfig("prefill_4096_at_128k", seed=3, B=1, T=4096, L=131072, first_pos=126976)
DECODE_1M = GroupConfig("decode_1m_b4", seed=4, B=4, T=1, L=1048576, first_pos=1048575)
MTP = MtpConfig("mtp_draft_b16_128k", seed=5, B=16, L=131072)

MTP_ROUNDS = MtpRoundsConfig("mtp_rounds_b16_128k", seed=6, B=16, L0=131072)

CONFIGS = {c.name: c for c in (TINY, DECODE_128K, PREFILL, DECODE_1M, MTP, MTP_ROUNDS)}


def group_bytes_per_query(cfg: GroupConfig, idx_elem: int = 2, kv_elem: int = 2) -> int:
    """Algorithmic HBM bytes one query token costs in a decode group step:
    the whole index-key scan, the gathered latent rows of every layer, the
    attention queries and outputs, the indexer query/weights and the index
    list.  The score buffer is an implementation detail and is excluded.
    idx_elem / kv_elem: bytes per element of the index and latent caches
    (2 for bf16, 1 for E4M3)."""
    k_scan = cfg.L * cfg.D * idx_elem
    gather = cfg.n_layers * cfg.k * cfg.Dqk * kv_elem
    q_att = cfg.n_layers * cfg.Hq * cfg.Dqk * 2
    out = cfg.n_layers * cfg.Hq * cfg.Dv * 2
    q_idx_w = cfg.H * cfg.D * idx_elem + cfg.H * 4
    idx = cfg.k * 4
    return k_scan + gather + q_att + out + q_idx_w + idx
