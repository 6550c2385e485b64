"""Shared helpers for the GPU parity tests (marshalling and comparisons only)."""
import numpy as np
import torch

import oracle

DEV = torch.device("cuda:0")
ATTN_TOL = 2e-2     # max|o_gpu - o_ref| <= ATTN_TOL * max|o_ref| (bf16 output, fp32 accumulate)
LSE_TOL = 5e-3      # absolute, natural-log units
VERIFY_SUM_TOL = 2e-6
RATIO_BAND = 1e-5   # relative band around u = p/q where either decision is correct
CDF_BAND = 1e-5     # absolute band around u*sum(r) where either CDF step is correct


def say(msg):
    print(msg, flush=True)


def bf16_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)


def f32_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(DEV)


def i32_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def assert_attn_close(got: np.ndarray, ref: np.ndarray, what=""):
    err = np.abs(got.astype(np.float64) - ref).max()
    scale = np.abs(ref).max()
    assert err <= ATTN_TOL * scale, "%s max err %.4g > %.3g * %.4g" % (what, err, ATTN_TOL, scale)
    return err, scale


def check_topk_properties(idx: np.ndarray, scores: np.ndarray, pos: np.ndarray, k: int):
    """Properties of a correct top-k that hold at any size, checked against the
    scores the same GPU run produced: ascending unique visible positions, the
    right count, nothing better left out, ties resolved towards lower positions."""
    for r in range(idx.shape[0]):
        p = int(pos[r])
        n = min(p + 1, scores.shape[1])
        sel = idx[r][idx[r] >= 0]
        assert sel.size == min(k, n)
        assert np.all(idx[r][sel.size:] == -1)
        assert np.all(np.diff(sel) > 0) and sel[0] >= 0 and sel[-1] <= p
        if n <= k:
            continue
        s = scores[r, :n]
        mask = np.zeros(n, bool)
        mask[sel] = True
        thr = s[mask].min()
        assert s[~mask].max() <= thr
        tied_out = np.nonzero((~mask) & (s == thr))[0]
        tied_in = np.nonzero(mask & (s == thr))[0]
        if tied_out.size:
            assert tied_in.max() < tied_out.min()


def inv_cdf_valid(r: np.ndarray, u: float, v: int) -> bool:
    c = np.cumsum(r)
    thr = u * c[-1]
    if v < 0 or v >= r.size or r[v] <= 0:
        return False
    lo = c[v - 1] if v > 0 else 0.0
    return lo <= thr + CDF_BAND and c[v] > thr - CDF_BAND


def check_verify(min_sum, n_acc, nxt, target, draft, tokens, u_acc, u_res):
    """GPU verification vs the oracle; decisions inside the fp32 ambiguity band
    may go either way, the rest must match exactly."""
    ref = oracle.mtp_verify(target, draft, tokens, u_acc, u_res)
    np.testing.assert_allclose(min_sum, ref["min_sum"], atol=VERIFY_SUM_TOL, rtol=0)
    B, S, V = draft.shape
    for b in range(B):
        ratio = ref["ratio"][b]
        amb = np.abs(u_acc[b] - ratio) <= RATIO_BAND * np.maximum(1.0, ratio)
        acc = u_acc[b] < ratio
        na = int(n_acc[b])
        # every decision up to the GPU's stopping point must be acceptable
        for i in range(na):
            assert acc[i] or amb[i], (b, i, "accepted a clear rejection")
        if na < S:
            assert (not acc[na]) or amb[na], (b, na, "rejected a clear acceptance")
        if na == int(ref["n_acc"][b]) and int(nxt[b]) == int(ref["next_tok"][b]):
            continue
        # different but possibly valid: check the GPU token against its own path's distribution
        if na < S:
            p = oracle.softmax_row(target[b, na])
            q = oracle.softmax_row(draft[b, na])
            r = np.maximum(p - q, 0.0)
        else:
            r = oracle.softmax_row(target[b, S])
        assert inv_cdf_valid(r, float(u_res[b]), int(nxt[b])), (b, na, int(nxt[b]), int(ref["next_tok"][b]))
