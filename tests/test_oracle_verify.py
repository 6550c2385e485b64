"""Pins for the oracle's MTP verification (CPU only).

Sum-min identities, scipy's softmax, and a Monte-Carlo check of the
speculative-sampling theorem: with draft tokens drawn from q, the rule must
accept with probability sum_v min(p_v, q_v) and every emitted token must be
distributed as the target p.  A wrong ratio, a wrong residual or a wrong
bonus distribution fails the chi-square checks."""
import numpy as np
import pytest
from scipy import special, stats

import oracle


def test_softmax_matches_scipy(rng):
    x = (rng.standard_normal(151552) * 2).astype(np.float32)
    np.testing.assert_allclose(oracle.softmax_row(x), special.softmax(x.astype(np.float64)), rtol=1e-12)


def test_min_sum_identities(rng):
    B, S, V = 3, 4, 1000
    t = (rng.standard_normal((B, S + 1, V)) * 2).astype(np.float32)
    d = (rng.standard_normal((B, S, V)) * 2).astype(np.float32)
    tok = rng.integers(0, V, (B, S)).astype(np.int32)
    u = rng.random((B, S)).astype(np.float32)
    ur = rng.random(B).astype(np.float32)
    r = oracle.mtp_verify(t, d, tok, u, ur)
    p = special.softmax(t[:, :S].astype(np.float64), axis=-1)
    q = special.softmax(d.astype(np.float64), axis=-1)
    np.testing.assert_allclose(r["min_sum"], np.minimum(p, q).sum(-1), rtol=1e-12)
    np.testing.assert_allclose(r["min_sum"], 1 - 0.5 * np.abs(p - q).sum(-1), rtol=1e-10)
    np.testing.assert_allclose(r["ratio"], np.take_along_axis(p / q, tok[..., None], -1)[..., 0], rtol=1e-12)
    # identical distributions: sum-min is 1 and every draft is accepted
    r2 = oracle.mtp_verify(np.concatenate([d, t[:, S:]], 1), d, tok, u, ur)
    np.testing.assert_allclose(r2["min_sum"], 1.0, rtol=1e-12)
    assert np.all(r2["n_acc"] == S)


def test_disjoint_supports_give_zero():
    V = 64
    t = np.full((1, 2, V), -1e4, np.float32)
    d = np.full((1, 1, V), -1e4, np.float32)
    t[0, :, : V // 2] = 0.0
    d[0, 0, V // 2:] = 0.0
    r = oracle.mtp_verify(t, d, np.array([[40]], np.int32), np.array([[0.5]], np.float32),
                          np.array([0.3], np.float32))
    assert r["min_sum"][0, 0] == 0.0
    assert r["n_acc"][0] == 0                       # p(x)=0: always rejected
    assert 0 <= r["next_tok"][0] < V // 2            # residual = p, supported on the first half


def _simulate(rng, N, S, V, rho):
    tl = (rng.standard_normal((S + 1, V)) * 1.5).astype(np.float32)
    dl = (rho * tl[:S] + np.sqrt(1 - rho ** 2) * rng.standard_normal((S, V)) * 1.5).astype(np.float32)
    p = special.softmax(tl.astype(np.float64), axis=-1)
    q = special.softmax(dl.astype(np.float64), axis=-1)
    tok = np.stack([rng.choice(V, size=N, p=q[i]) for i in range(S)], 1).astype(np.int32)
    u = rng.random((N, S)).astype(np.float32)
    ur = rng.random(N).astype(np.float32)
    T = np.ascontiguousarray(np.broadcast_to(tl, (N, S + 1, V)))
    D = np.ascontiguousarray(np.broadcast_to(dl, (N, S, V)))
    r = oracle.mtp_verify(T, D, tok, u, ur)
    return p, q, tok, r


def _chi2_ok(samples, probs):
    counts = np.bincount(samples, minlength=probs.size)
    exp = probs * samples.size
    keep = exp > 5
    chi2 = ((counts[keep] - exp[keep]) ** 2 / exp[keep]).sum() + 0.0
    dof = keep.sum() - 1
    return stats.chi2.sf(chi2, dof) > 1e-4, chi2, dof


@pytest.mark.parametrize("rho", [0.0, 0.8])
def test_speculative_sampling_theorem(rng, rho):
    N, S, V = 200_000, 3, 7
    p, q, tok, r = _simulate(rng, N, S, V, rho)
    n_acc, nxt = r["n_acc"], r["next_tok"]
    ms = np.minimum(p[:S], q).sum(-1)
    np.testing.assert_allclose(r["min_sum"][0], ms, rtol=1e-12)
    # acceptance probability of the first draft equals sum-min
    acc0 = (n_acc >= 1).mean()
    assert abs(acc0 - ms[0]) < 5 * np.sqrt(ms[0] * (1 - ms[0]) / N)
    # P(n_acc >= i+1 | n_acc >= i) = sum-min of step i (steps independent here)
    for i in range(1, S):
        sub = n_acc >= i
        rate = (n_acc[sub] >= i + 1).mean()
        assert abs(rate - ms[i]) < 5 * np.sqrt(ms[i] * (1 - ms[i]) / sub.sum())
    # the first emitted token is distributed as p_0
    y0 = np.where(n_acc >= 1, tok[:, 0], nxt)
    ok, chi2, dof = _chi2_ok(y0, p[0])
    assert ok, (chi2, dof)
    # the emitted token at position i, given the first i were accepted, ~ p_i
    for i in range(1, S + 1):
        sub = n_acc >= i
        yi = np.where(n_acc[sub] >= i + 1, tok[sub, i] if i < S else -1, nxt[sub])
        ok, chi2, dof = _chi2_ok(yi, p[i])
        assert ok, (i, chi2, dof)


def test_resample_is_inverse_cdf_of_residual():
    # Hand-built case: p = [.5,.3,.2], q = [.2,.3,.5]; draft token 2 with
    # u=0.9 > p/q = 0.4 is rejected; residual max(p-q,0) = [.3,0,0] -> token 0.
    p = np.array([0.5, 0.3, 0.2])
    q = np.array([0.2, 0.3, 0.5])
    t = np.log(np.stack([p, p]))[None].astype(np.float32)
    d = np.log(q)[None, None].astype(np.float32)
    r = oracle.mtp_verify(t, d, np.array([[2]], np.int32), np.array([[0.9]], np.float32),
                          np.array([0.99], np.float32))
    assert r["n_acc"][0] == 0 and r["next_tok"][0] == 0
    # u=0.3 < 0.4: accepted; then the bonus token is InvCDF(p, u_res):
    # cumsum [.5,.8,1.0] > 0.6 first at index 1
    r = oracle.mtp_verify(t, d, np.array([[2]], np.int32), np.array([[0.3]], np.float32),
                          np.array([0.6], np.float32))
    assert r["n_acc"][0] == 1 and r["next_tok"][0] == 1


def test_out_of_vocabulary_token_is_rejected():
    # A token outside [0, V) has target probability 0: ratio 0, rejected for any u.
    # Hand-built p = [.5,.3,.2], q = [.2,.3,.5]: the residual [.3,0,0] gives token 0.
    p = np.array([0.5, 0.3, 0.2])
    q = np.array([0.2, 0.3, 0.5])
    t = np.log(np.stack([p, p]))[None].astype(np.float32)
    d = np.log(q)[None, None].astype(np.float32)
    for x in (-1, 3, 1 << 20):
        r = oracle.mtp_verify(t, d, np.array([[x]], np.int32), np.array([[1e-6]], np.float32),
                              np.array([0.5], np.float32))
        assert r["ratio"][0, 0] == 0.0 and r["n_acc"][0] == 0 and r["next_tok"][0] == 0, x
    # q == p: the residual has no mass, so the sample comes from p itself;
    # cumsum [.5,.8,1.0] > 0.75 first at index 1
    r = oracle.mtp_verify(t, np.log(p)[None, None].astype(np.float32), np.array([[7]], np.int32),
                          np.array([[0.5]], np.float32), np.array([0.75], np.float32))
    assert r["n_acc"][0] == 0 and r["next_tok"][0] == 1


def test_inverse_cdf_boundary_is_strict():
    # InvCDF takes the smallest v whose cumulative mass is strictly above u*total:
    # p = [.5, .5] and u = .5 lands exactly on the first step, so the answer is 1.
    t = np.zeros((1, 2, 2), np.float32)
    d = np.zeros((1, 1, 2), np.float32)
    r = oracle.mtp_verify(t, d, np.array([[0]], np.int32), np.array([[0.5]], np.float32),
                          np.array([0.5], np.float32))
    assert r["n_acc"][0] == 1 and r["next_tok"][0] == 1
