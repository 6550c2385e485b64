"""Pins for the oracle's multi-round MTP pieces (CPU only): the target-only
verification rule, the cache commit and one composed round.

Target-only is pinned to numpy's argmax by brute force and to closed-form
cases; the commit to numpy slice assignment; the round to the functions it
is composed of, including that the next round's indexer sees the kept rows."""
import numpy as np
import pytest

import oracle
import synth


def _target_only_numpy(target, draft_tokens):
    B, S1, V = target.shape
    n, nxt = np.zeros(B, np.int32), np.zeros(B, np.int32)
    for b in range(B):
        i = 0
        while i < S1 - 1 and draft_tokens[b, i] == np.argmax(target[b, i]):
            i += 1
        n[b], nxt[b] = i, np.argmax(target[b, i])
    return n, nxt


def test_target_only_matches_numpy_argmax(rng):
    B, S, V = 64, 7, 500
    t = (rng.standard_normal((B, S + 1, V)) * 2).astype(np.float32)
    am = t[:, :S].argmax(-1).astype(np.int32)
    # drafts equal to the argmax with probability 0.7, else another token
    other = (am + rng.integers(1, V, (B, S))) % V
    tok = np.where(rng.random((B, S)) < 0.7, am, other).astype(np.int32)
    n, nxt = oracle.mtp_verify_target_only(t, tok)
    n2, nxt2 = _target_only_numpy(t, tok)
    np.testing.assert_array_equal(n, n2)
    np.testing.assert_array_equal(nxt, nxt2)
    assert len(set(n.tolist())) > 3  # a spread of acceptance lengths


def test_target_only_closed_forms(rng):
    S, V = 7, 100
    t = (rng.standard_normal((2, S + 1, V))).astype(np.float32)
    am = t.argmax(-1).astype(np.int32)
    tok = am[:, :S].copy()
    tok[1, 0] = (tok[1, 0] + 1) % V          # sequence 1 misses at the first draft
    n, nxt = oracle.mtp_verify_target_only(t, tok)
    assert n.tolist() == [S, 0]
    assert nxt.tolist() == [am[0, S], am[1, 0]]


def test_target_only_ties_go_to_the_lowest_index():
    V = 10
    t = np.zeros((1, 2, V), np.float32)
    t[0, 0, [3, 6]] = 5.0                    # two equal maxima: the first choice is 3
    t[0, 1, [2, 8]] = 1.0
    n, nxt = oracle.mtp_verify_target_only(t, np.array([[6]], np.int32))
    assert n[0] == 0 and nxt[0] == 3
    n, nxt = oracle.mtp_verify_target_only(t, np.array([[3]], np.int32))
    assert n[0] == 1 and nxt[0] == 2


def test_rejection_sampling_accepts_identical_distributions_where_target_only_may_not(rng):
    # the two rules differ exactly as the pages describe: with a flat target
    # and a draft drawn from the same distribution, rejection sampling keeps
    # every draft, target-only keeps a draft only when it is the argmax
    B, S, V = 32, 7, 50
    t = (rng.standard_normal((B, S + 1, V)) * 0.1).astype(np.float32)  # flat
    d = t[:, :S].copy()
    tok = np.stack([synth.gumbel_argmax(9, 1, d[b]) for b in range(B)]).astype(np.int32)
    r = oracle.mtp_verify(t, d, tok, rng.random((B, S)).astype(np.float32), rng.random(B).astype(np.float32))
    assert np.all(r["n_acc"] == S)
    n, _ = oracle.mtp_verify_target_only(t, tok)
    n2, _ = _target_only_numpy(t, tok)
    np.testing.assert_array_equal(n, n2)
    assert n.mean() < 1.0


@pytest.mark.parametrize("dtype", [np.uint16, np.uint8])
def test_commit_matches_slice_assignment(rng, dtype):
    B, S, L, Dk, Dv = 3, 7, 64, 128, 576
    k_cache = rng.integers(0, 200, (B, L, Dk)).astype(dtype)
    kv_cache = rng.integers(0, 200, (B, L, Dv)).astype(dtype)
    new_k = rng.integers(0, 200, (B, S + 1, Dk)).astype(dtype)
    new_kv = rng.integers(0, 200, (B, S + 1, Dv)).astype(dtype)
    q_pos = np.array([10, 30, L - 4], np.int32)   # the last one runs into the capacity
    n_acc = np.array([0, 7, 5], np.int32)
    want_k, want_kv = k_cache.copy(), kv_cache.copy()
    for b in range(B):
        for j in range(n_acc[b] + 1):
            pos = q_pos[b] + 1 + j
            if pos < L:
                want_k[b, pos], want_kv[b, pos] = new_k[b, j], new_kv[b, j]
    nxt = oracle.mtp_commit(n_acc, q_pos, new_k, new_kv, k_cache, kv_cache)
    np.testing.assert_array_equal(k_cache, want_k)
    np.testing.assert_array_equal(kv_cache, want_kv)
    assert nxt.tolist() == [11, 38, L - 1]


def test_round_next_indexer_sees_the_kept_rows(rng):
    # after a round, the rows appended at q_pos+1 .. q_pos+n+1 are visible to the
    # next round's step-1 query (at the new position) and can enter its top-k
    B, S, L, k, V = 2, 7, 512, 16, 300
    cfg = synth.GroupConfig("round", seed=8, B=B, T=1, L=L, first_pos=200, k=k)
    k_cache = cfg.k_idx().copy()
    kv_cache = cfg.kv(0).copy()
    q_pos = np.array([[200], [300]], np.int32)
    # make the candidate key rows score above everything cached
    new_k = np.full((B, S + 1, 128), 0x4040, np.uint16)     # 3.0 everywhere
    qi = np.full((B, 1, 32, 128), 0x3F80, np.uint16)        # 1.0 everywhere
    w = np.ones((B, 1, 32), np.float32)
    new_kv = synth.normal_bf16(8, 99, (B, S + 1, 576))
    q_steps = [synth.normal_bf16(8, 50 + i, (B, 1, 64, 576)) for i in range(S)]
    t = (rng.standard_normal((B, S + 1, V)) * 2).astype(np.float32)
    am = t.argmax(-1).astype(np.int32)
    tok = am[:, :S].copy()
    tok[0, 3] = (tok[0, 3] + 1) % V                         # sequence 0 keeps 3 drafts, sequence 1 all 7
    r = oracle.mtp_round(qi, w, k_cache, q_pos, k, q_steps, kv_cache, cfg.sm_scale, t, None, tok, None, None,
                         new_k, new_kv, rule="target_only")
    assert r["n_acc"].tolist() == [3, 7]
    assert r["q_pos_next"].tolist() == [204, 308]
    r2_scores = oracle.indexer_scores(qi, w, k_cache, r["q_pos_next"].reshape(B, 1))
    idx = oracle.topk(r2_scores, r["q_pos_next"].reshape(B, 1), k)
    for b, (p0, n) in enumerate([(200, 3), (300, 7)]):
        kept = set(range(p0 + 1, p0 + n + 2))
        assert kept <= set(idx[b, 0].tolist())
        np.testing.assert_array_equal(kv_cache[b, p0 + 1:p0 + n + 2], new_kv[b, :n + 1])
