"""Pins for the oracle's indexer scores (CPU only).

The oracle writes the definition out; these tests tie it to things other
than itself: numpy GEMV/GEMM special cases, closed forms on hand-built
inputs, linearity in the head weights and the causal mask."""
import numpy as np
import pytest

import oracle
import synth


def bf16(x):
    """float array of bf16-exact values -> bf16 bit patterns."""
    f = np.asarray(x, np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def test_single_head_is_relu_gemv(rng):
    # H=1, w=1: score = max(0, K q) — a textbook matrix-vector product.
    L, D = 300, 128
    q = rng.integers(-3, 4, size=(1, 1, 1, D)).astype(np.float32)
    k = rng.integers(-3, 4, size=(1, L, D)).astype(np.float32)
    w = np.ones((1, 1, 1), np.float32)
    pos = np.array([[L - 1]], np.int32)
    got = oracle.indexer_scores(bf16(q), w, bf16(k), pos)
    want = np.maximum(k[0] @ q[0, 0, 0], 0.0)
    np.testing.assert_array_equal(got[0, 0], want.astype(np.float32))


def test_nonnegative_inputs_collapse_to_one_gemm(rng):
    # All entries >= 0 => every head dot >= 0, so ReLU is the identity and
    # score = k_s . (sum_h w_h q_h): one numpy matmul, exact for these ints.
    B, T, H, D, L = 2, 3, 32, 128, 257
    q = rng.integers(0, 4, size=(B, T, H, D)).astype(np.float32)
    k = rng.integers(0, 4, size=(B, L, D)).astype(np.float32)
    w = synth.pow2_f32(7, 99, (B, T, H))
    pos = np.full((B, T), L - 1, np.int32)
    got = oracle.indexer_scores(bf16(q), w, bf16(k), pos)
    qw = np.einsum("bth,bthd->btd", w.astype(np.float64), q.astype(np.float64))
    want = np.einsum("bld,btd->btl", k.astype(np.float64), qw)
    np.testing.assert_array_equal(got, want.astype(np.float32))


@pytest.mark.parametrize("c", [-3.0, -1.0, 0.0, 2.0, 3.0])
def test_relu_is_per_head_closed_form(c):
    # q_0 = e_0, q_1 = -e_0, key = c e_0: dots are c and -c, so
    # score = w0*max(c,0) + w1*max(-c,0).  A ReLU taken after the weighted
    # sum, or a dropped head, gives a different value.
    D, H = 128, 2
    q = np.zeros((1, 1, H, D), np.float32)
    q[0, 0, 0, 0] = 1.0
    q[0, 0, 1, 0] = -1.0
    k = np.zeros((1, 1, D), np.float32)
    k[0, 0, 0] = c
    w = np.array([[[0.5, 0.25]]], np.float32)
    got = oracle.indexer_scores(bf16(q), w, bf16(k), np.zeros((1, 1), np.int32))
    assert got[0, 0, 0] == np.float32(0.5 * max(c, 0.0) + 0.25 * max(-c, 0.0))


def test_one_hot_selects_dimension():
    # q_h = a_h e_{d_h}, k_s = b_s e_{e_s}: score = sum over heads with d_h == e_s of w_h*max(0, a_h b_s).
    D, H, L = 128, 4, 6
    q = np.zeros((1, 1, H, D), np.float32)
    dims = [3, 3, 70, 127]
    amps = [2.0, -1.0, 3.0, 1.0]
    for h in range(H):
        q[0, 0, h, dims[h]] = amps[h]
    k = np.zeros((1, L, D), np.float32)
    key_dim = [3, 70, 127, 5, 3, 70]
    key_amp = [1.0, -2.0, 3.0, 1.0, -3.0, 1.0]
    for s in range(L):
        k[0, s, key_dim[s]] = key_amp[s]
    w = np.array([[[1.0, 0.5, 0.25, 0.125]]], np.float32)
    got = oracle.indexer_scores(bf16(q), w, bf16(k), np.array([[L - 1]], np.int32))[0, 0]
    for s in range(L):
        want = sum(w[0, 0, h] * max(0.0, amps[h] * key_amp[s]) for h in range(H) if dims[h] == key_dim[s])
        assert got[s] == np.float32(want), s


def test_linear_in_head_weights(rng):
    B, T, H, D, L = 1, 2, 32, 128, 200
    q = bf16(rng.integers(-3, 4, size=(B, T, H, D)))
    k = bf16(rng.integers(-3, 4, size=(B, L, D)))
    w1 = synth.pow2_f32(1, 1, (B, T, H))
    w2 = synth.pow2_f32(1, 2, (B, T, H))
    pos = np.full((B, T), L - 1, np.int32)
    s1 = oracle.indexer_scores(q, w1, k, pos).astype(np.float64)
    s2 = oracle.indexer_scores(q, w2, k, pos).astype(np.float64)
    s12 = oracle.indexer_scores(q, w1 + w2, k, pos).astype(np.float64)
    np.testing.assert_array_equal(s12, s1 + s2)
    s3 = oracle.indexer_scores(q, 2 * w1, k, pos).astype(np.float64)
    np.testing.assert_array_equal(s3, 2 * s1)


def test_causal_mask_and_grid():
    cfg = synth.TINY
    L = 1024
    q = cfg.q_idx()
    w = cfg.w()
    k = synth.int_bf16(cfg.seed, synth.T_K_IDX, (1, L, cfg.D))
    pos = np.array([[0, 1, 5, 100, 511, 700, 1000, 1023]], np.int32)
    s = oracle.indexer_scores(q, w, k, pos)
    for t in range(8):
        p = pos[0, t]
        assert np.all(np.isneginf(s[0, t, p + 1:]))
        fin = s[0, t, : p + 1]
        assert np.all(np.isfinite(fin)) and np.all(fin >= 0)
        # integer dots times 2^-k weights: every score sits on the 2^-4 grid
        assert np.all(fin * 16 == np.round(fin * 16))
        assert fin.max() <= 32 * 128 * 9


def test_key_batch_stride_uses_each_sequence(rng):
    # Two sequences with different caches: each query must read its own.
    B, T, H, D, L = 2, 1, 32, 128, 64
    q = bf16(np.ones((B, T, H, D)))
    k = np.zeros((B, L, D), np.float32)
    k[0] = 1.0
    k[1] = 2.0
    w = np.ones((B, T, H), np.float32)
    s = oracle.indexer_scores(q, w, bf16(k), np.full((B, T), L - 1, np.int32))
    assert np.all(s[0] == 32 * 128) and np.all(s[1] == 32 * 256)
