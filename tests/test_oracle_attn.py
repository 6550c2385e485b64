"""Pins for the oracle's sparse absorbed-MLA attention (CPU only).

When every visible position is selected (k >= p+1) sparse attention is
dense causal attention; torch's CPU scaled_dot_product_attention in fp64
is the textbook reference for that.  Other pins: one-hot logits, identical
rows, permutation invariance of the index list, masked entries."""
import numpy as np
import torch

import oracle
import synth

Hq, Dqk, Dv = 64, 576, 512


def f32(u16):
    return synth.bf16_to_f32(u16).astype(np.float64)


def test_dense_causal_equals_sdpa():
    # Sequence of L rows, T queries at positions p_t; k >= L so top-k keeps
    # every visible row: the sparse path must equal dense causal attention.
    B, T, L, k = 2, 3, 40, 64
    scale = 1.0 / 16
    q = synth.normal_bf16(11, 1, (B, T, Hq, Dqk))
    kv = synth.normal_bf16(11, 2, (B, L, Dqk))
    pos = np.array([[5, 20, 39], [0, 1, 39]], np.int32)
    idx = np.full((B, T, k), -1, np.int32)
    for b in range(B):
        for t in range(T):
            idx[b, t, : pos[b, t] + 1] = np.arange(pos[b, t] + 1)
    out, lse = oracle.sparse_mla_attn(q, kv, idx, scale)
    qt = torch.from_numpy(f32(q)).permute(0, 2, 1, 3)             # [B, Hq, T, Dqk]
    K = torch.from_numpy(f32(kv))[:, None].expand(B, Hq, L, Dqk)   # one latent row for all heads
    Vv = torch.from_numpy(f32(kv)[..., :Dv])[:, None].expand(B, Hq, L, Dv)
    mask = torch.from_numpy(np.arange(L)[None, None, None, :] <= pos[:, None, :, None])
    ref = torch.nn.functional.scaled_dot_product_attention(qt, K, Vv, attn_mask=mask, scale=scale)
    ref = ref.permute(0, 2, 1, 3).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)
    logits = np.einsum("bthd,bld->bthl", f32(q), f32(kv)) * scale
    logits = np.where(np.arange(L)[None, None, None, :] <= pos[:, :, None, None], logits, -np.inf)
    ref_lse = np.log(np.exp(logits - logits.max(-1, keepdims=True)).sum(-1)) + logits.max(-1)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12)


def test_one_hot_logit_returns_that_row():
    L, k = 16, 8
    q = np.zeros((1, 1, Hq, Dqk), np.float32)
    q[..., 0] = 64.0
    kv = synth.bf16_to_f32(synth.normal_bf16(3, 3, (1, L, Dqk))).copy()
    kv[..., 0] = 0.0
    kv[0, 9, 0] = 64.0                                 # logit 4096 vs 0: others underflow to 0
    to16 = lambda a: (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    idx = np.array([[[1, 4, 9, 12, -1, 15, 0, 2]]], np.int32)
    out, _ = oracle.sparse_mla_attn(to16(q), to16(kv), idx, 1.0)
    np.testing.assert_array_equal(out[0, 0], np.broadcast_to(kv[0, 9, :Dv].astype(np.float64), (Hq, Dv)))


def test_identical_rows():
    L, k = 32, 16
    row = synth.normal_bf16(4, 4, (Dqk,))
    kv = np.broadcast_to(row, (1, L, Dqk)).copy()
    q = synth.normal_bf16(4, 5, (1, 1, Hq, Dqk))
    idx = np.arange(k, dtype=np.int32)[None, None] * 2
    out, _ = oracle.sparse_mla_attn(q, kv, idx, 1.0 / 16)
    np.testing.assert_allclose(out[0, 0], np.broadcast_to(f32(row)[:Dv], (Hq, Dv)), rtol=1e-14, atol=1e-14)


def test_permutation_invariant_and_masked_entries(rng):
    L, k = 500, 64
    q = synth.normal_bf16(5, 1, (1, 2, Hq, Dqk))
    kv = synth.normal_bf16(5, 2, (1, L, Dqk))
    sel = rng.choice(L, size=(2, 48), replace=False).astype(np.int32)
    idx = np.full((1, 2, k), -1, np.int32)
    idx[0, :, :48] = np.sort(sel, axis=1)
    idx[0, 1, 60] = L + 7          # out of range: masked
    out1, lse1 = oracle.sparse_mla_attn(q, kv, idx, 1.0 / 16)
    perm = idx.copy()
    for t in range(2):
        perm[0, t] = rng.permutation(perm[0, t])
    out2, lse2 = oracle.sparse_mla_attn(q, kv, perm, 1.0 / 16)
    np.testing.assert_allclose(out1, out2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse1, lse2, rtol=1e-13)
    # explicit dense reference over just the chosen rows
    rows = f32(kv)[0, idx[0, 0, :48]]
    z = f32(q)[0, 0] @ rows.T / 16
    pr = np.exp(z - z.max(1, keepdims=True))
    pr /= pr.sum(1, keepdims=True)
    np.testing.assert_allclose(out1[0, 0], pr @ rows[:, :Dv], rtol=1e-11, atol=1e-13)


def test_nothing_visible_gives_zero():
    q = synth.normal_bf16(6, 1, (1, 1, Hq, Dqk))
    kv = synth.normal_bf16(6, 2, (1, 8, Dqk))
    idx = np.full((1, 1, 4), -1, np.int32)
    out, lse = oracle.sparse_mla_attn(q, kv, idx, 1.0 / 16)
    assert np.all(out == 0) and np.all(np.isneginf(lse))
