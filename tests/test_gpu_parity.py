"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs — small cases element by element, ragged shapes and edge
cases.  Bit-exact for scores and indices; attention within 2e-2 of the
output scale; verification exact outside the fp32 ambiguity band."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import (DEV, LSE_TOL, assert_attn_close, bf16_dev, check_topk_properties, check_verify, f32_dev,
                         host, i32_dev, inv_cdf_valid, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    import long_context_sparse_scores_amd as m
    assert torch.cuda.is_available()
    return m


# ------------------------------------------------------------------ indexer
def test_indexer_tiny_bit_exact(dsa):
    cfg = synth.TINY
    say("indexer tiny %s" % cfg.name)
    qi, w, ki, pos = cfg.q_idx(), cfg.w(), cfg.k_idx(), cfg.q_pos()
    got = host(dsa.indexer_scores(bf16_dev(qi), f32_dev(w), bf16_dev(ki), i32_dev(pos)))
    ref = oracle.indexer_scores(qi, w, ki, pos)
    np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_indexer_ragged_strided(dsa):
    B, T, L, Lc = 2, 3, 5000, 5104
    say("indexer ragged B=%d T=%d L=%d Lc=%d" % (B, T, L, Lc))
    qi = synth.int_bf16(31, 1, (B, T, 32, 128))
    w = synth.pow2_f32(31, 2, (B, T, 32))
    ki = synth.int_bf16(31, 3, (B, Lc, 128))
    pos = np.array([[0, 17, 4999], [2500, 4095, 4096]], np.int32)
    got = host(dsa.indexer_scores(bf16_dev(qi), f32_dev(w), bf16_dev(ki), i32_dev(pos), L=L))
    ref = oracle.indexer_scores(qi, w, ki, pos, L=L)
    np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_indexer_multi_query_ragged(dsa):
    # chunks of >= 8 queries take the multi-query path: a partial last group of 16
    # queries, a ragged key tail, a strided cache and positions all over the range
    B, T, L, Lc = 2, 21, 5000, 5104
    say("indexer multi-query B=%d T=%d L=%d" % (B, T, L))
    qi = synth.int_bf16(33, 1, (B, T, 32, 128))
    w = synth.pow2_f32(33, 2, (B, T, 32))
    ki = synth.int_bf16(33, 3, (B, Lc, 128))
    pos = np.stack([np.arange(T, dtype=np.int32) * 211 + 7, np.arange(T, dtype=np.int32) + 4979]).astype(np.int32)
    got = host(dsa.indexer_scores(bf16_dev(qi), f32_dev(w), bf16_dev(ki), i32_dev(pos), L=L))
    ref = oracle.indexer_scores(qi, w, ki, pos, L=L)
    np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("fp8", [False, True])
def test_indexer_multi_query_edges_guarded(dsa, fp8):
    # multi-query path at its edges: a key cache of exactly L rows (the last
    # tile reads past it), a key block of 63 keys, a last query group of 5, a
    # query at position 0 and one at the last key; the scores sit in a larger
    # buffer whose tail must stay untouched
    B, T, L = 2, 37, 4159
    say("indexer multi-query edges fp8=%s B=%d T=%d L=%d" % (fp8, B, T, L))
    qi = synth.int_bf16(34, 1, (B, T, 32, 128))
    w = synth.pow2_f32(34, 2, (B, T, 32))
    ki = synth.int_bf16(34, 3, (B, L, 128))
    pos = np.stack([np.arange(T, dtype=np.int32) * 113, L - T + np.arange(T, dtype=np.int32)]).astype(np.int32)
    guard = torch.full((B * T * L + 4096,), float("nan"), dtype=torch.float32, device=DEV)
    scores = guard[:B * T * L].view(B, T, L)
    if fp8:
        qi, ki = (synth.to_e4m3(synth.bf16_to_f32(a)) for a in (qi, ki))
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.uint8)).to(DEV)
        dsa.indexer_scores_fp8(dev(qi), f32_dev(w), dev(ki), i32_dev(pos), scores=scores)
    else:
        dsa.indexer_scores(bf16_dev(qi), f32_dev(w), bf16_dev(ki), i32_dev(pos), scores=scores)
    got = host(scores)
    ref = oracle.indexer_scores(qi, w, ki, pos, fp8=fp8)
    np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert torch.isnan(guard[B * T * L:]).all().item()


@pytest.mark.parametrize("fp8", [False, True])
def test_indexer_decode_edges_guarded(dsa, fp8):
    # per-query path (T < 8) at its edges: a key cache of exactly L rows whose
    # last block reads past it, a length that is no multiple of the 1024-key
    # blocks or the 16-key tiles, positions 0, in the middle and at the last
    # key; the scores sit in a larger buffer whose tail must stay untouched
    B, T, L = 3, 2, 3 * 1024 + 517
    say("indexer decode edges fp8=%s B=%d T=%d L=%d" % (fp8, B, T, L))
    qi = synth.int_bf16(35, 1, (B, T, 32, 128))
    w = synth.pow2_f32(35, 2, (B, T, 32))
    ki = synth.int_bf16(35, 3, (B, L, 128))
    pos = np.array([[0, L - 1], [1500, 2047], [L - 1, L - 2]], np.int32)
    guard = torch.full((B * T * L + 4096,), float("nan"), dtype=torch.float32, device=DEV)
    scores = guard[:B * T * L].view(B, T, L)
    if fp8:
        qi, ki = (synth.to_e4m3(synth.bf16_to_f32(a)) for a in (qi, ki))
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.uint8)).to(DEV)
        dsa.indexer_scores_fp8(dev(qi), f32_dev(w), dev(ki), i32_dev(pos), scores=scores)
    else:
        dsa.indexer_scores(bf16_dev(qi), f32_dev(w), bf16_dev(ki), i32_dev(pos), scores=scores)
    got = host(scores)
    ref = oracle.indexer_scores(qi, w, ki, pos, fp8=fp8)
    np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert torch.isnan(guard[B * T * L:]).all().item()


def test_indexer_negative_weights(dsa):
    # general weights (not the test distribution): still exact for integer inputs
    B, T, L = 1, 2, 777
    qi = synth.int_bf16(32, 1, (B, T, 32, 128))
    ki = synth.int_bf16(32, 3, (B, L, 128))
    w = (synth.pow2_f32(32, 2, (B, T, 32)) * np.where(np.arange(32) % 3 == 0, -1, 1)).astype(np.float32)
    pos = np.array([[776, 300]], np.int32)
    got = host(dsa.indexer_scores(bf16_dev(qi), f32_dev(w), bf16_dev(ki), i32_dev(pos)))
    ref = oracle.indexer_scores(qi, w, ki, pos)
    np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))


# ------------------------------------------------------------------ top-k
def _topk_case(dsa, scores, pos, k):
    got = host(dsa.topk(f32_dev(scores), i32_dev(pos), k))
    ref = oracle.topk(scores, pos, k)
    np.testing.assert_array_equal(got, ref)


def test_topk_tiny_from_oracle_scores(dsa):
    cfg = synth.TINY
    say("topk tiny")
    scores = oracle.indexer_scores(cfg.q_idx(), cfg.w(), cfg.k_idx(), cfg.q_pos())
    _topk_case(dsa, scores, cfg.q_pos(), cfg.k)


@pytest.mark.parametrize("k", [1, 7, 2048])
def test_topk_tie_heavy_multichunk(dsa, k):
    rng = np.random.default_rng(100 + k)
    B, T, L = 2, 3, 10000
    say("topk ties k=%d" % k)
    scores = (rng.integers(0, 8, size=(B, T, L)) / 16).astype(np.float32)
    pos = np.array([[L - 1, 4096, 8191], [3, 2047, 9000]], np.int32)
    _topk_case(dsa, scores, pos, k)


def test_topk_signed_and_special_values(dsa):
    rng = np.random.default_rng(7)
    B, T, L, k = 1, 4, 9000, 2048
    say("topk signed")
    s = rng.standard_normal((B, T, L)).astype(np.float32)
    s[0, 0, ::5] = -0.0
    s[0, 0, 1::5] = 0.0
    s[0, 1, :] = 1.5                     # all equal
    s[0, 2, ::3] = -np.inf
    s[0, 3] = np.arange(L, dtype=np.float32)  # increasing
    pos = np.array([[L - 1, L - 1, L - 1, L - 1]], np.int32)
    _topk_case(dsa, s, pos, k)


def test_topk_short_rows(dsa):
    rng = np.random.default_rng(8)
    s = rng.standard_normal((1, 3, 3000)).astype(np.float32)
    pos = np.array([[0, 999, 2047]], np.int32)
    say("topk short rows")
    _topk_case(dsa, s, pos, 2048)


def test_topk_candidate_overflow(dsa):
    # a row's candidate list (keys whose top digit is the threshold's or
    # above) holds max(4096, L/8) entries; fully tied rows overflow it and are
    # selected from the whole row instead
    rng = np.random.default_rng(13)
    B, T, L = 1, 4, 40000
    say("topk candidate overflow")
    s = rng.standard_normal((B, T, L)).astype(np.float32)
    s[0, 0] = 2.0                                                          # 40000 tied candidates
    s[0, 1] = np.where(rng.random(L) < 0.5, 1.0, 1.25).astype(np.float32)  # two values
    s[0, 2, ::2] = -0.0
    pos = np.array([[L - 1, L - 1, 30000, 20000]], np.int32)
    _topk_case(dsa, s, pos, 2048)


@pytest.mark.parametrize("n_tied", [11, 100])
def test_topk_ties_straddling_cut(dsa, n_tied):
    # distinct scores, except n_tied keys equal to the one ranked 2045th: only
    # the lowest positions among them are kept (a wave ranks up to 64 ties;
    # more go through the radix passes over positions)
    rng = np.random.default_rng(16 + n_tied)
    B, T, L, k = 1, 2, 30000, 2048
    say("topk %d ties straddling the cut" % n_tied)
    s = rng.permutation(L).astype(np.float32)[None, None].repeat(T, 1) / 7.0
    for t in range(T):
        order = np.argsort(-s[0, t], kind="stable")
        v = s[0, t, order[k - 4]]
        s[0, t, rng.choice(order[k + 500:], n_tied - 1, replace=False)] = v
    pos = np.array([[L - 1, 25000]], np.int32)
    _topk_case(dsa, s, pos, k)


def test_topk_candidates_beyond_lds(dsa):
    # 14000 keys share the threshold's top digit: more candidates than the
    # selection holds in LDS (12288), fewer than the list's capacity (L/8 = 16384)
    rng = np.random.default_rng(15)
    B, T, L, n_hot = 1, 3, 131072, 14000
    say("topk candidate list read from memory")
    s = (rng.standard_normal((B, T, L)) * 0.1).astype(np.float32)
    hot = rng.choice(L, n_hot, replace=False)
    s[0, 0, hot] = (1.0 + 0.2 * rng.random(n_hot)).astype(np.float32)                   # distinct
    s[0, 1, hot] = (1.0 + rng.integers(0, 16, n_hot) / 128).astype(np.float32)          # ties straddle K*
    s[0, 2, hot] = 1.125                                                                 # all tied
    pos = np.array([[L - 1, L - 1, 120000]], np.int32)
    _topk_case(dsa, s, pos, 2048)


def test_topk_candidates_clustered_in_slices(dsa):
    # Up to 256 rows are cut into slices of 16384 keys (8 per 128K row), each
    # with a region of L/8/8 = 2048 candidates and a first read of 12288/8 = 1536
    # per region by the selecting workgroup.  Candidates bunched in one slice:
    # more than that first read (row 0), more than the region (row 1, its
    # slice's scores are read again), spread over three slices (row 2), and
    # a ragged row whose last active slice is short (row 3).
    rng = np.random.default_rng(17)
    B, T, L = 1, 4, 131072
    say("topk candidates clustered in slices")
    s = (rng.random((B, T, L)) * 0.5).astype(np.float32)
    s[0, 0, 7 * 16384 + rng.choice(16384, 1800, replace=False)] = (4.0 + rng.random(1800)).astype(np.float32)
    s[0, 1, 3 * 16384 + rng.choice(16384, 2500, replace=False)] = (4.0 + rng.random(2500)).astype(np.float32)
    for sl in (1, 4, 6):
        s[0, 2, sl * 16384 + rng.choice(16384, 600, replace=False)] = (4.0 + rng.random(600)).astype(np.float32)
    s[0, 3, 100000 + rng.choice(3000, 1700, replace=False)] = (4.0 + rng.random(1700)).astype(np.float32)
    pos = np.array([[L - 1, L - 1, L - 1, 103000]], np.int32)
    _topk_case(dsa, s, pos, 1500)


@pytest.mark.parametrize("L", [262144, 262145])
def test_topk_long_rows(dsa, L):
    rng = np.random.default_rng(L)
    say("topk L=%d" % L)
    s = (rng.integers(0, 64, size=(1, 2, L)) / 8).astype(np.float32)
    pos = np.array([[L - 1, 100000]], np.int32)
    _topk_case(dsa, s, pos, 2048)


def test_topk_long_slices(dsa):
    # 512 rows of 66000 keys: one slice per row, long enough for the fine-bin
    # histogram; clustered values (few top-digit bins), ties and ragged rows.
    # The oracle checks a sample of the rows.
    rng = np.random.default_rng(16)
    B, T, L = 1, 512, 66000
    say("topk %d rows x %d (fine-bin histogram)" % (T, L))
    s = (1.0 + rng.integers(0, 4096, size=(B, T, L)) / 1024).astype(np.float32)
    s[0, 1::5] = (2.0 + rng.integers(0, 3, size=(T // 5 + 1, L))[: len(range(1, T, 5))]).astype(np.float32)
    pos = np.full((B, T), L - 1, np.int32)
    pos[0, ::7] = rng.integers(1000, L, size=len(range(0, T, 7)))
    got = host(dsa.topk(f32_dev(s), i32_dev(pos), 2048))
    rows = np.array([0, 1, 2, 6, 7, 11, 100, 255, 256, 301, 510, 511])
    ref = oracle.topk(s[:, rows], pos[:, rows], 2048)
    np.testing.assert_array_equal(got[:, rows], ref)


def test_topk_many_rows(dsa):
    # 600 rows of ragged visible lengths, tied rows overflowing the candidate list
    rng = np.random.default_rng(14)
    B, T, L = 1, 600, 5000
    say("topk %d rows" % (B * T))
    s = (rng.integers(0, 16, size=(B, T, L)) / 4).astype(np.float32)
    s[0, ::7] = 3.0
    pos = (np.arange(T, dtype=np.int32) * 37 % L)[None]
    pos[0, :5] = L - 1
    _topk_case(dsa, s, pos, 1000)


@pytest.mark.parametrize("L", [4098, 4099])
def test_topk_many_rows_key_loads(dsa, L):
    # 300 ragged rows on the many-row path with a length that is not a
    # multiple of 4: rows then do not all start 16-byte aligned, and the
    # streaming passes load one key per lane instead of four
    rng = np.random.default_rng(L)
    B, T = 1, 300
    say("topk %d rows of %d keys" % (T, L))
    s = (rng.integers(0, 64, size=(B, T, L)) / 8).astype(np.float32)
    s[0, ::11] = 5.0
    pos = ((np.arange(T, dtype=np.int32) * 53 + 2100) % L)[None]
    pos[0, :3] = L - 1
    _topk_case(dsa, s, pos, 2048)


# ------------------------------------------------------------------ attention
def test_attn_tiny_layers(dsa):
    cfg = synth.TINY
    say("attn tiny")
    scores = oracle.indexer_scores(cfg.q_idx(), cfg.w(), cfg.k_idx(), cfg.q_pos())
    idx = oracle.topk(scores, cfg.q_pos(), cfg.k)
    for l in range(2):
        q, kv = cfg.q_attn(l), cfg.kv(l)
        out, lse = dsa.sparse_mla_attn(bf16_dev(q), bf16_dev(kv), i32_dev(idx), cfg.sm_scale, want_lse=True)
        ref, ref_lse = oracle.sparse_mla_attn(q, kv, idx, cfg.sm_scale)
        assert_attn_close(host(out), ref, "layer %d" % l)
        np.testing.assert_allclose(host(lse), ref_lse, atol=LSE_TOL, rtol=0)


def test_attn_masked_ragged(dsa):
    rng = np.random.default_rng(9)
    B, T, L, k = 2, 2, 3000, 100
    say("attn masked ragged")
    q = synth.normal_bf16(41, 1, (B, T, 64, 576))
    kv = synth.normal_bf16(41, 2, (B, L, 576))
    idx = np.stack([np.sort(rng.choice(L, size=(T, k), replace=False), axis=1) for _ in range(B)]).astype(np.int32)
    idx[0, 0, 90:] = -1
    idx[0, 1, 5] = L + 3          # out of range: masked
    idx[1, 0, :] = -1             # nothing visible: zeros
    idx[1, 1, ::2] = -7
    out, lse = dsa.sparse_mla_attn(bf16_dev(q), bf16_dev(kv), i32_dev(idx), 1 / 16, want_lse=True)
    ref, ref_lse = oracle.sparse_mla_attn(q, kv, idx, 1 / 16)
    g = host(out)
    assert np.all(g[1, 0] == 0)
    assert_attn_close(g, ref)
    fin = np.isfinite(ref_lse)
    assert np.all(np.isneginf(host(lse)[~fin]))
    np.testing.assert_allclose(host(lse)[fin], ref_lse[fin], atol=LSE_TOL, rtol=0)


@pytest.mark.parametrize("B,T,k", [(3, 1, 20), (5, 1, 700), (4, 5, 2048), (33, 1, 600)])
def test_attn_head_groups(dsa, B, T, k):
    # Batches under 32 queries split each query's heads over two workgroups:
    # one tile (a single split per query), short and long splits; 33 queries
    # keep whole-query workgroups.  Masked and missing entries in every list.
    rng = np.random.default_rng(60 + B)
    L = 4000
    say("attn head groups B=%d T=%d k=%d" % (B, T, k))
    q = synth.normal_bf16(60, 1, (B, T, 64, 576))
    kv = synth.normal_bf16(60, 2, (B, L, 576))
    idx = np.sort(rng.choice(L, size=(B, T, k)), axis=2).astype(np.int32)
    idx[..., 1] = -1
    idx[0, 0, k // 2:] = L + 5
    out, lse = dsa.sparse_mla_attn(bf16_dev(q), bf16_dev(kv), i32_dev(idx), 1 / 16, want_lse=True)
    ref, ref_lse = oracle.sparse_mla_attn(q, kv, idx, 1 / 16)
    assert_attn_close(host(out), ref)
    np.testing.assert_allclose(host(lse), ref_lse, atol=LSE_TOL, rtol=0)


@pytest.mark.parametrize("B", [28, 32])
def test_attn_split_launch_either_side_of_streaming(dsa, B):
    # 28 x 2048 rows (63 MiB) keep plain gathers, 32 x 2048 (72 MiB) stream
    # them past the caches: the same kernel with another load hint, checked
    # here with masked, out-of-range and duplicated entries
    rng = np.random.default_rng(60 + B)
    T, L, k = 1, 3000, 2048
    say("attn split launch B=%d" % B)
    q = synth.normal_bf16(43, 1, (B, T, 64, 576))
    kv = synth.normal_bf16(43, 2, (B, L, 576))
    idx = np.stack([np.sort(rng.choice(L, size=(T, k), replace=False), axis=1) for _ in range(B)]).astype(np.int32)
    idx[0, 0, 1500:] = -1
    idx[1, 0, 7] = L + 11         # out of range: masked
    idx[2, 0, 100:200] = idx[2, 0, 99]  # a repeated row counts once per occurrence
    out, lse = dsa.sparse_mla_attn(bf16_dev(q), bf16_dev(kv), i32_dev(idx), 1 / 16, want_lse=True)
    ref, ref_lse = oracle.sparse_mla_attn(q, kv, idx, 1 / 16)
    assert_attn_close(host(out), ref)
    np.testing.assert_allclose(host(lse), ref_lse, atol=LSE_TOL, rtol=0)


def test_attn_dense_case(dsa):
    # k >= p+1: every visible row selected, sparse attention == dense causal attention
    B, T, L, k = 1, 3, 500, 512
    say("attn dense")
    q = synth.normal_bf16(42, 1, (B, T, 64, 576))
    kv = synth.normal_bf16(42, 2, (B, L, 576))
    pos = np.array([[10, 255, 499]], np.int32)
    scores = np.zeros((B, T, L), np.float32)
    idx = oracle.topk(scores, pos, k)
    got = host(dsa.sparse_mla_attn(bf16_dev(q), bf16_dev(kv), i32_dev(idx), 1 / 16))
    ref, _ = oracle.sparse_mla_attn(q, kv, idx, 1 / 16)
    assert_attn_close(got, ref)


def test_attn_many_queries_direct_path(dsa):
    # enough queries that each gets one split (the direct, combine-free kernel)
    rng = np.random.default_rng(10)
    B, T, L, k = 1, 600, 4000, 256
    say("attn direct path T=%d" % T)
    q = synth.normal_bf16(43, 1, (B, T, 64, 576))
    kv = synth.normal_bf16(43, 2, (B, L, 576))
    idx = np.sort(rng.choice(L, size=(B, T, k)), axis=2).astype(np.int32)
    assert dsa.attn_workspace_size(B, T, k) == 0
    got = host(dsa.sparse_mla_attn(bf16_dev(q), bf16_dev(kv), i32_dev(idx), 1 / 16))
    sample = [0, 1, 299, 599]
    ref, _ = oracle.sparse_mla_attn(q[:, sample], kv, idx[:, sample], 1 / 16)
    assert_attn_close(got[:, sample], ref)


def _growing_rows(seed, B, L):
    """Latent rows whose magnitude doubles every 256 positions: with sorted index
    lists the logits keep outgrowing the running reference maximum, so the
    online softmax has to move it (and rescale the accumulators) many times."""
    kv = synth.normal_bf16(seed, 2, (B, L, 576))
    scale = np.exp2(np.arange(L) // 256).astype(np.float32)[None, :, None]
    v = synth.bf16_to_f32(kv) * scale
    return (v.view(np.uint32) >> 16).astype(np.uint16)  # exact: scaling by a power of two


@pytest.mark.parametrize("T", [40, 300])
def test_attn_reference_moves(dsa, T):
    # T=40: several splits of several tiles each; T=300: one workgroup per query
    rng = np.random.default_rng(11 + T)
    B, L, k = 1, 4096, 1024
    say("attn reference moves T=%d" % T)
    q = synth.normal_bf16(44, 1, (B, T, 64, 576))
    kv = _growing_rows(44, B, L)
    idx = np.sort(np.stack([rng.choice(L, size=k, replace=False) for _ in range(T)]), axis=1)[None].astype(np.int32)
    out, lse = dsa.sparse_mla_attn(bf16_dev(q), bf16_dev(kv), i32_dev(idx), 1 / 16, want_lse=True)
    sample = [0, T // 2, T - 1]
    ref, ref_lse = oracle.sparse_mla_attn(q[:, sample], kv, idx[:, sample], 1 / 16)
    assert_attn_close(host(out)[:, sample], ref)
    np.testing.assert_allclose(host(lse)[:, sample], ref_lse, atol=LSE_TOL * np.abs(ref_lse).max(), rtol=0)


def test_attn_direct_ragged_k(dsa):
    # one workgroup per query with a list that ends inside a tile, some entries masked
    rng = np.random.default_rng(12)
    B, T, L, k = 1, 300, 3000, 100
    say("attn direct ragged k=%d" % k)
    q = synth.normal_bf16(45, 1, (B, T, 64, 576))
    kv = synth.normal_bf16(45, 2, (B, L, 576))
    idx = np.sort(rng.choice(L, size=(B, T, k)), axis=2).astype(np.int32)
    idx[0, 7, 50:] = -1
    idx[0, 8, :] = -1
    assert dsa.attn_workspace_size(B, T, k) == 0
    out, lse = dsa.sparse_mla_attn(bf16_dev(q), bf16_dev(kv), i32_dev(idx), 1 / 16, want_lse=True)
    sample = [0, 7, 8, 299]
    ref, ref_lse = oracle.sparse_mla_attn(q[:, sample], kv, idx[:, sample], 1 / 16)
    got = host(out)[:, sample]
    assert np.all(got[0, 2] == 0) and np.all(np.isneginf(host(lse)[0, 8]))
    assert_attn_close(got, ref)


def _unordered_list(rng, L, k, T):
    """Index lists in no particular order, with repeated rows and masked
    entries (-1 and positions >= L) spread through them."""
    idx = rng.integers(2, L, size=(1, T, k)).astype(np.int32)
    idx[0, :, 1::9] = idx[0, :, 0::9][:, :idx[0, :, 1::9].shape[1]]  # every ninth pair repeats a row
    idx[0, :, 5::13] = -1
    idx[0, :, 7::29] = L + 11
    return idx


@pytest.mark.parametrize("T", [3, 300])
def test_attn_unordered_duplicates_masked(dsa, T):
    # The entry point accepts any order: a permuted list with repeated rows
    # (each counted once per occurrence) and masked entries in the middle.
    # T=3: split lists and the combine; T=300: one workgroup per whole list.
    rng = np.random.default_rng(50 + T)
    B, L, k = 1, 5000, 700
    say("attn unordered, duplicates, masked T=%d" % T)
    q = synth.normal_bf16(51, 1, (B, T, 64, 576))
    kv = synth.normal_bf16(51, 2, (B, L, 576))
    idx = _unordered_list(rng, L, k, T)
    out, lse = dsa.sparse_mla_attn(bf16_dev(q), bf16_dev(kv), i32_dev(idx), 1 / 16, want_lse=True)
    sample = list(range(T)) if T < 8 else [0, 150, 299]
    ref, ref_lse = oracle.sparse_mla_attn(q[:, sample], kv, idx[:, sample], 1 / 16)
    assert_attn_close(host(out)[:, sample], ref)
    np.testing.assert_allclose(host(lse)[:, sample], ref_lse, atol=LSE_TOL, rtol=0)
    # the same multiset of rows in ascending order gives the same result (within rounding)
    srt = np.sort(idx, axis=2)
    out2 = host(dsa.sparse_mla_attn(bf16_dev(q), bf16_dev(kv), i32_dev(srt), 1 / 16))
    assert_attn_close(out2[:, sample], ref)


def test_attn_nonfinite_rows_not_selected(dsa):
    # Rows 0 and 1 hold NaN and Inf and are never selected; masked entries
    # (which gather row 0) must not carry them into the output.
    rng = np.random.default_rng(52)
    B, T, L, k = 1, 3, 3000, 300
    say("attn non-finite rows not selected")
    q = synth.normal_bf16(53, 1, (B, T, 64, 576))
    kv = synth.normal_bf16(53, 2, (B, L, 576))
    kv[0, 0, :] = 0x7FC0  # bf16 NaN
    kv[0, 1, :] = 0x7F80  # bf16 +Inf
    idx = np.sort(rng.choice(np.arange(2, L), size=(B, T, k)), axis=2).astype(np.int32)
    idx[0, 0, ::3] = -1
    idx[0, 1, -40:] = L + 5
    idx[0, 2, :] = -1
    idx[0, 2, 17] = 1234
    out, lse = dsa.sparse_mla_attn(bf16_dev(q), bf16_dev(kv), i32_dev(idx), 1 / 16, want_lse=True)
    got = host(out)
    assert np.all(np.isfinite(got)) and np.all(np.isfinite(host(lse)))
    ref, ref_lse = oracle.sparse_mla_attn(q, kv, idx, 1 / 16)
    assert_attn_close(got, ref)
    np.testing.assert_allclose(host(lse), ref_lse, atol=LSE_TOL, rtol=0)


# ------------------------------------------------------------------ IndexShare group
def test_group_tiny(dsa):
    cfg = synth.TINY
    say("group tiny")
    qi, w, ki, pos = cfg.q_idx(), cfg.w(), cfg.k_idx(), cfg.q_pos()
    qs = [cfg.q_attn(l) for l in range(cfg.n_layers)]
    kvs = [cfg.kv(l) for l in range(cfg.n_layers)]
    dq = [bf16_dev(q) for q in qs]
    dkv = [bf16_dev(kv) for kv in kvs]
    idx, outs, lses = dsa.layer_group(bf16_dev(qi), f32_dev(w), bf16_dev(ki), i32_dev(pos), cfg.k, dq, dkv,
                                      cfg.sm_scale, want_lse=True)
    _, ref_idx, ref_outs, ref_lses = oracle.layer_group(qi, w, ki, pos, cfg.k, qs, kvs, cfg.sm_scale)
    np.testing.assert_array_equal(host(idx), ref_idx)
    for l in range(cfg.n_layers):
        assert_attn_close(host(outs[l]), ref_outs[l], "layer %d" % l)
        np.testing.assert_allclose(host(lses[l]), ref_lses[l], atol=LSE_TOL, rtol=0)
        # every layer consumed the one shared list: bitwise equal to a standalone call with it
        alone = dsa.sparse_mla_attn(dq[l], dkv[l], idx, cfg.sm_scale)
        assert torch.equal(alone.view(torch.int16), outs[l].view(torch.int16))


def test_group_eight_layers(dsa):
    # the largest group the entry point takes: one index list feeding eight layers
    cfg = synth.TINY
    n = 8
    say("group tiny, %d layers" % n)
    qi, w, ki, pos = cfg.q_idx(), cfg.w(), cfg.k_idx(), cfg.q_pos()
    qs = [cfg.q_attn(l) for l in range(n)]
    kvs = [cfg.kv(l) for l in range(n)]
    idx, outs, _ = dsa.layer_group(bf16_dev(qi), f32_dev(w), bf16_dev(ki), i32_dev(pos), cfg.k,
                                   [bf16_dev(q) for q in qs], [bf16_dev(kv) for kv in kvs], cfg.sm_scale)
    _, ref_idx, ref_outs, _ = oracle.layer_group(qi, w, ki, pos, cfg.k, qs, kvs, cfg.sm_scale)
    np.testing.assert_array_equal(host(idx), ref_idx)
    for l in range(n):
        assert_attn_close(host(outs[l]), ref_outs[l], "layer %d" % l)


def test_group_on_side_stream_and_in_graph(dsa):
    # The entry points only enqueue work on the caller's stream: on a side
    # stream, and captured in a graph replayed several times with eager work
    # between the replays, the group gives the eager result bit for bit.
    cfg = synth.TINY
    say("group on a side stream and in a graph")
    qi, w, ki, pos = bf16_dev(cfg.q_idx()), f32_dev(cfg.w()), bf16_dev(cfg.k_idx()), i32_dev(cfg.q_pos())
    dq = [bf16_dev(cfg.q_attn(l)) for l in range(cfg.n_layers)]
    dkv = [bf16_dev(cfg.kv(l)) for l in range(cfg.n_layers)]
    idx0, outs0, _ = dsa.layer_group(qi, w, ki, pos, cfg.k, dq, dkv, cfg.sm_scale)
    torch.cuda.synchronize()

    def same(idx, outs):
        return torch.equal(idx, idx0) and all(torch.equal(a.view(torch.int16), b.view(torch.int16))
                                              for a, b in zip(outs, outs0))

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        idx1, outs1, _ = dsa.layer_group(qi, w, ki, pos, cfg.k, dq, dkv, cfg.sm_scale)
    side.synchronize()
    assert same(idx1, outs1)

    idx2 = torch.full_like(idx0, -7)
    outs2 = [torch.zeros_like(o) for o in outs0]
    ws = torch.empty(dsa.layer_group_workspace_size(
        dsa.make_group_args(qi, w, ki, pos, cfg.k, dq, dkv, cfg.sm_scale, idx2, outs2, None)),
        dtype=torch.uint8, device=DEV)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dsa.layer_group(qi, w, ki, pos, cfg.k, dq, dkv, cfg.sm_scale, ws=ws, idx_out=idx2, outs=outs2)
    for r in range(3):
        idx2.fill_(-7)
        for o in outs2:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert same(idx2, outs2), r
        dsa.layer_group(qi, w, ki, pos, cfg.k, dq, dkv, cfg.sm_scale)  # eager work between replays
        torch.cuda.synchronize()


# ------------------------------------------------------------------ verification
@pytest.mark.parametrize("rho", [0.0, 0.9, 1.0])
def test_verify_small(dsa, rho):
    rng = np.random.default_rng(int(rho * 10) + 50)
    B, S, V = 8, 3, 1000
    say("verify small rho=%.1f" % rho)
    t = (rng.standard_normal((B, S + 1, V)) * 2).astype(np.float32)
    d = (rho * t[:, :S] + np.sqrt(1 - rho * rho) * rng.standard_normal((B, S, V)) * 2).astype(np.float32)
    tok = rng.integers(0, V, (B, S)).astype(np.int32)
    tok[:, 0] = np.argmax(d[:, 0], -1)
    u = rng.random((B, S)).astype(np.float32)
    ur = rng.random(B).astype(np.float32)
    ms, na, nx = dsa.mtp_draft_verify(f32_dev(t), f32_dev(d), i32_dev(tok), f32_dev(u), f32_dev(ur))
    check_verify(host(ms), host(na), host(nx), t, d, tok, u, ur)


@pytest.mark.parametrize("S", [1, 20, 64])
def test_verify_draft_lengths(dsa, S):
    rng = np.random.default_rng(60 + S)
    B, V = 5, 3000
    say("verify S=%d" % S)
    t = (rng.standard_normal((B, S + 1, V)) * 2).astype(np.float32)
    d = (0.95 * t[:, :S] + 0.3 * rng.standard_normal((B, S, V))).astype(np.float32)
    tok = np.argmax(d + rng.gumbel(size=d.shape), axis=-1).astype(np.int32)
    u = rng.random((B, S)).astype(np.float32)
    ur = rng.random(B).astype(np.float32)
    ms, na, nx = dsa.mtp_draft_verify(f32_dev(t), f32_dev(d), i32_dev(tok), f32_dev(u), f32_dev(ur))
    check_verify(host(ms), host(na), host(nx), t, d, tok, u, ur)


def test_verify_mtp_vocab(dsa):
    cfg = synth.MtpConfig("mtp_small", seed=5, B=3, L=1024)
    say("verify vocab %d" % cfg.V)
    t = cfg.target_logits()
    d = cfg.draft_logits(t)
    tok = cfg.draft_tokens(d)
    u, ur = cfg.u_accept(), cfg.u_resample()
    ms, na, nx = dsa.mtp_draft_verify(f32_dev(t), f32_dev(d), i32_dev(tok), f32_dev(u), f32_dev(ur))
    check_verify(host(ms), host(na), host(nx), t, d, tok, u, ur)


def test_verify_ragged_vocab(dsa):
    # V not a multiple of 4 (element-wise loads) and a ragged last chunk
    rng = np.random.default_rng(71)
    B, S, V = 4, 5, 8195
    say("verify V=%d" % V)
    t = (rng.standard_normal((B, S + 1, V)) * 2).astype(np.float32)
    d = (0.8 * t[:, :S] + 0.6 * rng.standard_normal((B, S, V)) * 2).astype(np.float32)
    tok = np.argmax(d + rng.gumbel(size=d.shape), axis=-1).astype(np.int32)
    u = rng.random((B, S)).astype(np.float32)
    ur = rng.random(B).astype(np.float32)
    ms, na, nx = dsa.mtp_draft_verify(f32_dev(t), f32_dev(d), i32_dev(tok), f32_dev(u), f32_dev(ur))
    check_verify(host(ms), host(na), host(nx), t, d, tok, u, ur)


def test_verify_vocab_beyond_64_chunks(dsa):
    # V = 600001: 74 chunks of 8192, so the accept block's chunk scan runs over
    # two 64-chunk groups; V odd takes the element-wise loads
    rng = np.random.default_rng(73)
    B, S, V = 3, 2, 600001
    say("verify V=%d" % V)
    t = (rng.standard_normal((B, S + 1, V)) * 2).astype(np.float32)
    d = (0.5 * t[:, :S] + 0.9 * rng.standard_normal((B, S, V)) * 2).astype(np.float32)
    tok = np.argmax(d + rng.gumbel(size=d.shape), axis=-1).astype(np.int32)
    u = rng.random((B, S)).astype(np.float32)
    ur = np.array([0.02, 0.6, 0.995], np.float32)
    ms, na, nx = dsa.mtp_draft_verify(f32_dev(t), f32_dev(d), i32_dev(tok), f32_dev(u), f32_dev(ur))
    check_verify(host(ms), host(na), host(nx), t, d, tok, u, ur)


def test_verify_residual_without_mass_samples_p(dsa):
    # draft == target and a rejected out-of-vocabulary token: max(p - q, 0) has no
    # mass, so the resample draws from p of the rejected step
    rng = np.random.default_rng(72)
    B, S, V = 3, 2, 20000
    t = rng.standard_normal((B, S + 1, V)).astype(np.float32)
    d = t[:, :S].copy()
    tok = np.full((B, S), V + 1, np.int32)
    u = np.full((B, S), 0.5, np.float32)
    ur = np.array([0.1, 0.5, 0.97], np.float32)
    say("verify residual without mass")
    ms, na, nx = dsa.mtp_draft_verify(f32_dev(t), f32_dev(d), i32_dev(tok), f32_dev(u), f32_dev(ur))
    assert np.all(host(na) == 0)
    for b in range(B):
        assert inv_cdf_valid(oracle.softmax_row(t[b, 0]), float(ur[b]), int(host(nx)[b])), b
    check_verify(host(ms), host(na), host(nx), t, d, tok, u, ur)


def test_verify_out_of_vocab_token_rejected(dsa):
    rng = np.random.default_rng(3)
    B, S, V = 1, 2, 100
    t = rng.standard_normal((B, S + 1, V)).astype(np.float32)
    d = rng.standard_normal((B, S, V)).astype(np.float32)
    tok = np.array([[V + 5, 3]], np.int32)
    u = np.full((B, S), 0.01, np.float32)
    ur = np.array([0.5], np.float32)
    _, na, nx = dsa.mtp_draft_verify(f32_dev(t), f32_dev(d), i32_dev(tok), f32_dev(u), f32_dev(ur))
    assert int(host(na)[0]) == 0 and 0 <= int(host(nx)[0]) < V


@pytest.mark.parametrize("fill", ["zeros", "bytes_ab", "neg_inf_words"])
def test_group_workspace_state(dsa, fill):
    # The decode indexer adds the top-k histogram onto what the previous call
    # left in the workspace (zero, with a stamp of the shape).  A workspace
    # that holds anything else on its first use -- zeros, bytes 0xAB, or the
    # bits of -inf floats, whose 2048-word sums wrap to exactly 0 -- gives the
    # exact result through a recount, and so do the second call of the shape
    # and the first call after a change of shape.
    say("group workspace state: %s" % fill)
    lib = dsa.lib()
    stream = torch.cuda.current_stream(DEV).cuda_stream
    shapes = [(3, 9000, 0), (3, 9000, 1), (2, 12000, 0), (3, 9000, 0)]
    cases = {}
    for B, L, _ in shapes:
        if (B, L) in cases:
            continue
        qi = synth.int_bf16(90 + L, 1, (B, 1, 32, 128))
        w = synth.pow2_f32(90 + L, 2, (B, 1, 32))
        ki = synth.int_bf16(90 + L, 3, (B, L, 128))
        pos = np.full((B, 1), L - 1, np.int32)
        pos[0, 0] = L // 3
        q = synth.normal_bf16(90 + L, 4, (B, 1, 64, 576))
        kv = synth.normal_bf16(90 + L, 5, (B, L, 576))
        _, ref_idx, ref_outs, _ = oracle.layer_group(qi, w, ki, pos, 2048, [q], [kv], 1 / 16)
        cases[(B, L)] = ((bf16_dev(qi), f32_dev(w), bf16_dev(ki), i32_dev(pos), [bf16_dev(q)], [bf16_dev(kv)]),
                         ref_idx, ref_outs[0])
    nbytes = max(dsa.layer_group_workspace_size(dsa.make_group_args(
        *d[:4], 2048, d[4], d[5], 1 / 16, torch.empty((B, 1, 2048), dtype=torch.int32, device=DEV),
        [torch.empty((B, 1, 64, 512), dtype=torch.bfloat16, device=DEV)])) for (B, L), (d, _, _) in cases.items())
    if fill == "zeros":
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    elif fill == "bytes_ab":
        ws = torch.full((nbytes,), 0xAB, dtype=torch.uint8, device=DEV)
    else:
        ws = torch.full((nbytes // 4,), float("-inf"), dtype=torch.float32, device=DEV).view(torch.uint8)
    for call, (B, L, _) in enumerate(shapes):
        d, ref_idx, ref_out = cases[(B, L)]
        idx = torch.full((B, 1, 2048), -9, dtype=torch.int32, device=DEV)
        out = torch.zeros((B, 1, 64, 512), dtype=torch.bfloat16, device=DEV)
        a = dsa.make_group_args(*d[:4], 2048, d[4], d[5], 1 / 16, idx, [out])
        assert lib.dsa_layer_group(ctypes.byref(a), ws.data_ptr(), nbytes, stream) == 0, dsa.last_error()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(idx), ref_idx, err_msg="call %d B=%d L=%d" % (call, B, L))
        assert_attn_close(host(out), ref_out, "call %d" % call)


def test_group_without_indexshare(dsa):
    # share = 0, standard DSA: every layer runs its own indexer and top-k over
    # its own index queries, weights and index-key cache.  Each layer's list is
    # bit-exact against the oracle's indexer and top-k for that layer, the
    # lists differ between layers, and each output matches the oracle's
    # attention with that layer's list.
    cfg = synth.TINY
    n = 4
    say("group without IndexShare, %d layers" % n)
    B, T, L = cfg.B, cfg.T, cfg.L
    pos = cfg.q_pos()
    qis = [synth.int_bf16(60 + l, 1, (B, T, 32, 128)) for l in range(n)]
    ws_ = [synth.pow2_f32(60 + l, 2, (B, T, 32)) for l in range(n)]
    kis = [synth.int_bf16(60 + l, 3, (B, L, 128)) for l in range(n)]
    qs = [cfg.q_attn(l) for l in range(n)]
    kvs = [cfg.kv(l) for l in range(n)]
    idxs, outs, lses = dsa.layer_group_unshared([bf16_dev(x) for x in qis], [f32_dev(x) for x in ws_],
                                                [bf16_dev(x) for x in kis], i32_dev(pos), cfg.k,
                                                [bf16_dev(q) for q in qs], [bf16_dev(kv) for kv in kvs], cfg.sm_scale,
                                                want_lse=True)
    got_idx = [host(i) for i in idxs]
    for l in range(n):
        ref_idx = oracle.topk(oracle.indexer_scores(qis[l], ws_[l], kis[l], pos), pos, cfg.k)
        np.testing.assert_array_equal(got_idx[l], ref_idx, err_msg="layer %d" % l)
        ref, ref_lse = oracle.sparse_mla_attn(qs[l], kvs[l], ref_idx, cfg.sm_scale)
        assert_attn_close(host(outs[l]), ref, "layer %d" % l)
        np.testing.assert_allclose(host(lses[l]), ref_lse, atol=LSE_TOL, rtol=0)
    for l in range(1, n):
        assert not np.array_equal(got_idx[l], got_idx[0]), "layer %d selected the same rows as layer 0" % l


def _sweep_shape(seed):
    # a seeded shape: batch, queries per sequence, keys, k and ragged positions
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 5))
    T = int(rng.choice([1, 1, 2, 5, 9]))
    L = int(rng.choice([17, 300, 1023, 2049, 4100, 6001]))
    k = int(rng.choice([1, 5, 33, 100, 256, 700, 2048]))
    pos = rng.integers(0, L, size=(B, T)).astype(np.int32)
    pos[0, -1] = L - 1
    return B, T, L, k, pos


@pytest.mark.parametrize("seed", range(8))
def test_group_shape_sweep(dsa, seed):
    # Seeded shapes across the launch configurations (split or whole lists,
    # one to sixteen splits, k below or above the visible keys, ragged
    # positions, lengths that are not multiples of a tile): the shared list
    # bit-exact against the oracle, every query's output of two layers within
    # tolerance.
    B, T, L, k, pos = _sweep_shape(seed)
    say("group sweep seed=%d B=%d T=%d L=%d k=%d" % (seed, B, T, L, k))
    qi = synth.int_bf16(200 + seed, 1, (B, T, 32, 128))
    w = synth.pow2_f32(200 + seed, 2, (B, T, 32))
    ki = synth.int_bf16(200 + seed, 3, (B, L, 128))
    qs = [synth.normal_bf16(200 + seed, 4 + l, (B, T, 64, 576)) for l in range(2)]
    kvs = [synth.normal_bf16(200 + seed, 6 + l, (B, L, 576)) for l in range(2)]
    idx, outs, lses = dsa.layer_group(bf16_dev(qi), f32_dev(w), bf16_dev(ki), i32_dev(pos), k,
                                      [bf16_dev(q) for q in qs], [bf16_dev(kv) for kv in kvs], 1 / 16,
                                      want_lse=True)
    _, ref_idx, ref_outs, ref_lses = oracle.layer_group(qi, w, ki, pos, k, qs, kvs, 1 / 16)
    np.testing.assert_array_equal(host(idx), ref_idx)
    for l in range(2):
        assert_attn_close(host(outs[l]), ref_outs[l], "layer %d" % l)
        fin = np.isfinite(ref_lses[l])
        np.testing.assert_allclose(host(lses[l])[fin], ref_lses[l][fin], atol=LSE_TOL, rtol=0)


@pytest.mark.parametrize("B", [32, 40, 64, 100])
def test_group_batch_sizes(dsa, B):
    # Batches of 32+ one-token queries: each list is split in 8 (B = 32),
    # 7 (B = 40, a shorter last part), 4 (B = 64) or 3 (B = 100) parts whose
    # partials a combine launch merges.  Lists bit-exact against the oracle, outputs within
    # tolerance on sampled queries and bit-equal to the standalone entry point.
    L, k = 3000, 2048
    say("group B=%d" % B)
    qi = synth.int_bf16(100 + B, 1, (B, 1, 32, 128))
    w = synth.pow2_f32(100 + B, 2, (B, 1, 32))
    ki = synth.int_bf16(100 + B, 3, (B, L, 128))
    pos = np.full((B, 1), L - 1, np.int32)
    pos[1, 0] = 1000
    pos[2, 0] = 5  # fewer visible keys than k: -1 padded list
    qs = [synth.normal_bf16(100 + B, 4 + l, (B, 1, 64, 576)) for l in range(2)]
    kvs = [synth.normal_bf16(100 + B, 6 + l, (B, L, 576)) for l in range(2)]
    dq, dkv = [bf16_dev(q) for q in qs], [bf16_dev(kv) for kv in kvs]
    idx, outs, lses = dsa.layer_group(bf16_dev(qi), f32_dev(w), bf16_dev(ki), i32_dev(pos), k, dq, dkv, 1 / 16,
                                      want_lse=True)
    ref_idx = oracle.topk(oracle.indexer_scores(qi, w, ki, pos), pos, k)
    np.testing.assert_array_equal(host(idx), ref_idx)
    sample = [0, 1, 2, B - 1]
    for l in range(2):
        ref, ref_lse = oracle.sparse_mla_attn(qs[l][sample], kvs[l][sample], ref_idx[sample], 1 / 16)
        assert_attn_close(host(outs[l])[sample], ref, "layer %d" % l)
        np.testing.assert_allclose(host(lses[l])[sample], ref_lse, atol=LSE_TOL, rtol=0)
        alone = dsa.sparse_mla_attn(dq[l], dkv[l], idx, 1 / 16)
        assert torch.equal(alone.view(torch.int16), outs[l].view(torch.int16)), "layer %d" % l
