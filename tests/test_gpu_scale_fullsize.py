"""GPU parity at the workloads' full sizes, through the C ABI.

* decode 128K (B=32, L=131072, 4 layers): the exact launch the benchmark times
  (``dsa_layer_group``).
* decode 1M (B=4, L=1048576).
* chunked prefill (4096 queries at positions 126976..131071).
* the MTP draft round (B=16, 7 steps over the backbone cache) plus
  verification at V=151552.

The oracle is too slow for whole outputs at these sizes.  Sampled rows are
therefore compared with it one by one: scores and indices bit-exact,
attention within the stated tolerance.  Properties that hold at any size are
checked on every row (or on a large sample for prefill).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import (DEV, LSE_TOL, assert_attn_close, bf16_dev, check_topk_properties, check_verify, f32_dev,
                         host, i32_dev, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    import long_context_sparse_scores_amd as m
    assert torch.cuda.is_available()
    return m


def _device_group_inputs(cfg):
    """Every tensor of one group on the device, the caches generated one layer at a time."""
    B, L = cfg.B, cfg.L
    d = {"q_idx": bf16_dev(cfg.q_idx()), "w": f32_dev(cfg.w()), "pos": i32_dev(cfg.q_pos())}
    d["k_idx"] = bf16_dev(cfg.k_idx())
    d["qs"] = [bf16_dev(cfg.q_attn(l)) for l in range(cfg.n_layers)]
    host_kv = np.empty((B, L, cfg.Dqk), np.uint16)
    d["kvs"] = []
    for l in range(cfg.n_layers):
        cfg.kv(l, out=host_kv)
        d["kvs"].append(bf16_dev(host_kv))
    del host_kv
    torch.cuda.synchronize()
    return d


def _check_index_rows(cfg, rows_bt, scores_gpu, idx_gpu):
    """Oracle scores and top-k of the sampled (b, t) rows, bit-exact."""
    qi, w, pos = cfg.q_idx(), cfg.w(), cfg.q_pos()
    by_b = {}
    for b, t in rows_bt:
        by_b.setdefault(b, []).append(t)
    for b, ts in by_b.items():
        ki = cfg.k_idx_rows(b)[None]
        ts = np.array(ts)
        ref_s = oracle.indexer_scores(qi[b:b + 1, ts], w[b:b + 1, ts], ki, pos[b:b + 1, ts])
        ref_i = oracle.topk(ref_s, pos[b:b + 1, ts], cfg.k)
        for j, t in enumerate(ts):
            say("  oracle row b=%d t=%d" % (b, t))
            np.testing.assert_array_equal(scores_gpu[b, t].view(np.uint32), ref_s[0, j].view(np.uint32))
            np.testing.assert_array_equal(idx_gpu[b, t], ref_i[0, j])


def _check_attn_rows(cfg, pairs, q_host, out_gpu, lse_gpu, idx_gpu):
    """Oracle attention of sampled (layer, b, t) over the rows the GPU selected,
    regenerated from the seed (the oracle never sees the whole cache)."""
    for l, b, t in pairs:
        sel = idx_gpu[b, t]
        sel = sel[sel >= 0]
        kv_sel = cfg.kv_rows(l, b, sel)[None]
        ident = np.arange(sel.size, dtype=np.int32)[None, None]
        ref, ref_lse = oracle.sparse_mla_attn(q_host[l][b:b + 1, t:t + 1], kv_sel, ident, cfg.sm_scale)
        err, scale = assert_attn_close(out_gpu[l][b, t], ref[0, 0], "layer %d b %d t %d" % (l, b, t))
        say("  attn layer %d b=%d t=%d: max err %.3g of scale %.3g" % (l, b, t, err, scale))
        if lse_gpu is not None:
            np.testing.assert_allclose(lse_gpu[l][b, t], ref_lse[0, 0], atol=LSE_TOL, rtol=0)


def _run_group(dsa, cfg, want_lse=True):
    say("group %s: generating inputs" % cfg.name)
    d = _device_group_inputs(cfg)
    say("group %s: dsa_layer_group" % cfg.name)
    idx, outs, lses = dsa.layer_group(d["q_idx"], d["w"], d["k_idx"], d["pos"], cfg.k, d["qs"], d["kvs"],
                                      cfg.sm_scale, want_lse=want_lse)
    # the same kernels called one entry point at a time: the group's shared list is this one, bitwise
    scores = dsa.indexer_scores(d["q_idx"], d["w"], d["k_idx"], d["pos"])
    idx_alone = dsa.topk(scores, d["pos"], cfg.k)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx_alone)
    return d, idx, outs, lses, scores


def _gpu_topk_invariants(idx, pos, k):
    """Checked on the device for every row: ascending unique visible positions, exact count."""
    valid = idx >= 0
    n = valid.sum(dim=2)
    want = torch.clamp(pos.to(torch.int64) + 1, max=k)
    assert torch.equal(n.to(torch.int64), want)
    d = idx[..., 1:] - idx[..., :-1]
    both = valid[..., 1:] & valid[..., :-1]
    assert bool((d[both] > 0).all())
    assert bool((idx.max(dim=2).values <= pos).all())


def test_fullsize_decode_128k_group(dsa):
    cfg = synth.DECODE_128K
    d, idx, outs, lses, scores = _run_group(dsa, cfg)
    sc, ix = host(scores), host(idx)
    say("decode 128K: properties of all %d rows" % (cfg.B * cfg.T))
    _gpu_topk_invariants(idx, d["pos"], cfg.k)
    check_topk_properties(ix.reshape(-1, cfg.k), sc.reshape(-1, cfg.L), cfg.q_pos().reshape(-1), cfg.k)
    _check_index_rows(cfg, [(0, 0), (13, 0), (31, 0)], sc, ix)
    q_host = [cfg.q_attn(l) for l in range(cfg.n_layers)]
    out_h = [host(o) for o in outs]
    lse_h = [host(x) for x in lses]
    _check_attn_rows(cfg, [(0, 0, 0), (1, 7, 0), (2, 31, 0), (3, 13, 0)], q_host, out_h, lse_h, ix)
    # each layer of the group is bitwise the standalone attention call with the shared list
    for l in (0, 3):
        alone = dsa.sparse_mla_attn(d["qs"][l], d["kvs"][l], idx, cfg.sm_scale)
        assert torch.equal(alone.view(torch.int16), outs[l].view(torch.int16))
    assert all(bool(torch.isfinite(o.float()).all()) for o in outs)


def test_fullsize_decode_1m_group(dsa):
    cfg = synth.DECODE_1M
    d, idx, outs, lses, scores = _run_group(dsa, cfg)
    sc, ix = host(scores), host(idx)
    _gpu_topk_invariants(idx, d["pos"], cfg.k)
    check_topk_properties(ix.reshape(-1, cfg.k), sc.reshape(-1, cfg.L), cfg.q_pos().reshape(-1), cfg.k)
    _check_index_rows(cfg, [(0, 0), (3, 0)], sc, ix)
    q_host = [cfg.q_attn(l) for l in range(cfg.n_layers)]
    _check_attn_rows(cfg, [(0, 0, 0), (3, 3, 0), (1, 2, 0)], q_host, [host(o) for o in outs],
                     [host(x) for x in lses], ix)


def test_fullsize_prefill_4096(dsa):
    cfg = synth.PREFILL
    d, idx, outs, lses, scores = _run_group(dsa, cfg, want_lse=False)
    _gpu_topk_invariants(idx, d["pos"], cfg.k)
    rng = np.random.default_rng(11)
    sample_t = np.unique(np.concatenate([[0, 1, 2047, 2048, 4095], rng.choice(cfg.T, 59, replace=False)]))
    sc = host(scores[0, torch.from_numpy(sample_t).to(DEV)])
    ix_all = host(idx)
    say("prefill: properties of %d sampled rows" % sample_t.size)
    check_topk_properties(ix_all[0, sample_t], sc, cfg.q_pos()[0, sample_t], cfg.k)
    # oracle rows: the first, the last and two in between
    ot = [0, 2047, 4095, int(sample_t[7])]
    sc_full = {t: host(scores[0, t]) for t in ot}
    qi, w, pos = cfg.q_idx(), cfg.w(), cfg.q_pos()
    ki = cfg.k_idx_rows(0)[None]
    ts = np.array(ot)
    ref_s = oracle.indexer_scores(qi[:, ts], w[:, ts], ki, pos[:, ts])
    ref_i = oracle.topk(ref_s, pos[:, ts], cfg.k)
    for j, t in enumerate(ot):
        say("  oracle prefill row t=%d" % t)
        np.testing.assert_array_equal(sc_full[t].view(np.uint32), ref_s[0, j].view(np.uint32))
        np.testing.assert_array_equal(ix_all[0, t], ref_i[0, j])
    q_host = [cfg.q_attn(l) for l in range(cfg.n_layers)]
    out_h = [host(o) for o in outs]
    _check_attn_rows(cfg, [(0, 0, 0), (1, 0, 4095), (2, 0, 2047), (3, 0, int(sample_t[7]))], q_host, out_h, None,
                     ix_all)


def test_fullsize_mtp_round(dsa):
    cfg = synth.MTP
    B, L, S = cfg.B, cfg.L, cfg.S
    say("mtp: generating inputs")
    qi, w, pos = cfg.q_idx(), cfg.w(), cfg.q_pos()
    d_qi, d_w, d_pos = bf16_dev(qi), f32_dev(w), i32_dev(pos)
    d_ki = bf16_dev(cfg.k_idx())
    d_kv = bf16_dev(cfg.kv())
    q_steps = cfg.q_steps()
    d_q = bf16_dev(q_steps)
    # step 1: the MTP indexer over the backbone index keys, top-k once
    say("mtp: step-1 indexer + top-k")
    scores = dsa.indexer_scores(d_qi, d_w, d_ki, d_pos)
    idx1 = dsa.topk(scores, d_pos, cfg.k)
    before = idx1.clone()
    # steps 1..S: attention over the backbone latent rows with the step-1 list
    outs = []
    for s in range(S):
        outs.append(dsa.sparse_mla_attn(d_q[:, s:s + 1].contiguous(), d_kv, idx1, cfg.sm_scale))
    torch.cuda.synchronize()
    assert torch.equal(before, idx1)          # every step read the same, unchanged list
    ix = host(idx1)
    assert ix.max() < L and ix.max() <= pos.max()   # only backbone positions: no draft row exists
    _gpu_topk_invariants(idx1, d_pos, cfg.k)
    sc = host(scores)
    check_topk_properties(ix.reshape(-1, cfg.k), sc.reshape(-1, L), pos.reshape(-1), cfg.k)
    for b in (0, 15):
        ref_s = oracle.indexer_scores(qi[b:b + 1], w[b:b + 1], cfg.k_idx_rows(b)[None], pos[b:b + 1])
        np.testing.assert_array_equal(sc[b].view(np.uint32), ref_s[0].view(np.uint32))
        np.testing.assert_array_equal(ix[b], oracle.topk(ref_s, pos[b:b + 1], cfg.k)[0])
    for s, b in ((0, 0), (3, 5), (6, 15)):
        sel = ix[b, 0]
        kv_sel = cfg.kv_rows(b, sel)[None]
        ident = np.arange(sel.size, dtype=np.int32)[None, None]
        ref, _ = oracle.sparse_mla_attn(q_steps[b:b + 1, s:s + 1], kv_sel, ident, cfg.sm_scale)
        err, scale = assert_attn_close(host(outs[s])[b, 0], ref[0, 0], "mtp step %d b %d" % (s, b))
        say("  mtp step %d b=%d: max err %.3g of scale %.3g" % (s, b, err, scale))
    # verification of the round's drafts at the full vocabulary
    say("mtp: verification V=%d" % cfg.V)
    t = cfg.target_logits()
    dr = cfg.draft_logits(t)
    tok = cfg.draft_tokens(dr)
    u, ur = cfg.u_accept(), cfg.u_resample()
    ms, na, nx = dsa.mtp_draft_verify(f32_dev(t), f32_dev(dr), i32_dev(tok), f32_dev(u), f32_dev(ur))
    check_verify(host(ms), host(na), host(nx), t, dr, tok, u, ur)
