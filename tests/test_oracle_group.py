"""Pins for the oracle's IndexShare group and the synthetic generator."""
import json
import os

import numpy as np

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")


def small_group(L=600, T=3, k=128, layers=4, seed=21):
    cfg = synth.GroupConfig("t", seed=seed, B=2, T=T, L=L, first_pos=L - T, k=k, n_layers=layers)
    return cfg, cfg.q_idx(), cfg.w(), cfg.k_idx(), cfg.q_pos(), [cfg.q_attn(l) for l in range(layers)], \
        [cfg.kv(l) for l in range(layers)]


def test_group_is_indexer_then_topk_then_each_layer():
    cfg, qi, w, ki, pos, qs, kvs = small_group()
    scores, idx, outs, lses = oracle.layer_group(qi, w, ki, pos, cfg.k, qs, kvs, cfg.sm_scale)
    np.testing.assert_array_equal(scores, oracle.indexer_scores(qi, w, ki, pos))
    np.testing.assert_array_equal(idx, oracle.topk(scores, pos, cfg.k))
    for l in range(cfg.n_layers):
        o, s = oracle.sparse_mla_attn(qs[l], kvs[l], idx, cfg.sm_scale)
        np.testing.assert_array_equal(outs[l], o)       # one shared index list, bit for bit
        np.testing.assert_array_equal(lses[l], s)
    # layers differ (own q and cache), the index list does not
    assert not np.array_equal(outs[0], outs[1])


def test_page_constants_drive_the_shapes():
    g = json.load(open(GOLDEN))
    c = synth.DECODE_128K
    assert c.k == g["index_topk"]["value"]
    assert c.D == g["index_head_dim"]["value"]
    assert c.H == g["index_n_heads"]["value"]
    assert c.n_layers == g["index_topk_freq"]["value"]
    assert c.Dv == g["kv_lora_rank"]["value"]
    assert c.Hq == g["attn_heads"]["value"]
    assert synth.MTP.S == g["mtp_steps"]["value"]
    # sm_scale: 1/sqrt(head dim 256) from the MLA section
    assert c.sm_scale == 1.0 / np.sqrt(g["attn_head_dim"]["value"])


def test_kv_cache_estimate_pins_the_576_bf16_row():
    # The MLA section's ~88GB (compressed) and ~5TB (uncompressed) at 1M context
    # over 78 layers follow from a 576-value bf16 latent row and 64x256 heads.
    g = json.load(open(GOLDEN))
    toks, layers = 2 ** 20, g["n_layers"]["value"]
    row = synth.DECODE_128K.Dqk
    comp = toks * layers * row * 2
    full = toks * layers * g["attn_heads"]["value"] * g["attn_head_dim"]["value"] * 2 * 2
    assert abs(comp / 2 ** 30 - g["kv_cache_1m_compressed_gb"]["value"]) < 1.0      # 87.75 GiB
    assert abs(full / 1e12 - g["kv_cache_1m_uncompressed_tb"]["value"]) < 0.5        # 5.36 TB
    assert abs(full / comp - g["kv_compression_ratio"]["value"]) < 0.5                # 56.9
    assert abs(2 ** 20 / synth.DECODE_128K.k - g["attention_fraction_1m"]["value"]) < 25  # 512


def test_generator_is_counter_based_and_sliceable():
    a = synth.normal_bf16(9, 3, (1000,))
    b = synth.normal_bf16(9, 3, (400,), start=600)
    np.testing.assert_array_equal(a[600:], b)
    assert not np.array_equal(a, synth.normal_bf16(9, 4, (1000,)))
    assert not np.array_equal(a, synth.normal_bf16(10, 3, (1000,)))
    rows = synth.normal_bf16_rows(9, 3, np.array([0, 576, 10]), 5)
    np.testing.assert_array_equal(rows[1], a[576:581])
    x = synth.bf16_to_f32(synth.normal_bf16(1, 1, (2_000_000,))).astype(np.float64)
    assert abs(x.mean()) < 3e-3 and abs(x.std() - 1) < 3e-3
    i = synth.bf16_to_f32(synth.int_bf16(1, 2, (700_000,)))
    assert set(np.unique(i)) == set(range(-3, 4))
    w = synth.pow2_f32(1, 3, (100_000,))
    assert set(np.unique(w)) == {1.0, 0.5, 0.25, 0.125, 0.0625}
    u = synth.uniform_f32(1, 4, (1_000_000,))
    assert u.min() > 0 and u.max() < 1 and abs(u.mean() - 0.5) < 2e-3


def test_group_bytes_per_query_decode_128k():
    # index-K scan + 4 layers x 2048 gathered 1152-byte rows + q/out/q_idx/w/idx
    assert synth.group_bytes_per_query(synth.DECODE_128K) == 43_565_184
