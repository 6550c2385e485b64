"""Pins for the oracle's E4M3 (OCP 8-bit float) paths (CPU only).

The FP8 cache format is the one the GLM context-window page names for its KV
cache ("Le contexte d'un million de tokens", section on agent reinforcement
learning).  The decoder is tied to torch's float8_e4m3fn dtype on every code
and to code points of the OCP definition; the FP8 indexer and attention are
tied to their bf16 counterparts on values that both formats hold exactly (every
E4M3 value is a bf16 value), so a mistake in how the FP8 variants read their
elements fails an equality here, and the bf16 functions carry their own pins."""
import numpy as np
import pytest
import torch

import oracle
import synth


def bf16(x):
    f = np.asarray(x, np.float32)
    assert np.array_equal((f.view(np.uint32) & 0xFFFF), np.zeros(f.shape, np.uint32))
    return (f.view(np.uint32) >> 16).astype(np.uint16)


ALL = np.arange(256, dtype=np.uint8)
FINITE = ALL[(ALL & 0x7F) != 0x7F]


def torch_e4m3(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_decode_matches_torch_on_every_code():
    got = oracle.e4m3_decode(ALL)
    want = torch_e4m3(ALL)
    nan = (ALL & 0x7F) == 0x7F
    assert np.isnan(got[nan]).all() and np.isnan(want[nan]).all()
    np.testing.assert_array_equal(got[~nan], want[~nan])
    np.testing.assert_array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


@pytest.mark.parametrize("code,value", [
    (0x38, 1.0), (0x40, 2.0), (0x44, 3.0), (0x48, 4.0), (0x30, 0.5),
    (0x7E, 448.0),            # largest finite: 1.75 * 2^8
    (0x08, 2.0 ** -6),        # smallest normal
    (0x07, 0.875 * 2.0 ** -6),  # largest subnormal
    (0x01, 2.0 ** -9),        # smallest subnormal
    (0x00, 0.0), (0xB8, -1.0), (0xC4, -3.0), (0xFE, -448.0)])
def test_decode_ocp_code_points(code, value):
    assert oracle.e4m3_decode(np.array([code], np.uint8))[0] == value


def test_decode_nan_and_negative_zero():
    v = oracle.e4m3_decode(np.array([0x7F, 0xFF, 0x80], np.uint8))
    assert np.isnan(v[0]) and np.isnan(v[1])
    assert v[2] == 0.0 and np.signbit(v[2])


def test_decode_is_monotone_over_positive_codes():
    v = oracle.e4m3_decode(np.arange(0x00, 0x7F, dtype=np.uint8))
    assert (np.diff(v) > 0).all()


def test_input_encoder_round_trips_and_matches_torch():
    # The seeded-input encoder (not part of the oracle) must invert the
    # decoder on every finite code and agree with torch's rounding in range.
    vals = oracle.e4m3_decode(FINITE).astype(np.float32)
    enc = synth.to_e4m3(vals)
    np.testing.assert_array_equal(oracle.e4m3_decode(enc), vals.astype(np.float64))
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(20000) * rng.choice([0.01, 1.0, 50.0], 20000)).astype(np.float32)
    x = np.clip(x, -440.0, 440.0)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(synth.to_e4m3(x), want)
    assert synth.to_e4m3(np.array([1e6, -1e6], np.float32)).tolist() == [0x7E, 0xFE]


def _random_finite_codes(rng, shape, max_code=0x5F):
    """Random finite E4M3 codes with |value| <= decode(max_code)."""
    return (rng.integers(0, max_code + 1, size=shape) | (rng.integers(0, 2, size=shape) << 7)).astype(np.uint8)


def test_fp8_indexer_equals_bf16_indexer_on_shared_values():
    rng = np.random.default_rng(11)
    B, T, H, D, L = 2, 3, 32, 128, 300
    qc = _random_finite_codes(rng, (B, T, H, D))
    kc = _random_finite_codes(rng, (B, L, D))
    w = synth.pow2_f32(5, 17, (B, T, H))
    pos = np.array([[L - 1, 150, 0], [L - 1, L - 2, 7]], np.int32)
    got = oracle.indexer_scores(qc, w, kc, pos, fp8=True)
    qb = bf16(oracle.e4m3_decode(qc).astype(np.float32))
    kb = bf16(oracle.e4m3_decode(kc).astype(np.float32))
    want = oracle.indexer_scores(qb, w, kb, pos)
    np.testing.assert_array_equal(got, want)


def test_fp8_indexer_on_generated_integer_inputs_equals_bf16():
    cfg = synth.GroupConfig("fp8_idx", seed=4, B=2, T=2, L=512, first_pos=500, k=64)
    pos = cfg.q_pos()
    got = oracle.indexer_scores(cfg.q_idx_fp8(), cfg.w(), cfg.k_idx_fp8(), pos, fp8=True)
    want = oracle.indexer_scores(cfg.q_idx(), cfg.w(), cfg.k_idx(), pos)
    np.testing.assert_array_equal(got, want)


def test_fp8_attention_equals_bf16_attention_on_shared_values():
    rng = np.random.default_rng(12)
    B, T, Hq, Dqk, L, k = 2, 2, 8, 576, 200, 48
    q = synth.normal_bf16(9, 1, (B, T, Hq, Dqk))
    kvc = synth.to_e4m3(rng.standard_normal((B, L, Dqk)).astype(np.float32))
    idx = np.sort(rng.choice(L, size=(B, T, k)), axis=-1).astype(np.int32)
    idx[0, 0, :5] = -1
    out, lse = oracle.sparse_mla_attn(q, kvc, idx, 0.0417, kv_fp8=True)
    kvb = bf16(oracle.e4m3_decode(kvc).astype(np.float32))
    out2, lse2 = oracle.sparse_mla_attn(q, kvb, idx, 0.0417)
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)


def test_fp8_group_equals_bf16_group_on_shared_values():
    cfg = synth.GroupConfig("fp8_group", seed=5, B=1, T=2, L=256, first_pos=200, k=32, n_layers=2)
    rng = np.random.default_rng(13)
    pos = cfg.q_pos()
    kvc = [synth.to_e4m3(rng.standard_normal((cfg.B, cfg.L, cfg.Dqk)).astype(np.float32)) for _ in range(2)]
    kvb = [bf16(oracle.e4m3_decode(c).astype(np.float32)) for c in kvc]
    qs = [cfg.q_attn(l) for l in range(2)]
    s8, i8, o8, l8 = oracle.layer_group(cfg.q_idx_fp8(), cfg.w(), cfg.k_idx_fp8(), pos, cfg.k, qs, kvc,
                                        cfg.sm_scale, idx_fp8=True, kv_fp8=True)
    sb, ib, ob, lb = oracle.layer_group(cfg.q_idx(), cfg.w(), cfg.k_idx(), pos, cfg.k, qs, kvb, cfg.sm_scale)
    np.testing.assert_array_equal(s8, sb)
    np.testing.assert_array_equal(i8, ib)
    for a, b in zip(o8 + l8, ob + lb):
        np.testing.assert_array_equal(a, b)
