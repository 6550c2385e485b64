"""GPU parity of the multi-round MTP loop against the CPU oracle: target-only
verification, the cache commit, and whole rounds chained on the device
(indexer -> top-k -> draft attention steps -> verification -> commit), with the
host reading nothing between rounds."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import (ATTN_TOL, DEV, RATIO_BAND, assert_attn_close, bf16_dev, f32_dev, host, i32_dev, say,
                         inv_cdf_valid)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    import long_context_sparse_scores_amd as m
    assert torch.cuda.is_available()
    return m


def u8_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.uint8)).to(DEV)


# ------------------------------------------------------------------ target-only verification
@pytest.mark.parametrize("V", [151552, 1000, 8193])
def test_target_only_matches_oracle(dsa, V):
    rng = np.random.default_rng(V)
    B, S = 16, 7
    say("target-only verify B=%d S=%d V=%d" % (B, S, V))
    t = (rng.standard_normal((B, S + 1, V)) * 2).astype(np.float32)
    # equal maxima in two chunks (and inside one chunk): the lower index is the first choice
    top = t.max() + 1.0
    t[0, 0, [V - 1, 5]] = top
    t[1, 2, [17, 18]] = top
    am = t[:, :S].argmax(-1).astype(np.int32)
    other = (am + rng.integers(1, V, (B, S))) % V
    tok = np.where(rng.random((B, S)) < 0.75, am, other).astype(np.int32)
    tok[0, 0], tok[1, :3] = 5, am[1, :3]
    n, nxt = dsa.mtp_verify_target_only(f32_dev(t), i32_dev(tok))
    rn, rnxt = oracle.mtp_verify_target_only(t, tok)
    np.testing.assert_array_equal(host(n), rn)
    np.testing.assert_array_equal(host(nxt), rnxt)
    assert rn[0] >= 1 and rn[1] >= 3


# ------------------------------------------------------------------ commit
@pytest.mark.parametrize("fp8", [False, True])
def test_commit_matches_oracle(dsa, fp8):
    rng = np.random.default_rng(5 + fp8)
    B, S, L = 6, 7, 300
    say("commit fp8=%s" % fp8)
    dt = np.uint8 if fp8 else np.uint16
    k_cache = rng.integers(0, 250, (B, L, 128)).astype(dt)
    kv_cache = rng.integers(0, 250, (B, L, 576)).astype(dt)
    new_k = rng.integers(0, 250, (B, S + 1, 128)).astype(dt)
    new_kv = rng.integers(0, 250, (B, S + 1, 576)).astype(dt)
    q_pos = np.array([0, 10, 100, L - 9, L - 4, L - 1], np.int32)  # the last two run into the capacity
    n_acc = np.array([7, 0, 3, 7, 7, 2], np.int32)
    dev = u8_dev if fp8 else (lambda a: torch.from_numpy(a.view(np.int16)).to(DEV))
    dk, dkv = dev(k_cache), dev(kv_cache)
    out = dsa.mtp_commit(i32_dev(n_acc), i32_dev(q_pos), dev(new_k), dev(new_kv), dk, dkv)
    ref_out = oracle.mtp_commit(n_acc, q_pos, new_k, new_kv, k_cache, kv_cache)
    np.testing.assert_array_equal(host(out), ref_out)
    np.testing.assert_array_equal(dk.cpu().numpy().view(dt), k_cache)
    np.testing.assert_array_equal(dkv.cpu().numpy().view(dt), kv_cache)


# ------------------------------------------------------------------ whole rounds
class Rounds:
    """Seeded inputs of R rounds: step-1 indexer query, S draft attention
    queries, correlated target/draft logits, draft tokens drawn from the draft,
    uniforms, and the candidate cache rows the verifying pass produces."""

    def __init__(self, seed, B, R, S, V, rho=0.9, boost=11.0):
        self.B, self.R, self.S, self.V = B, R, S, V
        rng = np.random.default_rng(seed)
        self.q_idx = [synth.int_bf16(seed, 100 + r, (B, 1, 32, 128)) for r in range(R)]
        self.w = [synth.pow2_f32(seed, 200 + r, (B, 1, 32)) for r in range(R)]
        self.q_steps = [[synth.normal_bf16(seed, 1000 + 16 * r + i, (B, 1, 64, 576)) for i in range(S)]
                        for r in range(R)]
        # N(0, 2^2) logits with one favoured token per position (+boost), so
        # that the target's first choice is often the token the draft draws
        self.target = []
        for _ in range(R):
            t = (rng.standard_normal((B, S + 1, V)) * 2).astype(np.float32)
            fav = rng.integers(0, V, (B, S + 1))
            np.put_along_axis(t, fav[..., None], np.take_along_axis(t, fav[..., None], -1) + boost, -1)
            self.target.append(t)
        self.draft = [(rho * t[:, :S] + np.sqrt(1 - rho * rho) * rng.standard_normal((B, S, V)) * 2)
                      .astype(np.float32) for t in self.target]
        self.tok = [synth.gumbel_argmax(seed, 300 + r, d).astype(np.int32) for r, d in enumerate(self.draft)]
        self.u = [rng.random((B, S)).astype(np.float32) for _ in range(R)]
        self.ur = [rng.random(B).astype(np.float32) for _ in range(R)]
        self.new_k = [synth.int_bf16(seed, 400 + r, (B, S + 1, 128)) for r in range(R)]
        self.new_kv = [synth.normal_bf16(seed, 500 + r, (B, S + 1, 576)) for r in range(R)]

    def clear_margins(self, rng):
        """Move acceptance uniforms away from p/q so that every decision is clear
        of the fp32 band (decisions only; the oracle decides which is right)."""
        for r in range(self.R):
            ratio = oracle.mtp_verify(self.target[r], self.draft[r], self.tok[r], self.u[r], self.ur[r])["ratio"]
            close = np.abs(self.u[r] - ratio) <= 100 * RATIO_BAND * np.maximum(1.0, ratio)
            self.u[r][close] = np.where(ratio[close] > 0.5, 0.01, 0.99).astype(np.float32)


def _oracle_rounds(cfg, rd, k_cache, kv_cache, q_pos, rule):
    res = []
    for r in range(rd.R):
        out = oracle.mtp_round(rd.q_idx[r], rd.w[r], k_cache, q_pos.reshape(-1, 1), cfg.k, rd.q_steps[r], kv_cache,
                               cfg.sm_scale, rd.target[r], rd.draft[r], rd.tok[r], rd.u[r], rd.ur[r], rd.new_k[r],
                               rd.new_kv[r], rule=rule)
        res.append(out)
        q_pos = out["q_pos_next"]
    return res, q_pos


@pytest.mark.parametrize("rule,entry", [("rejection", "separate"), ("target_only", "separate"),
                                        ("rejection", "group")])
def test_rounds_chained_on_device_match_oracle(dsa, rule, entry):
    # entry "group": the draft path of a round is one dsa_layer_group call whose
    # layers are the draft steps (all over the one latent cache), as bench.py runs it
    B, R, S, V, L = 3, 4, 7, 3000, 6144
    cfg = synth.GroupConfig("rounds", seed=12, B=B, T=1, L=L, first_pos=0, k=256)
    rd = Rounds(77, B, R, S, V)
    rd.clear_margins(np.random.default_rng(1))
    q_pos0 = np.array([4000, 5200, 3000], np.int32)
    k_cache, kv_cache = cfg.k_idx().copy(), cfg.kv(0).copy()
    say("rounds %s via %s entry points: GPU" % (rule, entry))
    dk, dkv = bf16_dev(k_cache), bf16_dev(kv_cache)
    qp = [i32_dev(q_pos0), torch.empty(B, dtype=torch.int32, device=DEV)]
    gpu = []
    for r in range(R):
        cur, nxt_buf = qp[r % 2], qp[(r + 1) % 2]
        pos2 = cur.view(B, 1)
        if entry == "group":
            idx, outs, _ = dsa.layer_group(bf16_dev(rd.q_idx[r]), f32_dev(rd.w[r]), dk, pos2, cfg.k,
                                           [bf16_dev(q) for q in rd.q_steps[r]], [dkv] * S, cfg.sm_scale)
        else:
            scores = dsa.indexer_scores(bf16_dev(rd.q_idx[r]), f32_dev(rd.w[r]), dk, pos2)
            idx = dsa.topk(scores, pos2, cfg.k)
            outs = [dsa.sparse_mla_attn(bf16_dev(q), dkv, idx, cfg.sm_scale) for q in rd.q_steps[r]]
        if rule == "rejection":
            _, n_acc, nt = dsa.mtp_draft_verify(f32_dev(rd.target[r]), f32_dev(rd.draft[r]), i32_dev(rd.tok[r]),
                                                f32_dev(rd.u[r]), f32_dev(rd.ur[r]))
        else:
            n_acc, nt = dsa.mtp_verify_target_only(f32_dev(rd.target[r]), i32_dev(rd.tok[r]))
        dsa.mtp_commit(n_acc, cur, bf16_dev(rd.new_k[r]), bf16_dev(rd.new_kv[r]), dk, dkv, q_pos_out=nxt_buf)
        gpu.append((idx, outs, n_acc, nt))
    torch.cuda.synchronize()
    say("rounds %s: oracle" % rule)
    ref, q_final = _oracle_rounds(cfg, rd, k_cache, kv_cache, q_pos0.copy(), rule)
    for r in range(R):
        idx, outs, n_acc, nt = gpu[r]
        np.testing.assert_array_equal(host(idx), ref[r]["idx"], err_msg="round %d index list" % r)
        np.testing.assert_array_equal(host(n_acc), ref[r]["n_acc"], err_msg="round %d acceptance" % r)
        got_nt, ref_nt = host(nt), ref[r]["next_tok"]
        for b in range(B):  # a resampled token may differ only inside the fp32 CDF band
            if got_nt[b] != ref_nt[b]:
                assert rule == "rejection"
                na = int(ref[r]["n_acc"][b])
                p = oracle.softmax_row(rd.target[r][b, na])
                rr = np.maximum(p - oracle.softmax_row(rd.draft[r][b, na]), 0.0) if na < S else p
                assert inv_cdf_valid(rr, float(rd.ur[r][b]), int(got_nt[b]))
        for i in (0, S - 1):
            assert_attn_close(host(outs[i]), ref[r]["outs"][i], "round %d step %d" % (r, i))
    np.testing.assert_array_equal(host(qp[R % 2]), q_final)
    np.testing.assert_array_equal(dk.view(torch.int16).cpu().numpy().view(np.uint16), k_cache)
    np.testing.assert_array_equal(dkv.view(torch.int16).cpu().numpy().view(np.uint16), kv_cache)
    acc = np.array([ref[r]["n_acc"] for r in range(R)])
    say("rounds %s: acceptance lengths %s" % (rule, (acc + 1).tolist()))
