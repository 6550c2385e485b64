"""The no-allocation group entry point (dsa_layer_group_noalloc) against
dsa_layer_group on the same inputs, through the C ABI: the same kernels run
on the library's static per-GPU scratch instead of a caller workspace, so the
index lists and every layer's output must be equal bit for bit.  Two calls in
a row, the second smaller than the first (the scratch keeps the first call's
contents)."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from gpu_helpers import DEV, bf16_dev, f32_dev, i32_dev, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    import long_context_sparse_scores_amd as m
    assert torch.cuda.is_available()
    return m


def _inputs(seed, B, L, n_layers):
    q_idx = synth.int_bf16(seed, 1, (B, 1, 32, 128))
    w = synth.pow2_f32(seed, 2, (B, 1, 32))
    k_idx = synth.int_bf16(seed, 3, (B, L, 128))
    pos = np.full((B, 1), L - 1, np.int32)
    pos[0, 0] = L // 3  # a shorter row too
    qs = [synth.normal_bf16(seed, 10 + l, (B, 1, 64, 576)) for l in range(n_layers)]
    kvs = [synth.normal_bf16(seed, 20 + l, (B, L, 576)) for l in range(n_layers)]
    return (bf16_dev(q_idx), f32_dev(w), bf16_dev(k_idx), i32_dev(pos), [bf16_dev(q) for q in qs],
            [bf16_dev(kv) for kv in kvs])


def _outputs(B, k, n_layers):
    idx = torch.full((B, 1, k), -9, dtype=torch.int32, device=DEV)
    outs = [torch.zeros((B, 1, 64, 512), dtype=torch.bfloat16, device=DEV) for _ in range(n_layers)]
    return idx, outs


@pytest.mark.parametrize("calls", [[(8, 40000, 3), (3, 9000, 2)]])
def test_noalloc_group_matches_workspace_group(dsa, calls):
    lib = dsa.lib()
    stream = torch.cuda.current_stream(DEV).cuda_stream
    k = 2048
    for seed, (B, L, n) in enumerate(calls, start=80):
        say("no-allocation group B=%d L=%d layers=%d" % (B, L, n))
        q_idx, w, k_idx, pos, qs, kvs = _inputs(seed, B, L, n)
        idx_a, outs_a = _outputs(B, k, n)
        a = dsa.make_group_args(q_idx, w, k_idx, pos, k, qs, kvs, 1 / 16, idx_a, outs_a)
        assert dsa.layer_group_workspace_size(a) <= dsa.NOALLOC_SCRATCH_BYTES
        assert lib.dsa_layer_group_noalloc(ctypes.byref(a), stream) == 0, dsa.last_error()
        idx_b, outs_b = _outputs(B, k, n)
        dsa.layer_group(q_idx, w, k_idx, pos, k, qs, kvs, 1 / 16, idx_out=idx_b, outs=outs_b)
        torch.cuda.synchronize()
        assert torch.equal(idx_a, idx_b)
        assert int((idx_a[0, 0] >= 0).sum()) == min(k, L // 3 + 1)
        for l in range(n):
            assert torch.equal(outs_a[l].view(torch.int16), outs_b[l].view(torch.int16)), "layer %d" % l
