"""The host C code under AddressSanitizer and UndefinedBehaviorSanitizer.

The oracle (oracle/oracle.c) and the input generator (synth/synth.c) are
rebuilt with -fsanitize=address,undefined into a temporary directory and
every exported function is driven on small, ragged inputs (a partial key
tile, masked and repeated index entries, k above the visible count, a vocab
that is not a multiple of anything, E4M3 rows) in a child process with the
sanitizer runtimes preloaded.  Any report fails the test.  Runs on the CPU
only; the GPU code is not built with sanitizers."""
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]

DRIVER = textwrap.dedent('''
    import sys
    import numpy as np
    sys.path.insert(0, ROOT)
    import oracle, synth
    oracle._LIB_PATH = ORACLE_SO
    synth._LIB_PATH = SYNTH_SO
    rng = np.random.default_rng(0)
    B, T, L, k = 2, 3, 333, 64
    qi = synth.int_bf16(7, 1, (B, T, 32, 128))
    w = synth.pow2_f32(7, 2, (B, T, 32))
    ki = synth.int_bf16(7, 3, (B, L + 5, 128))
    pos = np.array([[0, 40, L - 1], [L - 1, 200, 63]], np.int32)
    s = oracle.indexer_scores(qi, w, ki, pos, L=L)
    idx = oracle.topk(s, pos, k)
    idx[0, 1, 3] = -1
    idx[1, 2, 5] = L + 2
    idx[1, 0, 7] = idx[1, 0, 6]
    q = synth.normal_bf16(7, 4, (B, T, 64, 576))
    kv = synth.normal_bf16(7, 5, (B, L, 576))
    oracle.sparse_mla_attn(q, kv, idx, 1 / 16)
    oracle.layer_group(qi, w, ki[:, :L], pos, k, [q, q], [kv, kv], 1 / 16)
    q8, k8 = synth.to_e4m3(synth.bf16_to_f32(qi)), synth.to_e4m3(synth.bf16_to_f32(ki))
    oracle.indexer_scores(q8, w, k8, pos, L=L, fp8=True)
    kv8 = synth.to_e4m3(synth.bf16_to_f32(kv))
    oracle.sparse_mla_attn(q, kv8, idx, 1 / 16, kv_fp8=True)
    oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    S, V = 3, 1001
    tgt = synth.normal_f32(7, 6, (B, S + 1, V), scale=2.0)
    dft = synth.mix_f32(7, 7, tgt[:, :S], 0.9, 0.43589, 2.0)
    tok = synth.gumbel_argmax(7, 8, dft)
    tok[1, 2] = V + 3
    ua, ur = synth.uniform_f32(7, 9, (B, S)), synth.uniform_f32(7, 10, (B,))
    oracle.mtp_verify(tgt, dft, tok, ua, ur)
    oracle.mtp_verify_target_only(tgt, tok)
    kc = synth.int_bf16(7, 11, (B, 50, 128))
    kvc = synth.normal_bf16(7, 12, (B, 50, 576))
    nk, nkv = synth.int_bf16(7, 13, (B, S + 1, 128)), synth.normal_bf16(7, 14, (B, S + 1, 576))
    oracle.mtp_commit(np.array([S, 0], np.int32), np.array([45, 10], np.int32), nk, nkv, kc, kvc)
    synth.raw_u64(7, 15, 17)
    synth.normal_bf16_rows(7, 16, np.array([0, 576, 1153]), 576)
    synth.int_bf16_rows(7, 17, np.array([3, 130]), 128)
    print("driver done", flush=True)
''')


def _runtime(name):
    path = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_and_synth_under_sanitizers(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    libs = {}
    for name, src, extra in (("oracle", "oracle/oracle.c", []), ("synth", "synth/synth.c", ["-ffp-contract=off"])):
        out = str(tmp_path / ("lib%s_san.so" % name))
        subprocess.run(["gcc"] + SAN + extra + ["-fopenmp", "-shared", "-fPIC", "-Wall", "-Werror", "-o", out,
                                               os.path.join(ROOT, src), "-lm"], check=True)
        libs[name] = out
    script = tmp_path / "driver.py"
    script.write_text("ROOT = %r\nORACLE_SO = %r\nSYNTH_SO = %r\n" % (ROOT, libs["oracle"], libs["synth"]) + DRIVER)
    env = dict(os.environ, LD_PRELOAD=asan + ":" + ubsan, OMP_NUM_THREADS="2",
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, str(script)], capture_output=True, text=True, env=env, timeout=600)
    report = r.stdout + r.stderr
    assert r.returncode == 0 and "driver done" in r.stdout, report[-4000:]
    assert "AddressSanitizer" not in report and "runtime error" not in report, report[-4000:]
