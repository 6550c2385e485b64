#!/usr/bin/env python3
"""Benchmark of the DSA sparse-attention hot path on one MI355X.

A step is one IndexShare group on the decode workload at 128K context:
indexer scoring of every cached key, top-2048 selection, then sparse
absorbed-MLA attention for each of the 4 layers with the shared index list
(dsa_layer_group), for batch 32 with one query token per sequence.  Inputs
are synthetic and seeded (synth/), resident in HBM before timing starts.

Prints ONE JSON line: throughput in query tokens per second, the HBM
roofline of the dominant kernel (the index-key scan), a per-phase breakdown
and the CPU oracle timed on a bounded sample of the same workload.  The
default run then times decode_1m_b4, prefill_4096_at_128k and
mtp_draft_b16_128k the same way (fewer steps, shorter oracle samples) and
reports each under "extra_workloads"; --no-extras skips them.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

Other workloads (--workload): decode_1m_b4 and tiny_decode_8k time the same
group step; prefill_4096_at_128k times it for a 4096-query chunk and reports
the fraction of the bf16 MFMA peak; mtp_draft_b16_128k times one MTP draft
round (step-1 indexer and top-k over the backbone index keys, 7 attention
steps over the backbone latent cache with the step-1 list, verification);
mtp_rounds_b16_128k times 8 chained rounds of draft -> verify -> commit (the
kept rows appended on the device) with rejection sampling and, for an A/B,
with the target-only rule.  --index-fp8 / --kv-fp8 run the group workloads
over E4M3 index-key / latent caches.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, published
MFMA_FP8_PEAK_TFLOPS = 5000.0   # MI355X dense fp8 matrix peak, published
PREFILL_MIN_QUERIES = 8         # chunks of at least this many queries per sequence take the tile kernel
METRIC = "query-tokens/sec per 4-layer DSA group at 128K ctx; % of HBM roofline"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # Untimed steps first: from idle the GPU needs about 30 ms of work to reach
    # its steady clocks (decode 128K x 32: 0.2892 ms per step after 10 warm-up
    # steps, 0.2849 after 100, 0.2841 after 1000, 50 timed steps each).
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="decode_128k_b32",
                    help="decode_128k_b32 (default), decode_1m_b4, prefill_4096_at_128k, tiny_decode_8k, "
                         "mtp_draft_b16_128k, mtp_rounds_b16_128k")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time for the oracle sample")
    ap.add_argument("--indexer-only", action="store_true", help="time only the indexer (for counter runs)")
    ap.add_argument("--index-fp8", action="store_true", help="E4M3 index queries and keys (FP8 index cache)")
    ap.add_argument("--kv-fp8", action="store_true", help="E4M3 latent rows (FP8 latent cache)")
    ap.add_argument("--no-nonshared", action="store_true", help="skip timing the group without IndexShare")
    ap.add_argument("--no-extras", action="store_true",
                    help="time only the headline workload (default run: also decode_1m_b4, prefill_4096_at_128k "
                         "and mtp_draft_b16_128k under extra_workloads)")
    ap.add_argument("--extra-cpu-seconds", type=float, default=4.0, help="oracle sample time per extra workload")
    ap.add_argument("--copy-calibrate", action="store_true",
                    help="only run 5 device-to-device copies of 1 GiB (reference for HBM byte counters)")
    ap.add_argument("--write-traffic", metavar="DIR",
                    help="no GPU work: read rocprofv3 --pmc output folders DIR/fetch, DIR/write (FETCH_SIZE, "
                         "WRITE_SIZE of an --indexer-only run of this workload), DIR/cfetch, DIR/cwrite (the same "
                         "of --copy-calibrate) and, if present, DIR/gfetch, DIR/gwrite (a group run); write "
                         "profiles/<indexer>_<workload>_traffic.json and print the per-kernel table")
    return ap.parse_args()


def traffic_from_profiles(kernel: str, workload: str):
    """HBM bytes per launch measured with rocprofv3 counters, if a summary for
    this kernel, workload and kernel source exists under profiles/."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "%s_%s_traffic.json" % (kernel, workload))
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src = os.path.join(ROOT, "long_context_sparse_scores_amd", "csrc", rec.get("source", ""))
    if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest() != rec.get("source_sha256"):
        return None       # the kernel changed since the counters were taken
    return rec.get("bytes_per_launch")


# Workloads timed after the headline in the default run, each reported under
# "extra_workloads" with its own roofline and oracle baseline.
EXTRA_WORKLOADS = ("decode_1m_b4", "prefill_4096_at_128k", "mtp_draft_b16_128k")


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only (requested --gpus %d); the multi-GPU "
              "context-parallel path is a design, not a measured configuration." % args.gpus, file=sys.stderr)
        sys.exit(2)

    if args.write_traffic:
        write_traffic(args)
        return

    import torch

    if args.copy_calibrate:
        copy_calibrate(torch)
        return

    import synth

    line = run_workload(synth.CONFIGS[args.workload], args)
    if line is None:
        return
    if (args.workload == "decode_128k_b32" and not args.no_extras and not args.index_fp8 and not args.kv_fp8):
        extras = {}
        for name in EXTRA_WORKLOADS:
            torch.cuda.empty_cache()
            sub = argparse.Namespace(**vars(args))
            # the GPU is at its steady clocks by now; a few warm-up steps per workload suffice
            sub.steps, sub.warmup = max(5, args.steps // 2), max(2, min(args.warmup // 2, 10))
            sub.cpu_seconds = args.extra_cpu_seconds
            sub.workload = name
            sub.cpu_queries = 8 if name.startswith("prefill") else None
            r = run_workload(synth.CONFIGS[name], sub)
            extras[name] = {key: r[key] for key in ("metric", "value", "unit", "ms_per_step", "steps", "warmup",
                                                    "config", "hbm_roofline_frac", "algorithmic_bytes_per_step",
                                                    "mfma", "roofline", "breakdown", "indexshare",
                                                    "draft_steps_per_s", "mean_acceptance_length", "cpu_baseline")
                            if key in r}
        line["extra_workloads"] = extras
    print(json.dumps(line), flush=True)


def run_workload(cfg, args):
    """Time one workload; returns its JSON record (None for counter-only runs)."""
    import synth

    if isinstance(cfg, synth.MtpConfig):
        return bench_mtp(cfg, args)
    if isinstance(cfg, synth.MtpRoundsConfig):
        return bench_mtp_rounds(cfg, args)
    return bench_group(cfg, args)


def bench_group(cfg, args):
    """One dsa_layer_group per step (indexer, top-k, every layer's attention)."""
    import ctypes

    import numpy as np
    import torch

    import long_context_sparse_scores_amd as dsa
    import synth

    dev = torch.device("cuda:0")
    B, T, L, k, nl = cfg.B, cfg.T, cfg.L, cfg.k, cfg.n_layers
    log("bench: workload %s B=%d T=%d L=%d k=%d layers=%d" % (cfg.name, B, T, L, k, nl))

    def to_dev(a):
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

    t0 = time.time()
    idx_elem = 1 if args.index_fp8 else 2   # bytes per index-cache element
    if args.index_fp8:
        q_idx = torch.from_numpy(cfg.q_idx_fp8()).to(dev)
        k_idx = torch.from_numpy(cfg.k_idx_fp8()).to(dev)
    else:
        q_idx = to_dev(cfg.q_idx())
        k_idx = to_dev(cfg.k_idx())
    w = torch.from_numpy(cfg.w()).to(dev)
    q_pos = torch.from_numpy(cfg.q_pos()).to(dev)
    qs = [to_dev(cfg.q_attn(l)) for l in range(nl)]
    kv_elem = 1 if args.kv_fp8 else 2   # bytes per latent-cache element
    kvs = []
    if args.kv_fp8:  # E4M3 rows, converted one sequence at a time
        for l in range(nl):
            kvs.append(torch.empty((B, L, cfg.Dqk), dtype=torch.uint8, device=dev))
            for b in range(B):
                kvs[l][b].copy_(torch.from_numpy(cfg.kv_seq_fp8(l, b)[0]))
    else:
        host_kv = np.empty((B, L, cfg.Dqk), np.uint16)
        for l in range(nl):
            cfg.kv(l, out=host_kv)
            kvs.append(to_dev(host_kv))
        del host_kv
    torch.cuda.synchronize()
    log("bench: inputs generated and resident in HBM (%.1f s)" % (time.time() - t0))

    idx = torch.empty((B, T, k), dtype=torch.int32, device=dev)
    outs = [torch.empty((B, T, cfg.Hq, cfg.Dv), dtype=torch.bfloat16, device=dev) for _ in range(nl)]
    args_c = dsa.make_group_args(q_idx, w, k_idx, q_pos, k, qs, kvs, cfg.sm_scale, idx, outs)
    ws_bytes = dsa.layer_group_workspace_size(args_c)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)  # zero-filled before first use
    lib = dsa.lib()
    stream = torch.cuda.current_stream(dev).cuda_stream
    argp = ctypes.byref(args_c)

    def group_step():
        rc = lib.dsa_layer_group(argp, ws.data_ptr(), ws_bytes, stream)
        if rc != 0:
            raise RuntimeError(dsa.last_error())

    scores = ws[: B * T * L * 4].view(torch.float32).view(B, T, L)

    indexer_fn = dsa.indexer_scores_fp8 if args.index_fp8 else dsa.indexer_scores

    def indexer_step():
        indexer_fn(q_idx, w, k_idx, q_pos, scores=scores)

    # ---------------- timed group steps
    if not args.indexer_only:
        for _ in range(args.warmup):
            group_step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            group_step()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        log("bench: group step %.3f ms" % ms)

    # ---------------- dominant kernel: the index-key scan, timed alone on the same stream
    for _ in range(args.warmup):
        indexer_step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        indexer_step()
    e1.record()
    torch.cuda.synchronize()
    idx_ms = e0.elapsed_time(e1) / args.steps
    idx_bytes = B * T * (L * cfg.D * idx_elem + cfg.H * cfg.D * idx_elem + cfg.H * 4)
    log("bench: indexer %.3f ms, %.1f GB/s" % (idx_ms, idx_bytes / idx_ms / 1e6))
    if args.indexer_only:
        return None

    # ---------------- per-phase breakdown (same kernels, called one entry point at a time)
    topk_ws = torch.empty(dsa.topk_workspace_size(B, T, L, k), dtype=torch.uint8, device=dev)
    attn_ws = torch.empty(max(256, dsa.attn_workspace_size(B, T, k)), dtype=torch.uint8, device=dev)
    phase = np.zeros(2 + nl)
    reps = max(5, args.steps // 5)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3 + nl)] for _ in range(reps + 2)]
    # Group steps queued first keep the GPU busy while the host queues the
    # phases, so no event sees the GPU idle waiting for the next launch.
    for _ in range(20):
        group_step()
    for r in range(reps + 2):
        ev = evs[r]
        ev[0].record()
        indexer_step()
        ev[1].record()
        dsa.topk(scores, q_pos, k, idx=idx, ws=topk_ws)
        ev[2].record()
        for l in range(nl):
            dsa.sparse_mla_attn(qs[l], kvs[l], idx, cfg.sm_scale, out=outs[l], ws=attn_ws)
            ev[3 + l].record()
    torch.cuda.synchronize()
    for ev in evs[2:]:
        phase += [ev[i].elapsed_time(ev[i + 1]) for i in range(2 + nl)]
    phase /= reps
    breakdown = {"indexer_ms": round(phase[0], 4), "topk_ms": round(phase[1], 4),
                 "attn_ms_per_layer": [round(x, 4) for x in phase[2:]]}
    log("bench: breakdown %s" % breakdown)

    # ---------------- without IndexShare (dsa_layer_group with share = 0): every layer runs its own
    # indexer and top-k over its own index queries, weights and index-key cache; the measured saving
    ns_ms = None
    if not args.no_nonshared and T == 1:
        def layer_keys(l):
            kb = synth.int_bf16(cfg.seed, synth.T_K_IDX + 100 + l, (B, L, cfg.D))
            return torch.from_numpy(synth.to_e4m3(synth.bf16_to_f32(kb))).to(dev) if args.index_fp8 else to_dev(kb)

        def layer_queries(l):
            qb = synth.int_bf16(cfg.seed, synth.T_K_IDX + 200 + l, (B, T, cfg.H, cfg.D))
            return torch.from_numpy(synth.to_e4m3(synth.bf16_to_f32(qb))).to(dev) if args.index_fp8 else to_dev(qb)

        k_idx_l = [k_idx] + [layer_keys(l) for l in range(1, nl)]
        q_idx_l = [q_idx] + [layer_queries(l) for l in range(1, nl)]
        w_l = [w] + [torch.from_numpy(synth.pow2_f32(cfg.seed, synth.T_K_IDX + 300 + l, (B, T, cfg.H))).to(dev)
                     for l in range(1, nl)]
        idx_l = [torch.empty_like(idx) for _ in range(nl)]
        args_ns = dsa.make_group_args(q_idx_l, w_l, k_idx_l, q_pos, k, qs, kvs, cfg.sm_scale, idx_l, outs)
        argp_ns = ctypes.byref(args_ns)

        def nonshared_step():
            rc = lib.dsa_layer_group(argp_ns, ws.data_ptr(), ws_bytes, stream)
            if rc != 0:
                raise RuntimeError(dsa.last_error())

        for _ in range(2):
            nonshared_step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            nonshared_step()
        e1.record()
        torch.cuda.synchronize()
        ns_ms = e0.elapsed_time(e1) / reps
        del k_idx_l, q_idx_l, w_l, idx_l, args_ns, argp_ns
        log("bench: without IndexShare %.3f ms per group (shared %.3f ms)" % (ns_ms, ms))

    qtok = B * T
    value = qtok / (ms / 1e3)
    if T == 1:
        step_bytes = qtok * synth.group_bytes_per_query(cfg, idx_elem=idx_elem, kv_elem=kv_elem)
    else:
        # a chunk of queries shares one key scan and gathers rows out of the same
        # cached layers: count each cache byte once, plus per-query inputs and outputs
        step_bytes = (B * L * cfg.D * idx_elem + qtok * (cfg.H * cfg.D * idx_elem + cfg.H * 4 + k * 4)
                      + nl * (B * min(L, T * k) * cfg.Dqk * kv_elem + qtok * cfg.Hq * (cfg.Dqk + cfg.Dv) * 2))
    achieved = idx_bytes / (idx_ms / 1e3) / 1e9
    pos = cfg.q_pos().astype(np.int64)
    idx_flops = int(((np.minimum(pos, L - 1) + 1) * cfg.H * cfg.D * 2).sum())
    attn_flops = nl * qtok * cfg.Hq * k * (cfg.Dqk + cfg.Dv) * 2
    if T >= PREFILL_MIN_QUERIES:
        # a chunk of queries runs the matrix-core tile kernel: one key scan for the
        # whole chunk, bound by the matrix peak of its input type rather than by HBM
        idx_tflops = idx_flops / (idx_ms / 1e3) / 1e12
        peak = MFMA_FP8_PEAK_TFLOPS if args.index_fp8 else MFMA_BF16_PEAK_TFLOPS
        roofline = {"kernel": "indexer_prefill_fp8_kernel" if args.index_fp8 else "indexer_prefill_kernel",
                    "bound": "mfma", "achieved": round(idx_tflops, 1), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(idx_tflops / peak, 4), "traffic": None, "flops_per_launch": idx_flops,
                    "avg_launch_ms": round(idx_ms, 4)}
    else:
        roofline = {"kernel": "indexer_decode_fp8_kernel" if args.index_fp8 else "indexer_decode_kernel",
                    "bound": "hbm", "achieved": round(achieved, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": traffic_from_profiles("indexer_fp8" if args.index_fp8 else "indexer", cfg.name),
                    "bytes_per_launch": idx_bytes, "avg_launch_ms": round(idx_ms, 4)}
        if T > 1:
            roofline["note"] = "each query row rescans the keys (through the caches); bytes count them per query"
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {(False, False): "bf16", (True, False): "fp8(e4m3) index scan, bf16 attention",
                  (False, True): "bf16 index scan, bf16 attention over e4m3 rows",
                  (True, True): "fp8(e4m3) index scan, bf16 attention over e4m3 rows"}[(args.index_fp8, args.kv_fp8)],
        "data": "synthetic (seeded counter-based generator; GLM-5.2 shapes)",
        "config": {"workload": cfg.name, "index_cache": "e4m3" if args.index_fp8 else "bf16",
                   "latent_cache": "e4m3" if args.kv_fp8 else "bf16",
                   "batch": B, "query_tokens_per_seq": T, "context": L, "topk": k,
                   "layers_per_group": nl, "index_heads": cfg.H, "index_dim": cfg.D, "attn_heads": cfg.Hq,
                   "latent_dim": cfg.Dqk, "value_dim": cfg.Dv},
        "hbm_roofline_frac": round(step_bytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
        "algorithmic_bytes_per_step": step_bytes,
        "roofline": roofline,
        "breakdown": breakdown,
        "cpu_baseline": None,
    }
    if ns_ms is not None:
        line["indexshare"] = {"shared_ms": round(ms, 4), "non_shared_ms": round(ns_ms, 4),
                              "speedup": round(ns_ms / ms, 3),
                              "note": "non-shared: dsa_layer_group with share = 0, an indexer and top-k per layer "
                                      "over that layer's own index queries, weights and index-key cache"}
    if T > 1:  # a prefill chunk is a dense contraction: report the matrix-core fraction as well
        tflops = (idx_flops + attn_flops) / (ms / 1e3) / 1e12
        line["mfma"] = {"flops_per_step": idx_flops + attn_flops, "achieved_tflops": round(tflops, 1),
                        "peak_tflops": MFMA_BF16_PEAK_TFLOPS, "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                        "indexer_tflops": round(idx_flops / (idx_ms / 1e3) / 1e12, 1)}
    if not args.no_cpu:
        prefill = cfg.T >= PREFILL_MIN_QUERIES
        line["cpu_baseline"] = cpu_baseline(
            cfg, args.cpu_seconds, index_fp8=args.index_fp8, kv_fp8=args.kv_fp8,
            queries=getattr(args, "cpu_queries", None) or (64 if prefill else None),
            single_thread=args.workload == "decode_128k_b32")
    return line


def copy_calibrate(torch):
    """A plain copy of known size: its FETCH_SIZE / WRITE_SIZE readings per
    dispatch, divided by 1 GiB, calibrate the same counters on other kernels."""
    dev = torch.device("cuda:0")
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("bench: 5 copies of %d bytes done" % n)


def read_counter(folder, counter):
    """Per-dispatch values of one rocprofv3 counter: {kernel name: [values in
    dispatch order]}, summed over the rows of each dispatch."""
    import csv
    import glob
    per = {}
    for f in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                key = (int(r["Dispatch_Id"]), r["Kernel_Name"])
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (d, name) in sorted(per):
        out.setdefault(name, []).append(per[(d, name)])
    return out


def short_kernel_name(name):
    return name.replace("void ", "").replace("dsa::(anonymous namespace)::", "").split("(")[0].strip()


def write_traffic(args):
    """HBM bytes per launch from FETCH_SIZE / WRITE_SIZE (KiB per dispatch),
    each scaled by 1 GiB over its own reading for a 1 GiB device copy."""
    import hashlib
    import synth
    d = args.write_traffic
    gib = 1 << 30

    def mean_after(vals, skip):
        v = vals[skip:] if len(vals) > skip else vals
        return sum(v) / len(v)

    copy_name = lambda m: next(n for n in m if "copyBuffer" in n or "copy" in n.lower())
    cf, cw = read_counter(os.path.join(d, "cfetch"), "FETCH_SIZE"), read_counter(os.path.join(d, "cwrite"), "WRITE_SIZE")
    cf_kib, cw_kib = mean_after(cf[copy_name(cf)], 1), mean_after(cw[copy_name(cw)], 1)
    ff, wf = gib / (cf_kib * 1024), gib / (cw_kib * 1024)  # true bytes per counted byte
    kname = "indexer_decode_fp8_kernel" if args.index_fp8 else "indexer_decode_kernel"
    fe, wr = read_counter(os.path.join(d, "fetch"), "FETCH_SIZE"), read_counter(os.path.join(d, "write"), "WRITE_SIZE")
    kf = next(n for n in fe if kname in n)
    kw = next(n for n in wr if kname in n)
    f_kib, w_kib = mean_after(fe[kf], 2), mean_after(wr[kw], 2)
    cfg = synth.CONFIGS[args.workload]
    key_bytes = 128 if args.index_fp8 else 256
    rows = cfg.B * cfg.T
    alg = cfg.B * cfg.L * key_bytes + rows * 32 * (128 if args.index_fp8 else 256) + rows * 32 * 4
    src = "indexer.hip"
    fpre = " --index-fp8" if args.index_fp8 else ""
    rec = {
        "kernel": kname,
        "workload": cfg.name,
        "source": src,
        "source_sha256": hashlib.sha256(open(os.path.join(ROOT, "long_context_sparse_scores_amd", "csrc", src),
                                             "rb").read()).hexdigest(),
        "dispatches_counted": [len(fe[kf]) - 2, len(wr[kw]) - 2],
        "fetch_size_kib_per_launch_raw": round(f_kib, 2),
        "write_size_kib_per_launch_raw": round(w_kib, 2),
        "copy_calibration": {"bytes_copied": gib, "fetch_size_kib_raw": round(cf_kib, 2),
                             "write_size_kib_raw": round(cw_kib, 2), "fetch_factor": round(ff, 5),
                             "write_factor": round(wf, 5)},
        "fetch_bytes_per_launch": int(f_kib * 1024 * ff),
        "write_bytes_per_launch": int(w_kib * 1024 * wf),
        "algorithmic_bytes_per_launch": alg,
        "commands": [
            "rocprofv3 --pmc FETCH_SIZE -d %s/fetch -o run --output-format csv -- python3 bench.py --workload %s%s "
            "--no-cpu --indexer-only --steps 5 --warmup 1" % (d, cfg.name, fpre),
            "rocprofv3 --pmc WRITE_SIZE -d %s/write -o run --output-format csv -- python3 bench.py --workload %s%s "
            "--no-cpu --indexer-only --steps 5 --warmup 1" % (d, cfg.name, fpre),
            "rocprofv3 --pmc FETCH_SIZE -d %s/cfetch -o run --output-format csv -- python3 bench.py --copy-calibrate" % d,
            "rocprofv3 --pmc WRITE_SIZE -d %s/cwrite -o run --output-format csv -- python3 bench.py --copy-calibrate" % d,
            "python3 bench.py --write-traffic %s --workload %s%s" % (d, cfg.name, fpre),
        ],
        "note": "per-launch averages over the indexer dispatches after the first two; the counters read KiB per "
                "dispatch; each is scaled by 1 GiB / (its reading for a 1 GiB device copy). The written bytes are "
                "the fp32 score rows (B*T*L*4).",
    }
    rec["bytes_per_launch"] = rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
    out = os.path.join(ROOT, "profiles", "%s_%s_traffic.json" % ("indexer_fp8" if args.index_fp8 else "indexer",
                                                                 cfg.name))
    with open(out, "w") as fh:
        json.dump(rec, fh, indent=1)
    log("bench: wrote %s" % out)
    gf, gw = os.path.join(d, "gfetch"), os.path.join(d, "gwrite")
    if os.path.isdir(gf) and os.path.isdir(gw):
        fe, wr = read_counter(gf, "FETCH_SIZE"), read_counter(gw, "WRITE_SIZE")
        print("| kernel | dispatches | fetched MB per launch | written MB per launch |")
        print("|---|---|---|---|")
        for n in sorted(fe, key=lambda n: -mean_after(fe[n], 2)):
            if "copy" in n.lower() or "fill" in n.lower():
                continue
            w = wr.get(n, [0.0])
            print("| %s | %d | %.1f | %.1f |" % (short_kernel_name(n), len(fe[n]), mean_after(fe[n], 2) * 1024 * ff / 1e6,
                                              mean_after(w, 2) * 1024 * wf / 1e6))


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def omp_set_threads(n):
    """OpenMP threads for the oracle's next parallel regions started by this thread."""
    import ctypes
    ctypes.CDLL("libgomp.so.1").omp_set_num_threads(int(n))


def cpu_baseline(cfg, target_s, index_fp8=False, kv_fp8=False, queries=None, single_thread=False):
    """The CPU oracle (oracle/, plain C fp64 + OpenMP), untuned, on query
    tokens of the same workload, each through the whole pipeline: indexer over
    its visible keys, top-k, and the attention of every layer.  Runs tokens
    until about target_s seconds on all host threads.  queries: a seeded
    sample of that many query rows of each sequence (long prefill chunks),
    else the rows in order.  single_thread: also time one query token on one
    thread.  index_fp8 / kv_fp8: E4M3 caches, as the GPU run reads them."""
    import numpy as np

    import oracle

    threads = int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count())
    rows = np.arange(cfg.T)
    if queries is not None and queries < cfg.T:
        rows = np.sort(np.random.default_rng(cfg.seed).choice(cfg.T, size=queries, replace=False))
    qi_all = cfg.q_idx_fp8() if index_fp8 else cfg.q_idx()
    w_all, pos_all = cfg.w(), cfg.q_pos()
    q_all = [cfg.q_attn(l) for l in range(cfg.n_layers)]

    def run(b, sel):
        ki = (cfg.k_idx_rows_fp8(b) if index_fp8 else cfg.k_idx_rows(b))[None]
        kvs = [cfg.kv_seq_fp8(l, b) if kv_fp8 else cfg.kv_seq(l, b) for l in range(cfg.n_layers)]
        t0 = time.perf_counter()
        oracle.layer_group(qi_all[b:b + 1, sel], w_all[b:b + 1, sel], ki, pos_all[b:b + 1, sel], cfg.k,
                           [q[b:b + 1, sel] for q in q_all], kvs, cfg.sm_scale, idx_fp8=index_fp8, kv_fp8=kv_fp8)
        return time.perf_counter() - t0

    done, spent, b, j = 0, 0.0, 0, 0
    per_call = min(len(rows), 4)  # a few query rows per call, scaled by query tokens
    while spent < target_s and b < cfg.B:
        sel = rows[j:j + per_call]
        spent += run(b, sel)
        done += len(sel)
        j += len(sel)
        if j >= len(rows):
            b, j = b + 1, 0
        log("bench: cpu oracle %d query token(s), %.2f s" % (done, spent))
    res = {"value": round(done / spent, 3), "unit": "query-tokens/s", "cores": threads, "kind": "oracle",
           "cpu_model": cpu_model(),
           "sample": "%d query tokens of %s (%d sequences x %d tokens%s), the whole pipeline per token: indexer "
                     "over the visible keys, top-%d, %d attention layers; fp64 plain C with OpenMP on %d threads"
                     % (done, cfg.name, cfg.B, cfg.T,
                        "; a seeded sample of %d of each sequence's %d query rows, the rate extrapolates to all of "
                        "them" % (len(rows), cfg.T) if len(rows) < cfg.T else "", cfg.k, cfg.n_layers, threads)}
    if single_thread:
        omp_set_threads(1)
        try:
            t1 = run(0, rows[:1])
        finally:
            omp_set_threads(threads)
        log("bench: cpu oracle 1 query token on one thread, %.2f s" % t1)
        res["single_thread"] = {"value": round(1.0 / t1, 4), "unit": "query-tokens/s", "cores": 1,
                                "sample": "query token 0 of sequence 0 of %s, the whole pipeline" % cfg.name}
    return res


def bench_mtp(cfg, args):
    """One MTP draft round per step, B sequences: the step-1 indexer and top-k
    over the backbone index keys, attention of the 7 draft steps over the
    backbone latent rows with the step-1 list, then verification of the 7
    drafts (sum-min, accept loop, resample) over the full vocabulary."""
    import numpy as np
    import torch

    import long_context_sparse_scores_amd as dsa
    import synth

    if args.index_fp8 or args.kv_fp8:
        raise SystemExit("bench.py: --index-fp8 / --kv-fp8 apply to the group workloads, not to %s" % cfg.name)
    dev = torch.device("cuda:0")
    B, L, S, V, k = cfg.B, cfg.L, cfg.S, cfg.V, cfg.k
    log("bench: workload %s B=%d L=%d steps=%d V=%d" % (cfg.name, B, L, S, V))

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    t0 = time.time()
    q_idx, w, pos = bf(cfg.q_idx()), torch.from_numpy(cfg.w()).to(dev), torch.from_numpy(cfg.q_pos()).to(dev)
    k_idx, kv = bf(cfg.k_idx()), bf(cfg.kv())
    q_steps = [bf(np.ascontiguousarray(cfg.q_steps()[:, s:s + 1])) for s in range(S)]
    target = cfg.target_logits()
    draft = cfg.draft_logits(target)
    tok = cfg.draft_tokens(draft)
    t_d, d_d = torch.from_numpy(target).to(dev), torch.from_numpy(draft).to(dev)
    tok_d = torch.from_numpy(tok).to(dev)
    u_d, ur_d = torch.from_numpy(cfg.u_accept()).to(dev), torch.from_numpy(cfg.u_resample()).to(dev)
    torch.cuda.synchronize()
    log("bench: inputs generated and resident in HBM (%.1f s)" % (time.time() - t0))

    scores = torch.empty((B, 1, L), dtype=torch.float32, device=dev)
    idx = torch.empty((B, 1, k), dtype=torch.int32, device=dev)
    outs = [torch.empty((B, 1, cfg.Hq, cfg.Dv), dtype=torch.bfloat16, device=dev) for _ in range(S)]
    topk_ws = torch.empty(dsa.topk_workspace_size(B, 1, L, k), dtype=torch.uint8, device=dev)
    attn_ws = torch.empty(max(256, dsa.attn_workspace_size(B, 1, k)), dtype=torch.uint8, device=dev)
    ver_ws = torch.empty(dsa.verify_workspace_size(B, S, V), dtype=torch.uint8, device=dev)
    # the draft path is one dsa_layer_group call whose layers are the S draft
    # steps: indexer and top-k once over the backbone keys, then S attention
    # launches over the one backbone latent cache with the step-1 list
    gargs = dsa.make_group_args(q_idx, w, k_idx, pos, k, q_steps, [kv] * S, cfg.sm_scale, idx, outs)
    g_bytes = dsa.layer_group_workspace_size(gargs)
    g_ws = torch.zeros(g_bytes, dtype=torch.uint8, device=dev)
    lib = dsa.lib()
    stream = torch.cuda.current_stream(dev).cuda_stream
    import ctypes
    gptr = ctypes.byref(gargs)

    def indexer_step():
        dsa.indexer_scores(q_idx, w, k_idx, pos, scores=scores)

    def round_step():
        rc = lib.dsa_layer_group(gptr, g_ws.data_ptr(), g_bytes, stream)
        if rc != 0:
            raise RuntimeError(dsa.last_error())
        return dsa.mtp_draft_verify(t_d, d_d, tok_d, u_d, ur_d, ws=ver_ws)

    def timed(fn, steps):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    ms = timed(round_step, args.steps)
    idx_ms = timed(indexer_step, args.steps)
    # per-phase breakdown, each entry point timed on its own
    topk_ms = timed(lambda: dsa.topk(scores, pos, k, idx=idx, ws=topk_ws), args.steps)
    attn_ms = timed(lambda: dsa.sparse_mla_attn(q_steps[1], kv, idx, cfg.sm_scale, out=outs[1], ws=attn_ws), args.steps)
    ver_ms = timed(lambda: dsa.mtp_draft_verify(t_d, d_d, tok_d, u_d, ur_d, ws=ver_ws), args.steps)
    breakdown = {"indexer_ms": round(idx_ms, 4), "topk_ms": round(topk_ms, 4), "attn_ms_per_step": round(attn_ms, 4),
                 "verify_ms": round(ver_ms, 4)}
    log("bench: breakdown %s" % breakdown)
    _, n_acc, _ = round_step()
    accept_len = float(n_acc.float().mean().item()) + 1.0
    step1 = L * cfg.D * 2 + cfg.H * cfg.D * 2 + cfg.H * 4 + k * 4
    attn_step = k * cfg.Dqk * 2 + cfg.Hq * cfg.Dqk * 2 + cfg.Hq * cfg.Dv * 2 + k * 4
    verify = (2 * S + 1) * V * 4 + S * 4 * 3 + 4
    seq_bytes = step1 + S * attn_step + verify
    idx_bytes = B * (L * cfg.D * 2 + cfg.H * cfg.D * 2 + cfg.H * 4)
    achieved = idx_bytes / (idx_ms / 1e3) / 1e9
    log("bench: round %.3f ms, indexer %.3f ms" % (ms, idx_ms))
    line = {
        "metric": "MTP draft rounds (sequence-rounds/s) at 128K ctx, 7 steps; % of HBM roofline",
        "value": round(B / (ms / 1e3), 1),
        "unit": "sequence-rounds/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded counter-based generator; GLM-5.2 shapes)",
        "config": {"workload": cfg.name, "batch": B, "context": L, "draft_steps": S, "vocab": V, "topk": k},
        "draft_steps_per_s": round(B * S / (ms / 1e3), 1),
        "mean_acceptance_length": round(accept_len, 3),
        "hbm_roofline_frac": round(B * seq_bytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
        "algorithmic_bytes_per_step": B * seq_bytes,
        "roofline": {"kernel": "indexer_decode_kernel", "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_from_profiles("indexer", cfg.name), "bytes_per_launch": idx_bytes,
                     "avg_launch_ms": round(idx_ms, 4)},
        "breakdown": breakdown,
        "cpu_baseline": None,
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline_mtp(cfg, args.cpu_seconds)
    return line


def bench_mtp_rounds(cfg, args):
    """A step is R chained MTP rounds for B sequences, all on the device: the
    step-1 indexer and top-k over the cache up to each sequence's position, S
    draft attention steps with that list (one dsa_layer_group call whose
    layers are the draft steps), verification of the S drafts, and the commit
    that appends the kept rows and advances the positions (the host reads
    nothing between rounds).  Every step starts from the same positions; the
    commit rewrites the same rows, so steps are identical.  The value is
    verified tokens per second (sum over sequences and rounds of n_accepted+1)
    with rejection sampling; the target-only rule is timed as an A/B."""
    import numpy as np
    import torch

    import ctypes

    import long_context_sparse_scores_amd as dsa
    import synth

    if args.index_fp8 or args.kv_fp8:
        raise SystemExit("bench.py: --index-fp8 / --kv-fp8 apply to the group workloads, not to %s" % cfg.name)
    dev = torch.device("cuda:0")
    B, L, R, S, V, k = cfg.B, cfg.L, cfg.R, cfg.S, cfg.V, cfg.k
    log("bench: workload %s B=%d L0=%d capacity=%d rounds=%d steps=%d V=%d" % (cfg.name, B, cfg.L0, L, R, S, V))

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    t0 = time.time()
    k_cache = bf(cfg.k_idx())
    kv_cache = torch.empty((B, L, cfg.Dqk), dtype=torch.bfloat16, device=dev)
    for b in range(B):
        kv_cache[b].copy_(bf(cfg.kv_seq(b)))
    rounds = []
    for r in range(R):
        t = cfg.target_logits(r)
        d = cfg.draft_logits(r, t)
        qs = cfg.q_steps(r)
        rounds.append({"q_idx": bf(cfg.q_idx(r)), "w": torch.from_numpy(cfg.w(r)).to(dev),
                       "q_steps": [bf(np.ascontiguousarray(qs[:, s:s + 1])) for s in range(S)],
                       "target": torch.from_numpy(t).to(dev), "draft": torch.from_numpy(d).to(dev),
                       "tok": torch.from_numpy(cfg.draft_tokens(r, d)).to(dev),
                       "u": torch.from_numpy(cfg.u_accept(r)).to(dev), "ur": torch.from_numpy(cfg.u_resample(r)).to(dev),
                       "new_k": bf(cfg.new_k(r)), "new_kv": bf(cfg.new_kv(r))})
        del t, d, qs
    q_pos0 = torch.from_numpy(cfg.q_pos0()).to(dev)
    torch.cuda.synchronize()
    log("bench: inputs generated and resident in HBM (%.1f s)" % (time.time() - t0))

    # positions: round 0 reads q_pos0, round r > 0 reads qp[r % 2]; the commit of
    # round r writes qp[(r + 1) % 2], so no copy resets them between steps
    qp = [torch.empty(B, dtype=torch.int32, device=dev) for _ in range(2)]
    pos_in = [q_pos0] + [qp[r % 2] for r in range(1, R)]
    idx = torch.empty((B, 1, k), dtype=torch.int32, device=dev)
    outs = [torch.empty((B, 1, cfg.Hq, cfg.Dv), dtype=torch.bfloat16, device=dev) for _ in range(S)]
    # the draft path of a round is one dsa_layer_group call with the S draft steps as
    # its layers: indexer and top-k once, S attention launches over the one cache
    gargs = [dsa.make_group_args(rounds[r]["q_idx"], rounds[r]["w"], k_cache, pos_in[r].view(B, 1), k,
                                 rounds[r]["q_steps"], [kv_cache] * S, cfg.sm_scale, idx, outs) for r in range(R)]
    gptr = [ctypes.byref(a) for a in gargs]
    g_bytes = max(dsa.layer_group_workspace_size(a) for a in gargs)
    g_ws = torch.zeros(g_bytes, dtype=torch.uint8, device=dev)  # zero-filled before first use
    ver_ws = torch.empty(max(dsa.verify_workspace_size(B, S, V), dsa.lib().mtp_verify_target_only_workspace_size(B, S, V)),
                         dtype=torch.uint8, device=dev)
    n_acc = torch.empty((R, B), dtype=torch.int32, device=dev)
    nxt = torch.empty((R, B), dtype=torch.int32, device=dev)
    min_sum = torch.empty((B, S), dtype=torch.float32, device=dev)
    lib = dsa.lib()
    stream = torch.cuda.current_stream(dev).cuda_stream

    def run_step(rule):
        for r in range(R):
            rd = rounds[r]
            rc = lib.dsa_layer_group(gptr[r], g_ws.data_ptr(), g_bytes, stream)
            if rc != 0:
                raise RuntimeError(dsa.last_error())
            if rule == "rejection":
                rc = lib.mtp_draft_verify(rd["target"].data_ptr(), rd["draft"].data_ptr(), rd["tok"].data_ptr(),
                                          rd["u"].data_ptr(), rd["ur"].data_ptr(), B, S, V, min_sum.data_ptr(),
                                          n_acc[r].data_ptr(), nxt[r].data_ptr(), ver_ws.data_ptr(),
                                          ver_ws.numel(), stream)
            else:
                rc = lib.mtp_verify_target_only(rd["target"].data_ptr(), rd["tok"].data_ptr(), B, S, V,
                                                n_acc[r].data_ptr(), nxt[r].data_ptr(), ver_ws.data_ptr(),
                                                ver_ws.numel(), stream)
            if rc != 0:
                raise RuntimeError(dsa.last_error())
            dsa.mtp_commit(n_acc[r], pos_in[r], rd["new_k"], rd["new_kv"], k_cache, kv_cache,
                           q_pos_out=qp[(r + 1) % 2])

    def timed(rule, steps):
        for _ in range(args.warmup):
            run_step(rule)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            run_step(rule)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        tokens = int((n_acc.to(torch.int64) + 1).sum().item())
        return ms, tokens, (n_acc.float() + 1).mean(dim=1).cpu().numpy()

    res = {}
    for rule in ("rejection", "target_only"):
        ms, tokens, per_round = timed(rule, args.steps)
        res[rule] = {"ms_per_step": round(ms, 4), "verified_tokens_per_step": tokens,
                     "verified_tokens_per_s": round(tokens / (ms / 1e3), 1),
                     "mean_acceptance_length": round(tokens / (B * R), 3),
                     "acceptance_length_per_round": [round(float(x), 3) for x in per_round]}
        log("bench: %s: %.3f ms per %d rounds, %d verified tokens, mean acceptance length %.3f"
            % (rule, ms, R, tokens, tokens / (B * R)))
    # the index-key scan of one round, timed alone (the roofline figure)
    rd0 = rounds[0]
    scores = torch.empty((B, 1, L), dtype=torch.float32, device=dev)

    def indexer_step():
        dsa.indexer_scores(rd0["q_idx"], rd0["w"], k_cache, q_pos0.view(B, 1), scores=scores)

    for _ in range(args.warmup):
        indexer_step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        indexer_step()
    e1.record()
    torch.cuda.synchronize()
    idx_ms = e0.elapsed_time(e1) / args.steps
    idx_bytes = B * (L * cfg.D * 2 + cfg.H * cfg.D * 2 + cfg.H * 4)
    achieved = idx_bytes / (idx_ms / 1e3) / 1e9
    main = res["rejection"]
    line = {
        "metric": "verified tokens/s in chained MTP rounds (draft 7 -> verify -> commit) at 128K ctx",
        "value": main["verified_tokens_per_s"],
        "unit": "verified-tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": main["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded counter-based generator; GLM-5.2 shapes; favoured-token logits)",
        "config": {"workload": cfg.name, "batch": B, "context_start": cfg.L0, "capacity": L, "rounds": R,
                   "draft_steps": S, "vocab": V, "topk": k, "rho": cfg.rho, "boost": cfg.boost},
        "rejection_sampling": res["rejection"],
        "target_only": res["target_only"],
        "roofline": {"kernel": "indexer_decode_kernel", "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None, "bytes_per_launch": idx_bytes, "avg_launch_ms": round(idx_ms, 4)},
        "cpu_baseline": None,
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline_mtp_rounds(cfg, args.cpu_seconds)
    return line


def cpu_baseline_mtp_rounds(cfg, target_s):
    """The oracle's composed round (indexer, top-k, S attention steps,
    rejection-sampling verification, commit) on whole sequences, one at a
    time, over the rounds until about target_s seconds; verified tokens/s."""
    import numpy as np

    import oracle

    threads = int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count())
    spent, tokens, done = 0.0, 0, 0
    for b in range(cfg.B):
        k_cache = cfg.k_idx()[b:b + 1].copy() if b == 0 else None
        if k_cache is None:
            break  # one sequence is enough for the bounded sample
        kv_cache = cfg.kv_seq(b)[None].copy()
        q_pos = cfg.q_pos0()[b:b + 1].copy()
        for r in range(cfg.R):
            t = cfg.target_logits(r)
            d = cfg.draft_logits(r, t)
            tok = cfg.draft_tokens(r, d)
            qs = cfg.q_steps(r)
            t0 = time.perf_counter()
            out = oracle.mtp_round(cfg.q_idx(r)[b:b + 1], cfg.w(r)[b:b + 1], k_cache, q_pos.reshape(1, 1), cfg.k,
                                   [np.ascontiguousarray(qs[b:b + 1, s:s + 1]) for s in range(cfg.S)], kv_cache,
                                   cfg.sm_scale, t[b:b + 1], d[b:b + 1], tok[b:b + 1], cfg.u_accept(r)[b:b + 1],
                                   cfg.u_resample(r)[b:b + 1], cfg.new_k(r)[b:b + 1], cfg.new_kv(r)[b:b + 1])
            spent += time.perf_counter() - t0
            tokens += int(out["n_acc"][0]) + 1
            q_pos = out["q_pos_next"]
            done += 1
            log("bench: cpu oracle round %d of sequence %d, %.2f s" % (r, b, spent))
            if spent >= target_s:
                break
    return {"value": round(tokens / spent, 3), "unit": "verified-tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": "%d round(s) of sequence 0 of %s, each the whole round: indexer over the visible keys, top-%d, "
                      "%d draft attention steps, rejection-sampling verification over V=%d, commit; fp64 plain C "
                      "with OpenMP" % (done, cfg.name, cfg.k, cfg.S, cfg.V)}


def cpu_baseline_mtp(cfg, target_s):
    """The CPU oracle on whole sequences of the MTP round: indexer over all
    keys, top-k, the 7 attention steps, verification."""
    import oracle
    import synth

    threads = int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count())
    target = cfg.target_logits()
    draft = cfg.draft_logits(target)
    tok = cfg.draft_tokens(draft)
    u, ur = cfg.u_accept(), cfg.u_resample()
    qsteps = cfg.q_steps()
    done, spent = 0, 0.0
    while spent < target_s and done < cfg.B:
        b = done
        t0 = time.perf_counter()
        sc = oracle.indexer_scores(cfg.q_idx()[b:b + 1], cfg.w()[b:b + 1], cfg.k_idx_rows(b)[None],
                                   cfg.q_pos()[b:b + 1])
        idx = oracle.topk(sc, cfg.q_pos()[b:b + 1], cfg.k)
        kv = synth.normal_bf16(cfg.seed, synth.T_KV, (1, cfg.L, cfg.Dqk), start=b * cfg.L * cfg.Dqk)
        for s in range(cfg.S):
            oracle.sparse_mla_attn(qsteps[b:b + 1, s:s + 1], kv, idx, cfg.sm_scale)
        oracle.mtp_verify(target[b:b + 1], draft[b:b + 1], tok[b:b + 1], u[b:b + 1], ur[b:b + 1])
        spent += time.perf_counter() - t0
        done += 1
        log("bench: cpu oracle %d sequence-round(s), %.2f s" % (done, spent))
    return {"value": round(done / spent, 4), "unit": "sequence-rounds/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": "%d of %d sequences of %s, the whole round per sequence; fp64 plain C with OpenMP"
                      % (done, cfg.B, cfg.name)}


if __name__ == "__main__":
    main()
