#!/usr/bin/env python3
"""Throughput of the decode-step MoE layer on one MI355X.

One step = one layer pass (router, top-k, routed experts, shared expert,
combine + residual + RMSNorm) over one batch of seeded synthetic tokens, with
every input resident in HBM.  Steps are replayed from HIP graphs and rotate
over several copies of the layer's weights, so consecutive steps never find
their weights in the 256 MB Infinity Cache (a decode pass reads each layer's
weights once).

By default it measures the metric's four points, 1, 16, 64 and 128 tokens
(decode_t1, decode_t16, wide_t64_e8m0, verify_t128), decode_t1 being the
headline, and prints ONE JSON line: effective HBM TB/s = algorithmic bytes
per step / time per step (touched routed-expert weights and scales +
shared-expert weights and scales + activations; the router weight is
reported apart).  The top-level fields are the headline's; "points" holds
every workload's record: µs per layer (K steps back to back) and the
p10/p50/p90 of the per-step time over replays of a multi-step graph, the
fraction of the published 8 TB/s and of a
streaming-read ceiling measured in the same run, the dominant kernel's
roofline with its counter traffic, MFMA utilisation on the grouped path,
the check of every output element against the CPU oracle, the health of the
bounded waits, and the CPU oracle's rate on a bounded sample.  A point whose
check fails or whose bounded waits gave up makes the line invalid (exit 1).

    python bench.py [--workload decode_t1] [--steps K] [--warmup W]
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E
MERGE_SHARED_MAX_TOKENS = 64  # the library's kMergeSharedMaxTokens
CHAIN_MAX_TOKENS = 16  # the library's kChainMaxTokens (split path: one expert launch)
# template arguments (NS, U, GR) of the library's gate_up MFMA launches (kNsGu, kUGu, kGR)
MFMA_GATE_UP_TILE = "4, 1, 1"
MFMA_ROUTED_TILE = "4, 1"  # NS, U of the routed-only gate_up launch
DENSE_MAX_GROUPS = 4  # 16-token groups per dense gate_up workgroup (kDenseMaxGroups)
GR2_MIN_MEAN = 10  # the library's kGr2MinMean
SHARED_ACT_MIN_MEAN = 10  # the library's kSharedActMinMean (two groups per pass)
SHARED_ACT_MIN_MEAN1 = 4  # the library's kSharedActMinMean1 (one group per pass)
MFMA_GATE_UP_WIDE_NS = 8  # the library's kNsGuWide (two groups, shared tiles)
FUSED_BOUNDARY_MAX_TOKENS = 16  # the library's kFusedBoundaryMaxTokens
METRIC = "µs per MoE layer and effective HBM TB/s (fraction of peak) at 1/16/64/128 tok"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def expert_bytes(H, I, e8m0):
    """Weight + scale bytes of one expert (w13 [2I,H] and w2 [H,I], fp8)."""
    sb = 1 if e8m0 else 4
    return 3 * H * I + sb * ((2 * I // 128) * (H // 128) + (H // 128) * (I // 128))


def step_bytes(sh, D):
    e8 = sh.scale_fmt == "e8m0"
    routed = D * expert_bytes(sh.H, sh.I, e8)
    shared = expert_bytes(sh.H, sh.Is, e8) if sh.Is else 0
    act = sh.T * 8 * sh.H + 2 * sh.H  # x, residual in; out, residual_out; gamma
    return routed, shared, act


def cpu_baseline(inp, sh, metric_bytes, seconds):
    import oracle
    from oracle import c_oracle

    c_oracle.build(force=False)
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or (os.cpu_count() or 1)
    model = cpu_model()
    if sh.E == 0:
        # a dense layer: the NumPy oracle (the C oracle is the MoE layer's)
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.moe_layer(inp)
            reps += 1
            elapsed = time.perf_counter() - t0
            if elapsed >= seconds:
                break
        per_step = elapsed / reps
        return {"value": metric_bytes / per_step / 1e12, "unit": "TB/s",
                "us_per_layer": per_step * 1e6, "cores": threads, "cpu_model": model,
                "kind": "oracle",
                "sample": "NumPy float64 dense-layer oracle, %d repetition(s) of the %s layer, "
                          "%.1f s (BLAS threads: up to %d)" % (reps, sh_name(sh), elapsed,
                                                               threads)}
    # token rows per repetition: whole step for small T, else a prefix
    rows = list(range(sh.T))
    t0 = time.perf_counter()
    c_oracle.moe_layer(inp, rows=rows[:1], threads=threads)
    t_one = time.perf_counter() - t0
    n_rows = max(1, min(sh.T, int(seconds / max(t_one, 1e-6))))
    reps, elapsed = 0, 0.0
    t0 = time.perf_counter()
    while True:
        c_oracle.moe_layer(inp, rows=rows[:n_rows], threads=threads)
        reps += 1
        elapsed = time.perf_counter() - t0
        if elapsed >= seconds or n_rows < sh.T:
            break
    per_step = elapsed / reps * (sh.T / n_rows)
    return {
        "value": metric_bytes / per_step / 1e12,
        "unit": "TB/s",
        "us_per_layer": per_step * 1e6,
        "cores": threads,
        "cpu_model": model,
        "kind": "oracle",
        "sample": "C float64 oracle, %d of %d token rows x %d repetition(s) of the %s layer, "
                  "%.1f s; time per full step scaled by tokens" % (n_rows, sh.T, reps,
                                                                    sh_name(sh), elapsed),
    }


def sources_digest():
    """sha256 over the HIP sources and the C header: a traffic figure taken
    with hardware counters holds only for the kernels it was taken on."""
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "moe_decode_layer_sigmoid_amd", "csrc")
    files = sorted(os.path.join(csrc, f) for f in os.listdir(csrc)
                   if f.endswith((".hip", ".h")))
    files.append(os.path.join(ROOT, "include", "moe_decode.h"))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


TRAFFIC_TAG = "traffic-record:"


def recorded_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` on `workload` from a counter summary
    under profiles/, if one was taken on the current sources."""
    pdir = os.path.join(ROOT, "profiles")
    if not os.path.isdir(pdir):
        return None
    digest = sources_digest()
    for f in sorted(os.listdir(pdir)):
        if not f.endswith(".md"):
            continue
        with open(os.path.join(pdir, f)) as fh:
            for line in fh:
                line = line.strip().strip("`")
                if not line.startswith(TRAFFIC_TAG):
                    continue
                rec = json.loads(line[len(TRAFFIC_TAG):])
                if (rec.get("workload") == workload and rec.get("kernel") == kernel
                        and rec.get("sources_sha256") == digest):
                    return rec
    return None


def _counter_mean(run_dir, kernel):
    import csv
    import glob

    vals = []
    for f in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if kernel in r["Kernel_Name"]:
                    vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit("no dispatch of %r in %s" % (kernel, run_dir))
    return sum(vals) / len(vals), len(vals)


def counters_summary(args):
    """Prints the traffic record of one kernel from four rocprofv3 --pmc runs:
    FETCH_SIZE and WRITE_SIZE of the workload, and of the copy calibration."""
    fetch, nf = _counter_mean(args.pmc_fetch, args.kernel)
    write, nw = _counter_mean(args.pmc_write, args.kernel)
    copy_kernel = "copyBuffer"
    cf, _ = _counter_mean(args.copy_fetch, copy_kernel)
    cw, _ = _counter_mean(args.copy_write, copy_kernel)
    copy_bytes = args.copy_calibration << 20
    fs = copy_bytes / (cf * 1024.0)
    ws = copy_bytes / (cw * 1024.0)
    rec = {"workload": args.workload, "kernel": args.kernel,
           "fetch_kib": round(fetch, 1), "write_kib": round(write, 1),
           "dispatches": [nf, nw], "copy_fetch_kib": round(cf, 1), "copy_write_kib": round(cw, 1),
           "fetch_scale": round(fs, 4), "write_scale": round(ws, 4),
           "bytes": int(round(fetch * 1024 * fs + write * 1024 * ws)),
           "sources_sha256": sources_digest()}
    print(TRAFFIC_TAG + json.dumps(rec))


def sh_name(sh):
    from synth import WORKLOADS

    for k, v in WORKLOADS.items():
        if v == sh:
            return k
    return "custom"


def cpu_model():
    """The host CPU's model name (Linux /proc/cpuinfo), for the CPU baseline."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


MFMA_TAG = "mfma-record:"
PEAK_BF16_MFMA_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
XCDS = 8  # MI355X accelerator complex dies


def recorded_mfma(workload, kernel):
    """MFMA counter record of `kernel` on `workload` (profiles/), if one was
    taken on the current sources."""
    pdir = os.path.join(ROOT, "profiles")
    if not os.path.isdir(pdir):
        return None
    digest = sources_digest()
    for f in sorted(os.listdir(pdir)):
        if not f.endswith(".md"):
            continue
        with open(os.path.join(pdir, f)) as fh:
            for line in fh:
                line = line.strip().strip("`")
                if not line.startswith(MFMA_TAG):
                    continue
                rec = json.loads(line[len(MFMA_TAG):])
                if (rec.get("workload") == workload and rec.get("kernel") == kernel
                        and rec.get("sources_sha256") == digest):
                    return rec
    return None


def _counter_means(run_dir, kernel):
    """Per-dispatch means of every counter rocprofv3 recorded for `kernel`."""
    import csv
    import glob

    vals = {}
    for f in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if kernel in r["Kernel_Name"]:
                    vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit("no dispatch of %r in %s" % (kernel, run_dir))
    return {k: (sum(v) / len(v), len(v)) for k, v in vals.items()}


def mfma_summary(args):
    """Prints the MFMA record of one kernel from rocprofv3 --pmc output
    directories (--pmc-dirs, comma-separated: one pass per counter group)."""
    counters, n = {}, 0
    for d in args.pmc_dirs.split(","):
        for name, (mean, cnt) in _counter_means(d, args.kernel).items():
            counters[name] = round(mean, 1)
            n = max(n, cnt)
    rec = {"workload": args.workload, "kernel": args.kernel, "counters": counters,
           "dispatches": n, "cu_count": args.cu_count, "xcds": XCDS,
           "sources_sha256": sources_digest()}
    print(MFMA_TAG + json.dumps(rec))


def percentile(v, q):
    return float(np.percentile(np.asarray(v, dtype=np.float64), q))


def read_ceiling(torch, md, gib=4, reps=12):
    """Streaming-read ceiling: the library's probe kernel over a `gib` GiB
    buffer, event-timed, median of `reps` launches (GB/s)."""
    nbytes = gib << 30
    nbytes -= nbytes % md.PROBE_STEP
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream()
    md.read_probe(buf, nbytes, sink, s)
    torch.cuda.synchronize()
    t = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(s)
        md.read_probe(buf, nbytes, sink, s)
        b.record(s)
        torch.cuda.synchronize()
        t.append(a.elapsed_time(b) * 1e-3)
    del buf
    torch.cuda.empty_cache()
    sec = float(np.median(t))
    return {"gbps": round(nbytes / sec / 1e9, 1), "bytes": nbytes, "launches": reps,
            "kernel": "moe_decode_read_probe (non-temporal 16-byte loads, 8 lanes per "
                      "128-byte line, 8 loads in flight per lane)",
            "frac_of_peak": round(nbytes / sec / 1e9 / PEAK_HBM_GBPS, 4)}


def dominant_kernel(md, sh, path_taken, D, routed_b, shared_b, act_b):
    """(readable name, rocprofv3 id, algorithmic bytes, algorithmic flops) of
    the kernel whose launches the measurement hook brackets."""
    T, H, k = sh.T, sh.H, sh.k
    e8 = "true" if sh.scale_fmt == "e8m0" else "false"
    sb = 1 if sh.scale_fmt == "e8m0" else 4
    if sh.E == 0:
        # a dense layer: the gate/up projection of its MLP (the router
        # kernel's gate_up tiles on the GEMV path, the shared-row MFMA launch)
        kb = (2 * sh.Is * H + sb * (2 * sh.Is // 128) * (H // 128) + T * H * 2 + T * sh.Is * 4)
        fl = 2 * T * 2 * sh.Is * H
        if path_taken == md.PATH_GROUPED:
            groups = (T + 15) // 16
            if groups == 1:  # one token group: the waves split the contraction
                return ("dense_gate_up_waves_mfma_kernel<E8> (dense MLP)",
                        "dense_gate_up_waves_mfma_kernel<%s>" % e8, kb, fl)
            gr = DENSE_MAX_GROUPS if groups >= DENSE_MAX_GROUPS else 2
            nb = 1 if gr == DENSE_MAX_GROUPS else 2  # blocks per round of loads
            return ("dense_gate_up_mfma_kernel<E8, GR, NB> (dense MLP)",
                    "dense_gate_up_mfma_kernel<%s, %d, %d>" % (e8, gr, nb), kb, fl)
        return ("router_kernel<NJ2, E8> (dense MLP gate_up tiles)",
                "router_kernel<%d, %s>" % ((H + 511) // 512, e8), kb, fl)
    if path_taken == md.PATH_GEMV:
        # one launch runs the whole step: its bytes are the step's (and the
        # router weight's)
        njd = (max(sh.I, sh.Is) + 1023) // 1024
        return ("decode_step_kernel<NJG, NJD, E8> (router, shared + routed experts, boundary)",
                "decode_step_kernel<%d, %d, %s>" % ((H + 1023) // 1024, njd, e8),
                routed_b + shared_b + act_b + sh.E * H * 2,
                6 * T * H * (k * sh.I + sh.Is) + 2 * T * sh.E * H)
    # gate/up projection: touched experts' w13 + scales, the token rows in,
    # the SwiGLU rows out (f32, or hi + lo bf16 planes)
    kb = D * (2 * sh.I * H + sb * (2 * sh.I // 128) * (H // 128)) + T * H * 2 + T * k * sh.I * 4
    fl = 2 * T * k * 2 * sh.I * H
    if path_taken == md.PATH_GROUPED and T <= MERGE_SHARED_MAX_TOKENS and H % 256 == 0:
        # one launch: the gate_up and down tiles of the touched experts and of
        # the shared expert's token passes (the boundary follows apart)
        if T <= FUSED_BOUNDARY_MAX_TOKENS:
            # with few tokens the boundary is in the same launch
            return ("grouped_chain_kernel<E8> (routed + shared experts, gate_up and down, "
                    "boundary)", "grouped_chain_kernel<%s>" % e8, routed_b + shared_b + act_b,
                    6 * T * H * (k * sh.I + sh.Is))
        return ("grouped_chain_kernel<E8> (routed + shared experts, gate_up and down)",
                "grouped_chain_kernel<%s>" % e8, routed_b + shared_b + T * H * 2,
                6 * T * H * (k * sh.I + sh.Is))
    if path_taken == md.PATH_GROUPED:
        # above 64 tokens the routed launch has routed rows only (ROWS = 2)
        # and the shared expert runs beside it (two 16-token groups per pass
        # once the routes average 10 or more tokens per expert)
        gr = 2 if T * sh.k >= GR2_MIN_MEAN * sh.E else 1
        # activation tiles shared per workgroup from a mean that depends on gr
        sa_min = SHARED_ACT_MIN_MEAN if gr == 2 else SHARED_ACT_MIN_MEAN1
        sa = "true" if T * sh.k >= sa_min * sh.E else "false"
        tile = MFMA_ROUTED_TILE
        if gr == 2 and sa == "true" and sh.I % (4 * 8 * MFMA_GATE_UP_WIDE_NS) == 0:
            tile = "%d, 1" % MFMA_GATE_UP_WIDE_NS  # wider waves (kNsGuWide)
        return ("gate_up_mfma_kernel<NS, U, GR, E8, ROWS> (routed experts)",
                "gate_up_mfma_kernel<%s, %d, %s, 2, %s>" % (tile, gr, e8, sa), kb, fl)
    if T <= CHAIN_MAX_TOKENS:
        # one launch streams the touched experts' gate_up and down weights and
        # the shared expert's down weights, and ends with the boundary (the
        # shared gate_up rides in the router launch)
        njd = (max(sh.I, sh.Is) + 1023) // 1024
        kb = routed_b + act_b
        if sh.Is:
            kb += H * sh.Is + sb * (H // 128) * (sh.Is // 128)
        return ("expert_chain_kernel<NJG, NJD, E8> (routed experts, shared down, boundary)",
                "expert_chain_kernel<%d, %d, %s>" % ((H + 1023) // 1024, njd, e8), kb,
                6 * T * k * H * sh.I + 2 * T * H * sh.Is)
    return ("gate_up_kernel<NJ, E8> (routed experts)",
            "gate_up_kernel<%d, %s>" % ((H + 1023) // 1024, e8), kb, fl)


def check_outputs(inp, sh, got):
    """The checked run against the oracles: expert ids on every token (the
    oracle router, near-ties excepted), and every element of out,
    residual_out and moe_out against the oracle run on the GPU's ids."""
    import oracle
    from oracle import c_oracle

    c_oracle.build(force=False)
    ids_ok, n_tie = True, 0
    if sh.E > 0:
        x = oracle.bf16_bits_to_f64(inp.hidden)
        sc = oracle.sigmoid(oracle.router_logits(x, oracle.bf16_bits_to_f64(inp.router_w)))
        oids = oracle.select_experts(sc, None, sh.k)
        gaps = oracle.score_gaps(sc, None, sh.k)
        for a, b, g in zip(got["ids"].tolist(), oids.tolist(), gaps):
            if g > 1e-4:
                ids_ok &= set(a) == set(b)
            else:
                n_tie += 1
        ref = c_oracle.moe_layer(inp, forced_ids=got["ids"])
    else:
        ref = oracle.moe_layer(inp)
    res = {"ids_match": bool(ids_ok), "near_ties": n_tie, "rows": sh.T}
    ok = ids_ok
    for name, key in (("out", "out"), ("residual_out", "h"), ("moe_out", "moe")):
        d = got[name] - ref[key]
        rel = float(np.linalg.norm(d) / max(np.linalg.norm(ref[key]), 1e-300))
        mx = float(np.abs(d).max() / max(np.sqrt(np.mean(ref[key] ** 2)), 1e-300))
        res[name] = {"rel_l2": round(rel, 6), "max_abs_over_rms": round(mx, 5)}
        ok &= rel <= 5e-3 and mx <= 3e-2
    res["pass"] = bool(ok)
    return res


def measure_point(name, args, ceiling):
    """Everything the line reports for one workload: the checked run, K timed
    steps (bracketed, then event per step), the dominant kernel's launches,
    the counter records, the CPU oracle's rate."""
    import torch

    import moe_decode_layer_sigmoid_amd as md
    import oracle
    from synth import WORKLOADS, make_layer

    sh = WORKLOADS[name]
    if args.tokens:
        sh = sh.replace(T=args.tokens)
    wname = name if not args.tokens else "%s@T%d" % (name, sh.T)
    T, H, E, k = sh.T, sh.H, sh.E, sh.k
    log("workload", wname, sh)
    t0 = time.perf_counter()
    inp = make_layer(sh, seed=0)
    log("inputs generated in %.1f s" % (time.perf_counter() - t0))

    def dev(a):
        if a is None:
            return None
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to("cuda")

    weights0 = {n: dev(getattr(inp, n)) for n in (
        "router_w", "router_bias", "w13", "w13_scale", "w2", "w2_scale", "sw13", "sw13_scale",
        "sw2", "sw2_scale", "gamma")}
    hidden = dev(inp.hidden)
    residual = dev(inp.residual)
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    res_out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    moe_out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    ids = torch.empty((T, max(k, 1)), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, max(k, 1)), dtype=torch.float32, device="cuda")

    path = {"auto": md.PATH_AUTO, "step": md.PATH_GEMV, "grouped": md.PATH_GROUPED,
            "split": md.PATH_GEMV_SPLIT}[args.path]
    plan = md.Plan(md.make_desc(H, E, k, sh.I, sh.Is, T, sh.scale_fmt, path, sh.limit, sh.rsf,
                                sh.eps), torch.cuda.current_device())

    def make_args(w):
        return plan.make_args(hidden=hidden, residual=residual, out=out, residual_out=res_out,
                              topk_ids=ids, topk_weights=wts, moe_out=moe_out, **w)

    # ---- one checked run: every token's ids, every output element
    plan.run_args(make_args(weights0), T)
    torch.cuda.synchronize()
    got_ids = ids.cpu().numpy()[:, :k]
    D = len(np.unique(got_ids)) if E else 0
    got = {"ids": got_ids,
           "out": oracle.bf16_bits_to_f64(out.cpu().numpy().view(np.uint16)),
           "residual_out": oracle.bf16_bits_to_f64(res_out.cpu().numpy().view(np.uint16)),
           "moe_out": oracle.bf16_bits_to_f64(moe_out.cpu().numpy().view(np.uint16))}
    waits_clean = not plan.check_waits()
    t0 = time.perf_counter()
    check = check_outputs(inp, sh, got)
    log("check (%.1f s): %s" % (time.perf_counter() - t0, json.dumps(check)))
    routed_b, shared_b, act_b = step_bytes(sh, D)
    metric_bytes = routed_b + shared_b + act_b

    # ---- weight copies so that no step finds its weights cached
    per_copy = sum(t.numel() * t.element_size() for t in weights0.values() if t is not None)
    copies = args.copies or max(2, min(16, math.ceil(1.5 * 2 ** 30 / metric_bytes)))
    free = torch.cuda.mem_get_info()[0]
    copies = max(1, min(copies, int(0.8 * free // per_copy)))
    weight_sets = [weights0] + [
        {n: (None if t is None else t.clone()) for n, t in weights0.items()}
        for _ in range(copies - 1)]
    arg_sets = [make_args(w) for w in weight_sets]
    log("weight copies %d (%.2f GB each), metric bytes/step %.2f MB, distinct experts %d" %
        (copies, per_copy / 1e9, metric_bytes / 1e6, D))

    # ---- graphs: one of `copies` consecutive steps (each on its own weight
    # copy), plus one of the remainder of K.  Inside a graph the steps'
    # kernels run back to back, as a decode step's layers do in one captured
    # step.
    K, W = args.steps, args.warmup
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())

    def capture(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            for i in range(n):
                plan.run_args(arg_sets[i % copies], T)
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=s):
                for i in range(n):
                    plan.run_args(arg_sets[i % copies], T)
        torch.cuda.synchronize()
        return g

    g_full = capture(copies)
    g_rem = capture(K % copies) if K % copies else None
    with torch.cuda.stream(s):
        for _ in range(max(1, -(-W // copies))):
            g_full.replay()
    torch.cuda.synchronize()
    log("warmup done (%d steps)" % (max(1, -(-W // copies)) * copies))
    # the replays queue behind a GPU-side spin, so host submission never sits
    # inside the timed region
    spin = int(2.4e6 * max(20.0, 0.05 * K))

    # (A) exactly K steps back to back between two events: the headline time
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    with torch.cuda.stream(s):
        torch.cuda._sleep(spin)
        ev0.record(s)
        for _ in range(K // copies):
            g_full.replay()
        if g_rem is not None:
            g_rem.replay()
        ev1.record(s)
        queued_a = not s.query()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_per_step = ev0.elapsed_time(ev1) / K
    tbps = metric_bytes / (ms_per_step * 1e-3) / 1e12
    log("timed %d steps: %.2f us/step, %.3f TB/s (wall %.1f ms incl. the spin)" %
        (K, ms_per_step * 1e3, tbps, t_wall * 1e3))

    # (B) the distribution: each replay of the `copies`-step graph between
    # its own two events (per-step time = replay time / copies)
    n_rep = max(1, K // copies)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_rep + 1)]
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        torch.cuda._sleep(spin)
        for i in range(n_rep):
            evs[i].record(s)
            g_full.replay()
        evs[n_rep].record(s)
        queued_b = not s.query()
    torch.cuda.synchronize()
    per_step = [evs[i].elapsed_time(evs[i + 1]) * 1e3 / copies for i in range(n_rep)]
    pct = {"p10": round(percentile(per_step, 10), 3), "p50": round(percentile(per_step, 50), 3),
           "p90": round(percentile(per_step, 90), 3), "samples": n_rep, "steps_per_sample": copies}
    log("per-step us over %d replays of %d steps: p10 %.2f p50 %.2f p90 %.2f" %
        (n_rep, copies, pct["p10"], pct["p50"], pct["p90"]))
    del g_full, g_rem

    # ---- dominant kernel: events stamped at its own start and end, eager
    # launches queued behind a spin on s
    n_ev = min(K, 200)
    kevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(n_ev)]
    with torch.cuda.stream(s):
        for b, e in kevs:
            b.record(s)
            e.record(s)
        torch.cuda.synchronize()
        torch.cuda._sleep(spin)
        for i, (b, e) in enumerate(kevs):
            plan.set_expert_events(b, e)
            plan.run_args(arg_sets[i % copies], T)
        plan.set_expert_events(None, None)
        queued_k = not s.query()
    torch.cuda.synchronize()
    kern_ms = float(np.mean([b.elapsed_time(e) for b, e in kevs]))
    if not (queued_a and queued_b and queued_k):
        log("note: the GPU caught up with the host while steps were being queued")
    waits_clean &= not plan.check_waits()
    path_taken = plan.path_for(T)
    kern_name, kern_id, kern_bytes, kern_flops = dominant_kernel(
        md, sh, path_taken, D, routed_b, shared_b, act_b)
    achieved = kern_bytes / (kern_ms * 1e-3) / 1e9
    log("%s: %.2f us avg over %d launches, %.1f GB/s" % (kern_name, kern_ms * 1e3, n_ev,
                                                         achieved))
    trec = recorded_traffic(wname, kern_id)
    traffic = trec["bytes"] if trec else None
    log("traffic record: %s" % ("bytes %d (%.3f x algorithmic)" % (traffic, traffic / kern_bytes)
                                if trec else "none for the current sources"))
    mfma = None
    if path_taken == md.PATH_GROUPED:
        mrec = recorded_mfma(wname, kern_id)
        useful = kern_flops / (kern_ms * 1e-3) / 1e12
        mfma = {"kernel": kern_id, "useful_tflops": round(useful, 2),
                "useful_frac_of_bf16_peak": round(useful / PEAK_BF16_MFMA_TFLOPS, 5)}
        if mrec:
            c = mrec["counters"]
            mops = c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16")
            if mops is not None:
                issued = mops * 512 / (kern_ms * 1e-3) / 1e12
                mfma["issued_tflops"] = round(issued, 2)
                mfma["issued_frac_of_bf16_peak"] = round(issued / PEAK_BF16_MFMA_TFLOPS, 5)
            busy, gui, cus = (c.get("SQ_VALU_MFMA_BUSY_CYCLES"), c.get("GRBM_GUI_ACTIVE"),
                              mrec.get("cu_count"))
            if busy is not None and gui and cus:
                # GRBM_GUI_ACTIVE reads the busy cycles of each XCD's GRBM,
                # summed over the XCDs; MFMA busy cycles are per SIMD (4 per CU)
                cycles = gui / mrec.get("xcds", XCDS)
                mfma["mfma_busy_frac"] = round(busy / (cycles * cus * 4), 5)
            mfma["counters"] = c
        else:
            mfma["counters"] = None
        log("mfma: %s" % json.dumps(mfma))

    point = {
        "workload": wname, "tokens": T, "hidden": H, "experts": E, "top_k": k,
        "intermediate": sh.I, "shared_intermediate": sh.Is, "scale_fmt": sh.scale_fmt,
        "expert_path": {1: "gemv-step", 2: "grouped", 3: "gemv-split"}.get(path_taken, "?"),
        "distinct_experts": D, "metric_bytes_per_step": metric_bytes, "router_bytes": E * H * 2,
        "weight_copies": copies,
        "us_per_layer": round(ms_per_step * 1e3, 3),
        "p10_us": pct["p10"], "p50_us": pct["p50"], "p90_us": pct["p90"],
        "percentile_samples": "%d replays of a %d-step graph" % (pct["samples"],
                                                                 pct["steps_per_sample"]),
        "tbps": round(tbps, 4),
        "frac_of_peak": round(tbps * 1e3 / PEAK_HBM_GBPS, 4),
        "frac_of_read_ceiling": (round(tbps * 1e3 / ceiling["gbps"], 4) if ceiling else None),
        "roofline": {
            "bound": "hbm", "kernel": kern_name, "kernel_id": kern_id,
            "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic,
            "bytes_per_launch": kern_bytes, "avg_launch_us": round(kern_ms * 1e3, 3),
        },
        "mfma": mfma,
        "waits_clean": bool(waits_clean),
        "check": check,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline ...")
        point["cpu_baseline"] = cpu_baseline(inp, sh, metric_bytes, args.cpu_seconds)
    plan.close()
    del arg_sets, weight_sets, weights0
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return point


HEADLINE = "decode_t1"
POINTS = ["decode_t1", "decode_t16", "wide_t64_e8m0", "verify_t128"]
# measured beside the metric's points, not part of it: the dense layer
EXTRA_POINTS = ["dense_t16"]


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="",
                    help="measure this workload only (default: the metric's four points, "
                         "decode_t1 as the headline)")
    ap.add_argument("--tokens", type=int, default=0,
                    help="override the workload's token count (a sweep point, not a headline)")
    ap.add_argument("--copies", type=int, default=0, help="weight copies to rotate (0: auto)")
    ap.add_argument("--cpu-seconds", type=float, default=8.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true", help="skip the read-ceiling probe")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the points measured beside the metric (the dense layer)")
    ap.add_argument("--path", default="auto", choices=["auto", "step", "grouped", "split"])
    ap.add_argument("--json-out", default=None)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 10 plain device copies of MIB MiB (a known-size reference "
                         "for hardware byte counters) and exit")
    ap.add_argument("--counters-summary", action="store_true",
                    help="print the traffic record of --kernel from rocprofv3 --pmc output "
                         "directories (--pmc-fetch, --pmc-write, --copy-fetch, --copy-write; "
                         "--copy-calibration gives the copy size) and exit; needs no GPU")
    ap.add_argument("--mfma-summary", action="store_true",
                    help="print the MFMA counter record of --kernel from the rocprofv3 --pmc "
                         "output directories in --pmc-dirs and exit; needs no GPU")
    ap.add_argument("--kernel", default="")
    ap.add_argument("--pmc-fetch", default="")
    ap.add_argument("--pmc-write", default="")
    ap.add_argument("--copy-fetch", default="")
    ap.add_argument("--copy-write", default="")
    ap.add_argument("--pmc-dirs", default="")
    ap.add_argument("--cu-count", type=int, default=256)
    args = ap.parse_args()

    if args.counters_summary:
        counters_summary(args)
        return
    if args.mfma_summary:
        mfma_summary(args)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this layer build runs on a single MI355X "
              "(no multi-GPU path); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n, "launches": 10}))
        return

    import moe_decode_layer_sigmoid_amd as md

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    md.lib()  # fails loudly when the HIP library is missing
    names = [args.workload] if args.workload else POINTS
    extra = [] if args.workload or args.no_extra else EXTRA_POINTS
    ceiling = None
    if not args.no_probe:
        ceiling = read_ceiling(torch, md)
        log("read ceiling: %.1f GB/s (%.1f%% of %.0f)" % (ceiling["gbps"],
                                                         100 * ceiling["frac_of_peak"],
                                                         PEAK_HBM_GBPS))
    points = [measure_point(n, args, ceiling) for n in names]
    extra_points = []
    for n in extra:
        # no CPU baseline for these (it is reported for the headline point)
        saved = args.no_cpu_baseline
        args.no_cpu_baseline = True
        extra_points.append(measure_point(n, args, ceiling))
        args.no_cpu_baseline = saved
    head = points[0]
    cpu = head.get("cpu_baseline")
    valid = all(p["waits_clean"] and p["check"]["pass"] for p in points + extra_points)
    rec = {
        "metric": METRIC,
        "value": head["tbps"],
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["us_per_layer"] * 1e-3, 6),
        "us_per_layer": head["us_per_layer"],
        "frac_of_peak": head["frac_of_peak"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3 weights x bf16 activations, f32 accumulate",
        "data": "synthetic (seeded N(0,1) activations, N(0,1/sqrt(K)) fp8 block-quantised "
                "weights)",
        "config": {k: head[k] for k in (
            "workload", "tokens", "hidden", "experts", "top_k", "intermediate",
            "shared_intermediate", "scale_fmt", "distinct_experts", "metric_bytes_per_step",
            "router_bytes", "weight_copies", "expert_path")},
        "roofline": head["roofline"],
        "percentiles_us": {"p10": head["p10_us"], "p50": head["p50_us"], "p90": head["p90_us"]},
        "read_ceiling": ceiling,
        "frac_of_read_ceiling": head["frac_of_read_ceiling"],
        "waits_clean": all(p["waits_clean"] for p in points + extra_points),
        "check": head["check"],
        "valid": valid,
        "points": points,
        "extra_points": extra_points,
    }
    rec["config"]["parallelism"] = "none (1 GPU)"
    if cpu is not None:
        rec["cpu_baseline"] = cpu
    line = json.dumps(rec)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")
    if not valid:
        log("INVALID: a bounded wait gave up or a checked output is outside the tolerance")
        sys.exit(1)


if __name__ == "__main__":
    main()
