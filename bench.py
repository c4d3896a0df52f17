#!/usr/bin/env python3
"""Throughput of the decode-step MoE layer on one MI355X.

One step = one layer pass (router, top-k, routed experts, shared expert,
combine + residual + RMSNorm) over one batch of seeded synthetic tokens, with
every input resident in HBM.  Steps are replayed from HIP graphs and rotate
over several copies of the layer's weights, so consecutive steps never find
their weights in the 256 MB Infinity Cache (a decode pass reads each layer's
weights once).

Prints ONE JSON line: effective HBM TB/s = algorithmic bytes per step /
time per step (touched routed-expert weights and scales + shared-expert
weights and scales + activations; the router weight is reported apart),
plus the roofline of the routed-expert kernels and the CPU oracle's rate on
a bounded sample of the same workload.

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
GR2_MIN_MEAN = 10  # the library's kGr2MinMean
MFMA_DENSE_TILE = "2, 1, 1"  # NS, U, GR of a dense layer's gate_up launch (kNsGuDense)
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
                "us_per_layer": per_step * 1e6, "cores": threads, "kind": "oracle",
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


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="decode_t1")
    ap.add_argument("--tokens", type=int, default=0,
                    help="override the workload's token count (a sweep point, not a headline)")
    ap.add_argument("--copies", type=int, default=0, help="weight copies to rotate (0: auto)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--path", default="auto", choices=["auto", "fused", "grouped", "split"])
    ap.add_argument("--json-out", default=None)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 10 plain device copies of MIB MiB (a known-size reference "
                         "for hardware byte counters) and exit")
    ap.add_argument("--counters-summary", action="store_true",
                    help="print the traffic record of --kernel from rocprofv3 --pmc output "
                         "directories (--pmc-fetch, --pmc-write, --copy-fetch, --copy-write; "
                         "--copy-calibration gives the copy size) and exit; needs no GPU")
    ap.add_argument("--kernel", default="")
    ap.add_argument("--pmc-fetch", default="")
    ap.add_argument("--pmc-write", default="")
    ap.add_argument("--copy-fetch", default="")
    ap.add_argument("--copy-write", default="")
    args = ap.parse_args()

    if args.counters_summary:
        counters_summary(args)
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
    import oracle
    from synth import WORKLOADS, make_layer

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    md.lib()  # fails loudly when the HIP library is missing
    sh = WORKLOADS[args.workload]
    if args.tokens:
        sh = sh.replace(T=args.tokens)
    T, H, E, k = sh.T, sh.H, sh.E, sh.k
    log("workload", args.workload, sh)

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
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, k), dtype=torch.float32, device="cuda")

    path = {"auto": md.PATH_AUTO, "fused": md.PATH_GEMV, "grouped": md.PATH_GROUPED,
            "split": md.PATH_GEMV_SPLIT}[args.path]
    plan = md.Plan(md.make_desc(H, E, k, sh.I, sh.Is, T, sh.scale_fmt, path, sh.limit, sh.rsf,
                                sh.eps), torch.cuda.current_device())

    def make_args(w):
        return plan.make_args(hidden=hidden, residual=residual, out=out, residual_out=res_out,
                              topk_ids=ids, topk_weights=wts, **w)

    # ---- one checked run: ids against the oracle router, one row against the oracle
    plan.run_args(make_args(weights0), T)
    torch.cuda.synchronize()
    got_ids = ids.cpu().numpy()
    D = len(np.unique(got_ids))
    routed_b, shared_b, act_b = step_bytes(sh, D)
    metric_bytes = routed_b + shared_b + act_b
    from oracle import c_oracle

    c_oracle.build(force=False)
    ref = (oracle.moe_layer(inp, rows=[0]) if E == 0 else
           c_oracle.moe_layer(inp, forced_ids=got_ids, rows=[0]))
    got0 = oracle.bf16_bits_to_f64(out[:1].cpu().numpy().view(np.uint16))
    rel0 = float(np.linalg.norm(got0 - ref["out"]) / np.linalg.norm(ref["out"]))
    ids_ok = True
    if E > 0:
        x = oracle.bf16_bits_to_f64(inp.hidden)
        sc = oracle.sigmoid(oracle.router_logits(x, oracle.bf16_bits_to_f64(inp.router_w)))
        oids = oracle.select_experts(sc, None, k)
        gaps = oracle.score_gaps(sc, None, k)
        ids_ok = all(set(a) == set(b) for a, b, g in zip(got_ids.tolist(), oids.tolist(), gaps)
                     if g > 1e-4)
    log("check: distinct experts %d, ids match %s, row-0 rel L2 %.2e" % (D, ids_ok, rel0))

    # ---- weight copies so that no step finds its weights cached
    per_copy = sum(t.numel() * t.element_size() for t in weights0.values() if t is not None)
    copies = args.copies or max(2, min(16, math.ceil(1.5 * 2 ** 30 / metric_bytes)))
    free = torch.cuda.mem_get_info()[0]
    copies = max(1, min(copies, int(0.8 * free // per_copy)))
    weight_sets = [weights0] + [
        {n: (None if t is None else t.clone()) for n, t in weights0.items()}
        for _ in range(copies - 1)]
    arg_sets = [make_args(w) for w in weight_sets]
    log("weight copies %d (%.2f GB each), metric bytes/step %.2f MB" %
        (copies, per_copy / 1e9, metric_bytes / 1e6))

    # ---- graphs: one of `copies` steps, plus one for the remainder of K
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

    def replay(nsteps):
        with torch.cuda.stream(s):
            for _ in range(nsteps // copies):
                g_full.replay()
            if nsteps % copies:
                g_rem.replay()

    with torch.cuda.stream(s):
        for _ in range(max(1, -(-W // copies))):
            g_full.replay()
        if g_rem is not None:
            g_rem.replay()
    torch.cuda.synchronize()
    log("warmup done")

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    ev0.record(s)
    replay(K)
    ev1.record(s)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_total = ev0.elapsed_time(ev1)
    ms_per_step = ms_total / K
    tbps = metric_bytes / (ms_per_step * 1e-3) / 1e12
    log("timed %d steps: %.3f ms total (wall %.3f ms), %.2f us/step, %.3f TB/s" %
        (K, ms_total, t_wall * 1e3, ms_per_step * 1e3, tbps))

    # ---- dominant kernel: HIP events around it, eager launches on s
    n_ev = min(K, 200)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n_ev)]
    with torch.cuda.stream(s):
        for b, e in evs:
            b.record(s)
            e.record(s)
        torch.cuda.synchronize()
        # The launches queue up behind a GPU-side spin, so that they run back
        # to back and host submission time never falls inside a bracket.
        torch.cuda._sleep(int(2.5e8))
        for i, (b, e) in enumerate(evs):
            plan.set_expert_events(b, e)
            plan.run_args(arg_sets[i % copies], T)
        plan.set_expert_events(None, None)
        queued_ahead = not s.query()
    torch.cuda.synchronize()
    kern_ms = float(np.mean([b.elapsed_time(e) for b, e in evs]))
    if not queued_ahead:
        log("note: the GPU caught up with the host during the bracketed launches")
    path_taken = plan.path_for(T)
    e8 = "true" if sh.scale_fmt == "e8m0" else "false"
    sb = 1 if sh.scale_fmt == "e8m0" else 4
    if E == 0:
        # a dense layer: the gate/up projection of its MLP (the router
        # kernel's gate_up tiles on the GEMV path, the shared-row MFMA launch)
        kern_bytes = (2 * sh.Is * H + sb * (2 * sh.Is // 128) * (H // 128) + T * H * 2
                      + T * sh.Is * 4)
        if path_taken == md.PATH_GROUPED:
            kern_name = "gate_up_mfma_kernel<NS, U, GR, E8, ROWS> (dense MLP)"
            kern_id = "gate_up_mfma_kernel<%s, %s, 1>" % (MFMA_DENSE_TILE, e8)
        else:
            kern_name = "router_kernel<NJ2, E8> (dense MLP gate_up tiles)"
            kern_id = "router_kernel<%d, %s>" % ((H + 511) // 512, e8)
    elif path_taken == md.PATH_GEMV:
        # one persistent kernel runs the whole step: its bytes are the step's
        kern_name = "decode_fused_kernel (router, shared + routed experts, boundary)"
        kern_id = "decode_fused_kernel<"
        kern_bytes = metric_bytes + E * H * 2
    else:
        # gate/up projection: touched experts' w13 + scales, the token rows
        # in, the SwiGLU rows out (f32, or hi + lo bf16 planes)
        sb = 1 if sh.scale_fmt == "e8m0" else 4
        kern_bytes = (D * (2 * sh.I * H + sb * (2 * sh.I // 128) * (H // 128))
                      + T * H * 2 + T * k * sh.I * 4)
        if path_taken == md.PATH_GROUPED and T <= MERGE_SHARED_MAX_TOKENS and H % 256 == 0:
            # one launch: the gate_up and down tiles of the touched experts and
            # of the shared expert's token passes (the boundary follows apart)
            kern_name = "grouped_chain_kernel<E8> (routed + shared experts, gate_up and down)"
            kern_id = "grouped_chain_kernel<%s>" % e8
            kern_bytes = routed_b + shared_b + T * H * 2
        elif path_taken == md.PATH_GROUPED:
            # above 64 tokens the routed launch has routed rows only (ROWS =
            # 2) and the shared expert runs beside it
            # (two 16-token groups per pass once the routes average 10 or
            # more tokens per expert)
            kern_name = "gate_up_mfma_kernel<NS, U, GR, E8, ROWS> (routed experts)"
            gr = 2 if T * sh.k >= GR2_MIN_MEAN * sh.E else 1
            kern_id = "gate_up_mfma_kernel<%s, %d, %s, 2>" % (MFMA_ROUTED_TILE, gr, e8)
        elif T <= CHAIN_MAX_TOKENS:
            # one launch streams the touched experts' gate_up and down weights
            # and the shared expert's down weights, and ends with the boundary
            # (the shared gate_up rides in the router launch)
            kern_name = "expert_chain_kernel<NJG, NJD, E8> (routed experts, shared down, boundary)"
            njd = (max(sh.I, sh.Is) + 1023) // 1024
            kern_id = "expert_chain_kernel<%d, %d, %s>" % ((H + 1023) // 1024, njd, e8)
            kern_bytes = routed_b + act_b
            if sh.Is:
                kern_bytes += H * sh.Is + sb * (H // 128) * (sh.Is // 128)
        else:
            kern_name = "gate_up_kernel<NJ, E8> (routed experts)"
            kern_id = "gate_up_kernel<%d, %s>" % ((H + 1023) // 1024, e8)
    achieved = kern_bytes / (kern_ms * 1e-3) / 1e9
    log("%s: %.2f us avg over %d launches, %.1f GB/s" % (kern_name, kern_ms * 1e3, n_ev,
                                                         achieved))

    trec = recorded_traffic(args.workload if not args.tokens else "%s@T%d" % (args.workload, T),
                            kern_id)
    traffic = trec["bytes"] if trec else None
    log("traffic record: %s" % ("bytes %d (%.3f x algorithmic)" % (traffic, traffic / kern_bytes)
                                if trec else "none for the current sources"))

    rec = {
        "metric": METRIC,
        "value": round(tbps, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 6),
        "us_per_layer": round(ms_per_step * 1e3, 3),
        "frac_of_peak": round(tbps * 1e3 / PEAK_HBM_GBPS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3 weights x bf16 activations, f32 accumulate",
        "data": "synthetic (seeded N(0,1) activations, N(0,1/sqrt(K)) fp8 block-quantised weights)",
        "config": {
            "workload": args.workload + ("" if not args.tokens else "@T%d" % T), "tokens": T, "hidden": H, "experts": E, "top_k": k,
            "intermediate": sh.I, "shared_intermediate": sh.Is, "scale_fmt": sh.scale_fmt,
            "distinct_experts": D, "metric_bytes_per_step": metric_bytes,
            "router_bytes": E * H * 2, "weight_copies": copies,
            "expert_path": {1: "gemv-fused", 2: "grouped", 3: "gemv-split"}.get(path_taken, "?"),
            "parallelism": "none (1 GPU)",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": kern_name,
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "traffic": traffic,
            "bytes_per_launch": kern_bytes,
            "kernel_id": kern_id,
            "avg_launch_us": round(kern_ms * 1e3, 3),
        },
        "check": {"ids_match": bool(ids_ok), "row0_rel_l2": rel0},
    }
    if not args.no_cpu_baseline:
        log("cpu baseline ...")
        rec["cpu_baseline"] = cpu_baseline(inp, sh, metric_bytes, args.cpu_seconds)
    plan.close()
    line = json.dumps(rec)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()
