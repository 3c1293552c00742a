#!/usr/bin/env python3
"""Benchmark of the MI355X NVFP4 grouped GEMM.

Times the HIP library on the 8-group MoE-like workload (N = 4096, K = 7168,
M = 80, 176, 128, 72, 64, 248, 96, 160) with seeded synthetic inputs resident
in HBM, and prints one JSON line: TFLOP/s (2*sum(MNK)/t), the roofline of the
kernel (algorithmic bytes / measured kernel time against 8 TB/s HBM), and the
CPU oracle timed on a bounded sample as a baseline.

Cold-cache protocol: each step runs on one of R input/output replicas in
rotation, with R chosen so the replicas together exceed twice the 256 MB
Infinity Cache; a step never finds its operands in any cache.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

_REPO = os.path.dirname(os.path.abspath(__file__))
if _REPO not in sys.path:
    sys.path.insert(0, _REPO)

import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"fp4": 10100.0, "fp8": 5000.0, "f16": 2500.0}
MALL_BYTES = 256 << 20


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--config", type=int, default=1, help="workload index (default: the 8-group N=4096 K=7168 case)")
    p.add_argument("--warm-cache", action="store_true", help="reuse one replica (numbers labelled warm)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--all-configs", action="store_true", help="also report every workload on stderr")
    p.add_argument("--oracle-timing", action="store_true",
                   help="time the oracle on every workload with 1 thread and with all threads, then exit")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                   help="run one plain device-to-device copy of BYTES first (counter calibration)")
    return p.parse_args()


KERNEL_SOURCE = os.path.join(_REPO, "block_scaled_fp4_group_amd", "csrc", "nvfp4_group_gemm.hip")
PROFILES = os.path.join(_REPO, "profiles")


def kernel_source_sha():
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(workload_name):
    """HBM bytes per launch from the committed counter summary of this
    workload (FETCH_SIZE + WRITE_SIZE, each scaled by the same counter's
    reading for a plain copy of known size), or None when there is none or
    the kernel source has changed since the counters were taken."""
    path = os.path.join(PROFILES, "nvfp4_group_gemm_kernel_%s_traffic.txt" % workload_name)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith(" "):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != kernel_source_sha():
        return None
    try:
        return int(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def build_replicas(groups, reps, dev):
    import torch
    base = []
    for g in groups:
        base.append([torch.from_numpy(x).to(dev) for x in (g.a, g.b, g.sfa, g.sfb)])
    replicas = []
    for r in range(reps):
        rep = []
        for g, (a, b, sa, sb) in zip(groups, base):
            c = torch.empty((g.m, g.n), dtype=torch.float16, device=dev)
            if r == 0:
                rep.append((a, b, sa, sb, c))
            else:
                rep.append((a.clone(), b.clone(), sa.clone(), sb.clone(), c))
        replicas.append(rep)
    return replicas


def time_workload(w, steps, warmup, warm_cache):
    import torch
    import block_scaled_fp4_group_amd as nv
    dev = torch.device("cuda:0")
    groups = workloads.generate(w)
    nbytes = workloads.config_bytes(w.shapes)
    flops = workloads.config_flops(w.shapes)
    reps = 1 if warm_cache else max(2, -(-2 * MALL_BYTES // max(1, nbytes)) + 1)
    replicas = build_replicas(groups, reps, dev)
    descs = [[nv._descriptor(*g) for g in rep] for rep in replicas]
    stream = torch.cuda.current_stream()
    sid = stream.cuda_stream
    for i in range(warmup):
        nv.group_gemm_raw(descs[i % reps], sid)
    torch.cuda.synchronize()
    # timed region: exactly `steps` launches, one event pair on the launch
    # stream around all of them (per-launch events would add their own
    # dispatch overhead to every launch)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        nv.group_gemm_raw(descs[i % reps], sid)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    batch_ms = e0.elapsed_time(e1) / steps
    # distribution of single launches, measured after the timed region
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        nv.group_gemm_raw(descs[i % reps], sid)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    per = np.array([a.elapsed_time(b) for a, b in ev])       # ms, one launch each
    return dict(groups=groups, flops=flops, nbytes=nbytes, reps=reps, wall_ms=wall * 1e3 / steps,
                ev_ms_mean=float(batch_ms), ev_ms_median=float(np.median(per)), ev_ms_min=float(per.min()))


def roofline(flops, nbytes, seconds, traffic=None):
    """Binding roofline of the workload: HBM (algorithmic bytes at 8 TB/s) or
    dense FP4 MFMA, whichever takes longer; achieved = algorithmic bytes (or
    flops) per launch / mean launch time."""
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    t_fp4 = flops / (MFMA_PEAK_TFLOPS["fp4"] * 1e12)
    bound = "hbm" if t_hbm >= t_fp4 else "mfma"
    if bound == "hbm":
        ach = nbytes / seconds / 1e9
        return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic}
    ach = flops / seconds / 1e12
    pk = MFMA_PEAK_TFLOPS["fp4"]
    return {"bound": "mfma", "achieved": round(ach, 1), "peak": pk, "unit": "TFLOP/s",
            "frac": round(ach / pk, 4), "traffic": traffic}


def cpu_baseline(w, groups, budget_s=20.0):
    """The oracle as it stands, on the host cores, over whole groups of the
    same workload taken in order until about budget_s of wall time (at least
    one group), scaled to TFLOP/s."""
    import oracle
    fl, dt, used = 0.0, 0.0, 0
    for g in groups:
        t0 = time.perf_counter()
        oracle.gemm_group(g.a, g.sfa, g.b, g.sfb, g.m, g.n, g.k)
        dt += time.perf_counter() - t0
        fl += 2.0 * g.m * g.n * g.k
        used += 1
        if dt >= budget_s:
            break
    return {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.max_threads(),
            "kind": "oracle", "sample": "full fp64 oracle GEMM of %d of %d groups of %s (%.2f GFLOP), %.1f s wall"
            % (used, len(groups), w.name, fl / 1e9, dt)}


def oracle_timing():
    """The oracle as it stands on every workload, whole, once with one
    thread and once with all host threads: one JSON line each."""
    import oracle
    for w in workloads.CONFIGS:
        groups = workloads.generate(w)
        flops = workloads.config_flops(w.shapes)
        for nt in (1, oracle.max_threads()):
            t0 = time.perf_counter()
            for g in groups:
                oracle.gemm_group(g.a, g.sfa, g.b, g.sfb, g.m, g.n, g.k, nt)
            dt = time.perf_counter() - t0
            print(json.dumps({"workload": w.name, "threads": nt, "seconds": round(dt, 3),
                              "tflops": round(flops / dt / 1e12, 6), "kind": "oracle"}), flush=True)


def main():
    args = parse()
    if args.oracle_timing:
        oracle_timing()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only (the grouped GEMM shards by group or "
              "by N with no exchange; multi-GPU runs are not part of it). Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    w = workloads.CONFIGS[args.config]
    if args.calibrate_copy > 0:
        n = args.calibrate_copy // 4
        src = torch.ones(n, dtype=torch.int32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print("bench.py: calibration copy of %d bytes done" % (4 * n), file=sys.stderr, flush=True)
        del src, dst
    r = time_workload(w, args.steps, args.warmup, args.warm_cache)
    kern_s = r["ev_ms_mean"] * 1e-3
    tflops = r["flops"] / (r["wall_ms"] * 1e-3) / 1e12     # whole-job rate over the timed steps
    line = {
        "metric": "grouped NVFP4 GEMM TFLOP/s (2*sum(MNK)/t) and % of binding roofline, 1 MI355X",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["wall_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4 operands -> f16 mfma, f32 accumulate, f16 out",
        "data": "synthetic (seeded, uniform E2M1 codes, E4M3FN scales 2^e(1+m/8))",
        "config": {"workload": w.name, "groups": len(w.shapes), "shapes_mnk": [list(s) for s in w.shapes],
                   "cache": "warm" if args.warm_cache else "cold (%d rotating replicas)" % r["reps"],
                   "gflop": round(r["flops"] / 1e9, 3), "alg_bytes_mb": round(r["nbytes"] / 1e6, 3),
                   "kernel_ms_mean": round(r["ev_ms_mean"], 5),
                   "single_launch_ms_median": round(r["ev_ms_median"], 5),
                   "single_launch_ms_min": round(r["ev_ms_min"], 5)},
        "roofline": roofline(r["flops"], r["nbytes"], kern_s,
                             None if args.warm_cache else measured_traffic(w.name)),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, r["groups"])
    if args.all_configs:
        for i, wc in enumerate(workloads.CONFIGS):
            rc = time_workload(wc, max(10, args.steps // 2), 5, args.warm_cache)
            s = rc["ev_ms_mean"] * 1e-3
            rf = roofline(rc["flops"], rc["nbytes"], s)
            print(json.dumps({"workload": wc.name, "us": round(s * 1e6, 2),
                              "tflops": round(rc["flops"] / s / 1e12, 2),
                              "gbs": round(rc["nbytes"] / s / 1e9, 1), "roofline": rf,
                              "cache": "warm" if args.warm_cache else "cold"}), file=sys.stderr, flush=True)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
