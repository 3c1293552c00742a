#!/usr/bin/env python3
"""Benchmark of the MI355X NVFP4 grouped GEMM.

Times the HIP library on the 8-group MoE-like workload (N = 4096, K = 7168,
M = 80, 176, 128, 72, 64, 248, 96, 160) with seeded synthetic inputs resident
in HBM, and prints one JSON line with:
- TFLOP/s (2*sum(MNK)/t);
- the roofline of the kernel (algorithmic bytes / mean kernel time from HIP
  events on the launch stream, against 8 TB/s HBM);
- the same figures for every one of the five workloads (`config.per_workload`),
  each also as a fraction of the dense f16 MFMA peak the kernel computes on;
- the host cost of one call and of one graph replay of the small workload;
- for the four large workloads, the kernel time with B's scales in the
  optional window-major layout (`sfb_window_major_us`; the headline figures
  use the plain row-major scales the inputs come in);
- the CPU oracle timed on a bounded sample as a baseline.

Cold-cache protocol: each step runs on one of R input/output replicas in
rotation, with R chosen so the replicas together exceed twice the 256 MB
Infinity Cache; a step never finds its operands in any cache.

Other modes: --mfma-rates prints the measured sustained matrix-core rates and
clock; --summarize-trace FILE turns a rocprofv3 kernel trace of a default run
into per-workload kernel times; --oracle-timing times the oracle on every
workload.
"""
from __future__ import annotations

import argparse
import csv
import ctypes
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
HEADLINE = 1                   # index of the 8-group N=4096 K=7168 workload
PER_WORKLOAD_STEPS = 20
PER_WORKLOAD_WARMUP = 5
HOST_CALLS = 200


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", type=int, default=HEADLINE,
                   help="workload of the headline figures (default: the 8-group N=4096 K=7168 case)")
    p.add_argument("--warm-cache", action="store_true", help="reuse one replica (numbers labelled warm)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--headline-only", action="store_true", help="skip the per-workload array")
    p.add_argument("--oracle-timing", action="store_true",
                   help="time the oracle on every workload with 1 thread and with all threads, then exit")
    p.add_argument("--mfma-rates", action="store_true", help="measure sustained MFMA rates and clock, then exit")
    p.add_argument("--summarize-trace", metavar="KERNEL_TRACE_CSV",
                   help="per-workload kernel times from a rocprofv3 kernel trace of a default run, then exit")
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


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


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


def launches_per_step(w):
    """Kernel launches of one call (one per batch of up to 32 non-empty groups)."""
    n = sum(1 for (m, n_, k) in w.shapes if m and n_)
    return max(1, -(-n // 32))


def time_workload(w, steps, warmup, warm_cache, sfb_swizzled=False):
    """Protocol of one workload (the trace summary relies on its launch
    order): `warmup` untimed calls, `steps` timed calls bracketed by one
    event pair on the launch stream (and host wall time), then `steps`
    single calls each bracketed by its own events.  With sfb_swizzled, B's
    scales are first copied into the window-major layout (nvfp4_swizzle_scales,
    outside the timed calls) and passed with NVFP4_SFB_SWIZZLED."""
    import torch
    import block_scaled_fp4_group_amd as nv
    dev = torch.device("cuda:0")
    groups = workloads.generate(w)
    nbytes = workloads.config_bytes(w.shapes)
    flops = workloads.config_flops(w.shapes)
    reps = 1 if warm_cache else max(2, -(-2 * MALL_BYTES // max(1, nbytes)) + 1)
    replicas = build_replicas(groups, reps, dev)
    if sfb_swizzled:
        replicas = [[(a, b, sa, nv.swizzle_scales(sb), c) for (a, b, sa, sb, c) in rep] for rep in replicas]
        descs = [[nv._descriptor(*g, sfb_swizzled=True) for g in rep] for rep in replicas]
    else:
        descs = [[nv._descriptor(*g) for g in rep] for rep in replicas]
    stream = torch.cuda.current_stream()
    sid = stream.cuda_stream
    for i in range(warmup):
        nv.group_gemm_raw(descs[i % reps], sid)
    torch.cuda.synchronize()
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
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        nv.group_gemm_raw(descs[i % reps], sid)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    if nv.stream_errors(sid) != 0:
        raise RuntimeError("bench.py: a hand-off wait ran out during %s" % w.name)
    per = np.array([a.elapsed_time(b) for a, b in ev])       # ms, one call each
    return dict(groups=groups, flops=flops, nbytes=nbytes, reps=reps, wall_ms=wall * 1e3 / steps,
                ev_ms_mean=float(batch_ms), ev_ms_median=float(np.median(per)), ev_ms_min=float(per.min()),
                launches=launches_per_step(w))


def host_and_graph_cost(w):
    """Host time of one call (argument marshalling, plan cache hit, launch)
    measured over HOST_CALLS back-to-back calls without synchronising, and
    the device time of one replay of a captured call."""
    import torch
    import block_scaled_fp4_group_amd as nv
    dev = torch.device("cuda:0")
    groups = workloads.generate(w)
    rep = build_replicas(groups, 1, dev)[0]
    descs = [nv._descriptor(*g) for g in rep]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for _ in range(5):
            nv.group_gemm_raw(descs, s.cuda_stream)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(HOST_CALLS):
            nv.group_gemm_raw(descs, s.cuda_stream)
        host_us = (time.perf_counter() - t0) / HOST_CALLS * 1e6
        torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        nv.group_gemm_raw(descs, s.cuda_stream)
    torch.cuda.synchronize()
    for _ in range(5):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(HOST_CALLS):
        g.replay()
    e1.record(s)
    torch.cuda.synchronize()
    return round(host_us, 2), round(e0.elapsed_time(e1) / HOST_CALLS * 1e3, 2)


def roofline(flops, nbytes, seconds, traffic=None):
    """Binding roofline of the workload: HBM (algorithmic bytes at 8 TB/s) or
    dense FP4 MFMA, whichever takes longer; achieved = algorithmic bytes (or
    flops) per launch / mean launch time."""
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    t_fp4 = flops / (MFMA_PEAK_TFLOPS["fp4"] * 1e12)
    if t_hbm >= t_fp4:
        ach = nbytes / seconds / 1e9
        return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic}
    ach = flops / seconds / 1e12
    pk = MFMA_PEAK_TFLOPS["fp4"]
    return {"bound": "mfma", "achieved": round(ach, 1), "peak": pk, "unit": "TFLOP/s",
            "frac": round(ach / pk, 4), "traffic": traffic}


def workload_entry(w, r, warm_cache):
    s = r["ev_ms_mean"] * 1e-3
    tf = r["flops"] / s / 1e12
    rf = roofline(r["flops"], r["nbytes"], s)
    return {"workload": w.name, "us": round(s * 1e6, 2), "tflops": round(tf, 2),
            "gbs": round(r["nbytes"] / s / 1e9, 1), "bound": rf["bound"], "roofline_frac": rf["frac"],
            "hbm_frac": round(r["nbytes"] / s / 1e9 / HBM_PEAK_GBS, 4),
            "f16_mfma_frac": round(tf / MFMA_PEAK_TFLOPS["f16"], 4),
            "single_call_us_median": round(r["ev_ms_median"] * 1e3, 2),
            "cache": "warm" if warm_cache else "cold (%d replicas)" % r["reps"]}


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
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": "full fp64 oracle GEMM of %d of %d groups of %s (%.2f GFLOP), %.1f s wall"
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
                              "tflops": round(flops / dt / 1e12, 6), "kind": "oracle",
                              "cpu_model": cpu_model()}), flush=True)


def mfma_rates():
    import torch
    torch.cuda.init()
    path = os.path.join(_REPO, "block_scaled_fp4_group_amd", "libnvfp4gg_probe.so")
    if not os.path.exists(path):
        raise RuntimeError("libnvfp4gg_probe.so is not built; run __graft_entry__.build()")
    L = ctypes.CDLL(path)
    L.nvfp4_probe_mfma_rates.restype = ctypes.c_int
    L.nvfp4_probe_mfma_rates.argtypes = [ctypes.c_char_p, ctypes.c_int]
    buf = ctypes.create_string_buffer(8192)
    rc = L.nvfp4_probe_mfma_rates(buf, 8192)
    sys.stdout.write(buf.value.decode())
    if rc != 0:
        raise RuntimeError("mfma rate probe: a HIP call failed")


def trace_protocol(steps, warmup, headline_only, config=HEADLINE):
    """Kernel launches of a run in order: (label, count) blocks, the timed
    regions marked."""
    blocks = []

    def add(w, st, wu, tag=""):
        n = launches_per_step(w)
        blocks.append((w.name + tag + " warmup", wu * n, False))
        blocks.append((w.name + tag + " timed", st * n, True))
        blocks.append((w.name + tag + " single", st * n, False))
    add(workloads.CONFIGS[config], steps, warmup)
    if not headline_only:
        for i, w in enumerate(workloads.CONFIGS):
            add(w, PER_WORKLOAD_STEPS, PER_WORKLOAD_WARMUP)
            if i > 0:
                add(w, PER_WORKLOAD_STEPS, PER_WORKLOAD_WARMUP, " (window-major sfb)")
    return blocks


def summarize_trace(path, steps, warmup, headline_only, config=HEADLINE):
    """Mean kernel duration per timed region of a rocprofv3 --kernel-trace
    CSV of `bench.py --steps S --warmup W` (the GEMM kernel's dispatches in
    order; graph replays and host-cost calls come after the blocks)."""
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            name = r.get("Kernel_Name", "")
            if "nvfp4_group_gemm_kernel" in name or "nvfp4_direct_kernel" in name:
                rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    rows.sort()
    durs = [(e - s) / 1e3 for s, e in rows]
    i = 0
    print("kernel dispatches in trace: %d" % len(durs))
    for label, n, timed in trace_protocol(steps, warmup, headline_only, config):
        seg = durs[i:i + n]
        i += n
        if timed and seg:
            print("%-66s launches %3d  mean %8.2f us  median %8.2f us  min %8.2f us"
                  % (label, len(seg), float(np.mean(seg)), float(np.median(seg)), float(np.min(seg))))
    print("remaining dispatches (host-cost calls, graph replays): %d" % max(0, len(durs) - i))


def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.steps, args.warmup, args.headline_only, args.config)
        return
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
    if args.mfma_rates:
        mfma_rates()
        return
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
    per_workload = []
    if not args.headline_only:
        for i, wc in enumerate(workloads.CONFIGS):
            rc = time_workload(wc, PER_WORKLOAD_STEPS, PER_WORKLOAD_WARMUP, args.warm_cache)
            per_workload.append(workload_entry(wc, rc, args.warm_cache))
            del rc
            torch.cuda.empty_cache()
            if i > 0:
                # the optional window-major layout of B's scales (a one-time
                # copy of a weight operand's scales), timed right after the
                # plain layout the inputs come in, which the headline uses
                rc = time_workload(wc, PER_WORKLOAD_STEPS, PER_WORKLOAD_WARMUP, args.warm_cache,
                                   sfb_swizzled=True)
                per_workload[-1]["sfb_window_major_us"] = round(rc["ev_ms_mean"] * 1e3, 2)
                del rc
                torch.cuda.empty_cache()
        host_us, graph_us = host_and_graph_cost(workloads.CONFIGS[0])
        per_workload[0]["host_us_per_call"] = host_us
        per_workload[0]["graph_replay_us"] = graph_us
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
                   "single_launch_ms_min": round(r["ev_ms_min"], 5),
                   "f16_mfma_frac": round(r["flops"] / kern_s / 1e12 / MFMA_PEAK_TFLOPS["f16"], 4),
                   "per_workload": per_workload},
        "roofline": roofline(r["flops"], r["nbytes"], kern_s,
                             None if args.warm_cache else measured_traffic(w.name)),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, r["groups"])
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
