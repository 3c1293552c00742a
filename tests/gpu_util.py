"""Helpers for the GPU tests: move seeded groups to the device, run the HIP
library through its binding, and sample outputs for the oracle."""
from __future__ import annotations

import sys
from typing import List

import numpy as np


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


def device_args(groups, dev="cuda:0"):
    import torch
    args = []
    for g in groups:
        t = [torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in (g.a, g.b, g.sfa, g.sfb)]
        c = torch.full((g.m, g.n), float("nan"), dtype=torch.float16, device=dev)  # poison
        args.append(tuple(t) + (c,))
    return args


def run_gpu(groups, stream=None) -> List[np.ndarray]:
    import torch
    import block_scaled_fp4_group_amd as nv
    args = device_args(groups)
    nv.group_gemm(args, stream=stream)
    torch.cuda.synchronize()
    return [a[4].cpu().numpy().view(np.uint16) for a in args]


def sample_positions(m, n, count, rng, tile_rows=64, tile_cols=64):
    """Random positions plus every tile's corners and the ragged edges."""
    rows = list(rng.integers(0, m, count))
    cols = list(rng.integers(0, n, count))
    edge_r = sorted({0, m - 1} | {min(m - 1, x) for t in range(0, m, tile_rows) for x in (t, t + tile_rows - 1)})
    edge_c = sorted({0, n - 1} | {min(n - 1, x) for t in range(0, n, tile_cols) for x in (t, t + tile_cols - 1)})
    for r in edge_r:
        for c in edge_c[:: max(1, len(edge_c) // 64)]:
            rows.append(r); cols.append(c)
    for c in edge_c:
        rows.append(edge_r[len(edge_r) // 2]); cols.append(c)
    return np.array(rows, np.int32), np.array(cols, np.int32)
