"""Helpers for the GPU tests: move seeded groups to the device and run the
HIP library through its binding."""
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
    st = stream if stream is not None else torch.cuda.current_stream()
    assert nv.stream_errors(st.cuda_stream) == 0, "a hand-off wait ran out"
    return [a[4].cpu().numpy().view(np.uint16) for a in args]
