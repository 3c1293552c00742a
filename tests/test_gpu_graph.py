"""A call captured in a HIP graph and replayed: the partial sums of split
tiles are handed over through flags whose epoch lives in device memory, so
every replay gets a fresh epoch.  Four consecutive replays run on new inputs
(uploaded between them, with no other library call), and each must match an
eager call on the same inputs bit for bit."""
import numpy as np
import pytest

import workloads
from tests.conftest import gpu_available
from tests.gpu_util import device_args, log

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X")]

SHAPES = [(200, 512, 2048), (72, 1024, 4096), (130, 256, 1536)]   # every tile split


def test_graph_replays_match_eager():
    import torch
    import block_scaled_fp4_group_amd as nv
    base = workloads.generate(workloads.make_workload(SHAPES, (-4, 2), 11, "graph"))
    assert any(seg[7] == 2 for seg in nv.plan([nv.make_group(a=0x1000, b=0x1000, sfa=0x1000, sfb=0x1000, c=0x1000, m=m, n=n, k=k)
                                                for m, n, k in SHAPES], 256))
    args = device_args(base)
    descs = [nv._descriptor(*a) for a in args]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        nv.group_gemm_raw(descs, s.cuda_stream)     # creates this stream's workspace outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        nv.group_gemm_raw(descs, s.cuda_stream)
    torch.cuda.synchronize()
    def load(seed):
        fresh = workloads.generate(workloads.make_workload(SHAPES, (-4, 2), seed, "graph"))
        for (a, b, sa, sb, _), f in zip(args, fresh):
            for dst, src in ((a, f.a), (b, f.b), (sa, f.sfa), (sb, f.sfb)):
                dst.copy_(torch.from_numpy(np.ascontiguousarray(src)))
        torch.cuda.synchronize()

    # consecutive replays with no library call between them (only new inputs)
    replayed = []
    for rep in range(4):
        log("graph replay %d" % rep)
        load(100 + rep)
        g.replay()
        torch.cuda.synchronize()
        replayed.append([x[4].cpu().numpy().view(np.uint16).copy() for x in args])
    # then each replay against an eager call on the same inputs
    for rep in range(4):
        load(100 + rep)
        with torch.cuda.stream(s):
            nv.group_gemm_raw(descs, s.cuda_stream)
        torch.cuda.synchronize()
        eager = [x[4].cpu().numpy().view(np.uint16) for x in args]
        for i, (r, e) in enumerate(zip(replayed[rep], eager)):
            nd = int((r != e).sum())
            assert nd == 0, "replay %d group %d: %d outputs differ from the eager call" % (rep, i, nd)
