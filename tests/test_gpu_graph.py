"""Calls captured in a HIP graph and replayed.  The partial sums of split
tiles are handed over through flags whose epoch lives in device memory, so
every replay gets a fresh epoch.  Consecutive replays run on new inputs
(uploaded between them, with no other library call); every output of every
replay is compared with the oracle on those inputs, and with an eager call
bit for bit.  The allocation-free entry point is captured the same way on a
stream that has never been used, and the regular one refuses such a stream
(it needs its workspace) unless the launch is tiny enough for the direct
path, which needs none."""
import numpy as np
import pytest

import oracle
import workloads
from tests.compare import compare_fp16
from tests.conftest import gpu_available
from tests.gpu_util import device_args, log

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X")]

SHAPES = [(200, 512, 2048), (72, 1024, 4096), (130, 256, 1536)]   # every tile split
REPLAYS = 4


TINY = [(64, 128, 256), (128, 256, 256)]   # config 0's shapes: the direct path


def _fresh(seed, shapes=SHAPES):
    return workloads.generate(workloads.make_workload(shapes, (-4, 2), seed, "graph"))


def _load(args, groups):
    import torch
    for (a, b, sa, sb, _), f in zip(args, groups):
        for dst, src in ((a, f.a), (b, f.b), (sa, f.sfa), (sb, f.sfb)):
            dst.copy_(torch.from_numpy(np.ascontiguousarray(src)))
    torch.cuda.synchronize()


def _replay_and_check(g, args, descs, stream, eager_fn, shapes=SHAPES):
    import torch
    import block_scaled_fp4_group_amd as nv
    replayed = []
    for rep in range(REPLAYS):
        log("graph replay %d" % rep)
        _load(args, _fresh(100 + rep, shapes))
        g.replay()
        torch.cuda.synchronize()
        replayed.append([x[4].cpu().numpy().view(np.uint16).copy() for x in args])
    assert nv.stream_errors(stream.cuda_stream) == 0
    for rep in range(REPLAYS):
        groups = _fresh(100 + rep, shapes)
        r16, r64 = oracle.group_gemm(groups)
        for i, (got, rb, rx) in enumerate(zip(replayed[rep], r16, r64)):
            res = compare_fp16(got, rb, rx)
            assert res.failures == 0, "replay %d group %d against the oracle: %s" % (rep, i, res)
        _load(args, groups)
        eager_fn()
        torch.cuda.synchronize()
        for i, (r, x) in enumerate(zip(replayed[rep], args)):
            nd = int((r != x[4].cpu().numpy().view(np.uint16)).sum())
            assert nd == 0, "replay %d group %d: %d outputs differ from the eager call" % (rep, i, nd)


def test_graph_replays_match_oracle_and_eager():
    import torch
    import block_scaled_fp4_group_amd as nv
    assert any(seg[7] == 2 for seg in nv.plan([nv.make_group(a=0x1000, b=0x1000, sfa=0x1000, sfb=0x1000, c=0x1000,
                                                             m=m, n=n, k=k) for m, n, k in SHAPES], 256))
    args = device_args(_fresh(11))
    descs = [nv._descriptor(*a) for a in args]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        nv.group_gemm_raw(descs, s.cuda_stream)     # creates this stream's workspace outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        nv.group_gemm_raw(descs, s.cuda_stream)
    torch.cuda.synchronize()

    def eager():
        with torch.cuda.stream(s):
            nv.group_gemm_raw(descs, s.cuda_stream)
    _replay_and_check(g, args, descs, s, eager)


def test_noalloc_capture_on_a_new_stream():
    import torch
    import block_scaled_fp4_group_amd as nv
    args = device_args(_fresh(12))
    descs = [nv._descriptor(*a) for a in args]
    s = torch.cuda.Stream()                         # never used before: no workspace
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        nv.group_gemm_noalloc_raw(descs, s.cuda_stream)
    torch.cuda.synchronize()

    def eager():
        with torch.cuda.stream(s):
            nv.group_gemm_noalloc_raw(descs, s.cuda_stream)
    _replay_and_check(g, args, descs, s, eager)


def test_regular_entry_refuses_capture_without_workspace():
    import torch
    import block_scaled_fp4_group_amd as nv
    args = device_args(_fresh(13))
    descs = [nv._descriptor(*a) for a in args]
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with pytest.raises(nv.Nvfp4Error) as err:
        with torch.cuda.graph(g, stream=s):
            nv.group_gemm_raw(descs, s.cuda_stream)
    assert err.value.code == nv.NVFP4_EUNSUPPORTED
    torch.cuda.synchronize()


def test_direct_path_capture_on_a_new_stream():
    import torch
    import block_scaled_fp4_group_amd as nv
    args = device_args(_fresh(14, TINY))
    descs = [nv._descriptor(*a) for a in args]
    s = torch.cuda.Stream()                         # never used before: no workspace, none needed
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        nv.group_gemm_raw(descs, s.cuda_stream)
    torch.cuda.synchronize()

    def eager():
        with torch.cuda.stream(s):
            nv.group_gemm_raw(descs, s.cuda_stream)
    _replay_and_check(g, args, descs, s, eager, TINY)
