"""The allocation-free entry point (nvfp4_group_gemm_noalloc) against the
regular one, on the GPU through the C ABI: two calls in a row, the second on
a smaller input, each bit-identical to nvfp4_group_gemm on the same inputs
(both run the same kernels; only the workspace differs)."""
import numpy as np
import pytest

import workloads
from tests.compare import bits_equal
from tests.conftest import gpu_available
from tests.gpu_util import device_args, log

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X")]


def run_both(groups, label):
    import torch
    import block_scaled_fp4_group_amd as nv
    log("gpu case: no-alloc %s shapes=%s" % (label, [(g.m, g.n, g.k) for g in groups]))
    args_a = device_args(groups)
    args_b = [t[:4] + (torch.full_like(t[4], float("nan")),) for t in args_a]
    sid = torch.cuda.current_stream().cuda_stream
    nv.group_gemm_raw([nv._descriptor(*t) for t in args_a], sid)
    nv.group_gemm_noalloc_raw([nv._descriptor(*t) for t in args_b], sid)
    torch.cuda.synchronize()
    for i, (ta, tb) in enumerate(zip(args_a, args_b)):
        ref = ta[4].cpu().numpy().view(np.uint16)
        got = tb[4].cpu().numpy().view(np.uint16)
        nd, where = bits_equal(got, ref)
        assert nd == 0, "%s group %d: %d outputs differ from nvfp4_group_gemm at %s" % (label, i, nd, where)


def test_noalloc_matches_regular_entry_twice():
    # a large launch with split tiles, then a smaller one on the same static workspace
    run_both(workloads.generate(workloads.CONFIGS[1]), "moe8 n4096 k7168")
    run_both(workloads.generate(workloads.CONFIGS[0]), "two small groups")
