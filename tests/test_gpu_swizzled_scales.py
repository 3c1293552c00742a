"""The optional window-major layout of B's scales (nvfp4_swizzle_scales and
NVFP4_SFB_SWIZZLED): the layout against its definition, and GEMM results with
swizzled scales bit for bit against the same call with plain scales (the
arithmetic is the same; only where the scale bytes are read from changes),
on both kernels, on split tiles, through the exact recomputation, and
against the oracle."""
import numpy as np
import pytest

import oracle
import workloads
from tests.compare import compare_fp16
from tests.conftest import gpu_available
from tests.gpu_util import device_args, log

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X")]


def _layout(sf: np.ndarray, rows: int, k: int) -> np.ndarray:
    """The window-major layout written out (test-side restatement of the
    header's definition): [row block][window][row in block][16 bytes]."""
    nb = k // 16
    windows = -(-k // 256)
    rp = -(-rows // 32) * 32
    src = np.zeros((rp, windows * 16), np.uint8)
    src[:rows, :nb] = sf.reshape(rows, nb)
    src[rows:, :nb] = sf.reshape(rows, nb)[rows - 1]          # padding rows repeat the last row
    return src.reshape(rp // 32, 32, windows, 16).transpose(0, 2, 1, 3).reshape(-1)


@pytest.mark.parametrize("rows,k", [(1, 64), (33, 256), (100, 448), (4096, 7168), (17, 1024)])
def test_swizzle_layout(rows, k):
    import torch
    import block_scaled_fp4_group_amd as nv
    rng = np.random.default_rng(rows + k)
    sf = rng.integers(0, 256, size=(rows, k // 16), dtype=np.uint8)
    out = nv.swizzle_scales(torch.from_numpy(sf).cuda())
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    want = _layout(sf, rows, k)
    assert got.size == nv.swizzled_scale_bytes(rows, k) == want.size
    assert np.array_equal(got, want)


def _run(groups, swizzled, stream=None):
    import torch
    import block_scaled_fp4_group_amd as nv
    args = device_args(groups)
    descs = []
    keep = []
    for (a, b, sa, sb, c) in args:
        if swizzled and b.shape[0] > 0 and a.shape[1] > 0:
            sbz = nv.swizzle_scales(sb)
            keep.append(sbz)
            descs.append(nv._descriptor(a, b, sa, sbz, c, sfb_swizzled=True))
        else:
            descs.append(nv._descriptor(a, b, sa, sb, c))
    st = stream if stream is not None else torch.cuda.current_stream()
    nv.group_gemm_raw(descs, st.cuda_stream)
    torch.cuda.synchronize()
    assert nv.stream_errors(st.cuda_stream) == 0
    return [x[4].cpu().numpy().view(np.uint16) for x in args]


def _same(groups, label, path=None, check_oracle=False):
    from tests.test_gpu_parity import forced_path
    log("gpu case: swizzled sfb, %s" % label)
    with forced_path(path):
        plain = _run(groups, False)
        swz = _run(groups, True)
    for i, (x, y) in enumerate(zip(plain, swz)):
        nd = int((x != y).sum())
        assert nd == 0, "%s group %d: %d outputs differ from the plain-scale call" % (label, i, nd)
    if check_oracle:
        r16, r64 = oracle.group_gemm(groups)
        for i, (g, rb, rx) in enumerate(zip(swz, r16, r64)):
            rep = compare_fp16(g, rb, rx)
            assert rep.failures == 0, "%s group %d: %s" % (label, i, rep)
    return swz


@pytest.mark.parametrize("cfg", [1, 4])
def test_swizzled_sfb_full_configs(cfg):
    w = workloads.CONFIGS[cfg]
    _same(workloads.generate(w), w.name, check_oracle=True)


@pytest.mark.parametrize("path", ["main", "direct"])
def test_swizzled_sfb_small_shapes(path):
    from tests.test_gpu_parity import DIRECT_SHAPES
    groups = workloads.generate(workloads.make_workload(DIRECT_SHAPES, (-8, 4), 61, "swz_small"))
    _same(groups, "small shapes, %s path" % path, path=path, check_oracle=True)


def test_swizzled_sfb_split_tiles():
    from tests.test_gpu_parity import SPLIT_SHAPES
    groups = workloads.generate(workloads.make_workload(SPLIT_SHAPES, (-4, 2), 62, "swz_split"))
    _same(groups, "split tiles")


def test_swizzled_sfb_exact_recompute():
    """Cancelling outputs, recomputed exactly with scales read from the
    window-major layout (including a ragged N: columns past N in the last
    32-column block repeat the last column)."""
    m, n = 72, 500
    rows = [5, 30]
    cols = [s + (7 * i) % 32 for s in range(0, 480, 32) for i in range(6)] + [490, 499]
    g = workloads.cancelling(m, n, 8192, rows, cols, (-8, 3), seed=63)
    got = _same([g], "cancelling", check_oracle=True)[0].reshape(m, n).view(np.float16).astype(np.float64)
    assert np.all(got[np.ix_(rows, cols)] == 0.0)
