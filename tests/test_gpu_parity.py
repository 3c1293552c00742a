"""Parity of the HIP grouped GEMM with the oracle, on the GPU, through the
C ABI.  Tolerance: |gpu - ref| <= 2e-3*|ref| + 1e-2 (tests/compare.py), and
bit-exact where fp32 accumulation is provably exact."""
import numpy as np
import pytest

import oracle
import workloads
from tests.compare import bits_equal, compare_fp16
from tests.conftest import gpu_available
from tests.gpu_util import log, run_gpu

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X")]

FINITE_E4M3 = [x for x in range(256) if x not in (0x7F, 0xFF)]


def group(m, n, k, a=None, b=None, sfa=None, sfb=None):
    z = lambda r, c, v=0: np.full((r, c), v, np.uint8)
    return workloads.Group(m, n, k, z(m, k // 2) if a is None else a, z(n, k // 2) if b is None else b,
                           z(m, k // 16, 0x38) if sfa is None else sfa,
                           z(n, k // 16, 0x38) if sfb is None else sfb)


def check_full(groups, label, exact=False):
    log("gpu case: %s shapes=%s" % (label, [(g.m, g.n, g.k) for g in groups]))
    got = run_gpu(groups)
    r16, r64 = oracle.group_gemm(groups)
    for i, (gbits, rb, rx) in enumerate(zip(got, r16, r64)):
        if exact:
            nd, where = bits_equal(gbits, rb)
            assert nd == 0, "%s group %d: %d bit mismatches at %s" % (label, i, nd, where)
        rep = compare_fp16(gbits, rb, rx)
        assert rep.failures == 0, "%s group %d: %s" % (label, i, rep)
    return got


@pytest.mark.parametrize("side", ["a", "b"])
def test_decode_every_code_and_scale(side):
    """Each output isolates one (E2M1 code, E4M3FN scale) pair: bit-exact."""
    k = 64
    rows = 16 * len(FINITE_E4M3)
    codes = np.zeros((rows, k // 2), np.uint8)
    scales = np.full((rows, k // 16), 0x38, np.uint8)
    for r in range(rows):
        kk = (r * 7) % k                          # vary nibble position and scale block
        codes[r, kk // 2] = (r % 16) << (4 * (kk % 2))
        scales[r, kk // 16] = FINITE_E4M3[r // 16]
    other = np.full((16, k // 2), 0x22, np.uint8)   # every element 1.0
    if side == "a":
        g = group(rows, 16, k, a=codes, sfa=scales, b=other)
    else:
        g = group(16, rows, k, b=codes, sfb=scales, a=other)
    check_full([g], "decode-%s" % side, exact=True)


@pytest.mark.parametrize("seed", [0, 1])
def test_small_ragged_shapes(seed):
    rng = np.random.default_rng(seed)
    shapes = [(1, 17, 64), (65, 130, 320), (130, 64, 576), (200, 300, 1024), (16, 1, 128), (63, 65, 2048)]
    w = workloads.make_workload(shapes, e_range=(-8, 4), seed=seed)
    check_full(workloads.generate(w), "ragged seed %d" % seed)


@pytest.mark.parametrize("seed", range(4))
def test_random_shapes_full(seed):
    """Random groups (some empty, ragged M and N, K from 64 to 3072) through
    the whole schedule, compared element by element."""
    rng = np.random.default_rng(500 + seed)
    shapes = [(int(rng.integers(0, 260)), int(rng.integers(0, 700)), 64 * int(rng.integers(1, 49)))
              for _ in range(int(rng.integers(2, 9)))]
    w = workloads.make_workload(shapes, e_range=(-6, 3), seed=500 + seed)
    check_full(workloads.generate(w), "random seed %d" % seed)


def test_config0_full():
    check_full(workloads.generate(workloads.CONFIGS[0]), workloads.CONFIGS[0].name)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_config_full(cfg):
    """Every output of the workload at its full size, element by element
    against the oracle's correctly rounded fp16 (and its exact fp64 sum for
    the overflow band)."""
    w = workloads.CONFIGS[cfg]
    check_full(workloads.generate(w), w.name)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_bitexact_unit_scales_full_shape(cfg):
    """All scales 1.0: every term is a multiple of 0.25 and every partial sum
    lies below K * 36 < 2^22, so fp32 accumulation is exact in any order and
    every output of the full workload must equal the oracle bit for bit."""
    w = workloads.CONFIGS[cfg]
    src = workloads.generate(w)
    groups = [group(g.m, g.n, g.k, a=g.a, b=g.b) for g in src]
    check_full(groups, "unit scales, %s" % w.name, exact=True)


@pytest.mark.parametrize("cfg", [1, 4])
def test_bitexact_power_of_two_scales_full_shape(cfg):
    """Every scale drawn from {1/4, 1/2, 1} (E4M3FN 0x28, 0x30, 0x38), per
    16-element block: each term is a multiple of 2^-6 (0.25 times the
    smallest scale product 1/16), and every partial sum stays below
    K * 36 <= 2^18, under 2^24 quanta, so fp32 accumulation is exact in any
    order and every output must equal the oracle bit for bit, with the scale
    path exercised block by block at the full workload shapes."""
    w = workloads.CONFIGS[cfg]
    src = workloads.generate(w)
    rng = np.random.default_rng(30 + cfg)
    codes = np.array([0x28, 0x30, 0x38], np.uint8)
    groups = [group(g.m, g.n, g.k, a=g.a, b=g.b,
                    sfa=codes[rng.integers(0, 3, g.sfa.shape)], sfb=codes[rng.integers(0, 3, g.sfb.shape)])
              for g in src]
    check_full(groups, "power-of-two scales, %s" % w.name, exact=True)


def test_deterministic():
    groups = workloads.generate(workloads.make_workload([(100, 200, 1024), (7, 64, 4096)], (-8, 4), 3))
    log("gpu case: determinism")
    a = run_gpu(groups)
    b = run_gpu(groups)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_edge_cases():
    rng = np.random.default_rng(4)
    w = workloads.make_workload([(3, 5, 64), (1, 1, 64), (17, 129, 192)], (-4, 2), 4)
    groups = workloads.generate(w)
    groups.append(group(4, 9, 0))                                   # k == 0 -> +0
    groups.insert(1, group(0, 8, 64))                              # empty groups are skipped
    groups.insert(2, group(8, 0, 64))
    log("gpu case: edge cases")
    got = run_gpu(groups)
    r16, r64 = oracle.group_gemm(groups)
    for i, (gb, rb, rx) in enumerate(zip(got, r16, r64)):
        assert gb.shape == rb.shape
        rep = compare_fp16(gb, rb, rx)
        assert rep.failures == 0, "group %d: %s" % (i, rep)
    assert (got[-1] == 0).all()


def _random_codes_fixed_scale(rng, shapes, scale_code):
    groups = []
    for m, n, k in shapes:
        groups.append(group(m, n, k, a=rng.integers(0, 256, (m, k // 2), dtype=np.uint8),
                            b=rng.integers(0, 256, (n, k // 2), dtype=np.uint8),
                            sfa=np.full((m, k // 16), scale_code, np.uint8),
                            sfb=np.full((n, k // 16), scale_code, np.uint8)))
    return groups


@pytest.mark.parametrize("path", [None, "main"])
def test_overflow_to_infinity(path):
    """Every scale 24 (E4M3FN 0x5C) on both sides: rms(C) is about 8e4, so
    many outputs overflow fp16 to +-inf (round to nearest even past 65504)
    while the rest are large finite values.  Infinities must match the
    oracle's in sign, finite outputs its value within tolerance.  The
    launch is small enough for the direct kernel; path "main" forces the
    persistent one.  The non-finite error estimate sends every output of a
    wave through the exact recomputation, more than one list of 64."""
    rng = np.random.default_rng(11)
    groups = _random_codes_fixed_scale(rng, [(40, 96, 256), (130, 200, 512)], 0x5C)
    with forced_path(path):
        got = check_full(groups, "overflow, path %s" % path)
    r16, _ = oracle.group_gemm(groups)
    for gb, rb in zip(got, r16):
        ref = rb.view(np.float16)
        n_inf = int(np.isinf(ref).sum())
        assert 0.1 * ref.size < n_inf < 0.9 * ref.size, n_inf      # both kinds of output occur
        assert not np.isnan(gb.view(np.float16)).any()


def test_subnormal_scales_and_outputs_bitexact():
    """Every scale the smallest E4M3FN subnormal, 2^-9 (0x01): each product
    is a multiple of 2^-20 and every partial sum stays below 2^4, so fp32
    accumulation is exact in any order, and the fp16 results (many of them
    subnormal) must equal the oracle's correctly rounded values bit for bit."""
    rng = np.random.default_rng(12)
    groups = _random_codes_fixed_scale(rng, [(33, 70, 1024), (16, 48, 64)], 0x01)
    got = check_full(groups, "subnormal scales", exact=True)
    sub = sum(int(((np.abs(g.view(np.float16)) < 2.0 ** -14) & (g.view(np.float16) != 0)).sum()) for g in got)
    assert sub > 100, sub


def test_long_k_many_parts():
    """K = 32768 (64 folds of 512 k) on one small tile: the tile's 128 stage
    pairs spread over 128 workgroups, so its finalizer adds over a hundred
    partial sums; and a second group of two row tiles with K = 16384."""
    w = workloads.make_workload([(24, 80, 32768), (130, 64, 16384)], (-4, 2), 13, "long_k")
    check_full(workloads.generate(w), "long K")


def test_many_groups_multiple_launches():
    shapes = [(int(m), int(n), 64 * int(kk)) for m, n, kk in
              zip(np.arange(1, 41) * 3, 16 + np.arange(40) * 5, 1 + np.arange(40) % 5)]
    w = workloads.make_workload(shapes, (-6, 3), 5)
    check_full(workloads.generate(w), "40 groups")


def test_nondefault_stream():
    import torch
    groups = workloads.generate(workloads.make_workload([(70, 90, 512)], (-4, 2), 6))
    log("gpu case: side stream")
    s = torch.cuda.Stream()
    got = run_gpu(groups, stream=s)
    r16, r64 = oracle.group_gemm(groups)
    assert compare_fp16(got[0], r16[0], r64[0]).failures == 0


SPLIT_SHAPES = [(200, 512, 2048), (72, 1024, 4096), (130, 256, 1536)]


@pytest.mark.parametrize("spin_limit", [None, "0"])
def test_split_tiles_full(spin_limit):
    """Shapes small enough for the full oracle but with every tile shared by
    several workgroups (fewer (tile, 256-k) units than compute units), so the
    result is assembled from partial sums.  With NVFP4_SPIN_LIMIT=0 the
    finishing workgroup never waits and computes every other part itself:
    the recomputation path must give the same answer."""
    import os
    import block_scaled_fp4_group_amd as nv
    groups = workloads.generate(workloads.make_workload(SPLIT_SHAPES, (-4, 2), 7, "split_tiles"))
    fake = dict(a=0x10000, b=0x20000, sfa=0x30000, sfb=0x40000, c=0x50000)   # plan never dereferences
    segs = nv.plan([nv.make_group(m=g.m, n=g.n, k=g.k, **fake) for g in groups])
    assert any(s[7] == 2 for s in segs) and any(s[7] == 1 for s in segs)
    old = os.environ.get("NVFP4_SPIN_LIMIT")
    try:
        if spin_limit is not None:
            os.environ["NVFP4_SPIN_LIMIT"] = spin_limit
        check_full(groups, "split tiles, spin limit %s" % spin_limit)
    finally:
        if old is None:
            os.environ.pop("NVFP4_SPIN_LIMIT", None)
        else:
            os.environ["NVFP4_SPIN_LIMIT"] = old


def test_config1_recomputed_parts_full():
    """The 8-group K = 7168 workload with every missing part recomputed by
    the finishing workgroup (NVFP4_SPIN_LIMIT=0), every output compared."""
    import os
    old = os.environ.get("NVFP4_SPIN_LIMIT")
    os.environ["NVFP4_SPIN_LIMIT"] = "0"
    try:
        test_config_full(1)
    finally:
        if old is None:
            os.environ.pop("NVFP4_SPIN_LIMIT", None)
        else:
            os.environ["NVFP4_SPIN_LIMIT"] = old


# The direct path (tiny launches: every K <= 512 and few (tile, pair)
# units) against the oracle, and against the persistent path, which can be
# forced with NVFP4_PATH=main (and the direct path with =direct).
DIRECT_SHAPES = [(1, 17, 64), (65, 130, 320), (130, 64, 512), (16, 1, 128), (63, 65, 256), (64, 128, 256),
                 (128, 256, 256), (77, 300, 448), (200, 129, 192)]


class forced_path:
    def __init__(self, path):
        self.path = path

    def __enter__(self):
        import os
        self.old = os.environ.get("NVFP4_PATH")
        if self.path is None:
            os.environ.pop("NVFP4_PATH", None)
        else:
            os.environ["NVFP4_PATH"] = self.path

    def __exit__(self, *exc):
        import os
        if self.old is None:
            os.environ.pop("NVFP4_PATH", None)
        else:
            os.environ["NVFP4_PATH"] = self.old


@pytest.mark.parametrize("path", ["main", "direct"])
@pytest.mark.parametrize("seed", [0, 1])
def test_small_shapes_both_paths(seed, path):
    """Ragged small groups (M, N not multiples of 16, 32, 64 or 128; K from
    64 to 512, not all multiples of 128) in one launch, on each path."""
    groups = workloads.generate(workloads.make_workload(DIRECT_SHAPES, (-8, 4), 40 + seed, "direct"))
    with forced_path(path):
        check_full(groups, "small shapes, %s path, seed %d" % (path, seed))


def test_direct_path_matches_persistent_bitwise():
    """With K <= 256 (one stage pair, so no tile is split) both paths sum
    every output in the same order with the same roundings: bit for bit."""
    shapes = [(s[0], s[1], min(s[2], 256)) for s in DIRECT_SHAPES]
    groups = workloads.generate(workloads.make_workload(shapes, (-8, 4), 44, "direct_vs_main"))
    with forced_path("main"):
        a = check_full(groups, "persistent path, K <= 256")
    with forced_path("direct"):
        b = check_full(groups, "direct path, K <= 256")
    for i, (x, y) in enumerate(zip(a, b)):
        nd = int((x != y).sum())
        assert nd == 0, "group %d: %d outputs differ between the paths" % (i, nd)


def test_direct_path_cancelling_outputs():
    """The direct path's fix-up: outputs that cancel exactly at K = 512
    (scale exponents up to 4 put the typical output near 10^4) come out zero."""
    m, n = 64, 256
    rows, cols = [3, 40], [s + (7 * i) % 32 for s in range(0, n, 32) for i in range(5)]
    g = workloads.cancelling(m, n, 512, rows, cols, (-8, 4), seed=9)
    with forced_path("direct"):
        got = check_full([g], "direct path, cancelling")[0].reshape(m, n).view(np.float16).astype(np.float64)
    zeros = got[np.ix_(rows, cols)]
    assert np.all(zeros == 0.0), "%d cancelling outputs are not zero" % int((zeros != 0).sum())


# Outputs that cancel exactly (workloads.cancelling): their fp32 sums carry
# rounding errors near the absolute tolerance, so they are recomputed
# exactly and must come out as zero.  Scale exponents -8..3 and K = 8192
# put the tile's typical output near 10^4; the small scales make the
# partial sums inexact in fp32 (with exponents >= 0 every sum here would be
# a multiple of 2^-8 below 2^16, exact in fp32, and cancel exactly anyway).
CANCEL_K = 8192
CANCEL_E = (-8, 3)


def _cancel_cols(per_slice, n):
    """`per_slice` columns in every 32-column slice (one wave's columns)."""
    return [s + (7 * i) % 32 for s in range(0, n, 32) for i in range(per_slice)]


def _check_cancelling(g, rows, cols, label):
    got = check_full([g], label)[0].reshape(g.m, g.n).view(np.float16).astype(np.float64)
    zeros = got[np.ix_(rows, cols)]
    assert np.all(zeros == 0.0), "%s: %d of %d cancelling outputs are not zero, largest %g" % (
        label, int((zeros != 0).sum()), zeros.size, float(np.abs(zeros).max()))


@pytest.mark.parametrize("per_slice", [1, 2, 3, 5, 8, 9, 17])
def test_cancelling_outputs_per_wave(per_slice):
    """One row and `per_slice` columns per wave whose outputs are exactly
    zero: every batch width of the exact recomputation (1, 2, up to 4, up to
    8 outputs, and more than one batch)."""
    m, n = 72, 512
    rows, cols = [5], _cancel_cols(per_slice, n)
    g = workloads.cancelling(m, n, CANCEL_K, rows, cols, CANCEL_E, seed=per_slice)
    _check_cancelling(g, rows, cols, "cancelling, %d per wave" % per_slice)


def test_cancelling_outputs_beyond_one_list():
    """40 cancelling rows and every column symmetric: more than 64 outputs
    of one wave to recompute, so the later lists take the out-of-line copy."""
    m, n = 72, 256
    rows, cols = list(range(8, 48)), list(range(n))
    g = workloads.cancelling(m, n, CANCEL_K, rows, cols, CANCEL_E, seed=3)
    _check_cancelling(g, rows, cols, "cancelling, 40 rows x all columns")


def test_handoff_timeouts_are_counted():
    """Forcing the waves' A hand-off waits to give up at once
    (NVFP4_SYNC_SPIN_LIMIT=0; the kernel still exits normally, only its sums
    may be wrong) is reported by nvfp4_stream_errors, which then reads zero
    again; a normal call afterwards reports nothing."""
    import os
    import torch
    import block_scaled_fp4_group_amd as nv
    from tests.gpu_util import device_args
    groups = workloads.generate(workloads.CONFIGS[3])
    log("gpu case: forced hand-off timeouts shapes=%s" % [(g.m, g.n, g.k) for g in groups])
    args = device_args(groups)
    sid = torch.cuda.current_stream().cuda_stream
    old = os.environ.get("NVFP4_SYNC_SPIN_LIMIT")
    os.environ["NVFP4_SYNC_SPIN_LIMIT"] = "0"
    try:
        nv.group_gemm(args)
    finally:
        if old is None:
            os.environ.pop("NVFP4_SYNC_SPIN_LIMIT", None)
        else:
            os.environ["NVFP4_SYNC_SPIN_LIMIT"] = old
    assert nv.stream_errors(sid) > 0
    assert nv.stream_errors(sid) == 0
    check_full(workloads.generate(workloads.CONFIGS[0]), "after forced timeouts")
