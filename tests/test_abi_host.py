"""Host-side checks of the C ABI (no GPU needed): the library loads and
exports every entry point the header declares, argument validation returns
the documented codes, and the work plan covers every output exactly once."""
import os
import re

import numpy as np
import pytest

import block_scaled_fp4_group_amd as nv

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    names = set()
    inc = os.path.join(REPO, "include")
    for fn in os.listdir(inc):
        if fn.endswith(".h"):
            text = open(os.path.join(inc, fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(nvfp4_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    lib = nv.lib()
    names = header_functions()
    assert "nvfp4_group_gemm" in names and len(names) >= 5
    for name in names:
        assert hasattr(lib, name), name


# fake, suitably aligned device addresses: validation never dereferences them
A, B, SA, SB, C = 0x10000, 0x20000, 0x30000, 0x40000, 0x50000


def G(m, n, k, **kw):
    args = dict(a=A, b=B, sfa=SA, sfb=SB, c=C, m=m, n=n, k=k)
    args.update(kw)
    return nv.make_group(**args)


@pytest.mark.parametrize("groups,code", [
    ([G(4, 4, 64)], nv.NVFP4_OK),
    ([], nv.NVFP4_OK),
    ([G(-1, 4, 64)], nv.NVFP4_EINVAL),
    ([G(4, -1, 64)], nv.NVFP4_EINVAL),
    ([G(4, 4, -16)], nv.NVFP4_EINVAL),
    ([G(4, 4, 24)], nv.NVFP4_EINVAL),                   # k % 16 != 0
    ([G(4, 4, 64, c=0)], nv.NVFP4_EINVAL),
    ([G(4, 4, 64, a=0)], nv.NVFP4_EINVAL),
    ([G(4, 4, 64, sfb=0)], nv.NVFP4_EINVAL),
    ([G(4, 4, 64, flags=2)], nv.NVFP4_EINVAL),          # unknown flag
    ([G(4, 4, 64, flags=nv.NVFP4_SFB_SWIZZLED)], nv.NVFP4_OK),
    ([G(4, 4, 64, flags=nv.NVFP4_SFB_SWIZZLED, sfb=SB + 4)], nv.NVFP4_EUNSUPPORTED),  # window-major sfb: 16 B
    ([G(4, 4, 64, sfb=SB + 4)], nv.NVFP4_OK),           # plain sfb: 4 B is enough
    ([G(0, 4, 64, a=0, b=0, c=0)], nv.NVFP4_OK),          # empty group: pointers unused
    ([G(4, 0, 64, c=0)], nv.NVFP4_OK),
    ([G(4, 4, 0, a=0, b=0, sfa=0, sfb=0)], nv.NVFP4_OK),  # k == 0 writes zeros
    ([G(4, 4, 48)], nv.NVFP4_EUNSUPPORTED),             # k % 64 != 0
    ([G(4, 4, 64, a=A + 8)], nv.NVFP4_EUNSUPPORTED),    # misaligned codes
    ([G(4, 4, 64, sfa=SA + 2)], nv.NVFP4_EUNSUPPORTED), # misaligned scales
    ([G(4, 4, 64, c=C + 2)], nv.NVFP4_EUNSUPPORTED),
    ([G(4, 4, 64), G(4, 4, 24)], nv.NVFP4_EINVAL),      # error in a later group
])
def test_validate_codes(groups, code):
    rc, msg = nv.validate(groups)
    assert rc == code, msg
    if code:
        assert msg


def test_validate_negative_ng_and_null():
    lib = nv.lib()
    assert lib.nvfp4_validate(None, -1) == nv.NVFP4_EINVAL
    assert lib.nvfp4_validate(None, 2) == nv.NVFP4_EINVAL
    assert lib.nvfp4_validate(None, 0) == nv.NVFP4_OK
    assert lib.nvfp4_group_gemm(None, -3, None) == nv.NVFP4_EINVAL   # rejected before any HIP call
    assert b"negative" in lib.nvfp4_last_error()


def test_group_gemm_rejects_before_launch():
    with pytest.raises(nv.Nvfp4Error) as ei:
        nv.group_gemm_raw([G(4, 4, 24)])
    assert ei.value.code == nv.NVFP4_EINVAL


SHAPES = [
    [(64, 128, 256), (128, 256, 256)],
    [(m, 4096, 7168) for m in (80, 176, 128, 72, 64, 248, 96, 160)],
    [(1, 8192, 7168), (17, 8192, 7168), (129, 4096, 2048), (255, 2048, 4096),
     (512, 1024, 256), (33, 6144, 1536), (300, 3072, 7168), (8, 512, 512)],
    [(0, 5, 64), (3, 0, 64), (1, 1, 64), (65, 129, 64), (7, 3, 0)],
    [(16, 16, 64)] * 40,                                  # more groups than one launch holds
]


def _tile_key(seg):
    return seg[1], seg[2], seg[4]


@pytest.mark.parametrize("num_wg", [256, 1, 7, 100000])
@pytest.mark.parametrize("shapes", SHAPES)
def test_plan_covers_every_output_once(shapes, num_wg):
    """Every output element is written by exactly one segment (role 0 or 2),
    every tile's k range is covered exactly once by its segments, and the
    hand-off of partial sums cannot deadlock: each producer (role 1) is the
    first segment of its workgroup, whose index is above its finalizer's."""
    groups = [G(m, n, k) for (m, n, k) in shapes]
    segs = nv.plan(groups, num_wg)
    TR, TC = nv.tile_rows(), nv.tile_cols()
    cover = [np.zeros((m, n), np.int32) for (m, n, k) in shapes]
    by_tile = {}
    first_of_wg = {}
    for i, seg in enumerate(segs):
        wg, g, m0, rows, n0, kb, ke, role = seg
        m, n, k = shapes[g]
        assert 0 <= wg < num_wg
        assert 0 < rows <= TR and 0 <= m0 and m0 + rows <= m and 0 <= n0 < n and n0 % TC == 0
        kpad = 256 * max(1, -(-k // 256))      # k padded to whole 256-k stage pairs
        assert 0 <= kb < ke <= kpad and kb % 256 == 0 and ke % 256 == 0
        first_of_wg.setdefault(wg, i)
        by_tile.setdefault(_tile_key(seg), []).append(seg)
        if role in (0, 2):
            cover[g][m0:m0 + rows, n0:min(n, n0 + TC)] += 1
            assert kb == 0
        else:
            assert role == 1 and kb > 0 and first_of_wg[wg] == i
    for (m, n, k), cv in zip(shapes, cover):
        assert (cv == 1).all()
    for key, parts in by_tile.items():
        parts.sort(key=lambda s: s[5])
        assert parts[0][5] == 0 and all(a[6] == b[5] for a, b in zip(parts, parts[1:]))
        k = shapes[key[0]][2]
        assert parts[-1][6] == 256 * max(1, -(-k // 256))
        head = parts[0]
        assert head[7] == (0 if len(parts) == 1 else 2)
        assert all(p[0] > head[0] for p in parts[1:])
        # one segment per workgroup and tile
        assert len({p[0] for p in parts}) == len(parts)


PAIR_CLK = [0, 4212, 4634, 4648, 4880, 5305, 5622, 6141, 6988]


def test_plan_balances_work():
    """The partition balances the workgroups' modelled times.  The model,
    in clocks: start-up 3500; a fill of 5850 for a workgroup's first
    segment and 9400 for each later one; per pair 4212, 4634, 4648, 4880,
    5305, 5622, 6141, 6988 for 1..8 row blocks of 16; after a segment 7900
    to publish a part of a split tile, or 7200 to store a tile plus 6000
    per other part to sum.  At least 95% of the
    compute units get work (the greedy fill may leave a few idle when whole
    tiles pack better), and the slowest is within 12% of the mean of those
    with work."""
    from collections import defaultdict
    for shapes in ([(m, 4096, 7168) for m in (80, 176, 128, 72, 64, 248, 96, 160)],
                   [(1, 8192, 7168), (17, 8192, 7168), (129, 4096, 2048), (255, 2048, 4096),
                    (512, 1024, 256), (33, 6144, 1536), (300, 3072, 7168), (8, 512, 512)]):
        segs = nv.plan([G(*s) for s in shapes], 256)
        by_wg = defaultdict(list)
        parts = defaultdict(int)
        for seg in segs:
            by_wg[seg[0]].append(seg)
            parts[_tile_key(seg)] += 1
        t = np.zeros(256)
        for wg, own in by_wg.items():
            x = 3500.0
            for i, (_, g, m0, rows, n0, kb, ke, role) in enumerate(own):
                x += (5850 if i == 0 else 9400) + (ke - kb) // 256 * PAIR_CLK[-(-rows // 16)]
                x += 7900 if role == 1 else 7200 + 6000 * (parts[_tile_key(own[i])] - 1)
            t[wg] = x
        assert (t > 0).mean() >= 0.95
        assert t.max() <= 1.12 * t[t > 0].mean()


def test_plan_leaves_finalizers_their_tail():
    """Under the same model, the last part of every split tile is published
    early enough that the finalizer's sum of it (6000) and its store (7200)
    still end within the makespan: a last part that ran up to the makespan
    would make its finalizer the slowest workgroup."""
    from collections import defaultdict
    for shapes in ([(m, 4096, 7168) for m in (80, 176, 128, 72, 64, 248, 96, 160)],
                   [(384, 3072, 4096), (512, 3072, 4096)],
                   [(1, 8192, 7168), (17, 8192, 7168), (129, 4096, 2048), (255, 2048, 4096),
                    (512, 1024, 256), (33, 6144, 1536), (300, 3072, 7168), (8, 512, 512)]):
        segs = nv.plan([G(*s) for s in shapes], 256)
        by_wg = defaultdict(list)
        parts = defaultdict(int)
        for seg in segs:
            by_wg[seg[0]].append(seg)
            parts[_tile_key(seg)] += 1
        end, last_publish = {}, []
        for wg, own in by_wg.items():
            x = 3500.0
            for i, (_, g, m0, rows, n0, kb, ke, role) in enumerate(own):
                x += (5850 if i == 0 else 9400) + (ke - kb) // 256 * PAIR_CLK[-(-rows // 16)]
                x += 7900 if role == 1 else 7200 + 6000 * (parts[_tile_key(own[i])] - 1)
                if role == 1 and ke == shapes[g][2]:
                    last_publish.append(x)
            end[wg] = x
        makespan = max(end.values())
        assert last_publish, "no split tiles: the case tests nothing"
        assert max(last_publish) + 6000 + 7200 <= makespan * 1.001


def test_plan_rejects_invalid():
    with pytest.raises(nv.Nvfp4Error):
        nv.plan([G(4, 4, 24)])

def test_plan_cache_keys_on_sizes():
    """The host keeps the last partition per thread; a plan for other sizes
    or another unit count in between must not leak into the next one."""
    a = [(m, 4096, 7168) for m in (80, 176, 128, 72, 64, 248, 96, 160)]
    b = [(1, 8192, 7168), (17, 8192, 7168), (129, 4096, 2048), (255, 2048, 4096)]
    c = [(m, 4096, 7168) for m in (80, 176, 128, 72, 64, 248, 96, 161)]   # one size differs
    first = nv.plan([G(*s) for s in a], 256)
    other = nv.plan([G(*s) for s in b], 256)
    again = nv.plan([G(*s) for s in a], 256)
    assert first == again and first != other
    fewer = nv.plan([G(*s) for s in a], 200)
    assert max(seg[0] for seg in fewer) < 200
    assert nv.plan([G(*s) for s in a], 256) == first
    near = nv.plan([G(*s) for s in c], 256)
    assert near != first
    assert nv.plan([G(*s) for s in c], 256) == near

@pytest.mark.parametrize("seed", range(24))
def test_plan_random_shapes(seed):
    """Random launches: every output element is written once, each tile's k
    range is covered once in order, a split tile has exactly one finalizer
    (its first part), and no workgroup runs a producer part after a
    finalizer part (so no finalizer can wait on a waiting workgroup)."""
    rng = np.random.default_rng(1000 + seed)
    ng = int(rng.integers(1, 13))
    shapes = [(int(rng.integers(0, 400)), int(rng.integers(0, 3000)), 64 * int(rng.integers(0, 120)))
              for _ in range(ng)]
    for num_wg in (1, 7, 64, 256):
        segs = nv.plan([G(*s) for s in shapes], num_wg)
        cover = [np.zeros((m, n), np.int8) for (m, n, k) in shapes]
        by_tile, by_wg = {}, {}
        for seg in segs:
            wg, g, m0, rows, n0, kb, ke, role = seg
            assert 0 <= wg < num_wg and 0 < rows and kb < ke
            by_tile.setdefault(_tile_key(seg), []).append(seg)
            by_wg.setdefault(wg, []).append(role)
            if role in (0, 2):
                cover[g][m0:m0 + rows, n0:n0 + 256] += 1
        for (m, n, k), cv in zip(shapes, cover):
            assert (cv == 1).all()
        for key, parts in by_tile.items():
            parts.sort(key=lambda q: q[5])
            k = shapes[key[0]][2]
            assert parts[0][5] == 0 and parts[-1][6] == 256 * max(1, -(-k // 256))
            assert all(a[6] == b[5] for a, b in zip(parts, parts[1:]))
            assert [q[7] for q in parts] == ([0] if len(parts) == 1 else [2] + [1] * (len(parts) - 1))
        for roles in by_wg.values():
            if 2 in roles:
                assert 1 not in roles[roles.index(2):]


def test_swizzled_scale_bytes():
    """ceil(rows / 32) * 32 rows of ceil(k / 256) windows of 16 bytes."""
    assert nv.swizzled_scale_bytes(1, 16) == 32 * 1 * 16
    assert nv.swizzled_scale_bytes(32, 256) == 32 * 1 * 16
    assert nv.swizzled_scale_bytes(33, 257 - 1 + 16) == 64 * 2 * 16
    assert nv.swizzled_scale_bytes(4096, 7168) == 4096 * 28 * 16
    assert nv.swizzled_scale_bytes(0, 64) == 0 and nv.swizzled_scale_bytes(8, 0) == 0


def test_swizzle_scales_rejects_before_launch():
    lib = nv.lib()
    assert lib.nvfp4_swizzle_scales(None, None, -1, 64, None) == nv.NVFP4_EINVAL
    assert lib.nvfp4_swizzle_scales(None, None, 4, 24, None) == nv.NVFP4_EINVAL
    assert lib.nvfp4_swizzle_scales(None, None, 4, 64, None) == nv.NVFP4_EINVAL
    assert lib.nvfp4_swizzle_scales(None, None, 0, 64, None) == nv.NVFP4_OK       # nothing to do
    assert lib.nvfp4_swizzle_scales(0x10000, 0x20008, 4, 64, None) == nv.NVFP4_EUNSUPPORTED
