"""Pins of the oracle's GEMM against computations that do not reuse it:
exact rational brute force, an independent decode + numpy matmul, closed-form
single-term cases, and algebraic invariants of the definition."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.test_oracle_formats import load_e2m1_table

E2M1 = load_e2m1_table()                                           # OCP table (golden)
E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def independent_decode(codes, scales, k):
    """code*scale from the golden E2M1 table and torch's E4M3FN decoder."""
    tab = np.array([E2M1[c] for c in range(16)])
    vals = np.empty((codes.shape[0], k))
    vals[:, 0::2] = tab[codes & 15]
    vals[:, 1::2] = tab[codes >> 4]
    return vals * np.repeat(E4M3[scales], 16, axis=1)


def rand_group(rng, m, n, k, any_scale=True):
    a = rng.integers(0, 256, (m, k // 2), dtype=np.uint8)
    b = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    if any_scale:   # every finite E4M3FN code, both signs, subnormals included
        finite = np.array([x for x in range(256) if x not in (0x7F, 0xFF)], dtype=np.uint8)
        sfa = rng.choice(finite, (m, k // 16)).astype(np.uint8)
        sfb = rng.choice(finite, (n, k // 16)).astype(np.uint8)
    else:
        sfa = workloads.encode_scale_e4m3fn(rng.integers(-8, 5, (m, k // 16)), rng.integers(0, 8, (m, k // 16)))
        sfb = workloads.encode_scale_e4m3fn(rng.integers(-8, 5, (n, k // 16)), rng.integers(0, 8, (n, k // 16)))
    return workloads.Group(m, n, k, a, b, sfa, sfb)


def fraction_gemm(g):
    """Exact rational sum, element by element, nibble by nibble."""
    out = np.zeros((g.m, g.n), dtype=object)
    for i in range(g.m):
        for j in range(g.n):
            s = Fraction(0)
            for k in range(g.k):
                ca = (g.a[i, k // 2] >> (4 * (k % 2))) & 15
                cb = (g.b[j, k // 2] >> (4 * (k % 2))) & 15
                s += (Fraction(E2M1[ca]) * Fraction(float(E4M3[g.sfa[i, k // 16]]))
                      * Fraction(E2M1[cb]) * Fraction(float(E4M3[g.sfb[j, k // 16]])))
            out[i, j] = s
    return out


@pytest.mark.parametrize("ng", [1, 3])
@pytest.mark.parametrize("k", [16, 32, 48])
def test_bruteforce_fraction_tiny(oracle_lib, ng, k):
    rng = np.random.default_rng(1000 + 10 * ng + k)
    for _ in range(ng):
        m, n = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        g = rand_group(rng, m, n, k)
        c16, c64 = oracle.gemm_group(g.a, g.sfa, g.b, g.sfb, m, n, k)
        exact = fraction_gemm(g)
        for i in range(m):
            for j in range(n):
                assert Fraction(c64[i, j]) == exact[i, j]                  # fp64 sum is exact here
                with np.errstate(over="ignore"):
                    ref = np.float64(float(exact[i, j])).astype(np.float16).view(np.uint16)
                assert c16[i, j] == ref


def test_independent_decode_matmul_config0(oracle_lib):
    """Full config-0 workload: oracle == independent decode + numpy matmul
    (fp64 sums are exact for these value ranges)."""
    for g in workloads.generate(workloads.CONFIGS[0]):
        c16, c64 = oracle.gemm_group(g.a, g.sfa, g.b, g.sfb, g.m, g.n, g.k)
        ref = independent_decode(g.a, g.sfa, g.k) @ independent_decode(g.b, g.sfb, g.k).T
        assert np.array_equal(c64, ref)
        with np.errstate(over="ignore"):
            assert np.array_equal(c16, ref.astype(np.float16).view(np.uint16))


def test_independent_decode_matmul_ragged(oracle_lib):
    rng = np.random.default_rng(7)
    for (m, n, k) in [(5, 7, 64), (17, 3, 256), (1, 33, 1024)]:
        g = rand_group(rng, m, n, k, any_scale=False)
        _, c64 = oracle.gemm_group(g.a, g.sfa, g.b, g.sfb, m, n, k)
        ref = independent_decode(g.a, g.sfa, k) @ independent_decode(g.b, g.sfb, k).T
        assert np.array_equal(c64, ref)


def test_single_term_closed_form(oracle_lib):
    """One nonzero k: C = e2m1(a) * sa * e2m1(b) * sb, for every A code and
    every finite scale byte, in both nibble positions and scale blocks."""
    k = 64
    finite = [x for x in range(256) if x not in (0x7F, 0xFF)]
    for kk in (0, 1, 17, 63):                    # low/high nibble, first/other scale blocks
        m = 16 * len(finite)
        a = np.zeros((m, k // 2), np.uint8)
        sfa = np.zeros((m, k // 16), np.uint8)
        for row in range(m):
            code, sbyte = row % 16, finite[row // 16]
            a[row, kk // 2] = code << (4 * (kk % 2))
            sfa[row, kk // 16] = sbyte
        b = np.zeros((1, k // 2), np.uint8)
        b[0, kk // 2] = 3 << (4 * (kk % 2))       # 1.5
        sfb = np.full((1, k // 16), 0x40, np.uint8)  # 2.0
        c16, c64 = oracle.gemm_group(a, sfa, b, sfb, m, 1, k)
        expect = np.array([E2M1[r % 16] * E4M3[finite[r // 16]] * 3.0 for r in range(m)])
        assert np.array_equal(c64[:, 0], expect)


def test_invariants(oracle_lib):
    rng = np.random.default_rng(11)
    g = rand_group(rng, 9, 13, 128, any_scale=False)
    c16, c64 = oracle.gemm_group(g.a, g.sfa, g.b, g.sfb, g.m, g.n, g.k)
    # doubling every normal SFA scale (exponent field +1) doubles the exact sums
    E = (g.sfa >> 3) & 15
    sfa2 = g.sfa.copy()
    ok = (E >= 1) & (E <= 13)
    sfa2[ok] += 8
    sfa_half = g.sfa.copy()
    sfa_half[~ok] = 0x38                           # make every scale normal-doublable
    _, base = oracle.gemm_group(g.a, sfa_half, g.b, g.sfb, g.m, g.n, g.k)
    sfa_half2 = sfa_half.copy(); sfa_half2 += 8
    _, dbl = oracle.gemm_group(g.a, sfa_half2, g.b, g.sfb, g.m, g.n, g.k)
    assert np.array_equal(dbl, 2 * base)
    # swapping the roles of A and B transposes C
    _, ct = oracle.gemm_group(g.b, g.sfb, g.a, g.sfa, g.n, g.m, g.k)
    assert np.array_equal(ct, c64.T)
    # a row of zero codes gives a +0 row
    a0 = g.a.copy(); a0[3] = 0
    z16, z64 = oracle.gemm_group(a0, g.sfa, g.b, g.sfb, g.m, g.n, g.k)
    assert (z16[3] == 0).all() and (z64[3] == 0).all()
    assert np.array_equal(np.delete(z16, 3, 0), np.delete(c16, 3, 0))
    # additivity over a K split at a 16-aligned point (exact in fp64)
    kh = 64
    _, lo = oracle.gemm_group(g.a[:, :kh // 2], g.sfa[:, :kh // 16], g.b[:, :kh // 2], g.sfb[:, :kh // 16], g.m, g.n, kh)
    _, hi = oracle.gemm_group(g.a[:, kh // 2:], g.sfa[:, kh // 16:], g.b[:, kh // 2:], g.sfb[:, kh // 16:], g.m, g.n, g.k - kh)
    assert np.array_equal(lo + hi, c64)
    # splitting N into separate groups gives identical bits
    parts = [oracle.gemm_group(g.a, g.sfa, g.b[s], g.sfb[s], g.m, len(range(*s.indices(g.n))), g.k)[0]
             for s in (slice(0, 5), slice(5, 13))]
    assert np.array_equal(np.concatenate(parts, axis=1), c16)


def test_group_list_independence(oracle_lib):
    rng = np.random.default_rng(5)
    gs = [rand_group(rng, m, n, k, any_scale=False) for (m, n, k) in [(3, 4, 64), (5, 2, 128), (1, 7, 32)]]
    r16, r64 = oracle.group_gemm(gs)
    p16, p64 = oracle.group_gemm(gs[::-1])
    for x, y in zip(r16, p16[::-1]):
        assert np.array_equal(x, y)


def test_degenerate_shapes(oracle_lib):
    c16, c64 = oracle.gemm_group(np.zeros((3, 0), np.uint8), np.zeros((3, 0), np.uint8),
                                 np.zeros((2, 0), np.uint8), np.zeros((2, 0), np.uint8), 3, 2, 0)
    assert (c16 == 0).all() and (c64 == 0).all() and not np.signbit(c64).any()
    c16, c64 = oracle.gemm_group(np.zeros((0, 8), np.uint8), np.zeros((0, 1), np.uint8),
                                 np.zeros((2, 8), np.uint8), np.zeros((2, 1), np.uint8), 0, 2, 16)
    assert c16.shape == (0, 2)


def test_entries_match_full(oracle_lib):
    rng = np.random.default_rng(9)
    g = rand_group(rng, 20, 30, 256, any_scale=False)
    c16, c64 = oracle.gemm_group(g.a, g.sfa, g.b, g.sfb, g.m, g.n, g.k)
    rows = rng.integers(0, g.m, 50)
    cols = rng.integers(0, g.n, 50)
    e16, e64 = oracle.gemm_entries(g, rows, cols)
    assert np.array_equal(e16, c16[rows, cols]) and np.array_equal(e64, c64[rows, cols])


def test_exactness_bound_of_workloads():
    """fp64 accumulation is exact for every benchmark workload: all terms are
    multiples of 2^-20 and K * max|term| < 2^33 (53-bit significand)."""
    for w in workloads.CONFIGS:
        e_hi = w.e_range[1]
        max_scale = 2.0 ** e_hi * (1 + 7 / 8)
        for (m, n, k) in w.shapes:
            bound = k * (6 * max_scale) ** 2
            assert bound < 2.0 ** 33, (w.name, bound)
