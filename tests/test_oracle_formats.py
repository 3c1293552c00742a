"""Pins of the oracle's number formats against sources other than itself:
the OCP E2M1 value table, torch's float8_e4m3fn decoder, numpy's float16
rounding, and the format facts (maxima, NaN codes, subnormal quantum)."""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_e2m1_table():
    vals = {}
    with open(os.path.join(GOLDEN, "e2m1_values.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            vals[int(c)] = float(v)
    assert sorted(vals) == list(range(16))
    return vals


def test_e2m1_matches_ocp_table(oracle_lib):
    table = load_e2m1_table()
    for code in range(16):
        got = oracle.e2m1_value(code)
        assert got == table[code], code
        assert math.copysign(1.0, got) == math.copysign(1.0, table[code]), code  # -0 for code 8


def test_e2m1_structure(oracle_lib):
    vals = [oracle.e2m1_value(c) for c in range(16)]
    assert vals[8] == 0.0 and math.copysign(1, vals[8]) < 0          # code 8 is -0
    assert all(vals[c + 8] == -vals[c] for c in range(8))             # sign bit is bit 3
    assert all(vals[c] < vals[c + 1] for c in range(7))               # monotone magnitudes
    assert max(vals) == 6.0 and min(v for v in vals if v > 0) == 0.5


def test_e4m3fn_matches_torch_all_codes(oracle_lib):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3fn_value(b) for b in range(256)])
    nan_ref, nan_got = np.isnan(ref), np.isnan(got)
    assert (nan_ref == nan_got).all()
    assert np.array_equal(got[~nan_got], ref[~nan_ref])
    assert np.array_equal(np.signbit(got[~nan_got]), np.signbit(ref[~nan_ref]))


def test_e4m3fn_format_facts(oracle_lib):
    vals = [oracle.e4m3fn_value(b) for b in range(256)]
    finite = [v for v in vals if not math.isnan(v)]
    assert len(finite) == 254
    assert [b for b in range(256) if math.isnan(vals[b])] == [0x7F, 0xFF]
    assert max(finite) == 448.0 and min(finite) == -448.0
    assert min(v for v in finite if v > 0) == 2.0 ** -9                 # smallest subnormal
    assert vals[0x08] == 2.0 ** -6                                      # smallest normal
    assert vals[0x38] == 1.0 and vals[0xB8] == -1.0
    assert not any(math.isinf(v) for v in vals)                         # "FN": no infinities


EDGE_F16 = [0.0, -0.0, 1.0, -1.0, 65504.0, 65519.99, 65520.0, -65520.0, 65536.0, 1e30, -1e30,
            2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.0000001, 3 * 2.0 ** -26, 2.0 ** -14,
            2.0 ** -14 - 2.0 ** -25, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 2049.0, 2051.0,
            4097.0, 6.103515625e-05, 5.960464477539063e-08, 0.1, 1.0 / 3.0]


def test_fp16_rne_matches_numpy(oracle_lib):
    rng = np.random.default_rng(123)
    xs = list(EDGE_F16)
    xs += list(rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 6, 20000))
    # exact ties at several binades, both parities
    for e in range(-24, 16):
        for mant in (1025, 1026, 1535, 2047):
            xs.append((mant + 0.5) * 2.0 ** (e - 10))
    with np.errstate(over="ignore"):
        ref = np.array(xs, dtype=np.float64).astype(np.float16).view(np.uint16)
    got = np.array([oracle.fp16_rne(x) for x in xs], dtype=np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(xs[i], hex(got[i]), hex(ref[i])) for i in bad[:5]]


def test_fp16_rne_specials(oracle_lib):
    assert oracle.fp16_rne(65504.0) == 0x7BFF
    assert oracle.fp16_rne(65519.99) == 0x7BFF
    assert oracle.fp16_rne(65520.0) == 0x7C00          # tie goes to the even neighbour: inf
    assert oracle.fp16_rne(-1e9) == 0xFC00
    assert oracle.fp16_rne(2.0 ** -25) == 0x0000        # tie between 0 and 2^-24 -> even (0)
    assert oracle.fp16_rne(3 * 2.0 ** -25) == 0x0002    # tie between 1 and 2 quanta -> 2
    assert oracle.fp16_rne(float("nan")) & 0x7C00 == 0x7C00


def test_input_scale_encoding_matches_torch():
    """The generator's integer E4M3FN encoder agrees with torch's RNE cast."""
    e = np.repeat(np.arange(-9, 9), 8)
    m = np.tile(np.arange(8), 18)
    keep = ~((e == 8) & (m == 7))
    e, m = e[keep], m[keep]
    mine = workloads.encode_scale_e4m3fn(e, m)
    ref = torch.tensor(2.0 ** e * (1 + m / 8), dtype=torch.float64).to(torch.float8_e4m3fn)
    assert np.array_equal(mine, ref.view(torch.uint8).numpy())


def test_workload_shapes_and_distribution():
    w = workloads.CONFIGS[4]
    gs = workloads.generate(w)
    assert [(g.m, g.n, g.k) for g in gs] == list(w.shapes)
    for g in gs:
        assert g.a.shape == (g.m, g.k // 2) and g.b.shape == (g.n, g.k // 2)
        assert g.sfa.shape == (g.m, g.k // 16) and g.sfb.shape == (g.n, g.k // 16)
    big = gs[0].b
    lo, hi = big & 15, big >> 4
    for nib in (lo, hi):
        counts = np.bincount(nib.ravel(), minlength=16) / nib.size
        assert np.all(np.abs(counts - 1 / 16) < 0.002)
    # config-4 scales reach subnormal E4M3FN codes (e = -8, -7)
    assert (gs[0].sfb < 8).any()
    # generation is deterministic
    again = workloads.generate(w)
    assert all(np.array_equal(x.b, y.b) and np.array_equal(x.sfa, y.sfa) for x, y in zip(gs, again))
