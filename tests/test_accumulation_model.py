"""The accumulation reading behind the kernel's accuracy fix-up, reproduced
from numpy alone (no GPU, no oracle code).

The kernel sums products in the matrix core.  Measured on gfx950 with
crafted inputs, an f16 MFMA step sums each lane's 8 products exactly and adds
that sum to the fp32 accumulator with one round-to-nearest-even.  The kernel
restarts those sums every 512 k and adds them into a separate fp32 total.
This file simulates exactly that rounding on real benchmark data (column
ranges of the workload groups, chosen to include the outputs where plain fp32
summation goes wrong) against the exact fp64 sum, and checks what the kernel
relies on:

1. plain fp32 summation (this model, no fix-up) leaves outputs outside the
   tolerance |d| <= 2e-3 |ref| + 1e-2 on the wide-scale workload, so a fix-up
   is needed at all;
2. per wave slice (a row tile x 32 columns) the error scale
   sigma = 2^-24 rms(C) sqrt(min(F, K)/16 + K/(2F)) bounds the error of every
   output that is small next to rms(C) with room to spare below the
   kernel's margin (kSigmaMargin, read from the kernel source);
3. with the kernel's rule -- outputs whose computed value c has
   2e-3 |c| + 1e-2 < margin * sigma are recomputed exactly -- every output is
   within tolerance.
"""
from __future__ import annotations

import os
import re

import numpy as np
import pytest

import workloads

FOLD_K = 512            # k between restarts of the MFMA sums
WAVE_COLS = 32          # columns of one wave slice
TILE_ROWS = 128         # most rows of one tile (rows spread evenly, rounded up to 16)
KERNEL = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "block_scaled_fp4_group_amd", "csrc", "nvfp4_group_gemm.hip")


def kernel_margin():
    m = re.search(r"constexpr float kSigmaMargin = ([0-9.]+)f;", open(KERNEL).read())
    assert m, "kSigmaMargin not found in the kernel source"
    return float(m.group(1))


def e2m1(c):
    # OCP MX E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit; e = 0 is subnormal
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, e.astype(np.int64) - 1))
    return np.where(s == 1, -mag, mag)


def e4m3fn(b):
    # E4M3FN: bias 7, subnormals at E = 0 (no infinities; the NaN codes are not used here)
    s = (b >> 7) & 1
    E = (b >> 3) & 15
    M = b & 7
    mag = np.where(E == 0, np.ldexp(M / 8.0, -6), np.ldexp(1.0 + M / 8.0, E.astype(np.int64) - 7))
    return np.where(s == 1, -mag, mag)


def decode(codes, scales, k):
    v = np.empty((codes.shape[0], k))
    v[:, 0::2] = e2m1(codes & 15)
    v[:, 1::2] = e2m1(codes >> 4)
    return v * np.repeat(e4m3fn(scales), 16, axis=1)


def hw_model_sum(A, B, fold=FOLD_K):
    """fp32 sums as the kernel forms them: exact 8-product groups added to an
    fp32 accumulator (RNE), the accumulator added into an fp32 total every
    `fold` k and at the end."""
    K = A.shape[1]
    acc = np.zeros((A.shape[0], B.shape[0]), np.float32)
    total = np.zeros_like(acc)
    for k in range(0, K, 8):
        acc = (acc.astype(np.float64) + A[:, k:k + 8] @ B[:, k:k + 8].T).astype(np.float32)
        if (k + 8) % fold == 0 or k + 8 == K:
            total = (total.astype(np.float64) + acc).astype(np.float32)
            acc[:] = 0
    return total.astype(np.float64)


def row_tiles(m):
    tiles = -(-m // TILE_ROWS)
    rows = 16 * -(-(-(-m // tiles)) // 16)
    return [(r0, min(m, r0 + rows)) for r0 in range(0, m, rows)]


# (workload, group, first column, last column): column ranges of whole wave
# slices; the first two hold the outputs where plain fp32 summation fails
CASES = [(4, 6, 1248, 1376), (4, 1, 5600, 5632), (4, 2, 0, 256), (3, 1, 0, 64), (1, 5, 0, 64)]


@pytest.fixture(scope="module")
def simulated():
    out = []
    gen = {}
    for cfg, gi, c0, c1 in CASES:
        if cfg not in gen:
            gen[cfg] = workloads.generate(workloads.CONFIGS[cfg])
        g = gen[cfg][gi]
        A = decode(g.a, g.sfa, g.k)
        B = decode(g.b[c0:c1], g.sfb[c0:c1], g.k)
        exact = A @ B.T
        approx = hw_model_sum(A, B)
        out.append((cfg, gi, c0, g.k, exact, approx))
    return out


def slices(m, ncols):
    for r0, r1 in row_tiles(m):
        for cs in range(0, ncols, WAVE_COLS):
            yield r0, r1, cs, cs + WAVE_COLS


def sigma_of(vals, K):
    rms = np.sqrt(np.mean(vals.astype(np.float64) ** 2))
    return 2.0 ** -24 * rms * np.sqrt(min(FOLD_K, K) / 16.0 + K / (2.0 * FOLD_K))


def test_plain_fp32_sums_break_the_tolerance(simulated):
    bad = 0
    for cfg, gi, c0, K, exact, approx in simulated:
        tol = 2e-3 * np.abs(exact) + 1e-2
        bad += int((np.abs(approx - exact) > tol).sum())
    assert bad >= 2, "the wide-scale workload should hold outputs fp32 summation gets wrong"


def test_sigma_bounds_small_outputs_with_room(simulated):
    margin = kernel_margin()
    worst = 0.0
    for cfg, gi, c0, K, exact, approx in simulated:
        for r0, r1, s0, s1 in slices(exact.shape[0], exact.shape[1]):
            e, a = exact[r0:r1, s0:s1], approx[r0:r1, s0:s1]
            sig = sigma_of(a, K)
            small = np.abs(e) < 0.05 * np.sqrt(np.mean(a ** 2))
            if small.any():
                worst = max(worst, float((np.abs(a - e)[small] / sig).max()))
    assert 0.0 < worst < 0.8 * margin, worst


def test_fixup_rule_leaves_every_output_in_tolerance(simulated):
    margin = kernel_margin()
    recomputed = 0
    for cfg, gi, c0, K, exact, approx in simulated:
        fixed = approx.copy()
        for r0, r1, s0, s1 in slices(exact.shape[0], exact.shape[1]):
            a = approx[r0:r1, s0:s1]
            thresh = (margin * sigma_of(a, K) - 1e-2) / 2e-3
            flag = np.abs(a) < thresh
            recomputed += int(flag.sum())
            fixed[r0:r1, s0:s1] = np.where(flag, exact[r0:r1, s0:s1], a)
        tol = 2e-3 * np.abs(exact) + 1e-2
        assert (np.abs(fixed - exact) <= tol).all(), (cfg, gi, c0)
    assert recomputed > 0
