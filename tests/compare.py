"""Comparison of GPU fp16 outputs with the oracle.

Tolerance of the benchmark spec: |gpu - ref| <= 2e-3 * |ref| + 1e-2, where
ref is the oracle's correctly rounded fp16.  Readings for the cases the
statement leaves open:
  * both infinite with the same sign: pass;
  * exactly one infinite: pass only when the exact sum lies in the overflow
    band |x| >= 65504 * (1 - 2e-3), where fp32 accumulation may legitimately
    land on either side of the fp16 overflow threshold;
  * any NaN: fail;
  * +0 and -0 are equal.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Tuple

import numpy as np

RTOL = 2e-3
ATOL = 1e-2
FP16_MAX = 65504.0


@dataclass
class Report:
    count: int
    failures: int
    worst_ratio: float
    examples: List[Tuple[int, float, float, float]] = field(default_factory=list)

    def __str__(self):
        return ("%d/%d outside tolerance, worst |d|/tol = %.3g, first: %s"
                % (self.failures, self.count, self.worst_ratio, self.examples[:5]))


def _f16(bits: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def compare_fp16(got_bits, ref_bits, ref_exact, rtol=RTOL, atol=ATOL) -> Report:
    g = _f16(got_bits).ravel()
    r = _f16(ref_bits).ravel()
    x = np.asarray(ref_exact, dtype=np.float64).ravel()
    if not (g.size == r.size == x.size):
        raise ValueError("size mismatch")
    nan = np.isnan(g) | np.isnan(r)
    ginf, rinf = np.isinf(g), np.isinf(r)
    both_inf = ginf & rinf & (np.sign(g) == np.sign(r))
    fin = ~(ginf | rinf | nan)
    tol = rtol * np.abs(r) + atol
    d = np.zeros_like(g)
    d[fin] = np.abs(g[fin] - r[fin])
    ok_fin = fin & (d <= tol)
    one_inf = (ginf ^ rinf) & ~nan & (np.abs(x) >= FP16_MAX * (1.0 - rtol))
    ok = (ok_fin | both_inf | one_inf) & ~nan
    bad = np.nonzero(~ok)[0]
    ratio = np.where(fin, d / tol, 0.0)
    worst = float(ratio.max()) if ratio.size else 0.0
    ex = [(int(i), float(g[i]), float(r[i]), float(x[i])) for i in bad[:8]]
    return Report(int(g.size), int(bad.size), worst, ex)


def bits_equal(got_bits, ref_bits) -> Tuple[int, List[int]]:
    """Number of elements whose fp16 bits differ, +0/-0 treated as equal."""
    g = np.ascontiguousarray(got_bits, dtype=np.uint16).ravel()
    r = np.ascontiguousarray(ref_bits, dtype=np.uint16).ravel()
    zero = ((g & 0x7FFF) == 0) & ((r & 0x7FFF) == 0)
    diff = np.nonzero((g != r) & ~zero)[0]
    return int(diff.size), [int(i) for i in diff[:8]]
