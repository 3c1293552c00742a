"""Seeded synthetic inputs for the NVFP4 grouped GEMM.

This module only *produces bytes*: packed E2M1 code bytes for A and B, and
E4M3FN scale bytes for SFA and SFB.  It holds none of the GEMM's arithmetic
(no decoding, no products, no sums, no rounding of results), so that both the
oracle and the GPU path can read identical inputs without sharing any code.

Workload shapes follow the five benchmark configurations of the NVFP4
grouped-GEMM task (the pages are submissions to that task; its own input
generator is not part of them).  Distributions:

* FP4 codes: every byte drawn uniformly from 0..255, i.e. both nibbles i.i.d.
  uniform over all 16 E2M1 codes (including -0, code 8).  Element k of a row
  lives in byte k//2; even k in the low nibble, odd k in the high nibble.
* Scales: value 2**e * (1 + m/8) with e uniform in [e_lo, e_hi] and m uniform
  in 0..7, encoded to the nearest E4M3FN byte (ties to even).  For e < -6 the
  value falls below the smallest normal E4M3FN number and the nearest
  encoding is a subnormal code.

Draw order for one workload, from a single ``numpy.random.default_rng(seed)``:
for each group in order: A bytes (row-major), B bytes, SFA exponents, SFA
mantissas, SFB exponents, SFB mantissas.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Sequence, Tuple

import numpy as np

__all__ = ["Group", "Workload", "CONFIGS", "make_workload", "encode_scale_e4m3fn",
           "generate", "cancelling", "config_flops", "config_bytes"]


@dataclass(frozen=True)
class Workload:
    name: str
    shapes: Tuple[Tuple[int, int, int], ...]   # (M, N, K) per group
    e_range: Tuple[int, int]                    # inclusive exponent range of the scales
    seed: int = 0


@dataclass
class Group:
    m: int
    n: int
    k: int
    a: np.ndarray    # uint8 [m, k//2]
    b: np.ndarray    # uint8 [n, k//2]
    sfa: np.ndarray  # uint8 [m, k//16]
    sfb: np.ndarray  # uint8 [n, k//16]


CONFIGS: List[Workload] = [
    Workload("nvfp4_gg_2x_small", ((64, 128, 256), (128, 256, 256)), (-4, 2)),
    Workload("nvfp4_gg_moe8_n4096_k7168",
             tuple((m, 4096, 7168) for m in (80, 176, 128, 72, 64, 248, 96, 160)), (-4, 2)),
    Workload("nvfp4_gg_moe8_n7168_k2048",
             tuple((m, 7168, 2048) for m in (40, 76, 168, 72, 164, 148, 196, 160)), (-4, 2)),
    Workload("nvfp4_gg_2x_m384_512_n3072_k4096", ((384, 3072, 4096), (512, 3072, 4096)), (-6, 3)),
    Workload("nvfp4_gg_ragged8",
             ((1, 8192, 7168), (17, 8192, 7168), (129, 4096, 2048), (255, 2048, 4096),
              (512, 1024, 256), (33, 6144, 1536), (300, 3072, 7168), (8, 512, 512)), (-8, 4)),
]


def encode_scale_e4m3fn(e: np.ndarray, m: np.ndarray) -> np.ndarray:
    """Nearest E4M3FN byte (ties to even) of the positive value 2**e * (1 + m/8).

    Integer-only encoding of an input value.  E4M3FN: 1 sign, 4 exponent
    (bias 7), 3 mantissa bits; the all-ones pattern S.1111.111 is NaN; the
    largest finite value is 448; subnormals are M * 2**-9.
    """
    e = np.asarray(e, dtype=np.int64)
    m = np.asarray(m, dtype=np.int64)
    if np.any((m < 0) | (m > 7)):
        raise ValueError("mantissa field out of range")
    if np.any(e > 8) or np.any((e == 8) & (m == 7)):
        raise ValueError("scale exceeds the largest finite E4M3FN value")
    out = np.empty(np.broadcast(e, m).shape, dtype=np.uint8)
    normal = e >= -6
    out[normal] = (((e[normal] + 7) << 3) | m[normal]).astype(np.uint8)
    # subnormal range: value = (8 + m) * 2**(e - 3) = q * 2**-9, q = (8 + m) / 2**shift
    sub = ~normal
    if np.any(sub):
        num = 8 + m[sub]
        shift = -(e[sub] + 6)              # >= 1
        q = num >> shift
        rem = num & ((np.int64(1) << shift) - 1)
        half = np.int64(1) << (shift - 1)
        up = (rem > half) | ((rem == half) & ((q & 1) == 1))
        q = q + up.astype(np.int64)
        # q == 8 is the smallest normal number 2**-6, whose byte is also 0x08
        out[sub] = q.astype(np.uint8)
    return out


def make_workload(shapes: Sequence[Tuple[int, int, int]], e_range=(-4, 2), seed: int = 0,
                  name: str = "custom") -> Workload:
    return Workload(name, tuple(tuple(int(x) for x in s) for s in shapes), tuple(e_range), seed)


def generate(w: Workload) -> List[Group]:
    """Draw every group's input bytes for workload ``w`` (see module docstring)."""
    rng = np.random.default_rng(w.seed)
    e_lo, e_hi = w.e_range
    groups = []
    for (m, n, k) in w.shapes:
        if k % 16:
            raise ValueError("K must be a multiple of 16 (one scale per 16 elements)")
        a = rng.integers(0, 256, size=(m, k // 2), dtype=np.uint8)
        b = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
        ea = rng.integers(e_lo, e_hi + 1, size=(m, k // 16))
        ma = rng.integers(0, 8, size=(m, k // 16))
        eb = rng.integers(e_lo, e_hi + 1, size=(n, k // 16))
        mb = rng.integers(0, 8, size=(n, k // 16))
        groups.append(Group(m, n, k, a, b, encode_scale_e4m3fn(ea, ma), encode_scale_e4m3fn(eb, mb)))
    return groups


def cancelling(m: int, n: int, k: int, rows, cols, e_range=(0, 3), seed: int = 0) -> Group:
    """One group whose outputs (r, c) for r in ``rows`` and c in ``cols`` are
    exactly zero while the rest are random (drawn as in ``generate``).

    For each listed row of A the second half of K repeats the first half
    with every code's sign bit flipped (byte XOR 0x88) and the same scales;
    for each listed column of B the second half repeats the first half
    unchanged.  The two halves of such an output's sum are then equal and
    opposite, whatever the values: large partial sums that cancel exactly.
    K must be a multiple of 32.
    """
    if k % 32:
        raise ValueError("K must be a multiple of 32")
    g = generate(make_workload([(m, n, k)], e_range, seed))[0]
    h, hs = k // 4, k // 32            # half of K in code bytes and in scale bytes
    a, b, sfa, sfb = g.a.copy(), g.b.copy(), g.sfa.copy(), g.sfb.copy()
    for r in rows:
        a[r, h:] = a[r, :h] ^ np.uint8(0x88)
        sfa[r, hs:] = sfa[r, :hs]
    for c in cols:
        b[c, h:] = b[c, :h]
        sfb[c, hs:] = sfb[c, :hs]
    return Group(m, n, k, a, b, sfa, sfb)


def config_flops(shapes) -> int:
    """2*M*N*K summed over groups (the benchmark's flop count)."""
    return sum(2 * m * n * k for (m, n, k) in shapes)


def config_bytes(shapes) -> int:
    """Algorithmic HBM bytes: FP4 codes and E4M3 scales of A and B read once,
    fp16 C written once."""
    return sum((m + n) * k // 2 + (m + n) * k // 16 + 2 * m * n for (m, n, k) in shapes)
