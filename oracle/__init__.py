"""Python access to the CPU oracle (``nvfp4_oracle.c``) through ctypes.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product package.  It shares no
code with the HIP library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import List, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_LIB = os.path.join(_HERE, "libnvfp4_oracle.so")
_lib = None

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_i32p = ctypes.POINTER(ctypes.c_int32)
_f64p = ctypes.POINTER(ctypes.c_double)


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (IEEE semantics: no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        L.oracle_e2m1_value.restype = ctypes.c_double
        L.oracle_e2m1_value.argtypes = [ctypes.c_uint]
        L.oracle_e4m3fn_value.restype = ctypes.c_double
        L.oracle_e4m3fn_value.argtypes = [ctypes.c_uint]
        L.oracle_fp16_rne.restype = ctypes.c_uint16
        L.oracle_fp16_rne.argtypes = [ctypes.c_double]
        L.oracle_dot.restype = ctypes.c_double
        L.oracle_dot.argtypes = [_u8p, _u8p, _u8p, _u8p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]
        L.oracle_gemm_group.restype = ctypes.c_int
        L.oracle_gemm_group.argtypes = [_u8p, _u8p, _u8p, _u8p, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_int64, _u16p, _f64p, ctypes.c_int]
        L.oracle_gemm_entries.restype = None
        L.oracle_gemm_entries.argtypes = [_u8p, _u8p, _u8p, _u8p, ctypes.c_int64, _i32p, _i32p,
                                          ctypes.c_int64, _u16p, _f64p, ctypes.c_int]
        L.oracle_max_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(arr, ptype):
    return arr.ctypes.data_as(ptype)


def _u8(arr) -> np.ndarray:
    arr = np.ascontiguousarray(arr, dtype=np.uint8)
    if arr.size == 0:                  # keep a valid pointer for empty inputs
        arr = np.zeros(1, np.uint8)
    return arr


def e2m1_value(code: int) -> float:
    return lib().oracle_e2m1_value(code)


def e4m3fn_value(byte: int) -> float:
    return lib().oracle_e4m3fn_value(byte)


def fp16_rne(x: float) -> int:
    return int(lib().oracle_fp16_rne(float(x)))


def gemm_group(a, sfa, b, sfb, m: int, n: int, k: int, nthreads: int = 0):
    """Returns (c16 bits uint16 [m, n], c64 float64 [m, n]) for one group."""
    c16 = np.zeros((m, n), dtype=np.uint16)
    c64 = np.zeros((m, n), dtype=np.float64)
    if m == 0 or n == 0:
        return c16, c64
    a, sfa, b, sfb = _u8(a), _u8(sfa), _u8(b), _u8(sfb)
    rc = lib().oracle_gemm_group(_p(a, _u8p), _p(sfa, _u8p), _p(b, _u8p), _p(sfb, _u8p),
                                 m, n, k, _p(c16, _u16p), _p(c64, _f64p), nthreads)
    if rc != 0:
        raise MemoryError("oracle_gemm_group failed to allocate")
    return c16, c64


def group_gemm(groups: Sequence, nthreads: int = 0):
    """Oracle over a list of groups (objects with m, n, k, a, b, sfa, sfb).
    Returns lists of (c16 bits, c64)."""
    out16: List[np.ndarray] = []
    out64: List[np.ndarray] = []
    for g in groups:
        c16, c64 = gemm_group(g.a, g.sfa, g.b, g.sfb, g.m, g.n, g.k, nthreads)
        out16.append(c16)
        out64.append(c64)
    return out16, out64


def gemm_entries(g, rows, cols, nthreads: int = 0):
    """Oracle values of selected outputs (rows[i], cols[i]) of one group."""
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    cols = np.ascontiguousarray(cols, dtype=np.int32)
    n = rows.size
    out16 = np.zeros(n, dtype=np.uint16)
    out64 = np.zeros(n, dtype=np.float64)
    if n == 0:
        return out16, out64
    if rows.min() < 0 or rows.max() >= g.m or cols.min() < 0 or cols.max() >= g.n:
        raise IndexError("sample index outside the group's output")
    a, sfa, b, sfb = _u8(g.a), _u8(g.sfa), _u8(g.b), _u8(g.sfb)
    lib().oracle_gemm_entries(_p(a, _u8p), _p(sfa, _u8p), _p(b, _u8p), _p(sfb, _u8p), g.k,
                              _p(rows, _i32p), _p(cols, _i32p), n, _p(out16, _u16p),
                              _p(out64, _f64p), nthreads)
    return out16, out64


def max_threads() -> int:
    return int(lib().oracle_max_threads())
