"""MI355X (gfx950) NVFP4 grouped GEMM -- Python binding of the C ABI in
include/nvfp4_group_gemm.h.

Argument marshalling only: every step of the computation runs in the HIP
kernels of libnvfp4gg.so.  PyTorch supplies device memory and the stream.
There is no fallback: if the library is missing, calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Iterable, List, Sequence, Tuple

__all__ = ["NVFP4_OK", "NVFP4_EINVAL", "NVFP4_EUNSUPPORTED", "NVFP4_EHIP", "NVFP4_SFB_SWIZZLED", "Nvfp4Error",
           "Nvfp4Group", "lib", "library_path", "group_gemm", "group_gemm_raw", "group_gemm_noalloc_raw",
           "validate", "swizzled_scale_bytes", "swizzle_scales",
           "plan", "release_workspace", "stream_errors", "tile_rows", "tile_cols", "make_group"]

NVFP4_OK, NVFP4_EINVAL, NVFP4_EUNSUPPORTED, NVFP4_EHIP = 0, 1, 2, 3
NVFP4_SFB_SWIZZLED = 1

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_PKG_DIR, "libnvfp4gg.so")
_lib = None


class Nvfp4Error(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__("nvfp4_group_gemm error %d: %s" % (code, message))
        self.code = code


class Nvfp4Group(ctypes.Structure):
    """Mirror of nvfp4_group_t."""
    _fields_ = [("a", ctypes.c_void_p), ("b", ctypes.c_void_p), ("sfa", ctypes.c_void_p),
                ("sfb", ctypes.c_void_p), ("c", ctypes.c_void_p), ("m", ctypes.c_int32),
                ("n", ctypes.c_int32), ("k", ctypes.c_int32), ("flags", ctypes.c_int32)]


def lib():
    """Load libnvfp4gg.so (built by __graft_entry__.build() or _build.py)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise RuntimeError("libnvfp4gg.so is not built (%s); run "
                               "`python -c 'import __graft_entry__ as g; g.build()'`" % library_path)
        L = ctypes.CDLL(library_path)
        gp = ctypes.POINTER(Nvfp4Group)
        L.nvfp4_group_gemm.restype = ctypes.c_int
        L.nvfp4_group_gemm.argtypes = [gp, ctypes.c_int, ctypes.c_void_p]
        L.nvfp4_group_gemm_noalloc.restype = ctypes.c_int
        L.nvfp4_group_gemm_noalloc.argtypes = [gp, ctypes.c_int, ctypes.c_void_p]
        L.nvfp4_validate.restype = ctypes.c_int
        L.nvfp4_validate.argtypes = [gp, ctypes.c_int]
        L.nvfp4_plan.restype = ctypes.c_int
        L.nvfp4_plan.argtypes = [gp, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_int32), ctypes.c_int]
        L.nvfp4_release_workspace.restype = ctypes.c_int
        L.nvfp4_release_workspace.argtypes = [ctypes.c_void_p]
        L.nvfp4_stream_errors.restype = ctypes.c_int
        L.nvfp4_stream_errors.argtypes = [ctypes.c_void_p]
        L.nvfp4_swizzled_scale_bytes.restype = ctypes.c_int64
        L.nvfp4_swizzled_scale_bytes.argtypes = [ctypes.c_int, ctypes.c_int]
        L.nvfp4_swizzle_scales.restype = ctypes.c_int
        L.nvfp4_swizzle_scales.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_void_p]
        L.nvfp4_tile_rows.restype = ctypes.c_int
        L.nvfp4_tile_cols.restype = ctypes.c_int
        L.nvfp4_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _last_error() -> str:
    return lib().nvfp4_last_error().decode(errors="replace")


def make_group(a=0, b=0, sfa=0, sfb=0, c=0, m=0, n=0, k=0, flags=0) -> Nvfp4Group:
    """A group descriptor from raw device addresses (ints) and sizes."""
    return Nvfp4Group(a or None, b or None, sfa or None, sfb or None, c or None, m, n, k, flags)


def _array(groups: Sequence[Nvfp4Group]):
    arr = (Nvfp4Group * max(1, len(groups)))(*groups)
    return arr


def group_gemm_raw(groups: Sequence[Nvfp4Group], stream: int = 0) -> None:
    """Call nvfp4_group_gemm with prepared descriptors on a raw hipStream_t."""
    arr = _array(groups)
    rc = lib().nvfp4_group_gemm(arr, len(groups), ctypes.c_void_p(stream or None))
    if rc != NVFP4_OK:
        raise Nvfp4Error(rc, _last_error())


def group_gemm_noalloc_raw(groups: Sequence[Nvfp4Group], stream: int = 0) -> None:
    """Call nvfp4_group_gemm_noalloc (no device allocation: the library's
    fixed per-GPU workspace; overlapping calls on one GPU race)."""
    arr = _array(groups)
    rc = lib().nvfp4_group_gemm_noalloc(arr, len(groups), ctypes.c_void_p(stream or None))
    if rc != NVFP4_OK:
        raise Nvfp4Error(rc, _last_error())


def validate(groups: Sequence[Nvfp4Group]) -> Tuple[int, str]:
    """Host-only argument check; returns (code, message)."""
    rc = lib().nvfp4_validate(_array(groups), len(groups))
    return rc, (_last_error() if rc else "")


def plan(groups: Sequence[Nvfp4Group], num_workgroups: int = 256) -> List[Tuple[int, ...]]:
    """Host-only work decomposition for a device with `num_workgroups` compute
    units: list of segments (workgroup, group, m0, rows, n0, k_begin, k_end,
    role); role 0 = whole tile, 1 = partial sum, 2 = finalizer."""
    arr = _array(groups)
    n = lib().nvfp4_plan(arr, len(groups), num_workgroups, None, 0)
    if n < 0:
        raise Nvfp4Error(-n, _last_error())
    buf = (ctypes.c_int32 * (8 * max(1, n)))()
    n2 = lib().nvfp4_plan(arr, len(groups), num_workgroups, buf, n)
    assert n2 == n
    return [tuple(buf[8 * i:8 * i + 8]) for i in range(n)]


def release_workspace(stream: int = 0) -> None:
    """Free the library's workspace of the current device and a raw
    hipStream_t (after the work queued on it)."""
    rc = lib().nvfp4_release_workspace(ctypes.c_void_p(stream or None))
    if rc != NVFP4_OK:
        raise Nvfp4Error(rc, _last_error())


def stream_errors(stream: int = 0) -> int:
    """Synchronise a raw hipStream_t and return (and clear) the count of
    hand-off waits that ran out since the last check (0 when all is well)."""
    rc = lib().nvfp4_stream_errors(ctypes.c_void_p(stream or None))
    if rc < 0:
        raise Nvfp4Error(-rc, _last_error())
    return rc


def swizzled_scale_bytes(rows: int, k: int) -> int:
    """Bytes of the window-major layout of a [rows][k/16] scale matrix."""
    return int(lib().nvfp4_swizzled_scale_bytes(rows, k))


def swizzle_scales(sf, rows: int = None, k: int = None, stream=None):
    """Window-major copy of a [rows, k/16] device tensor of scale bytes (a new
    uint8 device tensor of swizzled_scale_bytes(rows, k) bytes), for use as
    sfb with NVFP4_SFB_SWIZZLED.  Enqueued on `stream` (default: current)."""
    import torch
    if rows is None:
        rows, kb = sf.shape
        k = 16 * kb
    if sf.numel() and (not sf.is_cuda or not sf.is_contiguous() or sf.element_size() != 1):
        raise ValueError("sf must be a contiguous device tensor of bytes")
    out = torch.empty(max(1, swizzled_scale_bytes(rows, k)), dtype=torch.uint8, device=sf.device)
    if stream is None:
        stream = torch.cuda.current_stream()
    rc = lib().nvfp4_swizzle_scales(ctypes.c_void_p(sf.data_ptr() or None), ctypes.c_void_p(out.data_ptr()),
                                     rows, k, ctypes.c_void_p(stream.cuda_stream or None))
    if rc != NVFP4_OK:
        raise Nvfp4Error(rc, _last_error())
    return out


def tile_rows() -> int:
    return lib().nvfp4_tile_rows()


def tile_cols() -> int:
    return lib().nvfp4_tile_cols()


def _descriptor(a, b, sfa, sfb, c, sfb_swizzled=False) -> Nvfp4Group:
    import torch
    m, kb = a.shape
    n = b.shape[0]
    k = 2 * kb
    sfb_shape = (swizzled_scale_bytes(n, k),) if sfb_swizzled else (n, k // 16)
    for name, t, shape, dt in (("a", a, (m, kb), torch.uint8), ("b", b, (n, kb), torch.uint8),
                               ("sfa", sfa, (m, k // 16), None), ("sfb", sfb, sfb_shape, None),
                               ("c", c, (m, n), torch.float16)):
        if name == "sfb" and sfb_swizzled and t.numel() >= shape[0]:
            shape = tuple(t.shape)    # the swizzled buffer may be larger
        if tuple(t.shape) != shape:
            raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), shape))
        if dt is not None and t.dtype != dt:
            raise ValueError("%s has dtype %s, expected %s" % (name, t.dtype, dt))
        if t.element_size() != (2 if name == "c" else 1):
            raise ValueError("%s must hold 1-byte codes/scales (or fp16 for c)" % name)
        if t.numel() and not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
        if t.numel() and not t.is_cuda:
            raise ValueError("%s must be a device tensor" % name)
    return make_group(a.data_ptr(), b.data_ptr(), sfa.data_ptr(), sfb.data_ptr(), c.data_ptr(), m, n, k,
                      NVFP4_SFB_SWIZZLED if sfb_swizzled else 0)


def group_gemm(groups: Iterable, stream=None) -> None:
    """C_g = A_g * B_g^T for every (a, b, sfa, sfb, c) tuple of device tensors.

    a: uint8 [M, K/2], b: uint8 [N, K/2] (packed E2M1, low nibble = even k),
    sfa: [M, K/16], sfb: [N, K/16] (E4M3FN bytes, uint8 or float8_e4m3fn),
    c: float16 [M, N], written in place.  A sixth element True marks sfb as
    the window-major copy made by swizzle_scales.  Runs on `stream` (a torch
    stream, default: the current stream) without synchronising.
    """
    import torch
    descs = [_descriptor(*g) for g in groups]
    if stream is None:
        stream = torch.cuda.current_stream()
    group_gemm_raw(descs, stream.cuda_stream)
