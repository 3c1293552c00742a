"""Build step for the HIP library (gfx950).  Compiles csrc/*.hip into
libnvfp4gg.so inside the package directory with hipcc."""
from __future__ import annotations

import os
import subprocess

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
SRC = os.path.join(PKG_DIR, "csrc", "nvfp4_group_gemm.hip")
LIB = os.path.join(PKG_DIR, "libnvfp4gg.so")
# measurement probe (matrix-core rates and clock), loaded by bench.py only
PROBE_SRC = os.path.join(PKG_DIR, "csrc", "mfma_rate.hip")
PROBE_LIB = os.path.join(PKG_DIR, "libnvfp4gg_probe.so")
INCLUDE = os.path.join(REPO_DIR, "include")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 VALU ops are kept out of the generated code on purpose
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # private arrays stay in registers (or scratch), never in LDS, whose
    # every byte the kernel lays out itself
    "-mllvm", "-disable-promote-alloca-to-lds",
]


def _compile(src: str, lib: str, verbose: bool) -> str:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, "-I" + INCLUDE, src, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, lib)
    return lib


def build_library(verbose: bool = False) -> str:
    """The GEMM library, then the measurement probe."""
    _compile(SRC, LIB, verbose)
    _compile(PROBE_SRC, PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True))
