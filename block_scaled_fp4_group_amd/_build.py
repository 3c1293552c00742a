"""Build step for the HIP library (gfx950).  Compiles csrc/*.hip into
libnvfp4gg.so inside the package directory with hipcc."""
from __future__ import annotations

import os
import subprocess

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
SRC = os.path.join(PKG_DIR, "csrc", "nvfp4_group_gemm.hip")
LIB = os.path.join(PKG_DIR, "libnvfp4gg.so")
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


def build_library(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, "-I" + INCLUDE, SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True))
