"""Build the gfx950 HIP library ``libarnfp8.so`` in-tree with hipcc.

Flags: -O3, C++17, no fast-math (IEEE fp32 division and square root, denormals
kept), and packed-fp32 instruction selection switched off.
"""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SOURCES = [os.path.join(PKG, "csrc", "arnfp8.hip")]  # includes csrc/arnfp8_kernels.hpp
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libarnfp8.so")
ARCH = os.environ.get("ARNFP8_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def build(verbose: bool = False) -> str:
    """Compile every HIP source into ``all_reduce_rmsnorm_amd/libarnfp8.so``."""
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, f"-I{INCLUDE}", *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
