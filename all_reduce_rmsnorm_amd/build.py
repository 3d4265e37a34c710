"""Build the gfx950 HIP library ``libarnfp8.so`` in-tree with hipcc.

Flags: -O3, C++17, no fast-math (IEEE fp32 division and square root, denormals
kept), and packed-fp32 instruction selection switched off.
"""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
# Translation units, compiled in parallel and linked into one library.  The
# device code lives in csrc/arnfp8_kernels.hpp; each arnfp8_rows_*.hip holds
# one output format's kernel instances.
SOURCES = [os.path.join(PKG, "csrc", f) for f in
           ("arnfp8.hip", "arnfp8_rows_e4m3.hip", "arnfp8_rows_e5m2.hip", "arnfp8_rows_mxfp8.hip",
            "arnfp8_split.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libarnfp8.so")
# Achievable-bandwidth reference kernels for the benchmark, in a library of
# their own (not part of the product library).
REF_SOURCES = [os.path.join(PKG, "csrc", "arnfp8_ref_kernels.hip")]
REF_LIB_PATH = os.path.join(PKG, "libarnfp8_ref.so")
ARCH = os.environ.get("ARNFP8_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link ``all_reduce_rmsnorm_amd/libarnfp8.so``
    (and the benchmark's reference kernels, ``libarnfp8_ref.so``)."""
    obj_dir = os.path.join(PKG, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    procs, objs = [], {}
    for src in SOURCES + REF_SOURCES:
        obj = os.path.join(obj_dir, os.path.basename(src)[:-4] + ".o")
        cmd = [hipcc(), *HIPCC_FLAGS, "-c", f"-I{INCLUDE}", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd), src))
        objs[src] = obj
    failed = [src for p, src in procs if p.wait() != 0]
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    for srcs, path in ((SOURCES, LIB_PATH), (REF_SOURCES, REF_LIB_PATH)):
        tmp = path + ".tmp"
        link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC",
                *[objs[s] for s in srcs], "-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        subprocess.run(link, check=True)
        os.replace(tmp, path)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
