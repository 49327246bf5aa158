"""Builds the HIP library ``libets_topk.so`` in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "ets_topk.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libets_topk.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # packed fp32 instructions are disabled for every HIP source of this library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # LDS histogram atomics are aggregated by hand; keep the compiler from
    # rewriting them into wave reductions
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False) -> str:
    """Compile the library (always) and return its path."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
