"""Compile libtpshard.so (the C-ABI library) for gfx950 with hipcc, in-tree.

Usage: ``python -m attention_column_gemm_amd.build`` or ``build()`` from Python.
The library is written next to this file so that it travels with the source
tree; it is rebuilt on every call.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libtpshard.so")
ARCH = os.environ.get("TPSHARD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 VALU ops (v_pk_*_f32) are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libtpshard")


def build(verbose: bool = False, extra_flags=None) -> str:
    src = os.path.join(CSRC, "tp_shard.hip")
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra_flags or []), src, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
