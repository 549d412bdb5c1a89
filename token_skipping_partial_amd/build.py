"""Compile the HIP sources into the in-tree shared library `libdllm.so` (gfx950 only).

    python token_skipping_partial_amd/build.py

(run as a script, or through __graft_entry__.build(): importing the package first would load the
library that is about to be rebuilt).

hipcc cross-compiles for gfx950 without a GPU present. Packed fp32 instructions are disabled
(-packed-fp32-ops) for every device compilation.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libdllm.so")
SOURCES = ["api.hip", "saliency.hip", "select.hip", "gemm.hip", "attn.hip", "decode.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libdllm.so)")


def command(out: str = LIB) -> list:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-result",
        "-I", os.path.join(ROOT, "include"),
        *[os.path.join(CSRC, s) for s in SOURCES],
        "-L", "/opt/rocm/lib", "-lrocprofiler-sdk-roctx",
        "-o", out,
    ]


def build(verbose: bool = False) -> str:
    """Always recompiles; writes to a temporary name and renames, so a failed build never
    leaves a half-written library behind."""
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    if verbose and res.stderr.strip():
        sys.stderr.write(res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
