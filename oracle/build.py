"""Compile the C++ oracle (oracle/dllm_oracle.cpp) into oracle/liboracle_dllm.so with the host
compiler. Test infrastructure only: nothing in the HIP library links or loads it.

    python oracle/build.py

-ffp-contract=off keeps every product and sum a separately rounded IEEE operation, as written.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "dllm_oracle.cpp")
LIB = os.path.join(HERE, "liboracle_dllm.so")


def command(out: str = LIB) -> list:
    cxx = os.environ.get("CXX") or shutil.which("g++") or "g++"
    return [cxx, "-O2", "-std=c++17", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
            "-Wall", "-Wextra", SRC, "-o", out]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"oracle build failed with exit code {res.returncode}")
    if res.stderr.strip():
        sys.stderr.write(res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
