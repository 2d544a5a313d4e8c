"""Build the C++ oracle, oracle/liboracle.so, with g++ (test infrastructure).

Flags: -O2, C++17, OpenMP, and no floating-point contraction, so every
float64 multiply and add rounds as written (no fused multiply-add) and the
sums are taken in index order (no -ffast-math reassociation).
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.cpp")
LIB = os.path.join(HERE, "liboracle.so")
CXX = os.environ.get("CXX_ORACLE", "g++")
FLAGS = ["-O2", "-std=c++17", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
         "-fno-fast-math", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    r = subprocess.run([CXX, *FLAGS, SRC, "-o", tmp], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("g++ failed on the C++ oracle:\n" + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
