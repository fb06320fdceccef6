"""Build the C++ float64 oracle (``libttt_oracle.so``) with g++.

Test infrastructure: the library is loaded only by the tests, the package
smoke check and the benchmark's CPU-baseline leg.  No fast-math and no
target-specific flags: products and sums keep the IEEE float64 semantics of
the source (no contraction into FMA on the baseline x86-64 target).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ttt_oracle.cpp")
LIB = os.path.join(HERE, "libttt_oracle.so")
CXX = os.environ.get("ORACLE_CXX", "g++")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [CXX, "-O2", "-std=c++17", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-Wall", "-Wno-unknown-pragmas", SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"g++ failed for the oracle:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
