"""Compile the CPU oracle into ``oracle/liblf_oracle.so`` with g++.

Test infrastructure: the oracle is only ever loaded by the tests, the smoke
check and the CPU-baseline leg of the benchmark.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "lf_oracle.cpp")
LIB = os.path.join(HERE, "liblf_oracle.so")

CMD = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
       "-fno-fast-math", "-Wall", "-Wextra", "-o", LIB, SRC]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = CMD[:-3] + ["-o", tmp, SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
