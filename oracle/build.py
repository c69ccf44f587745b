"""Compile the oracle's plain C integer GEMM (test infrastructure only)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "int_gemm.c")
LIB = os.path.join(HERE, "liboracle_gemm.so")


def build(force: bool = False) -> str:
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared",
                               "-std=c99", "-Wall", "-o", tmp, SRC])
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force=True))
