"""Compile the plain-C oracle into oracle/liboracle.so (gcc, no GPU involved).

Flags: -O2 with -ffp-contract=off and no fast-math, so the compiler never fuses a
multiply and an add and every float expression rounds as written.  OpenMP only
spreads independent output rows over threads.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
HDR = os.path.join(HERE, "oracle.h")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
          "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(force: bool = True) -> str:
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= max(os.path.getmtime(SRC), os.path.getmtime(HDR)):
        return LIB
    tmp = LIB + f".tmp{os.getpid()}"
    subprocess.run(["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force="--if-stale" not in sys.argv))
