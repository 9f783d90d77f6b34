"""Compile the fp64 CPU oracle (plain C, gcc) into oracle/liboracle.so.

Test infrastructure: the HIP library never links or loads the result.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "vegas_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(force: bool = True) -> str:
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-std=c99", "-O2", "-fno-fast-math", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-D_POSIX_C_SOURCE=200809L", SRC, "-o", tmp, "-lpthread", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force="--if-stale" not in sys.argv))
