"""Build step for the CPU oracle (plain C, gcc, OpenMP) -- test infrastructure.

-ffp-contract=off keeps a*b+c as two rounded operations, which the int4
quantizer's fp32 definition needs; no fast-math anywhere.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kmr_oracle.c")
HDR = os.path.join(HERE, "kmr_oracle.h")
OUT = os.path.join(HERE, "liboracle.so")

CMD = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
       "-fno-fast-math", "-Wall", "-Wextra", "-o", OUT, SRC, "-lm"]


def build(force: bool = True) -> str:
    stale = (not os.path.exists(OUT)
             or os.path.getmtime(OUT) < max(os.path.getmtime(SRC), os.path.getmtime(HDR)))
    if force or stale:
        tmp = OUT + ".tmp"
        cmd = CMD[:]
        cmd[cmd.index(OUT)] = tmp
        subprocess.run(cmd, check=True)
        os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(force=True))
