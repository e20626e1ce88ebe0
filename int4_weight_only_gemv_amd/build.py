"""Build step for the HIP library libkmr.so (gfx950), in-tree.

hipcc compiles the one translation unit csrc/kmr.hip; the result sits next to
this file so that it travels with the source tree.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "kmr.hip")
OUT = os.path.join(HERE, "libkmr.so")
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 instructions are kept out of the generated code on purpose
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
]


def sources():
    d = os.path.join(HERE, "csrc")
    return [os.path.join(d, f) for f in sorted(os.listdir(d))] + [os.path.join(ROOT, "include", "kmr.h")]


def build(force: bool = True, extra=()) -> str:
    stale = not os.path.exists(OUT) or os.path.getmtime(OUT) < max(os.path.getmtime(s) for s in sources())
    if force or stale:
        tmp = OUT + ".tmp"
        cmd = [HIPCC, *FLAGS, *extra, SRC, "-o", tmp]
        subprocess.run(cmd, check=True)
        os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(force=True, extra=sys.argv[1:]))
