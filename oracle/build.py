"""Compile the CPU oracle (``nvfp4_oracle.c``) into ``liboracle.so`` with gcc.

Flags keep every binary32 operation IEEE round-to-nearest-even with
subnormals: no -ffast-math (which would also set FTZ/DAZ at start-up), no
floating-point contraction. Test infrastructure only.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "nvfp4_oracle.c")


def library_path() -> str:
    return os.path.join(HERE, "liboracle.so")


def build_oracle() -> str:
    out = library_path()
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-Wall",
           "-shared", "-fPIC", SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_oracle())
