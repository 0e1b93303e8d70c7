"""Build libnvfp4.so (the HIP kernels and the C ABI) in-tree for gfx950.

hipcc compiles every .hip source under csrc/ into one shared library next to
this file. Flags:
  --offload-arch=gfx950                 CDNA4 only, no other targets
  -O3 -ffp-contract=off                 no fused multiply-add contraction, so
                                        every product / quotient is rounded once
  (no -ffast-math)                      IEEE division, fp32 denormals kept
  -target-feature -packed-fp32-ops      keep the compiler from emitting packed
                                        fp32 VALU forms
"""
from __future__ import annotations

import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)


def library_path() -> str:
    """The in-tree libnvfp4.so (NVFP4_LIBRARY may name another build of it)."""
    return os.environ.get("NVFP4_LIBRARY") or os.path.join(HERE, "libnvfp4.so")


def build_library(verbose: bool = False, out: str = None, csrc: str = CSRC) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    out = out or os.path.join(HERE, "libnvfp4.so")
    tmp = out + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-ffp-contract=off", "-Wall",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", csrc,
           *sorted(glob.glob(os.path.join(csrc, "*.hip"))), "-o", tmp]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library(verbose=True))
