"""Build libnvfp4.so (the HIP kernels and the C ABI) in-tree for gfx950, and
the reference streaming kernels bench.py measures the HBM ceiling with
(bench_ref/libstream_ref.so, not part of the library).

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


BENCH_REF = os.path.join(HERE, "bench_ref")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
         "-Wall", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def library_path() -> str:
    """The in-tree libnvfp4.so."""
    return os.path.join(HERE, "libnvfp4.so")


def stream_ref_path() -> str:
    """The reference streaming kernels bench.py measures the HBM ceiling with."""
    return os.path.join(BENCH_REF, "libstream_ref.so")


def _hipcc(sources, out, includes, verbose):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + ".tmp"
    cmd = [hipcc, *FLAGS]
    for inc in includes:
        cmd += ["-I", inc]
    cmd += [*sources, "-o", tmp]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build_library(verbose: bool = False, out: str = None, csrc: str = CSRC) -> str:
    return _hipcc(sorted(glob.glob(os.path.join(csrc, "*.hip"))),
                  out or library_path(), [os.path.join(ROOT, "include"), csrc], verbose)


def build_stream_ref(verbose: bool = False) -> str:
    return _hipcc([os.path.join(BENCH_REF, "stream_ref.hip")], stream_ref_path(), [], verbose)


if __name__ == "__main__":
    print(build_library(verbose=True))
    print(build_stream_ref(verbose=True))
