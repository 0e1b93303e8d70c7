"""Compile the device-identity probes (nvfp4_identities.hip, test code) into
libnvfp4_identities.so next to this file, with the library's own compiler
flags, so that the probed inline functions compile as they do in the
kernels."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "precision_quantization_row_amd", "csrc")


def library_path() -> str:
    return os.path.join(HERE, "libnvfp4_identities.so")


def build_identities() -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    out = library_path()
    tmp = out + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-ffp-contract=off", "-Wall",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", CSRC, os.path.join(HERE, "nvfp4_identities.hip"), "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_identities())
