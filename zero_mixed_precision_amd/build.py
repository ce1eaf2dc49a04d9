"""Build the gfx950 shared libraries in place (hipcc cross-compiles without a GPU).

    python zero_mixed_precision_amd/build.py

(run as a script: importing the package first would load the library being
rebuilt)
Flags that carry meaning for the numerics:
  -ffp-contract=off                       no fused multiply-add contraction: one
                                          rounding per written operation
  -fhip-fp32-correctly-rounded-divide-sqrt  IEEE fp32 division and square root
  -fno-gpu-flush-denormals-to-zero        subnormals are kept
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                          no packed fp32 instructions
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
ARCH = os.environ.get("DSZERO_ARCH", "gfx950")

HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def compile_hip(src: str, out: str, includes=()) -> str:
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, *[f"-I{i}" for i in includes], "-o", tmp, src]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build_library() -> str:
    """libdszero.so: the kernels and the C ABI declared in include/dszero.h."""
    return compile_hip(os.path.join(PKG, "csrc", "dszero.hip"), os.path.join(PKG, "libdszero.so"),
                       includes=[os.path.join(ROOT, "include")])


if __name__ == "__main__":
    print(build_library(), file=sys.stderr)
