"""Builds tests/c/abi_driver, a plain-C program that drives libdszero.so through
include/dszero.h (test infrastructure: tests/test_gpu_c_abi.py runs it)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SRC = os.path.join(HERE, "abi_driver.c")
OUT = os.path.join(HERE, "abi_driver")


def build_driver() -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), "-D__HIP_PLATFORM_AMD__",
           SRC, "-o", OUT,
           "-L", os.path.join(ROOT, "zero_mixed_precision_amd"), "-ldszero",
           "-Wl,-rpath,$ORIGIN/../../zero_mixed_precision_amd",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    subprocess.run(cmd, check=True)
    return OUT


if __name__ == "__main__":
    print(build_driver())
