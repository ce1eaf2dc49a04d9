"""Builds the C test programs of the C ABI (test infrastructure):

  tests/c/abi_driver    plain C driving libdszero.so through include/dszero.h
                        on the GPU (tests/test_gpu_c_abi.py runs it)
  tests/c/host_checks   every host-only path of the library, linked against a
                        copy built with the host AddressSanitizer and
                        UndefinedBehaviorSanitizer (tests/test_host_sanitizers.py)
"""
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


HOST_SRC = os.path.join(HERE, "host_checks.c")
HOST_OUT = os.path.join(HERE, "host_checks")
ASAN_LIB = os.path.join(HERE, "libdszero_asan.so")


def build_host_checks() -> str:
    """The library with host-side sanitizers (device code as usual; each
    -fsanitize applies to the host pass only) and the program that drives it,
    both built by ROCm's clang so that they share one sanitizer runtime."""
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    clang = os.path.join(ROCM, "llvm", "bin", "clang")
    lib_cmd = [hipcc, "-O1", "-g", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950",
               "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
               "-Xarch_host", "-fno-omit-frame-pointer",
               "-I", os.path.join(ROOT, "include"), "-o", ASAN_LIB,
               os.path.join(ROOT, "zero_mixed_precision_amd", "csrc", "dszero.hip")]
    subprocess.run(lib_cmd, check=True, stderr=subprocess.DEVNULL)
    exe_cmd = [clang, "-std=c11", "-O1", "-g", "-Wall", "-Wextra", "-Werror", "-fsanitize=address,undefined",
               "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"), HOST_SRC, "-o", HOST_OUT,
               "-L", HERE, "-l:libdszero_asan.so", "-Wl,-rpath,$ORIGIN"]
    subprocess.run(exe_cmd, check=True)
    return HOST_OUT


if __name__ == "__main__":
    print(build_driver())
    print(build_host_checks())
