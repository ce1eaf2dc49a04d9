"""Build synth/libdssynth.so (device side of the seeded input generator).

    python synth/build.py
"""
import importlib.util
import os

HERE = os.path.dirname(os.path.abspath(__file__))
_spec = importlib.util.spec_from_file_location(
    "_dszero_build", os.path.join(os.path.dirname(HERE), "zero_mixed_precision_amd", "build.py"))
_build = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(_build)      # the compiler flags, without importing the package
compile_hip = _build.compile_hip


def build_library() -> str:
    return compile_hip(os.path.join(HERE, "csrc", "synth.hip"), os.path.join(HERE, "libdssynth.so"))


if __name__ == "__main__":
    print(build_library())
