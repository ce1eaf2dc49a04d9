"""Build synth/libdssynth.so (device side of the seeded input generator)."""
import os

from zero_mixed_precision_amd.build import compile_hip

HERE = os.path.dirname(os.path.abspath(__file__))


def build_library() -> str:
    return compile_hip(os.path.join(HERE, "csrc", "synth.hip"), os.path.join(HERE, "libdssynth.so"))


if __name__ == "__main__":
    print(build_library())
