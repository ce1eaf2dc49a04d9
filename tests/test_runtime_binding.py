"""The native libraries must launch on the HIP runtime that owns torch's memory
and streams, whatever the import order (a PyTorch-ROCm install carries its own
libamdhip64 besides the system one the libraries link against).  The dynamic
linker's binding trace shows which runtime each HIP call is bound to."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bindings(code: str) -> list:
    env = dict(os.environ, LD_BIND_NOW="1", LD_DEBUG="bindings")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                         timeout=300)
    assert out.returncode == 0, out.stderr[-2000:]
    return [line for line in out.stderr.splitlines()
            if ("libdszero.so" in line or "libdssynth.so" in line) and "binding file" in line
            and ("hipLaunchKernel" in line or "__hipRegisterFatBinary" in line)]


def test_library_loaded_before_torch_binds_to_torch_runtime():
    lines = _bindings("import zero_mixed_precision_amd\nimport synth\nsynth.device_lib()\nimport torch")
    assert len(lines) == 4, lines
    assert all("torch/lib/libamdhip64.so" in line for line in lines), lines
