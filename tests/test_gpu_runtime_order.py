"""Regression: with libdszero.so loaded before torch (a fresh process), the
step, a HIP-graph capture of it and the device generator still run on torch's
streams and match the oracle."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r'''
import zero_mixed_precision_amd            # loads libdszero.so before torch
import synth
synth.device_lib()                         # and libdssynth.so
import numpy as np
import torch
import __graft_entry__
__graft_entry__.smoke()
from zero_mixed_precision_amd import ShardStep, ZeroMPConfig
cfg = ZeroMPConfig(lr=1e-4, initial_scale_power=12, hysteresis=1)
a, b = ShardStep(10007, cfg), ShardStep(10007, cfg)
for s in (a, b):
    s.master.fill_(0.5)
g = torch.full((10007,), 3.0, dtype=torch.float16, device="cuda:0")
graph = b.graph([g])
for _ in range(3):
    a.step(g)
    graph.replay()
torch.cuda.synchronize()
assert torch.equal(a.master, b.master) and a.scaler().as_dict() == b.scaler().as_dict()
print("runtime order ok", flush=True)
'''


def test_library_first_then_torch_in_a_fresh_process():
    out = subprocess.run([sys.executable, "-c", SCRIPT], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, (out.stdout[-2000:], out.stderr[-3000:])
    assert "runtime order ok" in out.stdout
