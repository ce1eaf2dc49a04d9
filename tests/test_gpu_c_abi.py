"""The optimizer step driven from plain C through the C ABI (no Python, no
PyTorch in that process): tests/c/abi_driver runs steps on device memory from
hipMalloc on a stream of its own, and its outputs are compared with the oracle.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle
import synth
from synth.workloads import BETA1, BETA2, EPS, LR, MASTER_SIGMA
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

DRIVER = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "abi_driver")


@pytest.mark.parametrize("n,K,wd,clip,double", [(4099, 1, 0.0, 0.0, 0), (20_003, 3, 0.01, 0.0, 0),
                                                (65_541, 1, 0.0, 1.0, 0), (10_007, 2, 0.0, 1.0, 0),
                                                (30_011, 1, 0.01, 0.0, 1), (8_195, 2, 0.0, 0.0, 1),
                                                (12_347, 3, 0.01, 0.0, 2)])
def test_c_program_matches_oracle(tmp_path, n, K, wd, clip, double):
    """double = 1: ds_adam_step_double_buffered over two hipMalloc'd copies of
    the state; double = 2: the last micro-batch folded into the double-buffered
    pass; the driver writes out the copy that the state names current."""
    if not os.path.exists(DRIVER):
        pytest.fail(f"{DRIVER} is not built: run __graft_entry__.build()")
    steps, scale, window = 5, 2.0 ** 12, 2
    idx = np.arange(n)
    master = synth.host_master32(synth.stream_key(600 + K, synth.ARR_MASTER), idx, MASTER_SIGMA)
    spec = synth.GradSpec(0.05 if clip else 1e-3, scale)
    grads = np.empty((steps, K, n), np.uint16)
    for s in range(steps):
        for k in range(K):
            grads[s, k] = synth.host_grad16(synth.stream_key(601, synth.ARR_GRAD, s, k), idx, spec)
    grads[2, K - 1, n // 2] = 0x7C00                    # one overflowed step
    (tmp_path / "params.txt").write_text(
        f"{n} {K} {steps} {scale!r} {window} {LR!r} {BETA1!r} {BETA2!r} {EPS!r} {wd!r} {clip!r} {double}\n")
    master.tofile(tmp_path / "master.bin")
    grads.tofile(tmp_path / "grads.bin")
    gu.say(f"[c-abi] n={n} K={K} wd={wd} clip={clip} double={double}")
    r = subprocess.run([DRIVER, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "rejected as expected" in r.stdout

    o = oracle.State(master.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16),
                     oracle.Scaler(scale, 1.0, window, 1))
    trace = (tmp_path / "scaler.txt").read_text().split("\n")
    for s in range(steps):
        gs = [grads[s, k] for k in range(K)]
        ov = oracle.step(o, gs if K > 1 else gs[0], lr=LR, beta1=BETA1, beta2=BETA2, eps=EPS, weight_decay=wd,
                         max_grad_norm=clip)
        last, sc, applied, it, skipped = trace[s].split()
        assert (int(last) == 1) == ov and float(sc) == o.scaler.scale, (s, trace[s])
        assert (int(applied), int(it), int(skipped)) == (o.scaler.applied, o.scaler.s.iters, o.scaler.s.skipped)
    got = [np.fromfile(tmp_path / f, dtype=dt) for f, dt in (("master_out.bin", np.float32), ("m_out.bin", np.float32),
                                                              ("v_out.bin", np.float32), ("p16_out.bin", np.uint16))]
    if double:   # 4 of the 5 steps applied: copy 0 holds the state again
        assert "current copy: 0" in r.stdout, r.stdout
    du = gu.compare_arrays(f"c-abi n={n} K={K}", *got, o.master, o.m, o.v, o.p16)
    gu.say(f"[c-abi] n={n} K={K}: max ulp {du}")
