"""GPU parity of global-norm gradient clipping (fused sum of squares).

The device's sum of squares is an fp64 tree sum over fixed 4096-element
chunks; the oracle's is exact (then rounded once).  The two agree to a few
fp64 ulps of the total, the clip multiplier (an fp32 value) comes out the
same, and every array meets the usual bar.  The device sum itself must not
depend on the launch shape.
"""
import os

import numpy as np
import pytest

import oracle
import synth
from synth.workloads import BETA1, BETA2, EPS, LR, MASTER_SIGMA
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

HP = dict(lr=LR, beta1=BETA1, beta2=BETA2, eps=EPS)
SUMSQ_RTOL = 1e-13


@pytest.fixture(scope="module")
def torch():
    return gu.torch_mod()


def _grads(seed, n, sigma, scale):
    return synth.host_grad16(synth.stream_key(seed, synth.ARR_GRAD), np.arange(n), synth.GradSpec(sigma, scale))


class ClipDev:
    """Device state driven through the clipping entry points."""

    def __init__(self, torch, master, *, scale, K, window=1000):
        from zero_mixed_precision_amd import _lib
        self.L, self.torch, self.n, self.K = _lib, torch, master.size, K
        self.master = gu.dev_f32(torch, master)
        self.m = torch.zeros(self.n, device="cuda:0")
        self.v = torch.zeros(self.n, device="cuda:0")
        self.p16 = torch.zeros(self.n, dtype=torch.int16, device="cuda:0")
        self.acc = torch.empty(self.n, device="cuda:0")
        self.st = torch.zeros(_lib.ds_scaler_size(), dtype=torch.uint8, device="cuda:0")
        self.ws = torch.zeros((_lib.ds_sumsq_workspace_bytes(self.n) + 7) // 8, dtype=torch.float64,
                              device="cuda:0")
        _lib.ds_state_init(self.st, scale, 1.0, window, 1, 0, 1)

    def step(self, host_grads, max_norm, spans=None):
        L, n = self.L, self.n
        gs = [gu.dev_u16(self.torch, g) for g in host_grads]
        if self.K == 1:
            L.ds_check_overflow_sumsq(self.st, gs[0], L.DS_FP16, n, self.ws)
            grad, dt = gs[0], L.DS_FP16
        else:
            spans = spans or [(0, n)]
            for k, g in enumerate(gs):
                for start, size in spans:
                    a, gp = self.acc.data_ptr() + 4 * start, g.data_ptr() + 2 * start
                    if k == self.K - 1:
                        L.ds_accumulate_sumsq(a, gp, L.DS_FP16, size, k == 0, self.st, self.ws)
                    else:
                        L.ds_accumulate(a, gp, L.DS_FP16, size, k == 0)
            grad, dt = self.acc, L.DS_FP32
        L.ds_adam_step(self.st, self.master, self.m, self.v, self.p16, L.DS_FP16, grad, dt, n, LR, BETA1, BETA2, EPS,
                       0.0, max_norm, self.K)
        L.ds_update_loss_scale(self.st)
        return L.ds_state_read(self.st)


def _run(torch, n, K, max_norm, steps=3, sigma=0.05, scale=2.0 ** 10, spans=None, inject=None, seed=0):
    master = synth.host_master32(synth.stream_key(900 + seed, synth.ARR_MASTER), np.arange(n), MASTER_SIGMA)
    o = oracle.State(master.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16),
                     oracle.Scaler(scale, 1.0, 1000, 1))
    d = ClipDev(torch, master, scale=scale, K=K)
    sums = []
    for s in range(steps):
        hg = [_grads(1000 * seed + 10 * s + k, n, sigma * (s + 1), scale) for k in range(K)]
        if inject is not None and s == inject:
            hg[-1][n // 3] = 0x7C00
        ov = oracle.step(o, hg if K > 1 else hg[0], max_grad_norm=max_norm, **HP)
        sc = d.step(hg, max_norm, spans)
        gu.check_scaler(sc, o.scaler, ov, f"clip n={n} K={K} step {s}")
        if not ov and max_norm > 0:
            assert abs(sc.last_grad_sumsq - o.last_sumsq) <= SUMSQ_RTOL * o.last_sumsq, (sc.last_grad_sumsq, o.last_sumsq)
        sums.append(sc.last_grad_sumsq)
        gu.compare_arrays(f"clip n={n} K={K} step {s}", gu.host_f32(d.master), gu.host_f32(d.m),
                          gu.host_f32(d.v), gu.host_u16(d.p16), o.master, o.m, o.v, o.p16)
    return sums, d


@pytest.mark.parametrize("n", [1, 5, 4095, 4096, 4097, 12345, 65536 + 7, (1 << 20) + 3])
@pytest.mark.parametrize("max_norm", [1.0, 1e6])
def test_clipping_fp16_gradient(torch, n, max_norm):
    _run(torch, n, 1, max_norm, seed=n % 97)


@pytest.mark.parametrize("n", [3, 4097, 100_003, (1 << 20) + 3])
def test_clipping_accumulated_gradient(torch, n):
    spans = None
    if n == 100_003:
        spans = [(0, 40_000), (40_000, 24), (40_024, 60_000 - 24), (100_000, 3)]
    _run(torch, n, 4, 1.0, spans=spans, seed=5)


def test_clipping_with_overflow_skips(torch):
    sums, _ = _run(torch, 50_001, 1, 1.0, steps=4, inject=1, seed=6)
    assert not np.isfinite(sums[1])          # the skipped step's sum is not finite, then cleared
    assert np.isfinite(sums[2]) and np.isfinite(sums[3])


def test_sum_of_squares_does_not_depend_on_launch_shape(torch):
    from zero_mixed_precision_amd import _lib
    n = (1 << 20) + 77
    g = gu.dev_u16(torch, _grads(31, n, 0.05, 2.0 ** 10))
    rng = np.random.default_rng(0)
    a32 = gu.dev_f32(torch, (rng.standard_normal(n) * 100).astype(np.float32))
    ws = torch.zeros((_lib.ds_sumsq_workspace_bytes(n) + 7) // 8, dtype=torch.float64, device="cuda:0")
    st = torch.zeros(_lib.ds_scaler_size(), dtype=torch.uint8, device="cuda:0")
    results = {}
    for env in ({}, {"DSZERO_GRID": "1"}, {"DSZERO_GRID": "3"}, {"DSZERO_GRID": "700"}, {"DSZERO_NT": "0"}):
        old = {k: os.environ.get(k) for k in env}
        os.environ.update(env)
        try:
            out = []
            for grad, dt in ((g, _lib.DS_FP16), (a32, _lib.DS_FP32)):
                _lib.ds_state_init(st, 1.0, 1.0, 1, 1, 0, 1)
                _lib.ds_check_overflow_sumsq(st, grad, dt, n, ws)
                out.append(_lib.ds_state_read(st).grad_sumsq)
            acc = torch.zeros(n, device="cuda:0")
            _lib.ds_state_init(st, 1.0, 1.0, 1, 1, 0, 1)
            _lib.ds_accumulate_sumsq(acc, g, _lib.DS_FP16, n, True, st, ws)
            out.append(_lib.ds_state_read(st).grad_sumsq)
            results[str(env)] = out
        finally:
            for k, v in old.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v
    vals = list(results.values())
    assert all(v == vals[0] for v in vals), results
    exact16 = oracle.grad_sumsq(gu.host_u16(g))
    exact32 = oracle.grad_sumsq(gu.host_f32(a32))
    assert abs(vals[0][0] - exact16) <= SUMSQ_RTOL * exact16
    assert abs(vals[0][1] - exact32) <= SUMSQ_RTOL * exact32
    assert vals[0][2] == vals[0][0]           # accumulate of one micro-batch = the fp16 values


def test_shard_step_graph_with_clipping(torch):
    from zero_mixed_precision_amd import ShardStep, ZeroMPConfig
    n = 70_001
    cfg = ZeroMPConfig(lr=LR, betas=(BETA1, BETA2), eps=EPS, initial_scale_power=10, hysteresis=1,
                       gradient_clipping=1.0, gradient_accumulation_steps=2)
    master = synth.host_master32(synth.stream_key(55, synth.ARR_MASTER), np.arange(n), MASTER_SIGMA)
    s = ShardStep(n, cfg)
    s.master.copy_(torch.from_numpy(master))
    o = oracle.State(master.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16),
                     oracle.Scaler(2.0 ** 10, 1.0, 1000, 1))
    bufs = [torch.zeros(n, dtype=torch.float16, device="cuda:0") for _ in range(2)]
    graph = s.graph(bufs)
    for step in range(4):
        hg = [_grads(5000 + 2 * step + k, n, 0.05 * (step + 1), 2.0 ** 10) for k in range(2)]
        for b, h in zip(bufs, hg):
            b.copy_(torch.from_numpy(h.view(np.int16)).view(torch.float16))
        graph.replay()
        ov = oracle.step(o, hg, max_grad_norm=1.0, **HP)
        torch.cuda.synchronize()
        gu.check_scaler(s.scaler(), o.scaler, ov, f"graph clip step {step}")
        gu.compare_arrays(f"graph clip step {step}", gu.host_f32(s.master), gu.host_f32(s.m), gu.host_f32(s.v),
                          gu.host_u16(s.p16), o.master, o.m, o.v, o.p16)
