"""GPU parity of ds_accumulate_multi: several micro-batch gradients folded into
the fp32 accumulation buffer in one pass.

The fold's result is defined as that of the same gradients accumulated one by
one ("DeepSpeed" overview, core features: accumulation emulates a larger batch;
"DeepSpeed complete guide" section 5.1), so every case is checked bit for bit
against both the oracle's in-order fp32 accumulation and the library's own
single-gradient passes: the buffer, the fused inf/NaN flag and the sum of
squares for clipping.  Whole steps with folded accumulation match the oracle's
step with K micro-batches.
"""
import os

import numpy as np
import pytest

import oracle
import synth
from synth.workloads import BETA1, BETA2, EPS, LR, MASTER_SIGMA
from tests import gpu_util as gu
from tests._fp import f32_bits

pytestmark = pytest.mark.gpu

HP = dict(lr=LR, beta1=BETA1, beta2=BETA2, eps=EPS)


@pytest.fixture(scope="module")
def torch():
    t = gu.torch_mod()
    import zero_mixed_precision_amd  # noqa: F401
    return t


def _grads(seed, n, count, fmt):
    if fmt == "fp16":
        spec = synth.GradSpec(1e-3, 2.0 ** 15)
    else:
        spec = synth.GradSpec(1e-3, 1.0, fmt="bf16")
    gs = [synth.host_grad16(synth.stream_key(seed, synth.ARR_GRAD, k), np.arange(n), spec) for k in range(count)]
    rng = np.random.default_rng(seed)
    for g in gs:                                  # every finite pattern class mixed in
        pick = rng.random(n) < 0.2
        pat = rng.integers(0, 65536, n).astype(np.uint16)
        exp = 0x7C00 if fmt == "fp16" else 0x7F80
        pat = np.where((pat & exp) == exp, pat & ~np.uint16(0x4000), pat).astype(np.uint16)
        g[:] = np.where(pick, pat, g)
    return gs


def _run(torch, n, count, overwrite, check, sumsq, fmt, inject=None, env=None):
    from zero_mixed_precision_amd import _lib
    old = {k: os.environ.get(k) for k in (env or {})}
    os.environ.update(env or {})
    try:
        dt = _lib.DS_BF16 if fmt == "bf16" else _lib.DS_FP16
        gs = _grads(1000 + n % 977 + count, n, count, fmt)
        if inject is not None:
            gs[inject[0]][inject[1]] = 0x7C00 if fmt == "fp16" else 0x7F80
        rng = np.random.default_rng(n + count)
        acc0 = (rng.standard_normal(n) * 100).astype(np.float32)
        # the oracle's in-order accumulation
        acc_o = acc0.copy()
        for k, g in enumerate(gs):
            oracle.accumulate(acc_o, g, overwrite=(overwrite and k == 0), fmt=fmt)
        devg = [gu.dev_u16(torch, g) for g in gs]
        ws_n = (_lib.ds_sumsq_workspace_bytes(n) + 7) // 8 + 1
        out = []
        for mode in ("single", "fold"):
            acc = gu.dev_f32(torch, acc0)
            st = torch.zeros(_lib.ds_scaler_size(), dtype=torch.uint8, device="cuda:0")
            ws = torch.zeros(ws_n, dtype=torch.float64, device="cuda:0")
            _lib.ds_state_init(st, 1.0, 1.0, 1, 1, 0, 1)
            stp = st if (check or sumsq) else None
            if mode == "single":
                for k, g in enumerate(devg):
                    last = k == count - 1
                    if last and sumsq:
                        _lib.ds_accumulate_sumsq(acc, g, dt, n, overwrite and k == 0, st, ws)
                    else:
                        _lib.ds_accumulate(acc, g, dt, n, overwrite and k == 0, stp if last else None)
            else:
                _lib.ds_accumulate_multi(acc, devg, dt, n, overwrite, stp, ws if sumsq else None)
            sc = _lib.ds_state_read(st)
            out.append((gu.host_f32(acc), sc.overflow, sc.grad_sumsq))
        (a1, f1, s1), (a2, f2, s2) = out
        assert np.array_equal(f32_bits(a2), f32_bits(acc_o)), "fold vs oracle"
        assert np.array_equal(f32_bits(a1), f32_bits(a2)), "fold vs single passes"
        assert f1 == f2 and bool(f2) == (check and not np.isfinite(acc_o).all())
        if sumsq:
            assert s1 == s2 or (np.isnan(s1) and np.isnan(s2)), (s1, s2)   # same chunks, same order
            if np.isfinite(acc_o).all():
                exact = float(np.sum(acc_o.astype(np.float64) ** 2))
                assert abs(s2 - exact) <= 1e-12 * exact
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


@pytest.mark.parametrize("n", [1, 5, 4095, 4097, 12_345, (1 << 20) + 3])
@pytest.mark.parametrize("count", [1, 2, 3, 8])
def test_fold_equals_single_passes(torch, n, count):
    _run(torch, n, count, overwrite=True, check=True, sumsq=False, fmt="fp16")


@pytest.mark.parametrize("count", [2, 5, 7])
@pytest.mark.parametrize("overwrite,check,sumsq", [(False, False, False), (False, True, False), (True, True, True),
                                                   (False, True, True)])
def test_fold_variants(torch, count, overwrite, check, sumsq):
    _run(torch, 70_001, count, overwrite, check, sumsq, "fp16")


@pytest.mark.parametrize("count", [1, 4])
def test_fold_bf16(torch, count):
    _run(torch, 50_003, count, True, True, True, "bf16")


@pytest.mark.parametrize("k", [0, 2, 4])
def test_fold_flags_a_planted_infinity(torch, k):
    _run(torch, 40_009, 5, True, True, False, "fp16", inject=(k, 40_009 - 1 - k))


@pytest.mark.parametrize("env", [{"DSZERO_NT": "1"}, {"DSZERO_GRID": "1"}, {"DSZERO_GRID": "7"}])
def test_fold_launch_shape_invariance(torch, env):
    _run(torch, 300_007, 6, False, True, True, "fp16", env=env)


def test_whole_steps_with_folded_accumulation(torch):
    """K = 8 micro-batches per step accumulated as folds of 3 and 5 (bucketed
    calls, with an overflow in one step) or one fold of 8: every step matches
    the oracle's step with K = 8."""
    from zero_mixed_precision_amd import _lib
    n, K, steps = 100_003, 8, 5
    spans = [(0, 40_000), (40_000, 24), (40_024, 60_000 - 24), (100_000, 3)]
    master0 = synth.host_master32(synth.stream_key(4400, synth.ARR_MASTER), np.arange(n), MASTER_SIGMA)
    o = oracle.State(master0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16),
                     oracle.Scaler(2.0 ** 15, 1.0, 2, 1))
    d = gu.DevState(torch, master0, np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16),
                    init_scale=2.0 ** 15, window=2, K=K)
    spec = synth.GradSpec(1e-3, 2.0 ** 15)
    for s in range(steps):
        gs = [synth.host_grad16(synth.stream_key(4401, synth.ARR_GRAD, s, k), np.arange(n), spec) for k in range(K)]
        if s == 2:
            gs[6][77] = 0x7C00
        devg = [gu.dev_u16(torch, g) for g in gs]
        groups = [range(0, 3), range(3, 8)] if s % 2 == 0 else [range(0, 8)]
        for gi, grp in enumerate(groups):
            last = gi == len(groups) - 1
            for start, size in spans:
                ptrs = [devg[k].data_ptr() + 2 * start for k in grp]
                _lib.ds_accumulate_multi(d.acc.data_ptr() + 4 * start, ptrs, _lib.DS_FP16, size, gi == 0,
                                         d.state if last else None)
        _lib.ds_adam_step_fused(d.state, d.master, d.m, d.v, d.p16, _lib.DS_FP16, d.acc, _lib.DS_FP32, n, LR, None,
                                BETA1, BETA2, EPS, 0.0, 0.0, K)
        ov = oracle.step(o, gs, **HP)
        gu.check_scaler(d.scaler(), o.scaler, ov, f"fold step {s}")
        du = gu.compare_full(f"fold step {s}", d, o)
        assert max(du.values()) == 0, du


@pytest.mark.parametrize("clip", [0.0, 0.05])
def test_shard_step_folds_lists(torch, clip):
    """ShardStep.accumulate with lists (folds of 2, 1 and 2 of K = 5) and
    full_step (one fold of 5) give the oracle's steps; with clipping active the
    fold's sum of squares feeds the multiplier (within the usual bar)."""
    from zero_mixed_precision_amd import ShardStep, ZeroMPConfig
    n, K = 30_011, 5
    cfg = ZeroMPConfig(lr=LR, betas=(BETA1, BETA2), eps=EPS, initial_scale_power=14, loss_scale_window=2,
                       hysteresis=1, gradient_accumulation_steps=K, gradient_clipping=clip)
    master0 = synth.host_master32(synth.stream_key(4500, synth.ARR_MASTER), np.arange(n), MASTER_SIGMA)
    a, b = ShardStep(n, cfg), ShardStep(n, cfg)
    for sh in (a, b):
        sh.master.copy_(torch.from_numpy(master0))
        sh.p16.zero_()
    o = oracle.State(master0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16),
                     oracle.Scaler(2.0 ** 14, 1.0, 2, 1))
    spec = synth.GradSpec(1e-3, 2.0 ** 14)
    for s in range(4):
        gs = [synth.host_grad16(synth.stream_key(4501, synth.ARR_GRAD, s, k), np.arange(n), spec) for k in range(K)]
        if s == 1:
            gs[3][5] = 0x7C00
        dev = [gu.dev_u16(torch, g).view(torch.float16) for g in gs]
        a.accumulate(dev[0:2])
        a.accumulate(dev[2])
        a.accumulate(dev[3:5])
        a.step()
        b.full_step(dev)
        ov = oracle.step(o, gs, max_grad_norm=clip, **HP)
        torch.cuda.synchronize()
        assert a.scaler().as_dict() == b.scaler().as_dict()
        gu.check_scaler(a.scaler(), o.scaler, ov, f"ShardStep fold step {s}")
        for x, y in ((a.master, b.master), (a.m, b.m), (a.v, b.v)):
            assert torch.equal(x.view(torch.int32), y.view(torch.int32))
        du = gu.compare_arrays(f"ShardStep fold step {s}", gu.host_f32(a.master), gu.host_f32(a.m),
                               gu.host_f32(a.v), gu.host_u16(a.p16.view(torch.int16)), o.master, o.m, o.v, o.p16)
        if clip == 0.0:
            assert max(du.values()) == 0, du
