"""Pins of the oracle's learning-rate schedules (WarmupLR, WarmupDecayLR).

Pages: "DeepSpeed complete guide" section 4.1 (the scheduler block, WarmupLR
with warmup_min_lr / warmup_max_lr / warmup_num_steps) and section 4.4
(WarmupDecayLR with last_batch_iteration -1, total_num_steps 100000,
warmup_min_lr 0, warmup_max_lr 3e-4, warmup_num_steps 2000, linear warmup).
The pages name the parameters only; what fixes the oracle here:
  * the endpoints those parameters name (min at the start, max at the end of
    the warmup, min again at total_num_steps) and the page's example values;
  * exact rational values of a linear ramp (every warmup iteration of the
    page's example), within one fp32 ulp of the rounded result;
  * the constant-gradient closed form of Adam, where each applied step moves an
    element by lr(it) * g / (|g| + eps), so the final parameter pins which lr
    each step used (and that a skipped step does not advance the schedule);
  * torch.optim.Adam driven by torch.optim.lr_scheduler.LambdaLR (a library
    routine with its own iteration bookkeeping) over ten steps.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests._fp import f32_bits, ulp32

HERE = os.path.dirname(os.path.abspath(__file__))
B1, B2, EPS = 0.9, 0.999, 1e-8
S16 = 2.0 ** 16
f32 = lambda x: float(np.float32(x))


def _page_example():
    g = json.load(open(os.path.join(HERE, "golden", "scheduler_config.json")))
    blk = g["scheduler_section_4_4"]
    assert blk["type"] == "WarmupDecayLR" and blk["params"]["warmup_type"] == "linear"
    p = blk["params"]
    assert p["last_batch_iteration"] == -1
    return oracle.LrSchedule(oracle.LR_WARMUP_DECAY, p["warmup_min_lr"], p["warmup_max_lr"],
                             p["warmup_num_steps"], p["total_num_steps"]), p


def test_page_example_endpoints(oracle_lib):
    s, p = _page_example()
    W, T = p["warmup_num_steps"], p["total_num_steps"]
    assert s.at(0) == 0.0                       # the first applied step uses warmup_min_lr
    assert s.at(W) == f32(3e-4)                 # the peak at the end of the warmup
    assert s.at(W // 2) == f32(3e-4) / 2        # half way up
    assert s.at((W + T) // 2) == f32(3e-4) / 2  # half way down (98000 / 2 steps after the peak)
    for it in (T, T + 1, 10 * T, 2 ** 40):
        assert s.at(it) == 0.0                  # decayed to warmup_min_lr, and stays there


def _exact(min_lr, max_lr, gamma):
    lo, hi = Fraction(f32(min_lr)), Fraction(f32(max_lr))
    return lo + (hi - lo) * gamma


def test_page_example_is_linear_and_monotone(oracle_lib):
    s, p = _page_example()
    W, T = p["warmup_num_steps"], p["total_num_steps"]
    its = list(range(0, W + 1)) + list(range(W, T + 1, 97)) + [T - 1, T]
    vals = np.array([s.at(i) for i in its], dtype=np.float32)
    for it, v in zip(its, vals):
        gamma = Fraction(it, W) if it < W else Fraction(T - it, T - W)
        exact = _exact(0, 3e-4, gamma)
        assert abs(Fraction(float(v)) - exact) <= Fraction(float(ulp32(np.float32(exact)))), it
    rise = vals[: W + 1]
    fall = vals[W + 1:]
    assert np.all(np.diff(rise) > 0)
    assert np.all(np.diff(fall) <= 0)


def test_warmup_holds_the_peak(oracle_lib):
    s = oracle.LrSchedule(oracle.LR_WARMUP, 1e-5, 1e-3, 10)
    assert s.at(0) == f32(1e-5)
    for it in range(1, 10):
        exact = _exact(1e-5, 1e-3, Fraction(it, 10))
        assert abs(Fraction(s.at(it)) - exact) <= Fraction(float(ulp32(np.float32(exact))))
    assert all(s.at(it) == f32(1e-3) for it in range(10, 2000))
    assert s.at(2 ** 50) == f32(1e-3)


def test_no_warmup(oracle_lib):
    assert oracle.LrSchedule(oracle.LR_WARMUP, 0.0, 2e-4, 0).at(0) == f32(2e-4)
    d = oracle.LrSchedule(oracle.LR_WARMUP_DECAY, 0.0, 2e-4, 0, 100)
    assert d.at(0) == f32(2e-4) and d.at(50) == f32(2e-4) / 2 and d.at(100) == 0.0


def test_decay_ends_at_the_minimum(oracle_lib):
    d = oracle.LrSchedule(oracle.LR_WARMUP_DECAY, 1e-5, 3e-4, 5, 25)
    assert d.at(0) == f32(1e-5) and d.at(5) == f32(3e-4)
    assert d.at(25) == f32(1e-5) and d.at(26) == f32(1e-5) and d.at(10 ** 9) == f32(1e-5)
    # warmup == total: the divisor is held at 1, so the step after the peak is the minimum
    e = oracle.LrSchedule(oracle.LR_WARMUP_DECAY, 1e-5, 3e-4, 5, 5)
    assert e.at(5) == f32(1e-5) and e.at(4) < f32(3e-4)


def _state(p0, scale=S16, dynamic=True):
    n = p0.size
    return oracle.State(p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32),
                        np.zeros(n, np.uint16), oracle.Scaler(scale, 1.0, 1000, 1, dynamic=dynamic))


@pytest.mark.parametrize("kind", [oracle.LR_WARMUP, oracle.LR_WARMUP_DECAY])
def test_constant_gradient_closed_form_counts_applied_steps(oracle_lib, kind):
    """Constant g from m = v = 0: each applied step moves p by lr(it)*g/(|g|+eps) with it
    the number of steps applied before it; an overflowed step changes nothing and does
    not advance it."""
    rng = np.random.default_rng(11)
    n = 8192
    p0 = rng.normal(0, 0.02, n).astype(np.float32)
    g16 = (rng.normal(0, 1e-3, n) * S16).astype(np.float16).view(np.uint16)
    sched = oracle.LrSchedule(kind, 0.0, 1e-3, 4, 9)
    # a static scale keeps the unscaled gradient constant across the skips
    st = _state(p0, dynamic=False)
    # step 1 uses lr(0) = warmup_min_lr = 0: the moments move, the parameters do not
    assert not oracle.step(st, g16, lr=sched, beta1=B1, beta2=B2, eps=EPS)
    assert np.array_equal(f32_bits(st.master), f32_bits(p0)) and st.m.any()
    plan = [False, True, False, True, True, False, False, False, False, False, False]
    applied = 1
    for bad in plan:
        g = g16.copy()
        if bad:
            g[rng.integers(0, n)] = 0x7C00
        before = [a.copy() for a in (st.master, st.m, st.v, st.p16)]
        assert oracle.step(st, g, lr=sched, beta1=B1, beta2=B2, eps=EPS) == bad
        if bad:
            for a, b in zip(before, (st.master, st.m, st.v, st.p16)):
                assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
        else:
            applied += 1
    assert st.scaler.applied == applied == 9
    assert st.scaler.scale == S16
    g = g16.view(np.float16).astype(np.float64) / S16
    unit = g / (np.abs(g) + f32(EPS))
    moves, moves_iter = [], []
    it = 0
    for k, bad in enumerate([False] + plan):
        if not bad:
            moves.append(sched.at(it) * unit)
            moves_iter.append(sched.at(k) * unit)  # a schedule read at the all-steps count
            it += 1
    T = len(moves)
    bound = lambda total: T * ulp32(np.maximum(np.abs(p0), np.abs(st.master))) + 1e-5 * np.abs(total)
    total = np.sum(moves, axis=0)
    err = np.abs(st.master.astype(np.float64) - (p0.astype(np.float64) - total))
    assert np.all(err <= bound(total))
    total_iter = np.sum(moves_iter, axis=0)
    err_iter = np.abs(st.master.astype(np.float64) - (p0.astype(np.float64) - total_iter))
    assert np.mean(err_iter > bound(total_iter)) > 0.9


def test_matches_torch_lambda_lr(oracle_lib):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(12)
    n, T, W, total = 20000, 10, 3, 8
    max_lr = f32(3e-4)
    sched = oracle.LrSchedule(oracle.LR_WARMUP_DECAY, 0.0, max_lr, W, total)
    p0 = rng.normal(0, 0.02, n).astype(np.float32)
    st = _state(p0)
    param = torch.nn.Parameter(torch.from_numpy(p0.copy()))
    opt = torch.optim.Adam([param], lr=max_lr, betas=(f32(B1), f32(B2)), eps=f32(EPS), foreach=False)

    def gamma(it):
        return it / W if it < W else max(0.0, (total - it) / max(1, total - W))

    lam = torch.optim.lr_scheduler.LambdaLR(opt, gamma)
    for _ in range(T):
        g16 = (rng.normal(0, 1e-3, n) * S16).astype(np.float16).view(np.uint16)
        oracle.step(st, g16, lr=sched, beta1=B1, beta2=B2, eps=EPS)
        param.grad = torch.from_numpy(g16.view(np.float16).astype(np.float32) / np.float32(S16))
        opt.step()
        lam.step()
    ref = param.detach().numpy().astype(np.float64)
    move_ref, move = ref - p0, st.master.astype(np.float64) - p0
    assert np.abs(move_ref).max() > 3 * max_lr  # the schedule really moved the parameters
    assert np.all(np.abs(move - move_ref) <= 1e-6 * T * max_lr + 4 * ulp32(ref))
