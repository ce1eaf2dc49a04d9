"""Pins of the oracle's scaler and skip logic against torch's own loss scaler.

With one unit of hysteresis and a floor that never binds, the dynamic scaler
of "DeepSpeed complete guide" section 4.2 (halve on an overflow, double after
``loss_scale_window`` consecutive successes) is the rule of torch's
``GradScaler`` with backoff 0.5, growth 2 and growth interval W.  Torch
implements it independently (``torch._amp_update_scale_``, and
``GradScaler.step``, which unscales, looks for inf/NaN and leaves the
optimizer untouched on an overflow), so these tests pin:

  * the scale and success count after every step, over long random overflow
    patterns, for several windows;
  * the whole step loop (unscale, check, skip, Adam, scale update): the scale
    sequence, which steps were applied, Adam's step count (a skipped step does
    not advance the bias correction) and the parameters and moments, against
    ``GradScaler`` driving ``torch.optim.Adam`` on the CPU;
  * the static scale (``loss_scale`` > 0) against ``GradScaler`` held at a fixed
    scale: overflows still skip, the scale never moves.
"""
import numpy as np
import pytest

import oracle
from tests._fp import ulp32

torch = pytest.importorskip("torch")


@pytest.mark.parametrize("window,p_overflow,seed", [(1, 0.5, 1), (2, 0.3, 2), (3, 0.25, 3),
                                                     (7, 0.1, 4), (50, 0.01, 5)])
def test_scale_sequence_matches_torch_update_rule(oracle_lib, window, p_overflow, seed):
    rng = np.random.default_rng(seed)
    steps = 600
    overflow = rng.random(steps) < p_overflow
    init = 2.0 ** 20
    sc = oracle.Scaler(init, 2.0 ** -100, window, 1)
    t_scale = torch.tensor([init], dtype=torch.float32)
    t_growth = torch.zeros(1, dtype=torch.int32)
    halvings = growths = 0
    for s in range(steps):
        before = sc.scale
        sc.update(bool(overflow[s]))
        torch._amp_update_scale_(t_scale, t_growth, torch.tensor([float(overflow[s])]), 2.0, 0.5,
                                 window)
        assert sc.scale == t_scale.item(), f"step {s}"
        assert sc.s.good_steps == t_growth.item(), f"step {s}"
        halvings += sc.scale < before
        growths += sc.scale > before
    # the pattern exercised both directions, and the floor never took part
    assert halvings > 5 and growths > 5
    assert sc.s.skipped == int(overflow.sum()) and sc.applied == steps - int(overflow.sum())


@pytest.mark.parametrize("wd", [0.0, 0.01])
def test_step_loop_matches_torch_gradscaler_with_adam(oracle_lib, wd):
    rng = np.random.default_rng(11)
    n, T, window = 8192, 40, 5
    lr, b1, b2, eps = 1e-4, 0.9, 0.999, 1e-8
    mult = 2.0 ** 12            # the multiplier the synthetic gradients carry
    p0 = rng.normal(0, 0.02, n).astype(np.float32)
    st = oracle.State(p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32),
                      np.zeros(n, np.uint16), oracle.Scaler(mult, 1.0, window, 1))
    param = torch.nn.Parameter(torch.from_numpy(p0.copy()))
    f = lambda x: float(np.float32(x))
    cls = torch.optim.AdamW if wd else torch.optim.Adam
    opt = cls([param], lr=f(lr), betas=(f(b1), f(b2)), eps=f(eps), weight_decay=wd, foreach=False)
    gs = torch.amp.GradScaler("cpu", init_scale=mult, growth_factor=2.0, backoff_factor=0.5,
                              growth_interval=window)
    gs.scale(torch.ones(()))    # creates the scale tensor
    inject = {3: np.inf, 4: -np.inf, 17: np.nan, 26: np.inf}
    applied = 0
    for s in range(T):
        g = (rng.normal(0, 1e-3, n) * mult).astype(np.float16)
        if s in inject:
            g[rng.integers(0, n)] = inject[s]
        assert st.scaler.scale == gs.get_scale(), f"step {s}"
        ov = oracle.step(st, g.view(np.uint16), lr=lr, beta1=b1, beta2=b2, eps=eps,
                         weight_decay=wd)
        param.grad = torch.from_numpy(g.astype(np.float32))
        gs.step(opt)
        gs.update()
        assert ov == (s in inject)
        applied += not ov
        assert st.scaler.applied == applied == int(opt.state[param]["step"].item())
    assert st.scaler.scale == gs.get_scale()
    ref = param.detach().numpy()
    move_ref = ref.astype(np.float64) - p0
    move = st.master.astype(np.float64) - p0
    # the same bounds as the ten-step Adam comparison: rounding-order differences
    # stay far below 1e-6 of lr per step, a formula or skip mistake moves ~lr
    slack = (2 * T + 4) * ulp32(ref) if wd else 4 * ulp32(ref)
    assert np.all(np.abs(move - move_ref) <= 1e-6 * T * lr + slack)
    assert np.allclose(st.m, opt.state[param]["exp_avg"].numpy(), rtol=1e-5, atol=1e-10)
    assert np.allclose(st.v, opt.state[param]["exp_avg_sq"].numpy(), rtol=1e-5, atol=1e-15)


def test_planted_skip_mistake_is_caught(oracle_lib):
    """A step that applied Adam on an overflow (NaN moments) or advanced t on a
    skip would differ from torch by far more than the bounds above; check the
    bound separates them: one extra applied step moves parameters by ~lr."""
    rng = np.random.default_rng(12)
    n, lr = 4096, 1e-4
    p0 = rng.normal(0, 0.02, n).astype(np.float32)
    g = (rng.normal(0, 1e-3, n) * 2.0 ** 12).astype(np.float16).view(np.uint16)
    a = oracle.State(p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32),
                     np.zeros(n, np.uint16), oracle.Scaler(2.0 ** 12, 1.0, 5, 1))
    b = oracle.State(p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32),
                     np.zeros(n, np.uint16), oracle.Scaler(2.0 ** 12, 1.0, 5, 1))
    oracle.step(a, g, lr=lr, beta1=0.9, beta2=0.999, eps=1e-8)
    oracle.step(b, g, lr=lr, beta1=0.9, beta2=0.999, eps=1e-8)
    oracle.step(b, g, lr=lr, beta1=0.9, beta2=0.999, eps=1e-8)
    gap = np.abs(a.master.astype(np.float64) - b.master)
    assert np.median(gap) > 0.5 * lr > 1e-6 * 40 * lr + 4 * float(np.max(ulp32(a.master)))


def test_static_scale_matches_gradscaler_with_a_fixed_scale(oracle_lib):
    """loss_scale > 0 ("DeepSpeed complete guide" section 4.2: 0 selects dynamic
    scaling, so a positive value is a fixed scale): torch's GradScaler pinned to
    that scale after every step (update(new_scale=S)) still skips the optimizer on
    inf/NaN.  The oracle's static mode matches it: the same skipped steps, the
    same Adam step count, the scale never moves, parameters within the Adam bounds."""
    rng = np.random.default_rng(13)
    n, T, S = 4096, 24, 2.0 ** 10
    lr, b1, b2, eps = 1e-4, 0.9, 0.999, 1e-8
    p0 = rng.normal(0, 0.02, n).astype(np.float32)
    st = oracle.State(p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16),
                      oracle.Scaler(S, 1.0, 2, 1, dynamic=False))
    param = torch.nn.Parameter(torch.from_numpy(p0.copy()))
    f = lambda x: float(np.float32(x))
    opt = torch.optim.Adam([param], lr=f(lr), betas=(f(b1), f(b2)), eps=f(eps), foreach=False)
    gs = torch.amp.GradScaler("cpu", init_scale=S, growth_interval=2)
    gs.scale(torch.ones(()))
    inject = {1: np.inf, 2: np.nan, 3: -np.inf, 9: np.inf}
    for s in range(T):
        g = (rng.normal(0, 1e-3, n) * S).astype(np.float16)
        if s in inject:
            g[rng.integers(0, n)] = inject[s]
        ov = oracle.step(st, g.view(np.uint16), lr=lr, beta1=b1, beta2=b2, eps=eps)
        param.grad = torch.from_numpy(g.astype(np.float32))
        gs.step(opt)
        gs.update(new_scale=S)
        assert ov == (s in inject) and st.scaler.scale == S == gs.get_scale()
        assert st.scaler.applied == int(opt.state[param]["step"].item())
    assert st.scaler.applied == T - len(inject) and st.scaler.s.skipped == len(inject)
    ref = param.detach().numpy()
    assert np.all(np.abs((st.master.astype(np.float64) - p0) - (ref.astype(np.float64) - p0))
                  <= 1e-6 * T * lr + 4 * ulp32(ref))
