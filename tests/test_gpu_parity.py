"""GPU parity: the HIP path (through the C ABI) against the CPU oracle,
element by element, at sizes the oracle finishes in seconds.

Bar: overflow flags, skip decisions and the loss-scale sequence bit-exact;
fp32 master/m/v within 4 ulp; fp16 parameters within 1 ulp.  The max ulp
distance seen is printed (the design target is 0).
"""
import os

import numpy as np
import pytest

import oracle
import synth
from synth.workloads import BETA1, BETA2, EPS, LR, MASTER_SIGMA, WORKLOADS
from tests import gpu_util as gu
from tests._fp import f32_bits

pytestmark = pytest.mark.gpu

HP = dict(lr=LR, beta1=BETA1, beta2=BETA2, eps=EPS)


@pytest.fixture(scope="module")
def torch():
    t = gu.torch_mod()
    import zero_mixed_precision_amd  # noqa: F401  (fails loudly if libdszero.so is missing)
    return t


def _init_host(n, seed, sigma=MASTER_SIGMA):
    idx = np.arange(n)
    master = synth.host_master32(synth.stream_key(seed, synth.ARR_MASTER), idx, sigma)
    p16 = synth.host_grad16(synth.stream_key(seed, synth.ARR_P16), idx, synth.GradSpec(0.02, 1.0))
    return master, np.zeros(n, np.float32), np.zeros(n, np.float32), p16


def _pair(torch, n, seed, *, init_scale=2.0 ** 16, window=1000, K=1, hysteresis=1):
    master, m, v, p16 = _init_host(n, seed)
    o = oracle.State(master.copy(), m.copy(), v.copy(), p16.copy(),
                     oracle.Scaler(init_scale, 1.0, window, hysteresis))
    d = gu.DevState(torch, master, m, v, p16, init_scale=init_scale, window=window, K=K,
                    hysteresis=hysteresis)
    return o, d


def _mixed_grads(seed, n, spec):
    """Workload-like draws, with every finite fp16 pattern class mixed in."""
    g = synth.host_grad16(synth.stream_key(seed, synth.ARR_GRAD), np.arange(n), spec)
    rng = np.random.default_rng(seed)
    pick = rng.random(n) < 0.25
    pat = rng.integers(0, 65536, n).astype(np.uint16)
    pat = np.where((pat & 0x7C00) == 0x7C00, pat & 0x83FF, pat).astype(np.uint16)
    return np.where(pick, pat, g).astype(np.uint16)


# -- the tiny workload, every array compared after every step -----------------------

def test_tiny_workload_ten_steps_full_compare(torch):
    w = WORKLOADS["tiny"]
    n = w.psi
    idx = np.arange(n)
    master = synth.host_master32(w.master_key(), idx, MASTER_SIGMA)
    p16 = synth.host_grad16(w.p16_key(), idx, synth.GradSpec(0.02, 1.0))
    zeros = np.zeros(n, np.float32)
    o = oracle.State(master.copy(), zeros.copy(), zeros.copy(), p16.copy(),
                     oracle.Scaler(w.init_scale, w.min_scale, w.window, w.hysteresis))
    d = gu.DevState(torch, master, zeros, zeros, p16, init_scale=w.init_scale, window=w.window)
    worst = {}
    for s in range(1, w.steps + 1):
        g = synth.host_grad16(w.grad_key(s), idx, w.grad_spec)
        inj = w.injection(s)
        if inj is not None:
            g[inj[1]] = 0x7C00
        ov = oracle.step(o, g, **HP)
        assert ov == (inj is not None)
        d.step(gu.dev_u16(torch, g), HP)
        gu.check_scaler(d.scaler(), o.scaler, ov, f"tiny step {s}")
        du = gu.compare_full(f"tiny step {s}", d, o)
        worst = {k: max(worst.get(k, 0), x) for k, x in du.items()}
    gu.say("tiny workload: max ulp", worst)
    assert o.scaler.applied == 9 and o.scaler.scale == 2.0 ** 15


# -- ragged sizes, tails, both gradient dtypes ----------------------------------------

SIZES = list(range(1, 18)) + [63, 64, 65, 1023, 4097, 65536 + 7, (1 << 20) + 3, 3 * (1 << 18) + 5]


@pytest.mark.parametrize("n", SIZES)
def test_ragged_sizes_fp16_gradient(torch, n):
    o, d = _pair(torch, n, seed=1000 + n)
    spec = synth.GradSpec(1e-3, 2.0 ** 16)
    for s in range(3):
        g = _mixed_grads(7000 + 31 * n + s, n, spec)
        ov = oracle.step(o, g, **HP)
        d.step(gu.dev_u16(torch, g), HP)
        gu.check_scaler(d.scaler(), o.scaler, ov, f"n={n} step {s}")
        gu.compare_full(f"n={n} step {s}", d, o)


@pytest.mark.parametrize("n", [1, 3, 4, 5, 8, 17, 1023, 4097, (1 << 20) + 3])
@pytest.mark.parametrize("K", [2, 3, 8])
def test_ragged_sizes_accumulated_gradient(torch, n, K):
    o, d = _pair(torch, n, seed=2000 + n, init_scale=2.0 ** 15, window=2, K=K)
    spec = synth.GradSpec(1e-3, 2.0 ** 15)
    for s in range(3):
        gs = [_mixed_grads(9000 + 17 * n + 5 * s + k, n, spec) for k in range(K)]
        ov = oracle.step(o, gs, **HP)
        d.step([gu.dev_u16(torch, g) for g in gs], HP)
        gu.check_scaler(d.scaler(), o.scaler, ov, f"n={n} K={K} step {s}")
        gu.compare_full(f"n={n} K={K} step {s}", d, o)


def test_accumulate_buffer_bits_and_bucketed_calls(torch):
    """The fp32 accumulation buffer itself, built from bucketed sub-range calls."""
    from zero_mixed_precision_amd import _lib
    n, K = 100_003, 8
    spans = [(0, 40_000), (40_000, 24), (40_024, 60_000 - 24), (100_000, 3)]
    spec = synth.GradSpec(1e-3, 2.0 ** 15)
    gs = [_mixed_grads(50 + k, n, spec) for k in range(K)]
    gs[5][12] = 0x8000                       # -0
    acc_o = np.empty(n, np.float32)
    for k, g in enumerate(gs):
        oracle.accumulate(acc_o, g, overwrite=(k == 0))
    acc = torch.full((n,), 7.0, device="cuda:0")
    st = torch.zeros(_lib.ds_scaler_size(), dtype=torch.uint8, device="cuda:0")
    _lib.ds_state_init(st, 1.0, 1.0, 1, 1, 0, 1)
    for k, g in enumerate(gs):
        gd = gu.dev_u16(torch, g)
        for start, size in spans:
            _lib.ds_accumulate(acc.data_ptr() + 4 * start, gd.data_ptr() + 2 * start, _lib.DS_FP16, size, k == 0,
                               st if k == K - 1 else None)
    got = gu.host_f32(acc)
    assert np.array_equal(f32_bits(got), f32_bits(acc_o))
    assert not _lib.ds_state_read(st).overflow


# -- overflow: every special pattern at first / middle / last / tail positions -------

SPECIALS = {"+inf": 0x7C00, "-inf": 0xFC00, "qnan": 0x7E00, "snan": 0x7C01, "nan_payload": 0xFE5A}


@pytest.mark.parametrize("n", [37, 4096 + 7])
@pytest.mark.parametrize("name", sorted(SPECIALS))
def test_overflow_skips_bit_identically(torch, n, name):
    spec = synth.GradSpec(1e-3, 2.0 ** 16)
    for pos in (0, n // 2, n - 8, n - 1):
        o, d = _pair(torch, n, seed=3000 + pos)
        g0 = _mixed_grads(11 + pos, n, spec)
        oracle.step(o, g0, **HP)
        d.step(gu.dev_u16(torch, g0), HP)
        before = [gu.host_f32(d.master), gu.host_f32(d.m), gu.host_f32(d.v), gu.host_u16(d.p16)]
        g = _mixed_grads(12 + pos, n, spec)
        g[pos] = SPECIALS[name]
        assert oracle.step(o, g, **HP)
        d.step(gu.dev_u16(torch, g), HP)
        sc = d.scaler()
        gu.check_scaler(sc, o.scaler, True, f"{name} at {pos}")
        assert sc.scale == 2.0 ** 15 and sc.step == 1 and sc.skipped == 1
        after = [gu.host_f32(d.master), gu.host_f32(d.m), gu.host_f32(d.v), gu.host_u16(d.p16)]
        for a, b in zip(before, after):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"{name} at {pos}: state moved"


@pytest.mark.parametrize("h", [0x7BFF, 0xFBFF, 0x0001, 0x8001, 0x03FF, 0x8000, 0x0400])
def test_large_finite_and_subnormal_gradients_are_applied(torch, h):
    n = 4096 + 5
    spec = synth.GradSpec(1e-3, 2.0 ** 16)
    o, d = _pair(torch, n, seed=4000 + h)
    g = _mixed_grads(13 + h, n, spec)
    for pos in (0, 1000, n - 1):
        g[pos] = h
    assert not oracle.step(o, g, **HP)
    d.step(gu.dev_u16(torch, g), HP)
    gu.check_scaler(d.scaler(), o.scaler, False, hex(h))
    gu.compare_full(hex(h), d, o)


@pytest.mark.parametrize("n", [5, 4 * 1024 + 3, (1 << 20) + 1])
def test_fp32_overflow_check(torch, n):
    from zero_mixed_precision_amd import _lib
    rng = np.random.default_rng(n)
    base = rng.normal(0, 1, n).astype(np.float32)
    st = torch.zeros(_lib.ds_scaler_size(), dtype=torch.uint8, device="cuda:0")
    for pos in (0, n // 2, n - 1):
        for bits in (0x7F800000, 0xFF800000, 0x7FC00000, 0x7F800001, 0x7F7FFFFF, 0x00000001):
            a = base.copy()
            a.view(np.uint32)[pos] = bits
            _lib.ds_state_init(st, 1.0, 1.0, 1, 1, 0, 1)
            _lib.ds_check_overflow(st, gu.dev_f32(torch, a), _lib.DS_FP32, n)
            assert bool(_lib.ds_state_read(st).overflow) == oracle.any_nonfinite(a), (pos, hex(bits))


def test_fp16_overflow_check_all_patterns(torch):
    """Every fp16 pattern, each alone in a ragged array of finite values."""
    from zero_mixed_precision_amd import _lib
    n, stride, rows = 1027, 1032, 4096          # rows start 16-byte aligned (stride % 8 == 0)
    base = _mixed_grads(77, n, synth.GradSpec(1e-3, 2.0 ** 16))
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = np.zeros(pats.size, bool)
    want = np.zeros(pats.size, bool)
    for c0 in range(0, pats.size, rows):
        chunk = pats[c0:c0 + rows]
        a = np.zeros((chunk.size, stride), np.uint16)
        a[:, :n] = base
        pos = (np.arange(chunk.size) * 97) % n
        a[np.arange(chunk.size), pos] = chunk
        da = gu.dev_u16(torch, a.reshape(-1))
        states = torch.zeros((chunk.size, _lib.ds_scaler_size()), dtype=torch.uint8, device="cuda:0")
        for j in range(chunk.size):
            _lib.ds_check_overflow(states[j].data_ptr(), da.data_ptr() + 2 * stride * j, _lib.DS_FP16, n)
        got[c0:c0 + chunk.size] = states.cpu().numpy()[:, 28:32].copy().view(np.uint32)[:, 0] != 0
        want[c0:c0 + chunk.size] = [oracle.any_nonfinite(a[j, :n]) for j in range(chunk.size)]
    assert np.array_equal(got, want)
    assert want.sum() == 2048                     # 2 signs x 1024 fractions with exponent 31


# -- launch-shape invariance and determinism ---------------------------------------

def _run_variant(torch, n, env):
    old = {k: os.environ.get(k) for k in env}
    os.environ.update(env)
    try:
        o, d = _pair(torch, n, seed=5000)
        spec = synth.GradSpec(1e-3, 2.0 ** 16)
        for s in range(2):
            g = _mixed_grads(5100 + s, n, spec)
            d.step(gu.dev_u16(torch, g), HP)
        torch.cuda.synchronize()
        return [gu.host_f32(d.master), gu.host_f32(d.m), gu.host_f32(d.v), gu.host_u16(d.p16)]
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def test_grid_size_and_variant_invariance(torch):
    n = (1 << 20) + 3
    ref = _run_variant(torch, n, {})
    for env in [{"DSZERO_GRID": "1"}, {"DSZERO_GRID": "7"}, {"DSZERO_GRID": "100000"},
                {"DSZERO_UNROLL": "2"}, {"DSZERO_NT": "0"}, {"DSZERO_NT": "1"},
                {"DSZERO_UNROLL": "2", "DSZERO_GRID": "3", "DSZERO_NT": "1"},
                {}]:
        got = _run_variant(torch, n, env)
        for a, b in zip(ref, got):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), env


def test_snapshot_resume_is_bit_identical(torch):
    from zero_mixed_precision_amd import _lib
    n = 300_007
    spec = synth.GradSpec(1e-3, 2.0 ** 16)
    grads = [_mixed_grads(6000 + s, n, spec) for s in range(10)]
    grads[6][5] = 0x7C00
    o, d = _pair(torch, n, seed=6100, window=3)
    for g in grads[:5]:
        d.step(gu.dev_u16(torch, g), HP)
    snap_sc = d.scaler()
    snap = [d.master.clone(), d.m.clone(), d.v.clone(), d.p16.clone()]
    for g in grads[5:]:
        d.step(gu.dev_u16(torch, g), HP)
    full = [gu.host_f32(d.master), gu.host_f32(d.m), gu.host_f32(d.v), gu.host_u16(d.p16)]
    full_sc = d.scaler()
    # resume from the snapshot into fresh buffers and a fresh state
    _, r = _pair(torch, n, seed=6200, window=3)
    r.master.copy_(snap[0]); r.m.copy_(snap[1]); r.v.copy_(snap[2]); r.p16.copy_(snap[3])
    _lib.ds_state_write(r.state, snap_sc)
    for g in grads[5:]:
        r.step(gu.dev_u16(torch, g), HP)
    res = [gu.host_f32(r.master), gu.host_f32(r.m), gu.host_f32(r.v), gu.host_u16(r.p16)]
    for a, b in zip(full, res):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    assert r.scaler().as_dict() == full_sc.as_dict()
    # and the whole run matches the oracle
    for g in grads:
        oracle.step(o, g, **HP)
    gu.compare_arrays("resume", *full, o.master, o.m, o.v, o.p16)


# -- per-step scalars, weight decay, static scale ---------------------------------------

def test_bias_correction_scalars_bit_exact(torch):
    from zero_mixed_precision_amd import _lib
    ts = list(range(1, 3001)) + sorted({int(x) for x in np.logspace(3.5, 8, 150)})
    hps = [(1e-4, 0.9, 0.999), (3e-4, 0.95, 0.98), (1e-3, 0.5, 0.9999)]
    st = torch.zeros(_lib.ds_scaler_size(), dtype=torch.uint8, device="cuda:0")
    out = torch.zeros((len(hps), len(ts), 2), dtype=torch.float32, device="cuda:0")
    _lib.ds_state_init(st, 1.0, 1.0, 1, 1, 0, 1)
    base = _lib.ds_state_read(st)
    for a, (lr, b1, b2) in enumerate(hps):
        for j, t in enumerate(ts):
            base.step = t - 1
            _lib.ds_state_write(st, base)
            _lib.ds_adam_bias_scalars(st, lr, b1, b2, out[a, j].data_ptr())
    got = out.cpu().numpy()
    for a, (lr, b1, b2) in enumerate(hps):
        want = np.array([oracle.adam_scalars(t, lr, b1, b2) for t in ts], np.float32)
        assert np.array_equal(f32_bits(got[a]), f32_bits(want)), (lr, b1, b2)


def test_bias_correction_scalars_for_every_step_to_a_million(torch):
    """The device's per-step factors lr/(1-beta1^t) and 1/sqrt(1-beta2^t) (fp64,
    rounded once) equal the oracle's bit for bit for every applied step t =
    1..10^6, for three hyperparameter sets: this guards the lowering of the
    fp64 divide and square root.  The applied-step count advances on the
    device by one successful scaler update per t (static scale, no host
    round trip), and each t's pair is written to its own slot."""
    import ctypes

    from zero_mixed_precision_amd import _lib
    T = 10 ** 6
    hps = [(1e-4, 0.9, 0.999), (3e-4, 0.95, 0.98), (1e-3, 0.5, 0.9999)]
    L = _lib.lib
    out = torch.zeros((T, 2), dtype=torch.float32, device="cuda:0")
    st = torch.zeros(_lib.ds_scaler_size(), dtype=torch.uint8, device="cuda:0")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st_p, base = ctypes.c_void_p(st.data_ptr()), out.data_ptr()
    bias, update = L.ds_adam_bias_scalars, L.ds_update_loss_scale
    for lr, b1, b2 in hps:
        gu.say(f"[bias scalars] lr={lr} betas=({b1}, {b2}) t=1..{T}")
        _lib.ds_state_init(st, 1.0, 1.0, 1, 1, 0, 0)           # static scale: updates only advance t
        flr, fb1, fb2 = ctypes.c_float(lr), ctypes.c_float(b1), ctypes.c_float(b2)
        for j in range(T):
            if bias(st_p, flr, fb1, fb2, ctypes.c_void_p(base + 8 * j), stream) != 0 or update(st_p, stream) != 0:
                raise AssertionError(f"launch failed at t={j + 1}")
        got = out.cpu().numpy()
        assert _lib.ds_state_read(st).step == T
        want = oracle.adam_scalars_range(1, T, lr, b1, b2)
        bad = np.nonzero(f32_bits(got).ravel() != f32_bits(want).ravel())[0]
        assert bad.size == 0, (lr, b1, b2, "first differing t", int(bad[0] // 2) + 1)


@pytest.mark.parametrize("wd", [0.01, 0.1])
def test_weight_decay(torch, wd):
    n = 65536 + 9
    o, d = _pair(torch, n, seed=7000)
    spec = synth.GradSpec(1e-3, 2.0 ** 16)
    hp = dict(HP, weight_decay=wd)
    for s in range(4):
        g = _mixed_grads(7100 + s, n, spec)
        ov = oracle.step(o, g, **hp)
        d.step(gu.dev_u16(torch, g), hp)
        gu.check_scaler(d.scaler(), o.scaler, ov, f"wd step {s}")
        gu.compare_full(f"wd={wd} step {s}", d, o)


# lr, beta1, beta2, eps, weight decay at the edges of what the boundary accepts
DEGENERATE = {
    "lr_zero": (0.0, 0.9, 0.999, 1e-8, 0.0),            # moments move, parameters stay
    "lr_zero_with_decay": (0.0, 0.9, 0.999, 1e-8, 0.1),  # lr*wd = 0: the decay is an exact no-op
    "no_moment_memory": (1e-4, 0.0, 0.0, 1e-8, 0.0),    # m = g, v = g*g, both factors exactly 1
    "betas_one_half": (1e-4, 0.5, 0.5, 1e-8, 0.0),      # the Sterbenz edge of 1 - beta
    "betas_near_one": (1e-4, 0.99999994, 0.99999994, 1e-8, 0.0),  # the largest fp32 below 1
    "large_lr_and_eps": (1.0, 0.9, 0.999, 1.0, 0.0),
    "tiny_eps": (1e-4, 0.9, 0.999, 1e-30, 0.0),
    "subnormal_eps": (1e-4, 0.9, 0.999, 1e-40, 0.0),
    "large_decay": (1e-2, 0.9, 0.999, 1e-8, 10.0),      # lr*wd = 0.1
}


@pytest.mark.parametrize("name", sorted(DEGENERATE))
def test_degenerate_hyperparameters(torch, name):
    lr, b1, b2, eps, wd = DEGENERATE[name]
    n = 4096 * 3 + 5
    o, d = _pair(torch, n, seed=7500)
    spec = synth.GradSpec(1e-3, 2.0 ** 16)
    hp = dict(lr=lr, beta1=b1, beta2=b2, eps=eps, weight_decay=wd)
    for s in range(5):
        g = _mixed_grads(7600 + s, n, spec)
        if s == 2:
            g[n - 1] = 0x7C00
        ov = oracle.step(o, g, **hp)
        d.step(gu.dev_u16(torch, g), hp)
        gu.check_scaler(d.scaler(), o.scaler, ov, f"{name} step {s}")
        du = gu.compare_full(f"{name} step {s}", d, o)
        # both sides evaluate the same operations in the same order: no ulp apart
        assert max(du.values()) == 0, f"{name} step {s}: {du}"
    if lr == 0.0:
        master, _, _, p16 = _init_host(n, 7500)
        assert np.array_equal(f32_bits(o.master), f32_bits(master))


@pytest.mark.parametrize("t0", [10 ** 4, 10 ** 7, 2 ** 40])
def test_bias_correction_late_in_training(torch, t0):
    """Resumed at a large applied-step count: beta^t underflows to 0 and both
    factors become exactly lr and 1; the update is then plain lr*m/(sqrt(v)+eps)."""
    n = 4096 + 3
    o, d = _pair(torch, n, seed=7700)
    sc = d.scaler()
    sc.step = t0
    d.lib.ds_state_write(d.state, sc)
    o.scaler.s.applied = t0
    spec = synth.GradSpec(1e-3, 2.0 ** 16)
    for s in range(3):
        g = _mixed_grads(7800 + s, n, spec)
        ov = oracle.step(o, g, **HP)
        d.step(gu.dev_u16(torch, g), HP)
        gu.check_scaler(d.scaler(), o.scaler, ov, f"t0={t0} step {s}")
        du = gu.compare_full(f"t0={t0} step {s}", d, o)
        assert max(du.values()) == 0, f"t0={t0} step {s}: {du}"
    assert d.scaler().step == t0 + 3


def test_static_scale_and_hysteresis_two(torch):
    """Unexercised by the workloads; the device state machine still tracks the oracle's."""
    n = 1000
    spec = synth.GradSpec(1e-3, 2.0 ** 10)
    for dynamic, hyst in ((0, 1), (1, 2), (1, 3)):
        master, m, v, p16 = _init_host(n, 8000)
        o = oracle.State(master.copy(), m.copy(), v.copy(), p16.copy(),
                         oracle.Scaler(1024.0, 1.0, 2, hyst, dynamic=bool(dynamic)))
        d = gu.DevState(torch, master, m, v, p16, init_scale=1024.0, window=2, hysteresis=hyst,
                        dynamic=dynamic)
        for s in range(12):
            g = _mixed_grads(8100 + s, n, spec)
            if s in (1, 2, 3, 7):
                g[s] = 0x7C00
            ov = oracle.step(o, g, **HP)
            d.step(gu.dev_u16(torch, g), HP)
            gu.check_scaler(d.scaler(), o.scaler, ov, f"dyn={dynamic} H={hyst} step {s}")
        gu.compare_full(f"dyn={dynamic} H={hyst}", d, o)


def test_loss_scale_floor_below_powers_of_two(torch):
    """The guide's overflow-debugging floor (min_loss_scale 1e-8, hysteresis 2): after
    enough overflows the scale is fp32(1e-8), not a power of two, so the unscale
    multiplier 1/S is rounded; the device must round it as the oracle does."""
    n = 4099
    spec = synth.GradSpec(1e-3, 1.0)
    for window in (500, 2):
        master, m, v, p16 = _init_host(n, 8200)
        o = oracle.State(master.copy(), m.copy(), v.copy(), p16.copy(), oracle.Scaler(4096.0, 1e-8, window, 2))
        d = gu.DevState(torch, master, m, v, p16, init_scale=4096.0, window=window, hysteresis=2,
                        min_scale=1e-8)
        for s in range(86):
            g = _mixed_grads(8300 + s, n, spec)
            if s < 80:
                g[(s * 31) % n] = 0x7C00 if s % 2 else 0xFE00
            ov = oracle.step(o, g, **HP)
            d.step(gu.dev_u16(torch, g), HP)
            gu.check_scaler(d.scaler(), o.scaler, ov, f"floor W={window} step {s}")
        assert o.scaler.scale == (float(np.float32(1e-8)) * (8 if window == 2 else 1))
        gu.compare_full(f"floor W={window}", d, o)


@pytest.mark.parametrize("dynamic,hyst,consec,window", [(1, 1, 0, 3), (1, 2, 0, 4), (1, 3, 1, 2), (1, 2, 1, 5),
                                                         (0, 2, 0, 3)])
def test_scaler_state_machine_random_overflows(torch, dynamic, hyst, consec, window):
    """300 steps with random overflows (probability 0.3, runs of both kinds): the
    device's scaler follows the oracle's after every step, in every mode."""
    n = 40
    rng = np.random.default_rng(100 * hyst + 10 * consec + window + dynamic)
    master, m, v, p16 = _init_host(n, 8400)
    o = oracle.State(master.copy(), m.copy(), v.copy(), p16.copy(),
                     oracle.Scaler(2.0 ** 20, 4.0, window, hyst, dynamic=bool(dynamic),
                                   consecutive_hysteresis=bool(consec)))
    d = gu.DevState(torch, master, m, v, p16, init_scale=2.0 ** 20, window=window, hysteresis=hyst,
                    min_scale=4.0, dynamic=dynamic, consecutive_hysteresis=consec)
    spec = synth.GradSpec(1e-3, 2.0 ** 10)
    scales = set()
    for s in range(300):
        g = _mixed_grads(8500 + s, n, spec)
        if rng.random() < 0.3:
            g[rng.integers(0, n)] = rng.choice([0x7C00, 0xFC00, 0x7E00, 0xFD55])
        ov = oracle.step(o, g, **HP)
        d.step(gu.dev_u16(torch, g), HP)
        gu.check_scaler(d.scaler(), o.scaler, ov, f"dyn={dynamic} H={hyst} c={consec} W={window} step {s}")
        scales.add(o.scaler.scale)
    gu.compare_full(f"random overflows dyn={dynamic} H={hyst}", d, o)
    assert len(scales) >= (3 if dynamic else 1)


def _wild_f32(rng, n, nonneg=False):
    """fp32 values from every class: raw random bit patterns (every exponent,
    including inf and NaN), zeros and subnormals, values near the largest
    finite, and ordinary N(0, 0.02) values."""
    raw = rng.integers(0, 2 ** 32, n, dtype=np.uint64).astype(np.uint32)
    cls = rng.integers(0, 16, n)
    sign = raw & np.uint32(0x80000000)
    bits = raw.copy()                                                                    # 0..3: raw
    bits = np.where((cls >= 4) & (cls < 7), raw & np.uint32(0x807FFFFF), bits)            # 0 / subnormal
    bits = np.where((cls >= 7) & (cls < 9), (raw & np.uint32(0x80FFFFFF)) | np.uint32(0x7E000000), bits)
    bits = np.where(cls == 9, sign | np.uint32(0x7F800000), bits)                         # +-inf
    bits = np.where(cls == 10, raw | np.uint32(0x7FC00000), bits)                         # NaN
    normal = rng.normal(0, 0.02, n).astype(np.float32).view(np.uint32)
    bits = np.where(cls >= 11, normal, bits)
    if nonneg:
        bits = bits & np.uint32(0x7FFFFFFF)
    return bits.view(np.float32)


@pytest.mark.parametrize("scale,K,wd,pfmt", [(2.0 ** 16, 1, 0.0, "fp16"), (3000.0, 1, 0.1, "bf16"),
                                             (float(np.float32(1e-8)), 3, 0.0, "fp16"),
                                             (12345.0, 2, 0.01, "fp16")])
def test_adam_over_every_fp32_class(torch, scale, K, wd, pfmt):
    """Adam on master/m/v drawn from every fp32 class, gradients from every finite 16-bit
    class, scales that are not powers of two: the device's IEEE arithmetic (no flush to
    zero, correctly rounded divide and square root, infinities and NaNs propagated)
    matches the oracle's over the whole range (any NaN matches any NaN)."""
    rng = np.random.default_rng(int(scale) + 7 * K)
    n = 3 * 4096 + 77
    master, m = _wild_f32(rng, n), _wild_f32(rng, n)
    v = _wild_f32(rng, n, nonneg=True)
    v[:64] = -v[:64]                                     # a few negative second moments: sqrt -> NaN
    p16 = np.zeros(n, np.uint16)
    o = oracle.State(master.copy(), m.copy(), v.copy(), p16.copy(),
                     oracle.Scaler(scale, float(np.float32(1e-8)), 1000, 1), param_fmt=pfmt)
    d = gu.DevState(torch, master, m, v, p16, init_scale=scale, window=1000, min_scale=float(np.float32(1e-8)),
                    K=K, param_fmt=pfmt)
    hp = dict(HP, weight_decay=wd)
    for s in range(3):
        gs = []
        for k in range(K):
            h = rng.integers(0, 65536, n).astype(np.uint16)
            gs.append(np.where((h & 0x7C00) == 0x7C00, h & 0x83FF, h).astype(np.uint16))
        ov = oracle.step(o, gs if K > 1 else gs[0], **hp)
        assert not ov
        d.step([gu.dev_u16(torch, g) for g in gs] if K > 1 else gu.dev_u16(torch, gs[0]), hp)
        gu.check_scaler(d.scaler(), o.scaler, ov, f"wild step {s}")
        du = gu.compare_full(f"wild scale={scale} K={K} wd={wd} {pfmt} step {s}", d, o)
        gu.say(f"wild scale={scale} K={K} wd={wd} {pfmt} step {s}: max ulp {du}, "
               f"nan share {np.isnan(o.master).mean():.3f}")


@pytest.mark.parametrize("n,K,grid", [(1_000_003, 1, None), (1_000_003, 1, "1"), (300_001, 3, "7"),
                                      (300_001, 1, "100000"), (4096 * 4, 2, None), (5, 1, None)])
def test_fused_step_matches_separate_calls(torch, n, K, grid):
    """ds_adam_step_fused (Adam plus the scaler update in one kernel, the last block
    to finish advancing the scaler) against ds_adam_step + ds_update_loss_scale and the
    oracle, bit for bit, through overflowed steps and forced grids (one block; more
    blocks than tiles, so that blocks with no tile still count themselves)."""
    from zero_mixed_precision_amd import _lib
    env = {"DSZERO_GRID": grid} if grid else {}
    master, m, v, p16 = _init_host(n, 8600)
    o = oracle.State(master.copy(), m.copy(), v.copy(), p16.copy(), oracle.Scaler(4096.0, 1.0, 2, 1))
    sep = gu.DevState(torch, master, m, v, p16, init_scale=4096.0, window=2, K=K)
    fus = gu.DevState(torch, master, m, v, p16, init_scale=4096.0, window=2, K=K)
    spec = synth.GradSpec(1e-3, 4096.0)
    old = {k: os.environ.get(k) for k in env}
    os.environ.update(env)
    try:
        for s in range(8):
            gs = [_mixed_grads(8700 + 10 * s + k, n, spec) for k in range(K)]
            if s in (2, 5):
                gs[-1][(s * 131) % n] = 0x7C00
            ov = oracle.step(o, gs if K > 1 else gs[0], **HP)
            dg = [gu.dev_u16(torch, g) for g in gs]
            sep.step(dg if K > 1 else dg[0], HP)
            # the same sequence with the fused entry point
            if K == 1:
                _lib.ds_check_overflow(fus.state, dg[0], _lib.DS_FP16, n)
                grad, dt = dg[0], _lib.DS_FP16
            else:
                for k, g in enumerate(dg):
                    _lib.ds_accumulate(fus.acc, g, _lib.DS_FP16, n, k == 0, fus.state if k == K - 1 else None)
                grad, dt = fus.acc, _lib.DS_FP32
            _lib.ds_adam_step_fused(fus.state, fus.master, fus.m, fus.v, fus.p16, _lib.DS_FP16, grad, dt, n,
                                    HP["lr"], None, HP["beta1"], HP["beta2"], HP["eps"], 0.0, 0.0, K)
            sc = fus.scaler()
            gu.check_scaler(sc, o.scaler, ov, f"fused n={n} K={K} grid={grid} step {s}")
            assert sc.blocks_done == 0
            assert sc.as_dict() == sep.scaler().as_dict()
    finally:
        for k, val in old.items():
            if val is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = val
    for a, b in ((sep.master, fus.master), (sep.m, fus.m), (sep.v, fus.v), (sep.p16, fus.p16)):
        assert np.array_equal(a.cpu().numpy().view(np.uint8), b.cpu().numpy().view(np.uint8))
    gu.compare_full(f"fused n={n} K={K}", fus, o)


def test_fused_step_on_an_empty_partition_advances_the_scaler(torch):
    from zero_mixed_precision_amd import _lib
    st = torch.zeros(_lib.ds_scaler_size(), dtype=torch.uint8, device="cuda:0")
    _lib.ds_state_init(st, 1024.0, 1.0, 2, 1, 0, 1)
    for _ in range(2):
        _lib.ds_adam_step_fused(st, 0, 0, 0, 0, _lib.DS_FP16, 0, _lib.DS_FP16, 0, 1e-4, None, 0.9, 0.999, 1e-8,
                                0.0, 0.0, 1)
    sc = _lib.ds_state_read(st)
    assert sc.step == 2 and sc.iter == 2 and sc.scale == 2048.0


# -- the fp16 cast over every fp32 pattern ----------------------------------------------

def _enc16_parallel(pool, x, parts=8):
    out = np.empty(x.size, np.uint16)
    step = -(-x.size // parts)

    def work(k):
        out[k * step:(k + 1) * step] = oracle.enc16(x[k * step:(k + 1) * step])

    list(pool.map(work, range(parts)))
    return out


def test_fp16_cast_of_every_fp32_pattern(torch):
    """Zero gradient from m = v = 0 leaves master unchanged, so the kernel's fp16
    copy is its cast of the input; checked against the oracle's encoder on all
    2^32 fp32 patterns (NaN inputs: any NaN output)."""
    from concurrent.futures import ThreadPoolExecutor

    from zero_mixed_precision_amd import _lib
    chunk = 1 << 28
    m = torch.zeros(chunk, dtype=torch.float32, device="cuda:0")
    v = torch.zeros(chunk, dtype=torch.float32, device="cuda:0")
    p16 = torch.empty(chunk, dtype=torch.int16, device="cuda:0")
    g = torch.zeros(chunk, dtype=torch.int16, device="cuda:0")
    st = torch.zeros(_lib.ds_scaler_size(), dtype=torch.uint8, device="cuda:0")
    with ThreadPoolExecutor(8) as pool:
        for lo in range(0, 1 << 32, chunk):
            x = np.arange(lo, lo + chunk, dtype=np.uint32).view(np.float32)
            master = gu.dev_f32(torch, x)
            m.zero_()
            v.zero_()
            _lib.ds_state_init(st, 1.0, 1.0, 1000, 1, 0, 1)
            _lib.ds_adam_step(st, master, m, v, p16, _lib.DS_FP16, g, _lib.DS_FP16, chunk, LR, BETA1, BETA2, EPS,
                              0.0, 0.0, 1)
            got = gu.host_u16(p16)
            want = _enc16_parallel(pool, x)
            nan_in = np.isnan(x)
            assert np.array_equal(got[~nan_in], want[~nan_in]), hex(lo)
            gn = got[nan_in]
            assert np.all(((gn & 0x7C00) == 0x7C00) & ((gn & 0x03FF) != 0)), hex(lo)
            del master


# -- device input generator equals the host generator ---------------------------------

def test_device_generator_matches_host(torch):
    tabs = synth.DeviceTables(torch, "cuda:0")
    n = (1 << 20) + 5
    for spec in (synth.GradSpec(1e-3, 2.0 ** 16), synth.GradSpec(5e-4, 2.0 ** 16, heavy_tail=True)):
        key = synth.stream_key(42, synth.ARR_GRAD, 1, 0)
        out = torch.empty(n, dtype=torch.int16, device="cuda:0")
        synth.device_fill_grad16(torch, tabs, out, key, spec)
        assert np.array_equal(gu.host_u16(out), synth.host_grad16(key, np.arange(n), spec))
        # a window far beyond 2^32
        start = (1 << 33) + 12345
        out2 = torch.empty(1003, dtype=torch.int16, device="cuda:0")
        synth.device_fill_grad16(torch, tabs, out2, key, spec, start=start)
        assert np.array_equal(gu.host_u16(out2), synth.host_grad16(key, start + np.arange(1003), spec))
    key = synth.stream_key(42, synth.ARR_MASTER)
    outm = torch.empty(n, dtype=torch.float32, device="cuda:0")
    synth.device_fill_master32(torch, tabs, outm, key, MASTER_SIGMA)
    assert np.array_equal(f32_bits(gu.host_f32(outm)), f32_bits(synth.host_master32(key, np.arange(n), MASTER_SIGMA)))


def test_data_movement_reference_kernels(torch):
    """The bandwidth references move the bytes they claim to: the copy, and the
    step-shaped mix (a <- b, b <- c, c <- a, h <- g) over full tiles and a ragged last one."""
    rng = np.random.default_rng(5)
    n = 3 * 4096 + 1024 + 8
    g = rng.integers(-2 ** 15, 2 ** 15, n).astype(np.int16)
    a, b, c = (rng.standard_normal(n).astype(np.float32) for _ in range(3))
    dg, da, db, dc = (torch.from_numpy(x.copy()).to("cuda:0") for x in (g, a, b, c))
    dh = torch.zeros(n, dtype=torch.int16, device="cuda:0")
    synth.device_stream_mix(torch, dg, da, db, dc, dh)
    for dev, want in ((da, b), (db, c), (dc, a), (dh, g)):
        assert np.array_equal(dev.cpu().numpy(), want)
    src = torch.from_numpy(rng.integers(0, 2 ** 31, 4 * 1000 + 4).astype(np.int32)).to("cuda:0")
    dst = torch.zeros_like(src)
    synth.device_copy(torch, dst, src)
    assert torch.equal(dst, src)
