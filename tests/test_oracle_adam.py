"""Pins of the oracle's Adam update against closed forms and library routines.

What fixes the oracle here, other than itself:
  * closed forms of bias-corrected Adam (first step from m = v = 0; a constant
    gradient; a zero gradient), evaluated in fp64 from the mathematics;
  * the exact bias-correction values 1 - beta^t (80-digit decimals);
  * torch.optim.Adam / AdamW on the CPU (a library routine with a different
    operation order) over several steps;
  * a per-operation fp32 re-evaluation in numpy, which checks that the
    compiled C rounds once per operation (no contraction, no widening).
Pages: "DeepSpeed complete guide" section 2 (fp32 master, first and second
moments), section 4.1 (optimizer AdamW, eps 1e-8), section 5.1 (step()
updates the parameters after backward).
"""
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests._fp import f32_bits, ulp32

LR, B1, B2, EPS = 1e-4, 0.9, 0.999, 1e-8
S16 = 2.0 ** 16


def _fresh_state(p0, scale=S16, window=1000):
    n = p0.size
    return oracle.State(p0.astype(np.float32).copy(), np.zeros(n, np.float32),
                        np.zeros(n, np.float32), np.zeros(n, np.uint16),
                        oracle.Scaler(scale, 1.0, window, 1))


def _grads16(rng, n, sigma=1e-3, scale=S16):
    return (rng.normal(0, sigma, n) * scale).astype(np.float16).view(np.uint16)


def _all_finite_fp16_patterns(rng, n):
    h = rng.integers(0, 65536, n, dtype=np.uint32).astype(np.uint16)
    return np.where((h & 0x7C00) == 0x7C00, h & 0x83FF, h).astype(np.uint16)


# -- per-step scalars ---------------------------------------------------------

@pytest.mark.parametrize("t", [1, 2, 3, 7, 10, 50, 1000, 12345, 10 ** 6])
def test_bias_correction_scalars_match_exact_values(oracle_lib, t):
    """step_size = lr/(1 - beta1^t) and rbc2 = 1/sqrt(1 - beta2^t), from the fp32
    hyperparameter values, in 80-digit decimal arithmetic: within 1 fp32 ulp."""
    getcontext().prec = 80
    b1 = Decimal(float(np.float32(B1)))      # exact: every binary float is a finite decimal
    b2 = Decimal(float(np.float32(B2)))
    lr = Decimal(float(np.float32(LR)))
    step_exact = lr / (1 - b1 ** t)
    rbc2_exact = 1 / (1 - b2 ** t).sqrt()
    step_size, rbc2 = oracle.adam_scalars(t, LR, B1, B2)
    assert abs(Decimal(step_size) - step_exact) <= Decimal(float(ulp32(step_size)))
    assert abs(Decimal(rbc2) - rbc2_exact) <= Decimal(float(ulp32(rbc2)))


def test_one_minus_beta_constants(oracle_lib):
    # (1 - beta) in fp32 is exact for beta in [0.5, 1] (Sterbenz); pin the values used
    assert f32_bits(np.float32(1) - np.float32(B1))[()] == 0x3DCCCCD0
    assert f32_bits(np.float32(1) - np.float32(B2))[()] == 0x3A831200


# -- closed forms ---------------------------------------------------------------

def test_first_step_closed_form(oracle_lib):
    """t = 1 from m = v = 0: m_hat = g and v_hat = g^2, so the move is lr*g/(|g|+eps)."""
    rng = np.random.default_rng(1)
    n = 50000
    p0 = rng.normal(0, 0.02, n).astype(np.float32)
    g16 = np.concatenate([_grads16(rng, n // 2), _all_finite_fp16_patterns(rng, n - n // 2)])
    st = _fresh_state(p0)
    assert not oracle.step(st, g16, lr=LR, beta1=B1, beta2=B2, eps=EPS)
    g = g16.view(np.float16).astype(np.float64) / S16
    lr, eps = float(np.float32(LR)), float(np.float32(EPS))
    delta = lr * g / (np.abs(g) + eps)
    want = p0.astype(np.float64) - delta
    err = np.abs(st.master.astype(np.float64) - want)
    assert np.all(err <= ulp32(st.master) + 1e-6 * np.abs(delta))
    # the move is ~lr*sign(g) only where |g| >> eps; near eps it is smaller
    big = np.abs(g) > 1e-4
    assert np.allclose((p0 - st.master)[big], lr * np.sign(g[big]), rtol=1e-3, atol=0)
    small = (np.abs(g) > 0) & (np.abs(g) < 1e-9)
    assert small.any() and np.all(np.abs(p0 - st.master)[small] < 0.2 * lr)


def test_constant_gradient_closed_form(oracle_lib):
    """Constant g from m = v = 0: m_hat = g and v_hat = g^2 at every t, so after T
    applied steps p = p0 - T*lr*g/(|g|+eps)."""
    rng = np.random.default_rng(2)
    n, T = 20000, 50
    p0 = rng.normal(0, 0.02, n).astype(np.float32)
    g16 = _grads16(rng, n)
    st = _fresh_state(p0)
    for _ in range(T):
        assert not oracle.step(st, g16, lr=LR, beta1=B1, beta2=B2, eps=EPS)
    assert st.scaler.applied == T
    g = g16.view(np.float16).astype(np.float64) / S16
    lr, eps = float(np.float32(LR)), float(np.float32(EPS))
    delta = lr * g / (np.abs(g) + eps)
    want = p0.astype(np.float64) - T * delta
    err = np.abs(st.master.astype(np.float64) - want)
    assert np.all(err <= T * ulp32(np.maximum(np.abs(p0), np.abs(st.master))) + 1e-5 * T * np.abs(delta))


def test_zero_gradient_leaves_state_bit_identical(oracle_lib):
    rng = np.random.default_rng(3)
    n = 4096
    p0 = rng.normal(0, 0.02, n).astype(np.float32)
    st = _fresh_state(p0)
    for _ in range(3):
        oracle.step(st, np.zeros(n, np.uint16), lr=LR, beta1=B1, beta2=B2, eps=EPS)
    assert np.array_equal(f32_bits(st.master), f32_bits(p0))
    assert not st.m.any() and not st.v.any()
    assert np.array_equal(st.p16, p0.astype(np.float16).view(np.uint16))


# -- library cross-check ------------------------------------------------------

@pytest.mark.parametrize("wd", [0.0, 0.01])
def test_matches_torch_adam_over_ten_steps(oracle_lib, wd):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(4)
    n, T = 20000, 10
    p0 = rng.normal(0, 0.02, n).astype(np.float32)
    st = _fresh_state(p0)
    param = torch.nn.Parameter(torch.from_numpy(p0.copy()))
    cls = torch.optim.AdamW if wd else torch.optim.Adam
    # hyperparameters are fp32 values on the boundary; hand torch those same values
    # (it derives 1 - beta in double, which then equals the fp32 difference exactly)
    f = lambda x: float(np.float32(x))
    opt = cls([param], lr=f(LR), betas=(f(B1), f(B2)), eps=f(EPS), weight_decay=wd, foreach=False)
    for _ in range(T):
        g16 = _grads16(rng, n)
        oracle.step(st, g16, lr=LR, beta1=B1, beta2=B2, eps=EPS, weight_decay=wd)
        param.grad = torch.from_numpy(g16.view(np.float16).astype(np.float32) / np.float32(S16))
        opt.step()
    ref = param.detach().numpy()
    move_ref = ref.astype(np.float64) - p0
    move = st.master.astype(np.float64) - p0
    # each step moves an element by at most ~lr; rounding-order differences stay
    # far below 1e-6 of that per step, while a formula mistake shows up at ~lr
    # with decay, p is rounded twice per step in each implementation (decay, then
    # the Adam move), so the two may drift apart by up to ~2 ulp(p) per step
    slack = (2 * T + 4) * ulp32(ref) if wd else 4 * ulp32(ref)
    assert np.all(np.abs(move - move_ref) <= 1e-6 * T * LR + slack)
    state = opt.state[param]
    ref_m = state["exp_avg"].numpy()
    ref_v = state["exp_avg_sq"].numpy()
    # moments: torch updates m by lerp (another rounding order); allow a few ulps of
    # the gradient scale (|g| ~ 1e-3, g^2 ~ 1e-6) on top of a relative 1e-5
    assert np.allclose(st.m, ref_m, rtol=1e-5, atol=1e-10)
    assert np.allclose(st.v, ref_v, rtol=1e-5, atol=1e-15)
    assert np.array_equal(st.p16, st.master.astype(np.float16).view(np.uint16))


# -- compiled arithmetic: one fp32 rounding per operation ---------------------

def _numpy_f32_update(graw, p, m, v, *, inv, step_size, rbc2, omb1, omb2, b1, b2, eps):
    f = np.float32
    g = f(graw) * inv
    m = f(b1 * m) + f(omb1 * g)
    v = f(b2 * v) + f(omb2 * f(g * g))
    d = f(np.sqrt(v) * rbc2) + eps
    p = p - f(step_size * f(m / d))
    return f(p), f(m), f(v)


def test_sixteen_elements_match_per_operation_fp32(oracle_lib):
    rng = np.random.default_rng(5)
    f = np.float32
    for trial in range(200):
        n = 16
        p = rng.normal(0, 0.02, n).astype(np.float32)
        m = rng.normal(0, 1e-4, n).astype(np.float32)
        v = np.abs(rng.normal(0, 1e-7, n)).astype(np.float32)
        g16 = _all_finite_fp16_patterns(rng, n) if trial % 2 else _grads16(rng, n)
        t = int(rng.integers(1, 2000))
        scale = f(2.0 ** int(rng.integers(0, 24)))
        K = int(rng.choice([1, 2, 8]))
        mo, vo, po, p16 = m.copy(), v.copy(), p.copy(), np.zeros(n, np.uint16)
        oracle.adam(g16, po, mo, vo, p16, scale=scale, accum_steps=K, t=t, lr=LR, beta1=B1,
                    beta2=B2, eps=EPS)
        step_size, rbc2 = oracle.adam_scalars(t, LR, B1, B2)
        kw = dict(inv=f(f(1) / f(scale * f(K))), step_size=f(step_size), rbc2=f(rbc2),
                  omb1=f(1) - f(B1), omb2=f(1) - f(B2), b1=f(B1), b2=f(B2), eps=f(EPS))
        graw = g16.view(np.float16).astype(np.float32)
        for i in range(n):
            pe, me, ve = _numpy_f32_update(graw[i], p[i], m[i], v[i], **kw)
            assert f32_bits(pe) == f32_bits(po[i]) and f32_bits(me) == f32_bits(mo[i]) \
                and f32_bits(ve) == f32_bits(vo[i]), (trial, i)
        assert np.array_equal(p16, po.astype(np.float16).view(np.uint16))


# -- exact rational arithmetic, rounded by hand -----------------------------------

def _round_binary(x: Fraction, mant_bits: int, emin: int, emax: int) -> Fraction:
    """x rounded to nearest, ties to even, in a binary format with `mant_bits`
    fraction bits and normal exponents emin..emax (subnormals kept; overflow is
    not reached by these inputs and raises)."""
    if x == 0:
        return Fraction(0)
    sign, a = (-1, -x) if x < 0 else (1, x)
    e = a.numerator.bit_length() - a.denominator.bit_length()      # 2^e <= a < 2^(e+1) after the fix-up
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum = Fraction(2) ** (max(e, emin) - mant_bits)             # spacing of representable values near a
    scaled = a / quantum
    n = scaled.numerator // scaled.denominator
    rest = scaled - n
    if rest > Fraction(1, 2) or (rest == Fraction(1, 2) and n % 2 == 1):
        n += 1
    v = n * quantum
    if v >= Fraction(2) ** (emax + 1):
        raise OverflowError("rounds to infinity")
    return sign * v


def _f32(x: Fraction) -> Fraction:
    return _round_binary(x, 23, -126, 127)


def _f16(x: Fraction) -> Fraction:
    return _round_binary(x, 10, -14, 15)


def _sqrt_f32(x: Fraction) -> Fraction:
    """Correctly rounded fp32 square root of an fp32 value x >= 0, by integer square
    roots: the exact root lies in [s, s + 1) * 2^-k, narrow enough that both ends
    round alike unless the root is exact."""
    from math import isqrt
    if x == 0:
        return Fraction(0)
    k = 200
    scaled = x * Fraction(2) ** (2 * k)
    assert scaled.denominator == 1                                   # x is dyadic with < 400 fraction bits
    s = isqrt(scaled.numerator)
    lo, hi = Fraction(s, 2 ** k), Fraction(s + 1, 2 ** k)
    if s * s == scaled.numerator:
        return _f32(lo)
    r = _f32(lo)
    assert r == _f32(hi) or lo < r < hi, "rounding boundary inside the bracket"
    return r


def _exact_update(graw, p, m, v, *, inv, step_size, rbc2, omb1, omb2, b1, b2, eps, lrwd=None):
    """One element of the bias-corrected Adam update, every operation exact then rounded
    to fp32 (no shared rounding, no fused multiply-add), in the oracle's written order."""
    g = _f32(graw * inv)
    m = _f32(_f32(b1 * m) + _f32(omb1 * g))
    v = _f32(_f32(b2 * v) + _f32(omb2 * _f32(g * g)))
    if lrwd is not None:
        p = _f32(p - _f32(lrwd * p))
    den = _f32(_f32(_sqrt_f32(v) * rbc2) + eps)
    p = _f32(p - _f32(step_size * _f32(m / den)))
    return p, m, v


@pytest.mark.parametrize("wd", [0.0, 0.01])
def test_sixteen_elements_match_exact_rational_evaluation(oracle_lib, wd):
    """The compiled oracle equals an exact rational re-evaluation of the update rounded
    to fp32 by hand after every operation (binary16 for the parameter copy), bit for bit,
    on 16-element inputs over three steps: no contraction, no extra precision, and the
    IEEE rounding of divide and square root."""
    rng = np.random.default_rng(15)
    Q = lambda x: Fraction(float(x))                                 # exact value of a float
    f = np.float32
    for trial in range(12):
        n = 16
        p = rng.normal(0, 0.02, n).astype(np.float32)
        m = rng.normal(0, 1e-4, n).astype(np.float32)
        v = np.abs(rng.normal(0, 1e-7, n)).astype(np.float32)
        scale = 2.0 ** int(rng.integers(0, 20)) * (1.0 if trial % 3 else 1.5)   # some scales not powers of two
        K = int(rng.choice([1, 3, 8]))
        state = oracle.State(p.copy(), m.copy(), v.copy(), np.zeros(n, np.uint16),
                             oracle.Scaler(float(f(scale)), 1.0, 1000, 1))
        ep, em, ev = [Q(x) for x in p], [Q(x) for x in m], [Q(x) for x in v]
        for step in range(3):
            grads = [(_all_finite_fp16_patterns(rng, n) if (trial + k) % 2 else _grads16(rng, n, scale=scale))
                     for k in range(K)]
            t = state.scaler.applied + 1
            assert not oracle.step(state, grads if K > 1 else grads[0], lr=LR, beta1=B1, beta2=B2, eps=EPS,
                                   weight_decay=wd)
            step_size, rbc2 = oracle.adam_scalars(t, LR, B1, B2)
            S = Q(f(scale))
            kw = dict(inv=_f32(1 / _f32(S * K)), step_size=Q(step_size), rbc2=Q(rbc2),
                      omb1=_f32(1 - Q(f(B1))), omb2=_f32(1 - Q(f(B2))), b1=Q(f(B1)), b2=Q(f(B2)), eps=Q(f(EPS)),
                      lrwd=_f32(Q(f(LR)) * Q(f(wd))) if wd else None)
            for i in range(n):
                gsum = Fraction(0)
                for k in range(K):                                   # the fp32 sum over micro-batches, in order
                    gk = Q(grads[k].view(np.float16)[i])
                    gsum = gk if k == 0 else _f32(gsum + gk)
                ep[i], em[i], ev[i] = _exact_update(gsum, ep[i], em[i], ev[i], **kw)
            got = [(Q(a), Q(b), Q(c)) for a, b, c in zip(state.master, state.m, state.v)]
            assert got == list(zip(ep, em, ev)), (trial, step)
            want16 = [_f16(x) for x in ep]
            assert [Q(x) for x in state.p16.view(np.float16)] == want16, (trial, step)


# -- skip invariant on 16-element inputs -----------------------------------------

SPECIALS = {"+inf": 0x7C00, "-inf": 0xFC00, "qnan": 0x7E00, "snan": 0x7C01, "nan_payload": 0xFE5A}


@pytest.mark.parametrize("name", sorted(SPECIALS))
def test_overflow_skips_and_halves_at_every_position(oracle_lib, name):
    rng = np.random.default_rng(6)
    for pos in range(16):
        p0 = rng.normal(0, 0.02, 16).astype(np.float32)
        st = _fresh_state(p0)
        oracle.step(st, _grads16(rng, 16), lr=LR, beta1=B1, beta2=B2, eps=EPS)
        before = [a.copy() for a in (st.master, st.m, st.v, st.p16)]
        g16 = _grads16(rng, 16)
        g16[pos] = SPECIALS[name]
        assert oracle.step(st, g16, lr=LR, beta1=B1, beta2=B2, eps=EPS)
        for a, b in zip(before, (st.master, st.m, st.v, st.p16)):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
        assert st.scaler.scale == S16 / 2 and st.scaler.applied == 1 and st.scaler.s.skipped == 1


@pytest.mark.parametrize("h", [0x7BFF, 0xFBFF, 0x0001, 0x8001, 0x8000, 0x03FF])
def test_largest_finite_and_subnormal_are_not_overflow(oracle_lib, h):
    rng = np.random.default_rng(8)
    for pos in (0, 7, 15):
        st = _fresh_state(rng.normal(0, 0.02, 16).astype(np.float32))
        g16 = _grads16(rng, 16)
        g16[pos] = h
        assert not oracle.step(st, g16, lr=LR, beta1=B1, beta2=B2, eps=EPS)
        assert st.scaler.applied == 1


def test_empty_partition_is_a_no_op(oracle_lib):
    st = _fresh_state(np.zeros(0, np.float32))
    assert not oracle.step(st, np.zeros(0, np.uint16), lr=LR, beta1=B1, beta2=B2, eps=EPS)
    assert st.scaler.applied == 1


# -- stored worked example ---------------------------------------------------------

def test_worked_example_fixture(oracle_lib):
    """The stored 4-element example (written by tests/golden/make_worked_example.py
    from the oracle) still reproduces, and its first step obeys the closed form."""
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "adam_worked_example.json")
    ex = json.load(open(path))
    h32 = lambda xs: np.array([int(x, 16) for x in xs], np.uint32).view(np.float32)
    h16 = lambda xs: np.array([int(x, 16) for x in xs], np.uint16)
    p0 = h32(ex["inputs"]["master"])
    st = _fresh_state(p0)
    for k, s in enumerate(ex["steps"]):
        oracle.step(st, h16(s["grad16"]), lr=LR, beta1=B1, beta2=B2, eps=EPS)
        assert np.array_equal(f32_bits(st.master), f32_bits(h32(s["master"])))
        assert np.array_equal(f32_bits(st.m), f32_bits(h32(s["m"])))
        assert np.array_equal(f32_bits(st.v), f32_bits(h32(s["v"])))
        assert np.array_equal(st.p16, h16(s["p16"]))
        if k == 0:
            g = h16(s["grad16"]).view(np.float16).astype(np.float64) / S16
            delta = float(np.float32(LR)) * g / (np.abs(g) + float(np.float32(EPS)))
            assert np.all(np.abs(h32(s["master"]) - (p0 - delta)) <= ulp32(p0) + 1e-6 * np.abs(delta))


def test_scalars_range_equals_the_scalar_function():
    """The array form of the per-step factors is the per-step function, step by step."""
    for lr, b1, b2 in ((1e-4, 0.9, 0.999), (3e-4, 0.95, 0.98)):
        got = oracle.adam_scalars_range(1, 2000, lr, b1, b2)
        want = np.array([oracle.adam_scalars(t, lr, b1, b2) for t in range(1, 2001)], np.float32)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
        got = oracle.adam_scalars_range(10 ** 6 - 3, 4, lr, b1, b2)
        want = np.array([oracle.adam_scalars(t, lr, b1, b2) for t in range(10 ** 6 - 3, 10 ** 6 + 1)], np.float32)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
