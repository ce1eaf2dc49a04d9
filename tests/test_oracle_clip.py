"""Pins of the oracle's global-norm gradient clipping.

Pages: "DeepSpeed complete guide" section 4.1 (gradient_clipping 1.0) and
section 5.4 (the Accelerate plugin's gradient_clipping=1.0); section 5.1
(step() includes clipping).  Reading: the L2 norm of the whole unscaled
gradient is clipped to gradient_clipping with coefficient
min(1, max_norm / (norm + 1e-6)).

Fixed by: exact rational sums of squares (Python fractions), the closed form
of the first Adam step with clipping (the first moment is (1-beta1) * coef * g),
bit-identity with the unclipped step when the norm is below the limit, and
torch.nn.utils.clip_grad_norm_ followed by torch.optim.Adam.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests._fp import f32_bits, ulp32

LR, B1, B2, EPS = 1e-4, 0.9, 0.999, 1e-8


def _state(p0, scale):
    n = p0.size
    return oracle.State(p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32),
                        np.zeros(n, np.uint16), oracle.Scaler(scale, 1.0, 1000, 1))


def test_sumsq_fp16_is_exact():
    rng = np.random.default_rng(0)
    for trial in range(40):
        n = int(rng.integers(1, 3000))
        h = rng.integers(0, 65536, n).astype(np.uint16)
        h = np.where((h & 0x7C00) == 0x7C00, h & 0x83FF, h).astype(np.uint16)
        exact = sum(Fraction(float(x)) ** 2 for x in h.view(np.float16).astype(np.float64))
        assert oracle.grad_sumsq(h) == float(exact)
    assert oracle.grad_sumsq(np.array([0x7C00, 0], np.uint16)) == math.inf
    assert oracle.grad_sumsq(np.zeros(0, np.uint16)) == 0.0


def test_sumsq_fp32_is_exact():
    rng = np.random.default_rng(1)
    for trial in range(20):
        x = (rng.standard_normal(500) * 10.0 ** rng.integers(-20, 20, 500)).astype(np.float32)
        exact = sum(Fraction(float(v)) ** 2 for v in x)
        assert oracle.grad_sumsq(x) == float(exact)


def test_multiplier_without_clipping_is_the_unscale():
    for scale, K in ((2.0 ** 16, 1), (2.0 ** 15, 8), (3.0, 3)):
        inv = np.float32(1) / (np.float32(scale) * np.float32(K))
        assert oracle.clip_multiplier(123.0, scale, K, 0.0) == inv
        # a norm below the limit gives the unscale exactly
        assert oracle.clip_multiplier(1e-6, scale, K, 1.0) == inv


def test_clipped_norm_equals_the_limit():
    """After the multiplier, the unscaled gradient's norm is max_norm*norm/(norm+1e-6)."""
    rng = np.random.default_rng(2)
    S = 2.0 ** 10
    g = (rng.normal(0, 0.5, 100000) * S).astype(np.float16).view(np.uint16)
    sumsq = oracle.grad_sumsq(g)
    norm = math.sqrt(sumsq) / S
    assert norm > 10
    for max_norm in (1.0, 0.25, 5.0):
        mult = float(oracle.clip_multiplier(sumsq, S, 1, max_norm))
        got = math.sqrt(sumsq) * mult
        want = float(np.float32(max_norm)) * norm / (norm + 1e-6)
        assert abs(got - want) <= 1e-6 * want


def test_first_step_with_clipping_closed_form():
    """From m = v = 0 the first moment after one clipped step is (1-beta1)*coef*g."""
    rng = np.random.default_rng(3)
    S = 2.0 ** 12
    n = 20000
    g16 = (rng.normal(0, 0.3, n) * S).astype(np.float16).view(np.uint16)
    st = _state(rng.normal(0, 0.02, n).astype(np.float32), S)
    assert not oracle.step(st, g16, lr=LR, beta1=B1, beta2=B2, eps=EPS, max_grad_norm=1.0)
    g = g16.view(np.float16).astype(np.float64) / S
    norm = float(np.sqrt(np.sum(g * g)))
    coef = 1.0 / (norm + 1e-6)
    omb1 = float(np.float32(1) - np.float32(B1))
    want_m = omb1 * coef * g
    assert np.all(np.abs(st.m - want_m) <= 4 * ulp32(want_m) + 1e-30)
    # the clipped moments have unit norm up to rounding
    assert abs(np.sqrt(np.sum((st.m.astype(np.float64) / omb1) ** 2)) - norm * coef) < 1e-6


def test_unclipped_when_below_limit_is_bit_identical():
    rng = np.random.default_rng(4)
    n = 5000
    g16 = (rng.normal(0, 1e-3, n) * 2 ** 16).astype(np.float16).view(np.uint16)
    p0 = rng.normal(0, 0.02, n).astype(np.float32)
    a, b = _state(p0, 2.0 ** 16), _state(p0, 2.0 ** 16)
    oracle.step(a, g16, lr=LR, beta1=B1, beta2=B2, eps=EPS, max_grad_norm=1.0)   # norm ~0.07 < 1
    oracle.step(b, g16, lr=LR, beta1=B1, beta2=B2, eps=EPS)
    for x, y in ((a.master, b.master), (a.m, b.m), (a.v, b.v)):
        assert np.array_equal(f32_bits(x), f32_bits(y))


@pytest.mark.parametrize("K", [1, 4])
def test_matches_torch_clip_grad_norm_then_adam(K):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    n, T, S, max_norm = 30000, 8, 2.0 ** 8, 1.0
    f = lambda x: float(np.float32(x))
    p0 = rng.normal(0, 0.02, n).astype(np.float32)
    st = _state(p0, S)
    param = torch.nn.Parameter(torch.from_numpy(p0.copy()))
    opt = torch.optim.Adam([param], lr=f(LR), betas=(f(B1), f(B2)), eps=f(EPS), foreach=False)
    clipped_steps = 0
    for t in range(T):
        gs = [(rng.normal(0, 0.02 * (t + 1), n) * S).astype(np.float16).view(np.uint16) for _ in range(K)]
        oracle.step(st, gs if K > 1 else gs[0], lr=LR, beta1=B1, beta2=B2, eps=EPS, max_grad_norm=max_norm)
        total = np.zeros(n, np.float32)
        for g in gs:
            total = (total + g.view(np.float16).astype(np.float32)).astype(np.float32)
        param.grad = torch.from_numpy((total / np.float32(S * K)).astype(np.float32))
        norm = torch.nn.utils.clip_grad_norm_([param], max_norm)
        clipped_steps += int(float(norm) > max_norm)
        opt.step()
    assert clipped_steps >= T // 2
    ref = param.detach().numpy()
    move = st.master.astype(np.float64) - p0
    move_ref = ref.astype(np.float64) - p0
    assert np.all(np.abs(move - move_ref) <= 1e-5 * T * LR + 4 * ulp32(ref))
    assert np.allclose(st.m, opt.state[param]["exp_avg"].numpy(), rtol=1e-5, atol=1e-9)


def test_sumsq32_exact_units_matches_rational_sums():
    """The integer form of the fp32 sum of squares equals the exact rational sum
    (in units of 2^-298), across the whole exponent range, subnormals, zeros of
    either sign and the largest finite value; pieces add up to the whole."""
    rng = np.random.default_rng(7)
    unit = Fraction(1, 2 ** oracle.SUMSQ32_UNIT_BITS)
    specials = np.array([0.0, -0.0, 1e-45, -1e-45, 1.1754942e-38, 1.1754944e-38, 3.4028235e38, -1.0, 2.0 ** -126],
                        np.float32)
    for trial in range(12):
        n = int(rng.integers(1, 2500))
        bits = rng.integers(0, 2 ** 32, n, dtype=np.uint64).astype(np.uint32)
        bits = np.where(((bits >> 23) & 0xFF) == 0xFF, bits & 0x807FFFFF, bits).astype(np.uint32)
        x = np.concatenate([bits.view(np.float32), specials])
        exact = sum(Fraction(float(v)) ** 2 for v in x)
        units = oracle.sumsq32_exact_units(x)
        assert Fraction(units) * unit == exact
        assert oracle.units_to_float(units) == float(exact)
        cut = int(rng.integers(0, x.size))
        assert oracle.sumsq32_exact_units(x[:cut]) + oracle.sumsq32_exact_units(x[cut:]) == units
    # the accumulation buffer's values: sums of a few fp16 gradients
    g = (rng.standard_normal((8, 4000)) * 30).astype(np.float16).astype(np.float32).sum(axis=0, dtype=np.float32)
    assert oracle.units_to_float(oracle.sumsq32_exact_units(g)) == math.fsum((g.astype(np.float64) ** 2).tolist())
    assert oracle.sumsq32_exact_units(np.array([1.0, np.inf], np.float32)) is None
    assert oracle.sumsq32_exact_units(np.array([np.nan], np.float32)) is None
    assert oracle.sumsq32_exact_units(np.zeros(0, np.float32)) == 0


def test_sumsq32_exact_units_catches_a_dropped_term():
    """A plausible slip in the integer form (the cross term's factor) changes
    the sum: the three parts are all needed."""
    x = np.array([1.0 + 2.0 ** -23, 3.0, 1e-40], np.float32)
    exact = sum(Fraction(float(v)) ** 2 for v in x) * 2 ** oracle.SUMSQ32_UNIT_BITS
    assert oracle.sumsq32_exact_units(x) == exact
    M = (x.view(np.uint32) & 0x7FFFFF).astype(np.int64) + (1 << 23)
    assert int(((M[:2] >> 12) * (M[:2] & 0xFFF)).sum()) != 0      # the cross term is not zero here
