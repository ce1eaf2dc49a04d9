"""Pins of the oracle's dynamic loss scaler and gradient accumulation.

Scaler rules ("DeepSpeed complete guide" section 4.2, fp16 settings):
loss_scale 0 means dynamic; the initial scale is 2^initial_scale_power
(16 -> 65536, printed on the page); loss_scale_window is the number of
successful steps before the scale increases; hysteresis is the number of
overflows before it decreases; min_loss_scale is the floor.  Reading (factor
two both ways, as in "halves"/"doubles") is stated in oracle.c.  The expected
sequences below are derived by hand from those rules for each workload.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def run_sequence(init_pow, window, overflow_steps, steps, hysteresis=1, min_scale=1.0):
    sc = oracle.Scaler(2.0 ** init_pow, min_scale, window, hysteresis)
    used = []
    for s in range(1, steps + 1):
        used.append(sc.scale)
        sc.update(s in overflow_steps)
    return used, sc


def test_initial_scale_from_pages(oracle_lib):
    cfg = json.load(open(os.path.join(GOLDEN, "fp16_config.json")))
    power = cfg["fp16_section_4_2"]["initial_scale_power"]
    assert 2.0 ** power == cfg["meanings"]["initial_scale_power_16"] == 65536
    sc = oracle.Scaler(2.0 ** power)
    assert sc.scale == 65536.0 and sc.applied == 0


def test_tiny_partition_sequence(oracle_lib):
    # 2^16, window 1000, +inf in step 4, 10 steps
    used, sc = run_sequence(16, 1000, {4}, 10)
    assert [int(np.log2(u)) for u in used] == [16, 16, 16, 16, 15, 15, 15, 15, 15, 15]
    assert sc.scale == 2.0 ** 15 and sc.applied == 9 and sc.s.skipped == 1 and sc.s.iters == 10


@pytest.mark.parametrize("steps", [50, 20])
def test_no_overflow_long_window(oracle_lib, steps):
    used, sc = run_sequence(16, 1000, set(), steps)
    assert all(u == 2.0 ** 16 for u in used) and sc.applied == steps


def test_ragged_layout_sequence(oracle_lib):
    # 2^15, window 10, overflows in steps 3, 4, 17, 30 steps
    used, sc = run_sequence(15, 10, {3, 4, 17}, 30)
    want = [15, 15, 15, 14] + [13] * 10 + [14, 14, 14] + [13] * 10 + [14, 14, 14]
    assert [int(np.log2(u)) for u in used] == want
    assert sc.scale == 2.0 ** 14 and sc.applied == 27 and sc.s.skipped == 3


def test_heavy_tail_shard_sequence(oracle_lib):
    # 2^16, window 5, no overflow, 10 steps: grows after steps 5 and 10
    used, sc = run_sequence(16, 5, set(), 10)
    assert [int(np.log2(u)) for u in used] == [16] * 5 + [17] * 5
    assert sc.scale == 2.0 ** 18 and sc.applied == 10


def test_growth_after_exactly_window_successes(oracle_lib):
    for W in (1, 2, 3, 7):
        sc = oracle.Scaler(4.0, 1.0, W, 1)
        for k in range(W - 1):
            sc.update(False)
            assert sc.scale == 4.0
        sc.update(False)
        assert sc.scale == 8.0 and sc.s.good_steps == 0


def test_overflow_resets_the_success_run(oracle_lib):
    sc = oracle.Scaler(1024.0, 1.0, 3, 1)
    sc.update(False); sc.update(False)
    sc.update(True)
    assert sc.scale == 512.0 and sc.s.good_steps == 0
    sc.update(False); sc.update(False)
    assert sc.scale == 512.0
    sc.update(False)
    assert sc.scale == 1024.0


def test_floor_holds_and_overflow_keeps_skipping(oracle_lib):
    sc = oracle.Scaler(4.0, 1.0, 1000, 1)
    for _ in range(5):
        sc.update(True)
    assert sc.scale == 1.0 and sc.s.skipped == 5 and sc.applied == 0


def test_floor_below_the_powers_of_two_from_pages(oracle_lib):
    """The guide's gradient-overflow config (section 13.1: initial power 12, hysteresis 2,
    min_loss_scale 1e-8): halving from 2^12 passes 2^-26 (1.49e-8); the next halving
    (2^-27 = 7.45e-9) is below the floor, so the scale becomes fp32(1e-8) -- no longer a
    power of two -- and stays there under further overflows; growth doubles it exactly."""
    cfg = json.load(open(os.path.join(GOLDEN, "fp16_config.json")))["fp16_section_13_1"]
    H, floor = cfg["hysteresis"], cfg["min_loss_scale"]
    assert (cfg["initial_scale_power"], H, floor) == (12, 2, 1e-8)
    sc = oracle.Scaler(2.0 ** cfg["initial_scale_power"], floor, 3, H)
    scales = []
    for _ in range(2 * 40):
        sc.update(True)
        scales.append(sc.scale)
    # every second overflow halves (hysteresis 2)
    assert scales[2 * 38 - 1] == 2.0 ** -26 and scales[2 * 38] == 2.0 ** -26
    assert scales[2 * 39 - 1] == float(np.float32(1e-8))
    assert scales[-1] == float(np.float32(1e-8)) and sc.s.skipped == 80
    for _ in range(3):
        sc.update(False)
    assert sc.scale == 2 * float(np.float32(1e-8)) and sc.applied == 3


def test_hysteresis_two_halves_every_second_overflow(oracle_lib):
    """hysteresis = 2 (the pages' default): two overflows per decrease (the
    key's one-line meaning on the page)."""
    sc = oracle.Scaler(2.0 ** 16, 1.0, 1000, 2)
    seq = []
    for _ in range(4):
        sc.update(True)
        seq.append(sc.scale)
    assert seq == [2.0 ** 16, 2.0 ** 15, 2.0 ** 15, 2.0 ** 14]


def _closed_form(seq, H, W, consecutive):
    """The scaler's state after each step of an overflow sequence, counted
    over the sequence instead of stepped: the growth and hysteresis readings
    as run lengths.

    - growths: every maximal run of L successes doubles the scale floor(L / W)
      times (the success count restarts at an overflow and at each growth);
      the count left over is the current run's length mod W;
    - decreases without consecutive_hysteresis: successes never refill the
      count, which restarts only at a decrease, so O overflows in all halve
      the scale floor(O / H) times and leave H - O mod H units;
    - decreases with consecutive_hysteresis: a success refills the count, so
      every maximal run of R overflows halves floor(R / H) times and leaves
      H - R mod H units (H again once a success follows).
    Exponents are relative to the initial scale; the floor is never reached."""
    out = []
    growths = decreases = overflows = 0
    run_ok = run_ov = 0
    for i, ov in enumerate(seq):
        if ov:
            run_ov = run_ov + 1 if i and seq[i - 1] else 1
            run_ok = 0
            overflows += 1
            if consecutive:
                if run_ov % H == 0:
                    decreases += 1
                left = H - run_ov % H
            else:
                decreases = overflows // H
                left = H - overflows % H
        else:
            run_ok = run_ok + 1 if i and not seq[i - 1] else 1
            run_ov = 0
            if run_ok % W == 0:
                growths += 1
            left = H if consecutive else H - overflows % H
        out.append((growths - decreases, run_ok % W if not ov else 0, left,
                    overflows, i + 1 - overflows))
    return out


@pytest.mark.parametrize("consecutive", [False, True], ids=["spent_count", "consecutive_hysteresis"])
@pytest.mark.parametrize("H", [1, 2, 3, 5])
@pytest.mark.parametrize("W", [1, 2, 3, 7])
def test_scaler_matches_run_length_closed_form(oracle_lib, consecutive, H, W):
    """The hysteresis restart after a decrease, consecutive_hysteresis and
    growth checked at every step against the run-length counts above, on
    seeded random overflow sequences (overflow rates 0.1 to 0.9) and on
    structured ones (long runs of each kind, alternation).  The floor 2^-100
    and at most 80 steps keep the scale a power of two inside fp32's range, so
    scale == 2^(16 + growths - decreases) exactly."""
    rng = np.random.default_rng(1000 * H + 10 * W + consecutive)
    seqs = [list(rng.random(80) < p) for p in (0.1, 0.3, 0.5, 0.7, 0.9) for _ in range(4)]
    seqs += [[True] * 40 + [False] * 40, [False] * 40 + [True] * 40, [True, False] * 40,
             [True, True, False] * 26, ([False] * 6 + [True] * 4) * 8]
    for seq in seqs:
        sc = oracle.Scaler(2.0 ** 16, 2.0 ** -100, W, H, consecutive_hysteresis=consecutive)
        for i, (ov, want) in enumerate(zip(seq, _closed_form(seq, H, W, consecutive))):
            sc.update(bool(ov))
            e, good, left, skipped, applied = want
            s = sc.s
            ctx = f"H={H} W={W} consecutive={consecutive} step {i} of {''.join('x' if o else '.' for o in seq)}"
            assert s.scale == 2.0 ** (16 + e), ctx
            assert (s.good_steps, s.hyst_left, s.skipped, s.applied, s.iters) == (good, left, skipped, applied,
                                                                                 i + 1), ctx


def test_growth_is_not_capped(oracle_lib):
    """No upper bound on the scale (none is stated): with a window of one the
    scale doubles on every successful step up to fp32's largest power of two."""
    sc = oracle.Scaler(2.0 ** 16, 1.0, 1, 2)
    for k in range(1, 112):
        sc.update(False)
        assert sc.scale == 2.0 ** (16 + k)
    assert sc.scale == 2.0 ** 127


def test_static_scale_never_changes(oracle_lib):
    sc = oracle.Scaler(128.0, 1.0, 2, 1, dynamic=False)
    for ov in (False, False, True, False, False):
        sc.update(ov)
    assert sc.scale == 128.0 and sc.s.skipped == 1 and sc.applied == 4


# -- accumulation -------------------------------------------------------------------

def test_accumulate_matches_in_order_float32_adds(oracle_lib):
    rng = np.random.default_rng(11)
    n, K = 5000, 8
    gs = [(rng.normal(0, 1e-3, n) * 2 ** 15).astype(np.float16) for _ in range(K)]
    acc = np.empty(n, np.float32)
    for k, g in enumerate(gs):
        oracle.accumulate(acc, g.view(np.uint16), overwrite=(k == 0))
    want = gs[0].astype(np.float32)
    for g in gs[1:]:
        want = (want + g.astype(np.float32)).astype(np.float32)
    assert np.array_equal(acc.view(np.uint32), want.view(np.uint32))


def test_accumulate_overwrite_keeps_negative_zero(oracle_lib):
    acc = np.full(3, 5.0, np.float32)
    oracle.accumulate(acc, np.array([0x8000, 0x0000, 0x3C00], np.uint16), overwrite=True)
    assert acc.view(np.uint32).tolist() == [0x80000000, 0, 0x3F800000]


def test_accumulated_infinity_is_an_overflow(oracle_lib):
    n = 64
    acc = np.empty(n, np.float32)
    g = np.zeros(n, np.uint16)
    oracle.accumulate(acc, g, overwrite=True)
    g2 = g.copy(); g2[17] = 0x7C00
    oracle.accumulate(acc, g2, overwrite=False)
    g3 = g.copy(); g3[17] = 0xFC00
    oracle.accumulate(acc, g3, overwrite=False)
    assert np.isnan(acc[17]) and oracle.any_nonfinite(acc)


def test_step_with_microbatches_divides_by_k(oracle_lib):
    """K identical micro-batches equal one batch of that gradient: the sum is unscaled by S*K."""
    rng = np.random.default_rng(12)
    n, K = 3000, 8
    p0 = rng.normal(0, 0.02, n).astype(np.float32)
    g = (rng.normal(0, 1e-3, n) * 2 ** 15).astype(np.float16).view(np.uint16)
    a = oracle.State(p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32),
                     np.zeros(n, np.uint16), oracle.Scaler(2.0 ** 15, 1.0, 10, 1))
    b = oracle.State(p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32),
                     np.zeros(n, np.uint16), oracle.Scaler(2.0 ** 15, 1.0, 10, 1))
    hp = dict(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8)
    oracle.step(a, [g] * K, **hp)
    oracle.step(b, g, **hp)
    # K equal fp16 values sum exactly in fp32 (K = 8 is a power of two), so both unscale to g/S
    assert np.array_equal(a.master.view(np.uint32), b.master.view(np.uint32))
