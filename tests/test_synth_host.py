"""CPU checks of the seeded input generator (host side)."""
import numpy as np

import synth


def test_splitmix64_published_vector():
    # SplitMix64 seeded with 1234567: first five outputs of the reference generator
    want = [6457827717110365317, 3203168211198807973, 9817491932198370423,
            4593380528125082431, 16408922859458223821]
    assert [synth.mix64(1234567 + (i + 1) * synth.GOLDEN) for i in range(5)] == want
    assert synth.raw64(1234567, np.arange(5)).tolist() == want


def test_generator_is_a_function_of_index():
    key = synth.stream_key(9, synth.ARR_GRAD, 3, 0)
    spec = synth.GradSpec(1e-3, 2.0 ** 16)
    full = synth.host_grad16(key, np.arange(10000), spec)
    idx = np.array([0, 5, 9999, 1234])
    assert np.array_equal(synth.host_grad16(key, idx, spec), full[idx])
    other = synth.host_grad16(synth.stream_key(9, synth.ARR_GRAD, 4, 0), np.arange(10000), spec)
    assert (other != full).mean() > 0.9


def test_gradient_distribution():
    spec = synth.GradSpec(1e-3, 2.0 ** 16)
    g = synth.host_grad16(synth.stream_key(1, 2, 3), np.arange(1 << 20), spec)
    x = g.view(np.float16).astype(np.float64) / 2.0 ** 16
    assert np.all(np.isfinite(x))
    assert abs(x.mean()) < 1e-5 and abs(x.std() - 1e-3) < 2e-5
    assert np.abs(x).max() < 4.4e-3        # |z| <= 4.17 before the fp16 rounding


def test_heavy_tail_fraction():
    spec = synth.GradSpec(5e-4, 2.0 ** 16, heavy_tail=True)
    n = 1 << 21
    g = synth.host_grad16(synth.stream_key(5, 3, 1), np.arange(n), spec)
    x = np.abs(g.view(np.float16).astype(np.float64)) / 2.0 ** 16
    frac = (x > 5e-4 * 5).mean()         # beyond 5 sigma only the x100 draws remain
    assert 0.0006 < frac < 0.0011
    assert np.all(np.isfinite(x)) and x.max() < 65504 / 2.0 ** 16


def test_master_distribution():
    m = synth.host_master32(synth.stream_key(1, synth.ARR_MASTER), np.arange(1 << 20), 0.02)
    assert m.dtype == np.float32 and np.all(np.isfinite(m))
    assert abs(m.mean()) < 1e-4 and abs(m.std() - 0.02) < 2e-4
    assert np.unique(m).size > 500000


def test_tables_are_finite_at_every_workload_scale():
    for sigma, mult in [(1e-3, 2.0 ** 16), (1e-3, 2.0 ** 15), (5e-4, 2.0 ** 16)]:
        assert np.all(np.isfinite(synth.table16(sigma * mult).view(np.float16)))
    assert np.all(np.isfinite(synth.table16(5e-4 * 2.0 ** 16 * 100).view(np.float16)))


def test_inject_site_in_range():
    for s in range(50):
        k, i = synth.inject_site((4, synth.ARR_INJECT, s), 6_476_267_520, micro=8)
        assert 0 <= k < 8 and 0 <= i < 6_476_267_520
