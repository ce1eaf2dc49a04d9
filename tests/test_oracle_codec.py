"""Pins of the oracle's fp16 codec and non-finite test against library routines.

The pages fix the storage formats (fp16 parameters and gradients, fp32
master/moments: "DeepSpeed complete guide" section 2, memory table); the
oracle writes the binary16 codec from the IEEE 754 definition, and these tests
check it exhaustively against numpy's own conversions and ``isfinite``.
"""
import concurrent.futures as cf
import os

import numpy as np
import pytest

import oracle


def test_dec16_exhaustive_matches_numpy(oracle_lib):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.dec16(h)
    ref = h.view(np.float16).astype(np.float32)
    # numpy widens NaN payloads the same way, so every pattern matches bit for bit
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))


def test_dec16_spot_values(oracle_lib):
    cases = {0x0000: 0.0, 0x8000: -0.0, 0x0001: 2.0 ** -24, 0x03FF: 1023 * 2.0 ** -24,
             0x0400: 2.0 ** -14, 0x3C00: 1.0, 0xC000: -2.0, 0x7BFF: 65504.0,
             0x7C00: np.inf, 0xFC00: -np.inf}
    for h, want in cases.items():
        got = oracle.lib().zo_dec16(h)
        assert got == want and np.signbit(got) == np.signbit(want), hex(h)
    assert np.isnan(oracle.lib().zo_dec16(0x7E00))
    assert np.isnan(oracle.lib().zo_dec16(0x7C01))


def _enc_chunk(lo: int, count: int) -> int:
    bits = np.arange(lo, lo + count, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    ours = oracle.enc16(x)
    with np.errstate(over="ignore", invalid="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    nan_in = np.isnan(x)
    ok_num = np.array_equal(ours[~nan_in], ref[~nan_in])
    ours_nan = ours[nan_in]
    ok_nan = bool(np.all(((ours_nan & 0x7C00) == 0x7C00) & ((ours_nan & 0x03FF) != 0)))
    return int(ok_num and ok_nan)


def test_enc16_exhaustive_matches_numpy(oracle_lib):
    """All 2^32 fp32 patterns: round-to-nearest-even encode equals numpy's cast
    (NaN inputs: any quiet NaN output)."""
    chunk = 1 << 25
    workers = min(8, len(os.sched_getaffinity(0)))
    with cf.ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(lambda lo: _enc_chunk(lo, chunk), range(0, 1 << 32, chunk)))
    assert all(results)


def test_enc16_rounding_boundaries(oracle_lib):
    f = np.float32
    cases = [
        (f(65504.0), 0x7BFF), (f(65519.996), 0x7BFF), (f(65520.0), 0x7C00),
        (f(2.0 ** -24), 0x0001), (f(2.0 ** -25), 0x0000),            # tie -> even (0)
        (f(3 * 2.0 ** -25), 0x0002),                                   # tie 1.5 -> 2
        (f(np.nextafter(f(2.0 ** -25), f(1))), 0x0001),
        (f(1.0 + 2.0 ** -11), 0x3C00),                                 # tie -> even
        (f(1.0 + 3 * 2.0 ** -11), 0x3C02),                             # tie -> even (up)
        (f(-0.0), 0x8000), (f(np.inf), 0x7C00), (f(-np.inf), 0xFC00),
        (f(2.0 ** -14 - 2.0 ** -25), 0x0400),                          # carries into the normals
    ]
    for x, want in cases:
        assert oracle.lib().zo_enc16(x) == want, (x, hex(want))
    assert oracle.lib().zo_enc16(f(np.nan)) == 0x7E00


def test_nonfinite16_exhaustive_matches_isfinite(oracle_lib):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = ~np.isfinite(h.view(np.float16))
    # single-element arrays: the flag must equal the library's verdict for each pattern
    got = np.array([oracle.any_nonfinite(h[i:i + 1]) for i in range(65536)])
    assert np.array_equal(got, ref)


def test_nonfinite32_patterns_match_isfinite(oracle_lib):
    rng = np.random.default_rng(7)
    bits = np.concatenate([
        rng.integers(0, 1 << 32, 20000, dtype=np.uint64).astype(np.uint32),
        np.array([0x7F800000, 0xFF800000, 0x7FC00000, 0x7F800001, 0xFFFFFFFF, 0x7F7FFFFF,
                  0x00000001, 0x80000000], dtype=np.uint32)])
    x = bits.view(np.float32)
    got = np.array([oracle.any_nonfinite(x[i:i + 1]) for i in range(x.size)])
    assert np.array_equal(got, ~np.isfinite(x))
    assert not oracle.any_nonfinite(np.zeros(0, np.float32))
    assert not oracle.any_nonfinite(np.zeros(0, np.uint16))
