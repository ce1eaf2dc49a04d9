"""GPU test of ds_check_overflow_sumsq_noalloc, the check with the gradient's sum
of squares that keeps its partial sums in the library's own device array
instead of a caller workspace.  Through the C ABI it must give the same
overflow flag and the same fp64 sum of squares, bit for bit, as
ds_check_overflow_sumsq with a caller-owned workspace, on consecutive calls
(the array keeps the previous call's contents), the later ones smaller, in
every gradient format; the sum also meets the oracle's exact sum of squares
to 1e-13.  At the largest size the array takes, the two forms agree bit for
bit as well.
"""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    torch = gu.torch_mod()
    from zero_mixed_precision_amd import _lib
    return torch, _lib


def _grad(fmt, n, seed, inject=None):
    """Host gradient values of n elements (uint16 bits, or fp32 values)."""
    key = synth.stream_key(4242, synth.ARR_GRAD, seed)
    if fmt == "fp32":
        g = synth.host_master32(key, np.arange(n), 30.0)
        if inject is not None:
            g[inject] = np.float32(np.inf)
        return g
    g = synth.host_grad16(key, np.arange(n), synth.GradSpec(1e-3, 2.0 ** 15, fmt=fmt))
    if inject is not None:
        g[inject] = 0x7F80 if fmt == "bf16" else 0x7C00
    return g


def _scaler(torch, L):
    st = torch.zeros(L.ds_scaler_size(), dtype=torch.uint8, device="cuda:0")
    L.ds_state_init(st, 2.0 ** 15, 1.0, 1000, 1, 0, 1)
    return st


@pytest.mark.parametrize("fmt", ["fp16", "bf16", "fp32"])
def test_noalloc_matches_workspace_entry_point(env, fmt):
    torch, L = env
    dt = {"fp16": L.DS_FP16, "bf16": L.DS_BF16, "fp32": L.DS_FP32}[fmt]
    st_ws, st_na = _scaler(torch, L), _scaler(torch, L)
    # three calls in a row on the same two states: a large one (several groups
    # of chunk sums, a ragged tail), then two smaller ones, the last with a
    # non-finite value; each call adds its sum of squares to the state's
    for n, seed, inject in ((40_000_003, 1, None), (100_005, 2, None), (8_197, 3, 5_000)):
        g = _grad(fmt, n, seed, inject)
        gd = gu.dev_f32(torch, g) if fmt == "fp32" else gu.dev_u16(torch, g)
        ws = torch.empty((L.ds_sumsq_workspace_bytes(n) + 7) // 8, dtype=torch.float64, device="cuda:0")
        gu.say(f"[noalloc {fmt}] n={n} seed={seed} inject={inject}")
        L.ds_check_overflow_sumsq(st_ws, gd, dt, n, ws)
        L.ds_check_overflow_sumsq_noalloc(st_na, gd, dt, n)
        a, b = L.ds_state_read(st_ws), L.ds_state_read(st_na)
        assert a.overflow == b.overflow == (1 if inject is not None else 0)
        assert np.float64(a.grad_sumsq).view(np.uint64) == np.float64(b.grad_sumsq).view(np.uint64), \
            (fmt, n, a.grad_sumsq, b.grad_sumsq)
        assert b.sumsq_blocks_done == 0
        if seed == 1:   # the first call's sum is the state's whole sum
            exact = oracle.grad_sumsq(g, "bf16" if fmt == "bf16" else "fp16")
            assert abs(b.grad_sumsq - exact) <= 1e-13 * exact
        del gd, ws
    torch.cuda.synchronize()


def test_noalloc_through_the_raw_c_abi(env):
    """The entry point called with raw device addresses and torch's stream
    handle, as a C caller would, then a smaller call on the same stream."""
    torch, L = env
    stream = torch.cuda.current_stream()
    for n in (1_000_001, 4_099):
        g = _grad("fp16", n, 10 + n % 7)
        gd = gu.dev_u16(torch, g)
        st = _scaler(torch, L)
        rc = L.lib.ds_check_overflow_sumsq_noalloc(ctypes.c_void_p(st.data_ptr()), ctypes.c_void_p(gd.data_ptr()),
                                                   L.DS_FP16, n, ctypes.c_void_p(stream.cuda_stream))
        assert rc == L.DS_OK
        got = L.ds_state_read(st, stream)
        exact = oracle.grad_sumsq(g, "fp16")
        assert got.overflow == 0 and abs(got.grad_sumsq - exact) <= 1e-13 * exact
    assert L.lib.ds_check_overflow_sumsq_noalloc(ctypes.c_void_p(st.data_ptr()), ctypes.c_void_p(gd.data_ptr()),
                                                 L.DS_FP16, L.DS_NOALLOC_MAX_ELEMS + 1,
                                                 ctypes.c_void_p(stream.cuda_stream)) == L.DS_ERR_SIZE


def test_noalloc_at_its_maximum_size(env):
    """At exactly DS_NOALLOC_MAX_ELEMS fp16 elements (a 34 GB gradient drawn on
    the device), where the chunk sums and their group sums fill the library's
    array to its last slot: the same sum of squares, bit for bit, as the
    workspace form on a clean gradient, and the flag on one with an infinity
    in its last chunk (the maximum is a whole number of 8192-element chunks)."""
    torch, L = env
    n = L.DS_NOALLOC_MAX_ELEMS
    tabs = synth.DeviceTables(torch, "cuda:0")
    g = torch.empty(n, dtype=torch.int16, device="cuda:0")
    synth.device_fill_grad16(torch, tabs, g, synth.stream_key(4243, synth.ARR_GRAD, 0),
                             synth.GradSpec(1e-3, 2.0 ** 15))
    ws = torch.empty((L.ds_sumsq_workspace_bytes(n) + 7) // 8, dtype=torch.float64, device="cuda:0")
    for inject in (None, n - 3):
        if inject is not None:
            g[inject] = 0x7C00
        st_ws, st_na = _scaler(torch, L), _scaler(torch, L)
        gu.say(f"[noalloc max] n={n} inject={inject}")
        L.ds_check_overflow_sumsq(st_ws, g, L.DS_FP16, n, ws)
        L.ds_check_overflow_sumsq_noalloc(st_na, g, L.DS_FP16, n)
        a, b = L.ds_state_read(st_ws), L.ds_state_read(st_na)
        assert a.overflow == b.overflow == (0 if inject is None else 1)
        if inject is None:
            assert np.isfinite(a.grad_sumsq) and a.grad_sumsq > 0
            assert np.float64(a.grad_sumsq).view(np.uint64) == np.float64(b.grad_sumsq).view(np.uint64), \
                (a.grad_sumsq, b.grad_sumsq)
        assert b.sumsq_blocks_done == 0
    del g, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
