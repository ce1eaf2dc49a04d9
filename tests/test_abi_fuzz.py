"""Property tests of the C ABI's argument validation (host only).

A model of the rules in include/dszero.h decides, for random argument sets,
which rules are broken; the entry point must then return one of those rules'
codes (the header fixes what is an error, not which of several errors is
reported first).  Argument sets the model finds valid are not called unless
n == 0 (a no-op): the pointers are fake addresses, so these tests never launch
anything, and they skip themselves where a GPU is visible.
"""
import ctypes

import pytest

hyp = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402

from zero_mixed_precision_amd import _lib  # noqa: E402
from zero_mixed_precision_amd._lib import (DS_ERR_ALIAS, DS_ERR_ALIGN, DS_ERR_DTYPE, DS_ERR_HPARAM,  # noqa: E402
                                           DS_ERR_NULL, DS_ERR_SIZE, DS_OK)

L = _lib.lib
BASES = [0x1000_0000 * k for k in range(1, 8)]
FP16, FP32, BF16 = _lib.DS_FP16, _lib.DS_FP32, _lib.DS_BF16
ESIZE = {FP16: 2, BF16: 2, FP32: 4}
SCALER = 128


def _no_gpu():
    import torch
    return torch.cuda.device_count() == 0   # counts devices without initialising them


pytestmark = pytest.mark.skipif(not _no_gpu(), reason="fake device addresses: CPU-only test")

# weighted toward valid values, so that the later rules are reached too
MAX_N = 2 ** 40      # the largest n the library accepts
sizes = st.sampled_from([-7, -1, 0, 0, 1, 5, 8, 4096, 10 ** 6, 10 ** 6, MAX_N + 1, 2 ** 62])
dtypes = st.sampled_from([FP16] * 4 + [FP32] * 2 + [BF16] * 2 + [0, 4, -1])


def pointer(k):
    """Mostly an aligned base of its own; else None, a misaligned base, or a
    pointer into another array."""
    return st.sampled_from([BASES[k]] * 9 + [None, BASES[k] + 1, BASES[k] + 4, BASES[k] + 8] +
                           [BASES[j] + 16 for j in range(7) if j != k])


def overlap(a, an, b, bn):
    if a is None or b is None or an == 0 or bn == 0:
        return False
    return a < b + bn and b < a + an


def floats_in(valid, invalid):
    return st.sampled_from(list(valid) * 8 + list(invalid))


lrs = floats_in([0.0, 1e-4, 3e-4], [-1e-4, float("nan"), float("inf")])
betas = floats_in([0.0, 0.9, 0.999], [1.0, -0.1, float("nan"), 1.5])
epss = floats_in([1e-8, 1e-6], [0.0, -1e-8, float("inf"), float("nan")])
wds = floats_in([0.0, 0.01], [-0.01, float("nan")])
clips = floats_in([0.0, 1.0], [-1.0, float("inf")])
ksteps = st.sampled_from([1, 2, 8] * 6 + [0, -3])


def _check(rc, broken, ctx):
    if broken:
        assert rc in broken, (rc, broken, ctx)
    else:
        assert rc == DS_OK, (rc, ctx)


@settings(max_examples=1500, deadline=None)
@given(n=sizes, dt=dtypes, pdt=dtypes, st_p=pointer(5), ptrs=st.tuples(*[pointer(k) for k in range(5)]),
       lr=lrs, b1=betas, b2=betas, eps=epss, wd=wds, clip=clips, K=ksteps)
def test_adam_step_validation(n, dt, pdt, st_p, ptrs, lr, b1, b2, eps, wd, clip, K):
    broken = set()
    if n < 0 or n > MAX_N:
        broken.add(DS_ERR_SIZE)
    if dt not in ESIZE or pdt not in (FP16, BF16):
        broken.add(DS_ERR_DTYPE)
    bad_beta = lambda b: not (b == b and 0.0 <= b < 1.0)
    bad_ge0 = lambda x: not (x == x and x != float("inf") and x >= 0.0)
    if bad_ge0(lr) or bad_beta(b1) or bad_beta(b2) or not (eps == eps and eps != float("inf") and eps > 0) \
            or bad_ge0(wd) or bad_ge0(clip) or K < 1:
        broken.add(DS_ERR_HPARAM)
    if st_p is None:
        broken.add(DS_ERR_NULL)
    if n > 0:
        if any(p is None for p in ptrs):
            broken.add(DS_ERR_NULL)
        if any(p is not None and p % 16 for p in ptrs) or (st_p is not None and st_p % 8):
            broken.add(DS_ERR_ALIGN)
        es = ESIZE.get(dt, 2)
        sz = [4 * n, 4 * n, 4 * n, 2 * n, es * n, SCALER]
        allp = list(ptrs) + [st_p]
        if any(overlap(allp[i], sz[i], allp[j], sz[j]) for i in range(6) for j in range(i + 1, 6)):
            broken.add(DS_ERR_ALIAS)
    if not broken and n != 0:
        return                                   # valid: would launch; not called here
    master, m, v, p16, grad = ptrs
    rc = L.ds_adam_step(st_p, master, m, v, p16, pdt, grad, dt, n, lr, b1, b2, eps, wd, clip, K, None)
    _check(rc, broken, (n, dt, pdt, st_p, ptrs, lr, b1, b2, eps, wd, clip, K))


@settings(max_examples=800, deadline=None)
@given(n=sizes, gdt=dtypes, st_p=st.one_of(st.just(None), pointer(5)), acc=pointer(0), g=pointer(1),
       ow=st.sampled_from([0, 1]))
def test_accumulate_validation(n, gdt, st_p, acc, g, ow):
    broken = set()
    if n < 0 or n > MAX_N:
        broken.add(DS_ERR_SIZE)
    if gdt not in (FP16, BF16):
        broken.add(DS_ERR_DTYPE)
    if n > 0:
        if acc is None or g is None:
            broken.add(DS_ERR_NULL)
        if (acc is not None and acc % 16) or (g is not None and g % 16) or (st_p is not None and st_p % 8):
            broken.add(DS_ERR_ALIGN)
        if overlap(acc, 4 * n, g, 2 * n) or overlap(acc, 4 * n, st_p, SCALER) or overlap(g, 2 * n, st_p, SCALER):
            broken.add(DS_ERR_ALIAS)
    if not broken and n != 0:
        return
    rc = L.ds_accumulate(acc, g, gdt, n, ow, st_p, None)
    _check(rc, broken, (n, gdt, st_p, acc, g, ow))


@settings(max_examples=800, deadline=None)
@given(n=sizes, dt=dtypes, st_p=pointer(5), g=pointer(1), ws=pointer(3), ws_short=st.booleans())
def test_check_overflow_validation(n, dt, st_p, g, ws, ws_short):
    # the plain check
    broken = set()
    if n < 0 or n > MAX_N:
        broken.add(DS_ERR_SIZE)
    if dt not in ESIZE:
        broken.add(DS_ERR_DTYPE)
    if st_p is None:
        broken.add(DS_ERR_NULL)
    es = ESIZE.get(dt, 2)
    if n > 0:
        if g is None:
            broken.add(DS_ERR_NULL)
        if (g is not None and g % 16) or (st_p is not None and st_p % 8):
            broken.add(DS_ERR_ALIGN)
        if overlap(g, es * n, st_p, SCALER):
            broken.add(DS_ERR_ALIAS)
    if broken or n == 0:
        _check(L.ds_check_overflow(st_p, g, dt, n, None), broken, ("check", n, dt, st_p, g))
    # the check with the sum of squares: a workspace of 8 bytes per 4096 elements
    need = L.ds_sumsq_workspace_bytes(max(n, 0))
    ws_bytes = max(need - 8, 0) if ws_short else need
    if n > 0:
        if ws is None:
            broken.add(DS_ERR_NULL)
        elif ws % 8:
            broken.add(DS_ERR_ALIGN)
        if ws_short and need > 0:
            broken.add(DS_ERR_SIZE)
        if overlap(g, es * n, ws, need) or overlap(st_p, SCALER, ws, need):
            broken.add(DS_ERR_ALIAS)
    if broken or n == 0:
        rc = L.ds_check_overflow_sumsq(st_p, g, dt, n, ws, ws_bytes, None)
        _check(rc, broken, ("sumsq", n, dt, st_p, g, ws, ws_bytes))


@settings(max_examples=300, deadline=None)
@given(kind=st.sampled_from([0, 1, 2, 3, -1]), lo=floats_in([0.0, 1e-5], [-1e-5, float("nan")]),
       hi=floats_in([3e-4, 1e-3], [float("inf"), -1.0]), w=st.sampled_from([0, 5, 2000, -1]),
       t=st.sampled_from([0, 4, 5, 100000]), n=st.sampled_from([0, -1]))
def test_schedule_validation(kind, lo, hi, w, t, n):
    bad_ge0 = lambda x: not (x == x and x != float("inf") and x >= 0.0)
    broken = set()
    if n < 0 or n > MAX_N:
        broken.add(DS_ERR_SIZE)
    if kind not in (1, 2) or bad_ge0(lo) or bad_ge0(hi) or w < 0 or (kind == 2 and t < w):
        broken.add(DS_ERR_HPARAM)
    sched = _lib.DsLrSchedule(kind, 0, w, t, lo, hi)
    rc = L.ds_adam_step_sched(BASES[5], BASES[0], BASES[1], BASES[2], BASES[3], FP16, BASES[4], FP16, n,
                              ctypes.byref(sched), 0.9, 0.999, 1e-8, 0.0, 0.0, 1, None)
    _check(rc, broken, (kind, lo, hi, w, t, n))
