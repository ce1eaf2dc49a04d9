"""CPU tests of the C ABI: exported symbols, argument validation (every error
is returned before any device work, so these calls never reach the GPU), the
host-only layout/partition entry points against the packing oracle, and the
ds_config keys."""
import ctypes
import json
import os
import re

import numpy as np
import pytest

from oracle import packing
from zero_mixed_precision_amd import _lib, ZeroMPConfig, FlatLayout
from zero_mixed_precision_amd._lib import (DS_BF16, DS_ERR_ALIAS, DS_ERR_ALIGN, DS_ERR_DTYPE,
                                           DS_ERR_HPARAM, DS_ERR_NULL, DS_ERR_SIZE, DS_FP16, DS_FP32, DS_OK)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")
L = _lib.lib

# fake, never-dereferenced device addresses (validation fails before any launch)
A, B, C, D, E, ST = (0x10000000 * k for k in range(1, 7))


def _no_gpu():
    import torch
    return torch.cuda.device_count() == 0   # counts devices without initialising them


# The tests that hand the library fake device addresses run only where no GPU
# is visible: were a validation rule ever lost, the call must not reach a
# kernel that would dereference them.
fake_addresses = pytest.mark.skipif(not _no_gpu(), reason="fake device addresses: CPU-only test")
STREAM = None
HP = (1e-4, 0.9, 0.999, 1e-8, 0.0, 0.0, 1)


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "dszero.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ds_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    syms = declared_symbols()
    assert len(syms) >= 12
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for s in syms:
        assert hasattr(lib, s), s
    assert sorted(_lib.EXPORTED) == syms


def test_nothing_but_the_declared_abi_is_exported():
    """The library's dynamic symbol table holds the declared entry points and no
    C++ helper (the HIP compiler's own module id aside)."""
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    names = {line.split()[-1] for line in out.splitlines() if line.strip()}
    extra = {s for s in names if not s.startswith("ds_") and not s.startswith("__hip_cuid_")}
    assert not extra, sorted(extra)
    assert {s for s in names if s.startswith("ds_")} == set(declared_symbols())


def test_scaler_layout():
    assert L.ds_scaler_size() == 128 == ctypes.sizeof(_lib.DsScaler)
    offs = {n: getattr(_lib.DsScaler, n).offset for n, _ in _lib.DsScaler._fields_}
    assert offs["overflow"] == 28 and offs["step"] == 32 and offs["last_overflow"] == 60
    assert offs["grad_sumsq"] == 64 and offs["last_grad_sumsq"] == 72
    # the tickets and the double-buffered step's copy index; the 64-bit ticket is 8-byte aligned for its atomic
    assert offs["blocks_done"] == 80 and offs["sumsq_blocks_done"] == 84 and offs["current"] == 88
    assert offs["db_tickets"] == 96 and offs["db_tickets"] % 8 == 0


def test_status_strings():
    for s in range(8):
        assert _lib.status_string(s).startswith("DS_")
    assert "unknown" in _lib.status_string(99)


@fake_addresses
def test_accumulate_validation():
    acc = L.ds_accumulate
    assert acc(A, B, DS_FP16, -1, 1, None, STREAM) == DS_ERR_SIZE
    assert acc(A, B, DS_FP16, 0, 1, None, STREAM) == DS_OK                      # n == 0: nothing launched
    assert acc(None, B, DS_FP16, 5, 1, None, STREAM) == DS_ERR_NULL
    assert acc(A, None, DS_FP16, 5, 1, None, STREAM) == DS_ERR_NULL
    assert acc(A + 4, B, DS_FP16, 5, 1, None, STREAM) == DS_ERR_ALIGN
    assert acc(A, B + 2, DS_FP16, 5, 1, None, STREAM) == DS_ERR_ALIGN
    assert acc(A, B, DS_FP16, 5, 1, ST + 4, STREAM) == DS_ERR_ALIGN
    assert acc(A, A + 16, DS_FP16, 8, 1, None, STREAM) == DS_ERR_ALIAS          # acc [A, A+32) vs g16
    assert acc(A, B, DS_FP16, 8, 0, A + 16, STREAM) == DS_ERR_ALIAS             # state inside acc
    assert acc(A, B, DS_FP32, 8, 0, None, STREAM) == DS_ERR_DTYPE             # 16-bit gradients only
    assert acc(A, B, 9, 8, 0, None, STREAM) == DS_ERR_DTYPE


@fake_addresses
def test_accumulate_multi_validation():
    f = L.ds_accumulate_multi
    P = lambda *xs: (ctypes.c_void_p * len(xs))(*xs)
    ws = L.ds_sumsq_workspace_bytes(100)
    assert f(A, P(B, C), 2, DS_FP16, -1, 1, None, None, 0, STREAM) == DS_ERR_SIZE
    assert f(A, P(B, C), 2, DS_FP16, 2 ** 40 + 1, 1, None, None, 0, STREAM) == DS_ERR_SIZE
    assert f(A, P(B), 0, DS_FP16, 8, 1, None, None, 0, STREAM) == DS_ERR_SIZE            # count 1..8
    assert f(A, P(*[B] * 9), 9, DS_FP16, 8, 1, None, None, 0, STREAM) == DS_ERR_SIZE
    assert f(A, P(B, C), 2, DS_FP32, 8, 1, None, None, 0, STREAM) == DS_ERR_DTYPE        # 16-bit only
    assert f(A, P(B, C), 2, DS_FP16, 8, 1, None, D, ws, STREAM) == DS_ERR_NULL           # workspace needs st
    assert f(A, P(B, C), 2, DS_FP16, 0, 1, None, None, 0, STREAM) == DS_OK               # n == 0: nothing
    assert f(None, P(B, C), 2, DS_FP16, 8, 1, None, None, 0, STREAM) == DS_ERR_NULL
    assert f(A, None, 2, DS_FP16, 8, 1, None, None, 0, STREAM) == DS_ERR_NULL
    assert f(A, P(B, None), 2, DS_FP16, 8, 1, None, None, 0, STREAM) == DS_ERR_NULL
    assert f(A + 8, P(B, C), 2, DS_FP16, 8, 1, None, None, 0, STREAM) == DS_ERR_ALIGN
    assert f(A, P(B, C + 2), 2, DS_FP16, 8, 1, None, None, 0, STREAM) == DS_ERR_ALIGN
    assert f(A, P(B, C), 2, DS_FP16, 8, 1, ST + 4, None, 0, STREAM) == DS_ERR_ALIGN
    assert f(A, P(B, C), 2, DS_FP16, 100, 1, ST, D + 4, ws, STREAM) == DS_ERR_ALIGN
    assert f(A, P(B, C), 2, DS_FP16, 100, 1, ST, D, ws - 8, STREAM) == DS_ERR_SIZE     # short workspace
    assert f(A, P(B, A + 16), 2, DS_FP16, 64, 1, None, None, 0, STREAM) == DS_ERR_ALIAS  # a gradient inside acc
    assert f(A, P(B, C), 2, DS_FP16, 64, 0, A + 32, None, 0, STREAM) == DS_ERR_ALIAS     # state inside acc
    assert f(A, P(B, C), 2, DS_FP16, 64, 0, ST, C + 16, 16, STREAM) == DS_ERR_ALIAS      # workspace on a gradient


@fake_addresses
def test_check_overflow_validation():
    chk = L.ds_check_overflow
    assert chk(ST, A, DS_FP16, -1, STREAM) == DS_ERR_SIZE
    assert chk(ST, A, 4, 10, STREAM) == DS_ERR_DTYPE
    assert chk(ST, A, DS_BF16, -1, STREAM) == DS_ERR_SIZE
    assert chk(None, A, DS_FP16, 10, STREAM) == DS_ERR_NULL
    assert chk(ST, A, DS_FP16, 0, STREAM) == DS_OK
    assert chk(ST, None, DS_FP16, 10, STREAM) == DS_ERR_NULL
    assert chk(ST, A + 8, DS_FP32, 10, STREAM) == DS_ERR_ALIGN
    assert chk(ST + 4, A, DS_FP32, 10, STREAM) == DS_ERR_ALIGN
    assert chk(A + 32, A, DS_FP32, 10, STREAM) == DS_ERR_ALIAS


@fake_addresses
def test_sizes_beyond_any_device_are_refused():
    """n above 2^40 elements (more than any device holds) is DS_ERR_SIZE on every
    entry point that takes n, before any byte count is formed from it."""
    big = 2 ** 40 + 1
    ws = L.ds_sumsq_workspace_bytes(big)
    assert L.ds_accumulate(A, B, DS_FP16, big, 1, None, STREAM) == DS_ERR_SIZE
    assert L.ds_check_overflow(ST, A, DS_FP16, big, STREAM) == DS_ERR_SIZE
    assert L.ds_check_overflow_sumsq(ST, A, DS_FP16, big, B, ws, STREAM) == DS_ERR_SIZE
    assert L.ds_accumulate_sumsq(A, B, DS_FP16, big, 1, ST, C, ws, STREAM) == DS_ERR_SIZE
    for n in (big, 2 ** 62, 2 ** 63 - 1):
        assert _adam(n=n) == DS_ERR_SIZE
        assert L.ds_adam_step_fused(ST, A, B, C, D, DS_FP16, E, DS_FP16, n, 1e-4, None, *HP[1:], STREAM) \
            == DS_ERR_SIZE


def test_layout_and_partition_refuse_sizes_beyond_any_device():
    big = 2 ** 40
    for numels, cap, align in (([big + 1], 10, 1), ([big // 2, big // 2, 5], 10, 1), ([5], big + 1, 1),
                               ([5], 10, big + 1), ([2 ** 63 - 1, 2 ** 63 - 1], 10, 8)):
        with pytest.raises(_lib.DsError, match="SIZE"):
            _lib.ds_layout_greedy(numels, cap, align)
    assert _lib.ds_layout_greedy([big // 2 - 64, big // 2 - 64], int(2e8), 64)[4] == big - 128
    with pytest.raises(_lib.DsError, match="SIZE"):
        _lib.ds_partition_range(big + 1, 8, 0, 8)
    with pytest.raises(_lib.DsError, match="SIZE"):
        _lib.ds_partition_range(100, 8, 0, big + 1)
    # the largest total, the largest world: every rank's range is exact
    world = 2 ** 31 - 1
    per = -(-big // world)
    per = -(-per // 8) * 8
    for rank in (0, 1, big // per - 1, big // per, big // per + 1, world - 1):
        start, count = _lib.ds_partition_range(big, world, rank, 8)
        assert start == min(rank * per, big) and count == max(0, min(per, big - start))


def _adam(*, st=ST, ptrs=(A, B, C, D, E), dt=DS_FP16, pdt=DS_FP16, n=16, hp=HP):
    master, m, v, p16, grad = ptrs
    return L.ds_adam_step(st, master, m, v, p16, pdt, grad, dt, n, *hp, STREAM)


@fake_addresses
def test_adam_validation():
    assert _adam(n=-3) == DS_ERR_SIZE
    assert _adam(dt=0) == DS_ERR_DTYPE
    assert _adam(pdt=DS_FP32) == DS_ERR_DTYPE                       # the copy is 16-bit
    assert _adam(pdt=5) == DS_ERR_DTYPE
    assert _adam(n=0) == DS_OK
    assert _adam(st=None) == DS_ERR_NULL
    for k in range(5):
        ptrs = [A, B, C, D, E]
        ptrs[k] = None
        assert _adam(ptrs=tuple(ptrs)) == DS_ERR_NULL
        ptrs = [A, B, C, D, E]
        ptrs[k] += 8
        assert _adam(ptrs=tuple(ptrs)) == DS_ERR_ALIGN
    assert _adam(st=ST + 2) == DS_ERR_ALIGN
    assert _adam(ptrs=(A, A + 32, C, D, E)) == DS_ERR_ALIAS            # master [A, A+64) vs m
    assert _adam(ptrs=(A, B, C, D, D + 16)) == DS_ERR_ALIAS            # p16 vs grad
    assert _adam(st=E + 16) == DS_ERR_ALIAS                            # state inside grad


def _sched_call(sched, st=ST, n=1024, hp=HP[1:]):
    return L.ds_adam_step_sched(st, A, B, C, D, DS_FP16, E, DS_FP16, n,
                                ctypes.byref(sched) if sched is not None else None, *hp, STREAM)


@fake_addresses
def test_schedule_layout_and_validation():
    assert ctypes.sizeof(_lib.DsLrSchedule) == 32
    S = _lib.DsLrSchedule.make
    good = S(_lib.DS_LR_WARMUP_DECAY, 0.0, 3e-4, 2000, 100000)
    assert _sched_call(good, n=0) == DS_OK
    assert _sched_call(good, n=-1) == DS_ERR_SIZE
    assert _sched_call(None) == DS_ERR_NULL
    assert _sched_call(good, st=None) == DS_ERR_NULL
    for bad in [S(0, 0.0, 3e-4, 10, 20), S(3, 0.0, 3e-4, 10, 20), S(1, -1e-5, 3e-4, 10),
                S(1, 0.0, float("nan"), 10), S(1, 0.0, float("inf"), 10), S(1, 0.0, 3e-4, -1),
                S(2, 0.0, 3e-4, 10, 9)]:
        assert _sched_call(bad) == DS_ERR_HPARAM
    # total_num_steps is ignored by WarmupLR
    assert _sched_call(S(1, 0.0, 3e-4, 10, 9), n=0) == DS_OK
    # the other hyperparameters are checked as for the constant-lr step
    assert _sched_call(good, hp=(1.0, 0.999, 1e-8, 0.0, 0.0, 1)) == DS_ERR_HPARAM
    assert _sched_call(good, hp=(0.9, 0.999, 1e-8, 0.0, 0.0, 0)) == DS_ERR_HPARAM
    sc = L.ds_lr_scalars
    assert sc(None, ctypes.byref(good), 0.9, 0.999, A, STREAM) == DS_ERR_NULL
    assert sc(ST, None, 0.9, 0.999, A, STREAM) == DS_ERR_NULL
    assert sc(ST, ctypes.byref(good), 0.9, 0.999, None, STREAM) == DS_ERR_NULL
    assert sc(ST, ctypes.byref(S(7, 0.0, 1e-3, 1)), 0.9, 0.999, A, STREAM) == DS_ERR_HPARAM
    assert sc(ST, ctypes.byref(good), 0.9, 1.0, A, STREAM) == DS_ERR_HPARAM
    assert sc(ST, ctypes.byref(good), 0.9, 0.999, A + 2, STREAM) == DS_ERR_ALIGN
    assert sc(ST, ctypes.byref(good), 0.9, 0.999, ST + 120, STREAM) == DS_ERR_ALIAS


NAN, INF = float("nan"), float("inf")


@fake_addresses
@pytest.mark.parametrize("bad", [
    # lr, beta1, beta2, eps, weight_decay, max_grad_norm, accum_steps
    (-1e-4, 0.9, 0.999, 1e-8, 0.0, 0.0, 1), (NAN, 0.9, 0.999, 1e-8, 0.0, 0.0, 1),
    (INF, 0.9, 0.999, 1e-8, 0.0, 0.0, 1), (1e-4, 1.0, 0.999, 1e-8, 0.0, 0.0, 1),
    (1e-4, -0.1, 0.999, 1e-8, 0.0, 0.0, 1), (1e-4, 0.9, 1.0, 1e-8, 0.0, 0.0, 1),
    (1e-4, 0.9, NAN, 1e-8, 0.0, 0.0, 1), (1e-4, 0.9, 0.999, 0.0, 0.0, 0.0, 1),
    (1e-4, 0.9, 0.999, -1e-8, 0.0, 0.0, 1), (1e-4, 0.9, 0.999, INF, 0.0, 0.0, 1),
    (1e-4, 0.9, 0.999, 1e-8, -0.01, 0.0, 1), (1e-4, 0.9, 0.999, 1e-8, NAN, 0.0, 1),
    (1e-4, 0.9, 0.999, 1e-8, 0.0, 0.0, 0), (1e-4, 0.9, 0.999, 1e-8, 0.0, 0.0, -2),
    (1e-4, 0.9, 0.999, 1e-8, 0.0, -1.0, 1), (1e-4, 0.9, 0.999, 1e-8, 0.0, NAN, 1),
    (1e-4, 0.9, 0.999, 1e-8, 0.0, INF, 1),
])
def test_adam_hyperparameter_validation(bad):
    assert _adam(hp=bad) == DS_ERR_HPARAM


@fake_addresses
def test_sumsq_validation():
    ws_need = L.ds_sumsq_workspace_bytes(10000)
    # one fp64 per 1024-element chunk (10) and per group of 4096 chunk sums (1)
    assert ws_need == 8 * (10 + 1) and L.ds_sumsq_workspace_bytes(0) == 0
    assert L.ds_sumsq_workspace_bytes(1024 * 4096) == 8 * (4096 + 1)
    assert L.ds_sumsq_workspace_bytes(1024 * 4096 + 1) == 8 * (4097 + 2)
    WS = 0x70000000
    chk = L.ds_check_overflow_sumsq
    assert chk(ST, A, DS_FP16, -1, WS, ws_need, STREAM) == DS_ERR_SIZE
    assert chk(ST, A, 9, 10, WS, ws_need, STREAM) == DS_ERR_DTYPE
    assert chk(None, A, DS_FP16, 10, WS, ws_need, STREAM) == DS_ERR_NULL
    assert chk(ST, A, DS_FP16, 0, WS, ws_need, STREAM) == DS_OK
    assert chk(ST, A, DS_FP16, 10000, None, ws_need, STREAM) == DS_ERR_NULL
    assert chk(ST, A, DS_FP16, 10000, WS + 4, ws_need, STREAM) == DS_ERR_ALIGN
    assert chk(ST, A, DS_FP16, 10000, WS, ws_need - 8, STREAM) == DS_ERR_SIZE
    assert chk(ST, A + 8, DS_FP16, 10000, WS, ws_need, STREAM) == DS_ERR_ALIGN
    assert chk(ST, A, DS_FP16, 10000, A + 64, ws_need, STREAM) == DS_ERR_ALIAS
    assert chk(WS + 8, A, DS_FP16, 10000, WS, ws_need, STREAM) == DS_ERR_ALIAS   # state inside ws
    acc = L.ds_accumulate_sumsq
    assert acc(A, B, DS_FP16, -1, 1, ST, WS, ws_need, STREAM) == DS_ERR_SIZE
    assert acc(A, B, DS_FP16, 10000, 1, None, WS, ws_need, STREAM) == DS_ERR_NULL
    assert acc(A, B, DS_FP16, 0, 1, ST, WS, ws_need, STREAM) == DS_OK
    assert acc(None, B, DS_FP16, 10000, 1, ST, WS, ws_need, STREAM) == DS_ERR_NULL
    assert acc(A, B, DS_FP16, 10000, 1, ST, None, ws_need, STREAM) == DS_ERR_NULL
    assert acc(A, B + 4, DS_FP16, 10000, 1, ST, WS, ws_need, STREAM) == DS_ERR_ALIGN
    assert acc(A, B, DS_FP16, 10000, 1, ST, WS, 8, STREAM) == DS_ERR_SIZE
    assert acc(A, B, DS_FP16, 10000, 1, ST, A + 1024, ws_need, STREAM) == DS_ERR_ALIAS
    assert acc(A, A + 16, DS_FP16, 10000, 1, ST, WS, ws_need, STREAM) == DS_ERR_ALIAS
    assert acc(A, B, DS_FP32, 10000, 1, ST, WS, ws_need, STREAM) == DS_ERR_DTYPE


@fake_addresses
def test_state_and_scalar_validation():
    init = L.ds_state_init
    assert init(None, 65536.0, 1.0, 1000, 1, 0, 1, STREAM) == DS_ERR_NULL
    assert init(ST + 4, 65536.0, 1.0, 1000, 1, 0, 1, STREAM) == DS_ERR_ALIGN
    for args in [(0.0, 1.0, 1000, 1), (-1.0, 1.0, 1000, 1), (float("inf"), 1.0, 1000, 1),
                 (65536.0, 0.0, 1000, 1), (65536.0, float("nan"), 1000, 1), (65536.0, 1.0, 0, 1),
                 (65536.0, 1.0, 1000, 0)]:
        assert init(ST, *args, 0, 1, STREAM) == DS_ERR_HPARAM, args
    out = _lib.DsScaler()
    assert L.ds_state_read(None, ctypes.byref(out), STREAM) == DS_ERR_NULL
    assert L.ds_state_read(ST, None, STREAM) == DS_ERR_NULL
    assert L.ds_state_write(None, ctypes.byref(out), STREAM) == DS_ERR_NULL
    assert L.ds_state_write(ST + 1, ctypes.byref(out), STREAM) == DS_ERR_ALIGN
    assert L.ds_update_loss_scale(None, STREAM) == DS_ERR_NULL
    assert L.ds_update_loss_scale(ST + 4, STREAM) == DS_ERR_ALIGN
    assert L.ds_adam_bias_scalars(None, 1e-4, 0.9, 0.999, A, STREAM) == DS_ERR_NULL
    assert L.ds_adam_bias_scalars(ST, 1e-4, 0.9, 0.999, None, STREAM) == DS_ERR_NULL
    assert L.ds_adam_bias_scalars(ST, 1e-4, 1.5, 0.999, A, STREAM) == DS_ERR_HPARAM
    assert L.ds_adam_bias_scalars(ST, 1e-4, 0.9, 0.999, ST + 8, STREAM) == DS_ERR_ALIAS


# -- host-only entry points against the packing oracle --------------------------

def test_layout_matches_packing_oracle_on_the_ragged_layout():
    numels = packing.llama_like_numels()
    assert _lib.ds_layout_greedy(numels, int(2e8), 64) == tuple(packing.greedy_buckets(numels, int(2e8), 64))
    lay = FlatLayout(numels)
    assert lay.total == 6_476_267_520 and len(lay.buckets) == 38


def test_layout_matches_packing_oracle_on_random_layouts():
    rng = np.random.default_rng(3)
    for _ in range(500):
        k = int(rng.integers(0, 30))
        numels = [int(x) for x in rng.integers(0, 3000, k)]
        if k and rng.random() < 0.3:
            numels[int(rng.integers(0, k))] = int(rng.integers(3000, 9000))
        cap, align = int(rng.integers(1, 6000)), int(rng.choice([1, 2, 8, 64]))
        assert _lib.ds_layout_greedy(numels, cap, align) == tuple(packing.greedy_buckets(numels, cap, align))


def test_layout_validation():
    with pytest.raises(_lib.DsError):
        _lib.ds_layout_greedy([3, -1], 10, 1)
    with pytest.raises(_lib.DsError):
        _lib.ds_layout_greedy([3], 0, 1)
    with pytest.raises(_lib.DsError):
        _lib.ds_layout_greedy([3], 10, 0)


def test_partition_matches_packing_oracle():
    rng = np.random.default_rng(4)
    for _ in range(2000):
        total = int(rng.integers(0, 1 << 40))
        world = int(rng.integers(1, 1024))
        rank = int(rng.integers(0, world))
        align = int(rng.choice([1, 8, 64]))
        assert _lib.ds_partition_range(total, world, rank, align) == \
            packing.partition_range(total, world, rank, align)
    for bad in [(-1, 2, 0, 1), (10, 0, 0, 1), (10, 2, 2, 1), (10, 2, -1, 1), (10, 2, 0, 0)]:
        with pytest.raises(_lib.DsError):
            _lib.ds_partition_range(*bad)


def test_partition_buckets_clip():
    lay = FlatLayout([100, 100, 100], bucket_cap=150, align=4)
    start, count = 50, 200
    clipped = lay.buckets_in(start, count)
    assert sum(b.size for b in clipped) == count and clipped[0].start == 0


# -- ds_config keys ("DeepSpeed complete guide" sections 4.1-4.3) ------------------

def test_config_from_the_pages_fp16_block():
    g = json.load(open(os.path.join(GOLDEN, "fp16_config.json")))
    cfg = ZeroMPConfig.from_dict({"fp16": g["fp16_section_4_2"],
                                  "optimizer": {"type": "AdamW", "params": {"lr": 1e-4, "eps": 1e-8}},
                                  "zero_optimization": g["zero_optimization_section_4_1"]})
    assert cfg.dynamic and cfg.init_scale == 65536.0
    assert cfg.loss_scale_window == 1000 and cfg.hysteresis == 2 and cfg.min_loss_scale == 1
    assert cfg.reduce_bucket_size == 200_000_000 and cfg.stage == 2 and cfg.eps == 1e-8
    dbg = ZeroMPConfig.from_dict({"fp16": g["fp16_section_13_1"]})
    assert dbg.init_scale == 4096.0 and dbg.loss_scale_window == 500 and dbg.min_loss_scale == 1e-8
    static = ZeroMPConfig.from_dict({"fp16": {"enabled": True, "loss_scale": 128}})
    assert not static.dynamic and static.init_scale == 128.0


def test_config_rejects_auto_and_other_optimizers():
    with pytest.raises(ValueError):
        ZeroMPConfig.from_dict({"optimizer": {"type": "AdamW", "params": {"lr": "auto"}}})
    with pytest.raises(ValueError):
        ZeroMPConfig.from_dict({"optimizer": {"type": "SGD"}})
    with pytest.raises(ValueError):
        ZeroMPConfig.from_dict({"fp16": {"enabled": False}})


def test_config_scheduler_block_from_the_pages():
    g = json.load(open(os.path.join(GOLDEN, "scheduler_config.json")))
    cfg = ZeroMPConfig.from_dict({"scheduler": g["scheduler_section_4_4"]})
    assert (cfg.scheduler, cfg.warmup_min_lr, cfg.warmup_max_lr) == ("WarmupDecayLR", 0.0, 3e-4)
    assert (cfg.warmup_num_steps, cfg.total_num_steps) == (2000, 100000)
    sch = cfg.lr_schedule()
    assert (sch.kind, sch.warmup_num_steps, sch.total_num_steps) == (_lib.DS_LR_WARMUP_DECAY, 2000, 100000)
    assert abs(sch.warmup_max_lr - 3e-4) < 1e-10 and sch.warmup_min_lr == 0.0 and sch.reserved == 0
    warm = ZeroMPConfig.from_dict({"scheduler": {"type": "WarmupLR", "params": {"warmup_max_lr": 1e-3,
                                                                             "warmup_num_steps": 10}}})
    assert warm.lr_schedule().kind == _lib.DS_LR_WARMUP and warm.warmup_min_lr == 0.0
    assert ZeroMPConfig.from_dict({}).lr_schedule() is None
    # the section 4.1 block resolves its values through a trainer ("auto"): rejected here
    with pytest.raises(ValueError, match="auto"):
        ZeroMPConfig.from_dict({"scheduler": g["scheduler_section_4_1"]})
    # types the guide names without parameters or formula
    for kind in g["supported_types_section_4_4"]:
        if kind not in ("WarmupLR", "WarmupDecayLR"):
            with pytest.raises(ValueError, match="without its parameters"):
                ZeroMPConfig.from_dict({"scheduler": {"type": kind, "params": {}}})
    bad_params = [
        {"type": "Cosine", "params": {"warmup_max_lr": 1e-3, "warmup_num_steps": 1}},
        {"type": "WarmupLR", "params": {"warmup_num_steps": 1}},
        {"type": "WarmupDecayLR", "params": {"warmup_max_lr": 1e-3, "warmup_num_steps": 1}},
        {"type": "WarmupLR", "params": {"warmup_max_lr": 1e-3, "warmup_num_steps": 1, "warmup_type": "log"}},
        {"type": "WarmupLR", "params": {"warmup_max_lr": 1e-3, "warmup_num_steps": 1, "last_batch_iteration": 5}},
        {"type": "WarmupDecayLR", "params": {"warmup_max_lr": 1e-3, "warmup_num_steps": 10,
                                             "total_num_steps": 5}},
        {"type": "WarmupLR", "params": {"warmup_max_lr": -1e-3, "warmup_num_steps": 1}},
    ]
    for blk in bad_params:
        with pytest.raises(ValueError):
            ZeroMPConfig.from_dict({"scheduler": blk})


def test_batch_relation_from_the_pages():
    g = json.load(open(os.path.join(GOLDEN, "batch_relation.json")))
    cfg = ZeroMPConfig.from_dict({k: g[k] for k in ("train_micro_batch_size_per_gpu",
                                                    "gradient_accumulation_steps")})
    assert cfg.train_batch_size(g["world_size"]) == g["train_batch_size"] == 2048
    with pytest.raises(ValueError):
        ZeroMPConfig.from_dict({"train_batch_size": 1000, "world_size": 8,
                                "train_micro_batch_size_per_gpu": 4, "gradient_accumulation_steps": 64})


class _FakeDeviceTensor:
    """Stands in for a GPU tensor: the binding's checks read only these attributes,
    and every call below is rejected before its address is used."""
    is_cuda = True

    def __init__(self, nbytes, esize=2, contiguous=True):
        self._n, self._e, self._c = nbytes // esize, esize, contiguous

    def numel(self):
        return self._n

    def element_size(self):
        return self._e

    def is_contiguous(self):
        return self._c

    def data_ptr(self):
        return A


@fake_addresses
def test_binding_rejects_host_short_and_strided_tensors():
    """Python callers that pass tensors get an error, not a kernel reading an
    address it may not touch: host tensors, non-contiguous tensors and tensors
    shorter than the n elements the call covers are refused before the call."""
    torch = pytest.importorskip("torch")
    n = 1000
    st = _FakeDeviceTensor(128, 1)
    g = _FakeDeviceTensor(2 * n)
    f32 = lambda k=n: _FakeDeviceTensor(4 * k, 4)
    with pytest.raises(ValueError, match="GPU memory"):
        _lib.ds_check_overflow(torch.zeros(128, dtype=torch.uint8), g, DS_FP16, n, stream=0)
    with pytest.raises(ValueError, match="GPU memory"):
        _lib.ds_check_overflow(st, torch.zeros(n, dtype=torch.float16), DS_FP16, n, stream=0)
    with pytest.raises(ValueError, match="contiguous"):
        _lib.ds_check_overflow(st, _FakeDeviceTensor(2 * n, contiguous=False), DS_FP16, n, stream=0)
    with pytest.raises(ValueError, match="gradient"):
        _lib.ds_check_overflow(st, g, DS_FP32, n, stream=0)      # 4 bytes per element of fp32
    with pytest.raises(ValueError, match="ds_scaler"):
        _lib.ds_check_overflow(_FakeDeviceTensor(64, 1), g, DS_FP16, n, stream=0)
    with pytest.raises(ValueError, match="acc"):
        _lib.ds_accumulate(f32(n - 1), g, DS_FP16, n, True, None, stream=0)
    for short in range(5):
        arrays = [f32(), f32(), f32(), _FakeDeviceTensor(2 * n), g]
        arrays[short] = _FakeDeviceTensor(arrays[short].numel() * arrays[short].element_size() - 4,
                                          arrays[short].element_size())
        with pytest.raises(ValueError):
            _lib.ds_adam_step_fused(st, *arrays[:4], DS_FP16, arrays[4], DS_FP16, n, 1e-4, None, 0.9, 0.999,
                                    1e-8, 0.0, 0.0, 1, stream=0)
    with pytest.raises(ValueError, match="workspace"):
        _lib.ds_check_overflow_sumsq(st, _FakeDeviceTensor(200000), DS_FP16, 100000, _FakeDeviceTensor(8, 8),
                                     stream=0)
    with pytest.raises(ValueError, match="out2"):
        _lib.ds_adam_bias_scalars(st, 1e-4, 0.9, 0.999, _FakeDeviceTensor(4, 4), stream=0)
    # integers are raw addresses and pass through to the library's own validation
    with pytest.raises(_lib.DsError, match="SIZE"):
        _lib.ds_check_overflow(ST, A, DS_FP16, -1, stream=0)


@fake_addresses
def test_noalloc_check_validation():
    """ds_check_overflow_sumsq_noalloc validates like ds_check_overflow_sumsq and
    refuses sizes beyond its scratch array before any device work."""
    f = L.ds_check_overflow_sumsq_noalloc
    assert _lib.DS_NOALLOC_MAX_ELEMS == (2 ** 21 - 512) * 8192
    text = open(os.path.join(ROOT, "include", "dszero.h")).read()
    assert re.search(r"#define DS_NOALLOC_MAX_ELEMS %dLL" % _lib.DS_NOALLOC_MAX_ELEMS, text)
    assert f(ST, A, DS_FP16, -1, STREAM) == DS_ERR_SIZE
    assert f(ST, A, DS_FP16, _lib.DS_NOALLOC_MAX_ELEMS + 1, STREAM) == DS_ERR_SIZE
    assert f(ST, A, DS_FP16, 2 ** 40, STREAM) == DS_ERR_SIZE
    assert f(ST, A, 9, 10, STREAM) == DS_ERR_DTYPE
    assert f(None, A, DS_FP16, 10, STREAM) == DS_ERR_NULL
    assert f(ST, A, DS_FP16, 0, STREAM) == DS_OK
    assert f(ST, None, DS_FP16, 10, STREAM) == DS_ERR_NULL
    assert f(ST, A + 8, DS_FP16, 10, STREAM) == DS_ERR_ALIGN
    assert f(ST + 4, A, DS_FP16, 10, STREAM) == DS_ERR_ALIGN
    assert f(A + 64, A, DS_FP16, 10000, STREAM) == DS_ERR_ALIAS


@fake_addresses
def test_double_buffered_step_validation():
    """ds_adam_step_double_buffered validates its eight arrays (two copies of
    master, m, v and the 16-bit copy), the gradient and the state before any
    device work."""
    f = L.ds_adam_step_double_buffered
    V2 = ctypes.c_void_p * 2
    n = 1000
    base = [0x20000000 * k for k in range(1, 9)]
    mst, mm, vv, pp = V2(base[0], base[1]), V2(base[2], base[3]), V2(base[4], base[5]), V2(base[6], base[7])
    G = 0x20000000 * 9
    ok_hp = (1e-4, None, 0.9, 0.999, 1e-8, 0.0, 1)

    def call(st=ST, m2=mst, mo=mm, vo=vv, p2=pp, pdt=DS_FP16, g=G, dt=DS_FP16, nn=n, hp=ok_hp):
        lr, sched, b1, b2, eps, wd, K = hp
        return f(st, m2, mo, vo, p2, pdt, g, dt, nn, lr, sched, b1, b2, eps, wd, K, STREAM)

    assert call(nn=-1) == DS_ERR_SIZE
    assert call(nn=2 ** 40 + 1) == DS_ERR_SIZE
    assert call(dt=9) == DS_ERR_DTYPE
    assert call(pdt=DS_FP32) == DS_ERR_DTYPE
    assert call(st=None) == DS_ERR_NULL
    assert call(m2=None) == DS_ERR_NULL
    assert call(p2=V2(base[6], None)) == DS_ERR_NULL
    assert call(g=None) == DS_ERR_NULL
    assert call(m2=V2(base[0] + 4, base[1])) == DS_ERR_ALIGN
    assert call(st=ST + 4) == DS_ERR_ALIGN
    assert call(m2=V2(base[0], base[0] + 64)) == DS_ERR_ALIAS         # the two copies overlap
    assert call(vo=V2(base[4], base[2] + 16)) == DS_ERR_ALIAS         # v copy 1 inside m copy 0
    assert call(g=base[7] + 32) == DS_ERR_ALIAS                       # the gradient inside a p16 copy
    assert call(st=base[3] + 8) == DS_ERR_ALIAS                       # the state inside an m copy
    for bad in [(-1e-4, None, 0.9, 0.999, 1e-8, 0.0, 1), (1e-4, None, 1.0, 0.999, 1e-8, 0.0, 1),
                (1e-4, None, 0.9, 0.999, 0.0, 0.0, 1), (1e-4, None, 0.9, 0.999, 1e-8, -1.0, 1),
                (1e-4, None, 0.9, 0.999, 1e-8, 0.0, 0),
                (1e-4, ctypes.byref(_lib.DsLrSchedule.make(7, 0.0, 1e-3, 1)), 0.9, 0.999, 1e-8, 0.0, 1)]:
        assert call(hp=bad) == DS_ERR_HPARAM, bad


@fake_addresses
def test_fold_into_double_buffered_step_validation():
    """ds_accumulate_adam_double_buffered validates the eight state arrays, the
    running sum, the gradient list (1 to 8, consistent with accum_steps) and the
    state before any device work; ds_update_loss_scale_double_buffered checks
    its state pointer."""
    f = L.ds_accumulate_adam_double_buffered
    V2 = ctypes.c_void_p * 2
    n = 1000
    base = [0x20000000 * k for k in range(1, 9)]
    mst, mm, vv, pp = V2(base[0], base[1]), V2(base[2], base[3]), V2(base[4], base[5]), V2(base[6], base[7])
    ACC, G = 0x20000000 * 9, 0x20000000 * 10
    ok_hp = (1e-4, None, 0.9, 0.999, 1e-8, 0.0, 8)

    def grads(*ptrs):
        return (ctypes.c_void_p * max(len(ptrs), 1))(*ptrs), len(ptrs)

    def call(st=ST, m2=mst, mo=mm, vo=vv, p2=pp, pdt=DS_FP16, acc=ACC, gl=None, gdt=DS_FP16, nn=n, hp=ok_hp):
        lr, sched, b1, b2, eps, wd, K = hp
        g, count = gl if gl is not None else grads(G)
        return f(st, m2, mo, vo, p2, pdt, acc, g, count, gdt, nn, lr, sched, b1, b2, eps, wd, K, STREAM)

    assert call(nn=-1) == DS_ERR_SIZE
    assert call(nn=2 ** 40 + 1) == DS_ERR_SIZE
    assert call(gl=grads()) == DS_ERR_SIZE                              # no gradient
    assert call(gl=grads(*[G] * 9)) == DS_ERR_SIZE                      # more than 8
    assert call(gdt=DS_FP32) == DS_ERR_DTYPE
    assert call(pdt=9) == DS_ERR_DTYPE
    assert call(acc=None) == DS_ERR_HPARAM                              # 1 gradient, no sum, K = 8
    assert call(gl=grads(*[G] * 8)) == DS_ERR_HPARAM                    # a sum and all 8 gradients
    assert call(st=None) == DS_ERR_NULL
    assert call(m2=None) == DS_ERR_NULL
    assert call(p2=V2(base[6], None)) == DS_ERR_NULL
    assert call(gl=grads(None)) == DS_ERR_NULL
    assert call(m2=V2(base[0] + 4, base[1])) == DS_ERR_ALIGN
    assert call(acc=ACC + 8) == DS_ERR_ALIGN
    assert call(gl=grads(G + 8)) == DS_ERR_ALIGN
    assert call(st=ST + 4) == DS_ERR_ALIGN
    assert call(m2=V2(base[0], base[0] + 64)) == DS_ERR_ALIAS           # the two copies overlap
    assert call(acc=base[2] + 16) == DS_ERR_ALIAS                       # the sum inside an m copy
    assert call(gl=grads(ACC + 32)) == DS_ERR_ALIAS                     # a gradient inside the sum
    assert call(gl=grads(G, base[7] + 32)) == DS_ERR_ALIAS              # a gradient inside a p16 copy
    assert call(st=ACC + 8) == DS_ERR_ALIAS                             # the state inside the sum
    for bad in [(-1e-4, None, 0.9, 0.999, 1e-8, 0.0, 8), (1e-4, None, 1.0, 0.999, 1e-8, 0.0, 8),
                (1e-4, None, 0.9, 0.999, 0.0, 0.0, 8), (1e-4, None, 0.9, 0.999, 1e-8, -1.0, 8),
                (1e-4, None, 0.9, 0.999, 1e-8, 0.0, 0),
                (1e-4, ctypes.byref(_lib.DsLrSchedule.make(7, 0.0, 1e-3, 1)), 0.9, 0.999, 1e-8, 0.0, 8)]:
        assert call(hp=bad) == DS_ERR_HPARAM, bad
    assert call(nn=0) == DS_OK                                          # nothing to do: no launch
    assert L.ds_update_loss_scale_double_buffered(None, STREAM) == DS_ERR_NULL
    assert L.ds_update_loss_scale_double_buffered(ST + 4, STREAM) == DS_ERR_ALIGN
