"""GPU parity at the workloads' full sizes, on sampled elements.

The device runs the whole partition (one rank's ZeRO-2 share of 7B at N=64,
a full 7B state, the ragged Llama-like layout with 8 micro-batches, one
rank's ZeRO-1 share of 70B at N=8) in the default launch configuration.  The
oracle runs the same steps on a sample of element indices: 2^20 seeded
uniform indices, the first and last 4096 elements of the partition and of
every bucket, and every injected index.

Every element's update depends only on its own inputs and on the step's
overflow flag, so sampling is exact provided the oracle's flag is the global
one.  It is: the generator only emits entries of finite lookup tables (pinned
on the CPU), so the only non-finite gradients are the injected ones, and all of
those are in the sample; each full micro-batch buffer is also scanned with
torch's isfinite, which must find exactly the injected values.
"""
import numpy as np
import pytest

import oracle
import synth
from synth.workloads import BETA1, BETA2, EPS, LR, MASTER_SIGMA, WORKLOADS, ragged_numels
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

HP = dict(lr=LR, beta1=BETA1, beta2=BETA2, eps=EPS)


@pytest.fixture(scope="module")
def torch():
    t = gu.torch_mod()
    import zero_mixed_precision_amd  # noqa: F401
    return t


def sample_indices(w, buckets, extra=()):
    rng = np.random.default_rng(20261202 + w.cid)
    parts = [rng.integers(0, w.psi, 1 << 20), np.arange(4096), w.psi - 4096 + np.arange(4096), np.array(extra)]
    for start, size in buckets:
        parts += [start + np.arange(min(4096, size)), start + size - np.arange(1, min(4096, size) + 1)]
    for s in w.inject_steps:
        parts.append(np.array([w.injection(s)[1]]))
    return np.unique(np.concatenate(parts).astype(np.int64))


def run_sampled(torch, name, fused=False, bf16=False, fold=1, double=False, extra_inject=None):
    """double: the double-buffered step (K = 1); extra_inject: {step: index} of
    +inf gradients injected beside the workload's own."""
    from zero_mixed_precision_amd import _lib, FlatLayout

    # the largest cases hold up to 285 GB: release what earlier tests left in torch's cache first
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    w = WORKLOADS[name]
    n, K = w.psi, w.K
    # bf16 mode: bf16 gradients N(0, sigma) and bf16 parameter copy, no loss scaling (a static scale of 1)
    spec = synth.GradSpec(w.sigma, 1.0, w.heavy_tail, fmt="bf16") if bf16 else w.grad_spec
    fmt = "bf16" if bf16 else "fp16"
    dt16 = _lib.DS_BF16 if bf16 else _lib.DS_FP16
    init_scale, dynamic = (1.0, False) if bf16 else (w.init_scale, True)
    inf16 = 0x7F80 if bf16 else 0x7C00
    if w.ragged:
        lay = FlatLayout(ragged_numels())
        assert lay.total == n
        buckets = [(b.start, b.size) for b in lay.buckets]
    else:
        buckets = [(0, n)]
    extra_inject = extra_inject or {}
    I = sample_indices(w, buckets, list(extra_inject.values()))
    gu.say(f"[{name}] psi={n} K={K} steps={w.steps} sample={I.size} fused={fused} double={double} {fmt}")

    # oracle state on the sample
    o = oracle.State(synth.host_master32(w.master_key(), I, MASTER_SIGMA), np.zeros(I.size, np.float32),
                     np.zeros(I.size, np.float32), synth.host_grad16(w.p16_key(), I, synth.GradSpec(0.02, 1.0)),
                     oracle.Scaler(init_scale, w.min_scale, w.window, w.hysteresis, dynamic=dynamic), param_fmt=fmt)

    # device state over the whole partition
    tabs = synth.DeviceTables(torch, "cuda:0")
    master = torch.empty(n, dtype=torch.float32, device="cuda:0")
    synth.device_fill_master32(torch, tabs, master, w.master_key(), MASTER_SIGMA)
    m = torch.zeros(n, dtype=torch.float32, device="cuda:0")
    v = torch.zeros(n, dtype=torch.float32, device="cuda:0")
    p16 = torch.empty(n, dtype=torch.int16, device="cuda:0")
    synth.device_fill_grad16(torch, tabs, p16, w.p16_key(), synth.GradSpec(0.02, 1.0))
    g16 = torch.empty(n, dtype=torch.int16, device="cuda:0")
    # fold > 1: the micro-batches of a group are held at once and folded in one pass
    held = [g16] + [torch.empty(n, dtype=torch.int16, device="cuda:0") for _ in range(fold - 1)]
    # the running sum (not needed when one fold folds all K into the double-buffered pass)
    acc = torch.empty(n, dtype=torch.float32, device="cuda:0") if K > 1 and not (double and fold >= K) else None
    # the double-buffered step's second copy of the state (it holds no state yet)
    copy1 = [torch.empty(n, dtype=torch.float32, device="cuda:0") for _ in range(3)] + \
        [torch.empty(n, dtype=torch.int16, device="cuda:0")] if double else None
    st = torch.zeros(_lib.ds_scaler_size(), dtype=torch.uint8, device="cuda:0")
    _lib.ds_state_init(st, init_scale, w.min_scale, w.window, w.hysteresis, 0, int(dynamic))
    Id = torch.from_numpy(I).to("cuda:0")

    for s in range(1, w.steps + 1):
        inj = w.injection(s)
        if inj is None and s in extra_inject:
            inj = (0, int(extra_inject[s]))
        gs_host = []
        for k in range(K):
            buf = held[k % fold]
            synth.device_fill_grad16(torch, tabs, buf, w.grad_key(s, k), spec)
            gh = synth.host_grad16(w.grad_key(s, k), I, spec)
            if inj is not None and inj[0] == k:
                buf[inj[1]] = torch.tensor(inf16, dtype=torch.int32).to(torch.int16)
                gh[np.searchsorted(I, inj[1])] = inf16
            # the whole buffer's non-finite values are exactly the injected one (if any)
            assert gu.count_nonfinite16(torch, buf, fmt) == int(inj is not None and inj[0] == k), \
                f"[{name}] step {s} micro-batch {k}: non-finite values beyond the injected ones"
            gs_host.append(gh)
            group_end = k % fold == fold - 1 or k == K - 1
            if double and K > 1 and k == K - 1:
                # the last fold: summed onto the running sum (if any), checked, and fed to
                # the Adam pass, which writes the other copy; then the scaler update
                first = k - k % fold
                arrays = [[x.data_ptr() for x in (master, copy1[0])], [x.data_ptr() for x in (m, copy1[1])],
                          [x.data_ptr() for x in (v, copy1[2])], [x.data_ptr() for x in (p16, copy1[3])]]
                _lib.ds_accumulate_adam_double_buffered(st, *arrays, dt16, acc if first > 0 else None,
                                                        [held[j % fold] for j in range(first, k + 1)], dt16, n, LR,
                                                        None, BETA1, BETA2, EPS, 0.0, K)
                _lib.ds_update_loss_scale_double_buffered(st)
            elif double and K > 1 and group_end:
                first = k - k % fold
                for start, size in buckets:
                    _lib.ds_accumulate_multi(acc.data_ptr() + 4 * start,
                                             [held[j % fold].data_ptr() + 2 * start for j in range(first, k + 1)],
                                             dt16, size, first == 0, None)
            elif K > 1 and fold == 1:
                for start, size in buckets:
                    _lib.ds_accumulate(acc.data_ptr() + 4 * start, g16.data_ptr() + 2 * start, dt16, size,
                                       k == 0, st if k == K - 1 else None)
            elif K > 1 and (k % fold == fold - 1 or k == K - 1):
                first = k - k % fold
                for start, size in buckets:
                    _lib.ds_accumulate_multi(acc.data_ptr() + 4 * start,
                                             [held[j % fold].data_ptr() + 2 * start for j in range(first, k + 1)],
                                             dt16, size, first == 0, st if k == K - 1 else None)
        if K == 1 and not double:
            _lib.ds_check_overflow(st, g16, dt16, n)
        grad, dt = (g16, dt16) if K == 1 else (acc, _lib.DS_FP32)
        if double and K > 1:
            pass     # the step ended with the last fold above
        elif double:   # one kernel: the check, Adam into the other copy, the scaler update
            _lib.ds_adam_step_double_buffered(st, [master, copy1[0]], [m, copy1[1]], [v, copy1[2]],
                                              [p16, copy1[3]], dt16, grad, dt, n, LR, None, BETA1, BETA2, EPS,
                                              0.0, K)
        elif fused:   # one kernel: Adam, then the last block to finish advances the scaler
            _lib.ds_adam_step_fused(st, master, m, v, p16, dt16, grad, dt, n, LR, None, BETA1, BETA2, EPS,
                                    0.0, 0.0, K)
        else:
            _lib.ds_adam_step(st, master, m, v, p16, dt16, grad, dt, n, LR, BETA1, BETA2, EPS, 0.0, 0.0, K)
            _lib.ds_update_loss_scale(st)
        ov = oracle.step(o, gs_host if K > 1 else gs_host[0], fmt=fmt, **HP)
        assert ov == (inj is not None), f"[{name}] step {s}: oracle flag"
        got = _lib.ds_state_read(st)
        gu.check_scaler(got, o.scaler, ov, f"[{name}] step {s}")
        assert got.blocks_done == 0 and got.db_tickets == 0, f"[{name}] step {s}: block count not reset"
        cur = (master, m, v, p16) if not double or got.current == 0 else tuple(copy1)
        if double:
            assert got.current == o.scaler.applied % 2, f"[{name}] step {s}: current copy"
        if s in (1, w.steps // 2, w.steps) or (double and inj is not None):
            du = gu.compare_arrays(f"[{name}] step {s}", gu.host_f32(cur[0][Id]), gu.host_f32(cur[1][Id]),
                                   gu.host_f32(cur[2][Id]), gu.host_u16(cur[3][Id]), o.master, o.m, o.v, o.p16)
            gu.say(f"[{name}] {fmt} step {s}: scale 2^{int(np.log2(o.scaler.scale))} applied {o.scaler.applied} "
                   f"max ulp {du}")
    del master, m, v, p16, g16, held, acc, st, copy1, cur
    torch.cuda.empty_cache()
    return o.scaler


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "separate_update"])
def test_zero2_shard_of_7b(torch, fused):
    """fused=True is the launch bench.py times by default: the check kernel, then
    the Adam kernel whose last block advances the scaler."""
    sc = run_sampled(torch, "zero2_7b", fused=fused)
    assert sc.applied == 50 and sc.scale == 2.0 ** 16


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "separate_update"])
def test_full_7b_state(torch, fused):
    sc = run_sampled(torch, "full_7b", fused=fused)
    assert sc.applied == 20 and sc.scale == 2.0 ** 16


def test_ragged_layout_with_accumulation(torch):
    sc = run_sampled(torch, "ragged")
    assert sc.applied == 27 and sc.scale == 2.0 ** 14


def test_zero1_shard_of_70b_heavy_tail(torch):
    sc = run_sampled(torch, "zero1_70b")
    assert sc.applied == 10 and sc.scale == 2.0 ** 18


def test_zero1_shard_of_70b_fused_scaler_update(torch):
    """The fused Adam + scaler-update kernel at 8.75e9 elements (about 2.1 million
    blocks, each taking one ticket)."""
    sc = run_sampled(torch, "zero1_70b", fused=True)
    assert sc.applied == 10 and sc.scale == 2.0 ** 18


def test_zero2_shard_of_7b_double_buffered(torch):
    """The double-buffered step (overflow check fused into the Adam pass, the
    update written to the other copy) at the shard's full size, with +inf
    gradients injected at the partition's last element (the ragged tail that
    block 0 takes) in step 7 and at an interior element in step 30."""
    w = WORKLOADS["zero2_7b"]
    sc = run_sampled(torch, "zero2_7b", double=True, extra_inject={7: w.psi - 1, 30: 54_321_987})
    assert sc.applied == 48 and sc.s.skipped == 2


def test_zero2_shard_of_7b_bf16_double_buffered(torch):
    """bf16 gradients and parameter copy (a static scale of 1) through the
    double-buffered step at the shard's full size, with an injected infinity."""
    sc = run_sampled(torch, "zero2_7b", double=True, bf16=True, extra_inject={11: 98_765_431})
    assert sc.applied == 49 and sc.s.skipped == 1 and sc.scale == 1.0


def test_zero1_shard_of_70b_double_buffered(torch):
    """The launch bench.py --double-buffer times: 8.75e9 elements in both copies
    (245 GB of state beside the 17.5 GB gradient), with an overflow injected in
    step 4."""
    sc = run_sampled(torch, "zero1_70b", double=True, extra_inject={4: 6_123_456_789})
    assert sc.applied == 9 and sc.s.skipped == 1


@pytest.mark.parametrize("fold", [1, 8, 3])
def test_ragged_layout_double_buffered(torch, fold):
    """The launch bench.py --workload ragged [--fold F] times by default: two
    copies of the 130 GB state, the earlier micro-batches (or folds) summed per
    bucket, the last micro-batch (fold 1), all eight (fold 8, no running sum) or
    the last two (folds of 3, 3, 2) folded into the double-buffered Adam pass,
    with the workload's injected overflows (in steps 3, 4, 17)."""
    sc = run_sampled(torch, "ragged", fold=fold, double=True)
    assert sc.applied == 27 and sc.scale == 2.0 ** 14


def test_ragged_layout_bf16_double_buffered_fold_of_eight(torch):
    """bf16 gradients and parameter copy (a static scale of 1) on the ragged
    layout, all eight micro-batches summed inside the double-buffered Adam pass,
    with the workload's injected infinities."""
    sc = run_sampled(torch, "ragged", fold=8, double=True, bf16=True)
    assert sc.applied == 27 and sc.scale == 1.0


def test_ragged_layout_fused_scaler_update(torch):
    sc = run_sampled(torch, "ragged", fused=True)
    assert sc.applied == 27 and sc.scale == 2.0 ** 14


@pytest.mark.parametrize("fold", [8, 3])
def test_ragged_layout_folded_accumulation(torch, fold):
    """The launch bench.py --workload ragged --fold F times: the 8 micro-batches
    held at once and folded per bucket (fold 3: groups of 3, 3 and 2), with the
    injected overflows, at full size (eight 13 GB gradient buffers beside the
    130 GB state)."""
    sc = run_sampled(torch, "ragged", fused=True, fold=fold)
    assert sc.applied == 27 and sc.scale == 2.0 ** 14


def test_zero2_shard_of_7b_bf16_fused(torch):
    """bf16 mode at the shard's full size (the launch bench.py --bf16 times): bf16
    gradients and parameter copy, a static scale of 1, the fused scaler update."""
    sc = run_sampled(torch, "zero2_7b", fused=True, bf16=True)
    assert sc.applied == 50 and sc.scale == 1.0


def test_full_7b_bf16_fused(torch):
    sc = run_sampled(torch, "full_7b", fused=True, bf16=True)
    assert sc.applied == 20 and sc.scale == 1.0


def test_zero2_shard_of_7b_clipped(torch):
    """Global-norm clipping at the shard's full size (the launch bench.py --clip 1.0
    times).  The clipping coefficient depends on the whole gradient, so the host
    generates all 109,375,000 gradient values once and takes their exact sum of
    squares (oracle.grad_sumsq); the sampled elements are then updated with the
    oracle's multiplier.  The same gradient is applied in each of three steps (the
    state still moves every step); clipping is active (norm about 10, limit 1)."""
    from zero_mixed_precision_amd import _lib

    w = WORKLOADS["zero2_7b"]
    n, max_norm, steps = w.psi, 1.0, 3
    spec = w.grad_spec
    I = sample_indices(w, [(0, n)])
    key = w.grad_key(1, 0)
    g_full = synth.host_grad16(key, np.arange(n), spec)
    sumsq = oracle.grad_sumsq(g_full, "fp16")
    gs = g_full[I]
    del g_full
    gu.say(f"[zero2_7b clipped] sumsq {sumsq:.6g}, unscaled norm {np.sqrt(sumsq) / w.init_scale:.4g}")

    master0 = synth.host_master32(w.master_key(), I, MASTER_SIGMA)
    o = oracle.State(master0, np.zeros(I.size, np.float32), np.zeros(I.size, np.float32),
                     np.zeros(I.size, np.uint16), oracle.Scaler(w.init_scale, w.min_scale, w.window, w.hysteresis))
    tabs = synth.DeviceTables(torch, "cuda:0")
    master = torch.empty(n, dtype=torch.float32, device="cuda:0")
    synth.device_fill_master32(torch, tabs, master, w.master_key(), MASTER_SIGMA)
    m = torch.zeros(n, dtype=torch.float32, device="cuda:0")
    v = torch.zeros(n, dtype=torch.float32, device="cuda:0")
    p16 = torch.zeros(n, dtype=torch.int16, device="cuda:0")
    g16 = torch.empty(n, dtype=torch.int16, device="cuda:0")
    synth.device_fill_grad16(torch, tabs, g16, key, spec)
    ws = torch.zeros((_lib.ds_sumsq_workspace_bytes(n) + 7) // 8, dtype=torch.float64, device="cuda:0")
    st = torch.zeros(_lib.ds_scaler_size(), dtype=torch.uint8, device="cuda:0")
    _lib.ds_state_init(st, w.init_scale, w.min_scale, w.window, w.hysteresis, 0, 1)
    Id = torch.from_numpy(I).to("cuda:0")
    for s in range(steps):
        _lib.ds_check_overflow_sumsq(st, g16, _lib.DS_FP16, n, ws)
        _lib.ds_adam_step_fused(st, master, m, v, p16, _lib.DS_FP16, g16, _lib.DS_FP16, n, LR, None, BETA1, BETA2,
                                EPS, 0.0, max_norm, 1)
        got = _lib.ds_state_read(st)
        assert abs(got.last_grad_sumsq - sumsq) <= 1e-13 * sumsq, (got.last_grad_sumsq, sumsq)
        mult = oracle.clip_multiplier(sumsq, o.scaler.scale, 1, max_norm)
        assert mult < np.float32(1.0) / np.float32(w.init_scale)          # clipping is active
        oracle.adam_mult(gs, o.master, o.m, o.v, o.p16, mult=mult, t=o.scaler.applied + 1, lr=LR, beta1=BETA1,
                         beta2=BETA2, eps=EPS)
        o.scaler.update(False)
        gu.check_scaler(got, o.scaler, False, f"[zero2_7b clipped] step {s}")
        du = gu.compare_arrays(f"[zero2_7b clipped] step {s}", gu.host_f32(master[Id]), gu.host_f32(m[Id]),
                               gu.host_f32(v[Id]), gu.host_u16(p16[Id]), o.master, o.m, o.v, o.p16)
        gu.say(f"[zero2_7b clipped] step {s}: max ulp {du}")
    del master, m, v, p16, g16, ws, st
    torch.cuda.empty_cache()


def test_ragged_layout_clipped(torch):
    """Clipping on the ragged layout with 8 micro-batches at full size (the launch
    bench.py --workload ragged --clip 1.0 times): the last micro-batch's
    accumulation also gathers the sum of squares of the fp32 sum, bucket by
    bucket, into the state.  The whole sum cannot be formed on the GPU machine's
    host in a test, so the expected values were written beforehand by
    tests/golden/make_ragged_clip_sumsq.py, which regenerates every micro-batch
    gradient on the host, accumulates it with the oracle and sums the squares
    exactly (tests/golden/ragged_clip_sumsq.json: the running sum after each
    bucket and the total, rounded once).  The device's running sum must meet
    every one of them to 1e-12, and the sampled elements are updated by the
    oracle with the multiplier of the stored total; clipping is active (norm
    about 28, limit 1)."""
    import json
    import os

    from zero_mixed_precision_amd import _lib, FlatLayout

    w = WORKLOADS["ragged"]
    n, K, max_norm, steps = w.psi, w.K, 1.0, 2
    golden = json.load(open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                                         "ragged_clip_sumsq.json")))
    lay = FlatLayout(ragged_numels())
    buckets = [(b.start, b.size) for b in lay.buckets]
    assert golden["elements"] == n and golden["buckets"] == [list(b) for b in buckets]
    I = sample_indices(w, buckets)
    spec = w.grad_spec
    master0 = synth.host_master32(w.master_key(), I, MASTER_SIGMA)
    o = oracle.State(master0, np.zeros(I.size, np.float32), np.zeros(I.size, np.float32),
                     np.zeros(I.size, np.uint16), oracle.Scaler(w.init_scale, w.min_scale, w.window, w.hysteresis))
    tabs = synth.DeviceTables(torch, "cuda:0")
    master = torch.empty(n, dtype=torch.float32, device="cuda:0")
    synth.device_fill_master32(torch, tabs, master, w.master_key(), MASTER_SIGMA)
    m = torch.zeros(n, dtype=torch.float32, device="cuda:0")
    v = torch.zeros(n, dtype=torch.float32, device="cuda:0")
    p16 = torch.zeros(n, dtype=torch.int16, device="cuda:0")
    g16 = torch.empty(n, dtype=torch.int16, device="cuda:0")
    acc = torch.empty(n, dtype=torch.float32, device="cuda:0")
    ws = torch.zeros((_lib.ds_sumsq_workspace_bytes(n) + 7) // 8, dtype=torch.float64, device="cuda:0")
    st = torch.zeros(_lib.ds_scaler_size(), dtype=torch.uint8, device="cuda:0")
    _lib.ds_state_init(st, w.init_scale, w.min_scale, w.window, w.hysteresis, 0, 1)
    Id = torch.from_numpy(I).to("cuda:0")
    for s in range(1, steps + 1):
        want = golden["steps"][str(s)]
        running = [float.fromhex(x) for x in want["cumulative_by_bucket"]]
        total = float.fromhex(want["total"])
        acc_s = np.empty(I.size, np.float32)
        for k in range(K):
            key = w.grad_key(s, k)
            synth.device_fill_grad16(torch, tabs, g16, key, spec)
            assert gu.count_nonfinite16(torch, g16) == 0, (s, k)
            oracle.accumulate(acc_s, synth.host_grad16(key, I, spec), overwrite=(k == 0))
            for b, (start, size) in enumerate(buckets):
                a, gp = acc.data_ptr() + 4 * start, g16.data_ptr() + 2 * start
                if k == K - 1:
                    _lib.ds_accumulate_sumsq(a, gp, _lib.DS_FP16, size, k == 0, st, ws)
                    got = _lib.ds_state_read(st).grad_sumsq
                    assert abs(got - running[b]) <= 1e-12 * running[b], (s, b, got, running[b])
                else:
                    _lib.ds_accumulate(a, gp, _lib.DS_FP16, size, k == 0)
        got_pre = _lib.ds_state_read(st)
        assert got_pre.overflow == 0
        assert abs(got_pre.grad_sumsq - total) <= 1e-12 * total, (got_pre.grad_sumsq, total)
        _lib.ds_adam_step_fused(st, master, m, v, p16, _lib.DS_FP16, acc, _lib.DS_FP32, n, LR, None, BETA1, BETA2,
                                EPS, 0.0, max_norm, K)
        got = _lib.ds_state_read(st)
        mult = oracle.clip_multiplier(total, o.scaler.scale, K, max_norm)
        assert mult < np.float32(1.0) / np.float32(w.init_scale * K)      # clipping is active
        oracle.adam_mult(acc_s, o.master, o.m, o.v, o.p16, mult=mult, t=o.scaler.applied + 1, lr=LR, beta1=BETA1,
                         beta2=BETA2, eps=EPS)
        o.scaler.update(False)
        gu.check_scaler(got, o.scaler, False, f"[ragged clipped] step {s}")
        du = gu.compare_arrays(f"[ragged clipped] step {s}", gu.host_f32(master[Id]), gu.host_f32(m[Id]),
                               gu.host_f32(v[Id]), gu.host_u16(p16[Id]), o.master, o.m, o.v, o.p16)
        gu.say(f"[ragged clipped] step {s}: sumsq {total:.6g} (stored), device {got.last_grad_sumsq:.6g}, "
               f"max ulp {du}")
    del master, m, v, p16, g16, acc, ws, st
    torch.cuda.empty_cache()
