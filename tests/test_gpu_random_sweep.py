"""GPU parity over random combinations of every option of the step.

Each case draws, from its own seed: the partition size (empty, tiny, around
a tile, or up to 70,000 elements), the micro-batch count and bucket cuts, the
16-bit format (fp16 with dynamic scaling, bf16 with a static scale of 1), the
scaler settings (initial scale, window, hysteresis, consecutive hysteresis,
floor), Adam's hyperparameters (including beta 0 and weight decay), a
constant learning rate or a WarmupLR / WarmupDecayLR schedule, clipping (off,
active or never reached), the fused or the separate scaler update, one
accumulation pass per micro-batch or folds of several (ds_accumulate_multi),
without clipping the double-buffered step (ds_adam_step_double_buffered, the
check inside the Adam pass, two copies of the state) in place of the check and
the in-place update, or with K > 1 the last micro-batch or fold summed into
that pass per bucket (ds_accumulate_adam_double_buffered and
ds_update_loss_scale_double_buffered), and non-finite values planted in random steps,
micro-batches and positions.  The
device runs the step through the C ABI; the oracle runs the same steps.

Bar: scaler state exact after every step; without clipping every array
bit-identical; with clipping (the device's sum of squares is a tree sum, the
oracle's exact) the usual 4 fp32 ulp / 1 16-bit ulp.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

CASES = 200
STEPS = 4


@pytest.fixture(scope="module")
def torch():
    t = gu.torch_mod()
    import zero_mixed_precision_amd  # noqa: F401
    return t


def draw_case(seed):
    r = np.random.default_rng(1_000_003 * seed + 17)
    c = {}
    c["n"] = int(r.choice([0, 1, 7, 8, 4095, 4096, 4097, 8200, int(r.integers(9, 70_000))]))
    c["K"] = int(r.choice([1, 1, 2, 3]))
    c["fmt"] = "bf16" if r.random() < 0.3 else "fp16"
    if c["fmt"] == "fp16":
        c["dynamic"] = bool(r.random() < 0.85)
        c["scale"] = float(2.0 ** int(r.integers(4, 17)))
    else:
        c["dynamic"], c["scale"] = False, 1.0
    c["window"] = int(r.choice([1, 2, 3, 1000]))
    c["hyst"] = int(r.choice([1, 1, 2, 3]))
    c["consec"] = bool(r.random() < 0.3)
    c["min_scale"] = float(r.choice([1.0, 1e-8]))
    c["b1"] = float(r.choice([0.0, 0.5, 0.9, np.float32(r.uniform(0.5, 0.99))]))
    c["b2"] = float(r.choice([0.5, 0.99, 0.999, np.float32(r.uniform(0.9, 0.9999))]))
    c["eps"] = float(r.choice([1e-8, 1e-6, 1e-30]))
    c["wd"] = float(r.choice([0.0, 0.0, 0.01, 0.1]))
    if r.random() < 0.35:
        kind = int(r.choice([oracle.LR_WARMUP, oracle.LR_WARMUP_DECAY]))
        warm = int(r.integers(0, 4))
        c["sched"] = (kind, float(np.float32(r.uniform(0, 1e-4))), float(np.float32(r.uniform(1e-4, 1e-2))), warm,
                      warm + int(r.integers(0, 6)))
    else:
        c["sched"] = None
        c["lr"] = float(np.float32(r.uniform(0, 1e-2)))
    c["clip"] = float(r.choice([0.0, 0.0, 0.05, 1e9]))
    c["fused"] = bool(r.random() < 0.5)
    c["inject"] = {}
    for s in range(STEPS):
        if r.random() < 0.3 and c["n"] > 0:
            c["inject"][s] = (int(r.integers(0, c["K"])), int(r.integers(0, c["n"])), int(r.integers(0, 3)))
    # bucket cuts for the accumulation: multiples of 8 elements
    cuts = sorted({int(x) // 8 * 8 for x in r.integers(0, max(c["n"], 1), int(r.integers(0, 4)))} - {0})
    edges = [0] + [x for x in cuts if x < c["n"]] + [c["n"]]
    c["spans"] = [(a, b - a) for a, b in zip(edges[:-1], edges[1:]) if b > a]
    c["sigma"] = float(r.choice([1e-3, 3e-2]))
    # drawn apart, so that the cases above stay as they were: fold groups of
    # the K micro-batches (ds_accumulate_multi) instead of one pass each
    rf = np.random.default_rng(7_000_003 * seed + 5)
    if c["K"] > 1 and rf.random() < 0.5:
        cut = int(rf.integers(1, c["K"] + 1))
        c["groups"] = [list(range(0, cut)), list(range(cut, c["K"]))] if cut < c["K"] else [list(range(c["K"]))]
    else:
        c["groups"] = None
    # also drawn apart: the double-buffered step (only without clipping)
    rd = np.random.default_rng(9_000_011 * seed + 3)
    c["double"] = c["clip"] == 0.0 and bool(rd.random() < 0.5)
    rq = np.random.default_rng(11_000_027 * seed + 9)
    c["fold_into_pass"] = c["double"] and c["K"] > 1 and bool(rq.random() < 0.6)
    return c


NONFINITE = {"fp16": (0x7C00, 0xFC00, 0x7E00), "bf16": (0x7F80, 0xFF80, 0x7FC0)}


@pytest.mark.parametrize("seed", range(CASES))
def test_random_configuration(torch, seed):
    from zero_mixed_precision_amd import _lib

    c = draw_case(seed)
    n, K, fmt = c["n"], c["K"], c["fmt"]
    gu.say(f"[sweep {seed}] {c}")
    dt16 = _lib.DS_BF16 if fmt == "bf16" else _lib.DS_FP16
    idx = np.arange(n)
    master0 = synth.host_master32(synth.stream_key(4000 + seed, synth.ARR_MASTER), idx, 0.02)
    o = oracle.State(master0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16),
                     oracle.Scaler(c["scale"], c["min_scale"], c["window"], c["hyst"], dynamic=c["dynamic"],
                                   consecutive_hysteresis=c["consec"]), param_fmt=fmt)
    dev = "cuda:0"
    master = gu.dev_f32(torch, master0)
    m = torch.zeros(max(n, 1), device=dev)
    v = torch.zeros(max(n, 1), device=dev)
    p16 = torch.zeros(max(n, 1), dtype=torch.int16, device=dev)
    acc = torch.empty(max(n, 1), device=dev) if K > 1 else None
    # the double-buffered step's second copy (it holds no state yet)
    copy1 = ([torch.empty(max(n, 1), device=dev) for _ in range(3)] +
             [torch.empty(max(n, 1), dtype=torch.int16, device=dev)]) if c["double"] else None
    st = torch.zeros(_lib.ds_scaler_size(), dtype=torch.uint8, device=dev)
    ws = torch.zeros(max(1, (_lib.ds_sumsq_workspace_bytes(n) + 7) // 8), dtype=torch.float64, device=dev)
    _lib.ds_state_init(st, c["scale"], c["min_scale"], c["window"], c["hyst"], int(c["consec"]), int(c["dynamic"]))
    if c["sched"] is not None:
        kind, lo, hi, warm, total = c["sched"]
        lr_o = oracle.LrSchedule(kind, lo, hi, warm, total)
        sched = _lib.DsLrSchedule.make(kind, lo, hi, warm, total)
        lr = 0.0
    else:
        lr_o = lr = c["lr"]
        sched = None
    clip = c["clip"]
    spec = synth.GradSpec(c["sigma"], c["scale"] if fmt == "fp16" else 1.0, fmt=fmt)

    for s in range(STEPS):
        hg = [synth.host_grad16(synth.stream_key(5000 + seed, synth.ARR_GRAD, s, k), idx, spec) for k in range(K)]
        if s in c["inject"]:
            k, i, which = c["inject"][s]
            hg[k][i] = NONFINITE[fmt][which]
        ov = oracle.step(o, hg if K > 1 else hg[0], lr=lr_o, beta1=c["b1"], beta2=c["b2"], eps=c["eps"],
                         weight_decay=c["wd"], max_grad_norm=clip, fmt=fmt)
        gs = [gu.dev_u16(torch, g) if n > 0 else torch.zeros(1, dtype=torch.int16, device=dev) for g in hg]
        if K == 1 and c["double"]:   # the check runs inside the double-buffered pass
            grad, dt = gs[0], dt16
        elif c["fold_into_pass"]:    # earlier groups into the sum; the last one into the pass, per bucket
            grps = c["groups"] if c["groups"] is not None else [[k] for k in range(K)]
            for gi, grp in enumerate(grps[:-1]):
                for start, size in c["spans"]:
                    ptrs = [gs[k].data_ptr() + 2 * start for k in grp]
                    if len(ptrs) == 1:
                        _lib.ds_accumulate(acc.data_ptr() + 4 * start, ptrs[0], dt16, size, gi == 0, None)
                    else:
                        _lib.ds_accumulate_multi(acc.data_ptr() + 4 * start, ptrs, dt16, size, gi == 0, None)
            two = [[x.data_ptr() for x in (a, b)] for a, b in zip((master, m, v, p16), copy1)]
            for start, size in c["spans"]:
                _lib.ds_accumulate_adam_double_buffered(
                    st, *[[x + e * start for x in pair] for pair, e in zip(two, (4, 4, 4, 2))], dt16,
                    acc.data_ptr() + 4 * start if len(grps) > 1 else None,
                    [gs[k].data_ptr() + 2 * start for k in grps[-1]], dt16, size, lr, sched, c["b1"], c["b2"],
                    c["eps"], c["wd"], K)
            _lib.ds_update_loss_scale_double_buffered(st)
            grad, dt = None, None
        elif K == 1:
            if clip > 0:
                _lib.ds_check_overflow_sumsq(st, gs[0], dt16, n, ws)
            else:
                _lib.ds_check_overflow(st, gs[0], dt16, n)
            grad, dt = gs[0], dt16
        elif c["groups"] is not None:
            for gi, grp in enumerate(c["groups"]):
                last = gi == len(c["groups"]) - 1
                for start, size in c["spans"]:
                    _lib.ds_accumulate_multi(acc.data_ptr() + 4 * start, [gs[k].data_ptr() + 2 * start for k in grp],
                                             dt16, size, gi == 0, st if last else None,
                                             ws if (last and clip > 0) else None)
            grad, dt = acc, _lib.DS_FP32
        else:
            for k, g in enumerate(gs):
                last = k == K - 1
                for start, size in c["spans"]:
                    a, gp = acc.data_ptr() + 4 * start, g.data_ptr() + 2 * start
                    if last and clip > 0:
                        _lib.ds_accumulate_sumsq(a, gp, dt16, size, k == 0, st, ws)
                    else:
                        _lib.ds_accumulate(a, gp, dt16, size, k == 0, st if last else None)
            grad, dt = acc, _lib.DS_FP32
        args = (master, m, v, p16, dt16, grad, dt, n)
        tail = (c["b1"], c["b2"], c["eps"], c["wd"], clip, K)
        if c["fold_into_pass"]:
            pass                     # the step ended with the update above
        elif c["double"]:
            _lib.ds_adam_step_double_buffered(st, [master, copy1[0]], [m, copy1[1]], [v, copy1[2]],
                                              [p16, copy1[3]], dt16, grad, dt, n, lr, sched, c["b1"], c["b2"],
                                              c["eps"], c["wd"], K)
        elif c["fused"]:
            _lib.ds_adam_step_fused(st, *args, lr, sched, *tail)
        else:
            if sched is not None:
                _lib.ds_adam_step_sched(st, *args, sched, *tail)
            else:
                _lib.ds_adam_step(st, *args, lr, *tail)
            _lib.ds_update_loss_scale(st)
        ctx = f"[sweep {seed}] step {s}"
        got = _lib.ds_state_read(st)
        gu.check_scaler(got, o.scaler, ov, ctx)
        cur = (master, m, v, p16)
        if c["double"]:
            assert got.current == o.scaler.applied % 2 and got.db_tickets == 0, ctx
            cur = cur if got.current == 0 else tuple(copy1)
        if n > 0:
            du = gu.compare_arrays(ctx, gu.host_f32(cur[0][:n]), gu.host_f32(cur[1][:n]), gu.host_f32(cur[2][:n]),
                                   gu.host_u16(cur[3][:n]), o.master, o.m, o.v, o.p16)
            if clip == 0.0:
                assert max(du.values()) == 0, f"{ctx}: {du}"
