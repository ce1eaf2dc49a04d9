"""GPU parity of the learning-rate schedules (WarmupLR, WarmupDecayLR).

The device reads the schedule at its own applied-step count, so these tests
drive whole steps (with skipped ones in between) and compare every array with
the oracle after every step; the per-step scalars (lr, lr/(1-beta1^t),
1/sqrt(1-beta2^t)) are compared bit for bit over a long range of iterations;
a captured HIP graph is replayed across the warmup and the decay; and a run
resumed from a state snapshot continues the schedule where it stopped.
"""
import numpy as np
import pytest

import oracle
import synth
from synth.workloads import BETA1, BETA2, EPS, MASTER_SIGMA
from tests import gpu_util as gu
from tests._fp import f32_bits

pytestmark = pytest.mark.gpu

SCHEDULES = {
    # the guide's WarmupDecayLR example (section 4.4)
    "page_decay": ("WarmupDecayLR", 0.0, 3e-4, 2000, 100000),
    "warmup": ("WarmupLR", 1e-5, 1e-3, 10, 0),
    "decay_to_min": ("WarmupDecayLR", 1e-5, 3e-4, 5, 25),
    "no_warmup": ("WarmupDecayLR", 0.0, 2e-4, 0, 7),
    "short": ("WarmupDecayLR", 1e-5, 3e-4, 3, 8),
}


@pytest.fixture(scope="module")
def torch():
    t = gu.torch_mod()
    import zero_mixed_precision_amd  # noqa: F401
    return t


def _orc_sched(name):
    kind, lo, hi, w, t = SCHEDULES[name]
    k = oracle.LR_WARMUP if kind == "WarmupLR" else oracle.LR_WARMUP_DECAY
    return oracle.LrSchedule(k, lo, hi, w, t)


def _cfg_block(name):
    kind, lo, hi, w, t = SCHEDULES[name]
    params = dict(warmup_min_lr=lo, warmup_max_lr=hi, warmup_num_steps=w)
    if kind == "WarmupDecayLR":
        params["total_num_steps"] = t
    return {"type": kind, "params": params}


@pytest.mark.parametrize("name", sorted(SCHEDULES))
def test_schedule_scalars_bit_exact(torch, name):
    from zero_mixed_precision_amd import ZeroMPConfig, _lib
    sched = ZeroMPConfig.from_dict({"scheduler": _cfg_block(name)}).lr_schedule()
    orc = _orc_sched(name)
    w, t = sched.warmup_num_steps, sched.total_num_steps
    its = sorted(set(range(0, 600)) | {w - 1, w, w + 1, t - 1, t, t + 1, 1999, 2000, 2001, 51000, 99999,
                                        100000, 100001} | {int(x) for x in np.logspace(3, 8, 60)})
    its = [i for i in its if i >= 0]
    hps = [(BETA1, BETA2), (0.95, 0.98)]
    st = torch.zeros(_lib.ds_scaler_size(), dtype=torch.uint8, device="cuda:0")
    out = torch.zeros((len(hps), len(its), 3), dtype=torch.float32, device="cuda:0")
    _lib.ds_state_init(st, 1.0, 1.0, 1, 1, 0, 1)
    base = _lib.ds_state_read(st)
    for j, it in enumerate(its):
        base.step = it
        _lib.ds_state_write(st, base)
        for a, (b1, b2) in enumerate(hps):
            _lib.ds_lr_scalars(st, sched, b1, b2, out[a, j].data_ptr())
    got = out.cpu().numpy()
    for a, (b1, b2) in enumerate(hps):
        lrs = np.array([orc.at(i) for i in its], np.float32)
        want = np.array([(lr, *oracle.adam_scalars(i + 1, float(lr), b1, b2)) for i, lr in zip(its, lrs)],
                        np.float32)
        assert np.array_equal(f32_bits(got[a]), f32_bits(want)), (name, b1, b2)


def _pair(torch, n, cfg_dict, seed):
    from zero_mixed_precision_amd import ShardStep, ZeroMPConfig
    cfg = ZeroMPConfig.from_dict(cfg_dict)
    fmt = "bf16" if cfg.bf16 else "fp16"
    master0 = synth.host_master32(synth.stream_key(seed, synth.ARR_MASTER), np.arange(n), MASTER_SIGMA)
    d = ShardStep(n, cfg, device="cuda:0")
    d.master.copy_(torch.from_numpy(master0))
    d.p16.zero_()
    o = oracle.State(master0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16),
                     oracle.Scaler(cfg.init_scale, cfg.min_loss_scale, cfg.loss_scale_window, cfg.hysteresis,
                                   dynamic=cfg.dynamic, consecutive_hysteresis=cfg.consecutive_hysteresis),
                     param_fmt=fmt)
    return cfg, fmt, d, o


def _host_grads(seed, step, n, K, spec, inject):
    gs = [synth.host_grad16(synth.stream_key(seed, synth.ARR_GRAD, step, k), np.arange(n), spec)
          for k in range(K)]
    if inject:
        gs[-1][(step * 7919) % n] = 0x7F80 if spec.fmt == "bf16" else 0x7C00
    return gs


def _compare(ctx, d, o):
    gu.compare_arrays(ctx, gu.host_f32(d.master), gu.host_f32(d.m), gu.host_f32(d.v), gu.host_u16(d.p16),
                      o.master, o.m, o.v, o.p16)


CASES = {
    # schedule, K, weight decay, clipping, bf16
    "decay_fp16": ("short", 1, 0.0, 0.0, False),
    "warmup_k3_wd_clip": ("warmup", 3, 0.01, 1.0, False),
    "decay_min_bf16": ("decay_to_min", 1, 0.0, 0.0, True),
    "no_warmup_k2": ("no_warmup", 2, 0.0, 0.0, False),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_scheduled_steps_match_oracle(torch, case):
    sname, K, wd, clip, bf16 = CASES[case]
    n = 3 * 4096 * 4 + 5
    cfg_dict = {"optimizer": {"type": "AdamW", "params": {"lr": 1e-4, "betas": [BETA1, BETA2], "eps": EPS,
                                                         "weight_decay": wd}},
                "scheduler": _cfg_block(sname), "gradient_accumulation_steps": K, "gradient_clipping": clip}
    if bf16:
        cfg_dict["bf16"] = {"enabled": True}
    else:
        cfg_dict["fp16"] = {"enabled": True, "initial_scale_power": 12, "loss_scale_window": 4, "hysteresis": 1}
    cfg, fmt, d, o = _pair(torch, n, cfg_dict, seed=300 + sorted(CASES).index(case))
    spec = synth.GradSpec(1e-3, cfg.init_scale / K if not bf16 else 1.0, fmt=fmt)
    sched = _orc_sched(sname)
    for s in range(14):
        inject = s in (2, 6, 7)
        gs = _host_grads(4321, s, n, K, spec, inject)
        dev = [gu.dev_u16(torch, g) for g in gs]
        d.full_step(dev if K > 1 else dev[0])
        ov = oracle.step(o, gs if K > 1 else gs[0], lr=sched, beta1=BETA1, beta2=BETA2, eps=EPS,
                         weight_decay=wd, max_grad_norm=clip, fmt=fmt)
        assert ov == inject
        gu.check_scaler(d.scaler(), o.scaler, ov, f"{case} step {s}")
        _compare(f"{case} step {s}", d, o)
    assert o.scaler.applied == 11


def test_graph_replays_follow_the_schedule(torch):
    """One capture, many replays: each replay reads the schedule at the device's
    step count, so the lr changes across replays without touching the graph."""
    n = 100_003
    cfg_dict = {"optimizer": {"type": "Adam", "params": {"lr": 1e-4, "betas": [BETA1, BETA2], "eps": EPS}},
                "fp16": {"enabled": True, "initial_scale_power": 14, "loss_scale_window": 3, "hysteresis": 1},
                "scheduler": _cfg_block("short")}
    cfg, fmt, d, o = _pair(torch, n, cfg_dict, seed=55)
    sched = _orc_sched("short")
    buf = torch.zeros(n, dtype=torch.float16, device="cuda:0")
    spec = synth.GradSpec(1e-3, 2.0 ** 14)
    torch.cuda.synchronize()
    g = d.graph([buf])
    torch.cuda.synchronize()
    lrs = []
    for s in range(12):
        host = _host_grads(99, s, n, 1, spec, s in (3, 4))[0]
        buf.copy_(torch.from_numpy(host.view(np.int16)).view(torch.float16))
        lrs.append(sched.at(o.scaler.applied))
        g.replay()
        ov = oracle.step(o, host, lr=sched, beta1=BETA1, beta2=BETA2, eps=EPS)
        torch.cuda.synchronize()
        gu.check_scaler(d.scaler(), o.scaler, ov, f"graph step {s}")
        _compare(f"graph step {s}", d, o)
    assert len(set(lrs)) >= 6


def test_resume_continues_the_schedule(torch):
    """A fresh ShardStep given a snapshot of the arrays and the scaler state
    continues with the same learning rates, bit for bit."""
    from zero_mixed_precision_amd import ShardStep, _lib
    n = 40_961
    cfg_dict = {"optimizer": {"type": "Adam", "params": {"lr": 1e-4, "betas": [BETA1, BETA2], "eps": EPS}},
                "fp16": {"enabled": True, "initial_scale_power": 12, "loss_scale_window": 1000,
                         "hysteresis": 1},
                "scheduler": _cfg_block("decay_to_min")}
    cfg, fmt, a, _ = _pair(torch, n, cfg_dict, seed=66)
    spec = synth.GradSpec(1e-3, 2.0 ** 12)
    grads = [gu.dev_u16(torch, _host_grads(7, s, n, 1, spec, s == 1)[0]) for s in range(9)]
    for s in range(4):
        a.full_step(grads[s])
    b = ShardStep(n, cfg, device="cuda:0")
    for x, y in ((a.master, b.master), (a.m, b.m), (a.v, b.v), (a.p16, b.p16)):
        y.copy_(x)
    _lib.ds_state_write(b.state, a.scaler())
    for s in range(4, 9):
        a.full_step(grads[s])
        b.full_step(grads[s])
    torch.cuda.synchronize()
    for x, y in ((a.master, b.master), (a.m, b.m), (a.v, b.v)):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))
    assert torch.equal(a.p16.view(torch.int16), b.p16.view(torch.int16))
    assert a.scaler().as_dict() == b.scaler().as_dict()
