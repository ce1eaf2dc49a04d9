"""A long run: 2,000 steps of the whole step (fused scaler update, global-norm
clipping, a WarmupDecayLR schedule, dynamic loss scaling with hysteresis 2 and
random overflows) against the oracle, every array compared every 400 steps.
Over this horizon the bias correction approaches 1, the scale goes through
many growth and back-off cycles, and the schedule runs through its warmup,
its decay and past its end; no difference may build up."""
import numpy as np
import pytest

import oracle
import synth
from synth.workloads import BETA1, BETA2, EPS, MASTER_SIGMA
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    return gu.torch_mod()


def test_two_thousand_steps_match_the_oracle(torch):
    from zero_mixed_precision_amd import ShardStep, ZeroMPConfig
    n, steps = 65_541, 2000
    cfg = ZeroMPConfig.from_dict({
        "optimizer": {"type": "AdamW", "params": {"lr": 1e-4, "betas": [BETA1, BETA2], "eps": EPS,
                                                  "weight_decay": 0.01}},
        "scheduler": {"type": "WarmupDecayLR", "params": {"warmup_min_lr": 1e-5, "warmup_max_lr": 3e-4,
                                                          "warmup_num_steps": 100, "total_num_steps": 1500}},
        "fp16": {"enabled": True, "initial_scale_power": 12, "loss_scale_window": 50, "hysteresis": 2},
        "gradient_clipping": 1.0})
    rng = np.random.default_rng(2000)
    idx = np.arange(n)
    master0 = synth.host_master32(synth.stream_key(95, synth.ARR_MASTER), idx, MASTER_SIGMA)
    d = ShardStep(n, cfg, device="cuda:0")
    d.master.copy_(torch.from_numpy(master0))
    d.p16.zero_()
    o = oracle.State(master0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16),
                     oracle.Scaler(cfg.init_scale, cfg.min_loss_scale, cfg.loss_scale_window, cfg.hysteresis))
    sched = oracle.LrSchedule(oracle.LR_WARMUP_DECAY, 1e-5, 3e-4, 100, 1500)
    buf = torch.empty(n, dtype=torch.int16, device="cuda:0")
    overflows = 0
    # gradients drawn with a fixed multiplier 2^12 while the scale the step divides by moves (it grows to
    # 2^23 here): clipping is active while the scale is small and idle once it is large
    spec = synth.GradSpec(0.05, 2.0 ** 12)
    for s in range(steps):
        g = synth.host_grad16(synth.stream_key(96, synth.ARR_GRAD, s), idx, spec)
        if rng.random() < 0.02:
            g[rng.integers(0, n)] = rng.choice([0x7C00, 0xFC00, 0x7E00])
        buf.copy_(torch.from_numpy(g.view(np.int16)))
        d.step(buf)
        ov = oracle.step(o, g, lr=sched, beta1=BETA1, beta2=BETA2, eps=EPS, weight_decay=0.01, max_grad_norm=1.0)
        overflows += ov
        if (s + 1) % 400 == 0:
            gu.check_scaler(d.scaler(), o.scaler, ov, f"long run step {s}")
            du = gu.compare_arrays(f"long run step {s}", gu.host_f32(d.master), gu.host_f32(d.m),
                                   gu.host_f32(d.v), gu.host_u16(d.p16), o.master, o.m, o.v, o.p16)
            gu.say(f"[long run] step {s + 1}: t {o.scaler.applied}, scale {o.scaler.scale}, max ulp {du}")
    assert 10 < overflows < 80 and o.scaler.applied == steps - overflows


def test_two_thousand_double_buffered_steps_with_accumulation_match_the_oracle(torch):
    """The same horizon through ShardStep(double_buffer=True) with K = 2 (no
    clipping: the double-buffered form takes none): even steps hand both
    micro-batches over together (both summed inside the Adam pass), odd steps
    one at a time (the first into the running sum, the second inside the
    pass); the copy that holds the state is compared every 400 steps, and the
    copies switch on every applied step."""
    from zero_mixed_precision_amd import ShardStep, ZeroMPConfig
    n, steps, K = 65_541, 2000, 2
    cfg = ZeroMPConfig.from_dict({
        "optimizer": {"type": "AdamW", "params": {"lr": 1e-4, "betas": [BETA1, BETA2], "eps": EPS,
                                                  "weight_decay": 0.01}},
        "scheduler": {"type": "WarmupDecayLR", "params": {"warmup_min_lr": 1e-5, "warmup_max_lr": 3e-4,
                                                          "warmup_num_steps": 100, "total_num_steps": 1500}},
        "fp16": {"enabled": True, "initial_scale_power": 12, "loss_scale_window": 50, "hysteresis": 2},
        "gradient_accumulation_steps": K})
    rng = np.random.default_rng(2001)
    idx = np.arange(n)
    master0 = synth.host_master32(synth.stream_key(97, synth.ARR_MASTER), idx, MASTER_SIGMA)
    d = ShardStep(n, cfg, device="cuda:0", double_buffer=True)
    d.master.copy_(torch.from_numpy(master0))
    d.p16.zero_()
    o = oracle.State(master0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16),
                     oracle.Scaler(cfg.init_scale, cfg.min_loss_scale, cfg.loss_scale_window, cfg.hysteresis))
    sched = oracle.LrSchedule(oracle.LR_WARMUP_DECAY, 1e-5, 3e-4, 100, 1500)
    bufs = [torch.empty(n, dtype=torch.int16, device="cuda:0") for _ in range(K)]
    spec = synth.GradSpec(1e-3, 2.0 ** 12)
    overflows = 0
    for s in range(steps):
        gs = [synth.host_grad16(synth.stream_key(98, synth.ARR_GRAD, s, k), idx, spec) for k in range(K)]
        if rng.random() < 0.02:
            gs[rng.integers(0, K)][rng.integers(0, n)] = rng.choice([0x7C00, 0xFC00, 0x7E00])
        for b, g in zip(bufs, gs):
            b.copy_(torch.from_numpy(g.view(np.int16)))
        if s % 2 == 0:
            d.full_step(bufs)
        else:
            for b in bufs:
                d.accumulate(b)
            d.step()
        ov = oracle.step(o, gs, lr=sched, beta1=BETA1, beta2=BETA2, eps=EPS, weight_decay=0.01)
        overflows += ov
        if (s + 1) % 400 == 0:
            sc = d.scaler()
            gu.check_scaler(sc, o.scaler, ov, f"double-buffered long run step {s}")
            assert sc.current == o.scaler.applied % 2
            cur = d.current()
            du = gu.compare_arrays(f"double-buffered long run step {s}", gu.host_f32(cur[0]), gu.host_f32(cur[1]),
                                   gu.host_f32(cur[2]), gu.host_u16(cur[3]), o.master, o.m, o.v, o.p16)
            assert max(du.values()) == 0, du
            gu.say(f"[double-buffered long run] step {s + 1}: t {o.scaler.applied}, scale {o.scaler.scale}")
    assert 10 < overflows < 80 and o.scaler.applied == steps - overflows
