"""Independent partitions stepped concurrently: each ShardStep on a stream of
its own (default priority), driven from its own host thread, with the steps of
the two interleaved on the device.  The library keeps no mutable global state,
so each partition's result must equal the oracle's as if it ran alone.
"""
import threading

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


def _partition(torch, n, K, seed, clip, sched):
    from zero_mixed_precision_amd import ShardStep, ZeroMPConfig
    cfg_dict = {"optimizer": {"type": "Adam", "params": {"lr": 1e-4, "betas": [BETA1, BETA2], "eps": EPS}},
                "fp16": {"enabled": True, "initial_scale_power": 13, "loss_scale_window": 3, "hysteresis": 1},
                "gradient_accumulation_steps": K, "gradient_clipping": clip}
    if sched:
        cfg_dict["scheduler"] = {"type": "WarmupDecayLR", "params": {"warmup_min_lr": 0.0, "warmup_max_lr": 3e-4,
                                                                     "warmup_num_steps": 2, "total_num_steps": 6}}
    cfg = ZeroMPConfig.from_dict(cfg_dict)
    stream = torch.cuda.Stream()
    master0 = synth.host_master32(synth.stream_key(seed, synth.ARR_MASTER), np.arange(n), MASTER_SIGMA)
    d = ShardStep(n, cfg, device="cuda:0", stream=stream)
    with torch.cuda.stream(stream):
        d.master.copy_(torch.from_numpy(master0))
        d.p16.zero_()
    o = oracle.State(master0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16),
                     oracle.Scaler(2.0 ** 13, 1.0, 3, 1))
    lr = (oracle.LrSchedule(oracle.LR_WARMUP_DECAY, 0.0, 3e-4, 2, 6) if sched else 1e-4)
    spec = synth.GradSpec(1e-3, 2.0 ** 13)
    steps = 8
    host = [[synth.host_grad16(synth.stream_key(seed, synth.ARR_GRAD, s, k), np.arange(n), spec) for k in range(K)]
            for s in range(steps)]
    for s in (2, 5):
        host[s][K - 1][(s * 977) % n] = 0x7C00
    with torch.cuda.stream(stream):
        dev = [[torch.from_numpy(g.view(np.int16)).to("cuda:0") for g in gs] for gs in host]
    stream.synchronize()
    return dict(d=d, o=o, stream=stream, host=host, dev=dev, K=K, lr=lr, clip=clip, steps=steps)


def _drive(p, barrier, errors):
    try:
        barrier.wait()
        for gs in p["dev"]:
            p["d"].full_step(gs if p["K"] > 1 else gs[0])
    except Exception as e:  # surfaced by the main thread
        errors.append(e)


def test_two_partitions_on_two_streams_from_two_threads(torch):
    parts = [_partition(torch, 300_007, 1, 71, 0.0, True), _partition(torch, 150_001, 4, 72, 1.0, False)]
    torch.cuda.synchronize()
    barrier, errors = threading.Barrier(len(parts)), []
    threads = [threading.Thread(target=_drive, args=(p, barrier, errors)) for p in parts]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
        assert not t.is_alive(), "a driving thread did not finish"
    assert not errors, errors
    for p in parts:
        p["stream"].synchronize()
    for i, p in enumerate(parts):
        o = p["o"]
        for s, gs in enumerate(p["host"]):
            ov = oracle.step(o, gs if p["K"] > 1 else gs[0], lr=p["lr"], beta1=BETA1, beta2=BETA2, eps=EPS,
                             max_grad_norm=p["clip"])
        d = p["d"]
        gu.check_scaler(d.scaler(), o.scaler, ov, f"partition {i}")
        gu.compare_arrays(f"partition {i}", gu.host_f32(d.master), gu.host_f32(d.m), gu.host_f32(d.v),
                          gu.host_u16(d.p16), o.master, o.m, o.v, o.p16)
        assert o.scaler.applied == p["steps"] - 2
