"""One rank's share of a ragged layout, end to end: FlatLayout packs ragged
tensors into greedy buckets, partition() gives rank r of N its contiguous
range, buckets_in() clips the buckets to it, and ShardStep accumulates K
micro-batches bucket by bucket, checks, and steps; the result equals the
oracle's on the same range (the layout only decides how the work is cut)."""
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


@pytest.mark.parametrize("rank", [0, 1, 3])
def test_rank_share_of_a_ragged_layout(torch, rank):
    from zero_mixed_precision_amd import FlatLayout, ShardStep, ZeroMPConfig
    # a small Llama-like stack: 3 layers of q, k, v, o, gate, up, down, two norms (h = 96, f = 264)
    h, f = 96, 264
    numels = [x for _ in range(3) for x in (h * h,) * 4 + (f * h,) * 3 + (h, h)]
    lay = FlatLayout(numels, bucket_cap=40_000, align=64)
    assert len(lay.buckets) > 3
    world, K = 4, 3
    start, count = lay.partition(world, rank)
    assert count > 0 and start % 8 == 0
    buckets = lay.buckets_in(start, count)
    assert sum(b.size for b in buckets) == count
    cfg = ZeroMPConfig.from_dict({"optimizer": {"type": "Adam", "params": {"lr": 1e-4, "betas": [BETA1, BETA2],
                                                                           "eps": EPS}},
                                  "fp16": {"enabled": True, "initial_scale_power": 14, "loss_scale_window": 2,
                                           "hysteresis": 1},
                                  "gradient_accumulation_steps": K})
    idx = start + np.arange(count)
    master0 = synth.host_master32(synth.stream_key(90, synth.ARR_MASTER), idx, MASTER_SIGMA)
    d = ShardStep(count, cfg, device="cuda:0", buckets=buckets)
    d.master.copy_(torch.from_numpy(master0))
    d.p16.zero_()
    o = oracle.State(master0.copy(), np.zeros(count, np.float32), np.zeros(count, np.float32),
                     np.zeros(count, np.uint16), oracle.Scaler(2.0 ** 14, 1.0, 2, 1))
    spec = synth.GradSpec(1e-3, 2.0 ** 14)
    for s in range(5):
        gs = [synth.host_grad16(synth.stream_key(91, synth.ARR_GRAD, s, k), idx, spec) for k in range(K)]
        if s == 2:
            gs[1][count // 2] = 0x7C00           # an overflow in a middle micro-batch
        for g in gs:
            d.accumulate(gu.dev_u16(torch, g))
        d.step()
        ov = oracle.step(o, gs, lr=1e-4, beta1=BETA1, beta2=BETA2, eps=EPS)
        gu.check_scaler(d.scaler(), o.scaler, ov, f"rank {rank} step {s}")
        gu.compare_arrays(f"rank {rank} step {s}", gu.host_f32(d.master), gu.host_f32(d.m), gu.host_f32(d.v),
                          gu.host_u16(d.p16), o.master, o.m, o.v, o.p16)
    assert o.scaler.applied == 4


def test_misuse_is_refused_before_any_device_work(torch):
    """Host, short, wide or strided gradients and out-of-order calls raise, and
    leave the device state as it was."""
    from zero_mixed_precision_amd import ShardStep, ZeroMPConfig, _lib

    n = 4099
    one = ShardStep(n, ZeroMPConfig(lr=1e-4), device="cuda:0")
    three = ShardStep(n, ZeroMPConfig(lr=1e-4, gradient_accumulation_steps=3), device="cuda:0")
    g = torch.zeros(n, dtype=torch.float16, device="cuda:0")
    bad = [torch.zeros(n, dtype=torch.float16),                      # host memory
           torch.zeros(n - 1, dtype=torch.float16, device="cuda:0"),  # short
           torch.zeros(n, dtype=torch.float32, device="cuda:0"),      # not 16-bit
           torch.zeros(2 * n, dtype=torch.float16, device="cuda:0")[::2]]   # strided
    for b in bad:
        with pytest.raises(ValueError):
            one.step(b)
        with pytest.raises(ValueError):
            three.accumulate(b)
    with pytest.raises(RuntimeError):
        one.accumulate(g)                 # K = 1 takes the gradient in step()
    three.accumulate(g)
    with pytest.raises(RuntimeError):
        three.step()                      # one of three micro-batches
    three.accumulate(g)
    three.accumulate(g)
    with pytest.raises(RuntimeError):
        three.accumulate(g)               # a fourth
    # the binding refuses host tensors and short tensors as well
    with pytest.raises(ValueError):
        _lib.ds_check_overflow(one.state, g.cpu(), _lib.DS_FP16, n)
    with pytest.raises(ValueError):
        _lib.ds_adam_step_fused(one.state, one.master, one.m, one.v, one.p16, _lib.DS_FP16, g[:-8], _lib.DS_FP16,
                                n, 1e-4, None, 0.9, 0.999, 1e-8, 0.0, 0.0, 1)
    assert one.scaler().iter == 0 and three.scaler().iter == 0
    three.step()
    assert three.scaler().iter == 1 and three.scaler().step == 1
