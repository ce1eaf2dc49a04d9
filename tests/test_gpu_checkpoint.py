"""Checkpoint and resume of a shard ("DeepSpeed complete guide" section 5.2):
steps, save, more steps; a fresh shard loaded from the file and given the same
later steps ends bit-identical, and both match the oracle run straight through.
The scaler state travels with the file, so the loss scale, the applied-step
count t and the learning-rate schedule's position resume exactly."""
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


@pytest.mark.parametrize("bf16", [False, True])
def test_save_then_resume_is_bit_identical(torch, tmp_path, bf16):
    from zero_mixed_precision_amd import ShardStep, ZeroMPConfig
    n, K = 100_003, 2
    cfg_dict = {"optimizer": {"type": "AdamW", "params": {"lr": 1e-4, "betas": [BETA1, BETA2], "eps": EPS,
                                                         "weight_decay": 0.01}},
                "scheduler": {"type": "WarmupDecayLR", "params": {"warmup_min_lr": 1e-5, "warmup_max_lr": 3e-4,
                                                                  "warmup_num_steps": 3, "total_num_steps": 7}},
                "gradient_accumulation_steps": K, "gradient_clipping": 1.0}
    if bf16:
        cfg_dict["bf16"] = {"enabled": True}
    else:
        cfg_dict["fp16"] = {"enabled": True, "initial_scale_power": 12, "loss_scale_window": 2, "hysteresis": 1}
    cfg = ZeroMPConfig.from_dict(cfg_dict)
    fmt = "bf16" if bf16 else "fp16"
    master0 = synth.host_master32(synth.stream_key(77, synth.ARR_MASTER), np.arange(n), MASTER_SIGMA)
    spec = synth.GradSpec(0.05, cfg.init_scale, fmt=fmt)
    host = [[synth.host_grad16(synth.stream_key(78, synth.ARR_GRAD, s, k), np.arange(n), spec) for k in range(K)]
            for s in range(8)]
    host[2][1][n // 2] = 0x7F80 if bf16 else 0x7C00
    host[6][0][7] = 0x7F80 if bf16 else 0x7C00
    dev = [[gu.dev_u16(torch, g) for g in gs] for gs in host]

    a = ShardStep(n, cfg, device="cuda:0")
    a.master.copy_(torch.from_numpy(master0))
    a.p16.zero_()
    for s in range(4):
        a.full_step(dev[s])
    path = a.save_checkpoint(str(tmp_path), client_state={"epoch": 3, "note": "mid-run"})
    assert path.endswith("zero_shard_rank00000.safetensors") and "step_4" in path
    for s in range(4, 8):
        a.full_step(dev[s])

    b = ShardStep(n, cfg, device="cuda:0")
    got_path, client = b.load_checkpoint(str(tmp_path))          # the tag named by "latest"
    assert got_path == path and client == {"epoch": 3, "note": "mid-run"}
    for s in range(4, 8):
        b.full_step(dev[s])
    torch.cuda.synchronize()
    for x, y in ((a.master, b.master), (a.m, b.m), (a.v, b.v)):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))
    assert torch.equal(a.p16.view(torch.int16), b.p16.view(torch.int16))
    assert a.scaler().as_dict() == b.scaler().as_dict()

    o = oracle.State(master0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16),
                     oracle.Scaler(cfg.init_scale, cfg.min_loss_scale, cfg.loss_scale_window, cfg.hysteresis,
                                   dynamic=cfg.dynamic), param_fmt=fmt)
    sched = oracle.LrSchedule(oracle.LR_WARMUP_DECAY, 1e-5, 3e-4, 3, 7)
    for s in range(8):
        ov = oracle.step(o, host[s], lr=sched, beta1=BETA1, beta2=BETA2, eps=EPS, weight_decay=0.01,
                         max_grad_norm=1.0, fmt=fmt)
    gu.check_scaler(b.scaler(), o.scaler, ov, "resumed")
    gu.compare_arrays("resumed", gu.host_f32(b.master), gu.host_f32(b.m), gu.host_f32(b.v), gu.host_u16(b.p16),
                      o.master, o.m, o.v, o.p16)


def test_load_rejects_a_different_shard(torch, tmp_path):
    from zero_mixed_precision_amd import ShardStep, ZeroMPConfig
    cfg = ZeroMPConfig()
    a = ShardStep(4096, cfg, device="cuda:0")
    a.master.zero_()
    a.save_checkpoint(str(tmp_path), tag="t0")
    with pytest.raises(ValueError, match="elements"):
        ShardStep(4104, cfg, device="cuda:0").load_checkpoint(str(tmp_path), tag="t0")
    with pytest.raises(ValueError, match="parameter copy"):
        ShardStep(4096, ZeroMPConfig(bf16=True), device="cuda:0").load_checkpoint(str(tmp_path), tag="t0")


def test_load_on_a_raw_stream_handle_and_refuse_a_corrupt_scaler(torch, tmp_path):
    """A shard driven on a raw hipStream_t handle (an int) saves and loads; a file
    whose scaler state was tampered with (a zero loss scale) is refused before
    anything is written to the shard."""
    from safetensors import safe_open
    from safetensors.torch import save_file

    from zero_mixed_precision_amd import ShardStep, ZeroMPConfig
    n = 8192
    side = torch.cuda.Stream()
    cfg = ZeroMPConfig(lr=1e-4)
    g = gu.dev_u16(torch, synth.host_grad16(synth.stream_key(79, synth.ARR_GRAD), np.arange(n),
                                            synth.GradSpec(1e-3, cfg.init_scale)))
    a = ShardStep(n, cfg, device="cuda:0", stream=side.cuda_stream)
    a.master.copy_(torch.from_numpy(synth.host_master32(synth.stream_key(79, synth.ARR_MASTER), np.arange(n),
                                                        MASTER_SIGMA)))
    torch.cuda.synchronize()
    a.step(g)
    path = a.save_checkpoint(str(tmp_path), tag="good")
    b = ShardStep(n, cfg, device="cuda:0", stream=side.cuda_stream)
    b.load_checkpoint(str(tmp_path), tag="good")
    b.step(g)
    a.step(g)
    side.synchronize()
    assert torch.equal(a.master.view(torch.int32), b.master.view(torch.int32))
    assert a.scaler().as_dict() == b.scaler().as_dict()

    with safe_open(path, framework="pt", device="cpu") as f:
        meta = f.metadata()
        tensors = {k: f.get_tensor(k) for k in f.keys()}
    raw = tensors["scaler"].clone()
    raw[0:4] = 0                                   # scale = 0.0
    tensors["scaler"] = raw
    bad = tmp_path / "bad" / "zero_shard_rank00000.safetensors"
    bad.parent.mkdir()
    save_file(tensors, str(bad), metadata=meta)
    c = ShardStep(n, cfg, device="cuda:0", stream=side.cuda_stream)
    c.master.fill_(7.0)
    torch.cuda.synchronize()
    with pytest.raises(ValueError, match="loss-scaler"):
        c.load_checkpoint(str(tmp_path), tag="bad")
    assert bool((c.master == 7.0).all())
