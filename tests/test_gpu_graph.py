"""HIP-graph capture of a whole step: every replay matches eager execution.

The graph is replayed several times with the program's own eager work (new
gradients written into the captured buffers) and host synchronisation in
between, and each replay is compared bit for bit with an eager ShardStep fed
the same gradients, and with the oracle.
"""
import numpy as np
import pytest

import oracle
import synth
from synth.workloads import BETA1, BETA2, EPS, LR, MASTER_SIGMA
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    return gu.torch_mod()


@pytest.mark.parametrize("K,clip", [(1, 0.0), (4, 0.0), (1, 0.05), (4, 0.05)])
def test_graph_replays_match_eager_and_oracle(torch, K, clip):
    """clip > 0: the captured step also holds the sum-of-squares passes and their
    workspace (the unscaled gradient's norm is about 0.45, so clipping is active)."""
    from zero_mixed_precision_amd import ShardStep, ZeroMPConfig
    n = 200_003
    cfg = ZeroMPConfig(lr=LR, betas=(BETA1, BETA2), eps=EPS, initial_scale_power=15, loss_scale_window=3,
                       hysteresis=1, gradient_accumulation_steps=K, gradient_clipping=clip)
    idx = np.arange(n)
    master0 = synth.host_master32(synth.stream_key(77, synth.ARR_MASTER), idx, MASTER_SIGMA)
    eager, graphed = ShardStep(n, cfg), ShardStep(n, cfg)
    for s in (eager, graphed):
        s.master.copy_(torch.from_numpy(master0))
        s.p16.zero_()
    o = oracle.State(master0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32),
                     np.zeros(n, np.uint16), oracle.Scaler(2.0 ** 15, 1.0, 3, 1))
    spec = synth.GradSpec(1e-3, 2.0 ** 15)
    bufs = [torch.zeros(n, dtype=torch.float16, device="cuda:0") for _ in range(K)]
    torch.cuda.synchronize()
    g = graphed.graph(bufs)
    torch.cuda.synchronize()
    for step in range(6):
        host = [synth.host_grad16(synth.stream_key(78, synth.ARR_GRAD, step, k), idx, spec) for k in range(K)]
        if step in (2, 3):
            host[-1][step * 1000] = 0x7C00
        for b, h in zip(bufs, host):                      # eager work between replays
            b.copy_(torch.from_numpy(h.view(np.int16)).view(torch.float16))
        g.replay()
        eager.full_step([b.clone() for b in bufs])
        ov = oracle.step(o, host if K > 1 else host[0], lr=LR, beta1=BETA1, beta2=BETA2, eps=EPS,
                         max_grad_norm=clip)
        torch.cuda.synchronize()
        se, sg = eager.scaler(), graphed.scaler()
        assert se.as_dict() == sg.as_dict(), step
        gu.check_scaler(sg, o.scaler, ov, f"graph step {step}")
        for a, b in ((eager.master, graphed.master), (eager.m, graphed.m), (eager.v, graphed.v),
                     (eager.p16, graphed.p16)):
            assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16),
                               b.view(torch.int32) if b.dtype == torch.float32 else b.view(torch.int16)), step
        gu.compare_arrays(f"graph step {step}", gu.host_f32(graphed.master), gu.host_f32(graphed.m),
                          gu.host_f32(graphed.v), gu.host_u16(graphed.p16), o.master, o.m, o.v, o.p16)
