"""GPU parity of the double-buffered step (ds_adam_step_double_buffered): the
overflow check fused into the Adam pass, which reads the current copy of the
state and writes the update into the other one; the last block makes the
other copy current only if the step applied ("DeepSpeed complete guide"
section 2: fp32 master and moments, fp16 copy; section 4.2: dynamic loss
scaling, a gradient overflow skips the step).

Against the oracle's check -> Adam or skip -> scaler update: the current copy
bit for bit after every step, the copy index, the scaler state; a skipped step
leaves the current copy (and its index) untouched; launch-shape invariance;
every gradient and parameter format; schedules and weight decay; and the
same steps through ds_check_overflow + ds_adam_step_fused give identical bits.
"""
import numpy as np
import pytest

import oracle
import synth
from synth.workloads import BETA1, BETA2, EPS, LR, MASTER_SIGMA
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

HP = dict(lr=LR, beta1=BETA1, beta2=BETA2, eps=EPS)


@pytest.fixture(scope="module")
def torch():
    return gu.torch_mod()


class DbState:
    """Two device copies of one partition's state plus a ds_scaler."""

    def __init__(self, torch, master, p16, *, init_scale, window, hysteresis=1, dynamic=1, fmt="fp16",
                 param_fmt="fp16"):
        from zero_mixed_precision_amd import _lib
        self.torch, self.L, self.n = torch, _lib, master.size
        self.gdt = _lib.DS_BF16 if fmt == "bf16" else _lib.DS_FP16
        self.pdt = _lib.DS_BF16 if param_fmt == "bf16" else _lib.DS_FP16
        n1 = max(self.n, 1)
        self.master = [gu.dev_f32(torch, master), torch.full((n1,), 7.0, device="cuda:0")]
        self.m = [torch.zeros(n1, device="cuda:0"), torch.full((n1,), 7.0, device="cuda:0")]
        self.v = [torch.zeros(n1, device="cuda:0"), torch.full((n1,), 7.0, device="cuda:0")]
        self.p16 = [gu.dev_u16(torch, p16) if self.n else torch.zeros(1, dtype=torch.int16, device="cuda:0"),
                    torch.full((n1,), 0x1234, dtype=torch.int16, device="cuda:0")]
        self.state = torch.zeros(_lib.ds_scaler_size(), dtype=torch.uint8, device="cuda:0")
        _lib.ds_state_init(self.state, init_scale, 1.0, window, hysteresis, 0, dynamic)

    def step(self, grad, dt=None, K=1, lr=LR, sched=None, wd=0.0):
        L = self.L
        L.ds_adam_step_double_buffered(self.state, self.master, self.m, self.v, self.p16, self.pdt, grad,
                                       self.gdt if dt is None else dt, self.n, lr, sched, BETA1, BETA2, EPS, wd, K)

    def scaler(self):
        return self.L.ds_state_read(self.state)

    def current(self):
        c = self.scaler().current
        assert c in (0, 1)
        return (gu.host_f32(self.master[c][:self.n]), gu.host_f32(self.m[c][:self.n]),
                gu.host_f32(self.v[c][:self.n]), gu.host_u16(self.p16[c][:self.n])), c


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint32 if a.dtype == np.float32 else np.uint16)


def _run(torch, n, steps, *, fmt="fp16", param_fmt="fp16", inject=(), scale=2.0 ** 16, window=1000, wd=0.0,
         sched=None, seed=0):
    spec = synth.GradSpec(1e-3, scale, fmt=fmt)
    idx = np.arange(n)
    master0 = synth.host_master32(synth.stream_key(500 + seed, synth.ARR_MASTER), idx, MASTER_SIGMA)
    p160 = synth.host_grad16(synth.stream_key(500 + seed, synth.ARR_P16), idx, synth.GradSpec(0.02, 1.0, fmt=fmt))
    o = oracle.State(master0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32), p160.copy(),
                     oracle.Scaler(scale, 1.0, window, 1), param_fmt=param_fmt)
    d = DbState(torch, master0, p160, init_scale=scale, window=window, fmt=fmt, param_fmt=param_fmt)
    lr = sched if sched is not None else LR
    dsched = None
    if sched is not None:
        from zero_mixed_precision_amd import _lib
        dsched = _lib.DsLrSchedule.make(sched.kind, sched.min_lr, sched.max_lr, sched.warmup, sched.total)
    for s in range(steps):
        g = synth.host_grad16(synth.stream_key(600 + seed, synth.ARR_GRAD, s), idx, spec)
        if s in inject and n:
            g[(s * 7919) % n] = 0x7F80 if fmt == "bf16" else (0x7C00 if s % 2 else 0xFE01)
        before, c0 = d.current()
        d.step(gu.dev_u16(torch, g) if n else torch.zeros(8, dtype=torch.int16, device="cuda:0"),
               lr=LR, sched=dsched, wd=wd)
        ov = oracle.step(o, g, fmt=fmt, weight_decay=wd, **dict(HP, lr=lr))
        (master, m, v, p16), c1 = d.current()
        sc = d.scaler()
        gu.check_scaler(sc, o.scaler, ov, f"n={n} step {s}")
        assert sc.db_tickets == 0, f"n={n} step {s}: tickets not reset"
        if ov:
            assert c1 == c0, "a skipped step changed the current copy"
            for x, y in zip(before, (master, m, v, p16)):
                assert np.array_equal(_bits(x), _bits(y)), "a skipped step changed the current state"
        else:
            assert c1 == 1 - c0
        for x, y in zip((master, m, v, p16), (o.master, o.m, o.v, o.p16)):
            assert np.array_equal(_bits(x), _bits(y)), f"n={n} step {s}: state differs from the oracle"
    return d, o


@pytest.mark.parametrize("n", [0, 1, 3, 4, 5, 255, 1021, 4095, 4096, 4097, 8191, 70_003])
def test_ragged_sizes_against_the_oracle(torch, n):
    _run(torch, n, 4, inject=(2,))


def test_tiny_workload_with_an_overflow(torch):
    """The tiny workload's schedule (2^20 elements, 10 steps, +inf in step 4)."""
    d, o = _run(torch, 1 << 20, 10, inject=(3,))
    assert o.scaler.applied == 9 and d.scaler().scale == 2.0 ** 15


@pytest.mark.parametrize("fmt,param_fmt", [("bf16", "bf16"), ("fp16", "bf16"), ("bf16", "fp16")])
def test_formats(torch, fmt, param_fmt):
    _run(torch, 10_007, 5, fmt=fmt, param_fmt=param_fmt, scale=1.0 if fmt == "bf16" else 2.0 ** 16, inject=(1, 3))


def test_weight_decay_schedule_and_growth(torch):
    sched = oracle.LrSchedule(oracle.LR_WARMUP_DECAY, 1e-5, 3e-4, 3, 9)
    d, o = _run(torch, 33_333, 12, wd=0.01, sched=sched, window=3, inject=(5,))
    # growth after steps 2, 8 and 11 (three successes each), a halving at step 5
    assert o.scaler.scale == 2.0 ** 18


def test_accumulated_fp32_gradient(torch):
    """With K = 3 micro-batches summed into the fp32 buffer, the step reads the
    buffer (30 B per element) and checks it in the same pass."""
    from zero_mixed_precision_amd import _lib
    n, K, scale = 50_001, 3, 2.0 ** 12
    idx = np.arange(n)
    master0 = synth.host_master32(synth.stream_key(701, synth.ARR_MASTER), idx, MASTER_SIGMA)
    o = oracle.State(master0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16),
                     oracle.Scaler(scale, 1.0, 1000, 1))
    d = DbState(torch, master0, np.zeros(n, np.uint16), init_scale=scale, window=1000)
    acc = torch.empty(n, device="cuda:0")
    for s in range(4):
        gs = [synth.host_grad16(synth.stream_key(702, synth.ARR_GRAD, s, k), idx, synth.GradSpec(1e-3, scale))
              for k in range(K)]
        if s == 2:
            gs[1][n - 1] = 0x7C00
        for k, g in enumerate(gs):
            _lib.ds_accumulate(acc, gu.dev_u16(torch, g), _lib.DS_FP16, n, k == 0, None)
        d.step(acc, dt=_lib.DS_FP32, K=K)
        ov = oracle.step(o, gs, **HP)
        gu.check_scaler(d.scaler(), o.scaler, ov, f"K=3 step {s}")
        (master, m, v, p16), _ = d.current()
        for x, y in zip((master, m, v, p16), (o.master, o.m, o.v, o.p16)):
            assert np.array_equal(_bits(x), _bits(y)), f"K=3 step {s}"


def test_flag_raised_before_the_call_skips_the_step(torch):
    """A non-finite value found earlier in the step (here by ds_check_overflow
    on another gradient buffer of the partition) skips the step even though
    the gradient the pass reads is finite; the next, clean step applies."""
    from zero_mixed_precision_amd import _lib
    n = 40_000
    idx = np.arange(n)
    master0 = synth.host_master32(synth.stream_key(711, synth.ARR_MASTER), idx, MASTER_SIGMA)
    o = oracle.State(master0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16),
                     oracle.Scaler(2.0 ** 16, 1.0, 1000, 1))
    d = DbState(torch, master0, np.zeros(n, np.uint16), init_scale=2.0 ** 16, window=1000)
    other = np.zeros(999, np.uint16)
    other[998] = 0xFC00    # -inf
    for s in range(3):
        g = synth.host_grad16(synth.stream_key(712, synth.ARR_GRAD, s), idx, synth.GradSpec(1e-3, 2.0 ** 16))
        _, c0 = d.current()
        if s == 1:
            _lib.ds_check_overflow(d.state, gu.dev_u16(torch, other), _lib.DS_FP16, other.size)
        d.step(gu.dev_u16(torch, g))
        # the partition's gradient holds a non-finite value in step 1 (in the
        # other buffer): for the oracle, the same step with it in this one
        gi = g.copy()
        if s == 1:
            gi[0] = other[998]
        ov = oracle.step(o, gi, **HP)
        assert ov == (s == 1)
        gu.check_scaler(d.scaler(), o.scaler, ov, f"step {s}")
        after, c1 = d.current()
        assert c1 == (c0 if ov else 1 - c0)
        for x, y in zip(after, (o.master, o.m, o.v, o.p16)):
            assert np.array_equal(_bits(x), _bits(y)), f"step {s}"


def test_launch_shape_invariance(torch, monkeypatch):
    n = 3 * 4096 + 1029
    ref = None
    for env in [{}, {"DSZERO_GRID": "1"}, {"DSZERO_GRID": "5"}, {"DSZERO_GRID": "100000"}, {"DSZERO_NT": "1"},
                {"DSZERO_NT": "1", "DSZERO_GRID": "2"}]:
        for k in ("DSZERO_GRID", "DSZERO_NT"):
            monkeypatch.delenv(k, raising=False)
        for k, val in env.items():
            monkeypatch.setenv(k, val)
        d, _ = _run(torch, n, 3, inject=(1,))
        got = d.current()[0]
        if ref is None:
            ref = got
        for x, y in zip(got, ref):
            assert np.array_equal(_bits(x), _bits(y)), env


def test_same_bits_as_check_then_fused_adam(torch):
    """The same steps through ds_check_overflow + ds_adam_step_fused (in place)
    end in the same bits and the same scaler state."""
    from zero_mixed_precision_amd import _lib
    n = 200_003
    idx = np.arange(n)
    master0 = synth.host_master32(synth.stream_key(801, synth.ARR_MASTER), idx, MASTER_SIGMA)
    d = DbState(torch, master0, np.zeros(n, np.uint16), init_scale=2.0 ** 16, window=3)
    master, m, v = gu.dev_f32(torch, master0), torch.zeros(n, device="cuda:0"), torch.zeros(n, device="cuda:0")
    p16 = torch.zeros(n, dtype=torch.int16, device="cuda:0")
    st = torch.zeros(_lib.ds_scaler_size(), dtype=torch.uint8, device="cuda:0")
    _lib.ds_state_init(st, 2.0 ** 16, 1.0, 3, 1, 0, 1)
    for s in range(9):
        g = synth.host_grad16(synth.stream_key(802, synth.ARR_GRAD, s), idx, synth.GradSpec(1e-3, 2.0 ** 16))
        if s in (2, 6):
            g[(s * 104729) % n] = 0x7C00
        gd = gu.dev_u16(torch, g)
        d.step(gd)
        _lib.ds_check_overflow(st, gd, _lib.DS_FP16, n)
        _lib.ds_adam_step_fused(st, master, m, v, p16, _lib.DS_FP16, gd, _lib.DS_FP16, n, LR, None, BETA1, BETA2,
                                EPS, 0.0, 0.0, 1)
    (cm, cmm, cv, cp), _ = d.current()
    for x, y in zip((cm, cmm, cv, cp), (gu.host_f32(master), gu.host_f32(m), gu.host_f32(v), gu.host_u16(p16))):
        assert np.array_equal(_bits(x), _bits(y))
    a, b = d.scaler(), _lib.ds_state_read(st)
    for f in ("scale", "step", "iter", "skipped", "growth_count", "hysteresis_left", "last_overflow"):
        assert getattr(a, f) == getattr(b, f), f


def test_shard_step_double_buffered_graph_and_checkpoint(torch, tmp_path):
    """ShardStep(double_buffer=True) against the in-place ShardStep: the same bits
    after steps with an overflow, when the steps are replayed from a captured
    graph (eager work and synchronisation between replays), and across a
    checkpoint taken while copy 1 holds the state (after an overflowed step)."""
    from zero_mixed_precision_amd import ShardStep, ZeroMPConfig
    n = 123_457
    cfg = ZeroMPConfig.from_dict({"fp16": {"enabled": True, "initial_scale_power": 14, "loss_scale_window": 2},
                                  "optimizer": {"type": "AdamW", "params": {"lr": 2e-4, "weight_decay": 0.01}}})
    master0 = torch.from_numpy(synth.host_master32(synth.stream_key(901, synth.ARR_MASTER), np.arange(n),
                                                   MASTER_SIGMA)).to("cuda:0")
    host = [synth.host_grad16(synth.stream_key(902, synth.ARR_GRAD, s), np.arange(n), synth.GradSpec(1e-3, 2.0 ** 14))
            for s in range(8)]
    host[3][77] = 0x7C00
    ref, db, gr = ShardStep(n, cfg), ShardStep(n, cfg, double_buffer=True), ShardStep(n, cfg, double_buffer=True)
    for s in (ref, db, gr):
        s.master.copy_(master0)
        s.p16.zero_()
    buf = torch.empty(n, dtype=torch.int16, device="cuda:0")
    graph = gr.graph(buf)
    for s in range(8):
        g = gu.dev_u16(torch, host[s])
        ref.step(g)
        db.step(g)
        buf.copy_(g)
        graph.replay()
        torch.cuda.synchronize()
        want = [gu.host_f32(x) if x.dtype == torch.float32 else gu.host_u16(x) for x in ref.current()]
        for shard in (db, gr):
            got = [gu.host_f32(x) if x.dtype == torch.float32 else gu.host_u16(x) for x in shard.current()]
            for x, y in zip(got, want):
                assert np.array_equal(_bits(x), _bits(y)), f"step {s}"
            assert shard.scaler().scale == ref.scaler().scale
        if s == 3:
            assert db.scaler().current == 1      # 3 applied steps of 4 (step 3 overflowed): copy 1 holds the state
            db.save_checkpoint(str(tmp_path), tag="mid")
            resumed = ShardStep(n, cfg, double_buffer=True)
            resumed.load_checkpoint(str(tmp_path), tag="mid")
            assert resumed.scaler().current == 0
    for s in range(4, 8):
        resumed.step(gu.dev_u16(torch, host[s]))
    for x, y in zip(resumed.current(), db.current()):
        assert torch.equal(x.view(torch.int16) if x.dtype != torch.float32 else x.view(torch.int32),
                           y.view(torch.int16) if y.dtype != torch.float32 else y.view(torch.int32))
    with pytest.raises(ValueError, match="double_buffer"):
        ShardStep(n, ZeroMPConfig(gradient_clipping=1.0), double_buffer=True)
