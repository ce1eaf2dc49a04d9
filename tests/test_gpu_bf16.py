"""GPU parity of the bf16 path: bf16 gradients and parameter copy, no loss
scaling (a static scale of 1; a non-finite gradient still skips the step),
against the oracle, element by element."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle
import synth
from synth.workloads import BETA1, BETA2, EPS, LR, MASTER_SIGMA
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

HP = dict(lr=LR, beta1=BETA1, beta2=BETA2, eps=EPS)
BF16_SPECIALS = {"+inf": 0x7F80, "-inf": 0xFF80, "qnan": 0x7FC0, "snan": 0x7F81, "nan_payload": 0xFFC1}


@pytest.fixture(scope="module")
def torch():
    t = gu.torch_mod()
    import zero_mixed_precision_amd  # noqa: F401
    return t


def _grads(seed, n):
    """bf16 N(0, 1e-3) draws with every finite bf16 pattern class mixed in."""
    g = synth.host_grad16(synth.stream_key(seed, synth.ARR_GRAD), np.arange(n),
                          synth.GradSpec(1e-3, 1.0, fmt="bf16"))
    rng = np.random.default_rng(seed)
    pat = rng.integers(0, 65536, n).astype(np.uint16)
    pat = np.where((pat & 0x7F80) == 0x7F80, pat & 0x807F, pat).astype(np.uint16)
    return np.where(rng.random(n) < 0.25, pat, g).astype(np.uint16)


def _pair(torch, n, seed, K=1, fmt="bf16", param_fmt="bf16", scale=1.0, dynamic=0):
    idx = np.arange(n)
    master = synth.host_master32(synth.stream_key(seed, synth.ARR_MASTER), idx, MASTER_SIGMA)
    p16 = synth.host_grad16(synth.stream_key(seed, synth.ARR_P16), idx, synth.GradSpec(0.02, 1.0, fmt="bf16"))
    z = np.zeros(n, np.float32)
    o = oracle.State(master.copy(), z.copy(), z.copy(), p16.copy(),
                     oracle.Scaler(scale, 1.0, 1000, 1, dynamic=bool(dynamic)), param_fmt=param_fmt)
    d = gu.DevState(torch, master, z, z, p16, init_scale=scale, window=1000, dynamic=dynamic, K=K, fmt=fmt,
                    param_fmt=param_fmt)
    return o, d


@pytest.mark.parametrize("n", [1, 3, 8, 17, 1023, 4097, 65536 + 7, (1 << 20) + 3])
def test_bf16_gradients_and_copy(torch, n):
    o, d = _pair(torch, n, 300 + n)
    for s in range(3):
        g = _grads(400 + 7 * n + s, n)
        if s == 1:
            g[n // 2] = 0x7F80
        ov = oracle.step(o, g, fmt="bf16", **HP)
        assert ov == (s == 1)
        d.step(gu.dev_u16(torch, g), HP)
        gu.check_scaler(d.scaler(), o.scaler, ov, f"bf16 n={n} step {s}")
        assert d.scaler().scale == 1.0
        gu.compare_full(f"bf16 n={n} step {s}", d, o)


@pytest.mark.parametrize("n", [5, 4097, (1 << 20) + 3])
@pytest.mark.parametrize("K", [2, 8])
def test_bf16_accumulation(torch, n, K):
    o, d = _pair(torch, n, 500 + n, K=K)
    for s in range(3):
        gs = [_grads(600 + 11 * n + 3 * s + k, n) for k in range(K)]
        ov = oracle.step(o, gs, fmt="bf16", **HP)
        d.step([gu.dev_u16(torch, g) for g in gs], HP)
        gu.check_scaler(d.scaler(), o.scaler, ov, f"bf16 K={K} n={n} step {s}")
        gu.compare_full(f"bf16 K={K} n={n} step {s}", d, o)


@pytest.mark.parametrize("name", sorted(BF16_SPECIALS))
def test_bf16_overflow_skips_bit_identically(torch, name):
    n = 4096 + 7
    for pos in (0, n // 2, n - 1):
        o, d = _pair(torch, n, 700 + pos)
        d.step(gu.dev_u16(torch, _grads(701, n)), HP)
        oracle.step(o, _grads(701, n), fmt="bf16", **HP)
        before = [gu.host_f32(d.master), gu.host_f32(d.m), gu.host_f32(d.v), gu.host_u16(d.p16)]
        g = _grads(702 + pos, n)
        g[pos] = BF16_SPECIALS[name]
        assert oracle.step(o, g, fmt="bf16", **HP)
        d.step(gu.dev_u16(torch, g), HP)
        gu.check_scaler(d.scaler(), o.scaler, True, f"{name} at {pos}")
        after = [gu.host_f32(d.master), gu.host_f32(d.m), gu.host_f32(d.v), gu.host_u16(d.p16)]
        for a, b in zip(before, after):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


def test_bf16_overflow_check_all_patterns(torch):
    from zero_mixed_precision_amd import _lib
    n, stride, rows = 1027, 1032, 4096
    base = _grads(77, n)
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = np.zeros(pats.size, bool)
    want = np.zeros(pats.size, bool)
    for c0 in range(0, pats.size, rows):
        chunk = pats[c0:c0 + rows]
        a = np.zeros((chunk.size, stride), np.uint16)
        a[:, :n] = base
        pos = (np.arange(chunk.size) * 89) % n
        a[np.arange(chunk.size), pos] = chunk
        da = gu.dev_u16(torch, a.reshape(-1))
        states = torch.zeros((chunk.size, _lib.ds_scaler_size()), dtype=torch.uint8, device="cuda:0")
        for j in range(chunk.size):
            _lib.ds_check_overflow(states[j].data_ptr(), da.data_ptr() + 2 * stride * j, _lib.DS_BF16, n)
        got[c0:c0 + chunk.size] = states.cpu().numpy()[:, 28:32].copy().view(np.uint32)[:, 0] != 0
        want[c0:c0 + chunk.size] = [oracle.any_nonfinite(a[j, :n], "bf16") for j in range(chunk.size)]
    assert np.array_equal(got, want)
    assert want.sum() == 2 * 128                    # exponent 0xFF: 2 signs x 128 fractions


@pytest.mark.parametrize("fmt,param_fmt", [("fp16", "bf16"), ("bf16", "fp16")])
def test_mixed_formats(torch, fmt, param_fmt):
    n = 70_001
    scale = 2.0 ** 12 if fmt == "fp16" else 1.0
    o, d = _pair(torch, n, 900, K=2, fmt=fmt, param_fmt=param_fmt, scale=scale, dynamic=int(fmt == "fp16"))
    for s in range(2):
        if fmt == "fp16":
            gs = [synth.host_grad16(synth.stream_key(901 + s, k), np.arange(n), synth.GradSpec(1e-3, scale))
                  for k in range(2)]
        else:
            gs = [_grads(903 + 2 * s + k, n) for k in range(2)]
        ov = oracle.step(o, gs, fmt=fmt, **HP)
        d.step([gu.dev_u16(torch, g) for g in gs], HP)
        gu.check_scaler(d.scaler(), o.scaler, ov, f"{fmt}/{param_fmt} step {s}")
        gu.compare_full(f"{fmt}/{param_fmt} step {s}", d, o)


def test_bf16_clipping(torch):
    from zero_mixed_precision_amd import _lib
    n = 100_003
    o, d = _pair(torch, n, 950)
    ws = torch.zeros((_lib.ds_sumsq_workspace_bytes(n) + 7) // 8, dtype=torch.float64, device="cuda:0")
    for s in range(3):
        g = synth.host_grad16(synth.stream_key(951 + s, 1), np.arange(n), synth.GradSpec(0.05, 1.0, fmt="bf16"))
        ov = oracle.step(o, g, fmt="bf16", max_grad_norm=1.0, **HP)
        gd = gu.dev_u16(torch, g)
        _lib.ds_check_overflow_sumsq(d.state, gd, _lib.DS_BF16, n, ws)
        _lib.ds_adam_step(d.state, d.master, d.m, d.v, d.p16, _lib.DS_BF16, gd, _lib.DS_BF16, n, LR, BETA1,
                          BETA2, EPS, 0.0, 1.0, 1)
        _lib.ds_update_loss_scale(d.state)
        sc = d.scaler()
        gu.check_scaler(sc, o.scaler, ov, f"bf16 clip step {s}")
        assert abs(sc.last_grad_sumsq - o.last_sumsq) <= 1e-13 * o.last_sumsq
        gu.compare_full(f"bf16 clip step {s}", d, o)


def test_bf16_cast_of_every_fp32_pattern(torch):
    """Zero gradient from m = v = 0 leaves master unchanged, so the bf16 copy is the
    kernel's cast of the input: all 2^32 fp32 patterns against the oracle's encoder."""
    from zero_mixed_precision_amd import _lib
    chunk = 1 << 28
    m = torch.zeros(chunk, dtype=torch.float32, device="cuda:0")
    v = torch.zeros(chunk, dtype=torch.float32, device="cuda:0")
    p16 = torch.empty(chunk, dtype=torch.int16, device="cuda:0")
    g = torch.zeros(chunk, dtype=torch.int16, device="cuda:0")
    st = torch.zeros(_lib.ds_scaler_size(), dtype=torch.uint8, device="cuda:0")

    def enc(pool, x, parts=8):
        out = np.empty(x.size, np.uint16)
        step = -(-x.size // parts)

        def work(k):
            out[k * step:(k + 1) * step] = oracle.encbf16(x[k * step:(k + 1) * step])
        list(pool.map(work, range(parts)))
        return out

    with ThreadPoolExecutor(8) as pool:
        for lo in range(0, 1 << 32, chunk):
            x = np.arange(lo, lo + chunk, dtype=np.uint32).view(np.float32)
            master = gu.dev_f32(torch, x)
            m.zero_()
            v.zero_()
            _lib.ds_state_init(st, 1.0, 1.0, 1000, 1, 0, 0)
            _lib.ds_adam_step(st, master, m, v, p16, _lib.DS_BF16, g, _lib.DS_BF16, chunk, LR, BETA1, BETA2,
                              EPS, 0.0, 0.0, 1)
            got = gu.host_u16(p16)
            want = enc(pool, x)
            nan = np.isnan(x)
            assert np.array_equal(got[~nan], want[~nan]), hex(lo)
            gn = got[nan]
            assert np.all(((gn & 0x7F80) == 0x7F80) & ((gn & 0x7F) != 0)), hex(lo)
            del master
