"""Helpers shared by the GPU parity tests: device buffers, the ABI call
sequence of one step, and oracle-vs-device comparison at the stated bar
(flags, skips and loss scales bit-exact; fp32 master/m/v within 4 ulp;
fp16 parameters within 1 ulp)."""
from __future__ import annotations

import sys

import numpy as np

import oracle
from tests._fp import ulp_diff16, ulp_diff32

F32_ULP_TOL = 4
F16_ULP_TOL = 1


def torch_mod():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU test run without a visible GPU")
    return torch


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev_f32(torch, a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda:0")


def dev_u16(torch, a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).to("cuda:0")


def host_f32(t) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.float32, copy=False)


def host_u16(t) -> np.ndarray:
    return t.detach().cpu().view(__import__("torch").int16).numpy().view(np.uint16)


class DevState:
    """Device copy of one partition's state plus a ds_scaler."""

    def __init__(self, torch, master, m, v, p16, *, init_scale, window, hysteresis=1, min_scale=1.0,
                 dynamic=1, K=1, fmt="fp16", param_fmt="fp16", consecutive_hysteresis=0):
        from zero_mixed_precision_amd import _lib
        self.torch, self.lib = torch, _lib
        self.gdt = _lib.DS_BF16 if fmt == "bf16" else _lib.DS_FP16
        self.pdt = _lib.DS_BF16 if param_fmt == "bf16" else _lib.DS_FP16
        self.master, self.m, self.v = dev_f32(torch, master), dev_f32(torch, m), dev_f32(torch, v)
        self.p16 = dev_u16(torch, p16)
        self.n = master.size
        self.K = K
        self.acc = torch.empty(max(self.n, 1), dtype=torch.float32, device="cuda:0") if K > 1 else None
        self.state = torch.zeros(_lib.ds_scaler_size(), dtype=torch.uint8, device="cuda:0")
        _lib.ds_state_init(self.state, init_scale, min_scale, window, hysteresis, int(consecutive_hysteresis),
                           dynamic)

    def step(self, grads, hp, buckets=None, fused_check=True):
        """grads: one device fp16 tensor (K = 1) or a list of K of them."""
        L, n = self.lib, self.n
        if not isinstance(grads, (list, tuple)):
            grads = [grads]
        K = len(grads)
        assert K == self.K
        for g in grads:
            assert g.numel() >= n
        if K == 1:
            L.ds_check_overflow(self.state, grads[0], self.gdt, n)
            grad, dt = grads[0], self.gdt
        else:
            spans = buckets or [(0, n)]
            assert sum(s for _, s in spans) == n
            for k, g in enumerate(grads):
                last = k == K - 1
                for start, size in spans:
                    assert start % 8 == 0 and start + size <= n
                    L.ds_accumulate(self.acc.data_ptr() + 4 * start, g.data_ptr() + 2 * start, self.gdt, size,
                                    k == 0, self.state if (last and fused_check) else None)
            if not fused_check:
                L.ds_check_overflow(self.state, self.acc, L.DS_FP32, n)
            grad, dt = self.acc, L.DS_FP32
        L.ds_adam_step(self.state, self.master, self.m, self.v, self.p16, self.pdt, grad, dt, n, hp["lr"],
                       hp["beta1"], hp["beta2"], hp["eps"], hp.get("weight_decay", 0.0), 0.0, K)
        L.ds_update_loss_scale(self.state)

    def scaler(self):
        return self.lib.ds_state_read(self.state)


def count_nonfinite16(torch, t, fmt="fp16", chunk=1 << 28) -> int:
    """Non-finite values in a device buffer of 16-bit gradient bits, counted by
    torch's isfinite (a library routine, independent of the kernels and of the
    oracle) over chunks, so that no full-size temporary is made."""
    view = t.view(torch.bfloat16 if fmt == "bf16" else torch.float16)
    bad = 0
    for s in range(0, view.numel(), chunk):
        bad += int((~torch.isfinite(view[s:s + chunk])).sum().item())
    return bad


def check_scaler(dev_sc, orc: "oracle.Scaler", overflow: bool, ctx=""):
    s = orc.s
    assert bool(dev_sc.last_overflow) == bool(overflow), f"{ctx}: overflow flag"
    assert dev_sc.scale == s.scale, f"{ctx}: scale {dev_sc.scale} vs {s.scale}"
    assert dev_sc.step == s.applied and dev_sc.skipped == s.skipped and dev_sc.iter == s.iters, ctx
    assert dev_sc.growth_count == s.good_steps and dev_sc.hysteresis_left == s.hyst_left, ctx
    assert dev_sc.overflow == 0, ctx


def compare_arrays(ctx, master, m, v, p16, o_master, o_m, o_v, o_p16):
    """Element-by-element comparison; returns the max ulp distances seen."""
    du = {
        "master": int(ulp_diff32(master, o_master).max(initial=0)),
        "m": int(ulp_diff32(m, o_m).max(initial=0)),
        "v": int(ulp_diff32(v, o_v).max(initial=0)),
        "p16": int(ulp_diff16(p16, o_p16).max(initial=0)),
    }
    for k in ("master", "m", "v"):
        assert du[k] <= F32_ULP_TOL, f"{ctx}: {k} differs by {du[k]} ulp"
    assert du["p16"] <= F16_ULP_TOL, f"{ctx}: p16 differs by {du['p16']} ulp"
    return du


def compare_full(ctx, d: DevState, o: "oracle.State"):
    return compare_arrays(ctx, host_f32(d.master), host_f32(d.m), host_f32(d.v), host_u16(d.p16),
                          o.master, o.m, o.v, o.p16)
