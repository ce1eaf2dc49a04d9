"""Checkpoint and resume of one rank's optimizer shard.

"DeepSpeed complete guide" section 5.2: the engine saves its (distributed)
state under a directory and a tag, and loading returns the caller's client
state.  Here one rank's shard is one safetensors file per tag

    <save_dir>/<tag>/zero_shard_rank<rank>.safetensors

holding the flat fp32 master, Adam m and v, the 16-bit parameter copy and the
128-byte device scaler state (loss scale, counters, applied-step count t,
which also positions a learning-rate schedule), with the caller's client
state and the element count and formats as JSON metadata.  ``<save_dir>/latest``
names the last tag written.  safetensors holds raw arrays only: loading runs
nothing from the file.  The fp32 accumulation buffer is not saved: a
checkpoint is taken between steps, when it holds nothing.
"""
from __future__ import annotations

import ctypes
import json
import os

FORMAT = "zero-mp-shard-1"


def torch_stream(stream, torch):
    """The torch stream for a ShardStep's stream: None is torch's current
    stream, a raw hipStream_t handle (an int) is wrapped, a torch stream is
    used as it is."""
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, int):
        return torch.cuda.ExternalStream(stream)
    return stream


def validate_scaler(sc, where: str = "scaler state") -> None:
    """Refuse a restored loss-scaler state that the library would not have
    produced between steps ("DeepSpeed complete guide" section 4.2: a dynamic
    or static scale, loss_scale_window, hysteresis, min_loss_scale):
    ds_state_write copies it as it is, so a corrupt or foreign file could
    otherwise leave an unusable scale or disable growth.  Raises ValueError."""
    import math

    def bad(what):
        raise ValueError(f"{where}: invalid loss-scaler state ({what})")

    if not (math.isfinite(sc.scale) and sc.scale > 0):
        bad(f"scale {sc.scale}")
    if not (math.isfinite(sc.min_scale) and sc.min_scale > 0):
        bad(f"min_scale {sc.min_scale}")
    if sc.growth_window < 1:
        bad(f"growth_window {sc.growth_window}")
    if sc.hysteresis < 1:
        bad(f"hysteresis {sc.hysteresis}")
    if not 0 <= sc.growth_count < sc.growth_window:
        bad(f"growth_count {sc.growth_count} of window {sc.growth_window}")
    if not 1 <= sc.hysteresis_left <= sc.hysteresis:
        bad(f"hysteresis_left {sc.hysteresis_left} of {sc.hysteresis}")
    if sc.dynamic not in (0, 1) or sc.consecutive_hysteresis not in (0, 1):
        bad("dynamic / consecutive_hysteresis not 0 or 1")
    if min(sc.step, sc.iter, sc.skipped) < 0 or sc.step + sc.skipped != sc.iter:
        bad(f"step counts (applied {sc.step} + skipped {sc.skipped} != all {sc.iter})")
    if sc.overflow != 0 or sc.grad_sumsq != 0.0:
        bad("taken inside a step (overflow flag or gradient sum of squares pending)")


def _file(save_dir: str, tag: str, rank: int) -> str:
    return os.path.join(save_dir, str(tag), f"zero_shard_rank{int(rank):05d}.safetensors")


def save_checkpoint(step, save_dir: str, tag=None, client_state=None, rank: int = 0) -> str:
    """Write ``step``'s shard (a ShardStep) under ``save_dir``/``tag``; the default
    tag is ``step_<n>`` with n the steps taken so far (applied and skipped)."""
    import torch
    from safetensors.torch import save_file

    from . import _lib

    if step._micro != 0:
        raise RuntimeError("save_checkpoint between steps only (micro-batches are pending)")
    sc = step.scaler()                          # synchronises the step's stream
    if tag is None:
        tag = f"step_{sc.iter}"
    path = _file(save_dir, tag, rank)
    os.makedirs(os.path.dirname(path), exist_ok=True)
    raw = ctypes.string_at(ctypes.addressof(sc), ctypes.sizeof(sc))
    master, m, v, p16 = step.current()           # with double buffering: the copy holding the state
    tensors = {
        "master": master.detach().cpu(),
        "exp_avg": m.detach().cpu(),
        "exp_avg_sq": v.detach().cpu(),
        "param16": p16.detach().view(torch.int16).cpu(),
        "scaler": torch.frombuffer(bytearray(raw), dtype=torch.uint8).clone(),
    }
    meta = {
        "format": FORMAT,
        "numel": str(step.n),
        "half": "bf16" if step.pdt == _lib.DS_BF16 else "fp16",
        "scaler_bytes": str(len(raw)),
        "client_state": json.dumps(client_state if client_state is not None else {}),
    }
    save_file(tensors, path, metadata=meta)
    with open(os.path.join(save_dir, "latest"), "w") as f:
        f.write(str(tag))
    return path


def load_checkpoint(step, load_dir: str, tag=None, rank: int = 0):
    """Restore ``step``'s shard from ``load_dir``/``tag`` (default: the tag named by
    ``latest``); returns (path, client_state)."""
    import torch
    from safetensors import safe_open

    from . import _lib

    if tag is None:
        with open(os.path.join(load_dir, "latest")) as f:
            tag = f.read().strip()
    path = _file(load_dir, tag, rank)
    with safe_open(path, framework="pt", device="cpu") as f:
        meta = f.metadata() or {}
        if meta.get("format") != FORMAT:
            raise ValueError(f"{path}: not a shard checkpoint of this library")
        if int(meta["numel"]) != step.n:
            raise ValueError(f"{path}: {meta['numel']} elements, this shard has {step.n}")
        half = "bf16" if step.pdt == _lib.DS_BF16 else "fp16"
        if meta["half"] != half:
            raise ValueError(f"{path}: {meta['half']} parameter copy, this shard uses {half}")
        raw = f.get_tensor("scaler").numpy().tobytes()
        if len(raw) != _lib.ds_scaler_size():
            raise ValueError(f"{path}: scaler state of {len(raw)} bytes")
        arrays = {k: f.get_tensor(k) for k in ("master", "exp_avg", "exp_avg_sq", "param16")}
    sc = _lib.DsScaler.from_buffer_copy(raw)
    validate_scaler(sc, path)
    sc.current = 0                              # the arrays are restored into copy 0 (the attributes)
    with torch.cuda.stream(torch_stream(step.stream, torch)):
        step.master.copy_(arrays["master"])
        step.m.copy_(arrays["exp_avg"])
        step.v.copy_(arrays["exp_avg_sq"])
        step.p16.view(torch.int16).copy_(arrays["param16"])
    _lib.ds_state_write(step.state, sc, step.stream)
    step._micro = 0
    return path, json.loads(meta["client_state"])
