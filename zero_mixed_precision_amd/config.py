"""The ds_config.json keys the optimizer step consumes.

"DeepSpeed complete guide" section 4.1 (base structure: gradient_accumulation_steps,
gradient_clipping, fp16, bf16, optimizer, zero_optimization), section 4.2 (fp16 block: loss_scale 0 is
dynamic, initial scale 2^initial_scale_power, loss_scale_window,
hysteresis, consecutive_hysteresis, min_loss_scale; bf16 block: no loss scaling), section 4.3
(train_batch_size = micro batch x gradient_accumulation_steps x world size), sections 4.1 and 4.4
(scheduler block: WarmupLR, WarmupDecayLR with warmup_min_lr, warmup_max_lr, warmup_num_steps,
total_num_steps, linear warmup).
"auto" values are resolved by a trainer integration, which this library does
not have: they are rejected.
"""
from __future__ import annotations

from dataclasses import dataclass


def _val(d: dict, key: str, default):
    v = d.get(key, default)
    if v == "auto":
        raise ValueError(f"'{key}': \"auto\" needs a trainer integration; give a number")
    return v


@dataclass
class ZeroMPConfig:
    # bf16 block (section 4.2: bf16 needs no loss scaling): bf16 gradients and
    # parameter copy, a static loss scale of 1 (a non-finite gradient still skips)
    bf16: bool = False
    # fp16 block
    loss_scale: float = 0.0
    initial_scale_power: int = 16
    loss_scale_window: int = 1000
    hysteresis: int = 2
    consecutive_hysteresis: bool = False
    min_loss_scale: float = 1.0
    # optimizer block
    optimizer: str = "AdamW"
    lr: float = 1e-4
    betas: tuple = (0.9, 0.999)
    eps: float = 1e-8
    weight_decay: float = 0.0
    # scheduler block: None (constant lr), "WarmupLR" or "WarmupDecayLR"
    scheduler: str | None = None
    warmup_min_lr: float = 0.0
    warmup_max_lr: float = 0.0
    warmup_num_steps: int = 0
    total_num_steps: int = 0
    # global-norm clipping of the unscaled gradient (0: off)
    gradient_clipping: float = 0.0
    # batch / ZeRO
    gradient_accumulation_steps: int = 1
    train_micro_batch_size_per_gpu: int = 1
    reduce_bucket_size: int = int(2e8)
    stage: int = 2

    @property
    def dynamic(self) -> bool:
        return self.loss_scale == 0 and not self.bf16

    @property
    def init_scale(self) -> float:
        if self.bf16:
            return 1.0
        return 2.0 ** self.initial_scale_power if self.dynamic else float(self.loss_scale)

    def lr_schedule(self):
        """The scheduler block as a ds_lr_schedule, or None for a constant lr."""
        from ._lib import DS_LR_WARMUP, DS_LR_WARMUP_DECAY, DsLrSchedule

        if self.scheduler is None:
            return None
        kind = DS_LR_WARMUP if self.scheduler == "WarmupLR" else DS_LR_WARMUP_DECAY
        return DsLrSchedule.make(kind, self.warmup_min_lr, self.warmup_max_lr, self.warmup_num_steps,
                                 self.total_num_steps)

    def train_batch_size(self, world_size: int) -> int:
        return self.train_micro_batch_size_per_gpu * self.gradient_accumulation_steps * world_size

    @classmethod
    def from_dict(cls, cfg: dict) -> "ZeroMPConfig":
        fp16 = cfg.get("fp16", {})
        bf16 = bool(_val(cfg.get("bf16", {}), "enabled", False))
        fp16_on = bool(_val(fp16, "enabled", True)) if fp16 else not bf16
        if bf16 and fp16 and fp16_on:
            raise ValueError("fp16 and bf16 are both enabled")
        if not bf16 and not fp16_on:
            raise ValueError("neither fp16 nor bf16 is enabled: this step is the mixed-precision path")
        opt = cfg.get("optimizer", {})
        params = opt.get("params", {})
        zero = cfg.get("zero_optimization", {})
        kind = _val(opt, "type", "AdamW")
        if kind not in ("Adam", "AdamW"):
            raise ValueError(f"optimizer type {kind!r} is not Adam/AdamW")
        betas = tuple(float(b) for b in _val(params, "betas", (0.9, 0.999)))
        out = cls(
            bf16=bf16,
            loss_scale=float(_val(fp16, "loss_scale", 0.0)),
            initial_scale_power=int(_val(fp16, "initial_scale_power", 16)),
            loss_scale_window=int(_val(fp16, "loss_scale_window", 1000)),
            hysteresis=int(_val(fp16, "hysteresis", 2)),
            consecutive_hysteresis=bool(_val(fp16, "consecutive_hysteresis", False)),
            min_loss_scale=float(_val(fp16, "min_loss_scale", 1.0)),
            optimizer=kind,
            lr=float(_val(params, "lr", 1e-4)),
            betas=betas,
            eps=float(_val(params, "eps", 1e-8)),
            weight_decay=float(_val(params, "weight_decay", 0.0)),
            gradient_clipping=float(_val(cfg, "gradient_clipping", 0.0)),
            gradient_accumulation_steps=int(_val(cfg, "gradient_accumulation_steps", 1)),
            train_micro_batch_size_per_gpu=int(_val(cfg, "train_micro_batch_size_per_gpu", 1)),
            reduce_bucket_size=int(float(_val(zero, "reduce_bucket_size", 2e8))),
            stage=int(_val(zero, "stage", 2)),
        )
        sched = cfg.get("scheduler")
        if sched:
            _parse_scheduler(out, sched)
        if "train_batch_size" in cfg and cfg["train_batch_size"] != "auto":
            world = cfg.get("world_size")
            if world is not None and out.train_batch_size(int(world)) != int(cfg["train_batch_size"]):
                raise ValueError("train_batch_size != micro batch x accumulation steps x world size")
        return out


_NAMED_WITHOUT_FORMULA = ("LRRangeTest", "OneCycle", "WarmupCosineLR")


def _parse_scheduler(out: ZeroMPConfig, sched: dict) -> None:
    kind = _val(sched, "type", None)
    if kind in _NAMED_WITHOUT_FORMULA:
        raise ValueError(f"scheduler {kind!r} is named by the guide without its parameters; "
                         "WarmupLR and WarmupDecayLR are supported")
    if kind not in ("WarmupLR", "WarmupDecayLR"):
        raise ValueError(f"unknown scheduler type {kind!r}")
    p = sched.get("params", {})
    for key in ("warmup_max_lr", "warmup_num_steps") + (("total_num_steps",) if kind == "WarmupDecayLR" else ()):
        if key not in p:
            raise ValueError(f"scheduler {kind}: '{key}' is required")
    if _val(p, "warmup_type", "linear") != "linear":
        raise ValueError("only the linear warmup is supported")
    if int(_val(p, "last_batch_iteration", -1)) != -1:
        raise ValueError("last_batch_iteration must be -1: a resumed run takes its position from the "
                         "restored optimizer state")
    out.scheduler = kind
    out.warmup_min_lr = float(_val(p, "warmup_min_lr", 0.0))
    out.warmup_max_lr = float(_val(p, "warmup_max_lr", None))
    out.warmup_num_steps = int(_val(p, "warmup_num_steps", None))
    out.total_num_steps = int(_val(p, "total_num_steps", 0))
    if out.warmup_num_steps < 0 or out.warmup_min_lr < 0 or out.warmup_max_lr < 0:
        raise ValueError("scheduler rates and step counts must be >= 0")
    if kind == "WarmupDecayLR" and out.total_num_steps < out.warmup_num_steps:
        raise ValueError("total_num_steps must be >= warmup_num_steps")
