"""The five synthetic workloads of the optimizer step (input recipes only).

Sizes, distributions, step counts and injection schedules; no optimizer
arithmetic.  All share Adam lr 1e-4, betas (0.9, 0.999), eps 1e-8, no weight
decay, master ~ N(0, 0.02), m = v = 0.

  tiny      2^20 elements, one flat range, 10 steps, grads N(0,1e-3) x 2^16,
            one +inf at a seeded index in step 4; scale 2^16, window 1000
  zero2_7b  109,375,000 elements (one rank's ZeRO-2 share of a 7B model at
            N = 64), 50 steps, no overflow; scale 2^16, window 1000
  full_7b   7e9 elements (a whole 7B model state on one device), 20 steps
  ragged    32 layers of [4096x4096] x4, [11008x4096] x3, [4096] x2 in greedy
            2e8-element buckets (6,476,267,520 elements), K = 8 micro-batches
            N(0,1e-3) x 2^15 per step, 30 steps, +inf at a seeded
            (micro-batch, index) in steps 3, 4 and 17; scale 2^15, window 10
  zero1_70b 8.75e9 elements (one rank's ZeRO-1 share of a 70B model at
            N = 8), grads N(0,5e-4) x 2^16 with 0.1% of entries x100,
            10 steps; scale 2^16, window 5

The gradient multiplier is the workload's stated loss scale, fixed for the run.
"""
from __future__ import annotations

from dataclasses import dataclass, field

from . import ARR_GRAD, ARR_INJECT, ARR_MASTER, ARR_P16, GradSpec, inject_site, stream_key

LR, BETA1, BETA2, EPS, WD = 1e-4, 0.9, 0.999, 1e-8, 0.0
MASTER_SIGMA = 0.02


@dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    psi: int
    steps: int
    K: int
    sigma: float
    mult: float
    init_scale: float
    window: int
    inject_steps: tuple = ()
    heavy_tail: bool = False
    ragged: bool = False
    hysteresis: int = 1
    min_scale: float = 1.0

    @property
    def grad_spec(self) -> GradSpec:
        return GradSpec(self.sigma, self.mult, self.heavy_tail)

    def master_key(self) -> int:
        return stream_key(self.cid, ARR_MASTER)

    def p16_key(self) -> int:
        return stream_key(self.cid, ARR_P16)

    def grad_key(self, step: int, micro: int = 0) -> int:
        """step counts from 1."""
        return stream_key(self.cid, ARR_GRAD, step, micro)

    def injection(self, step: int):
        """(micro-batch, index) of the +inf injected in ``step``, or None."""
        if step not in self.inject_steps:
            return None
        return inject_site((self.cid, ARR_INJECT, step), self.psi, micro=self.K)


WORKLOADS = {
    w.name: w for w in [
        Workload(1, "tiny", 1 << 20, 10, 1, 1e-3, 2.0 ** 16, 2.0 ** 16, 1000, inject_steps=(4,)),
        Workload(2, "zero2_7b", 109_375_000, 50, 1, 1e-3, 2.0 ** 16, 2.0 ** 16, 1000),
        Workload(3, "full_7b", 7_000_000_000, 20, 1, 1e-3, 2.0 ** 16, 2.0 ** 16, 1000),
        Workload(4, "ragged", 6_476_267_520, 30, 8, 1e-3, 2.0 ** 15, 2.0 ** 15, 10,
                 inject_steps=(3, 4, 17), ragged=True),
        Workload(5, "zero1_70b", 8_750_000_000, 10, 1, 5e-4, 2.0 ** 16, 2.0 ** 16, 5, heavy_tail=True),
    ]
}


def ragged_numels(layers=32, hidden=4096, inter=11008):
    """Per-layer q, k, v, o [hidden x hidden]; gate, up, down [inter x hidden]; 2 norms [hidden]."""
    out = []
    for _ in range(layers):
        out += [hidden * hidden] * 4 + [inter * hidden] * 3 + [hidden] * 2
    return out
