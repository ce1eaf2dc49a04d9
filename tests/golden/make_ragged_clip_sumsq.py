"""Write ragged_clip_sumsq.json: the exact sum of squares of the fp32
accumulation buffer of the ragged Llama-like layout (6,476,267,520 elements in
38 greedy 2e8-element buckets, 8 fp16 micro-batch gradients N(0,1e-3) x 2^15
per step) for steps 1 and 2, per bucket and in total, computed by the oracle
alone ("DeepSpeed complete guide" section 4.1 gradient_clipping, section 4.3
gradient accumulation).  Run from the repository root:

    python tests/golden/make_ragged_clip_sumsq.py [--workers 8]

Every piece of the flat array is regenerated on the host from the seeded
generator (a pure function of stream key and element index), accumulated in
micro-batch order with ``oracle.accumulate`` and reduced exactly with
``oracle.sumsq32_exact_units``; the pieces' exact sums add up to each
bucket's, and each bucket's and the total are rounded once to fp64.  About
1e11 generated values: some ten minutes on 8 cores.
"""
import argparse
import json
import os
import sys
import time
from multiprocessing import Pool

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import oracle  # noqa: E402
import synth  # noqa: E402
from oracle import packing  # noqa: E402
from synth.workloads import WORKLOADS, ragged_numels  # noqa: E402

STEPS = (1, 2)
PIECE = 1 << 23
OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "ragged_clip_sumsq.json")


def piece_units(task):
    step, start, stop = task
    w = WORKLOADS["ragged"]
    idx = np.arange(start, stop, dtype=np.int64)
    acc = np.empty(idx.size, np.float32)
    for k in range(w.K):
        oracle.accumulate(acc, synth.host_grad16(w.grad_key(step, k), idx, w.grad_spec), overwrite=(k == 0))
    units = oracle.sumsq32_exact_units(acc)
    if units is None:
        raise RuntimeError(f"non-finite accumulation in step {step}, elements [{start}, {stop})")
    return units


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workers", type=int, default=min(8, os.cpu_count() or 1))
    args = ap.parse_args()
    w = WORKLOADS["ragged"]
    for s in STEPS:
        if w.injection(s) is not None:
            raise RuntimeError(f"step {s} has an injected overflow")
    _, _, starts, sizes, total = packing.greedy_buckets(ragged_numels(), 200_000_000, 64)
    if total != w.psi:
        raise RuntimeError("layout total differs from the workload's size")
    tasks = []
    for s in STEPS:
        for b, (b0, bn) in enumerate(zip(starts, sizes)):
            for a in range(b0, b0 + bn, PIECE):
                tasks.append((s, b, a, min(a + PIECE, b0 + bn)))
    t0 = time.time()
    sums = {}
    with Pool(args.workers) as pool:
        for i, units in enumerate(pool.imap(piece_units, [(s, a, z) for s, _, a, z in tasks], chunksize=1)):
            s, b = tasks[i][0], tasks[i][1]
            sums[(s, b)] = sums.get((s, b), 0) + units
            if i % 100 == 0:
                print(f"{i}/{len(tasks)} pieces, {time.time() - t0:.0f} s", flush=True)
    out = {
        "what": "exact sum of squares of the fp32 accumulation of the ragged workload's 8 fp16 micro-batch "
                "gradients, per bucket and in total, each rounded once to fp64 (oracle only)",
        "pages": "DeepSpeed complete guide, section 4.1 (gradient_clipping) and section 4.3 (gradient accumulation)",
        "workload": "ragged",
        "elements": w.psi,
        "micro_batches": w.K,
        "buckets": [[int(a), int(n)] for a, n in zip(starts, sizes)],
        "steps": {},
    }
    for s in STEPS:
        per = [sums[(s, b)] for b in range(len(starts))]
        cum, running = [], 0
        for u in per:
            running += u
            cum.append(float.hex(oracle.units_to_float(running)))
        out["steps"][str(s)] = {
            "total": float.hex(oracle.units_to_float(running)),
            "total_decimal": repr(oracle.units_to_float(running)),
            "cumulative_by_bucket": cum,
        }
    with open(OUT, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(f"wrote {OUT} in {time.time() - t0:.0f} s", flush=True)


if __name__ == "__main__":
    main()
