"""Packing oracle: flat contiguous layout, buckets and ZeRO partition ranges.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Pages: "DeepSpeed complete guide" section 2 (memory table: the model state is
five per-parameter arrays) and sections 2.2 / 4.1 (``contiguous_gradients``;
``reduce_bucket_size`` and ``allgather_bucket_size`` of 2e8, counted in
elements); section 2.1 (each of N ranks owns a 1/N shard of the optimizer
state and updates only that shard).

Readings (the pages give the keys, not the packing rule):
  * tensors are laid out in the order given, each starting at an offset that
    is a multiple of ``align`` elements (zero padding in between);
  * buckets are built greedily from whole tensors: a tensor joins the open
    bucket if the bucket, padded to ``align``, still holds at most ``cap``
    elements with it; otherwise the bucket closes and the tensor opens the
    next one (a tensor larger than ``cap`` gets a bucket of its own);
  * the flat array is the concatenation of the buckets; a ZeRO partition of
    rank r of N is the r-th of N equal contiguous ranges of the flat array,
    whose length is rounded up to ``align`` (the last range may be shorter).
"""
from __future__ import annotations


def round_up(x: int, a: int) -> int:
    return ((x + a - 1) // a) * a


def greedy_buckets(numels, cap: int, align: int):
    """Return (offsets, bucket_of, bucket_starts, bucket_sizes, total)."""
    offsets, bucket_of, starts, sizes = [], [], [], []
    open_start = 0     # first element of the open bucket
    open_end = 0       # end of the open bucket's last tensor (unpadded)
    open_count = 0     # tensors in the open bucket
    for n in numels:
        n = int(n)
        if n < 0:
            raise ValueError("negative tensor size")
        candidate_off = round_up(open_end, align)
        candidate_end = round_up(candidate_off + n, align)
        if open_count > 0 and candidate_end - open_start > cap:
            close = round_up(open_end, align)
            starts.append(open_start)
            sizes.append(close - open_start)
            open_start = close
            open_end = close
            open_count = 0
            candidate_off = open_start
        offsets.append(candidate_off)
        bucket_of.append(len(starts))
        open_end = candidate_off + n
        open_count += 1
    if open_count > 0:
        close = round_up(open_end, align)
        starts.append(open_start)
        sizes.append(close - open_start)
        open_end = close
    total = round_up(open_end, align)
    return offsets, bucket_of, starts, sizes, total


def partition_range(total: int, world: int, rank: int, align: int):
    """(start, count) of rank's contiguous share of a flat array of ``total``."""
    if world < 1 or not (0 <= rank < world):
        raise ValueError("bad world/rank")
    per = round_up(-(-total // world), align)
    start = min(rank * per, total)
    count = min(per, total - start)
    return start, count


def llama_like_numels(layers=32, hidden=4096, inter=11008):
    """Tensor sizes of the ragged Llama-like layout, in packing order: per layer
    q, k, v, o [hidden x hidden], gate, up, down [inter x hidden], two norms [hidden]."""
    out = []
    for _ in range(layers):
        out += [hidden * hidden] * 4 + [inter * hidden] * 3 + [hidden] * 2
    return out


# Model-state accounting ("DeepSpeed complete guide" section 2 memory table and
# sections 2.1-2.3): bytes per parameter of fp16 params (2), fp16 grads (2),
# fp32 master (4), Adam first moment (4), Adam second moment (4).
STATE_BYTES = {"fp16_param": 2, "fp16_grad": 2, "fp32_master": 4, "adam_m": 4, "adam_v": 4}


def model_state_bytes(psi: int) -> int:
    return sum(STATE_BYTES.values()) * psi


def zero_bytes_per_param(stage: int, world: int) -> float:
    """Per-GPU model-state bytes per parameter under ZeRO stage 0..3 with N ranks."""
    p, g = STATE_BYTES["fp16_param"], STATE_BYTES["fp16_grad"]
    opt = STATE_BYTES["fp32_master"] + STATE_BYTES["adam_m"] + STATE_BYTES["adam_v"]
    if stage == 0:
        return p + g + opt
    if stage == 1:
        return p + g + opt / world
    if stage == 2:
        return p + (g + opt) / world
    if stage == 3:
        return (p + g + opt) / world
    raise ValueError("stage must be 0..3")
