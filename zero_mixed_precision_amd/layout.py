"""Flat-partition layout: ragged tensors packed into contiguous buffers.

"DeepSpeed complete guide" section 2 (the model state is five per-parameter
arrays), sections 2.2 and 4.1 (contiguous_gradients; reduce_bucket_size and
allgather_bucket_size of 2e8 elements), sections 2.1-2.2 (each of N ranks owns
a contiguous 1/N share).  The packing itself runs in the native library
(``ds_layout_greedy``, ``ds_partition_range``); this class only holds the
result and hands out views.
"""
from __future__ import annotations

from dataclasses import dataclass

from . import _lib

DEFAULT_BUCKET = int(2e8)
DEFAULT_ALIGN = 64


@dataclass(frozen=True)
class Bucket:
    start: int
    size: int


class FlatLayout:
    def __init__(self, numels, bucket_cap: int = DEFAULT_BUCKET, align: int = DEFAULT_ALIGN):
        self.numels = [int(x) for x in numels]
        self.bucket_cap, self.align = int(bucket_cap), int(align)
        offs, bof, starts, sizes, total = _lib.ds_layout_greedy(self.numels, self.bucket_cap, self.align)
        self.offsets, self.bucket_of, self.total = offs, bof, total
        self.buckets = [Bucket(s, z) for s, z in zip(starts, sizes)]

    def view(self, flat, i: int):
        """Tensor i as a view of a flat array (any dtype)."""
        o = self.offsets[i]
        return flat[o:o + self.numels[i]]

    def partition(self, world: int, rank: int, align: int = 8):
        """(start, count) of rank's contiguous share of the flat array."""
        return _lib.ds_partition_range(self.total, world, rank, align)

    def buckets_in(self, start: int, count: int):
        """Buckets clipped to the element range [start, start + count)."""
        out = []
        for b in self.buckets:
            lo, hi = max(b.start, start), min(b.start + b.size, start + count)
            if hi > lo:
                out.append(Bucket(lo - start, hi - lo))
        return out
