"""Pins of the packing oracle (flat layout, greedy 2e8-element buckets, ZeRO
ranges) against the numbers the pages print and against the packing rule's
defining properties."""
import json
import os

import numpy as np
import pytest

from oracle import packing

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_memory_table_from_pages():
    g = json.load(open(os.path.join(GOLDEN, "memory_table.json")))
    assert packing.STATE_BYTES == g["bytes_per_param"]
    assert packing.model_state_bytes(1) == g["total_bytes_per_param"] == 16
    for ex in g["examples"]:
        got = packing.model_state_bytes(int(ex["params"]))
        # the page rounds: "about 112 GB", "about 1.1 TB"
        assert abs(got - ex["approx_bytes"]) / ex["approx_bytes"] < 0.025


def test_zero_stage_memory_from_pages():
    g = json.load(open(os.path.join(GOLDEN, "zero_stage_memory.json")))
    assert packing.zero_bytes_per_param(0, 64) == g["baseline_bytes_per_param"]
    for st in g["stages"]:
        got = packing.zero_bytes_per_param(st["stage"], st["N"])
        assert round(got, 1 if st["stage"] < 3 else 2) == st["approx_bytes_per_param"]
    # exact values behind the page's rounding
    assert packing.zero_bytes_per_param(1, 64) == 4.1875
    assert packing.zero_bytes_per_param(2, 64) == 2.21875


def test_shard_sizes_of_the_workloads():
    # one rank's share of a 7B model at N=64 and of a 70B model at N=8
    assert packing.partition_range(7_000_000_000, 64, 0, 8) == (0, 109_375_000)
    assert packing.partition_range(7_000_000_000, 64, 63, 8) == (63 * 109_375_000, 109_375_000)
    assert packing.partition_range(70_000_000_000, 8, 7, 8) == (7 * 8_750_000_000, 8_750_000_000)


def test_partition_ranges_tile_the_array():
    rng = np.random.default_rng(0)
    for _ in range(300):
        total = int(rng.integers(0, 10 ** 6))
        world = int(rng.integers(1, 70))
        align = int(rng.choice([1, 8, 64]))
        pos = 0
        for r in range(world):
            start, count = packing.partition_range(total, world, r, align)
            assert start == pos and count >= 0
            assert start % align == 0 or (start == total and count == 0)
            pos += count
        assert pos == total


def _check_layout(numels, cap, align):
    offs, bof, starts, sizes, total = packing.greedy_buckets(numels, cap, align)
    assert len(offs) == len(numels)
    # buckets tile [0, total) contiguously, each starting aligned
    assert starts[0] == 0 if starts else total == 0
    for b in range(len(starts)):
        assert starts[b] % align == 0 and sizes[b] % align == 0
        if b + 1 < len(starts):
            assert starts[b] + sizes[b] == starts[b + 1]
    if starts:
        assert starts[-1] + sizes[-1] == total
    prev_end = 0
    for i, (o, n, b) in enumerate(zip(offs, numels, bof)):
        assert o % align == 0 and o >= prev_end          # in order, aligned, no overlap
        assert o - prev_end < align or (i > 0 and bof[i - 1] != b)
        assert starts[b] <= o and o + n <= starts[b] + sizes[b]   # inside one bucket
        prev_end = o + n
    for b in range(len(starts)):
        members = [i for i in range(len(numels)) if bof[i] == b]
        assert members == list(range(members[0], members[-1] + 1))
        if len(members) > 1:
            assert sizes[b] <= cap                          # only a lone big tensor may exceed
        if b + 1 < len(starts):                             # greedy: next tensor did not fit
            nxt = members[-1] + 1
            end_with_next = packing.round_up(packing.round_up(starts[b] + sizes[b], 1) + numels[nxt], align)
            assert end_with_next - starts[b] > cap
    return offs, bof, starts, sizes, total


def test_ragged_llama_like_layout():
    numels = packing.llama_like_numels()
    assert len(numels) == 288
    assert sum(numels[:9]) == 202_383_360
    offs, bof, starts, sizes, total = _check_layout(numels, int(2e8), 64)
    assert total == 6_476_267_520 == sum(numels)
    assert len(starts) == 38
    hist = {}
    for s in sizes:
        hist[s] = hist.get(s, 0) + 1
    assert hist == {185_606_144: 20, 157_294_592: 11, 157_286_400: 6, 90_185_728: 1}
    assert sizes[0] == 157_286_400          # layer 0: q, k, v, o, gate, up


def test_random_layouts_satisfy_the_rule():
    rng = np.random.default_rng(1)
    for _ in range(200):
        k = int(rng.integers(1, 40))
        numels = [int(x) for x in rng.integers(0, 5000, k)]
        if rng.random() < 0.3:
            numels[int(rng.integers(0, k))] = int(rng.integers(5000, 20000))
        _check_layout(numels, int(rng.integers(1000, 9000)), int(rng.choice([1, 4, 64])))


def test_empty_layout():
    assert packing.greedy_buckets([], 100, 64) == ([], [], [], [], 0)
