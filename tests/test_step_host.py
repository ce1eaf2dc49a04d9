"""Host-side checks of ShardStep and the checkpoint loader (no GPU): the bucket
list must tile the partition, a gradient's float format must match the shard's
16-bit format, and a restored loss-scaler state must be one the library could
have produced between steps ("DeepSpeed complete guide" sections 2.2, 4.2 and
5.2)."""
import math

import pytest
import torch

from zero_mixed_precision_amd import FlatLayout, ShardStep, ZeroMPConfig, _lib
from zero_mixed_precision_amd.checkpoint import validate_scaler
from zero_mixed_precision_amd.step import buckets_or_all, check_grad_dtype


def test_buckets_that_tile_the_partition_are_kept():
    assert buckets_or_all(None, 100) == [(0, 100)]
    assert buckets_or_all([(0, 64), (64, 36)], 100) == [(0, 64), (64, 36)]
    lay = FlatLayout([4096 * 4096] * 4 + [4096] * 2)
    assert buckets_or_all(lay.buckets, lay.total) == [(b.start, b.size) for b in lay.buckets]


@pytest.mark.parametrize("buckets, n, what", [
    ([(0, 64), (72, 28)], 100, "does not start where"),          # a gap
    ([(0, 64), (56, 44)], 100, "does not start where"),          # an overlap
    ([(64, 36), (0, 64)], 100, "does not start where"),          # out of order
    ([(8, 92)], 100, "does not start where"),                    # not from 0
    ([(0, 64), (64, 40)], 100, "cover"),                         # past the end
    ([(0, 64)], 100, "cover"),                                   # short of the end
    ([(0, 60), (60, 40)], 100, "multiple of 8"),                 # misaligned start
    ([(0, -8), (-8, 108)], 100, "negative"),
])
def test_buckets_that_do_not_tile_the_partition_are_refused(buckets, n, what):
    with pytest.raises(ValueError, match=what):
        buckets_or_all(buckets, n)
    # the shard refuses them before it allocates anything
    with pytest.raises(ValueError, match=what):
        ShardStep(n, ZeroMPConfig(gradient_accumulation_steps=2), device="meta", buckets=buckets)


def test_the_layouts_absolute_buckets_are_refused_for_a_later_shard():
    """A rank's share takes buckets relative to its own start (buckets_in);
    the layout's absolute offsets would point past its arrays."""
    lay = FlatLayout([4096 * 64] * 8)
    start, count = lay.partition(world=2, rank=1)
    with pytest.raises(ValueError):
        buckets_or_all(lay.buckets, count)
    assert sum(s for _, s in buckets_or_all(lay.buckets_in(start, count), count)) == count


@pytest.mark.parametrize("bf16", [False, True])
def test_gradient_dtype_must_match_the_shard(bf16):
    check_grad_dtype(torch.int16, bf16, torch)
    check_grad_dtype(torch.bfloat16 if bf16 else torch.float16, bf16, torch)
    for wrong in (torch.float16 if bf16 else torch.bfloat16, torch.float32):
        with pytest.raises(ValueError, match="shard"):
            check_grad_dtype(wrong, bf16, torch)


def _between_steps(**kw):
    sc = _lib.DsScaler()
    sc.scale, sc.min_scale, sc.growth_window, sc.hysteresis, sc.hysteresis_left = 65536.0, 1.0, 1000, 2, 2
    sc.dynamic, sc.step, sc.iter, sc.skipped, sc.growth_count = 1, 40, 43, 3, 17
    for k, v in kw.items():
        setattr(sc, k, v)
    return sc


def test_a_scaler_state_between_steps_is_accepted():
    validate_scaler(_between_steps())
    validate_scaler(_between_steps(dynamic=0, scale=1.0, growth_count=0))
    validate_scaler(_between_steps(min_scale=1e-8, scale=1e-8))


@pytest.mark.parametrize("field, value", [
    ("scale", 0.0), ("scale", -2.0), ("scale", math.inf), ("scale", math.nan), ("min_scale", 0.0),
    ("growth_window", 0), ("hysteresis", 0), ("growth_count", 1000), ("growth_count", -1),
    ("hysteresis_left", 0), ("hysteresis_left", 3), ("dynamic", 2), ("consecutive_hysteresis", 5),
    ("iter", 44), ("step", -1), ("overflow", 1), ("grad_sumsq", 3.0),
])
def test_a_corrupt_scaler_state_is_refused(field, value):
    with pytest.raises(ValueError, match="loss-scaler"):
        validate_scaler(_between_steps(**{field: value}))
