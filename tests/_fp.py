"""Small floating-point helpers for the tests (ulp distances, bit views)."""
import numpy as np


def f32_bits(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)


def ulp32(x) -> np.ndarray:
    """Spacing of fp32 numbers at |x|."""
    return np.spacing(np.abs(np.asarray(x, dtype=np.float32))).astype(np.float64)


def ulp_diff32(a, b) -> np.ndarray:
    """Distance in fp32 ulps between two fp32 arrays (ordered-integer metric).
    NaN vs NaN counts as 0; NaN vs number as a huge value."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = np.ascontiguousarray(b, dtype=np.float32)
    ia = a.view(np.int32).astype(np.int64)
    ib = b.view(np.int32).astype(np.int64)
    ia = np.where(ia < 0, -(ia & 0x7FFFFFFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFFFFFF), ib)
    d = np.abs(ia - ib)
    na, nb = np.isnan(a), np.isnan(b)
    d = np.where(na & nb, 0, d)
    d = np.where(na ^ nb, 1 << 40, d)
    return d


def ulp_diff16(a, b) -> np.ndarray:
    """Distance in fp16 ulps between two arrays of fp16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.uint16)
    b = np.ascontiguousarray(b, dtype=np.uint16)
    ia = a.view(np.int16).astype(np.int64)
    ib = b.view(np.int16).astype(np.int64)
    ia = np.where(ia < 0, -(ia & 0x7FFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFF), ib)
    d = np.abs(ia - ib)
    na = ((a & 0x7C00) == 0x7C00) & ((a & 0x03FF) != 0)
    nb = ((b & 0x7C00) == 0x7C00) & ((b & 0x03FF) != 0)
    d = np.where(na & nb, 0, d)
    d = np.where(na ^ nb, 1 << 40, d)
    return d
