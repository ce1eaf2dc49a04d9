"""Seeded synthetic inputs for the ZeRO optimizer step (host and device sides).

This module is the one piece shared by the oracle's tests and the GPU path's
tests and benchmark.  It holds none of the optimizer's arithmetic: it only
draws numbers.  Random values are a pure function of (stream key, element
index), so any element can be regenerated on its own on the host, and the
device fill kernels in ``csrc/synth.hip`` write the very same bits.

Generator.  SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014; output mix with Vigna's published
constants): the state of element i is ``key + (i + 1) * 0x9E3779B97F4A7C15``
(mod 2^64) and its 64-bit output is the mix of that state.

Distributions.  A normal draw is the quantile-table lookup
``Phi^-1((j + 0.5) / 65536)`` for the low 16 bits j of the output (a
65,536-level discretisation of N(0, 1), |z| <= 4.17); the tables are built
once on the host in fp64 and uploaded, so host and device agree bit for bit
without evaluating any transcendental function on the device.
  * fp16 gradient  = fp16(z * sigma * loss_scale_mult)  (table per sigma/mult)
  * heavy tail     : when output bits 32..63 fall below 0.001 * 2^32, the
                     draw uses the table scaled by 100 instead
  * fp32 master    = fp32(z * sigma_master), then the low 8 fraction bits are
                     XORed with output bits 16..23 (about 2^24 distinct values)
  * fp16 initial parameter copy: any pattern will do (the step only writes
    it); it is drawn like a gradient from its own stream so a skipped step's
    "left unchanged" is observable.
"""
from __future__ import annotations

import ctypes
import functools
import os
import statistics

import numpy as np

SEED = 20261202
GOLDEN = 0x9E3779B97F4A7C15
M1 = 0xBF58476D1CE4E5B9
M2 = 0x94D049BB133111EB
MASK64 = (1 << 64) - 1
TAIL_THRESH = int(round(0.001 * 2 ** 32))  # Bernoulli(0.001) on 32 output bits

# array ids of the streams
ARR_MASTER, ARR_P16, ARR_GRAD, ARR_INJECT = 1, 2, 3, 4


def mix64(z: int) -> int:
    """SplitMix64 output mix of one 64-bit state (Python ints)."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * M1) & MASK64
    z = ((z ^ (z >> 27)) * M2) & MASK64
    return z ^ (z >> 31)


def stream_key(*parts: int, seed: int = SEED) -> int:
    """Key of the stream named by integer parts, e.g. (config, array, step, micro)."""
    k = seed & MASK64
    for p in parts:
        k = mix64((k ^ (int(p) & MASK64)) + GOLDEN)
    return k


def raw64(key: int, idx) -> np.ndarray:
    """64-bit outputs for element indices ``idx`` (uint64 array) of stream ``key``."""
    idx = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(key) + (idx + np.uint64(1)) * np.uint64(GOLDEN)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(M1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(M2)
        z = z ^ (z >> np.uint64(31))
    return z


@functools.lru_cache(maxsize=None)
def _quantiles() -> np.ndarray:
    nd = statistics.NormalDist()
    return np.array([nd.inv_cdf((j + 0.5) / 65536.0) for j in range(65536)], dtype=np.float64)


@functools.lru_cache(maxsize=None)
def table16(scale: float) -> np.ndarray:
    """uint16 bit patterns of fp16(q_j * scale), j = 0..65535 (all finite)."""
    t = (_quantiles() * float(scale)).astype(np.float16)
    if not np.all(np.isfinite(t)):
        raise ValueError("fp16 table overflows at scale %g" % scale)
    t.setflags(write=False)
    return t.view(np.uint16)


@functools.lru_cache(maxsize=None)
def tablebf16(scale: float) -> np.ndarray:
    """uint16 bit patterns of bf16(q_j * scale) (drawn through torch's bf16 cast)."""
    import torch
    t = torch.from_numpy(_quantiles() * float(scale)).to(torch.float32).to(torch.bfloat16)
    out = t.view(torch.int16).numpy().view(np.uint16).copy()
    out.setflags(write=False)
    return out


@functools.lru_cache(maxsize=None)
def table32(scale: float) -> np.ndarray:
    """uint32 bit patterns of fp32(q_j * scale), j = 0..65535."""
    t = (_quantiles() * float(scale)).astype(np.float32).view(np.uint32).copy()
    t.setflags(write=False)
    return t


class GradSpec:
    """Distribution of a 16-bit gradient: N(0, sigma) * mult, optional heavy tail,
    stored as fp16 (``fmt="fp16"``) or bf16."""

    def __init__(self, sigma: float, mult: float, heavy_tail: bool = False, fmt: str = "fp16"):
        self.sigma, self.mult, self.heavy_tail = float(sigma), float(mult), bool(heavy_tail)
        self.fmt = fmt

    def _table(self, scale):
        return tablebf16(scale) if self.fmt == "bf16" else table16(scale)

    @property
    def table(self) -> np.ndarray:
        return self._table(self.sigma * self.mult)

    @property
    def tail_table(self) -> np.ndarray:
        return self._table(self.sigma * self.mult * 100.0) if self.heavy_tail else self.table

    @property
    def tail_thresh(self) -> int:
        return TAIL_THRESH if self.heavy_tail else 0


# -- host side ----------------------------------------------------------------

def host_grad16(key: int, idx, spec: GradSpec) -> np.ndarray:
    """fp16 gradient bit patterns (uint16) at element indices ``idx``."""
    z = raw64(key, idx)
    j = (z & np.uint64(0xFFFF)).astype(np.int64)
    out = spec.table[j]
    if spec.heavy_tail:
        tail = (z >> np.uint64(32)) < np.uint64(spec.tail_thresh)
        out = np.where(tail, spec.tail_table[j], out)
    return np.ascontiguousarray(out, dtype=np.uint16)


def host_master32(key: int, idx, sigma: float) -> np.ndarray:
    """fp32 master values at element indices ``idx``."""
    z = raw64(key, idx)
    j = (z & np.uint64(0xFFFF)).astype(np.int64)
    bits = table32(sigma)[j] ^ ((z >> np.uint64(16)) & np.uint64(0xFF)).astype(np.uint32)
    return np.ascontiguousarray(bits).view(np.float32)


def inject_site(seed_parts, n: int, micro: int = 1):
    """(micro-batch k, element index) of an injected +inf, from its own stream."""
    z = mix64(stream_key(*seed_parts) + GOLDEN)
    return (z >> 48) % micro, (z & ((1 << 48) - 1)) % n


# -- device side ----------------------------------------------------------------

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libdssynth.so")
_dlib = None


def _bind_torch_hip_runtime() -> None:
    """Make PyTorch's HIP runtime the global definition of the HIP symbols
    before loading libdssynth.so, so its kernels launch on the runtime that
    owns torch's streams and memory (a PyTorch-ROCm install carries its own
    libamdhip64 besides the system one the library links against)."""
    try:
        import torch
    except ImportError:
        return
    path = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
    if os.path.exists(path):
        ctypes.CDLL(path, mode=ctypes.RTLD_GLOBAL)


def device_lib():
    """ctypes handle of libdssynth.so (device fill kernels); raises if not built."""
    global _dlib
    if _dlib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError("libdssynth.so is not built: run __graft_entry__.build()")
        _bind_torch_hip_runtime()
        L = ctypes.CDLL(_LIB_PATH)
        vp, i64, u64, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32
        L.synth_fill_grad16.argtypes = [vp, i64, i64, u64, vp, vp, u32, vp]
        L.synth_fill_master32.argtypes = [vp, i64, i64, u64, vp, vp]
        L.synth_copy.argtypes = [vp, vp, i64, vp]
        L.synth_stream_mix.argtypes = [vp, vp, vp, vp, vp, i64, vp]
        L.synth_stream_mix_shape.argtypes = [vp, vp, vp, vp, vp, i64, ctypes.c_int32, vp]
        for f in (L.synth_fill_grad16, L.synth_fill_master32, L.synth_copy, L.synth_stream_mix,
                  L.synth_stream_mix_shape):
            f.restype = ctypes.c_int
        _dlib = L
    return _dlib


def _stream_ptr(torch, stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"{what} failed with HIP error {rc}")


class DeviceTables:
    """Generator tables resident on one device (uploaded once per distribution)."""

    def __init__(self, torch, device):
        self.torch, self.device, self._cache = torch, device, {}

    def get(self, arr: np.ndarray):
        key = (arr.dtype.str, arr.size, arr.ctypes.data)
        t = self._cache.get(key)
        if t is None:
            # a private writable copy: the tables are read-only module constants
            host = self.torch.from_numpy(arr.view(np.int16 if arr.dtype == np.uint16 else np.int32).copy())
            t = host.to(self.device)
            self._cache[key] = (t, arr)  # keep arr alive so its address stays unique
        else:
            t = t[0]
        return t


def device_fill_grad16(torch, tables: DeviceTables, out, key: int, spec: GradSpec,
                       start: int = 0, stream=None) -> None:
    """Write the fp16 gradient of stream ``key`` for elements [start, start+numel) into ``out``."""
    tab = tables.get(spec.table)
    tail = tables.get(spec.tail_table)
    _check(device_lib().synth_fill_grad16(out.data_ptr(), out.numel(), int(start), key,
                                           tab.data_ptr(), tail.data_ptr(), spec.tail_thresh,
                                           _stream_ptr(torch, stream)), "synth_fill_grad16")


def device_fill_master32(torch, tables: DeviceTables, out, key: int, sigma: float,
                         start: int = 0, stream=None) -> None:
    tab = tables.get(table32(sigma))
    _check(device_lib().synth_fill_master32(out.data_ptr(), out.numel(), int(start), key,
                                             tab.data_ptr(), _stream_ptr(torch, stream)),
           "synth_fill_master32")


def device_copy(torch, dst, src, stream=None) -> None:
    """Plain 16-byte-vector copy (bandwidth and counter calibration)."""
    nbytes = src.numel() * src.element_size()
    if nbytes % 16 != 0 or dst.numel() * dst.element_size() < nbytes:
        raise ValueError("device_copy: the source must be a whole number of 16-byte vectors and fit in dst")
    _check(device_lib().synth_copy(dst.data_ptr(), src.data_ptr(), nbytes // 16,
                                   _stream_ptr(torch, stream)), "synth_copy")


def device_stream_mix(torch, g16, a, b, c, h16, stream=None, small_tiles=False) -> None:
    """Data movement of the optimizer step with no arithmetic: reads 14 B and
    writes 14 B per element (fp16 + 3 x fp32 in, 3 x fp32 + fp16 out), in
    256-lane blocks of 4 quads per lane (the step's tiling) or, with
    small_tiles, 64-lane blocks of one quad per lane."""
    n = a.numel()
    _check(device_lib().synth_stream_mix_shape(g16.data_ptr(), a.data_ptr(), b.data_ptr(), c.data_ptr(),
                                               h16.data_ptr(), n, int(bool(small_tiles)),
                                               _stream_ptr(torch, stream)),
           "synth_stream_mix")
