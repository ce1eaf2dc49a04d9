"""CPU oracle for the ZeRO mixed-precision optimizer step -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product path (``zero_mixed_precision_amd``) never imports,
links or calls it, and it shares no code with the GPU library.

The arithmetic lives in ``oracle.c`` (plain scalar C loops, fp32 per the
memory table of "DeepSpeed complete guide" section 2); this module is the
ctypes binding plus the step sequence of one ZeRO optimizer step:

    accumulate (K > 1)  ->  overflow check  ->  Adam or skip  ->  scaler update

("DeepSpeed complete guide" section 5.1: backward scales and accumulates,
step() updates; section 4.2: dynamic loss scaling; "DeepSpeed" overview, core
features: gradient accumulation and dynamic loss scaling).  The bucket packing
oracle is in ``oracle.packing``.

Parity pins: every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_*.py``.  The scaler's branches that the pages give only
the keys' one-line meaning for (what happens after a hysteresis >= 2
decrease, ``consecutive_hysteresis``, the uncapped growth) are pinned to the
run-length closed form of their reading at every step of seeded and
structured overflow sequences; the static scale is pinned against torch's loss
scaler held at a fixed scale, and the 1e-8 floor of the guide's section 13.1,
where the scale stops being a power of two, is pinned.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-fexcess-precision=standard", "-mno-fma"]


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc into liboracle.so (plain scalar code)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


class ZoScaler(ctypes.Structure):
    """Mirror of ``zo_scaler`` in oracle.c."""
    _fields_ = [
        ("scale", ctypes.c_float),
        ("min_scale", ctypes.c_float),
        ("window", ctypes.c_int32),
        ("good_steps", ctypes.c_int32),
        ("hysteresis", ctypes.c_int32),
        ("hyst_left", ctypes.c_int32),
        ("dynamic", ctypes.c_int32),
        ("consecutive_hysteresis", ctypes.c_int32),
        ("applied", ctypes.c_int64),
        ("iters", ctypes.c_int64),
        ("skipped", ctypes.c_int64),
    ]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
        L.zo_dec16.argtypes, L.zo_dec16.restype = [ctypes.c_uint16], f32
        L.zo_enc16.argtypes, L.zo_enc16.restype = [f32], ctypes.c_uint16
        L.zo_dec16_array.argtypes, L.zo_dec16_array.restype = [vp, vp, i64], None
        L.zo_enc16_array.argtypes, L.zo_enc16_array.restype = [vp, vp, i64], None
        L.zo_decbf16.argtypes, L.zo_decbf16.restype = [ctypes.c_uint16], f32
        L.zo_encbf16.argtypes, L.zo_encbf16.restype = [f32], ctypes.c_uint16
        L.zo_decbf16_array.argtypes, L.zo_decbf16_array.restype = [vp, vp, i64], None
        L.zo_encbf16_array.argtypes, L.zo_encbf16_array.restype = [vp, vp, i64], None
        L.zo_accumulate.argtypes, L.zo_accumulate.restype = [vp, vp, i64, i32, i32], None
        L.zo_any_nonfinite16.argtypes, L.zo_any_nonfinite16.restype = [vp, i64, i32], i32
        L.zo_any_nonfinite32.argtypes, L.zo_any_nonfinite32.restype = [vp, i64], i32
        L.zo_adam_scalars.argtypes = [i64, f32, f32, f32, ctypes.POINTER(f32), ctypes.POINTER(f32)]
        L.zo_adam_scalars.restype = None
        L.zo_adam_scalars_range.argtypes = [i64, i64, f32, f32, f32, vp]
        L.zo_adam_scalars_range.restype = None
        L.zo_adam.argtypes = [vp, i32, i64, vp, vp, vp, vp, i32, f32, i32, i64, f32, f32, f32, f32, f32]
        L.zo_adam.restype = None
        L.zo_adam_mult.argtypes = [vp, i32, i64, vp, vp, vp, vp, i32, f32, i64, f32, f32, f32, f32, f32]
        L.zo_adam_mult.restype = None
        L.zo_lr_schedule.argtypes = [i32, i64, f32, f32, i64, i64]
        L.zo_lr_schedule.restype = f32
        L.zo_scaler_init.argtypes = [ctypes.POINTER(ZoScaler), f32, f32, i32, i32, i32, i32]
        L.zo_scaler_init.restype = None
        L.zo_scaler_update.argtypes = [ctypes.POINTER(ZoScaler), i32]
        L.zo_scaler_update.restype = None
        L.zo_scaler_sizeof.argtypes, L.zo_scaler_sizeof.restype = [], i64
        _require(L.zo_scaler_sizeof() == ctypes.sizeof(ZoScaler))
        _lib = L
    return _lib


def _require(ok: bool) -> None:
    """Argument checks that guard the C calls (kept under ``python -O``)."""
    if not ok:
        raise ValueError("oracle: array of the wrong type, size or layout")


def _ptr(a: np.ndarray) -> int:
    _require(a.flags["C_CONTIGUOUS"])
    return a.ctypes.data


# -- element codecs ----------------------------------------------------------

def dec16(h: np.ndarray) -> np.ndarray:
    """binary16 bit patterns (uint16) -> float32, from the format definition."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().zo_dec16_array(_ptr(h), _ptr(out), h.size)
    return out


def enc16(x: np.ndarray) -> np.ndarray:
    """float32 -> binary16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().zo_enc16_array(_ptr(x), _ptr(out), x.size)
    return out


def decbf16(h: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 (exact)."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().zo_decbf16_array(_ptr(h), _ptr(out), h.size)
    return out


def encbf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().zo_encbf16_array(_ptr(x), _ptr(out), x.size)
    return out


# 16-bit formats: "fp16" (IEEE binary16) or "bf16" (upper half of binary32)
FMT = {"fp16": 0, "bf16": 1}


def decode(h: np.ndarray, fmt: str = "fp16") -> np.ndarray:
    return decbf16(h) if fmt == "bf16" else dec16(h)


# -- the four steps ------------------------------------------------------------

def accumulate(acc: np.ndarray, g16: np.ndarray, overwrite: bool, fmt: str = "fp16") -> None:
    _require(acc.dtype == np.float32 and g16.dtype == np.uint16 and acc.size == g16.size)
    lib().zo_accumulate(_ptr(acc), _ptr(g16), acc.size, int(bool(overwrite)), FMT[fmt])


def any_nonfinite(grad: np.ndarray, fmt: str = "fp16") -> bool:
    if grad.dtype == np.uint16:
        return bool(lib().zo_any_nonfinite16(_ptr(grad), grad.size, FMT[fmt]))
    _require(grad.dtype == np.float32)
    return bool(lib().zo_any_nonfinite32(_ptr(grad), grad.size))


def adam_scalars(t: int, lr: float, beta1: float, beta2: float) -> tuple[float, float]:
    """(step_size, rbc2) of applied step t, as fp32 values."""
    a, b = ctypes.c_float(), ctypes.c_float()
    lib().zo_adam_scalars(int(t), lr, beta1, beta2, ctypes.byref(a), ctypes.byref(b))
    return a.value, b.value


def adam_scalars_range(t0: int, count: int, lr: float, beta1: float, beta2: float) -> np.ndarray:
    """float32[count, 2]: (step_size, rbc2) of the applied steps t0 .. t0 + count - 1."""
    out = np.empty((int(count), 2), np.float32)
    lib().zo_adam_scalars_range(int(t0), int(count), lr, beta1, beta2, _ptr(out))
    return out


def _gfmt(grad, fmt):
    return 2 if grad.dtype == np.float32 else FMT[fmt]


def adam(grad, master, m, v, p16, *, scale, accum_steps, t, lr, beta1, beta2, eps,
         weight_decay=0.0, fmt="fp16", param_fmt="fp16") -> None:
    """One applied Adam step, in place on master/m/v/p16 (see oracle.c).  ``fmt`` is
    the format of a 16-bit gradient, ``param_fmt`` that of the parameter copy."""
    n = master.size
    for a, dt in ((master, np.float32), (m, np.float32), (v, np.float32), (p16, np.uint16)):
        _require(a.dtype == dt and a.size == n and a.flags["C_CONTIGUOUS"])
    _require(grad.size == n and grad.dtype in (np.uint16, np.float32))
    lib().zo_adam(_ptr(grad), _gfmt(grad, fmt), n, _ptr(master), _ptr(m), _ptr(v), _ptr(p16),
                  FMT[param_fmt], scale, int(accum_steps), int(t), lr, beta1, beta2, eps, weight_decay)


def adam_mult(grad, master, m, v, p16, *, mult, t, lr, beta1, beta2, eps, weight_decay=0.0,
              fmt="fp16", param_fmt="fp16") -> None:
    """One applied Adam step with an explicit gradient multiplier (fp32)."""
    n = master.size
    _require(grad.size == n and grad.dtype in (np.uint16, np.float32))
    lib().zo_adam_mult(_ptr(grad), _gfmt(grad, fmt), n, _ptr(master), _ptr(m), _ptr(v), _ptr(p16),
                       FMT[param_fmt], float(np.float32(mult)), int(t), lr, beta1, beta2, eps,
                       weight_decay)


# -- global-norm clipping ("DeepSpeed complete guide" section 4.1 and 5.4:
#    gradient_clipping; section 5.1: step() includes clipping) ----------------

def grad_sumsq(grad: np.ndarray, fmt: str = "fp16") -> float:
    """Sum of squares of the stored gradient values, exactly, rounded once to fp64.

    fp16: each value is M * 2^E with integers M < 2^11, E in [-24, 5]; the
    squares M^2 * 2^(2E) are summed exactly as integers per exponent (Python
    integers), then divided by 2^48 with one correct rounding.  bf16 and fp32:
    the squares are exact in fp64 and math.fsum adds them with one rounding.
    Non-finite gradients give inf or nan (their step is skipped anyway)."""
    if grad.dtype == np.uint16 and fmt == "bf16":
        grad = decbf16(grad)
    if grad.dtype == np.uint16:
        h = grad.astype(np.int64)
        e = (h >> 10) & 0x1F
        if np.any(e == 31):
            return float("inf")
        f = h & 0x3FF
        M = np.where(e == 0, f, f + 1024)
        E = np.where(e == 0, -24, e - 25)
        total = 0
        for ex in np.unique(E):
            total += int(np.sum(M[E == ex] ** 2)) << int(2 * ex + 48)
        return total / (1 << 48)
    _require(grad.dtype == np.float32)
    if not np.all(np.isfinite(grad)):
        return float("inf")
    return math.fsum((grad.astype(np.float64) ** 2).tolist())


# Every finite fp32 square is an integer multiple of 2^-298 (the smallest
# subnormal is 2^-149), so sums of fp32 squares are exact as Python integers
# in that unit.
SUMSQ32_UNIT_BITS = 298


def sumsq32_exact_units(grad: np.ndarray):
    """Exact sum of squares of fp32 values, as an integer count of 2^-298, or
    None if a value is not finite.  Partial results of disjoint pieces add up
    exactly, so a sum over an array too large to hold at once is the sum of
    its pieces' results; ``units_to_float`` rounds it once.

    From the binary32 definition: the value with exponent field e and fraction
    f is M * 2^(E - 150) with M = f + 2^23, E = e for e >= 1, and M = f, E = 1
    for e = 0, so its square is M^2 * 4^(E - 1) units.  M^2 < 2^48 is taken in
    three parts (M = Mh * 2^12 + Ml, M^2 = Mh^2 * 2^24 + Mh*Ml * 2^13 + Ml^2),
    each below 2^24, and every part is summed per exponent field in fp64,
    which is exact while a piece holds at most 2^29 values."""
    _require(grad.dtype == np.float32)
    bits = np.ascontiguousarray(grad).view(np.uint32)
    _require(bits.size <= 1 << 29)
    e = ((bits >> 23) & 0xFF).astype(np.int64)
    if np.any(e == 0xFF):
        return None
    f = (bits & 0x7FFFFF).astype(np.int64)
    M = np.where(e == 0, f, f + (1 << 23))
    Mh, Ml = M >> 12, M & 0xFFF
    parts = [np.bincount(e, weights=(w).astype(np.float64), minlength=256)
             for w in (Mh * Mh, Mh * Ml, Ml * Ml)]
    total = 0
    for ex in range(255):
        hh, hl, ll = (int(p[ex]) for p in parts)
        if hh or hl or ll:
            total += ((hh << 24) + (hl << 13) + ll) << (2 * (max(ex, 1) - 1))
    return total


def units_to_float(total_units: int) -> float:
    """An exact sum of squares in units of 2^-298, rounded once to fp64."""
    return total_units / (1 << SUMSQ32_UNIT_BITS)


def clip_multiplier(sumsq: float, scale: float, accum_steps: int, max_norm: float) -> np.float32:
    """fp32 gradient multiplier: inv = fp32(1/(S*K)) without clipping; with a
    positive max_norm, fp32(inv * min(1, max_norm / (norm + 1e-6))) where
    norm = sqrt(sumsq) * inv is the L2 norm of the unscaled gradient (fp64)."""
    inv = np.float32(1.0) / (np.float32(scale) * np.float32(accum_steps))
    if max_norm <= 0:
        return inv
    inv64 = float(inv)
    norm = math.sqrt(sumsq) * inv64
    ratio = float(np.float32(max_norm)) / (norm + 1e-6)
    coef = ratio if ratio < 1.0 else 1.0
    return np.float32(inv64 * coef)


class Scaler:
    """Dynamic loss scaler state machine (oracle.c ``zo_scaler``)."""

    def __init__(self, init_scale=2.0 ** 16, min_scale=1.0, window=1000, hysteresis=1,
                 dynamic=True, consecutive_hysteresis=False):
        self.s = ZoScaler()
        lib().zo_scaler_init(ctypes.byref(self.s), init_scale, min_scale, int(window),
                             int(hysteresis), int(bool(dynamic)), int(bool(consecutive_hysteresis)))

    def update(self, overflow: bool) -> None:
        lib().zo_scaler_update(ctypes.byref(self.s), int(bool(overflow)))

    @property
    def scale(self) -> float:
        return self.s.scale

    @property
    def applied(self) -> int:
        return self.s.applied

    def as_dict(self) -> dict:
        return self.s.as_dict()


LR_WARMUP, LR_WARMUP_DECAY = 1, 2


class LrSchedule:
    """Per-step learning rate of a WarmupLR (``kind=LR_WARMUP``) or WarmupDecayLR
    (``kind=LR_WARMUP_DECAY``) schedule (oracle.c ``zo_lr_schedule``).  The
    iteration is the number of applied Adam steps before the current one."""

    def __init__(self, kind, warmup_min_lr, warmup_max_lr, warmup_num_steps, total_num_steps=0):
        self.kind = int(kind)
        self.min_lr, self.max_lr = float(warmup_min_lr), float(warmup_max_lr)
        self.warmup, self.total = int(warmup_num_steps), int(total_num_steps)

    def at(self, it: int) -> float:
        return lib().zo_lr_schedule(self.kind, int(it), self.min_lr, self.max_lr, self.warmup,
                                    self.total)


class State:
    """The flat partition's model state (fp16 params, fp32 master/m/v) plus the scaler."""

    def __init__(self, master, m, v, p16, scaler: Scaler, param_fmt: str = "fp16"):
        self.master, self.m, self.v, self.p16, self.scaler = master, m, v, p16, scaler
        self.param_fmt = param_fmt
        self.last_sumsq = 0.0


def step(state: State, grads, *, lr, beta1, beta2, eps, weight_decay=0.0, max_grad_norm=0.0,
         fmt="fp16") -> bool:
    """One full ZeRO optimizer step of the oracle; returns the overflow flag.

    ``grads`` is one uint16 array (K = 1: the fp16 gradient is consumed
    directly) or a list of K uint16 micro-batch gradients (K > 1: summed into
    an fp32 buffer in micro-batch order first); ``fmt`` is their 16-bit format
    ("fp16" or "bf16").  ``lr`` is a number or an ``LrSchedule``, which is
    read at the count of steps applied so far.  ``max_grad_norm`` > 0 clips the unscaled gradient to
    that global L2 norm.  ``state.last_sumsq`` keeps
    the step's gradient sum of squares when clipping.
    """
    if isinstance(grads, np.ndarray):
        grads = [grads]
    K = len(grads)
    if K == 1:
        grad = np.ascontiguousarray(grads[0], dtype=np.uint16)
    else:
        grad = np.empty(state.master.size, np.float32)
        for k, g in enumerate(grads):
            accumulate(grad, np.ascontiguousarray(g, dtype=np.uint16), overwrite=(k == 0), fmt=fmt)
    overflow = any_nonfinite(grad, fmt)
    if not overflow:
        if isinstance(lr, LrSchedule):
            lr = lr.at(state.scaler.applied)
        kw = dict(t=state.scaler.applied + 1, lr=lr, beta1=beta1, beta2=beta2, eps=eps,
                  weight_decay=weight_decay, fmt=fmt, param_fmt=state.param_fmt)
        if max_grad_norm > 0:
            state.last_sumsq = grad_sumsq(grad, fmt)
            mult = clip_multiplier(state.last_sumsq, state.scaler.scale, K, max_grad_norm)
            adam_mult(grad, state.master, state.m, state.v, state.p16, mult=mult, **kw)
        else:
            adam(grad, state.master, state.m, state.v, state.p16, scale=state.scaler.scale,
                 accum_steps=K, **kw)
    state.scaler.update(overflow)
    return overflow
