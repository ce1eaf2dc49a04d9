"""ctypes binding of libdszero.so (include/dszero.h), same names as the C ABI.

Argument marshalling only: every entry point forwards to the native library,
which enqueues HIP kernels.  Pointers may be passed as integers or as torch
tensors (their ``data_ptr()``); ``stream`` defaults to torch's current HIP
stream.  A non-OK status raises ``DsError``.  If the library has not been
built, importing the binding raises -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdszero.so")

DS_OK, DS_ERR_NULL, DS_ERR_SIZE, DS_ERR_ALIGN, DS_ERR_DTYPE, DS_ERR_HPARAM, DS_ERR_ALIAS, DS_ERR_HIP = range(8)
DS_FP16, DS_FP32, DS_BF16 = 1, 2, 3

EXPORTED = (
    "ds_scaler_size", "ds_state_init", "ds_state_read", "ds_state_write", "ds_accumulate",
    "ds_check_overflow", "ds_adam_step", "ds_update_loss_scale", "ds_adam_bias_scalars",
    "ds_layout_greedy", "ds_partition_range", "ds_status_string", "ds_sumsq_workspace_bytes",
    "ds_check_overflow_sumsq", "ds_accumulate_sumsq", "ds_adam_step_sched", "ds_lr_scalars",
    "ds_adam_step_fused", "ds_accumulate_multi", "ds_check_overflow_sumsq_noalloc", "ds_adam_step_double_buffered",
    "ds_accumulate_adam_double_buffered", "ds_update_loss_scale_double_buffered",
)
DS_NOALLOC_MAX_ELEMS = 17175674880
DS_LR_WARMUP, DS_LR_WARMUP_DECAY = 1, 2


class DsScaler(ctypes.Structure):
    """Mirror of ``ds_scaler`` (128 bytes)."""
    _fields_ = [
        ("scale", ctypes.c_float),
        ("min_scale", ctypes.c_float),
        ("growth_window", ctypes.c_int32),
        ("growth_count", ctypes.c_int32),
        ("hysteresis", ctypes.c_int32),
        ("hysteresis_left", ctypes.c_int32),
        ("dynamic", ctypes.c_int32),
        ("overflow", ctypes.c_uint32),
        ("step", ctypes.c_int64),
        ("iter", ctypes.c_int64),
        ("skipped", ctypes.c_int64),
        ("consecutive_hysteresis", ctypes.c_int32),
        ("last_overflow", ctypes.c_uint32),
        ("grad_sumsq", ctypes.c_double),
        ("last_grad_sumsq", ctypes.c_double),
        ("blocks_done", ctypes.c_uint32),
        ("sumsq_blocks_done", ctypes.c_uint32),
        ("current", ctypes.c_uint32),
        ("reserved0", ctypes.c_uint32),
        ("db_tickets", ctypes.c_uint64),
        ("reserved", ctypes.c_uint8 * 24),
    ]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_ if not name.startswith("reserved")}


class DsLrSchedule(ctypes.Structure):
    """Mirror of ``ds_lr_schedule`` (32 bytes, host memory)."""
    _fields_ = [
        ("kind", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("warmup_num_steps", ctypes.c_int64),
        ("total_num_steps", ctypes.c_int64),
        ("warmup_min_lr", ctypes.c_float),
        ("warmup_max_lr", ctypes.c_float),
    ]

    @classmethod
    def make(cls, kind, warmup_min_lr, warmup_max_lr, warmup_num_steps, total_num_steps=0):
        return cls(int(kind), 0, int(warmup_num_steps), int(total_num_steps), float(warmup_min_lr),
                   float(warmup_max_lr))


class DsError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = int(status)
        super().__init__(f"{where}: {status_string(status)}")


def bind_torch_hip_runtime() -> None:
    """Put the HIP runtime that PyTorch uses into the global symbol scope.

    A PyTorch-ROCm install carries its own libamdhip64; the library is linked
    against the system one.  The dynamic linker binds the library's HIP calls
    (fatbinary registration, kernel launches) to the first definition in the
    global scope, so without this step the binding depends on import order: if
    libdszero.so loads before torch, its kernels go to a second runtime that
    knows nothing of torch's streams (and a hipStream_t of one runtime is not a
    stream of the other).  With torch's runtime global first, every launch uses
    the runtime that owns the caller's memory and streams.  Without torch (a
    plain C caller) the library uses the runtime it was linked against.
    """
    try:
        import torch
    except ImportError:
        return
    path = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
    if os.path.exists(path):
        ctypes.CDLL(path, mode=ctypes.RTLD_GLOBAL)


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                          "(python zero_mixed_precision_amd/build.py)")
    bind_torch_hip_runtime()
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
    sig = {
        "ds_scaler_size": ([], ctypes.c_size_t),
        "ds_state_init": ([vp, f32, f32, i32, i32, i32, i32, vp], ctypes.c_int),
        "ds_state_read": ([vp, ctypes.POINTER(DsScaler), vp], ctypes.c_int),
        "ds_state_write": ([vp, ctypes.POINTER(DsScaler), vp], ctypes.c_int),
        "ds_accumulate": ([vp, vp, ctypes.c_int, i64, i32, vp, vp], ctypes.c_int),
        "ds_check_overflow": ([vp, vp, ctypes.c_int, i64, vp], ctypes.c_int),
        "ds_adam_step": ([vp, vp, vp, vp, vp, ctypes.c_int, vp, ctypes.c_int, i64, f32, f32, f32, f32, f32,
                          f32, i32, vp], ctypes.c_int),
        "ds_sumsq_workspace_bytes": ([i64], ctypes.c_size_t),
        "ds_check_overflow_sumsq": ([vp, vp, ctypes.c_int, i64, vp, ctypes.c_size_t, vp], ctypes.c_int),
        "ds_check_overflow_sumsq_noalloc": ([vp, vp, ctypes.c_int, i64, vp], ctypes.c_int),
        "ds_adam_step_double_buffered": ([vp, ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(vp),
                                          ctypes.POINTER(vp), ctypes.c_int, vp, ctypes.c_int, i64, f32,
                                          ctypes.POINTER(DsLrSchedule), f32, f32, f32, f32, i32, vp], ctypes.c_int),
        "ds_accumulate_adam_double_buffered": ([vp, ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(vp),
                                                ctypes.POINTER(vp), ctypes.c_int, vp, ctypes.POINTER(vp), i32,
                                                ctypes.c_int, i64, f32, ctypes.POINTER(DsLrSchedule), f32, f32, f32,
                                                f32, i32, vp], ctypes.c_int),
        "ds_update_loss_scale_double_buffered": ([vp, vp], ctypes.c_int),
        "ds_accumulate_sumsq": ([vp, vp, ctypes.c_int, i64, i32, vp, vp, ctypes.c_size_t, vp], ctypes.c_int),
        "ds_accumulate_multi": ([vp, ctypes.POINTER(vp), i32, ctypes.c_int, i64, i32, vp, vp, ctypes.c_size_t, vp],
                                ctypes.c_int),
        "ds_update_loss_scale": ([vp, vp], ctypes.c_int),
        "ds_adam_bias_scalars": ([vp, f32, f32, f32, vp, vp], ctypes.c_int),
        "ds_adam_step_sched": ([vp, vp, vp, vp, vp, ctypes.c_int, vp, ctypes.c_int, i64,
                                ctypes.POINTER(DsLrSchedule), f32, f32, f32, f32, f32, i32, vp], ctypes.c_int),
        "ds_lr_scalars": ([vp, ctypes.POINTER(DsLrSchedule), f32, f32, vp, vp], ctypes.c_int),
        "ds_adam_step_fused": ([vp, vp, vp, vp, vp, ctypes.c_int, vp, ctypes.c_int, i64, f32,
                                ctypes.POINTER(DsLrSchedule), f32, f32, f32, f32, f32, i32, vp], ctypes.c_int),
        "ds_layout_greedy": ([vp, i32, i64, i64, vp, vp, vp, vp, ctypes.POINTER(i32),
                              ctypes.POINTER(i64)], ctypes.c_int),
        "ds_partition_range": ([i64, i32, i32, i64, ctypes.POINTER(i64), ctypes.POINTER(i64)],
                               ctypes.c_int),
        "ds_status_string": ([ctypes.c_int], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        try:
            fn = getattr(L, name)
        except AttributeError:
            raise ImportError(f"{LIB_PATH} does not export {name}: it is older than include/dszero.h; "
                              "rebuild it (python zero_mixed_precision_amd/build.py)") from None
        fn.argtypes, fn.restype = args, res
    if L.ds_scaler_size() != ctypes.sizeof(DsScaler):
        raise ImportError("ds_scaler layout mismatch between libdszero.so and the binding")
    return L


lib = _load()


def status_string(status: int) -> str:
    return lib.ds_status_string(int(status)).decode()


def _p(x, nbytes=0, what="pointer"):
    """Pointer argument: int, None, or a torch tensor.

    An int is passed through as it is (the caller vouches for it, as in C).  A
    tensor must live on the GPU, be contiguous and hold at least ``nbytes``
    bytes from its first element: a host tensor or a too-short one would
    otherwise reach the kernels as an address they may not read or write.
    """
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not getattr(x, "is_cuda", False):
        raise ValueError(f"{what}: expected a tensor in GPU memory, got one on {x.device}")
    if not x.is_contiguous():
        raise ValueError(f"{what}: expected a contiguous tensor")
    have = x.numel() * x.element_size()
    if nbytes > 0 and have < nbytes:
        raise ValueError(f"{what}: tensor holds {have} bytes, the call reads or writes {nbytes}")
    return x.data_ptr()


def _esize(dtype) -> int:
    return 4 if int(dtype) == DS_FP32 else 2


def _scaler(st):
    return _p(st, ctypes.sizeof(DsScaler), "ds_scaler state")


def _s(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ok(rc: int, where: str) -> None:
    if rc != DS_OK:
        raise DsError(rc, where)


def ds_scaler_size() -> int:
    return lib.ds_scaler_size()


def ds_state_init(st, init_scale, min_scale, growth_window, hysteresis, consecutive_hysteresis=0,
                  dynamic=1, stream=None) -> None:
    _ok(lib.ds_state_init(_scaler(st), init_scale, min_scale, int(growth_window), int(hysteresis),
                          int(consecutive_hysteresis), int(dynamic), _s(stream)), "ds_state_init")


def ds_state_read(st, stream=None) -> DsScaler:
    out = DsScaler()
    _ok(lib.ds_state_read(_scaler(st), ctypes.byref(out), _s(stream)), "ds_state_read")
    return out


def ds_state_write(st, value: DsScaler, stream=None) -> None:
    _ok(lib.ds_state_write(_scaler(st), ctypes.byref(value), _s(stream)), "ds_state_write")


def ds_accumulate(acc, g16, gdt, n, overwrite, st_or_null=None, stream=None) -> None:
    n = int(n)
    _ok(lib.ds_accumulate(_p(acc, 4 * n, "acc"), _p(g16, 2 * n, "gradient"), int(gdt), n, int(bool(overwrite)),
                          _scaler(st_or_null), _s(stream)), "ds_accumulate")


def ds_check_overflow(st, grad, dtype, n, stream=None) -> None:
    n = int(n)
    _ok(lib.ds_check_overflow(_scaler(st), _p(grad, _esize(dtype) * n, "gradient"), int(dtype), n, _s(stream)),
        "ds_check_overflow")


def _adam_arrays(master, m, v, p16, pdt, grad, dtype, n):
    """The five array arguments of the Adam entry points, checked for n elements."""
    return (_p(master, 4 * n, "master"), _p(m, 4 * n, "m"), _p(v, 4 * n, "v"), _p(p16, 2 * n, "p16"), int(pdt),
            _p(grad, _esize(dtype) * n, "gradient"), int(dtype), n)


def ds_adam_step(st, master, m, v, p16, pdt, grad, dtype, n, lr, beta1, beta2, eps, weight_decay,
                 max_grad_norm, accum_steps, stream=None) -> None:
    n = int(n)
    _ok(lib.ds_adam_step(_scaler(st), *_adam_arrays(master, m, v, p16, pdt, grad, dtype, n), lr, beta1, beta2,
                         eps, weight_decay, max_grad_norm, int(accum_steps), _s(stream)), "ds_adam_step")


def ds_adam_step_sched(st, master, m, v, p16, pdt, grad, dtype, n, sched: DsLrSchedule, beta1, beta2, eps,
                       weight_decay, max_grad_norm, accum_steps, stream=None) -> None:
    n = int(n)
    _ok(lib.ds_adam_step_sched(_scaler(st), *_adam_arrays(master, m, v, p16, pdt, grad, dtype, n),
                               ctypes.byref(sched), beta1, beta2, eps, weight_decay, max_grad_norm,
                               int(accum_steps), _s(stream)), "ds_adam_step_sched")


def ds_adam_step_fused(st, master, m, v, p16, pdt, grad, dtype, n, lr, sched, beta1, beta2, eps, weight_decay,
                       max_grad_norm, accum_steps, stream=None) -> None:
    """ds_adam_step (sched None) or ds_adam_step_sched, then the scaler update, in one kernel."""
    n = int(n)
    sched_p = ctypes.byref(sched) if sched is not None else None
    _ok(lib.ds_adam_step_fused(_scaler(st), *_adam_arrays(master, m, v, p16, pdt, grad, dtype, n), lr, sched_p,
                               beta1, beta2, eps, weight_decay, max_grad_norm, int(accum_steps), _s(stream)),
        "ds_adam_step_fused")


def _pair(arrs, nbytes, what):
    """Host array of the two copies' device addresses (tensors are checked as by _p)."""
    if len(arrs) != 2:
        raise ValueError(f"{what}: expected two copies")
    return (ctypes.c_void_p * 2)(*[_p(a, nbytes, f"{what}[{k}]") for k, a in enumerate(arrs)])


def ds_adam_step_double_buffered(st, master2, m2, v2, p16_2, pdt, grad, dtype, n, lr, sched, beta1, beta2, eps,
                                 weight_decay, accum_steps, stream=None) -> None:
    """The check fused into the Adam pass over two copies of the state: master2, m2, v2, p16_2 are pairs
    (copy 0, copy 1) of tensors or device addresses; the copy holding the state is the state's ``current``."""
    n = int(n)

    sched_p = ctypes.byref(sched) if sched is not None else None
    _ok(lib.ds_adam_step_double_buffered(_scaler(st), _pair(master2, 4 * n, "master"), _pair(m2, 4 * n, "m"),
                                         _pair(v2, 4 * n, "v"), _pair(p16_2, 2 * n, "p16"), int(pdt),
                                         _p(grad, _esize(dtype) * n, "gradient"), int(dtype), n, lr, sched_p,
                                         beta1, beta2, eps, weight_decay, int(accum_steps), _s(stream)),
        "ds_adam_step_double_buffered")


def ds_accumulate_adam_double_buffered(st, master2, m2, v2, p16_2, pdt, acc, grads, gdt, n, lr, sched, beta1, beta2,
                                       eps, weight_decay, accum_steps, stream=None) -> None:
    """The step's last micro-batches (``grads``: 1..8 tensors or device addresses, in order) folded into the
    double-buffered Adam pass; ``acc`` is the running sum of the earlier ones (or None when ``grads`` are all
    of them).  End the step with ds_update_loss_scale_double_buffered."""
    n = int(n)

    ptrs = (ctypes.c_void_p * max(len(grads), 1))(*[_p(g, 2 * n, f"gradient {k}") for k, g in enumerate(grads)])
    sched_p = ctypes.byref(sched) if sched is not None else None
    _ok(lib.ds_accumulate_adam_double_buffered(_scaler(st), _pair(master2, 4 * n, "master"), _pair(m2, 4 * n, "m"),
                                               _pair(v2, 4 * n, "v"), _pair(p16_2, 2 * n, "p16"), int(pdt),
                                               _p(acc, 4 * n, "acc"), ptrs, len(grads), int(gdt), n, lr, sched_p,
                                               beta1, beta2, eps, weight_decay, int(accum_steps), _s(stream)),
        "ds_accumulate_adam_double_buffered")


def ds_update_loss_scale_double_buffered(st, stream=None) -> None:
    _ok(lib.ds_update_loss_scale_double_buffered(_scaler(st), _s(stream)), "ds_update_loss_scale_double_buffered")


def ds_sumsq_workspace_bytes(n) -> int:
    return lib.ds_sumsq_workspace_bytes(int(n))


def _nbytes(ws, ws_bytes):
    if ws_bytes is not None:
        return int(ws_bytes)
    return ws.numel() * ws.element_size()


def ds_check_overflow_sumsq(st, grad, dtype, n, workspace, workspace_bytes=None, stream=None) -> None:
    n = int(n)
    _ok(lib.ds_check_overflow_sumsq(_scaler(st), _p(grad, _esize(dtype) * n, "gradient"), int(dtype), n,
                                    _p(workspace, ds_sumsq_workspace_bytes(max(n, 0)), "workspace"),
                                    _nbytes(workspace, workspace_bytes), _s(stream)),
        "ds_check_overflow_sumsq")


def ds_check_overflow_sumsq_noalloc(st, grad, dtype, n, stream=None) -> None:
    n = int(n)
    _ok(lib.ds_check_overflow_sumsq_noalloc(_scaler(st), _p(grad, _esize(dtype) * n, "gradient"), int(dtype), n,
                                            _s(stream)),
        "ds_check_overflow_sumsq_noalloc")


def ds_accumulate_sumsq(acc, g16, gdt, n, overwrite, st, workspace, workspace_bytes=None,
                        stream=None) -> None:
    n = int(n)
    _ok(lib.ds_accumulate_sumsq(_p(acc, 4 * n, "acc"), _p(g16, 2 * n, "gradient"), int(gdt), n,
                                int(bool(overwrite)), _scaler(st),
                                _p(workspace, ds_sumsq_workspace_bytes(max(n, 0)), "workspace"),
                                _nbytes(workspace, workspace_bytes), _s(stream)),
        "ds_accumulate_sumsq")


def ds_accumulate_multi(acc, grads, gdt, n, overwrite, st_or_null=None, workspace=None, workspace_bytes=None,
                        stream=None) -> None:
    """``grads``: a sequence of 1..8 micro-batch gradients (tensors or device
    addresses), folded into ``acc`` in one pass in this order."""
    n = int(n)
    ptrs = (ctypes.c_void_p * max(len(grads), 1))(*[_p(g, 2 * n, f"gradient {k}") for k, g in enumerate(grads)])
    ws_bytes = 0 if workspace is None else _nbytes(workspace, workspace_bytes)
    ws = None if workspace is None else _p(workspace, ds_sumsq_workspace_bytes(max(n, 0)), "workspace")
    _ok(lib.ds_accumulate_multi(_p(acc, 4 * n, "acc"), ptrs, len(grads), int(gdt), n, int(bool(overwrite)),
                                _scaler(st_or_null), ws, ws_bytes, _s(stream)), "ds_accumulate_multi")


def ds_update_loss_scale(st, stream=None) -> None:
    _ok(lib.ds_update_loss_scale(_scaler(st), _s(stream)), "ds_update_loss_scale")


def ds_adam_bias_scalars(st, lr, beta1, beta2, out2, stream=None) -> None:
    _ok(lib.ds_adam_bias_scalars(_scaler(st), lr, beta1, beta2, _p(out2, 8, "out2"), _s(stream)),
        "ds_adam_bias_scalars")


def ds_lr_scalars(st, sched: DsLrSchedule, beta1, beta2, out3, stream=None) -> None:
    _ok(lib.ds_lr_scalars(_scaler(st), ctypes.byref(sched), beta1, beta2, _p(out3, 12, "out3"), _s(stream)),
        "ds_lr_scalars")


def ds_layout_greedy(numels, cap, align):
    """Host-only greedy packing; returns (offsets, bucket_of, bucket_starts, bucket_sizes, total)."""
    n = len(numels)
    c_num = (ctypes.c_int64 * max(n, 1))(*[int(x) for x in numels])
    offs = (ctypes.c_int64 * max(n, 1))()
    bof = (ctypes.c_int32 * max(n, 1))()
    bst = (ctypes.c_int64 * max(n, 1))()
    bsz = (ctypes.c_int64 * max(n, 1))()
    nb, total = ctypes.c_int32(), ctypes.c_int64()
    _ok(lib.ds_layout_greedy(c_num, n, int(cap), int(align), offs, bof, bst, bsz, ctypes.byref(nb),
                             ctypes.byref(total)), "ds_layout_greedy")
    k = nb.value
    return list(offs[:n]), list(bof[:n]), list(bst[:k]), list(bsz[:k]), total.value


def ds_partition_range(total, world, rank, align):
    start, count = ctypes.c_int64(), ctypes.c_int64()
    _ok(lib.ds_partition_range(int(total), int(world), int(rank), int(align), ctypes.byref(start),
                               ctypes.byref(count)), "ds_partition_range")
    return start.value, count.value
