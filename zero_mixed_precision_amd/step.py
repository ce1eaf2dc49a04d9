"""ShardStep: one rank's ZeRO optimizer step over its flat partition.

Owns the partition's device arrays (torch tensors used as memory only) and the
device-resident loss-scaler state, and issues the per-step call sequence of
the C ABI on one HIP stream ("DeepSpeed complete guide" section 5.1: backward
scales and accumulates, step() updates):

    K > 1:  ds_accumulate per bucket for micro-batches 1..K (the last one also
            checks for inf/NaN), then the Adam step on the fp32 buffer;
            micro-batches handed over together (a list to accumulate(), or
            full_step()) are folded in one pass each (ds_accumulate_multi, up
            to 8 at a time, the same result with less memory traffic)
    K = 1:  ds_check_overflow on the fp16 gradient, then the Adam step on it

The Adam step covers the whole partition in one ds_adam_step_fused call,
whose kernel also advances the loss scaler (ds_update_loss_scale's work).
With ``double_buffer`` (no clipping) the shard keeps two copies of master, m,
v and the 16-bit copy, and the overflow check is fused into the Adam pass,
which writes the other copy; the device makes that copy current only if the
step applied.  K = 1: one ds_adam_step_double_buffered call (28 bytes per
element instead of 30).  K > 1: the micro-batches before the last call to
accumulate() are summed as above, and step() folds the last call's
gradients into the Adam pass (ds_accumulate_adam_double_buffered, which uses
the sum without storing it), then ds_update_loss_scale_double_buffered ends
the step (a fold of all 8 of 8 micro-batches: 42 bytes per element instead of
50).  ``current()`` returns the copy holding the state.

With gradient clipping configured the check passes are the _sumsq variants
(ds_accumulate_sumsq / ds_check_overflow_sumsq), which also gather the
gradient's sum of squares for the Adam step's global-norm clipping.  With a
scheduler block the Adam step reads the learning rate of the schedule on the
device.

No call synchronises the host; ``scaler()`` reads the state back (one copy).
``save_checkpoint``/``load_checkpoint`` write and restore the shard between
steps (safetensors files, see checkpoint.py).
``graph(grads)`` records the whole sequence for fixed gradient buffers into a
HIP graph, so a step costs one graph launch; it contains kernels only (no
memset or copy nodes).
"""
from __future__ import annotations

from . import _lib
from .config import ZeroMPConfig


def buckets_or_all(buckets, n):
    """(start, size) pairs of the accumulation buckets inside a partition of n
    elements (objects with .start/.size, or pairs), or the whole partition.

    The buckets must tile [0, n): sorted, the first at 0, each starting where
    the previous one ends, the sizes adding up to n, and every start a multiple
    of 8 elements (so that every array pointer the calls derive stays 16-byte
    aligned).  Anything else raises ValueError: the calls receive raw
    addresses, so a bucket past the end would be written out of bounds, and a
    gap would leave part of the accumulation buffer stale and unchecked."""
    if not buckets:
        return [(0, int(n))]
    pairs = [(int(b.start), int(b.size)) if hasattr(b, "start") else (int(b[0]), int(b[1])) for b in buckets]
    end = 0
    for start, size in pairs:
        if start != end:
            raise ValueError(f"bucket at {start} does not start where the previous one ends ({end}): "
                             "buckets must tile [0, n) in order")
        if size < 0:
            raise ValueError(f"bucket at {start} has a negative size")
        if start % 8:
            raise ValueError(f"bucket at {start} does not start on a multiple of 8 elements")
        end = start + size
    if end != n:
        raise ValueError(f"buckets cover [0, {end}), the partition has {n} elements")
    return pairs


def check_grad_dtype(dtype, bf16: bool, torch) -> None:
    """The fp16 and bf16 formats are exclusive ("DeepSpeed complete guide"
    section 4.2): a float16 gradient for a bf16 shard, or a bfloat16 one for an
    fp16 shard, would be read bit for bit in the other format, so it is
    refused.  int16 (and uint16) tensors pass as raw bit containers."""
    raw = (torch.int16,) + ((torch.uint16,) if hasattr(torch, "uint16") else ())
    if dtype in raw:
        return
    want = torch.bfloat16 if bf16 else torch.float16
    if dtype != want:
        raise ValueError(f"gradient of dtype {dtype} for a {'bf16' if bf16 else 'fp16'} shard "
                         f"(expected {want}, or int16 raw bits)")


class ShardStep:
    def __init__(self, n: int, cfg: ZeroMPConfig, device="cuda", buckets=None, stream=None, double_buffer=False):
        import torch

        self.double_buffer = bool(double_buffer)
        if self.double_buffer and float(cfg.gradient_clipping) > 0:
            raise ValueError("double_buffer takes no gradient clipping (clipping needs the whole gradient's norm "
                             "before the update)")

        # accumulation granularity: the reduce buckets inside this partition
        self.buckets = buckets_or_all(buckets, int(n))
        self.torch, self.n, self.cfg = torch, int(n), cfg
        self.K = int(cfg.gradient_accumulation_steps)
        self.stream = stream
        # 16-bit format of the gradients and of the parameter copy
        self.gdt = self.pdt = _lib.DS_BF16 if cfg.bf16 else _lib.DS_FP16
        f32 = dict(dtype=torch.float32, device=device)
        self.master = torch.empty(self.n, **f32)
        self.m = torch.zeros(self.n, **f32)
        self.v = torch.zeros(self.n, **f32)
        self.p16 = torch.empty(self.n, dtype=torch.bfloat16 if cfg.bf16 else torch.float16, device=device)
        self.acc = torch.empty(self.n, **f32) if self.K > 1 else None
        # double_buffer: a second copy of master, m, v and the 16-bit copy; the
        # state names the current one (initially copy 0, the attributes above)
        self._copies = None
        if self.double_buffer:
            self._copies = ((self.master, self.m, self.v, self.p16),
                            (torch.empty(self.n, **f32), torch.empty(self.n, **f32), torch.empty(self.n, **f32),
                             torch.empty(self.n, dtype=self.p16.dtype, device=device)))
        self.state = torch.zeros(_lib.ds_scaler_size(), dtype=torch.uint8, device=device)
        # learning-rate schedule (None: the constant cfg.lr), read on the device
        # at the applied-step count, so a skipped step does not advance it
        self.sched = cfg.lr_schedule()
        self.clip = float(cfg.gradient_clipping)
        self.ws = None
        if self.clip > 0:
            # chunk sums of the gradient's sum of squares (scratch, no initial contents)
            nbytes = _lib.ds_sumsq_workspace_bytes(self.n)
            self.ws = torch.zeros((nbytes + 7) // 8, dtype=torch.float64, device=device)
        self._ws_bytes = self.ws.numel() * 8 if self.ws is not None else 0
        self._micro = 0
        # double_buffer with K > 1: the step's last micro-batch gradients, folded
        # into the Adam pass by step(), and whether they are all K of them
        self._pending, self._pending_all = None, False
        _lib.ds_state_init(self.state, cfg.init_scale, cfg.min_loss_scale, cfg.loss_scale_window,
                           cfg.hysteresis, int(cfg.consecutive_hysteresis), int(cfg.dynamic),
                           self.stream)

    def _check_grad(self, g16) -> None:
        if g16 is None or g16.numel() != self.n or g16.element_size() != 2:
            raise ValueError(f"expected a 16-bit gradient of {self.n} elements")
        if g16.device != self.master.device or not g16.is_contiguous():
            raise ValueError(f"the gradient must be a contiguous tensor on {self.master.device}")
        check_grad_dtype(g16.dtype, self.cfg.bf16, self.torch)

    def accumulate(self, g16) -> None:
        """Add one fp16 micro-batch gradient (K > 1), or a list of up to 8 of them
        in micro-batch order, folded into the buffer in one pass (the same result
        as one call each, with less memory traffic); the call that completes the
        K micro-batches also checks the sum.  With double_buffer that call only
        records its gradients: step() folds them into the Adam pass, so they must
        stay unchanged until then."""
        if self.K == 1:
            raise RuntimeError("accumulate() is for gradient_accumulation_steps > 1; pass the gradient to step()")
        if isinstance(g16, (list, tuple)):
            self._fold(list(g16))
            return
        if self._micro >= self.K:
            raise RuntimeError(f"accumulate() called more than {self.K} times before step()")
        self._check_grad(g16)
        k = self._micro
        last = k == self.K - 1
        if last and self.double_buffer:
            self._pending, self._pending_all = [g16], False
            self._micro = k + 1
            return
        st, acc, g0 = self.state.data_ptr(), self.acc.data_ptr(), g16.data_ptr()
        for start, size in self.buckets:
            a, g = acc + 4 * start, g0 + 2 * start
            if last and self.ws is not None:
                _lib.ds_accumulate_sumsq(a, g, self.gdt, size, k == 0, st, self.ws.data_ptr(), self._ws_bytes,
                                         stream=self.stream)
            else:
                _lib.ds_accumulate(a, g, self.gdt, size, overwrite=(k == 0), st_or_null=st if last else None,
                                   stream=self.stream)
        self._micro = k + 1

    def _fold(self, grads) -> None:
        count = len(grads)
        if not 1 <= count <= 8:
            raise ValueError("a fold takes 1 to 8 micro-batch gradients")
        if self._micro + count > self.K:
            raise RuntimeError(f"{self._micro} + {count} micro-batches exceed gradient_accumulation_steps={self.K}")
        for g in grads:
            self._check_grad(g)
        first, last = self._micro == 0, self._micro + count == self.K
        if last and self.double_buffer:
            self._pending, self._pending_all = list(grads), first
            self._micro += count
            return
        st, acc = self.state.data_ptr(), self.acc.data_ptr()
        base = [g.data_ptr() for g in grads]
        for start, size in self.buckets:
            ws = self.ws.data_ptr() if (last and self.ws is not None) else None
            _lib.ds_accumulate_multi(acc + 4 * start, [b + 2 * start for b in base], self.gdt, size, first,
                                     st if last else None, ws, self._ws_bytes, stream=self.stream)
        self._micro += count

    def step(self, g16=None) -> None:
        """Finish the step: check (K = 1), gated Adam, scaler update."""
        c = self.cfg
        st = self.state.data_ptr()
        if self.double_buffer and self.K > 1:
            # the last micro-batches folded into the Adam pass, which checks their
            # sum and writes the other copy; then the scaler update swaps copies
            if self._micro != self.K or self._pending is None:
                raise RuntimeError(f"accumulate() must be called {self.K} times before step() "
                                   f"(called {self._micro} times)")
            a, b = self._copies
            _lib.ds_accumulate_adam_double_buffered(
                st, [a[0].data_ptr(), b[0].data_ptr()], [a[1].data_ptr(), b[1].data_ptr()],
                [a[2].data_ptr(), b[2].data_ptr()], [a[3].data_ptr(), b[3].data_ptr()], self.pdt,
                None if self._pending_all else self.acc.data_ptr(), [g.data_ptr() for g in self._pending],
                self.gdt, self.n, c.lr, self.sched, c.betas[0], c.betas[1], c.eps, c.weight_decay, self.K,
                self.stream)
            _lib.ds_update_loss_scale_double_buffered(st, self.stream)
            self._pending, self._pending_all, self._micro = None, False, 0
            return
        if self.double_buffer:
            # the check fused into the Adam pass, which writes the other copy
            self._check_grad(g16)
            a, b = self._copies
            _lib.ds_adam_step_double_buffered(st, [a[0].data_ptr(), b[0].data_ptr()],
                                              [a[1].data_ptr(), b[1].data_ptr()],
                                              [a[2].data_ptr(), b[2].data_ptr()],
                                              [a[3].data_ptr(), b[3].data_ptr()], self.pdt, g16.data_ptr(),
                                              self.gdt, self.n, c.lr, self.sched, c.betas[0], c.betas[1], c.eps,
                                              c.weight_decay, 1, self.stream)
            return
        if self.K == 1:
            self._check_grad(g16)
            grad, dt = g16.data_ptr(), self.gdt
            if self.ws is not None:
                _lib.ds_check_overflow_sumsq(st, grad, dt, self.n, self.ws.data_ptr(), self._ws_bytes,
                                             stream=self.stream)
            else:
                _lib.ds_check_overflow(st, grad, dt, self.n, self.stream)
        else:
            if self._micro != self.K:
                raise RuntimeError(f"accumulate() must be called {self.K} times before step() "
                                   f"(called {self._micro} times)")
            grad, dt = self.acc.data_ptr(), _lib.DS_FP32
        # the whole partition in one call: the Adam kernel also advances the scaler
        # (raw addresses: the arrays are this object's own, sized and placed at construction,
        # and the gradient was checked above, so the binding's per-tensor checks are skipped)
        _lib.ds_adam_step_fused(st, self.master.data_ptr(), self.m.data_ptr(), self.v.data_ptr(),
                                self.p16.data_ptr(), self.pdt, grad, dt, self.n,
                                c.lr, self.sched, c.betas[0], c.betas[1], c.eps, c.weight_decay,
                                c.gradient_clipping, self.K, self.stream)
        self._micro = 0

    def full_step(self, grads) -> None:
        """One whole step from K fp16 micro-batch gradients (a tensor when K = 1)."""
        if self.K == 1:
            self.step(grads[0] if isinstance(grads, (list, tuple)) else grads)
            return
        if len(grads) != self.K:
            raise ValueError(f"expected {self.K} micro-batch gradients, got {len(grads)}")
        for i in range(0, self.K, 8):           # all K are at hand: fold up to 8 per pass
            self.accumulate(list(grads[i:i + 8]))
        self.step()

    def graph(self, grads):
        """Record ``full_step(grads)`` into a HIP graph (torch.cuda.CUDAGraph).

        The gradient buffers are baked in by address: write the next step's
        gradients into the same tensors, then ``replay()``.  Replays use the
        hyperparameters as recorded; with a learning-rate schedule each replay
        still takes the schedule's lr at the device's applied-step count.
        """
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        saved, self.stream = self.stream, None      # launch on the capturing (current) stream
        try:
            with torch.cuda.graph(g, stream=side):
                self.full_step(grads)
        finally:
            self.stream = saved
        torch.cuda.current_stream().wait_stream(side)
        return g

    def scaler(self) -> _lib.DsScaler:
        return _lib.ds_state_read(self.state, self.stream)

    def current(self):
        """(master, m, v, p16) holding the state: the attributes of the same names,
        or with double_buffer the copy the state names (read back: one copy)."""
        if not self.double_buffer:
            return self.master, self.m, self.v, self.p16
        return self._copies[self.scaler().current & 1]

    def save_checkpoint(self, save_dir, tag=None, client_state=None, rank=0) -> str:
        """Save this shard between steps ("DeepSpeed complete guide" section 5.2); see checkpoint.py."""
        from .checkpoint import save_checkpoint
        return save_checkpoint(self, save_dir, tag, client_state, rank)

    def load_checkpoint(self, load_dir, tag=None, rank=0):
        """Restore this shard; returns (path, client_state)."""
        from .checkpoint import load_checkpoint
        return load_checkpoint(self, load_dir, tag, rank)
