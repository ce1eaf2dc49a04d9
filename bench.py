"""Benchmark of the ZeRO mixed-precision optimizer step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload zero1_70b] [--step-form auto]

One step = the whole per-rank hot path over one synthetic batch: the inf/NaN
check of the gradient (K > 1: fused into the bucketed fp16 -> fp32
accumulation of the last micro-batch), the gated Adam update with the fp16
copy, and the loss-scale update.  Without clipping the default
(--step-form auto) is the double-buffered form: the check fused into the
Adam pass, which reads the copy of master/m/v/p16 that holds the state and
writes the other one (K = 1: 28 B per element in one launch; K > 1: the last
micro-batch or fold also summed inside that pass, the sum never stored).  It
needs 30 bytes of device memory per element instead of 16, so it is used
where the second copy and the gradient buffers fit, and (K = 1) where the
gradient is larger than the 256 MB Infinity Cache (a smaller one is still
cached when the in-place form reads it again, which makes that form as fast)
or where the whole state fits in that cache (the step is then launch-bound,
and the double-buffered form is one launch instead of two).
The in-place form (the check or the accumulation with its fused check, then
the Adam pass that rewrites the one copy) is then timed after it on the copy
that holds the state and reported as ``in_place_form``; --step-form in_place
makes it the timed form.  Inputs are resident in HBM before the timed region;
gradients are drawn on the device (distinct buffers, reused cyclically when
they do not all fit).

The default workload is zero1_70b: one rank's ZeRO-1 share of a 70B model at
N = 8, 8.75e9 elements (140 GB of state, 262.5 GB with the second copy), the
largest single-GPU workload.

Prints one JSON line.  ``value`` is parameters updated per second (Gparams/s)
over the timed steps; ``roofline`` is the Adam kernel's algorithmic HBM
bandwidth (28 B/element with an fp16 gradient, 30 with the fp32 buffer) over
its average duration, timed with HIP events on the launch stream, against
the 8 TB/s HBM3E peak; ``traffic`` comes from the committed rocprofv3 counter
summary when it was taken on the current kernel source; the median and minimum
launch times sit beside it, ``roofline.step`` gives the whole step's
algorithmic bytes per element over the wall time per step, and
``roofline.references`` three data-movement references timed on the same
arrays after the timed region: the step's 14 B read + 14 B written per
element with no arithmetic (in the step's 256 x 4 tiling, and in 64-lane
blocks of one quad per lane, the copy's shape), a plain copy with one 16-byte
vector per lane, and the runtime's device-to-device copy
(``torch.Tensor.copy_``, which is hipMemcpyAsync).  ``step_ms_*`` and ``pre_adam_ms_*`` (the check, or the
accumulation with its fused check; nothing in the double-buffered form) come
from an untimed pass with events around each part.  ``graph_replay`` times the
same steps replayed from HIP graphs (one per position in the cycle of gradient
buffers).  ``cpu_baseline`` times the CPU oracle on a bounded slice of the
same workload on the host cores the process may use.

    python bench.py --mode copy    # plain-copy and step-shaped data-movement references
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
INFINITY_CACHE_BYTES = 256 << 20   # MI355X's last-level (MALL) cache
METRIC = "Gparams/s per Adam step + achieved HBM GB/s (% of MI355X peak)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "adam_traffic.json")
KERNEL_SRC = os.path.join(ROOT, "zero_mixed_precision_amd", "csrc", "dszero.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def load_traffic(workload: str, half: str, kernel: str, fold: int = 1):
    """Per-launch HBM bytes of the Adam kernel from the committed counter summary,
    or None if it is missing, was taken on another kernel source, or on another
    workload, 16-bit format, fold or kernel (another instance of the pass)."""
    try:
        data = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    for rec in data.get("records", [data]):
        if (rec.get("kernel_source_sha256_16") == kernel_source_hash() and rec.get("workload") == workload
                and rec.get("half") == half and rec.get("fold", 1) == fold
                and re.search(r"\b%s<" % kernel, rec.get("kernel", ""))):
            return rec.get("traffic_bytes_per_launch")
    return None


HEADROOM_BYTES = 4 << 30   # device memory left free beside the run's arrays


def grad_ring(n: int, K: int, fold: int, steps: int, warmup: int, max_buffers: int) -> int:
    """Gradient buffers wanted: a ring of distinct draws (a real step rewrites one
    contiguous gradient buffer) of at least 2 GiB, far beyond the 256 MB Infinity
    Cache, never fewer than one fold holds, and no more than the run draws or the
    caller allows."""
    return min(max(2, -(-(2 << 30) // (2 * n)), fold), (steps + warmup) * K, max_buffers)


def double_wanted(step_form: str, clip: float, K: int, n: int) -> bool:
    """Whether to try the double-buffered form: never with clipping (it needs the
    whole gradient's norm before the update); "double" asks for it; "auto" takes
    it with K > 1, and with K = 1 where the gradient is larger than the Infinity
    Cache (a smaller one is still cached when the in-place form's Adam pass reads
    it again after the check, which makes that form as fast) or where the whole
    state fits in it (the step is then launch-bound, and the double-buffered
    form is one launch instead of two)."""
    if clip > 0:
        return False
    launch_bound = 16 * n <= INFINITY_CACHE_BYTES
    return step_form == "double" or (step_form == "auto" and (K > 1 or 2 * n > INFINITY_CACHE_BYTES or launch_bound))


def needs_running_sum(K: int, fold: int, double: bool) -> bool:
    """The fp32 running sum is needed with K > 1, except when the double-buffered
    form folds all K micro-batches into its Adam pass."""
    return K > 1 and not (double and fold >= K)


def room_beside_second_copy(n: int, K: int, fold: int, ring: int) -> int:
    """Bytes that must stay free once the second copy is allocated: the gradient
    buffers, the running sum if the form needs one, and the headroom."""
    return ring * 2 * n + (4 * n if needs_running_sum(K, fold, True) else 0) + HEADROOM_BYTES


def buffers_that_fit(free: int, n: int, ring: int) -> int:
    return max(1, min(int((free - HEADROOM_BYTES) // (2 * n)), ring))


def fold_bytes(sizes) -> int:
    """Algorithmic bytes per element of the accumulation passes over groups of
    micro-batches of these sizes: 2f + 4 for the first (it overwrites the
    running sum), 2f + 8 for each later one (it reads and writes it)."""
    return sum(2 * f + (4 if i == 0 else 8) for i, f in enumerate(sizes))


# ----------------------------------------------------------------------------
# GPU leg
# ----------------------------------------------------------------------------

def gpu_run(args):
    import numpy as np
    import torch

    import synth
    from synth.workloads import BETA1, BETA2, EPS, LR, MASTER_SIGMA, WD, WORKLOADS, ragged_numels
    from zero_mixed_precision_amd import _lib, FlatLayout

    w = WORKLOADS[args.workload]
    n, K = w.psi, w.K
    # bf16 mode: bf16 gradients and parameter copy, no loss scaling (static scale 1)
    gdt16 = _lib.DS_BF16 if args.bf16 else _lib.DS_FP16
    gspec = synth.GradSpec(w.sigma, 1.0, w.heavy_tail, fmt="bf16") if args.bf16 else w.grad_spec
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    log(f"device: {props.name} CUs={props.multi_processor_count} mem={props.total_memory / 2**30:.0f} GiB")
    stream = torch.cuda.current_stream()
    tabs = synth.DeviceTables(torch, dev)

    master = torch.empty(n, dtype=torch.float32, device=dev)
    synth.device_fill_master32(torch, tabs, master, w.master_key(), MASTER_SIGMA)
    m = torch.zeros(n, dtype=torch.float32, device=dev)
    v = torch.zeros(n, dtype=torch.float32, device=dev)
    p16 = torch.empty(n, dtype=torch.int16, device=dev)
    synth.device_fill_grad16(torch, tabs, p16, w.p16_key(), synth.GradSpec(0.02, 1.0))
    st = torch.zeros(_lib.ds_scaler_size(), dtype=torch.uint8, device=dev)
    if args.bf16:
        _lib.ds_state_init(st, 1.0, 1.0, w.window, w.hysteresis, 0, 0)
    else:
        _lib.ds_state_init(st, w.init_scale, w.min_scale, w.window, w.hysteresis, 0, 1)
    if w.ragged:
        buckets = [(b.start, b.size) for b in FlatLayout(ragged_numels()).buckets]
    else:
        buckets = [(0, n)]
    if not 1 <= args.fold <= 8:
        sys.exit("bench.py: --fold takes 1..8")
    fold = min(args.fold, K)
    ring = grad_ring(n, K, fold, args.steps, args.warmup, args.max_grad_buffers)

    # double-buffered step (no clipping): a second copy of master, m, v and the
    # 16-bit copy; the overflow check is fused into the Adam pass, and with K > 1
    # so is the accumulation of the last micro-batch (or of the last fold); it is
    # used if the second copy leaves room for the gradient buffers and the
    # running sum the step needs
    double = False
    copy1 = None
    if args.step_form == "double" and args.clip > 0:
        log("bench.py: the double-buffered step takes no clipping; using the in-place form")
    if double_wanted(args.step_form, args.clip, K, n):
        try:
            copy1 = [torch.empty(n, dtype=torch.float32, device=dev) for _ in range(3)] + \
                    [torch.empty(n, dtype=torch.int16, device=dev)]
            if torch.cuda.mem_get_info(dev)[0] < room_beside_second_copy(n, K, fold, ring):
                raise torch.cuda.OutOfMemoryError("no room for the gradient buffers beside two copies")
            double = True
        except torch.cuda.OutOfMemoryError as e:
            copy1 = None
            torch.cuda.empty_cache()
            log(f"bench.py: two copies of the state do not fit ({str(e).splitlines()[0][:120]}); "
                "using the in-place form")
    acc = torch.empty(n, dtype=torch.float32, device=dev) if needs_running_sum(K, fold, double) else None

    nbuf = buffers_that_fit(torch.cuda.mem_get_info(dev)[0], n, ring)
    if fold > nbuf:
        sys.exit(f"bench.py: --fold {fold} needs {fold} gradient buffers at once; {nbuf} fit")
    grads = []
    for b in range(nbuf):
        g = torch.empty(n, dtype=torch.int16, device=dev)
        s, k = divmod(b, K)
        synth.device_fill_grad16(torch, tabs, g, w.grad_key(s + 1, k), gspec)
        grads.append(g)
    torch.cuda.synchronize()
    log(f"workload {w.name}: psi={n} K={K} grad buffers={nbuf} (of {(args.steps + args.warmup) * K} micro-batches) "
        f"step form={'double-buffered' if double else 'in place'}")

    hp = (LR, BETA1, BETA2, EPS, WD, args.clip)
    ws = None
    if args.clip > 0:   # global-norm clipping: the check passes also gather the sum of squares
        ws = torch.zeros((_lib.ds_sumsq_workspace_bytes(n) + 7) // 8, dtype=torch.float64, device=dev)
    ev = []
    # raw device addresses for the calls in the step loop: every array is fixed for
    # the run (checked once here), so the binding's per-call tensor checks stay out
    # of the host's launch loop
    for t, nb in ((master, 4 * n), (m, 4 * n), (v, 4 * n), (p16, 2 * n), (st, _lib.ds_scaler_size())):
        if not (t.is_cuda and t.is_contiguous() and t.numel() * t.element_size() >= nb):
            raise RuntimeError("bench.py: a state array is not a contiguous device tensor of the expected size")
    st_p, master_p, m_p, v_p, p16_p = (t.data_ptr() for t in (st, master, m, v, p16))
    # the arrays the in-place form updates (the current copy when there are two)
    ip = [master_p, m_p, v_p, p16_p]
    if double:
        V2 = ctypes.c_void_p * 2
        copies = (ip[:], [t.data_ptr() for t in copy1])
        db_arrays = tuple(V2(copies[0][k], copies[1][k]) for k in range(4))
        db_step = _lib.lib.ds_adam_step_double_buffered
        db_fold = _lib.lib.ds_accumulate_adam_double_buffered
        db_update = _lib.lib.ds_update_loss_scale_double_buffered
    acc_p = acc.data_ptr() if acc is not None else None
    ws_p, ws_bytes = (ws.data_ptr(), ws.numel() * 8) if ws is not None else (None, 0)
    grad_p = [g.data_ptr() for g in grads]

    step_ev, pre_ev = [], []   # whole steps; their check (K = 1) or accumulation + check (K > 1) part

    def one_step(i, timed, q=stream, whole=False, form=None, evs=None):
        dbl = double if form is None else form == "double"
        if whole:
            s0 = torch.cuda.Event(enable_timing=True)
            s0.record(q)
        base = i * K
        if dbl and K == 1:
            g = grad_p[base % nbuf]
            gptr, dt = g, gdt16
        elif dbl:   # every fold but the last into the running sum; the last goes into the Adam pass
            groups = [list(range(g0, min(g0 + fold, K))) for g0 in range(0, K, fold)]
            for gi, grp in enumerate(groups[:-1]):
                for start, size in buckets:
                    gp = [grad_p[(base + k) % nbuf] + 2 * start for k in grp]
                    if len(gp) == 1:
                        _lib.ds_accumulate(acc_p + 4 * start, gp[0], gdt16, size, gi == 0, None, q)
                    else:
                        _lib.ds_accumulate_multi(acc_p + 4 * start, gp, gdt16, size, gi == 0, None, None, 0,
                                                 stream=q)
            last = (ctypes.c_void_p * len(groups[-1]))(*[grad_p[(base + k) % nbuf] for k in groups[-1]])
            last_acc = acc_p if len(groups) > 1 else None
        elif K == 1:
            g = grad_p[base % nbuf]
            if ws is None:
                _lib.ds_check_overflow(st_p, g, gdt16, n, q)
            else:
                _lib.ds_check_overflow_sumsq(st_p, g, gdt16, n, ws_p, ws_bytes, stream=q)
            gptr, dt = g, gdt16
        elif fold == 1:
            for k in range(K):
                g = grad_p[(base + k) % nbuf]
                for start, size in buckets:
                    a, gp = acc_p + 4 * start, g + 2 * start
                    if k == K - 1 and ws is not None:
                        _lib.ds_accumulate_sumsq(a, gp, gdt16, size, k == 0, st_p, ws_p, ws_bytes, stream=q)
                    else:
                        _lib.ds_accumulate(a, gp, gdt16, size, k == 0, st_p if k == K - 1 else None, q)
            gptr, dt = acc_p, _lib.DS_FP32
        else:   # groups of `fold` micro-batches, each folded into the buffer in one pass
            for g0 in range(0, K, fold):
                grp = [grad_p[(base + k) % nbuf] for k in range(g0, min(g0 + fold, K))]
                final = g0 + fold >= K
                for start, size in buckets:
                    _lib.ds_accumulate_multi(acc_p + 4 * start, [g + 2 * start for g in grp], gdt16, size, g0 == 0,
                                             st_p if final else None, ws_p if (final and ws is not None) else None,
                                             ws_bytes, stream=q)
            gptr, dt = acc_p, _lib.DS_FP32
        if whole:
            c1 = torch.cuda.Event(enable_timing=True)
            c1.record(q)
        if timed:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(q)
        # the Adam kernel also advances the loss scaler (one launch for both)
        if dbl and K == 1:   # and performs the overflow check, writing the other copy
            rc = db_step(st_p, *db_arrays, gdt16, gptr, dt, n, hp[0], None, *hp[1:5], K, q.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"ds_adam_step_double_buffered: {_lib.ds_status_string(rc)}")
        elif dbl:            # the last fold, the check and Adam into the other copy
            rc = db_fold(st_p, *db_arrays, gdt16, last_acc, last, len(last), gdt16, n, hp[0], None, *hp[1:5], K,
                         q.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"ds_accumulate_adam_double_buffered: {_lib.ds_status_string(rc)}")
        else:
            _lib.ds_adam_step_fused(st_p, *ip, gdt16, gptr, dt, n, hp[0], None, *hp[1:], K, q)
        if timed:
            b.record(q)
            (ev if evs is None else evs).append((a, b))
        if dbl and K > 1:    # then the one-work-item scaler update, which switches copies if the step applied
            rc = db_update(st_p, q.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"ds_update_loss_scale_double_buffered: {_lib.ds_status_string(rc)}")
        if whole:
            s1 = torch.cuda.Event(enable_timing=True)
            s1.record(q)
            step_ev.append((s0, s1))
            pre_ev.append((s0, c1))

    for i in range(args.warmup):
        one_step(i, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.warmup, args.warmup + args.steps):
        one_step(i, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    sc = _lib.ds_state_read(st, stream)

    # per-step device time (median, min) in a pass of its own, so that the
    # extra events stay out of the timed region; with --step-log, one JSON line
    # per step of that pass (reading the scaler synchronises every step)
    log_f = open(args.step_log, "w") if args.step_log else None
    for i in range(args.steps):
        if log_f is not None:
            used = _lib.ds_state_read(st, stream).scale
        one_step(i, False, whole=True)
        if log_f is not None:
            after = _lib.ds_state_read(st, stream)
            a, b = step_ev[-1]
            log_f.write(json.dumps({"step": int(after.iter), "scale": used, "overflow": int(after.last_overflow),
                                    "t": int(after.step), "growth_count": int(after.growth_count),
                                    "skipped": int(after.skipped), "step_ms": round(a.elapsed_time(b), 4)}) + "\n")
    torch.cuda.synchronize()
    if log_f is not None:
        log_f.close()

    # the same steps replayed from HIP graphs: one graph per position in the
    # cycle of gradient buffers, each captured once (kernels only), replayed in
    # order, and reported beside the eager rate (on short steps a replay costs
    # more than the launches it replaces; on long ones it changes nothing)
    cycle = nbuf // math.gcd(nbuf, K)
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    graphs = []
    for c in range(cycle):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=side):
            one_step(c, False, side)
        graphs.append(gr)
    stream.wait_stream(side)
    for i in range(args.warmup):
        graphs[i % cycle].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        graphs[i % cycle].replay()
    torch.cuda.synchronize()
    gwall = time.perf_counter() - t0
    del graphs

    # with two copies, the in-place form (check, then the in-place Adam pass) on
    # the copy that holds the state, timed the same way after the rest
    in_place = None
    groups_sizes = [min(fold, K - g0) for g0 in range(0, K, fold)]
    ip_step_bytes = 30 if K == 1 else fold_bytes(groups_sizes) + 30
    if double:
        # keep the copy that holds the state; the in-place form updates it (and,
        # with K > 1, needs the running sum, which may take the other copy's room)
        cur = _lib.ds_state_read(st, stream).current
        keep = (master, m, v, p16) if cur == 0 else tuple(copy1)
        master, m, v, p16 = keep
        copy1 = keep = None
        torch.cuda.empty_cache()
        if K > 1 and acc is None:
            acc = torch.empty(n, dtype=torch.float32, device=dev)
            acc_p = acc.data_ptr()
        ip[:] = [t.data_ptr() for t in (master, m, v, p16)]
        ip_ev = []
        for i in range(args.warmup):
            one_step(i, False, form="in_place")
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.warmup, args.warmup + args.steps):
            one_step(i, True, form="in_place", evs=ip_ev)
        torch.cuda.synchronize()
        ip_wall = time.perf_counter() - t0
        ip_adam_s = sum(a.elapsed_time(b) for a, b in ip_ev) / len(ip_ev) / 1e3
        ip_bpe = 28 if K == 1 else 30
        in_place = {
            "step_form": ("check, then the in-place Adam pass" if K == 1 else
                          "accumulation with the fused check, then the in-place Adam pass")
                         + " (one copy of the state)",
            "value": round(n * args.steps / ip_wall / 1e9, 3),
            "ms_per_step": round(ip_wall / args.steps * 1e3, 4),
            "kernel": "adam_kernel",
            "avg_launch_ms": round(ip_adam_s * 1e3, 4),
            "achieved": round(ip_bpe * n / ip_adam_s / 1e9, 1),
            "frac": round(ip_bpe * n / ip_adam_s / 1e9 / PEAK_HBM_GBS, 4),
            "traffic": load_traffic(w.name, "bf16" if args.bf16 else "fp16", "adam_kernel", fold),
            "step": {"bytes_per_elem": ip_step_bytes,
                     "achieved": round(ip_step_bytes * n * args.steps / ip_wall / 1e9, 1),
                     "frac": round(ip_step_bytes * n * args.steps / ip_wall / 1e9 / PEAK_HBM_GBS, 4)},
        }

    adam_ms = [a.elapsed_time(b) for a, b in ev]
    adam_avg_s = sum(adam_ms) / len(adam_ms) / 1e3
    adam_sorted = sorted(adam_ms)
    step_sorted = sorted(a.elapsed_time(b) for a, b in step_ev)
    pre_sorted = sorted(a.elapsed_time(b) for a, b in pre_ev)

    # data-movement references, after the timed region, on the same arrays
    # (they scramble them; the run is over): the step's 14 B read + 14 B
    # written per element with no arithmetic; a plain copy of master into m
    # with one 16-byte vector per lane; the same copy by the runtime
    # (torch's copy_ of a contiguous tensor on one device is hipMemcpyAsync)
    def timed(fn, reps):
        for _ in range(2):
            fn()
        evs = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            evs.append((a, b))
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in evs) / len(evs) / 1e3

    nm = n - n % 4
    mix_args = (grads[0][:nm], master[:nm], m[:nm], v[:nm], p16[:nm])
    mix_s = timed(lambda: synth.device_stream_mix(torch, *mix_args, stream=stream), 8)
    mix_gbs = 28 * nm / mix_s / 1e9
    mix64_s = timed(lambda: synth.device_stream_mix(torch, *mix_args, stream=stream, small_tiles=True), 8)
    mix64_gbs = 28 * nm / mix64_s / 1e9
    copy_s = timed(lambda: synth.device_copy(torch, m[:nm], master[:nm], stream=stream), 8)
    memcpy_s = timed(lambda: m[:nm].copy_(master[:nm]), 8)
    copy_gbs, memcpy_gbs = 8 * nm / copy_s / 1e9, 8 * nm / memcpy_s / 1e9
    if double and K > 1:   # the last fold with the Adam pass: its gradients, the running sum if any, the state
        last = groups_sizes[-1]
        bytes_per_elem = 2 * last + (30 if len(groups_sizes) > 1 else 26)
        step_bytes = fold_bytes(groups_sizes[:-1]) + bytes_per_elem
        kernel = "fold_adam_db_kernel"
    elif double:
        bytes_per_elem = step_bytes = 28
        kernel = "adam_db_kernel"
    else:
        bytes_per_elem = 28 if K == 1 else 30
        step_bytes = ip_step_bytes
        kernel = "adam_kernel"
    achieved = bytes_per_elem * n / adam_avg_s / 1e9
    traffic = load_traffic(w.name, "bf16" if args.bf16 else "fp16", kernel, fold)
    out = {
        "metric": METRIC,
        "value": round(n * args.steps / wall / 1e9, 3),
        "unit": "Gparams/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "step_ms_median": round(step_sorted[len(step_sorted) // 2], 4),
        "step_ms_min": round(step_sorted[0], 4),
        "pre_adam_ms_median": round(pre_sorted[len(pre_sorted) // 2], 4),
        "pre_adam_ms_min": round(pre_sorted[0], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "psi": n,
            "micro_batches": K,
            "fold": fold,
            "grad": ("bf16 N(0,%g)" % w.sigma if args.bf16 else "fp16 N(0,%g) x %g" % (w.sigma, w.mult))
                    + (" heavy tail" if w.heavy_tail else ""),
            "state": "fp32 master/m/v, %s params" % ("bf16" if args.bf16 else "fp16"),
            "adam": {"lr": LR, "betas": [BETA1, BETA2], "eps": EPS, "weight_decay": WD},
            "gradient_clipping": args.clip,
            "half": "bf16" if args.bf16 else "fp16",
            "step_form": ("double-buffered: the overflow check fused into the Adam pass, which writes the "
                          "second copy of the state" if double and K == 1 else
                          "double-buffered: the earlier micro-batches accumulated, the last fold summed, checked "
                          "and fed to the Adam pass, which writes the second copy of the state" if double else
                          "check (or accumulation with the fused check), then the in-place Adam pass"),
            "parallelism": "one GPU's ZeRO partition",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": kernel,
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "alg_bytes_per_launch": bytes_per_elem * n,
            "avg_launch_ms": round(adam_avg_s * 1e3, 4),
            "median_launch_ms": round(adam_sorted[len(adam_sorted) // 2], 4),
            "min_launch_ms": round(adam_sorted[0], 4),
            "step": {"bytes_per_elem": step_bytes,
                     "achieved": round(step_bytes * n * args.steps / wall / 1e9, 1),
                     "frac": round(step_bytes * n * args.steps / wall / 1e9 / PEAK_HBM_GBS, 4)},
            "references": {"step_shaped_no_arithmetic_gbs": round(mix_gbs, 1),
                           "step_shaped_no_arithmetic_64x1_gbs": round(mix64_gbs, 1),
                           "copy_one_vector_per_lane_gbs": round(copy_gbs, 1),
                           "runtime_d2d_copy_gbs": round(memcpy_gbs, 1),
                           "bytes": nm * 8},
        },
        "in_place_form": in_place,
        "graph_replay": {"graphs": cycle, "ms_per_step": round(gwall / args.steps * 1e3, 4),
                         "value": round(n * args.steps / gwall / 1e9, 3)},
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                   "compute_units": props.multi_processor_count,
                   "memory_gib": round(props.total_memory / 2 ** 30, 1)},
        "scaler_after": {"scale": sc.scale, "applied_steps": sc.step, "skipped": sc.skipped},
    }
    del grads, master, m, v, p16, acc, copy1
    torch.cuda.empty_cache()
    return out


# ----------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded slice of the same workload
# ----------------------------------------------------------------------------

def cpu_share():
    """Host CPUs this process may use: its affinity set, bounded by a cgroup CPU
    quota when one is set (cgroup v2 cpu.max or v1 cfs quota), and by the
    machine's OMP_NUM_THREADS when that states a smaller share."""
    n = len(os.sched_getaffinity(0))
    info = {"affinity_cpus": n}
    quota = None
    try:
        q, period = open("/sys/fs/cgroup/cpu.max").read().split()[:2]
        if q != "max":
            quota = int(q) / int(period)
    except (OSError, ValueError):
        try:
            q = int(open("/sys/fs/cgroup/cpu/cpu.cfs_quota_us").read())
            period = int(open("/sys/fs/cgroup/cpu/cpu.cfs_period_us").read())
            if q > 0:
                quota = q / period
        except (OSError, ValueError):
            pass
    if quota is not None:
        info["cgroup_cpu_quota"] = quota
        n = min(n, max(1, int(quota)))
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        info["omp_num_threads"] = int(omp)
        n = min(n, int(omp))
    return max(1, n), info


def cpu_baseline(workload: str, min_seconds: float, slice_elems: int):
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle
    import synth
    from synth.workloads import BETA1, BETA2, EPS, LR, MASTER_SIGMA, WD, WORKLOADS

    w = WORKLOADS[workload]
    n = min(slice_elems, w.psi)
    threads, share = cpu_share()
    idx = np.arange(n)
    master = synth.host_master32(w.master_key(), idx, MASTER_SIGMA)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    p16 = np.zeros(n, np.uint16)
    grads = [synth.host_grad16(w.grad_key(s + 1), idx, w.grad_spec) for s in range(2)]
    del idx
    sc = oracle.Scaler(w.init_scale, w.min_scale, w.window, w.hysteresis)
    cuts = np.linspace(0, n, threads + 1).astype(np.int64)
    sl = [slice(int(a), int(b)) for a, b in zip(cuts[:-1], cuts[1:])]
    pool = ThreadPoolExecutor(threads)

    def step(g):
        flags = list(pool.map(lambda s: oracle.any_nonfinite(g[s]), sl))
        ov = any(flags)
        if not ov:
            t = sc.applied + 1

            def upd(s):
                oracle.adam(g[s], master[s], m[s], v[s], p16[s], scale=sc.scale, accum_steps=1, t=t,
                            lr=LR, beta1=BETA1, beta2=BETA2, eps=EPS, weight_decay=WD)
            list(pool.map(upd, sl))
        sc.update(ov)

    steps = 0
    t0 = time.perf_counter()
    while True:
        step(grads[steps % 2])
        steps += 1
        if steps >= 2 and time.perf_counter() - t0 >= min_seconds:
            break
    el = time.perf_counter() - t0
    pool.shutdown()

    # the same step on one thread over a slice 1/threads as long (the oracle's
    # loop is per element, so the rate does not depend on the length)
    n1 = max(1, n // threads)
    g1 = [g[:n1].copy() for g in grads]
    st1 = [synth.host_master32(w.master_key(), np.arange(n1), MASTER_SIGMA), np.zeros(n1, np.float32),
           np.zeros(n1, np.float32), np.zeros(n1, np.uint16)]
    sc1 = oracle.Scaler(w.init_scale, w.min_scale, w.window, w.hysteresis)
    steps1 = 0
    t1 = time.perf_counter()
    while True:
        g = g1[steps1 % 2]
        ov = oracle.any_nonfinite(g)
        if not ov:
            oracle.adam(g, *st1, scale=sc1.scale, accum_steps=1, t=sc1.applied + 1, lr=LR, beta1=BETA1,
                        beta2=BETA2, eps=EPS, weight_decay=WD)
        sc1.update(ov)
        steps1 += 1
        if steps1 >= 2 and time.perf_counter() - t1 >= min_seconds / 4:
            break
    el1 = time.perf_counter() - t1
    return {
        "value": round(n * steps / el / 1e9, 4),
        "unit": "Gparams/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{n}-element slice of {workload} (K=1 steps: check + Adam + scaler update), "
                  f"{steps} steps in {el:.1f} s on {threads} threads",
        "cpu_share": share,
        "single_thread_value": round(n1 * steps1 / el1 / 1e9, 4),
        "single_thread_sample": f"{n1}-element slice, {steps1} steps in {el1:.1f} s on 1 thread",
        "cpu_model": cpu_model(),
    }


def cpu_model() -> str:
    """lscpu's model name with the socket, core and thread counts, else /proc/cpuinfo's."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        kv = dict(line.split(":", 1) for line in out.splitlines() if ":" in line)
        kv = {k.strip(): v.strip() for k, v in kv.items()}
        name = kv.get("Model name", "")
        if name:
            extra = ", ".join(f"{k} {kv[k]}" for k in ("CPU(s)", "Socket(s)", "Core(s) per socket",
                                                         "Thread(s) per core", "CPU family", "Model")
                              if k in kv)
            return f"{name} ({extra})" if extra else name
    except (OSError, ValueError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ----------------------------------------------------------------------------
# data-movement references
# ----------------------------------------------------------------------------

def copy_mode(args):
    """Data-movement references on their own arrays: a 4 GiB copy by the plain
    copy kernel and by the runtime (hipMemcpyAsync through torch's copy_), and
    the step's 14 B read + 14 B written per element with no arithmetic on a
    109M-element partition."""
    import torch

    import synth
    dev = torch.device("cuda:0")
    res = {}

    def timed(fn, reps=10):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps / 1e3

    nbytes = 4 << 30
    src = torch.empty(nbytes // 4, dtype=torch.int32, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for name, fn in (("copy_one_vector_per_lane", lambda: synth.device_copy(torch, dst, src)),
                     ("runtime_d2d_copy", lambda: dst.copy_(src))):
        t = timed(fn)
        res[name] = {"bytes_read": nbytes, "bytes_written": nbytes, "avg_ms": round(t * 1e3, 4),
                     "GBps": round(2 * nbytes / t / 1e9, 1)}
    del src, dst
    n = 109_375_000
    g = torch.zeros(n, dtype=torch.int16, device=dev)
    h = torch.zeros(n, dtype=torch.int16, device=dev)
    x, y, z = (torch.zeros(n, dtype=torch.float32, device=dev) for _ in range(3))
    t = timed(lambda: synth.device_stream_mix(torch, g, x, y, z, h))
    res["step_shaped_mix"] = {"elements": n, "bytes_per_elem": 28, "avg_ms": round(t * 1e3, 4),
                              "GBps": round(28 * n / t / 1e9, 1)}
    print(json.dumps({"mode": "copy", **res}), flush=True)


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="zero1_70b")
    ap.add_argument("--mode", default="step", choices=["step", "copy"])
    ap.add_argument("--max-grad-buffers", type=int, default=8)
    ap.add_argument("--bf16", action="store_true",
                    help="bf16 gradients and parameter copy, no loss scaling")
    ap.add_argument("--clip", type=float, default=0.0,
                    help="gradient_clipping max norm (0: the workloads' setting, no clipping)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--cpu-slice", type=int, default=109_375_000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--step-form", default="auto", choices=["auto", "double", "in_place"],
                    help="double: two copies of the state, the overflow check (and with K > 1 the last "
                         "micro-batch or fold) fused into the Adam pass (ds_adam_step_double_buffered, "
                         "ds_accumulate_adam_double_buffered; no clipping); in_place: the check (or the "
                         "accumulation), then the in-place Adam pass; auto (default): double where it applies, "
                         "the second copy fits and (K = 1) the gradient is larger than the 256 MB Infinity Cache "
                         "or the whole state fits in it, then the in-place form timed after it on the copy that "
                         "holds the state")
    ap.add_argument("--double-buffer", dest="step_form", action="store_const", const="double",
                    help="the same as --step-form double")
    ap.add_argument("--fold", type=int, default=1,
                    help="micro-batches folded into the accumulation buffer per pass (1..8; K > 1 workloads; "
                         "needs that many gradient buffers held at once)")
    ap.add_argument("--step-log", default=None,
                    help="write one JSON line per step (scale used, overflow, t, growth count, device time) "
                         "from an untimed pass")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported; the benchmark measures one GPU's "
              "partition (ranks only exchange the 4-byte overflow flag, which needs a second GPU)",
              file=sys.stderr)
        sys.exit(2)
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: launched with WORLD_SIZE > 1; the benchmark measures one GPU", file=sys.stderr)
        sys.exit(2)
    if args.mode == "copy":
        copy_mode(args)
        return
    out = gpu_run(args)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded slice ...")
        out["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_seconds, args.cpu_slice)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
