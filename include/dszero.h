/*
 * dszero.h -- C ABI of the MI355X (gfx950) ZeRO mixed-precision optimizer step.
 *
 * One GPU's share of ZeRO data-parallel training: the optimizer step that each
 * rank runs on its own contiguous 1/N partition of the model state, gated by
 * dynamic loss scaling and fed by fp16 gradient accumulation into an fp32
 * buffer.
 *
 * Pages cited (by title and section):
 *   [Guide]    "DeepSpeed complete guide" (youngju.dev, Japanese)
 *   [Overview] "DeepSpeed" project overview (aibars.net, Japanese), core features
 *
 * Model state per element of a partition ([Guide] section 2, memory table):
 * fp16 parameter copy (p16), fp16 gradient, fp32 master parameter, fp32 Adam
 * first moment (m), fp32 Adam second moment (v).  In bf16 mode ([Guide]
 * section 4.2, bf16 settings) the 16-bit parameter copy and gradients are
 * bf16 instead and no loss scaling is applied (a static scale of 1).  With
 * ZeRO-1/2 each rank owns a contiguous 1/N range of these arrays and updates
 * only that range ([Guide] sections 2.1 and 2.2).
 *
 * Conventions shared by every entry point:
 *  - Memory.  Array arguments are DEVICE pointers owned by the caller; the
 *    library never allocates, frees or keeps them.  Work is enqueued
 *    asynchronously on `stream` (a hipStream_t; NULL is the default stream)
 *    and uses the buffers until the stream reaches it.
 *  - Layout.  Arrays are flat and contiguous, element i of every array belongs
 *    to the same parameter.  16-bit values are bit patterns (uint16_t) of IEEE
 *    binary16 (DS_FP16) or bf16 (DS_BF16: the upper half of an IEEE binary32);
 *    fp32 values are IEEE binary32.
 *  - Alignment.  Every array pointer must be 16-byte aligned; a ds_scaler
 *    pointer must be 8-byte aligned.
 *  - Errors.  Every call validates all arguments before any device work, so a
 *    call that returns an error has had no effect.  n < 0, or n > 2^40
 *    (more elements than any device holds) -> DS_ERR_SIZE;
 *    n == 0 -> DS_OK and nothing is launched; a NULL array with n > 0 ->
 *    DS_ERR_NULL; a misaligned pointer -> DS_ERR_ALIGN; overlapping arrays ->
 *    DS_ERR_ALIAS; an unknown dtype -> DS_ERR_DTYPE; an out-of-range
 *    hyperparameter -> DS_ERR_HPARAM; a failed HIP launch or copy ->
 *    DS_ERR_HIP (the enqueue failed; earlier work is unaffected).
 *  - Data is not an error: inf/NaN gradients set the overflow flag.
 *  - Per-step order on one stream: all ds_accumulate calls, then any number of
 *    ds_check_overflow calls (disjoint ranges), then any number of
 *    ds_adam_step calls (disjoint ranges, all reading the same state), then
 *    exactly one ds_update_loss_scale; or, for a partition updated by a
 *    single call, one ds_adam_step_fused in place of both.  No host
 *    synchronisation is needed inside a step: the skip decision is taken on
 *    the device.
 *  - Thread safety: the library keeps no mutable global state.  Calls that
 *    share a ds_scaler must be ordered on one stream.
 *  - Launch-shape knobs, read from the environment at each call (for tests
 *    and tuning; results are bit-identical under every setting):
 *    DSZERO_GRID=<blocks> pins the block count of every kernel of the call
 *    (the kernels loop over their tiles or chunks); DSZERO_UNROLL=2 halves
 *    the tile of ds_adam_step to 2048 elements (256 lanes x 2 quads; by
 *    default 4096 elements as 256 lanes x 4 quads, or 512 x 2 for
 *    ds_adam_step_fused without non-temporal hints); DSZERO_NT=0|1 turns the
 *    non-temporal load/store hints of the read/write kernels off or on
 *    (default: on above 2^24 elements, off at and below, where the state
 *    stays in the Infinity Cache between steps).
 */
#ifndef DSZERO_H
#define DSZERO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
/* A C caller may pass any int where an enum is expected; giving the enums a
 * fixed underlying type makes every such value representable in C++ (so the
 * library can reject it as DS_ERR_DTYPE and the like) with the same 4-byte
 * layout as the C enums. */
#define DS_ENUM_BASE : int32_t
#else
#define DS_ENUM_BASE
#endif

typedef enum ds_status DS_ENUM_BASE {
    DS_OK = 0,
    DS_ERR_NULL = 1,
    DS_ERR_SIZE = 2,
    DS_ERR_ALIGN = 3,
    DS_ERR_DTYPE = 4,
    DS_ERR_HPARAM = 5,
    DS_ERR_ALIAS = 6,
    DS_ERR_HIP = 7
} ds_status;

typedef enum ds_dtype DS_ENUM_BASE { DS_FP16 = 1, DS_FP32 = 2, DS_BF16 = 3 } ds_dtype;

/*
 * Per-step device state, 128 bytes, kept in caller-owned DEVICE memory so that
 * the kernels read the scale, the overflow flag and the gradient norm without
 * a host sync.  The loss-scaler fields follow the fp16 block of ds_config.json
 * ([Guide] section 4.2: loss_scale 0 = dynamic, initial scale
 * 2^initial_scale_power, loss_scale_window = successful steps before the scale
 * grows, hysteresis = overflows before it shrinks, min_loss_scale = floor).
 * grad_sumsq accumulates the sum of squares of the step's (still scaled)
 * gradient for global-norm clipping ([Guide] section 4.1 gradient_clipping).
 */
typedef struct ds_scaler {
    float scale;                    /* S: loss scale the next step unscales by        */
    float min_scale;                /* floor of S (min_loss_scale)                    */
    int32_t growth_window;          /* W: successful steps before S doubles           */
    int32_t growth_count;           /* successful steps since last overflow or growth */
    int32_t hysteresis;             /* H: overflows needed before S halves            */
    int32_t hysteresis_left;        /* overflows still tolerated before S halves      */
    int32_t dynamic;                /* 1: dynamic scaling; 0: static S                */
    uint32_t overflow;              /* OR of non-finite findings of the current step  */
    int64_t step;                   /* applied Adam steps (t of the last update)      */
    int64_t iter;                   /* all steps, applied or skipped                  */
    int64_t skipped;                /* skipped steps                                  */
    int32_t consecutive_hysteresis; /* 1: a successful step refills hysteresis_left   */
    uint32_t last_overflow;         /* overflow flag consumed by the last update      */
    double grad_sumsq;              /* sum of squares of the step's gradient so far   */
    double last_grad_sumsq;         /* grad_sumsq consumed by the last update         */
    uint32_t blocks_done;           /* ds_adam_step_fused: blocks finished (0 between steps) */
    uint32_t sumsq_blocks_done;     /* sum-of-squares second pass: blocks finished (0 between calls) */
    uint32_t current;               /* ds_adam_step_double_buffered: copy holding the state (0 or 1) */
    uint32_t reserved0;             /* zero                                           */
    uint64_t db_tickets;            /* ds_adam_step_double_buffered: blocks finished (low 32 bits) and
                                       blocks that found a non-finite gradient (high 32 bits); 0 between steps */
    uint8_t reserved[24];           /* zero                                           */
} ds_scaler;

/* sizeof(ds_scaler) as compiled into the library (128). */
size_t ds_scaler_size(void);

/*
 * Initialise a scaler ([Guide] section 4.2).  init_scale = 2^initial_scale_power,
 * min_scale = min_loss_scale, growth_window = loss_scale_window, hysteresis,
 * consecutive_hysteresis, dynamic = (loss_scale == 0); for a static scale pass
 * the fixed scale as init_scale and dynamic = 0.  Sets step = iter = skipped = 0
 * and clears the flag and the gradient sum of squares.  Asynchronous (a
 * one-thread kernel writes the struct).
 * DS_ERR_HPARAM: init_scale or min_scale not finite or <= 0, growth_window < 1,
 * hysteresis < 1.
 */
ds_status ds_state_init(ds_scaler* st, float init_scale, float min_scale, int32_t growth_window,
                        int32_t hysteresis, int32_t consecutive_hysteresis, int32_t dynamic,
                        void* stream);

/* Copy the device state into *host_out (host memory) and synchronise `stream`. */
ds_status ds_state_read(const ds_scaler* st, ds_scaler* host_out, void* stream);

/* Overwrite the device state with *host_in (resume from a snapshot).  The
 * struct is passed by value to a one-thread kernel, so host_in may be freed as
 * soon as the call returns. */
ds_status ds_state_write(ds_scaler* st, const ds_scaler* host_in, void* stream);

/*
 * Gradient accumulation ([Overview] core features: accumulating micro-batch
 * gradients emulates a larger batch; [Guide] section 5.1: backward handles
 * the accumulation; section 4.3: gradient_accumulation_steps).
 *   overwrite != 0 : acc[i] = float(g16[i])            (first micro-batch)
 *   overwrite == 0 : acc[i] = acc[i] + float(g16[i])   (later micro-batches, in order)
 * acc: fp32[n], g16: 16-bit[n] of type gdt (DS_FP16 or DS_BF16; the widening
 * is exact).  If st is not NULL the same pass ORs "acc[i] is not finite" into
 * st->overflow (use it on the last micro-batch: the check of the step then
 * costs no extra pass).  Errors: see the conventions; acc, g16 and st must not
 * overlap; gdt other than DS_FP16/DS_BF16 -> DS_ERR_DTYPE.
 */
ds_status ds_accumulate(float* acc, const uint16_t* g16, ds_dtype gdt, int64_t n, int32_t overwrite,
                        ds_scaler* st_or_null, void* stream);

/*
 * Overflow check ([Overview] core features: dynamic loss scaling; [Guide]
 * section 13.1, gradient overflow in fp16): ORs "some grad[i] is +-inf or NaN"
 * into st->overflow.  grad: fp16[n] (dt = DS_FP16), bf16[n] (DS_BF16) or
 * fp32[n] (DS_FP32).  The largest finite value (65504 in fp16) is not an
 * overflow.  Does nothing more once the flag is already set for this step.
 */
ds_status ds_check_overflow(ds_scaler* st, const void* grad, ds_dtype dt, int64_t n, void* stream);

/*
 * Fused mixed-precision Adam step over n elements ([Guide] section 2: fp32
 * master, first and second moments, fp16 parameter copy; section 4.1:
 * optimizer AdamW with lr, betas, eps, weight_decay; section 5.1: step()).
 * If st->overflow is set the kernel writes nothing (the step is skipped).
 * Otherwise, with S = st->scale, K = accum_steps and t = st->step + 1:
 *   g      = grad[i] / (S*K)                     (unscale; grad fp16 or fp32)
 *            (with max_grad_norm > 0 the multiplier 1/(S*K) is scaled by the
 *             global-norm clipping coefficient below)
 *   m[i]   = beta1*m[i] + (1-beta1)*g
 *   v[i]   = beta2*v[i] + (1-beta2)*g*g
 *   master = master - lr*weight_decay*master     (only if weight_decay != 0)
 *   master = master - lr/(1-beta1^t) * m[i] / (sqrt(v[i])/sqrt(1-beta2^t) + eps)
 *   p16[i] = fp16(master[i]) or bf16(master[i])  (pdt; round to nearest even)
 * in IEEE fp32, one rounding per operation; the two bias-correction factors
 * are evaluated in fp64 and rounded once.  master/m/v: fp32[n] in place;
 * p16: 16-bit[n] out, of type pdt (DS_FP16 or DS_BF16); grad: [n] in, of
 * type dt (DS_FP16, DS_BF16, or DS_FP32 for the accumulation buffer).  st is
 * read only (t and S advance in ds_update_loss_scale).
 * Global-norm clipping ([Guide] sections 4.1 and 5.4 gradient_clipping,
 * section 5.1 step() includes clipping): with max_grad_norm > 0, using the
 * step's st->grad_sumsq (filled by ds_check_overflow_sumsq or
 * ds_accumulate_sumsq over the whole partition) and inv = fp32(1/(S*K)):
 *   norm = sqrt(grad_sumsq) * inv                         (fp64)
 *   coef = min(1, max_grad_norm / (norm + 1e-6))          (fp64)
 *   the multiplier of the gradient becomes fp32(inv * coef)
 * max_grad_norm = 0 disables clipping (the multiplier is inv).
 * DS_ERR_HPARAM: lr, weight_decay or max_grad_norm negative or not finite,
 * beta1 or beta2 outside [0, 1), eps not finite or <= 0, accum_steps < 1.
 */
ds_status ds_adam_step(const ds_scaler* st, float* master, float* m, float* v, uint16_t* p16,
                       ds_dtype pdt, const void* grad, ds_dtype dt, int64_t n, float lr, float beta1,
                       float beta2, float eps, float weight_decay, float max_grad_norm,
                       int32_t accum_steps, void* stream);

/*
 * Learning-rate schedules ([Guide] section 4.1: the scheduler block of the
 * base ds_config.json, WarmupLR; section 4.4: WarmupDecayLR with
 * warmup_min_lr, warmup_max_lr, warmup_num_steps, total_num_steps and a
 * linear warmup).  The pages give the parameters, not the formula; the
 * schedule read here: with it = st->step, the count of Adam steps applied
 * before this one (a fresh run starts at 0; a skipped step does not advance
 * it, so the schedule stays on the device and resumes with the state),
 *   gamma = it / warmup_num_steps                    while it < warmup_num_steps
 *         = 1                                        afterwards, DS_LR_WARMUP
 *         = max(0, (total - it) / max(1, total - warmup_num_steps))
 *                                                    afterwards, DS_LR_WARMUP_DECAY
 *   lr    = warmup_min_lr + (warmup_max_lr - warmup_min_lr) * gamma
 * in fp64, rounded once to fp32; that lr then enters the step like a
 * constant lr.  A host struct, read during the call and not kept.
 * Valid: kind one of the two below, both rates finite and >= 0,
 * warmup_num_steps >= 0, and for DS_LR_WARMUP_DECAY total_num_steps >=
 * warmup_num_steps; anything else is DS_ERR_HPARAM.
 */
typedef enum ds_lr_kind DS_ENUM_BASE { DS_LR_WARMUP = 1, DS_LR_WARMUP_DECAY = 2 } ds_lr_kind;

typedef struct ds_lr_schedule {
    int32_t kind;             /* ds_lr_kind */
    int32_t reserved;         /* set to 0 */
    int64_t warmup_num_steps; /* applied steps of the linear rise */
    int64_t total_num_steps;  /* DS_LR_WARMUP_DECAY: where the fall ends; else ignored */
    float warmup_min_lr;      /* lr of the first step, and the end of the fall */
    float warmup_max_lr;      /* the peak, reached after the warmup */
} ds_lr_schedule;

/*
 * ds_adam_step with the learning rate taken from `sched` (a HOST pointer) at
 * the device's applied-step count, so a whole step, schedule included, runs
 * without a host round trip (and can be captured once into a graph and
 * replayed).  Every other argument, the arithmetic and the errors are those
 * of ds_adam_step; sched NULL is DS_ERR_NULL, an invalid schedule
 * DS_ERR_HPARAM.
 */
ds_status ds_adam_step_sched(const ds_scaler* st, float* master, float* m, float* v, uint16_t* p16,
                             ds_dtype pdt, const void* grad, ds_dtype dt, int64_t n,
                             const ds_lr_schedule* sched, float beta1, float beta2, float eps,
                             float weight_decay, float max_grad_norm, int32_t accum_steps,
                             void* stream);

/*
 * ds_adam_step (sched_or_null NULL: constant lr) or ds_adam_step_sched
 * (sched_or_null: a host ds_lr_schedule, lr ignored) followed by
 * ds_update_loss_scale, in one kernel: for a partition updated by a single
 * call per step, which then calls no ds_update_loss_scale of its own.  Each
 * block of the kernel, when done, takes a ticket from st->blocks_done (one
 * atomic add); the block with the last ticket advances the scaler exactly as
 * ds_update_loss_scale does and sets the count back to 0.  Arithmetic,
 * results and errors are those of the two calls it replaces; with n == 0
 * only the scaler advances.  st is read and written.
 */
ds_status ds_adam_step_fused(ds_scaler* st, float* master, float* m, float* v, uint16_t* p16, ds_dtype pdt,
                             const void* grad, ds_dtype dt, int64_t n, float lr,
                             const ds_lr_schedule* sched_or_null, float beta1, float beta2, float eps,
                             float weight_decay, float max_grad_norm, int32_t accum_steps, void* stream);

/*
 * A whole step for a caller that keeps two copies (0 and 1) of the fp32
 * master, m and v arrays and of the 16-bit parameter copy (30 bytes of device
 * memory per element instead of 16), in one HBM pass: the overflow check of
 * the gradient is fused into the Adam pass ([Guide] section 2, section 4.2
 * dynamic loss scaling, section 5.1 step()).  st->current names the copy that
 * holds the state.  The kernel reads the gradient and the current copy once,
 * tests whether some gradient value is +-inf or NaN, and writes the Adam
 * update of every element (the arithmetic of ds_adam_step) into the other
 * copy; each block's finding travels in its ticket (st->db_tickets), and the
 * last block to finish advances the scaler as ds_update_loss_scale does with
 * the OR of all findings and st->overflow and, if the step applied (no
 * overflow), makes the other copy current.  A skipped step leaves the current
 * copy bit-identical (only the other copy, which holds no state, is written)
 * and t unchanged.
 * The step moves 28 bytes per element with an fp16 gradient instead of the
 * 30 of ds_check_overflow + ds_adam_step_fused.  Call it once per step for the
 * whole partition, in place of ds_check_overflow and ds_adam_step_fused (a flag
 * already raised earlier in the step, e.g. by a fused accumulation check, also
 * skips it).  No gradient clipping (it needs the whole gradient's norm before
 * the update).
 * master2, m2, v2: HOST arrays of 2 DEVICE pointers to fp32[n]; p16_2: HOST
 * array of 2 DEVICE pointers to 16-bit[n] of type pdt; the eight arrays, grad
 * and st must not overlap.  lr / sched_or_null, betas, eps, weight_decay,
 * accum_steps, grad and dt: as for ds_adam_step_fused.  With n == 0 only the
 * scaler advances (and the copies swap if the step applied).  The copy that
 * is current after a call is read back with ds_state_read (st.current).
 * Errors: as for ds_adam_step_fused; a NULL host array -> DS_ERR_NULL.
 */
ds_status ds_adam_step_double_buffered(ds_scaler* st, float* const* master2, float* const* m2, float* const* v2,
                                       uint16_t* const* p16_2, ds_dtype pdt, const void* grad, ds_dtype dt,
                                       int64_t n, float lr, const ds_lr_schedule* sched_or_null, float beta1,
                                       float beta2, float eps, float weight_decay, int32_t accum_steps,
                                       void* stream);

/*
 * The last micro-batches of a step folded into the double-buffered Adam pass
 * ([Guide] section 4.3 gradient accumulation, [Overview] gradient
 * accumulation; [Guide] section 4.2 dynamic loss scaling, section 5.1
 * step()).  The gradient of element i is the fp32 sum, in micro-batch order,
 * of acc_or_null[i] (the running sum of the step's earlier micro-batches as
 * ds_accumulate / ds_accumulate_multi leave it; NULL when grads are all of the
 * step's micro-batches, the first of them then starting the sum) and of
 * grads[0][i] .. grads[count-1][i]: the sum ds_accumulate would have formed,
 * which is used, not stored.  The pass ORs "some sum is +-inf or NaN" into
 * st->overflow and writes the Adam update of every element of [0, n) (the
 * arithmetic of ds_adam_step with that sum as the fp32 gradient) into the copy
 * of master, m, v and the 16-bit copy that does not hold the state
 * (st->current names the one that does); nothing else in st changes.  Call it
 * once for the partition, or once per bucket (disjoint ranges, each with its
 * own offsets into every array), then ds_update_loss_scale_double_buffered
 * exactly once.  The step's earlier micro-batches go through ds_accumulate
 * (with st_or_null NULL or not: a flag raised there also skips the step).
 * Bytes per element: 2 * count + 30 with the running sum (read only), 2 *
 * count + 26 without, against 2 * count + 8 (or + 4) for the fold and 30 for
 * the Adam pass done separately.  No gradient clipping (it needs the whole
 * gradient's norm before the update).
 * master2, m2, v2, p16_2, pdt, lr / sched_or_null, betas, eps, weight_decay,
 * accum_steps (K, the unscale divisor), stream: as for
 * ds_adam_step_double_buffered.  grads: HOST array of count (1-8) DEVICE
 * pointers to 16-bit[n] of format gdt (fp16 or bf16); they may repeat but
 * must not overlap acc, st or the eight state arrays, which must not overlap
 * one another.  acc_or_null: DEVICE fp32[n] or NULL.
 * Errors: count outside 1..8 -> DS_ERR_SIZE; gdt or pdt not a 16-bit format ->
 * DS_ERR_DTYPE; acc_or_null NULL with count != accum_steps, or non-NULL with
 * count >= accum_steps -> DS_ERR_HPARAM; otherwise as for
 * ds_adam_step_double_buffered.  With n == 0 nothing is launched.
 */
ds_status ds_accumulate_adam_double_buffered(ds_scaler* st, float* const* master2, float* const* m2,
                                             float* const* v2, uint16_t* const* p16_2, ds_dtype pdt,
                                             const float* acc_or_null, const uint16_t* const* grads, int32_t count,
                                             ds_dtype gdt, int64_t n, float lr, const ds_lr_schedule* sched_or_null,
                                             float beta1, float beta2, float eps, float weight_decay,
                                             int32_t accum_steps, void* stream);

/*
 * End of a double-buffered step taken with ds_accumulate_adam_double_buffered
 * ([Guide] section 4.2): advance the scaler by the step's flag as
 * ds_update_loss_scale does and, if the step applied (no overflow), make the
 * other copy current (st->current ^= 1).  Call exactly once per step.
 * Errors: st NULL -> DS_ERR_NULL; st not 8-byte aligned -> DS_ERR_ALIGN.
 */
ds_status ds_update_loss_scale_double_buffered(ds_scaler* st, void* stream);

/*
 * End of a step: advance the scaler by the step's overflow flag, then clear
 * the flag ([Guide] section 4.2).  Overflow: skipped += 1, growth_count = 0;
 * if dynamic, one more overflow is charged to the hysteresis and, when it is
 * used up, S = max(S/2, min_scale) and the hysteresis restarts.  No overflow:
 * step += 1; if dynamic, growth_count += 1 and at growth_window S doubles and
 * growth_count restarts (consecutive_hysteresis refills the hysteresis).
 * iter += 1, last_overflow = flag and last_grad_sumsq = grad_sumsq in both
 * cases; grad_sumsq restarts at 0.  Call exactly once per step.
 */
ds_status ds_update_loss_scale(ds_scaler* st, void* stream);

/*
 * Gradient sum of squares for global-norm clipping, fused into the passes
 * that already read the gradient.  Both add sum(x_i^2) over their n values
 * (the stored, still loss-scaled gradient: fp16 values, or the fp32
 * accumulation) into st->grad_sumsq, in fp64.  The sum is taken over fixed
 * chunks of consecutive elements (8192 for the check, 1024 for the
 * accumulation), each reduced in a fixed order, then over groups of 4096
 * chunk sums and the group sums, each in a fixed order, so the result does
 * not depend on the launch shape.  Several calls per step (disjoint ranges,
 * e.g. buckets) add up in call order.
 *
 * workspace: caller-owned DEVICE scratch of at least
 * ds_sumsq_workspace_bytes(n) bytes (one fp64 partial sum per chunk and per
 * group), 8-byte aligned, no initial contents needed.  Each call is two
 * kernels: the pass over the data writes the chunk sums, a second pass adds
 * them by groups, and its last block to finish adds the group sums (taking
 * one ticket per block from st->sumsq_blocks_done, which it leaves at 0).
 * One workspace serves every call on one stream (calls that may run at the
 * same time need their own).
 * Errors as for the plain entry points; DS_ERR_NULL / DS_ERR_SIZE /
 * DS_ERR_ALIGN / DS_ERR_ALIAS also cover the workspace.
 */
size_t ds_sumsq_workspace_bytes(int64_t n);

/* ds_check_overflow plus the sum of squares of grad (fp16, bf16 or fp32), one pass. */
ds_status ds_check_overflow_sumsq(ds_scaler* st, const void* grad, ds_dtype dt, int64_t n,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * ds_check_overflow_sumsq without a caller workspace, for callers that cannot
 * allocate device memory: code under stream or graph capture, tight serving
 * loops, harnesses that forbid allocation.  The call allocates nothing: the
 * chunk and group sums go to a scratch array of 2^21 fp64 values (16 MiB)
 * that the library holds in each device's memory until the process ends.
 * Flag and sum of squares are bit-identical to those of
 * ds_check_overflow_sumsq.  n may be at most DS_NOALLOC_MAX_ELEMS (2,096,640
 * chunks of 8192 elements); a larger n is DS_ERR_SIZE.  The first call on a
 * device (the device of `stream`, or the current one for the null stream)
 * looks up the address of that device's array and keeps it; DS_ERR_HIP if
 * that fails.  Every call on one device shares that device's array, which
 * keeps the last call's contents: calls that may run at the same time on one
 * device (other streams, other threads) race and give wrong sums, so order
 * them on one stream.  Nothing in the array needs to start at zero: every
 * chunk and group sum is written before it is read.
 */
#define DS_NOALLOC_MAX_ELEMS 17175674880LL
ds_status ds_check_overflow_sumsq_noalloc(ds_scaler* st, const void* grad, ds_dtype dt, int64_t n, void* stream);

/* ds_accumulate with the fused overflow check (st required) plus the sum of
 * squares of the accumulated values, one pass: use it for the last
 * micro-batch of a clipped step. */
ds_status ds_accumulate_sumsq(float* acc, const uint16_t* g16, ds_dtype gdt, int64_t n,
                              int32_t overwrite, ds_scaler* st, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * Several micro-batch gradients folded into the accumulation buffer in one
 * pass (gradient accumulation as for ds_accumulate: [Overview] core features;
 * [Guide] sections 4.3 and 5.1):
 *   acc[i] = (overwrite ? float(g_0[i]) : acc[i] + float(g_0[i]))
 *            + float(g_1[i]) + ... + float(g_{count-1}[i])
 * with every add an fp32 add in this order, so the result is bit for bit that
 * of `count` consecutive ds_accumulate calls.  A caller that can hold `count`
 * 16-bit micro-batch gradients at once (grads[k] is the k-th in micro-batch
 * order) moves 2 * count + 8 bytes per element (2 * count + 4 when
 * overwriting) instead of 10 bytes per micro-batch.
 * grads: HOST array of `count` (1..8) DEVICE pointers to 16-bit[n] arrays of
 * type gdt; they may repeat or overlap one another but not acc, st or the
 * workspace.  st_or_null: as for ds_accumulate (the fused inf/NaN check of the
 * result).  workspace_or_null: as for ds_accumulate_sumsq (requires st; adds
 * the sum of squares of the result to st->grad_sumsq, same chunks, so the
 * value equals that of a ds_accumulate_sumsq pass producing the same acc).
 * Errors: count outside 1..8 -> DS_ERR_SIZE; otherwise as ds_accumulate and
 * ds_accumulate_sumsq.
 */
ds_status ds_accumulate_multi(float* acc, const uint16_t* const* grads, int32_t count, ds_dtype gdt, int64_t n,
                              int32_t overwrite, ds_scaler* st_or_null, void* workspace_or_null,
                              size_t workspace_bytes, void* stream);

/*
 * The bias-correction scalars the next applied step will use, evaluated on
 * the device exactly as ds_adam_step does (t = st->step + 1):
 * out2[0] = fp32(lr / (1 - beta1^t)), out2[1] = fp32(1 / sqrt(1 - beta2^t)).
 * out2: device float[2].  For diagnostics and tests.
 */
ds_status ds_adam_bias_scalars(const ds_scaler* st, float lr, float beta1, float beta2,
                               float* out2, void* stream);

/*
 * The scheduled learning rate and bias-correction scalars the next applied
 * step will use, evaluated on the device exactly as ds_adam_step_sched does:
 * out3[0] = lr, out3[1] = fp32(lr / (1 - beta1^t)),
 * out3[2] = fp32(1 / sqrt(1 - beta2^t)), t = st->step + 1.
 * sched: host struct; out3: device float[3].  For diagnostics and tests.
 */
ds_status ds_lr_scalars(const ds_scaler* st, const ds_lr_schedule* sched, float beta1, float beta2,
                        float* out3, void* stream);

/*
 * Flat layout of ragged tensors in contiguous buffers with greedy buckets
 * ([Guide] sections 2.2 and 4.1: contiguous_gradients, reduce_bucket_size and
 * allgather_bucket_size of 2e8 elements).  Host-only, no device work.
 * Tensors keep their order; tensor i starts at offsets[i], a multiple of
 * `align` elements.  A tensor joins the open bucket if the bucket, padded to
 * `align`, then holds at most `cap` elements; otherwise the bucket closes and
 * the tensor opens the next one (a tensor larger than cap gets its own
 * bucket).  Outputs (host arrays of `count` entries, caller-owned): offsets,
 * bucket_of; bucket_start and bucket_size (first *n_buckets entries used);
 * *total = padded length of the flat array.  DS_ERR_SIZE: count < 0, a
 * negative size, cap < 1, align < 1, cap or align above 2^40, or sizes whose
 * sum plus count * (align - 1) exceeds 2^40 (nothing is written then).
 */
ds_status ds_layout_greedy(const int64_t* numels, int32_t count, int64_t cap, int64_t align,
                           int64_t* offsets, int32_t* bucket_of, int64_t* bucket_start,
                           int64_t* bucket_size, int32_t* n_buckets, int64_t* total);

/*
 * ZeRO partition of a flat array of `total` elements over `world` ranks
 * ([Guide] sections 2.1 and 2.2: each rank owns a contiguous 1/N share):
 * rank r gets [r*per, min((r+1)*per, total)) with per = ceil(total/world)
 * rounded up to `align`.  Host-only.  DS_ERR_SIZE: total outside
 * [0, 2^40], world < 1, rank outside [0, world), align outside [1, 2^40].
 */
ds_status ds_partition_range(int64_t total, int32_t world, int32_t rank, int64_t align,
                             int64_t* start, int64_t* count);

/* Static string naming a status code. */
const char* ds_status_string(ds_status s);

#ifdef __cplusplus
}
#endif

#endif /* DSZERO_H */
