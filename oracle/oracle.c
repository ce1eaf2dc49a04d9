/*
 * oracle.c -- plain, slow, scalar CPU oracle for the ZeRO mixed-precision
 * optimizer step.  TEST INFRASTRUCTURE ONLY: nothing in the product path may
 * link, load or call this file; only the tests, the smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header, table or
 * constant with the GPU library.
 *
 * Pages cited (by title and section):
 *   [Guide]    "DeepSpeed complete guide" (youngju.dev, Japanese)
 *   [Overview] "DeepSpeed" project overview (aibars.net, Japanese), core-features list
 *
 * Precision.  [Guide] section 2, memory table, fixes the precision of every
 * array: fp16 parameters and gradients, fp32 master parameters, fp32 Adam
 * first and second moments.  The update is therefore evaluated in IEEE fp32
 * with round-to-nearest-even, one rounding per operation, in the order written
 * below (build with -ffp-contract=off, no fast-math).  The per-step bias
 * correction scalars are evaluated in fp64 and rounded once to fp32.
 *
 * Pins (tests/test_oracle_*.py) fix every function against the pages' values,
 * closed forms, exhaustive library comparisons and brute force.  The branches
 * of zo_scaler_update that the pages give only a one-line meaning for (the
 * restart of the hysteresis count after a decrease, consecutive_hysteresis,
 * the uncapped growth) are pinned to their reading's run-length closed form:
 * the readings themselves are choices the pages leave open.
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared -ffp-contract=off -fno-fast-math
 *            -o liboracle.so oracle.c -lm
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary16 <-> binary32, written from the format's definition.      */
/* ------------------------------------------------------------------------ */

/* Decode one binary16 pattern.  Fields: sign s (1 bit), biased exponent e
 * (5 bits, bias 15), fraction f (10 bits).
 *   e == 0        : (-1)^s * 2^-14 * (f / 1024)           (zero, subnormal)
 *   0 < e < 31    : (-1)^s * 2^(e-15) * (1 + f / 1024)    (normal)
 *   e == 31, f==0 : (-1)^s * infinity
 *   e == 31, f!=0 : NaN; the fraction is carried into the top of the binary32
 *                   fraction (the widening keeps the payload).
 * Every finite binary16 value is exactly representable in binary32, so the
 * arithmetic below is exact. */
float zo_dec16(uint16_t h)
{
    uint32_t s = (uint32_t)(h >> 15) & 1u;
    uint32_t e = (uint32_t)(h >> 10) & 0x1Fu;
    uint32_t f = (uint32_t)h & 0x3FFu;
    float mag;
    if (e == 31u) {
        uint32_t bits = (s << 31) | 0x7F800000u | (f << 13);
        float out;
        memcpy(&out, &bits, sizeof out);
        return out;
    }
    if (e == 0u)
        mag = ldexpf((float)f, -24);                   /* 2^-14 * f/2^10 */
    else
        mag = ldexpf((float)(1024u + f), (int)e - 25); /* 2^(e-15) * (1024+f)/2^10 */
    return s ? -mag : mag;
}

/* Round a non-negative float holding an integer-plus-fraction below 2^23 to
 * the nearest integer, ties to the even integer. */
static uint32_t round_half_even(float q)
{
    float fl = floorf(q);
    float frac = q - fl; /* exact: q and fl share the exponent range */
    uint32_t r = (uint32_t)fl;
    if (frac > 0.5f || (frac == 0.5f && (r & 1u)))
        r += 1u;
    return r;
}

/* Encode one binary32 value as binary16, rounding to nearest, ties to even.
 * Largest finite binary16 is 65504 = (2 - 2^-10) * 2^15; its half-unit is 16,
 * so magnitudes of 65520 and above round to infinity.  Below 2^-14 the
 * binary16 grid is uniform with spacing 2^-24 (subnormals).  NaN encodes as
 * the quiet NaN 0x7E00 with the input's sign. */
uint16_t zo_enc16(float x)
{
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    if (isnan(x))
        return (uint16_t)(sign | 0x7E00u);
    float a = fabsf(x);
    if (a >= 65520.0f)
        return (uint16_t)(sign | 0x7C00u);
    if (a < 0x1p-14f) {
        /* units of 2^-24; scaling by a power of two is exact */
        uint32_t r = round_half_even(a * 0x1p24f); /* 0..1024; 1024 is the smallest normal */
        return (uint16_t)(sign | r);
    }
    int ex;
    (void)frexpf(a, &ex);                  /* a = mant * 2^ex, mant in [0.5, 1) */
    int E = ex - 1;                        /* a in [2^E, 2^(E+1)), E in [-14, 15] */
    uint32_t r = round_half_even(ldexpf(a, 10 - E)); /* 1024..2048 */
    /* r == 2048 carries into the exponent field, which is the correct result */
    uint32_t bits = ((uint32_t)(E + 15) << 10) + (r - 1024u);
    return (uint16_t)(sign | bits);
}

/* bf16 ("brain float"): the upper 16 bits of an IEEE binary32 (sign, 8-bit
 * exponent, 7 fraction bits).  Decoding appends 16 zero bits, exactly. */
float zo_decbf16(uint16_t b)
{
    uint32_t bits = (uint32_t)b << 16;
    float out;
    memcpy(&out, &bits, sizeof out);
    return out;
}

/* Encode binary32 as bf16, rounding to nearest, ties to even.  For values of
 * one sign the binary32 encoding is monotonic in the bit pattern, and the bf16
 * values are exactly the binary32 values whose low 16 bits are zero, so
 * rounding the magnitude to the nearest multiple of 2^16 in the integer
 * representation (ties to an even upper half) is rounding the value; a carry
 * out of the fraction moves to the next binade, and past the largest finite
 * value to infinity, as it should.  NaN encodes as the quiet NaN 0x7FC0 with
 * the input's sign. */
uint16_t zo_encbf16(float x)
{
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    if (isnan(x))
        return (uint16_t)(((u >> 16) & 0x8000u) | 0x7FC0u);
    uint32_t upper = u >> 16, lower = u & 0xFFFFu;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))
        upper += 1u;
    return (uint16_t)upper;
}

/* 16-bit formats of the gradient and of the parameter copy */
enum { ZO_FP16 = 0, ZO_BF16 = 1, ZO_FP32 = 2 };

static float dec_fmt(uint16_t h, int32_t fmt) { return fmt == ZO_BF16 ? zo_decbf16(h) : zo_dec16(h); }
static uint16_t enc_fmt(float x, int32_t fmt) { return fmt == ZO_BF16 ? zo_encbf16(x) : zo_enc16(x); }

void zo_decbf16_array(const uint16_t *h, float *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = zo_decbf16(h[i]);
}

void zo_encbf16_array(const float *x, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = zo_encbf16(x[i]);
}

void zo_dec16_array(const uint16_t *h, float *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = zo_dec16(h[i]);
}

void zo_enc16_array(const float *x, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = zo_enc16(x[i]);
}

/* ------------------------------------------------------------------------ */
/* Gradient accumulation ([Overview] core features: gradient accumulation    */
/* sums micro-batch gradients to emulate a larger batch; [Guide] section 5.1 */
/* training loop, backward handles accumulation; section 4.3 batch relation).*/
/* ------------------------------------------------------------------------ */

/* acc[i] = dec(g[i])            when overwrite != 0 (first micro-batch)
 * acc[i] = acc[i] + dec(g[i])   otherwise (later micro-batches, in order)
 * g is fp16 (fmt 0) or bf16 (fmt 1). */
void zo_accumulate(float *acc, const uint16_t *g, int64_t n, int32_t overwrite, int32_t fmt)
{
    for (int64_t i = 0; i < n; ++i) {
        float gi = dec_fmt(g[i], fmt);
        if (overwrite)
            acc[i] = gi;
        else
            acc[i] = acc[i] + gi;
    }
}

/* ------------------------------------------------------------------------ */
/* Overflow check ([Overview] core features: dynamic loss scaling; [Guide]   */
/* section 4.2 fp16 settings and section 13.1 "gradient overflow (fp16)").   */
/* The step overflows when any gradient value is not finite (+-inf or NaN).  */
/* ------------------------------------------------------------------------ */

int32_t zo_any_nonfinite16(const uint16_t *g, int64_t n, int32_t fmt)
{
    int32_t flag = 0;
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(dec_fmt(g[i], fmt)))
            flag = 1;
    return flag;
}

int32_t zo_any_nonfinite32(const float *g, int64_t n)
{
    int32_t flag = 0;
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(g[i]))
            flag = 1;
    return flag;
}

/* ------------------------------------------------------------------------ */
/* Adam (Kingma & Ba, bias-corrected), fp32 state per [Guide] section 2.     */
/* ------------------------------------------------------------------------ */

/* b^t by binary exponentiation: walk the bits of t from the least
 * significant, multiplying the running square into the result for each set
 * bit.  fp64 multiplies only, so any IEEE machine gets the same bits. */
static double pow_by_squaring(double b, int64_t t)
{
    double r = 1.0;
    while (t > 0) {
        if (t & 1)
            r = r * b;
        b = b * b;
        t >>= 1;
    }
    return r;
}

/* Per-step scalars of applied step t (t >= 1):
 *   step_size = lr / (1 - beta1^t)        (folds the first-moment correction)
 *   rbc2      = 1 / sqrt(1 - beta2^t)     (folds the second-moment correction)
 * evaluated in fp64 and rounded once to fp32. */
void zo_adam_scalars(int64_t t, float lr, float beta1, float beta2,
                     float *step_size, float *rbc2)
{
    double b1t = pow_by_squaring((double)beta1, t);
    double b2t = pow_by_squaring((double)beta2, t);
    *step_size = (float)((double)lr / (1.0 - b1t));
    *rbc2 = (float)(1.0 / sqrt(1.0 - b2t));
}

/* zo_adam_scalars for the applied steps t0, t0 + 1, ..., t0 + count - 1:
 * out2[2 j] = step_size, out2[2 j + 1] = rbc2 of step t0 + j. */
void zo_adam_scalars_range(int64_t t0, int64_t count, float lr, float beta1, float beta2, float *out2)
{
    for (int64_t j = 0; j < count; ++j)
        zo_adam_scalars(t0 + j, lr, beta1, beta2, &out2[2 * j], &out2[2 * j + 1]);
}

/* One applied Adam step over n elements of a flat partition.
 *
 * Algorithm (bias-corrected Adam, epsilon outside the square root):
 *   g      = grad / (S * K)                  unscale: loss scale S, K micro-batches
 *   m      = beta1 m + (1 - beta1) g
 *   v      = beta2 v + (1 - beta2) g^2
 *   p      = p - lr wd p                     (decoupled decay, AdamW; skipped when wd == 0)
 *   p      = p - lr/(1-beta1^t) * m / (sqrt(v)/sqrt(1-beta2^t) + eps)
 *   p16    = fp16(p) or bf16(p)              round to nearest even
 * The textbook form m_hat / (sqrt(v_hat) + eps) is regrouped so that each
 * element takes one divide and one square root; the regrouping is exact in
 * real arithmetic.  Each line below is one fp32 rounding, evaluated in the
 * written order.
 *
 * gfmt: grad is fp16 bits (0), bf16 bits (1) or the fp32 accumulation buffer
 * (2); pfmt: the parameter copy is fp16 (0) or bf16 (1).
 * zo_adam_mult takes the gradient multiplier (1/(S*K), or that times the
 * clipping coefficient) as `inv`; zo_adam computes 1/(S*K) itself. */
void zo_adam_mult(const void *grad, int32_t gfmt, int64_t n,
                  float *master, float *m, float *v, uint16_t *p16, int32_t pfmt,
                  float inv, int64_t t,
                  float lr, float beta1, float beta2, float eps, float weight_decay)
{
    float step_size, rbc2;
    zo_adam_scalars(t, lr, beta1, beta2, &step_size, &rbc2);
    float omb1 = 1.0f - beta1;
    float omb2 = 1.0f - beta2;
    float lrwd = lr * weight_decay;

    for (int64_t i = 0; i < n; ++i) {
        float graw = gfmt == ZO_FP32 ? ((const float *)grad)[i]
                                     : dec_fmt(((const uint16_t *)grad)[i], gfmt);
        float g = graw * inv;

        float m1 = beta1 * m[i];
        float m2 = omb1 * g;
        float mi = m1 + m2;

        float gg = g * g;
        float v1 = beta2 * v[i];
        float v2 = omb2 * gg;
        float vi = v1 + v2;

        float p = master[i];
        if (weight_decay != 0.0f) {
            float decay = lrwd * p;
            p = p - decay;
        }
        float root = sqrtf(vi);
        float den0 = root * rbc2;
        float den = den0 + eps;
        float ratio = mi / den;
        float delta = step_size * ratio;
        p = p - delta;

        m[i] = mi;
        v[i] = vi;
        master[i] = p;
        p16[i] = enc_fmt(p, pfmt);
    }
}

/* The unclipped step: the gradient multiplier is 1 / (S * K) in fp32. */
void zo_adam(const void *grad, int32_t gfmt, int64_t n,
             float *master, float *m, float *v, uint16_t *p16, int32_t pfmt,
             float scale, int32_t accum_steps, int64_t t,
             float lr, float beta1, float beta2, float eps, float weight_decay)
{
    float inv = 1.0f / (scale * (float)accum_steps);
    zo_adam_mult(grad, gfmt, n, master, m, v, p16, pfmt, inv, t, lr, beta1, beta2, eps,
                 weight_decay);
}

/* ------------------------------------------------------------------------ */
/* Learning-rate schedules ([Guide] section 4.1, the "scheduler" block with  */
/* WarmupLR; section 4.4, WarmupDecayLR with warmup_min_lr, warmup_max_lr,   */
/* warmup_num_steps, total_num_steps and a linear warmup).  The pages give   */
/* the parameters, not the formula; this is the plain reading of them.       */
/* ------------------------------------------------------------------------ */

enum { ZO_LR_WARMUP = 1, ZO_LR_WARMUP_DECAY = 2 };

/* lr of schedule iteration `it`, the count of Adam steps applied before this
 * one (a fresh run starts at 0; skipped steps do not count).  A fraction
 * gamma in [0, 1] places lr between warmup_min_lr and warmup_max_lr:
 *   while it < warmup:          gamma = it / warmup          (linear rise)
 *   afterwards, WarmupLR:       gamma = 1                    (hold the peak)
 *   afterwards, WarmupDecayLR:  gamma = (total - it) / (total - warmup),
 *                               at least 0; the divisor at least 1
 *   lr = min_lr + (max_lr - min_lr) * gamma
 * all in fp64, rounded once to fp32. */
float zo_lr_schedule(int32_t kind, int64_t it, float min_lr, float max_lr, int64_t warmup,
                     int64_t total)
{
    double gamma = 1.0;
    if (it < warmup) {
        gamma = (double)it / (double)warmup;
    } else if (kind == ZO_LR_WARMUP_DECAY) {
        int64_t span = total - warmup;
        double left = (double)(total - it);
        gamma = left / (double)(span > 1 ? span : 1);
        if (gamma < 0.0)
            gamma = 0.0;
    }
    double lo = (double)min_lr;
    double range = (double)max_lr - lo;
    return (float)(lo + range * gamma);
}

/* ------------------------------------------------------------------------ */
/* Dynamic loss scaler ([Guide] section 4.2 fp16 settings: loss_scale 0 means */
/* dynamic, initial scale 2^initial_scale_power, loss_scale_window counts the */
/* successful steps before an increase, hysteresis counts the overflows      */
/* before a decrease, min_loss_scale is the floor).                           */
/* ------------------------------------------------------------------------ */

typedef struct zo_scaler {
    float scale;        /* S, the loss scale of the next step */
    float min_scale;    /* floor of S */
    int32_t window;     /* successful steps before S doubles */
    int32_t good_steps; /* successful steps since the last overflow or growth */
    int32_t hysteresis; /* overflows needed before S halves */
    int32_t hyst_left;  /* overflows still tolerated before S halves */
    int32_t dynamic;    /* 1: dynamic scaling; 0: S fixed */
    int32_t consecutive_hysteresis; /* 1: a successful step refills hyst_left */
    int64_t applied;    /* Adam steps applied so far (t of the last update) */
    int64_t iters;      /* all steps, applied or skipped */
    int64_t skipped;    /* skipped steps */
} zo_scaler;

void zo_scaler_init(zo_scaler *s, float init_scale, float min_scale, int32_t window,
                    int32_t hysteresis, int32_t dynamic, int32_t consecutive_hysteresis)
{
    s->scale = init_scale;
    s->min_scale = min_scale;
    s->window = window;
    s->good_steps = 0;
    s->hysteresis = hysteresis;
    s->hyst_left = hysteresis;
    s->dynamic = dynamic;
    s->consecutive_hysteresis = consecutive_hysteresis;
    s->applied = 0;
    s->iters = 0;
    s->skipped = 0;
}

/* Advance the scaler past one step whose overflow flag was `overflow`.
 *  overflow: the step was skipped; the success run restarts; with dynamic
 *            scaling one more overflow is charged against the hysteresis and,
 *            once it is used up, S halves (not below the floor) and the
 *            hysteresis restarts.
 *  success : one more applied step; with dynamic scaling the success run
 *            grows and, when it reaches the window, S doubles and the run
 *            restarts. */
void zo_scaler_update(zo_scaler *s, int32_t overflow)
{
    s->iters += 1;
    if (overflow) {
        s->skipped += 1;
        s->good_steps = 0;
        if (s->dynamic) {
            if (s->hyst_left <= 1) {
                float half = s->scale * 0.5f;
                s->scale = half > s->min_scale ? half : s->min_scale;
                s->hyst_left = s->hysteresis;
            } else {
                s->hyst_left -= 1;
            }
        }
    } else {
        s->applied += 1;
        if (s->dynamic) {
            if (s->consecutive_hysteresis)
                s->hyst_left = s->hysteresis;
            s->good_steps += 1;
            if (s->good_steps == s->window) {
                s->scale = s->scale * 2.0f;
                s->good_steps = 0;
            }
        }
    }
}

int64_t zo_scaler_sizeof(void) { return (int64_t)sizeof(zo_scaler); }
