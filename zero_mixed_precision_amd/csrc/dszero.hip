// dszero.hip -- gfx950 (MI355X) kernels and C ABI of the ZeRO mixed-precision
// optimizer step.  Declarations, argument meaning and error behaviour are in
// include/dszero.h.
//
// Pages cited (by title and section):
//   [Guide]    "DeepSpeed complete guide" (youngju.dev, Japanese)
//   [Overview] "DeepSpeed" project overview (aibars.net, Japanese), core features
//
// Every kernel here is a single streaming pass over HBM: the step moves
// 28 bytes per element (fp16 gradient + fp32 master/m/v in, fp32 master/m/v +
// fp16 copy out) for a handful of fp32 operations, so the design goals are
// full-width coalesced accesses and the right amount of traffic in flight,
// not ALU throughput.  Elements are handled in quads of four: each lane moves
// one 16-byte vector per fp32 array (8 bytes per fp16 array) per quad, so
// every wave-wide load or store covers one contiguous 1 KiB (fp32) or 512 B
// (fp16) span.  Each block owns one tile of consecutive quads and issues all
// of the tile's loads before any arithmetic; the grid has one block per tile
// (up to 2^31 work-items per launch, the blocks loop past that), and loads and
// stores are marked non-temporal (streamed data is touched once) on
// partitions above 2^24 elements, whose step traffic is about twice the
// Infinity Cache or more.  Tile shapes, measured on MI355X against each other
// in one process (launch shapes of 64-1024 lanes x 1-4 quads, and 8 elements
// per lane with 16-byte 16-bit accesses, which is 30 % slower for Adam):
//   * Adam: 256 lanes x 4 quads (4096 elements); every shape tried lies within
//     1.5 % of it at 1e8-9e9 elements.  On the smaller, cache-resident
//     partitions the fused Adam kernel covers the same tile with 512 lanes x 2
//     quads.
//   * accumulation (one or several micro-batch gradients into the fp32
//     buffer): one wave, one quad per lane (256 elements): 4-15 % faster than
//     256 x 4 or 512 x 2 on 1.9e8- and 8.75e9-element ranges.  Their
//     sum-of-squares forms take one 1024-element chunk per 256-lane block.
//   * the double-buffered Adam pass: the Adam tile; each block takes one
//     ticket (a 64-bit atomic add on one address, about 12 ns each,
//     serialised), which the 2.1 million blocks of an 8.75e9-element
//     partition hide under the stream but 64 x 1 blocks would not.
//   * the last micro-batches folded into the double-buffered pass: one wave,
//     one quad per lane, like the accumulation (64-512 lanes x 1-2 quads
//     within 4 % at 4e9 elements); it takes no ticket.
// The read-only overflow check uses 1024-lane blocks, one 16-byte vector per
// lane, and ordinary (cache-allocating) loads on purpose: the fp16 gradient
// it reads is read again by the Adam pass right after it, and a partition's
// gradient of up to ~256 MB (e.g. 109M elements) is then served from the
// Infinity Cache instead of HBM (measured: 198 -> 214 Gparams/s per step at
// 109M elements).  Its sum-of-squares form takes 8192-element chunks, 512
// lanes x 2 vectors.
//
// Numerics: IEEE fp32, round to nearest even, one rounding per operation in
// the written order (built with -ffp-contract=off; fp32 division and square
// root are the correctly rounded forms); the bias-correction factors are
// evaluated in fp64 and rounded once; fp16 <-> fp32 conversions are the
// hardware's exact widening and round-to-nearest-even narrowing.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "dszero.h"

#pragma clang fp contract(off)

static_assert(sizeof(ds_scaler) == 128, "ds_scaler must stay 128 bytes");
static_assert(sizeof(ds_lr_schedule) == 32, "ds_lr_schedule is 32 bytes");

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kStepBlock = 256;    // lanes per block of the Adam kernel (4 quads per lane)
// The fused Adam kernel on a cache-resident partition (temporal accesses)
// covers the same 4096-element tile with 512 lanes x 2 quads: twice the waves
// per CU hide more of the latency of a short kernel (step kernel time at 2^20 /
// 2^22 / 2^24 elements: 11.5 / 24.5 / 73.9 us vs 12.0 / 27.4 / 74.8 us with
// 256 x 4); on streamed partitions the two shapes tie or 256 x 4 wins.
constexpr int kSmallBlock = 512;
static_assert(2 * kSmallBlock == 4 * kStepBlock, "both shapes cover one 4096-element tile per block");
constexpr int kCheckBlock = 1024;  // lanes per block of the read-only check
// Accumulation: one wave per block, one quad per lane (256-element tiles).
constexpr int kAccBlock = 64;
constexpr int kFoldAdamBlock = 64;   // fold + double-buffered Adam: lanes per block
constexpr int kFoldAdamUnroll = 1;   // and quads per lane
// Sum-of-squares forms of the accumulation: one chunk of 1024 elements per
// block, 256 lanes x 1 quad.
constexpr int kAccSumsqBlock = 256;
constexpr int64_t kAccChunk = 4 * kAccSumsqBlock;
// Check with the sum of squares: one chunk of 8192 elements per block, 512
// lanes x 2 16-byte vectors (16-bit formats) or 4 (fp32).
constexpr int kCheckSumsqBlock = 512;
constexpr int64_t kCheckChunk = 8192;
// Second pass of the sum of squares: each 256-lane block adds one group of
// 4096 chunk sums (16 per lane, loaded before the adds), the last block to
// finish adds the group sums.
constexpr int kFinishBlock = 256;
constexpr int kFinishPerLane = 16;
constexpr int64_t kGroup = int64_t(kFinishBlock) * kFinishPerLane;
// A dispatch counts its grid in work-items with 32 bits; launches stay within
// 2^31 of them and the kernels loop over the tiles past that.
constexpr int64_t kMaxWorkItems = int64_t(1) << 31;
// Largest n any entry point accepts: 2^40 elements is far beyond one GPU's
// memory (4 TiB of fp32), and keeps every byte count the validation computes
// (at most 16 bytes per element) far from overflowing.
constexpr int64_t kMaxElems = int64_t(1) << 40;

// ---------------------------------------------------------------------------
// memory helpers
// ---------------------------------------------------------------------------

template <bool NT, typename T>
__device__ __forceinline__ T load(const T* p)
{
    if constexpr (NT)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}

template <bool NT, typename T>
__device__ __forceinline__ void store(T* p, T v)
{
    if constexpr (NT)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}

__device__ __forceinline__ float h2f(uint32_t bits)
{
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
}

__device__ __forceinline__ uint32_t f2h(float x)
{
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(x)));
}

// Element formats: 16-bit arrays are fp16 (IEEE binary16) or bf16 (the top
// half of a binary32); gradients may also be fp32 (the accumulation buffer).
constexpr int kF16 = 0, kBF16 = 1, kF32 = 2;

// bf16 -> fp32 is exact (append 16 zero bits); fp32 -> bf16 rounds to nearest
// even (hardware conversion).
__device__ __forceinline__ uint32_t f2bf(float x)
{
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(x)));
}

template <int FMT>
__device__ __forceinline__ float dec1(uint32_t bits)
{
    if constexpr (FMT == kBF16)
        return __uint_as_float((bits & 0xFFFFu) << 16);
    else
        return h2f(bits);
}

template <int FMT>
__device__ __forceinline__ uint32_t enc1(float x)
{
    if constexpr (FMT == kBF16)
        return f2bf(x);
    else
        return f2h(x);
}

template <int FMT>
__device__ __forceinline__ f32x4 widen4(u32x2 w)
{
    if constexpr (FMT == kBF16)
        return f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                     __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u)};
    else
        return f32x4{h2f(w.x & 0xFFFFu), h2f(w.x >> 16), h2f(w.y & 0xFFFFu), h2f(w.y >> 16)};
}

template <int FMT>
__device__ __forceinline__ u32x2 narrow4(f32x4 p)
{
    return u32x2{enc1<FMT>(p.x) | (enc1<FMT>(p.y) << 16), enc1<FMT>(p.z) | (enc1<FMT>(p.w) << 16)};
}

// Non-finite tests on raw bits: an exponent field of all ones is +-inf or NaN.
// Adding one unit to an all-ones exponent carries into the sign position, and
// into nothing else, so one add and one mask test both halves of a word.
__device__ __forceinline__ uint32_t nonfinite_f16x2(uint32_t w)
{
    return ((w & 0x7C007C00u) + 0x04000400u) & 0x80008000u;
}

__device__ __forceinline__ uint32_t nonfinite_bf16x2(uint32_t w)
{
    return ((w & 0x7F807F80u) + 0x00800080u) & 0x80008000u;
}

template <int FMT>
__device__ __forceinline__ uint32_t nonfinite16x2(uint32_t w)
{
    if constexpr (FMT == kBF16)
        return nonfinite_bf16x2(w);
    else
        return nonfinite_f16x2(w);
}

__device__ __forceinline__ uint32_t nonfinite_f32(uint32_t w)
{
    return ((w & 0x7F800000u) + 0x00800000u) & 0x80000000u;
}

__device__ __forceinline__ uint32_t nonfinite_f32x4(f32x4 x)
{
    return nonfinite_f32(__float_as_uint(x.x)) | nonfinite_f32(__float_as_uint(x.y)) |
           nonfinite_f32(__float_as_uint(x.z)) | nonfinite_f32(__float_as_uint(x.w));
}

// One atomic OR per wave that saw a non-finite value, issued by the lowest
// lane that saw one.
__device__ __forceinline__ void raise_flag(ds_scaler* st, uint32_t bad)
{
    const uint64_t mask = __ballot(bad != 0u);
    if (mask != 0ull && __lane_id() == static_cast<unsigned>(__ffsll(static_cast<long long>(mask)) - 1))
        atomicOr(&st->overflow, 1u);
}

// ---------------------------------------------------------------------------
// gradient sum of squares (global-norm clipping), deterministic
// ---------------------------------------------------------------------------

// Sum over a block in a fixed order: a fixed xor butterfly inside each wave,
// then the TPB / 64 wave sums combined by a fixed butterfly in the first wave.
// The result is meaningful in thread 0.  Every thread of the block must call
// it.  One barrier per call: `lds` holds two buffers of TPB / 64 doubles and
// consecutive calls of a block alternate `parity`, so a call never writes the
// buffer the previous call may still be reading.
template <int TPB>
__device__ __forceinline__ double block_sum_fixed(double x, double* lds, int parity)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        x = x + __shfl_xor(x, off);
    constexpr int kWaves = TPB / 64;
    if constexpr (kWaves == 1) {
        return x;
    } else {
        double* buf = lds + parity * kWaves;
        if ((threadIdx.x & 63) == 0)
            buf[threadIdx.x >> 6] = x;
        __syncthreads();
        double t = 0.0;
        if (threadIdx.x < 64) {
            t = threadIdx.x < kWaves ? buf[threadIdx.x] : 0.0;
#pragma unroll
            for (int off = kWaves / 2; off > 0; off >>= 1)
                t = t + __shfl_xor(t, off);
        }
        return t;
    }
}

__device__ __forceinline__ double sq(float x)
{
    const double d = static_cast<double>(x);
    return d * d;  // exact: a 24-bit significand squared fits in 53 bits
}

__device__ __forceinline__ double sq4(const f32x4& x)
{
    return ((sq(x.x) + sq(x.y)) + sq(x.z)) + sq(x.w);
}

// sq4 for values whose squares are exact in fp32 (widened fp16): the same
// result, with the squares taken in fp32.
__device__ __forceinline__ double sq4_exact32(const f32x4& x)
{
    return ((static_cast<double>(x.x * x.x) + static_cast<double>(x.y * x.y)) + static_cast<double>(x.z * x.z)) +
           static_cast<double>(x.w * x.w);
}

// Second pass of the sum of squares over the nparts chunk sums in part[]:
// block g adds group g (chunk sums g * kGroup ... + kGroup - 1; lane l takes
// j * kFinishBlock + l of the group for j = 0..15, in j order, then the fixed
// block sum) into part2[g]; every block then takes a ticket, and the block
// that takes the last one adds the group sums in a fixed order into
// st->grad_sumsq and sets the ticket count back to 0.  The chunking is fixed
// by n, so the result depends on neither grid.  The fences order each
// block's group sum before its ticket, and the last block's reads after it
// (the L2 caches of the XCDs are not coherent with one another).
__global__ __launch_bounds__(kFinishBlock) void sumsq_finish_kernel(ds_scaler* __restrict__ st,
                                                                    const double* __restrict__ part,
                                                                    int64_t nparts, double* part2)
{
    __shared__ double lds[2 * (kFinishBlock / 64)];
    __shared__ uint32_t is_last;
    const int64_t ngroups = (nparts + kGroup - 1) / kGroup;
    int parity = 0;
    for (int64_t g = blockIdx.x; g < ngroups; g += gridDim.x) {
        double x[kFinishPerLane];
#pragma unroll
        for (int j = 0; j < kFinishPerLane; ++j) {
            const int64_t i = g * kGroup + static_cast<int64_t>(j) * kFinishBlock + threadIdx.x;
            x[j] = i < nparts ? part[i] : 0.0;
        }
        double s = 0.0;
#pragma unroll
        for (int j = 0; j < kFinishPerLane; ++j)
            s = s + x[j];
        s = block_sum_fixed<kFinishBlock>(s, lds, parity);
        parity ^= 1;
        if (threadIdx.x == 0)
            part2[g] = s;
    }
    if (threadIdx.x == 0) {
        __threadfence();
        is_last = atomicAdd(&st->sumsq_blocks_done, 1u) == gridDim.x - 1u ? 1u : 0u;
    }
    __syncthreads();
    if (is_last) {
        __threadfence();
        double s = 0.0;
        for (int64_t g = threadIdx.x; g < ngroups; g += kFinishBlock)
            s = s + part2[g];
        s = block_sum_fixed<kFinishBlock>(s, lds, parity);
        if (threadIdx.x == 0) {
            st->grad_sumsq = st->grad_sumsq + s;
            st->sumsq_blocks_done = 0u;
        }
    }
}

// ---------------------------------------------------------------------------
// loss-scaler state machine ([Guide] section 4.2), one work-item
// ---------------------------------------------------------------------------

__device__ __forceinline__ void advance_scaler_with(ds_scaler* st, uint32_t flag)
{
    ds_scaler s = *st;
    const uint32_t ov = flag != 0u ? 1u : 0u;
    s.iter += 1;
    if (ov) {
        s.skipped += 1;
        s.growth_count = 0;
        if (s.dynamic) {
            if (s.hysteresis_left <= 1) {
                const float half = s.scale * 0.5f;
                s.scale = half > s.min_scale ? half : s.min_scale;
                s.hysteresis_left = s.hysteresis;
            } else {
                s.hysteresis_left -= 1;
            }
        }
    } else {
        s.step += 1;
        if (s.dynamic) {
            if (s.consecutive_hysteresis)
                s.hysteresis_left = s.hysteresis;
            s.growth_count += 1;
            if (s.growth_count == s.growth_window) {
                s.scale = s.scale * 2.0f;
                s.growth_count = 0;
            }
        }
    }
    s.last_overflow = ov;
    s.overflow = 0u;
    s.last_grad_sumsq = s.grad_sumsq;
    s.grad_sumsq = 0.0;
    *st = s;
}

__device__ __forceinline__ void advance_scaler(ds_scaler* st) { advance_scaler_with(st, st->overflow); }

__global__ void update_scale_kernel(ds_scaler* st) { advance_scaler(st); }

// The double-buffered step's scaler update on an empty partition: advance,
// and make the other copy current if the step applied.
__global__ void update_scale_swap_kernel(ds_scaler* st)
{
    const uint32_t ov = st->overflow;
    const uint32_t cur = st->current & 1u;
    advance_scaler_with(st, ov);
    if (ov == 0u)
        st->current = cur ^ 1u;
}

// ---------------------------------------------------------------------------
// Adam
// ---------------------------------------------------------------------------

struct AdamHyper {
    float lr, beta1, beta2, eps, weight_decay, max_grad_norm;
    int32_t accum_steps;
    // learning-rate schedule (lr_kind 0: the constant lr above; else a
    // ds_lr_kind, with lr playing warmup_max_lr)
    int32_t lr_kind;
    float lr_min;
    int64_t lr_warmup, lr_total;
};

struct AdamConsts {
    float inv;        // 1 / (S * K), times the clipping coefficient when clipping
    float b1, b2;     // beta1, beta2
    float omb1, omb2; // 1 - beta1, 1 - beta2
    float lrwd;       // lr * weight_decay
    float step_size;  // lr / (1 - beta1^t)
    float rbc2;       // 1 / sqrt(1 - beta2^t)
    float eps;
};

// beta1^t and beta2^t by binary exponentiation over the bits of t, least
// significant first (fp64 multiplies only), then the two bias-correction
// factors in fp64, each rounded once to fp32.
__device__ __forceinline__ void bias_scalars(int64_t t, float lr, float beta1, float beta2,
                                             float* step_size, float* rbc2)
{
    double r1 = 1.0, r2 = 1.0, x1 = static_cast<double>(beta1), x2 = static_cast<double>(beta2);
    for (int64_t e = t; e > 0; e >>= 1) {
        if (e & 1) {
            r1 = r1 * x1;
            r2 = r2 * x2;
        }
        x1 = x1 * x1;
        x2 = x2 * x2;
    }
    *step_size = static_cast<float>(static_cast<double>(lr) / (1.0 - r1));
    *rbc2 = static_cast<float>(1.0 / sqrt(1.0 - r2));
}

// Learning rate of schedule iteration `it` (Adam steps applied before this
// one): gamma in [0, 1] rises linearly over the warmup, then holds at 1
// (WarmupLR) or falls linearly to 0 at lr_total (WarmupDecayLR);
// lr = lr_min + (lr_max - lr_min) * gamma in fp64, rounded once.
__device__ __forceinline__ float schedule_lr(int64_t it, const AdamHyper& h)
{
    double gamma = 1.0;
    if (it < h.lr_warmup) {
        gamma = static_cast<double>(it) / static_cast<double>(h.lr_warmup);
    } else if (h.lr_kind == DS_LR_WARMUP_DECAY) {
        const int64_t span = h.lr_total - h.lr_warmup;
        const double left = static_cast<double>(h.lr_total - it);
        gamma = left / static_cast<double>(span > 1 ? span : 1);
        if (gamma < 0.0)
            gamma = 0.0;
    }
    const double lo = static_cast<double>(h.lr_min);
    const double range = static_cast<double>(h.lr) - lo;
    return static_cast<float>(lo + range * gamma);
}

__device__ __forceinline__ float step_lr(const ds_scaler* st, const AdamHyper& h)
{
    return h.lr_kind == 0 ? h.lr : schedule_lr(st->step, h);
}

__device__ __forceinline__ AdamConsts make_consts(const ds_scaler* st, const AdamHyper& h)
{
    AdamConsts c;
    const float lr = step_lr(st, h);
    c.inv = 1.0f / (st->scale * static_cast<float>(h.accum_steps));
    if (h.max_grad_norm > 0.0f) {
        // global-norm clipping of the unscaled gradient
        const double inv64 = static_cast<double>(c.inv);
        const double norm = sqrt(st->grad_sumsq) * inv64;
        const double ratio = static_cast<double>(h.max_grad_norm) / (norm + 1e-6);
        const double coef = ratio < 1.0 ? ratio : 1.0;
        c.inv = static_cast<float>(inv64 * coef);
    }
    c.b1 = h.beta1;
    c.b2 = h.beta2;
    c.omb1 = 1.0f - h.beta1;
    c.omb2 = 1.0f - h.beta2;
    c.lrwd = lr * h.weight_decay;
    c.eps = h.eps;
    bias_scalars(st->step + 1, lr, h.beta1, h.beta2, &c.step_size, &c.rbc2);
    return c;
}

// One element, [Guide] section 2 state: fp32 master p, moments m and v.
template <bool WD>
__device__ __forceinline__ void adam1(float graw, float& p, float& m, float& v, const AdamConsts& c)
{
    const float g = graw * c.inv;
    const float m1 = c.b1 * m;
    const float m2 = c.omb1 * g;
    m = m1 + m2;
    const float gg = g * g;
    const float v1 = c.b2 * v;
    const float v2 = c.omb2 * gg;
    v = v1 + v2;
    if constexpr (WD) {
        const float decay = c.lrwd * p;
        p = p - decay;
    }
    const float root = sqrtf(v);
    const float den0 = root * c.rbc2;
    const float den = den0 + c.eps;
    const float ratio = m / den;
    const float delta = c.step_size * ratio;
    p = p - delta;
}

template <bool WD>
__device__ __forceinline__ void adam4(const f32x4& g, f32x4& p, f32x4& m, f32x4& v, const AdamConsts& c)
{
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        float pk = p[k], mk = m[k], vk = v[k];
        adam1<WD>(g[k], pk, mk, vk, c);
        p[k] = pk;
        m[k] = mk;
        v[k] = vk;
    }
}

template <int GF, bool NT>
__device__ __forceinline__ f32x4 load_grad4(const void* grad, int64_t q)
{
    if constexpr (GF == kF32)
        return load<NT>(static_cast<const f32x4*>(grad) + q);
    else
        return widen4<GF>(load<NT>(static_cast<const u32x2*>(grad) + q));
}

template <int GF>
__device__ __forceinline__ float load_grad1(const void* grad, int64_t i)
{
    if constexpr (GF == kF32)
        return static_cast<const float*>(grad)[i];
    else
        return dec1<GF>(static_cast<const uint16_t*>(grad)[i]);
}

// Gated fused step: if the step's overflow flag is set, write nothing; else
// update every element of [0, n) once.  Tiles of U x TPB quads are dealt to
// blocks round-robin; block 0 also takes the quads of the last, partial tile
// and the final n % 4 elements.  With FUSE the kernel also ends the step:
// every block, when done (whether or not the step is skipped), takes a ticket
// from st->blocks_done with one atomic add, and the block that takes the last
// ticket, after every other block has read the scaler state, advances the
// scaler (as update_scale_kernel does) and resets the count.  No block waits
// for another.
template <int GF, int PF, bool WD, bool NT, int TPB, int U, bool FUSE>
__global__ __launch_bounds__(TPB) void adam_kernel(ds_scaler* __restrict__ st,
                                                   float* __restrict__ master,
                                                   float* __restrict__ mom1,
                                                   float* __restrict__ mom2,
                                                   uint16_t* __restrict__ p16,
                                                   const void* __restrict__ grad, int64_t n,
                                                   AdamHyper hp)
{
    if (st->overflow == 0u) {
        const AdamConsts c = make_consts(st, hp);

        f32x4* P = reinterpret_cast<f32x4*>(master);
        f32x4* M = reinterpret_cast<f32x4*>(mom1);
        f32x4* V = reinterpret_cast<f32x4*>(mom2);
        u32x2* H = reinterpret_cast<u32x2*>(p16);

        constexpr int T = U * TPB;  // quads per tile
        const int64_t nq = n >> 2;
        const int64_t ntiles = nq / T;
        for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
            const int64_t q0 = tile * T + threadIdx.x;
            f32x4 g[U], p[U], m[U], v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = q0 + u * TPB;
                g[u] = load_grad4<GF, NT>(grad, i);
                p[u] = load<NT>(P + i);
                m[u] = load<NT>(M + i);
                v[u] = load<NT>(V + i);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = q0 + u * TPB;
                adam4<WD>(g[u], p[u], m[u], v[u], c);
                store<NT>(P + i, p[u]);
                store<NT>(M + i, m[u]);
                store<NT>(V + i, v[u]);
                store<NT>(H + i, narrow4<PF>(p[u]));
            }
        }
        if (blockIdx.x == 0) {
            for (int64_t q = ntiles * T + threadIdx.x; q < nq; q += TPB) {
                f32x4 g = load_grad4<GF, NT>(grad, q);
                f32x4 p = load<NT>(P + q), m = load<NT>(M + q), v = load<NT>(V + q);
                adam4<WD>(g, p, m, v, c);
                store<NT>(P + q, p);
                store<NT>(M + q, m);
                store<NT>(V + q, v);
                store<NT>(H + q, narrow4<PF>(p));
            }
            if (static_cast<int64_t>(threadIdx.x) < (n & 3)) {
                const int64_t i = (nq << 2) + threadIdx.x;
                float p = master[i], m = mom1[i], v = mom2[i];
                adam1<WD>(load_grad1<GF>(grad, i), p, m, v, c);
                master[i] = p;
                mom1[i] = m;
                mom2[i] = v;
                p16[i] = static_cast<uint16_t>(enc1<PF>(p));
            }
        }
    }
    if constexpr (FUSE) {
        // every lane of this block has read the scaler state (make_consts) by now
        __syncthreads();
        if (threadIdx.x == 0 && atomicAdd(&st->blocks_done, 1u) == gridDim.x - 1u) {
            st->blocks_done = 0u;
            advance_scaler(st);
        }
    }
}

// Double-buffered step (ds_adam_step_double_buffered): copies 0 and 1 of
// master, m, v and the 16-bit parameter copy; st->current names the copy that
// holds the state.  One pass reads the gradient and the current copy, ORs the
// gradient's non-finite test into the flag (the overflow check, fused: it needs
// no pass of its own because nothing is written to the current copy) and writes
// the update into the other copy.  Every block then takes a ticket; the block
// with the last one reads the step's flag, advances the scaler and, if the step
// applied, makes the other copy current.  A block's flag travels in its
// ticket (one 64-bit atomic add on st->db_tickets: one in the low half, and
// one in the high half if the block saw a non-finite value), so the last
// block reads every block's finding from the value its own add returns and no
// block needs a memory fence.  A flag raised before the call (st->overflow)
// also skips the step.
// Same tiling and arithmetic as adam_kernel.
struct DbArrays {
    float* master[2];
    float* m[2];
    float* v[2];
    uint16_t* p16[2];
};

template <int GF, int PF, bool WD, bool NT, int TPB, int U>
__global__ __launch_bounds__(TPB) void adam_db_kernel(ds_scaler* __restrict__ st, DbArrays a,
                                                      const void* __restrict__ grad, int64_t n, AdamHyper hp)
{
    const AdamConsts c = make_consts(st, hp);
    const uint32_t cur = st->current & 1u;
    const f32x4* P = reinterpret_cast<const f32x4*>(cur ? a.master[1] : a.master[0]);
    const f32x4* M = reinterpret_cast<const f32x4*>(cur ? a.m[1] : a.m[0]);
    const f32x4* V = reinterpret_cast<const f32x4*>(cur ? a.v[1] : a.v[0]);
    f32x4* Po = reinterpret_cast<f32x4*>(cur ? a.master[0] : a.master[1]);
    f32x4* Mo = reinterpret_cast<f32x4*>(cur ? a.m[0] : a.m[1]);
    f32x4* Vo = reinterpret_cast<f32x4*>(cur ? a.v[0] : a.v[1]);
    uint16_t* p16o = cur ? a.p16[0] : a.p16[1];
    u32x2* H = reinterpret_cast<u32x2*>(p16o);

    constexpr int T = U * TPB;  // quads per tile
    const int64_t nq = n >> 2;
    const int64_t ntiles = nq / T;
    uint32_t bad = 0u;
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int64_t q0 = tile * T + threadIdx.x;
        f32x4 g[U], p[U], m[U], v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = q0 + u * TPB;
            g[u] = load_grad4<GF, NT>(grad, i);
            p[u] = load<NT>(P + i);
            m[u] = load<NT>(M + i);
            v[u] = load<NT>(V + i);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = q0 + u * TPB;
            bad |= nonfinite_f32x4(g[u]);
            adam4<WD>(g[u], p[u], m[u], v[u], c);
            store<NT>(Po + i, p[u]);
            store<NT>(Mo + i, m[u]);
            store<NT>(Vo + i, v[u]);
            store<NT>(H + i, narrow4<PF>(p[u]));
        }
    }
    if (blockIdx.x == 0) {
        for (int64_t q = ntiles * T + threadIdx.x; q < nq; q += TPB) {
            f32x4 g = load_grad4<GF, NT>(grad, q);
            f32x4 p = load<NT>(P + q), m = load<NT>(M + q), v = load<NT>(V + q);
            bad |= nonfinite_f32x4(g);
            adam4<WD>(g, p, m, v, c);
            store<NT>(Po + q, p);
            store<NT>(Mo + q, m);
            store<NT>(Vo + q, v);
            store<NT>(H + q, narrow4<PF>(p));
        }
        if (static_cast<int64_t>(threadIdx.x) < (n & 3)) {
            const int64_t i = (nq << 2) + threadIdx.x;
            const float* ps = reinterpret_cast<const float*>(P);
            const float* ms = reinterpret_cast<const float*>(M);
            const float* vs = reinterpret_cast<const float*>(V);
            float p = ps[i], m = ms[i], v = vs[i];
            const float g = load_grad1<GF>(grad, i);
            bad |= nonfinite_f32(__float_as_uint(g));
            adam1<WD>(g, p, m, v, c);
            reinterpret_cast<float*>(Po)[i] = p;
            reinterpret_cast<float*>(Mo)[i] = m;
            reinterpret_cast<float*>(Vo)[i] = v;
            p16o[i] = static_cast<uint16_t>(enc1<PF>(p));
        }
    }
    // One ticket per block, carrying the block's flag: each wave's OR goes to
    // LDS; once the barrier has passed every lane has read the scaler state.
    __shared__ uint32_t wave_bad[TPB / 64];
    const bool wave_any = __ballot(bad != 0u) != 0ull;
    if (__lane_id() == 0u)
        wave_bad[threadIdx.x / 64] = wave_any ? 1u : 0u;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t block_bad = 0u;
#pragma unroll
        for (int w = 0; w < TPB / 64; ++w)
            block_bad |= wave_bad[w];
        const unsigned long long mine = 1ull | (block_bad ? (1ull << 32) : 0ull);
        const unsigned long long before =
            atomicAdd(reinterpret_cast<unsigned long long*>(&st->db_tickets), mine);
        if (static_cast<uint32_t>(before) == gridDim.x - 1u) {
            const uint32_t ov = ((before + mine) >> 32) != 0ull || st->overflow != 0u ? 1u : 0u;
            st->db_tickets = 0ull;
            advance_scaler_with(st, ov);
            if (ov == 0u)
                st->current = cur ^ 1u;
        }
    }
}

__global__ void bias_scalars_kernel(const ds_scaler* st, float lr, float beta1, float beta2, float* out2)
{
    float a, b;
    bias_scalars(st->step + 1, lr, beta1, beta2, &a, &b);
    out2[0] = a;
    out2[1] = b;
}

__global__ void lr_scalars_kernel(const ds_scaler* st, AdamHyper hp, float* out3)
{
    const float lr = step_lr(st, hp);
    float a, b;
    bias_scalars(st->step + 1, lr, hp.beta1, hp.beta2, &a, &b);
    out3[0] = lr;
    out3[1] = a;
    out3[2] = b;
}

// ---------------------------------------------------------------------------
// overflow check
// ---------------------------------------------------------------------------

// fp16/bf16: 8 elements per 16-byte vector; fp32: 4.  One vector per lane per
// grid-stride step; block 0 also tests the elements after the last vector.
template <int GF, bool NT, int TPB>
__global__ __launch_bounds__(TPB) void check_kernel(ds_scaler* __restrict__ st,
                                                    const void* __restrict__ grad, int64_t n)
{
    if (st->overflow != 0u)
        return;  // already decided for this step
    constexpr bool F32 = GF == kF32;
    constexpr int kPer = F32 ? 4 : 8;
    const u32x4* G = static_cast<const u32x4*>(grad);
    const int64_t nv = n / kPer;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * TPB;
    uint32_t bad = 0u;
    for (int64_t q = static_cast<int64_t>(blockIdx.x) * TPB + threadIdx.x; q < nv; q += stride) {
        const u32x4 w = load<NT>(G + q);
        if constexpr (F32)
            bad |= nonfinite_f32(w.x) | nonfinite_f32(w.y) | nonfinite_f32(w.z) | nonfinite_f32(w.w);
        else
            bad |= nonfinite16x2<GF>(w.x) | nonfinite16x2<GF>(w.y) | nonfinite16x2<GF>(w.z) |
                   nonfinite16x2<GF>(w.w);
    }
    if (blockIdx.x == 0 && static_cast<int64_t>(threadIdx.x) < n - nv * kPer) {
        const int64_t i = nv * kPer + threadIdx.x;
        if constexpr (F32)
            bad |= nonfinite_f32(static_cast<const uint32_t*>(grad)[i]);
        else
            bad |= nonfinite16x2<GF>(static_cast<const uint16_t*>(grad)[i]);
    }
    raise_flag(st, bad);
}

// Overflow check plus the chunk sums of squares.  A chunk is kCheckChunk =
// 8192 elements, TPB = 512 lanes x kVecs 16-byte vectors (16-bit formats: 2
// vectors of 8, fp32: 4 of 4); vector j of lane l is vector j * TPB + l of
// the chunk, so each of the kVecs loads is one contiguous span across the
// block, and each lane sums its elements in order.  An fp16 value squared is
// exact in fp32 (at most 22 significant bits, between 2^-48 and 65504^2), so
// fp16 squares are taken in fp32 and widened for the fp64 sum -- the same
// values as fp64 squares, for less fp64 work; bf16 and fp32 squares are taken
// in fp64.  One block per chunk; measured at 8.75e9 elements in one process:
// 6.5 TB/s, against 6.1-6.2 with 1024 lanes x 2 vectors per 16,384 elements
// and a two-barrier block sum, 6.3-6.5 with chunks of one wave (no barrier)
// and 6.8 for the plain check.
// One 16-byte vector of the gradient: ORs its non-finite test into `bad` and
// adds the sums of its squares to `s`, four elements at a time in element
// order.
template <int GF>
__device__ __forceinline__ void check_sq_vec(const u32x4& w, uint32_t& bad, double& s)
{
    if constexpr (GF == kF32) {
        bad |= nonfinite_f32(w.x) | nonfinite_f32(w.y) | nonfinite_f32(w.z) | nonfinite_f32(w.w);
        s = s + sq4(f32x4{__uint_as_float(w.x), __uint_as_float(w.y), __uint_as_float(w.z), __uint_as_float(w.w)});
    } else {
        bad |= nonfinite16x2<GF>(w.x) | nonfinite16x2<GF>(w.y) | nonfinite16x2<GF>(w.z) | nonfinite16x2<GF>(w.w);
        const f32x4 a = widen4<GF>(u32x2{w.x, w.y});
        const f32x4 b = widen4<GF>(u32x2{w.z, w.w});
        if constexpr (GF == kF16) {
            s = s + sq4_exact32(a);
            s = s + sq4_exact32(b);
        } else {
            s = s + sq4(a);
            s = s + sq4(b);
        }
    }
}

template <int GF, int TPB>
__global__ __launch_bounds__(TPB) void check_sumsq_kernel(ds_scaler* __restrict__ st,
                                                          const void* __restrict__ grad, int64_t n,
                                                          double* __restrict__ part)
{
    constexpr bool F32 = GF == kF32;
    constexpr int kPer = F32 ? 4 : 8;
    constexpr int kVecs = static_cast<int>(kCheckChunk / (static_cast<int64_t>(TPB) * kPer));
    static_assert(static_cast<int64_t>(TPB) * kVecs * kPer == kCheckChunk, "one chunk per block");
    __shared__ double lds[2 * (TPB / 64)];
    const u32x4* G = static_cast<const u32x4*>(grad);
    const int64_t nfull = n / kCheckChunk;
    uint32_t bad = 0u;
    int parity = 0;
    // whole chunks: every vector in bounds, all loads issued before the arithmetic
    for (int64_t c = blockIdx.x; c < nfull; c += gridDim.x) {
        const int64_t v0 = c * (kCheckChunk / kPer) + threadIdx.x;
        double s = 0.0;
        u32x4 w[kVecs];
#pragma unroll
        for (int j = 0; j < kVecs; ++j)
            w[j] = G[v0 + static_cast<int64_t>(j) * TPB];
#pragma unroll
        for (int j = 0; j < kVecs; ++j)
            check_sq_vec<GF>(w[j], bad, s);
        const double cs = block_sum_fixed<TPB>(s, lds, parity);
        parity ^= 1;
        if (threadIdx.x == 0)
            part[c] = cs;
    }
    // the last, partial chunk, by block 0 after its whole chunks: whole vectors
    // as above, then element by element (kept out of the loop above, where the
    // extra paths cost the whole-chunk pass 9 % in time)
    if (blockIdx.x == 0 && nfull * kCheckChunk < n) {
        const int64_t v0 = nfull * (kCheckChunk / kPer) + threadIdx.x;
        double s = 0.0;
        for (int j = 0; j < kVecs; ++j) {
            const int64_t v = v0 + static_cast<int64_t>(j) * TPB;
            if ((v + 1) * kPer <= n) {
                check_sq_vec<GF>(G[v], bad, s);
            } else {
                for (int k = 0; k < kPer; ++k) {
                    const int64_t i = v * kPer + k;
                    if (i < n) {
                        if constexpr (F32) {
                            const uint32_t bits = static_cast<const uint32_t*>(grad)[i];
                            bad |= nonfinite_f32(bits);
                            s = s + sq(__uint_as_float(bits));
                        } else {
                            const uint32_t bits = static_cast<const uint16_t*>(grad)[i];
                            bad |= nonfinite16x2<GF>(bits);
                            s = s + sq(dec1<GF>(bits));
                        }
                    }
                }
            }
        }
        const double cs = block_sum_fixed<TPB>(s, lds, parity);
        if (threadIdx.x == 0)
            part[nfull] = cs;
    }
    raise_flag(st, bad);
}

// ---------------------------------------------------------------------------
// gradient accumulation
// ---------------------------------------------------------------------------

// count (1..8) micro-batch gradients folded into the fp32 buffer in one
// pass: acc = (OVERWRITE ? g_0 : acc + g_0) + g_1 + ... + g_{count-1}, every
// add an fp32 add in this order, so the result is bit for bit that of count
// consecutive single-gradient passes, for 2 * count + 8 (or + 4 when
// overwriting) bytes per element instead of 10 * count.  One quad per lane,
// one tile of TPB quads per block, every gradient's loads issued before the
// first add.  With CHECK the pass ORs "a result is not finite" into the
// overflow flag; with SUMSQ (which needs CHECK and a tile of kAccChunk
// elements) each tile is one chunk of the sum of squares of the result,
// written to part[tile].  The gradient list is indexed with compile-time
// indices only (no dynamic indexing of the kernel argument, so no scratch).
constexpr int kMaxFold = 8;
struct GradList {
    const uint16_t* p[kMaxFold];
    int32_t count;
};

// One quad of a fold of F gradients (F known at compile time): the loads of
// the accumulation buffer and of every gradient are issued before the adds.
template <int GF, bool OVERWRITE, bool NT, int F>
__device__ __forceinline__ f32x4 fold_quad(f32x4* A, const GradList& gl, int64_t q)
{
    f32x4 r;
    if constexpr (!OVERWRITE)
        r = load<NT>(A + q);
    u32x2 raw[F];
#pragma unroll
    for (int k = 0; k < F; ++k)
        raw[k] = load<NT>(reinterpret_cast<const u32x2*>(gl.p[k]) + q);
    if constexpr (OVERWRITE)
        r = widen4<GF>(raw[0]);
    else
        r = r + widen4<GF>(raw[0]);
#pragma unroll
    for (int k = 1; k < F; ++k)
        r = r + widen4<GF>(raw[k]);
    return r;
}

// The pass over [0, n) for a fold of F gradients: tiles of TPB quads dealt to
// blocks round-robin; block 0 also takes the quads after the last whole tile
// (fewer than TPB) and the last n % 4 elements.
template <int GF, bool OVERWRITE, bool CHECK, bool SUMSQ, bool NT, int TPB, int F>
__device__ __forceinline__ void accumulate_pass(float* __restrict__ acc, const GradList& gl, int64_t n,
                                                ds_scaler* __restrict__ st, double* __restrict__ part, double* lds)
{
    f32x4* A = reinterpret_cast<f32x4*>(acc);
    const int64_t nq = n >> 2;
    const int64_t ntiles = nq / TPB;
    uint32_t bad = 0u;
    int parity = 0;
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int64_t q = tile * TPB + threadIdx.x;
        const f32x4 r = fold_quad<GF, OVERWRITE, NT, F>(A, gl, q);
        if constexpr (CHECK)
            bad |= nonfinite_f32x4(r);
        store<NT>(A + q, r);
        if constexpr (SUMSQ) {
            const double cs = block_sum_fixed<TPB>(sq4(r), lds, parity);
            parity ^= 1;
            if (threadIdx.x == 0)
                part[tile] = cs;
        }
    }
    if (blockIdx.x == 0) {
        double s = 0.0;
        const int64_t q = ntiles * TPB + threadIdx.x;
        if (q < nq) {
            const f32x4 r = fold_quad<GF, OVERWRITE, NT, F>(A, gl, q);
            if constexpr (CHECK)
                bad |= nonfinite_f32x4(r);
            if constexpr (SUMSQ)
                s = s + sq4(r);
            store<NT>(A + q, r);
        }
        if (static_cast<int64_t>(threadIdx.x) < (n & 3)) {
            const int64_t i = (nq << 2) + threadIdx.x;
            float r = dec1<GF>(gl.p[0][i]);
            if constexpr (!OVERWRITE)
                r = acc[i] + r;
#pragma unroll
            for (int k = 1; k < F; ++k)
                r = r + dec1<GF>(gl.p[k][i]);
            if constexpr (CHECK)
                bad |= nonfinite_f32(__float_as_uint(r));
            if constexpr (SUMSQ)
                s = s + sq(r);
            acc[i] = r;
        }
        if constexpr (SUMSQ) {
            if (ntiles * TPB * 4 < n) {          // a last, partial chunk exists
                const double cs = block_sum_fixed<TPB>(s, lds, parity);
                if (threadIdx.x == 0)
                    part[ntiles] = cs;
            }
        }
    }
    if constexpr (CHECK)
        raise_flag(st, bad);
}

// MULTI = false: exactly one gradient.  MULTI = true: gl.count (2..8)
// gradients, the pass chosen by a block-uniform switch, so every form is
// straight-line code with all of its loads in flight together.
template <int GF, bool OVERWRITE, bool CHECK, bool SUMSQ, bool NT, bool MULTI, int TPB>
__global__ __launch_bounds__(TPB) void accumulate_kernel(float* __restrict__ acc, GradList gl, int64_t n,
                                                         ds_scaler* __restrict__ st, double* __restrict__ part)
{
    static_assert(!SUMSQ || (CHECK && 4 * TPB == kAccChunk), "a tile is one chunk");
    __shared__ double lds[SUMSQ ? 2 * (TPB / 64) : 1];
    if constexpr (!MULTI) {
        accumulate_pass<GF, OVERWRITE, CHECK, SUMSQ, NT, TPB, 1>(acc, gl, n, st, part, lds);
    } else {
        switch (gl.count) {
        case 2: accumulate_pass<GF, OVERWRITE, CHECK, SUMSQ, NT, TPB, 2>(acc, gl, n, st, part, lds); break;
        case 3: accumulate_pass<GF, OVERWRITE, CHECK, SUMSQ, NT, TPB, 3>(acc, gl, n, st, part, lds); break;
        case 4: accumulate_pass<GF, OVERWRITE, CHECK, SUMSQ, NT, TPB, 4>(acc, gl, n, st, part, lds); break;
        case 5: accumulate_pass<GF, OVERWRITE, CHECK, SUMSQ, NT, TPB, 5>(acc, gl, n, st, part, lds); break;
        case 6: accumulate_pass<GF, OVERWRITE, CHECK, SUMSQ, NT, TPB, 6>(acc, gl, n, st, part, lds); break;
        case 7: accumulate_pass<GF, OVERWRITE, CHECK, SUMSQ, NT, TPB, 7>(acc, gl, n, st, part, lds); break;
        default: accumulate_pass<GF, OVERWRITE, CHECK, SUMSQ, NT, TPB, 8>(acc, gl, n, st, part, lds); break;
        }
    }
}

// The step's last micro-batches folded into the double-buffered Adam pass
// (ds_accumulate_adam_double_buffered).  Per element, the gradient is the fp32
// sum, in micro-batch order, of the running sum in acc (HAS_ACC; without it
// the first of the F gradients starts the sum) and of the F 16-bit gradients
// of gl; the sum is tested, fed to Adam (the arithmetic of adam_kernel), which
// reads the current copy of master, m, v and writes the other copy and its
// 16-bit parameter copy, and is not stored.  Tiles of U x TPB quads are dealt
// to blocks round-robin, every load of a tile issued before its arithmetic;
// block 0 also takes the quads after the last whole tile and the last n % 4
// elements.  A non-finite sum raises st->overflow (one atomic per wave that
// saw one); the scaler and the copy index are left to the one-thread update
// that ends the step, so a step may take one such pass per bucket.
template <int GF, int PF, bool WD, bool HAS_ACC, bool NT, int TPB, int U, int F>
__device__ __forceinline__ void fold_adam_pass(const DbArrays& a, uint32_t cur, const float* __restrict__ acc,
                                               const GradList& gl, int64_t n, const AdamConsts& c, uint32_t& bad)
{
    const f32x4* P = reinterpret_cast<const f32x4*>(cur ? a.master[1] : a.master[0]);
    const f32x4* M = reinterpret_cast<const f32x4*>(cur ? a.m[1] : a.m[0]);
    const f32x4* V = reinterpret_cast<const f32x4*>(cur ? a.v[1] : a.v[0]);
    f32x4* Po = reinterpret_cast<f32x4*>(cur ? a.master[0] : a.master[1]);
    f32x4* Mo = reinterpret_cast<f32x4*>(cur ? a.m[0] : a.m[1]);
    f32x4* Vo = reinterpret_cast<f32x4*>(cur ? a.v[0] : a.v[1]);
    uint16_t* p16o = cur ? a.p16[0] : a.p16[1];
    u32x2* H = reinterpret_cast<u32x2*>(p16o);
    const f32x4* A = reinterpret_cast<const f32x4*>(acc);

    constexpr int T = U * TPB;  // quads per tile
    const int64_t nq = n >> 2;
    const int64_t ntiles = nq / T;
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int64_t q0 = tile * T + threadIdx.x;
        f32x4 r[U], p[U], m[U], v[U];
        u32x2 raw[U][F];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = q0 + u * TPB;
            if constexpr (HAS_ACC)
                r[u] = load<NT>(A + i);
#pragma unroll
            for (int k = 0; k < F; ++k)
                raw[u][k] = load<NT>(reinterpret_cast<const u32x2*>(gl.p[k]) + i);
            p[u] = load<NT>(P + i);
            m[u] = load<NT>(M + i);
            v[u] = load<NT>(V + i);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = q0 + u * TPB;
            if constexpr (HAS_ACC)
                r[u] = r[u] + widen4<GF>(raw[u][0]);
            else
                r[u] = widen4<GF>(raw[u][0]);
#pragma unroll
            for (int k = 1; k < F; ++k)
                r[u] = r[u] + widen4<GF>(raw[u][k]);
            bad |= nonfinite_f32x4(r[u]);
            adam4<WD>(r[u], p[u], m[u], v[u], c);
            store<NT>(Po + i, p[u]);
            store<NT>(Mo + i, m[u]);
            store<NT>(Vo + i, v[u]);
            store<NT>(H + i, narrow4<PF>(p[u]));
        }
    }
    if (blockIdx.x == 0) {
        for (int64_t q = ntiles * T + threadIdx.x; q < nq; q += TPB) {
            f32x4 r;
            if constexpr (HAS_ACC)
                r = load<NT>(A + q) + widen4<GF>(load<NT>(reinterpret_cast<const u32x2*>(gl.p[0]) + q));
            else
                r = widen4<GF>(load<NT>(reinterpret_cast<const u32x2*>(gl.p[0]) + q));
#pragma unroll
            for (int k = 1; k < F; ++k)
                r = r + widen4<GF>(load<NT>(reinterpret_cast<const u32x2*>(gl.p[k]) + q));
            f32x4 p = load<NT>(P + q), m = load<NT>(M + q), v = load<NT>(V + q);
            bad |= nonfinite_f32x4(r);
            adam4<WD>(r, p, m, v, c);
            store<NT>(Po + q, p);
            store<NT>(Mo + q, m);
            store<NT>(Vo + q, v);
            store<NT>(H + q, narrow4<PF>(p));
        }
        if (static_cast<int64_t>(threadIdx.x) < (n & 3)) {
            const int64_t i = (nq << 2) + threadIdx.x;
            float r = dec1<GF>(gl.p[0][i]);
            if constexpr (HAS_ACC)
                r = acc[i] + r;
#pragma unroll
            for (int k = 1; k < F; ++k)
                r = r + dec1<GF>(gl.p[k][i]);
            const float* ps = reinterpret_cast<const float*>(P);
            const float* ms = reinterpret_cast<const float*>(M);
            const float* vs = reinterpret_cast<const float*>(V);
            float p = ps[i], m = ms[i], v = vs[i];
            bad |= nonfinite_f32(__float_as_uint(r));
            adam1<WD>(r, p, m, v, c);
            reinterpret_cast<float*>(Po)[i] = p;
            reinterpret_cast<float*>(Mo)[i] = m;
            reinterpret_cast<float*>(Vo)[i] = v;
            p16o[i] = static_cast<uint16_t>(enc1<PF>(p));
        }
    }
}

// gl.count (1..8) chosen by a block-uniform switch, so each form is
// straight-line code with every load of a tile in flight together.
template <int GF, int PF, bool WD, bool HAS_ACC, bool NT, int TPB, int U>
__global__ __launch_bounds__(TPB) void fold_adam_db_kernel(ds_scaler* __restrict__ st, DbArrays a,
                                                           const float* __restrict__ acc, GradList gl, int64_t n,
                                                           AdamHyper hp)
{
    const AdamConsts c = make_consts(st, hp);
    const uint32_t cur = st->current & 1u;
    uint32_t bad = 0u;
    switch (gl.count) {
    case 1: fold_adam_pass<GF, PF, WD, HAS_ACC, NT, TPB, U, 1>(a, cur, acc, gl, n, c, bad); break;
    case 2: fold_adam_pass<GF, PF, WD, HAS_ACC, NT, TPB, U, 2>(a, cur, acc, gl, n, c, bad); break;
    case 3: fold_adam_pass<GF, PF, WD, HAS_ACC, NT, TPB, U, 3>(a, cur, acc, gl, n, c, bad); break;
    case 4: fold_adam_pass<GF, PF, WD, HAS_ACC, NT, TPB, U, 4>(a, cur, acc, gl, n, c, bad); break;
    case 5: fold_adam_pass<GF, PF, WD, HAS_ACC, NT, TPB, U, 5>(a, cur, acc, gl, n, c, bad); break;
    case 6: fold_adam_pass<GF, PF, WD, HAS_ACC, NT, TPB, U, 6>(a, cur, acc, gl, n, c, bad); break;
    case 7: fold_adam_pass<GF, PF, WD, HAS_ACC, NT, TPB, U, 7>(a, cur, acc, gl, n, c, bad); break;
    default: fold_adam_pass<GF, PF, WD, HAS_ACC, NT, TPB, U, 8>(a, cur, acc, gl, n, c, bad); break;
    }
    raise_flag(st, bad);
}

__global__ void write_state_kernel(ds_scaler* st, ds_scaler value) { *st = value; }

// ---------------------------------------------------------------------------
// host helpers
// ---------------------------------------------------------------------------

long env_long(const char* name, long dflt)
{
    const char* s = std::getenv(name);
    if (s == nullptr || *s == '\0')
        return dflt;
    char* end = nullptr;
    long v = std::strtol(s, &end, 10);
    return (end != s) ? v : dflt;
}

// Blocks for `units` units of work (tiles, sum-of-squares chunks or groups,
// or the check's groups of kCheckBlock vectors) of a kernel with `tpb` lanes
// per block: one block per unit, at least one, at most kMaxWorkItems / tpb
// (the kernels loop past that).  DSZERO_GRID pins the block count (launch-
// shape invariance tests, sweeps).
unsigned grid_blocks(int64_t units, int tpb)
{
    const int64_t cap = kMaxWorkItems / tpb;
    const long forced = env_long("DSZERO_GRID", 0);
    int64_t b = forced > 0 ? static_cast<int64_t>(forced) : units;
    if (b > cap)
        b = cap;
    if (b < 1)
        b = 1;
    return static_cast<unsigned>(b);
}

// Quads per lane of the Adam kernel (default 4; DSZERO_UNROLL=2 halves the tile).
int variant_unroll() { return env_long("DSZERO_UNROLL", 4) == 2 ? 2 : 4; }
// Non-temporal hints on the read/write kernels' streams: on by default above
// kTemporalMaxElems elements, where a step's 28-30 B per element is more than
// twice the 256 MB Infinity Cache and every array is streamed once; off
// below, where a small partition's state stays in the cache between steps.
// DSZERO_NT=0|1 forces either.
constexpr int64_t kTemporalMaxElems = int64_t(1) << 24;
bool variant_nt(int64_t n)
{
    const long forced = env_long("DSZERO_NT", -1);
    if (forced >= 0)
        return forced != 0;
    return n > kTemporalMaxElems;
}

int64_t tiles_of(int64_t n, int unroll) { return (n >> 2) / (static_cast<int64_t>(unroll) * kStepBlock); }

bool size_ok(int64_t n) { return n >= 0 && n <= kMaxElems; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlap(const void* a, uint64_t abytes, const void* b, uint64_t bbytes)
{
    if (a == nullptr || b == nullptr || abytes == 0 || bbytes == 0)
        return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + bbytes && b0 < a0 + abytes;
}

bool finite_ge0(float x) { return std::isfinite(x) && x >= 0.0f; }
bool beta_ok(float b) { return std::isfinite(b) && b >= 0.0f && b < 1.0f; }

ds_status launched()
{
    return hipGetLastError() == hipSuccess ? DS_OK : DS_ERR_HIP;
}

// Kernel dispatch: runtime formats and switches -> template instances.

int fmt_of(ds_dtype dt) { return dt == DS_BF16 ? kBF16 : (dt == DS_FP32 ? kF32 : kF16); }
bool is16(ds_dtype dt) { return dt == DS_FP16 || dt == DS_BF16; }
bool known(ds_dtype dt) { return dt == DS_FP16 || dt == DS_BF16 || dt == DS_FP32; }
uint64_t esize(ds_dtype dt) { return dt == DS_FP32 ? 4 : 2; }

struct AdamArgs {
    ds_scaler* st;   // written only by the fused form
    float *master, *m, *v;
    uint16_t* p16;
    const void* grad;
    int64_t n;
    AdamHyper hp;
};

template <int GF, int PF, bool WD, bool NT>
void launch_adam4(int unroll, bool fuse, unsigned blocks, hipStream_t s, const AdamArgs& a)
{
    if (fuse) {  // one 4096-element tile per block in either shape (the grid does not change)
        if constexpr (NT)
            adam_kernel<GF, PF, WD, NT, kStepBlock, 4, true><<<blocks, kStepBlock, 0, s>>>(a.st, a.master, a.m, a.v, a.p16, a.grad, a.n, a.hp);
        else
            adam_kernel<GF, PF, WD, NT, kSmallBlock, 2, true><<<blocks, kSmallBlock, 0, s>>>(a.st, a.master, a.m, a.v, a.p16, a.grad, a.n, a.hp);
    }
    else if (unroll == 2)
        adam_kernel<GF, PF, WD, NT, kStepBlock, 2, false><<<blocks, kStepBlock, 0, s>>>(a.st, a.master, a.m, a.v, a.p16, a.grad, a.n, a.hp);
    else
        adam_kernel<GF, PF, WD, NT, kStepBlock, 4, false><<<blocks, kStepBlock, 0, s>>>(a.st, a.master, a.m, a.v, a.p16, a.grad, a.n, a.hp);
}

template <int GF, int PF>
void launch_adam2(bool wd, bool nt, int unroll, bool fuse, unsigned blocks, hipStream_t s, const AdamArgs& a)
{
    if (wd) {
        if (nt) launch_adam4<GF, PF, true, true>(unroll, fuse, blocks, s, a);
        else    launch_adam4<GF, PF, true, false>(unroll, fuse, blocks, s, a);
    } else {
        if (nt) launch_adam4<GF, PF, false, true>(unroll, fuse, blocks, s, a);
        else    launch_adam4<GF, PF, false, false>(unroll, fuse, blocks, s, a);
    }
}

void launch_adam(int gf, int pf, bool wd, bool nt, int unroll, bool fuse, unsigned blocks, hipStream_t s,
                 const AdamArgs& a)
{
    if (pf == kBF16) {
        if (gf == kF16)       launch_adam2<kF16, kBF16>(wd, nt, unroll, fuse, blocks, s, a);
        else if (gf == kBF16) launch_adam2<kBF16, kBF16>(wd, nt, unroll, fuse, blocks, s, a);
        else                  launch_adam2<kF32, kBF16>(wd, nt, unroll, fuse, blocks, s, a);
    } else {
        if (gf == kF16)       launch_adam2<kF16, kF16>(wd, nt, unroll, fuse, blocks, s, a);
        else if (gf == kBF16) launch_adam2<kBF16, kF16>(wd, nt, unroll, fuse, blocks, s, a);
        else                  launch_adam2<kF32, kF16>(wd, nt, unroll, fuse, blocks, s, a);
    }
}

template <int GF, int PF, bool WD>
void launch_adam_db3(bool nt, unsigned blocks, hipStream_t s, ds_scaler* st, const DbArrays& a, const void* grad,
                     int64_t n, const AdamHyper& hp)
{
    // the fused Adam kernel's shapes: 256 x 4 streamed, 512 x 2 on a cache-resident partition
    if (nt)
        adam_db_kernel<GF, PF, WD, true, kStepBlock, 4><<<blocks, kStepBlock, 0, s>>>(st, a, grad, n, hp);
    else
        adam_db_kernel<GF, PF, WD, false, kSmallBlock, 2><<<blocks, kSmallBlock, 0, s>>>(st, a, grad, n, hp);
}

template <int GF, int PF>
void launch_adam_db2(bool wd, bool nt, unsigned blocks, hipStream_t s, ds_scaler* st, const DbArrays& a,
                     const void* grad, int64_t n, const AdamHyper& hp)
{
    if (wd) launch_adam_db3<GF, PF, true>(nt, blocks, s, st, a, grad, n, hp);
    else    launch_adam_db3<GF, PF, false>(nt, blocks, s, st, a, grad, n, hp);
}

void launch_adam_db(int gf, int pf, bool wd, bool nt, unsigned blocks, hipStream_t s, ds_scaler* st,
                    const DbArrays& a, const void* grad, int64_t n, const AdamHyper& hp)
{
    if (pf == kBF16) {
        if (gf == kF16)       launch_adam_db2<kF16, kBF16>(wd, nt, blocks, s, st, a, grad, n, hp);
        else if (gf == kBF16) launch_adam_db2<kBF16, kBF16>(wd, nt, blocks, s, st, a, grad, n, hp);
        else                  launch_adam_db2<kF32, kBF16>(wd, nt, blocks, s, st, a, grad, n, hp);
    } else {
        if (gf == kF16)       launch_adam_db2<kF16, kF16>(wd, nt, blocks, s, st, a, grad, n, hp);
        else if (gf == kBF16) launch_adam_db2<kBF16, kF16>(wd, nt, blocks, s, st, a, grad, n, hp);
        else                  launch_adam_db2<kF32, kF16>(wd, nt, blocks, s, st, a, grad, n, hp);
    }
}

template <int GF, int PF, bool WD, bool HA>
void launch_fold_adam4(bool nt, unsigned blocks, hipStream_t s, ds_scaler* st, const DbArrays& a, const float* acc,
                       const GradList& gl, int64_t n, const AdamHyper& hp)
{
    constexpr int TPB = kFoldAdamBlock, U = kFoldAdamUnroll;
    if (nt) fold_adam_db_kernel<GF, PF, WD, HA, true, TPB, U><<<blocks, TPB, 0, s>>>(st, a, acc, gl, n, hp);
    else    fold_adam_db_kernel<GF, PF, WD, HA, false, TPB, U><<<blocks, TPB, 0, s>>>(st, a, acc, gl, n, hp);
}

template <int GF, int PF>
void launch_fold_adam3(bool wd, bool ha, bool nt, unsigned blocks, hipStream_t s, ds_scaler* st, const DbArrays& a,
                       const float* acc, const GradList& gl, int64_t n, const AdamHyper& hp)
{
    if (wd) {
        if (ha) launch_fold_adam4<GF, PF, true, true>(nt, blocks, s, st, a, acc, gl, n, hp);
        else    launch_fold_adam4<GF, PF, true, false>(nt, blocks, s, st, a, acc, gl, n, hp);
    } else {
        if (ha) launch_fold_adam4<GF, PF, false, true>(nt, blocks, s, st, a, acc, gl, n, hp);
        else    launch_fold_adam4<GF, PF, false, false>(nt, blocks, s, st, a, acc, gl, n, hp);
    }
}

void launch_fold_adam(int gf, int pf, bool wd, bool nt, unsigned blocks, hipStream_t s, ds_scaler* st,
                      const DbArrays& a, const float* acc, const GradList& gl, int64_t n, const AdamHyper& hp)
{
    const bool ha = acc != nullptr;
    if (gf == kBF16) {
        if (pf == kBF16) launch_fold_adam3<kBF16, kBF16>(wd, ha, nt, blocks, s, st, a, acc, gl, n, hp);
        else             launch_fold_adam3<kBF16, kF16>(wd, ha, nt, blocks, s, st, a, acc, gl, n, hp);
    } else {
        if (pf == kBF16) launch_fold_adam3<kF16, kBF16>(wd, ha, nt, blocks, s, st, a, acc, gl, n, hp);
        else             launch_fold_adam3<kF16, kF16>(wd, ha, nt, blocks, s, st, a, acc, gl, n, hp);
    }
}

template <int GF, bool OW, bool CK, bool SQ>
void launch_acc3(bool nt, hipStream_t s, float* acc, const GradList& gl, int64_t n, ds_scaler* st, double* part)
{
    constexpr int TPB = SQ ? kAccSumsqBlock : kAccBlock;
    const unsigned blocks = grid_blocks((n >> 2) / TPB, TPB);
    if (gl.count == 1) {
        if (nt) accumulate_kernel<GF, OW, CK, SQ, true, false, TPB><<<blocks, TPB, 0, s>>>(acc, gl, n, st, part);
        else    accumulate_kernel<GF, OW, CK, SQ, false, false, TPB><<<blocks, TPB, 0, s>>>(acc, gl, n, st, part);
    } else {
        if (nt) accumulate_kernel<GF, OW, CK, SQ, true, true, TPB><<<blocks, TPB, 0, s>>>(acc, gl, n, st, part);
        else    accumulate_kernel<GF, OW, CK, SQ, false, true, TPB><<<blocks, TPB, 0, s>>>(acc, gl, n, st, part);
    }
}

// Accumulation pass: `ck` fuses the non-finite check of the result, a
// non-null `part` (which needs `ck`) the chunk sums of squares.
template <int GF>
void launch_acc(bool ow, bool ck, bool nt, hipStream_t s, float* acc, const GradList& gl, int64_t n, ds_scaler* st,
                double* part)
{
    if (part != nullptr) {
        if (ow) launch_acc3<GF, true, true, true>(nt, s, acc, gl, n, st, part);
        else    launch_acc3<GF, false, true, true>(nt, s, acc, gl, n, st, part);
    } else if (ck) {
        if (ow) launch_acc3<GF, true, true, false>(nt, s, acc, gl, n, st, nullptr);
        else    launch_acc3<GF, false, true, false>(nt, s, acc, gl, n, st, nullptr);
    } else {
        if (ow) launch_acc3<GF, true, false, false>(nt, s, acc, gl, n, nullptr, nullptr);
        else    launch_acc3<GF, false, false, false>(nt, s, acc, gl, n, nullptr, nullptr);
    }
}

int64_t acc_chunks(int64_t n) { return (n + kAccChunk - 1) / kAccChunk; }
int64_t check_chunks(int64_t n) { return (n + kCheckChunk - 1) / kCheckChunk; }
int64_t finish_groups(int64_t nparts) { return (nparts + kGroup - 1) / kGroup; }

// Workspace of a sum of squares over n elements: the chunk sums of the
// finer chunking (the accumulation's, 1024 elements) followed by the group
// sums of the second pass.
uint64_t sumsq_ws_bytes(int64_t n)
{
    if (n <= 0)
        return 0;
    const int64_t p = acc_chunks(n);
    return 8 * static_cast<uint64_t>(p + finish_groups(p));
}

// validation shared by the sum-of-squares entry points
ds_status check_workspace(const void* ws, size_t ws_bytes, int64_t n)
{
    if (ws == nullptr)
        return DS_ERR_NULL;
    if (!aligned(ws, 8))
        return DS_ERR_ALIGN;
    if (ws_bytes < sumsq_ws_bytes(n))
        return DS_ERR_SIZE;
    return DS_OK;
}

// Second pass of a sum of squares whose first pass wrote `nparts` chunk sums
// at ws: the group sums go right after them.
ds_status launch_finish(ds_scaler* st, double* ws, int64_t nparts, hipStream_t s)
{
    const unsigned blocks = grid_blocks(finish_groups(nparts), kFinishBlock);
    sumsq_finish_kernel<<<blocks, kFinishBlock, 0, s>>>(st, ws, nparts, ws + nparts);
    return launched();
}

// Launches of the validated accumulation entry points: the pass over the
// data, then (with a workspace) the second pass of the sum of squares.
ds_status launch_accumulate(float* acc, const GradList& gl, ds_dtype gdt, int64_t n, bool overwrite,
                            ds_scaler* st_or_null, double* ws_or_null, hipStream_t s)
{
    const bool nt = variant_nt(n);
    const bool ck = st_or_null != nullptr;
    if (gdt == DS_BF16)
        launch_acc<kBF16>(overwrite, ck, nt, s, acc, gl, n, st_or_null, ws_or_null);
    else
        launch_acc<kF16>(overwrite, ck, nt, s, acc, gl, n, st_or_null, ws_or_null);
    if (ws_or_null == nullptr)
        return launched();
    if (launched() != DS_OK)
        return DS_ERR_HIP;
    return launch_finish(st_or_null, ws_or_null, acc_chunks(n), s);
}

// Launch of the validated check with the sum of squares (workspace ws of at
// least sumsq_ws_bytes(n) bytes).
ds_status launch_check_sumsq(ds_scaler* st, const void* grad, ds_dtype dt, int64_t n, double* ws, hipStream_t s)
{
    constexpr int TPB = kCheckSumsqBlock;
    const int64_t chunks = check_chunks(n);
    const unsigned blocks = grid_blocks(chunks, TPB);
    if (dt == DS_FP16)
        check_sumsq_kernel<kF16, TPB><<<blocks, TPB, 0, s>>>(st, grad, n, ws);
    else if (dt == DS_BF16)
        check_sumsq_kernel<kBF16, TPB><<<blocks, TPB, 0, s>>>(st, grad, n, ws);
    else
        check_sumsq_kernel<kF32, TPB><<<blocks, TPB, 0, s>>>(st, grad, n, ws);
    if (launched() != DS_OK)
        return DS_ERR_HIP;
    return launch_finish(st, ws, chunks, s);
}

bool schedule_ok(const ds_lr_schedule& q)
{
    if (q.kind != DS_LR_WARMUP && q.kind != DS_LR_WARMUP_DECAY)
        return false;
    if (!finite_ge0(q.warmup_min_lr) || !finite_ge0(q.warmup_max_lr) || q.warmup_num_steps < 0)
        return false;
    return q.kind != DS_LR_WARMUP_DECAY || q.total_num_steps >= q.warmup_num_steps;
}

// Validation and launch shared by the constant-lr and scheduled entry points
// (a schedule is checked by its entry point; hp.lr is the constant lr or the
// schedule's peak).
ds_status adam_step(const ds_scaler* st, float* master, float* m, float* v, uint16_t* p16,
                    ds_dtype pdt, const void* grad, ds_dtype dt, int64_t n, const AdamHyper& hp,
                    bool fuse, void* stream)
{
    const float beta1 = hp.beta1, beta2 = hp.beta2, eps = hp.eps;
    const float weight_decay = hp.weight_decay, max_grad_norm = hp.max_grad_norm;
    const int32_t accum_steps = hp.accum_steps;
    if (!size_ok(n))
        return DS_ERR_SIZE;
    if (!known(dt) || !is16(pdt))
        return DS_ERR_DTYPE;
    if (!finite_ge0(hp.lr) || !beta_ok(beta1) || !beta_ok(beta2) || !std::isfinite(eps) ||
        eps <= 0.0f || !finite_ge0(weight_decay) || !finite_ge0(max_grad_norm) || accum_steps < 1)
        return DS_ERR_HPARAM;
    if (st == nullptr)
        return DS_ERR_NULL;
    if (n == 0) {
        if (!fuse)
            return DS_OK;
        if (!aligned(st, 8))
            return DS_ERR_ALIGN;
        update_scale_kernel<<<1, 1, 0, static_cast<hipStream_t>(stream)>>>(const_cast<ds_scaler*>(st));
        return launched();
    }
    if (master == nullptr || m == nullptr || v == nullptr || p16 == nullptr || grad == nullptr)
        return DS_ERR_NULL;
    if (!aligned(master, 16) || !aligned(m, 16) || !aligned(v, 16) || !aligned(p16, 16) ||
        !aligned(grad, 16) || !aligned(st, 8))
        return DS_ERR_ALIGN;
    const uint64_t un = static_cast<uint64_t>(n);
    const void* ptrs[6] = {master, m, v, p16, grad, st};
    const uint64_t sizes[6] = {4 * un, 4 * un, 4 * un, 2 * un, esize(dt) * un, sizeof(ds_scaler)};
    for (int i = 0; i < 6; ++i)
        for (int j = i + 1; j < 6; ++j)
            if (overlap(ptrs[i], sizes[i], ptrs[j], sizes[j]))
                return DS_ERR_ALIAS;

    hipStream_t s = static_cast<hipStream_t>(stream);
    const int unroll = fuse ? 4 : variant_unroll();
    const bool nt = variant_nt(n);
    const unsigned blocks = grid_blocks(tiles_of(n, unroll), fuse && !nt ? kSmallBlock : kStepBlock);
    const bool wd = weight_decay != 0.0f;
    const AdamArgs args{const_cast<ds_scaler*>(st), master, m, v, p16, grad, n, hp};
    launch_adam(fmt_of(dt), fmt_of(pdt), wd, nt, unroll, fuse, blocks, s, args);
    return launched();
}

}  // namespace

// ---------------------------------------------------------------------------
// statically allocated scratch of ds_check_overflow_sumsq_noalloc
// ---------------------------------------------------------------------------

// The chunk and group sums of that entry point: 2^21 fp64 values (16 MiB),
// held in each device's memory for the life of the process.  In host code the
// array's name stands for no device address; the address of a device's copy
// is looked up once per device (scratch_on) and passed to the kernels.
constexpr int64_t kScratchDoubles = int64_t(1) << 21;
static __device__ __align__(256) double scratch[kScratchDoubles];
static_assert(DS_NOALLOC_MAX_ELEMS % kCheckChunk == 0, "the limit is a whole number of chunks");
static_assert(DS_NOALLOC_MAX_ELEMS / kCheckChunk + (DS_NOALLOC_MAX_ELEMS / kCheckChunk + kGroup - 1) / kGroup <=
                  kScratchDoubles, "the largest accepted n fits in the scratch array");
static_assert((DS_NOALLOC_MAX_ELEMS / kCheckChunk + 1) + (DS_NOALLOC_MAX_ELEMS / kCheckChunk + kGroup) / kGroup >
                  kScratchDoubles, "the limit is the largest n that fits");

namespace {

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
std::atomic<double*> scratch_ptr[kMaxDevices];

// Device address of device `dev`'s copy of `scratch`: looked up on the first
// call for that device, with that device current (and the caller's current
// device restored), then kept.
ds_status scratch_on(int dev, double** out)
{
    if (dev < 0 || dev >= kMaxDevices)
        return DS_ERR_HIP;
    double* p = scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(scratch_mutex);
        p = scratch_ptr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            int cur = -1;
            if (hipGetDevice(&cur) != hipSuccess)
                return DS_ERR_HIP;
            if (cur != dev && hipSetDevice(dev) != hipSuccess)
                return DS_ERR_HIP;
            void* addr = nullptr;
            const hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
            const bool restored = cur == dev || hipSetDevice(cur) == hipSuccess;
            if (e != hipSuccess || addr == nullptr || !restored)
                return DS_ERR_HIP;
            p = static_cast<double*>(addr);
            scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return DS_OK;
}

// The device a stream's work runs on (the current device for the null stream).
ds_status stream_device(hipStream_t s, int* dev)
{
    if (s == nullptr)
        return hipGetDevice(dev) == hipSuccess ? DS_OK : DS_ERR_HIP;
    return hipStreamGetDevice(s, dev) == hipSuccess ? DS_OK : DS_ERR_HIP;
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------

extern "C" {

size_t ds_scaler_size(void) { return sizeof(ds_scaler); }

const char* ds_status_string(ds_status s)
{
    switch (s) {
    case DS_OK: return "DS_OK";
    case DS_ERR_NULL: return "DS_ERR_NULL: null pointer";
    case DS_ERR_SIZE: return "DS_ERR_SIZE: invalid size";
    case DS_ERR_ALIGN: return "DS_ERR_ALIGN: pointer not aligned";
    case DS_ERR_DTYPE: return "DS_ERR_DTYPE: unknown dtype";
    case DS_ERR_HPARAM: return "DS_ERR_HPARAM: hyperparameter out of range";
    case DS_ERR_ALIAS: return "DS_ERR_ALIAS: arrays overlap";
    case DS_ERR_HIP: return "DS_ERR_HIP: HIP launch or copy failed";
    }
    return "unknown ds_status";
}

ds_status ds_state_init(ds_scaler* st, float init_scale, float min_scale, int32_t growth_window,
                        int32_t hysteresis, int32_t consecutive_hysteresis, int32_t dynamic,
                        void* stream)
{
    if (st == nullptr)
        return DS_ERR_NULL;
    if (!aligned(st, 8))
        return DS_ERR_ALIGN;
    if (!std::isfinite(init_scale) || init_scale <= 0.0f || !std::isfinite(min_scale) ||
        min_scale <= 0.0f || growth_window < 1 || hysteresis < 1)
        return DS_ERR_HPARAM;
    ds_scaler s;
    std::memset(&s, 0, sizeof s);
    s.scale = init_scale;
    s.min_scale = min_scale;
    s.growth_window = growth_window;
    s.hysteresis = hysteresis;
    s.hysteresis_left = hysteresis;
    s.dynamic = dynamic ? 1 : 0;
    s.consecutive_hysteresis = consecutive_hysteresis ? 1 : 0;
    write_state_kernel<<<1, 1, 0, static_cast<hipStream_t>(stream)>>>(st, s);
    return launched();
}

ds_status ds_state_read(const ds_scaler* st, ds_scaler* host_out, void* stream)
{
    if (st == nullptr || host_out == nullptr)
        return DS_ERR_NULL;
    if (!aligned(st, 8))
        return DS_ERR_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (hipMemcpyAsync(host_out, st, sizeof(ds_scaler), hipMemcpyDeviceToHost, s) != hipSuccess)
        return DS_ERR_HIP;
    return hipStreamSynchronize(s) == hipSuccess ? DS_OK : DS_ERR_HIP;
}

ds_status ds_state_write(ds_scaler* st, const ds_scaler* host_in, void* stream)
{
    if (st == nullptr || host_in == nullptr)
        return DS_ERR_NULL;
    if (!aligned(st, 8))
        return DS_ERR_ALIGN;
    ds_scaler value = *host_in;
    value.blocks_done = 0u;         // between steps the fused form's block count is 0
    value.sumsq_blocks_done = 0u;   // and so is the sum of squares' second pass's
    value.db_tickets = 0ull;        // and the double-buffered step's
    write_state_kernel<<<1, 1, 0, static_cast<hipStream_t>(stream)>>>(st, value);
    return launched();
}

ds_status ds_accumulate(float* acc, const uint16_t* g16, ds_dtype gdt, int64_t n, int32_t overwrite,
                        ds_scaler* st_or_null, void* stream)
{
    if (!size_ok(n))
        return DS_ERR_SIZE;
    if (!is16(gdt))
        return DS_ERR_DTYPE;
    if (n == 0)
        return DS_OK;
    if (acc == nullptr || g16 == nullptr)
        return DS_ERR_NULL;
    if (!aligned(acc, 16) || !aligned(g16, 16) || (st_or_null != nullptr && !aligned(st_or_null, 8)))
        return DS_ERR_ALIGN;
    const uint64_t un = static_cast<uint64_t>(n);
    if (overlap(acc, 4 * un, g16, 2 * un) || overlap(acc, 4 * un, st_or_null, sizeof(ds_scaler)) ||
        overlap(g16, 2 * un, st_or_null, sizeof(ds_scaler)))
        return DS_ERR_ALIAS;
    GradList gl{};
    gl.p[0] = g16;
    gl.count = 1;
    return launch_accumulate(acc, gl, gdt, n, overwrite != 0, st_or_null, nullptr,
                             static_cast<hipStream_t>(stream));
}

ds_status ds_check_overflow(ds_scaler* st, const void* grad, ds_dtype dt, int64_t n, void* stream)
{
    if (!size_ok(n))
        return DS_ERR_SIZE;
    if (!known(dt))
        return DS_ERR_DTYPE;
    if (st == nullptr)
        return DS_ERR_NULL;
    if (n == 0)
        return DS_OK;
    if (grad == nullptr)
        return DS_ERR_NULL;
    if (!aligned(grad, 16) || !aligned(st, 8))
        return DS_ERR_ALIGN;
    if (overlap(grad, esize(dt) * static_cast<uint64_t>(n), st, sizeof(ds_scaler)))
        return DS_ERR_ALIAS;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t vecs = n / (dt == DS_FP32 ? 4 : 8);
    const unsigned blocks = grid_blocks((vecs + kCheckBlock - 1) / kCheckBlock, kCheckBlock);
    // ordinary loads: leave the gradient in the Infinity Cache for the Adam pass
    if (dt == DS_FP16)
        check_kernel<kF16, false, kCheckBlock><<<blocks, kCheckBlock, 0, s>>>(st, grad, n);
    else if (dt == DS_BF16)
        check_kernel<kBF16, false, kCheckBlock><<<blocks, kCheckBlock, 0, s>>>(st, grad, n);
    else
        check_kernel<kF32, false, kCheckBlock><<<blocks, kCheckBlock, 0, s>>>(st, grad, n);
    return launched();
}

ds_status ds_adam_step(const ds_scaler* st, float* master, float* m, float* v, uint16_t* p16,
                       ds_dtype pdt, const void* grad, ds_dtype dt, int64_t n, float lr, float beta1,
                       float beta2, float eps, float weight_decay, float max_grad_norm,
                       int32_t accum_steps, void* stream)
{
    const AdamHyper hp{lr, beta1, beta2, eps, weight_decay, max_grad_norm, accum_steps, 0, 0.0f, 0, 0};
    return adam_step(st, master, m, v, p16, pdt, grad, dt, n, hp, false, stream);
}

ds_status ds_adam_step_sched(const ds_scaler* st, float* master, float* m, float* v, uint16_t* p16,
                             ds_dtype pdt, const void* grad, ds_dtype dt, int64_t n,
                             const ds_lr_schedule* sched, float beta1, float beta2, float eps,
                             float weight_decay, float max_grad_norm, int32_t accum_steps,
                             void* stream)
{
    if (sched == nullptr)
        return DS_ERR_NULL;
    if (!schedule_ok(*sched))
        return DS_ERR_HPARAM;
    const AdamHyper hp{sched->warmup_max_lr, beta1, beta2, eps, weight_decay, max_grad_norm, accum_steps,
                 sched->kind, sched->warmup_min_lr, sched->warmup_num_steps, sched->total_num_steps};
    return adam_step(st, master, m, v, p16, pdt, grad, dt, n, hp, false, stream);
}

ds_status ds_adam_step_fused(ds_scaler* st, float* master, float* m, float* v, uint16_t* p16, ds_dtype pdt,
                             const void* grad, ds_dtype dt, int64_t n, float lr,
                             const ds_lr_schedule* sched_or_null, float beta1, float beta2, float eps,
                             float weight_decay, float max_grad_norm, int32_t accum_steps, void* stream)
{
    if (sched_or_null != nullptr) {
        if (!schedule_ok(*sched_or_null))
            return DS_ERR_HPARAM;
        const ds_lr_schedule& q = *sched_or_null;
        const AdamHyper hp{q.warmup_max_lr, beta1, beta2, eps, weight_decay, max_grad_norm, accum_steps,
                           q.kind, q.warmup_min_lr, q.warmup_num_steps, q.total_num_steps};
        return adam_step(st, master, m, v, p16, pdt, grad, dt, n, hp, true, stream);
    }
    const AdamHyper hp{lr, beta1, beta2, eps, weight_decay, max_grad_norm, accum_steps, 0, 0.0f, 0, 0};
    return adam_step(st, master, m, v, p16, pdt, grad, dt, n, hp, true, stream);
}

ds_status ds_adam_step_double_buffered(ds_scaler* st, float* const* master2, float* const* m2, float* const* v2,
                                       uint16_t* const* p16_2, ds_dtype pdt, const void* grad, ds_dtype dt,
                                       int64_t n, float lr, const ds_lr_schedule* sched_or_null, float beta1,
                                       float beta2, float eps, float weight_decay, int32_t accum_steps,
                                       void* stream)
{
    AdamHyper hp{lr, beta1, beta2, eps, weight_decay, 0.0f, accum_steps, 0, 0.0f, 0, 0};
    if (sched_or_null != nullptr) {
        if (!schedule_ok(*sched_or_null))
            return DS_ERR_HPARAM;
        const ds_lr_schedule& q = *sched_or_null;
        hp = AdamHyper{q.warmup_max_lr, beta1, beta2, eps, weight_decay, 0.0f, accum_steps,
                       q.kind, q.warmup_min_lr, q.warmup_num_steps, q.total_num_steps};
    }
    if (!size_ok(n))
        return DS_ERR_SIZE;
    if (!known(dt) || !is16(pdt))
        return DS_ERR_DTYPE;
    if (!finite_ge0(hp.lr) || !beta_ok(beta1) || !beta_ok(beta2) || !std::isfinite(eps) || eps <= 0.0f ||
        !finite_ge0(weight_decay) || accum_steps < 1)
        return DS_ERR_HPARAM;
    if (st == nullptr)
        return DS_ERR_NULL;
    if (!aligned(st, 8))
        return DS_ERR_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (n == 0) {
        update_scale_swap_kernel<<<1, 1, 0, s>>>(st);
        return launched();
    }
    if (master2 == nullptr || m2 == nullptr || v2 == nullptr || p16_2 == nullptr || grad == nullptr)
        return DS_ERR_NULL;
    DbArrays a{};
    for (int k = 0; k < 2; ++k) {
        if (master2[k] == nullptr || m2[k] == nullptr || v2[k] == nullptr || p16_2[k] == nullptr)
            return DS_ERR_NULL;
        a.master[k] = master2[k];
        a.m[k] = m2[k];
        a.v[k] = v2[k];
        a.p16[k] = p16_2[k];
    }
    const void* ptrs[10] = {a.master[0], a.master[1], a.m[0], a.m[1], a.v[0], a.v[1], a.p16[0], a.p16[1], grad, st};
    for (int i = 0; i < 10; ++i)
        if (!aligned(ptrs[i], i == 9 ? 8 : 16))
            return DS_ERR_ALIGN;
    const uint64_t un = static_cast<uint64_t>(n);
    const uint64_t sizes[10] = {4 * un, 4 * un, 4 * un, 4 * un, 4 * un, 4 * un, 2 * un, 2 * un, esize(dt) * un,
                                sizeof(ds_scaler)};
    for (int i = 0; i < 10; ++i)
        for (int j = i + 1; j < 10; ++j)
            if (overlap(ptrs[i], sizes[i], ptrs[j], sizes[j]))
                return DS_ERR_ALIAS;
    const bool nt = variant_nt(n);
    const unsigned blocks = grid_blocks(tiles_of(n, 4), nt ? kStepBlock : kSmallBlock);
    launch_adam_db(fmt_of(dt), fmt_of(pdt), weight_decay != 0.0f, nt, blocks, s, st, a, grad, n, hp);
    return launched();
}

ds_status ds_accumulate_adam_double_buffered(ds_scaler* st, float* const* master2, float* const* m2,
                                             float* const* v2, uint16_t* const* p16_2, ds_dtype pdt,
                                             const float* acc_or_null, const uint16_t* const* grads, int32_t count,
                                             ds_dtype gdt, int64_t n, float lr, const ds_lr_schedule* sched_or_null,
                                             float beta1, float beta2, float eps, float weight_decay,
                                             int32_t accum_steps, void* stream)
{
    AdamHyper hp{lr, beta1, beta2, eps, weight_decay, 0.0f, accum_steps, 0, 0.0f, 0, 0};
    if (sched_or_null != nullptr) {
        if (!schedule_ok(*sched_or_null))
            return DS_ERR_HPARAM;
        const ds_lr_schedule& q = *sched_or_null;
        hp = AdamHyper{q.warmup_max_lr, beta1, beta2, eps, weight_decay, 0.0f, accum_steps,
                       q.kind, q.warmup_min_lr, q.warmup_num_steps, q.total_num_steps};
    }
    if (!size_ok(n) || count < 1 || count > kMaxFold)
        return DS_ERR_SIZE;
    if (!is16(gdt) || !is16(pdt))
        return DS_ERR_DTYPE;
    if (!finite_ge0(hp.lr) || !beta_ok(beta1) || !beta_ok(beta2) || !std::isfinite(eps) || eps <= 0.0f ||
        !finite_ge0(weight_decay) || accum_steps < 1)
        return DS_ERR_HPARAM;
    // without the running sum these are all of the step's micro-batches; with
    // it, the last of them
    if (acc_or_null == nullptr ? count != accum_steps : count >= accum_steps)
        return DS_ERR_HPARAM;
    if (st == nullptr)
        return DS_ERR_NULL;
    if (!aligned(st, 8))
        return DS_ERR_ALIGN;
    if (n == 0)
        return DS_OK;
    if (master2 == nullptr || m2 == nullptr || v2 == nullptr || p16_2 == nullptr || grads == nullptr)
        return DS_ERR_NULL;
    DbArrays a{};
    for (int k = 0; k < 2; ++k) {
        if (master2[k] == nullptr || m2[k] == nullptr || v2[k] == nullptr || p16_2[k] == nullptr)
            return DS_ERR_NULL;
        a.master[k] = master2[k];
        a.m[k] = m2[k];
        a.v[k] = v2[k];
        a.p16[k] = p16_2[k];
    }
    GradList gl{};
    for (int32_t k = 0; k < count; ++k) {
        if (grads[k] == nullptr)
            return DS_ERR_NULL;
        if (!aligned(grads[k], 16))
            return DS_ERR_ALIGN;
        gl.p[k] = grads[k];
    }
    gl.count = count;
    // the eight state arrays, the running sum and the state must not overlap
    // one another or a gradient (the gradients, only read, may repeat)
    const void* ptrs[10] = {a.master[0], a.master[1], a.m[0], a.m[1], a.v[0], a.v[1], a.p16[0], a.p16[1],
                            acc_or_null, st};
    for (int i = 0; i < 10; ++i)
        if (ptrs[i] != nullptr && !aligned(ptrs[i], i == 9 ? 8 : 16))
            return DS_ERR_ALIGN;
    const uint64_t un = static_cast<uint64_t>(n);
    const uint64_t sizes[10] = {4 * un, 4 * un, 4 * un, 4 * un, 4 * un, 4 * un, 2 * un, 2 * un,
                                acc_or_null != nullptr ? 4 * un : 0, sizeof(ds_scaler)};
    for (int i = 0; i < 10; ++i) {
        for (int j = i + 1; j < 10; ++j)
            if (overlap(ptrs[i], sizes[i], ptrs[j], sizes[j]))
                return DS_ERR_ALIAS;
        for (int32_t k = 0; k < count; ++k)
            if (overlap(ptrs[i], sizes[i], grads[k], 2 * un))
                return DS_ERR_ALIAS;
    }
    const bool nt = variant_nt(n);
    const unsigned blocks = grid_blocks((n >> 2) / (kFoldAdamBlock * kFoldAdamUnroll), kFoldAdamBlock);
    launch_fold_adam(fmt_of(gdt), fmt_of(pdt), weight_decay != 0.0f, nt, blocks, static_cast<hipStream_t>(stream),
                     st, a, acc_or_null, gl, n, hp);
    return launched();
}

ds_status ds_update_loss_scale_double_buffered(ds_scaler* st, void* stream)
{
    if (st == nullptr)
        return DS_ERR_NULL;
    if (!aligned(st, 8))
        return DS_ERR_ALIGN;
    update_scale_swap_kernel<<<1, 1, 0, static_cast<hipStream_t>(stream)>>>(st);
    return launched();
}

size_t ds_sumsq_workspace_bytes(int64_t n)
{
    return static_cast<size_t>(sumsq_ws_bytes(n));
}

ds_status ds_check_overflow_sumsq(ds_scaler* st, const void* grad, ds_dtype dt, int64_t n,
                                  void* workspace, size_t workspace_bytes, void* stream)
{
    if (!size_ok(n))
        return DS_ERR_SIZE;
    if (!known(dt))
        return DS_ERR_DTYPE;
    if (st == nullptr)
        return DS_ERR_NULL;
    if (n == 0)
        return DS_OK;
    if (grad == nullptr)
        return DS_ERR_NULL;
    if (!aligned(grad, 16) || !aligned(st, 8))
        return DS_ERR_ALIGN;
    if (const ds_status w = check_workspace(workspace, workspace_bytes, n); w != DS_OK)
        return w;
    const uint64_t gb = esize(dt) * static_cast<uint64_t>(n);
    const uint64_t wb = sumsq_ws_bytes(n);
    if (overlap(grad, gb, st, sizeof(ds_scaler)) || overlap(grad, gb, workspace, wb) ||
        overlap(st, sizeof(ds_scaler), workspace, wb))
        return DS_ERR_ALIAS;
    return launch_check_sumsq(st, grad, dt, n, static_cast<double*>(workspace), static_cast<hipStream_t>(stream));
}

ds_status ds_check_overflow_sumsq_noalloc(ds_scaler* st, const void* grad, ds_dtype dt, int64_t n, void* stream)
{
    if (n < 0 || n > DS_NOALLOC_MAX_ELEMS)
        return DS_ERR_SIZE;
    if (!known(dt))
        return DS_ERR_DTYPE;
    if (st == nullptr)
        return DS_ERR_NULL;
    if (n == 0)
        return DS_OK;
    if (grad == nullptr)
        return DS_ERR_NULL;
    if (!aligned(grad, 16) || !aligned(st, 8))
        return DS_ERR_ALIGN;
    if (overlap(grad, esize(dt) * static_cast<uint64_t>(n), st, sizeof(ds_scaler)))
        return DS_ERR_ALIAS;
    hipStream_t s = static_cast<hipStream_t>(stream);
    int dev = -1;
    if (stream_device(s, &dev) != DS_OK)
        return DS_ERR_HIP;
    double* ws = nullptr;
    if (scratch_on(dev, &ws) != DS_OK)
        return DS_ERR_HIP;
    const uint64_t wb = 8 * static_cast<uint64_t>(kScratchDoubles);
    if (overlap(grad, esize(dt) * static_cast<uint64_t>(n), ws, wb) || overlap(st, sizeof(ds_scaler), ws, wb))
        return DS_ERR_ALIAS;
    return launch_check_sumsq(st, grad, dt, n, ws, s);
}

ds_status ds_accumulate_sumsq(float* acc, const uint16_t* g16, ds_dtype gdt, int64_t n, int32_t overwrite,
                              ds_scaler* st, void* workspace, size_t workspace_bytes, void* stream)
{
    if (!size_ok(n))
        return DS_ERR_SIZE;
    if (!is16(gdt))
        return DS_ERR_DTYPE;
    if (st == nullptr)
        return DS_ERR_NULL;
    if (n == 0)
        return DS_OK;
    if (acc == nullptr || g16 == nullptr)
        return DS_ERR_NULL;
    if (!aligned(acc, 16) || !aligned(g16, 16) || !aligned(st, 8))
        return DS_ERR_ALIGN;
    if (const ds_status w = check_workspace(workspace, workspace_bytes, n); w != DS_OK)
        return w;
    const uint64_t un = static_cast<uint64_t>(n);
    const uint64_t wb = sumsq_ws_bytes(n);
    const void* ptrs[4] = {acc, g16, st, workspace};
    const uint64_t sizes[4] = {4 * un, 2 * un, sizeof(ds_scaler), wb};
    for (int i = 0; i < 4; ++i)
        for (int j = i + 1; j < 4; ++j)
            if (overlap(ptrs[i], sizes[i], ptrs[j], sizes[j]))
                return DS_ERR_ALIAS;
    GradList gl{};
    gl.p[0] = g16;
    gl.count = 1;
    return launch_accumulate(acc, gl, gdt, n, overwrite != 0, st, static_cast<double*>(workspace),
                             static_cast<hipStream_t>(stream));
}

ds_status ds_accumulate_multi(float* acc, const uint16_t* const* grads, int32_t count, ds_dtype gdt, int64_t n,
                              int32_t overwrite, ds_scaler* st_or_null, void* workspace_or_null,
                              size_t workspace_bytes, void* stream)
{
    if (!size_ok(n) || count < 1 || count > kMaxFold)
        return DS_ERR_SIZE;
    if (!is16(gdt))
        return DS_ERR_DTYPE;
    if (workspace_or_null != nullptr && st_or_null == nullptr)
        return DS_ERR_NULL;
    if (n == 0)
        return DS_OK;
    if (acc == nullptr || grads == nullptr)
        return DS_ERR_NULL;
    for (int32_t k = 0; k < count; ++k)
        if (grads[k] == nullptr)
            return DS_ERR_NULL;
    if (!aligned(acc, 16) || (st_or_null != nullptr && !aligned(st_or_null, 8)))
        return DS_ERR_ALIGN;
    for (int32_t k = 0; k < count; ++k)
        if (!aligned(grads[k], 16))
            return DS_ERR_ALIGN;
    const bool sumsq = workspace_or_null != nullptr;
    if (sumsq) {
        if (const ds_status w = check_workspace(workspace_or_null, workspace_bytes, n); w != DS_OK)
            return w;
    }
    // written: acc, the state, the workspace; read: the gradients (which may
    // repeat or overlap one another)
    const uint64_t un = static_cast<uint64_t>(n);
    const uint64_t wb = sumsq ? sumsq_ws_bytes(n) : 0;
    const void* out[3] = {acc, st_or_null, workspace_or_null};
    const uint64_t out_bytes[3] = {4 * un, st_or_null != nullptr ? sizeof(ds_scaler) : 0, wb};
    for (int i = 0; i < 3; ++i) {
        for (int j = i + 1; j < 3; ++j)
            if (overlap(out[i], out_bytes[i], out[j], out_bytes[j]))
                return DS_ERR_ALIAS;
        for (int32_t k = 0; k < count; ++k)
            if (overlap(out[i], out_bytes[i], grads[k], 2 * un))
                return DS_ERR_ALIAS;
    }
    GradList gl{};
    for (int32_t k = 0; k < count; ++k)
        gl.p[k] = grads[k];
    gl.count = count;
    return launch_accumulate(acc, gl, gdt, n, overwrite != 0, st_or_null, static_cast<double*>(workspace_or_null),
                             static_cast<hipStream_t>(stream));
}

ds_status ds_update_loss_scale(ds_scaler* st, void* stream)
{
    if (st == nullptr)
        return DS_ERR_NULL;
    if (!aligned(st, 8))
        return DS_ERR_ALIGN;
    update_scale_kernel<<<1, 1, 0, static_cast<hipStream_t>(stream)>>>(st);
    return launched();
}

ds_status ds_adam_bias_scalars(const ds_scaler* st, float lr, float beta1, float beta2, float* out2,
                               void* stream)
{
    if (st == nullptr || out2 == nullptr)
        return DS_ERR_NULL;
    if (!aligned(st, 8) || !aligned(out2, 8))
        return DS_ERR_ALIGN;
    if (!finite_ge0(lr) || !beta_ok(beta1) || !beta_ok(beta2))
        return DS_ERR_HPARAM;
    if (overlap(st, sizeof(ds_scaler), out2, 2 * sizeof(float)))
        return DS_ERR_ALIAS;
    bias_scalars_kernel<<<1, 1, 0, static_cast<hipStream_t>(stream)>>>(st, lr, beta1, beta2, out2);
    return launched();
}

ds_status ds_lr_scalars(const ds_scaler* st, const ds_lr_schedule* sched, float beta1, float beta2,
                        float* out3, void* stream)
{
    if (st == nullptr || sched == nullptr || out3 == nullptr)
        return DS_ERR_NULL;
    if (!aligned(st, 8) || !aligned(out3, 4))
        return DS_ERR_ALIGN;
    if (!schedule_ok(*sched) || !beta_ok(beta1) || !beta_ok(beta2))
        return DS_ERR_HPARAM;
    if (overlap(st, sizeof(ds_scaler), out3, 3 * sizeof(float)))
        return DS_ERR_ALIAS;
    const AdamHyper hp{sched->warmup_max_lr, beta1, beta2, 1.0f, 0.0f, 0.0f, 1,
                       sched->kind, sched->warmup_min_lr, sched->warmup_num_steps,
                       sched->total_num_steps};
    lr_scalars_kernel<<<1, 1, 0, static_cast<hipStream_t>(stream)>>>(st, hp, out3);
    return launched();
}

ds_status ds_layout_greedy(const int64_t* numels, int32_t count, int64_t cap, int64_t align,
                           int64_t* offsets, int32_t* bucket_of, int64_t* bucket_start,
                           int64_t* bucket_size, int32_t* n_buckets, int64_t* total)
{
    if (count < 0 || cap < 1 || align < 1)
        return DS_ERR_SIZE;
    if (n_buckets == nullptr || total == nullptr)
        return DS_ERR_NULL;
    if (count > 0 && (numels == nullptr || offsets == nullptr || bucket_of == nullptr ||
                      bucket_start == nullptr || bucket_size == nullptr))
        return DS_ERR_NULL;
    if (cap > kMaxElems || align > kMaxElems)
        return DS_ERR_SIZE;
    // every tensor, padded, must fit in kMaxElems together: a bound on the
    // flat length that keeps all of the arithmetic below in range
    int64_t bound = 0;
    for (int32_t i = 0; i < count; ++i) {
        if (numels[i] < 0 || numels[i] > kMaxElems)
            return DS_ERR_SIZE;
        bound += numels[i] + align - 1;
        if (bound > kMaxElems)
            return DS_ERR_SIZE;
    }
    auto up = [align](int64_t x) { return (x + align - 1) / align * align; };
    int32_t nb = 0;
    int64_t start = 0;     // first element of the open bucket
    int64_t end = 0;       // end of the last tensor placed (unpadded)
    int32_t members = 0;   // tensors in the open bucket
    for (int32_t i = 0; i < count; ++i) {
        int64_t off = up(end);
        if (members > 0 && up(off + numels[i]) - start > cap) {
            bucket_start[nb] = start;
            bucket_size[nb] = up(end) - start;
            ++nb;
            start = up(end);
            off = start;
            members = 0;
        }
        offsets[i] = off;
        bucket_of[i] = nb;
        end = off + numels[i];
        ++members;
    }
    if (members > 0) {
        bucket_start[nb] = start;
        bucket_size[nb] = up(end) - start;
        ++nb;
    }
    *n_buckets = nb;
    *total = up(end);
    return DS_OK;
}

ds_status ds_partition_range(int64_t total, int32_t world, int32_t rank, int64_t align, int64_t* start,
                             int64_t* count)
{
    if (!size_ok(total) || world < 1 || rank < 0 || rank >= world || align < 1 || align > kMaxElems)
        return DS_ERR_SIZE;
    if (start == nullptr || count == nullptr)
        return DS_ERR_NULL;
    int64_t per = (total + world - 1) / world;
    per = (per + align - 1) / align * align;
    // rank * per, clamped to total without forming a product beyond it
    const int64_t s0 = (per == 0 || rank > total / per) ? total : static_cast<int64_t>(rank) * per;
    int64_t c = total - s0;
    if (c > per)
        c = per;
    *start = s0;
    *count = c;
    return DS_OK;
}

}  // extern "C"
