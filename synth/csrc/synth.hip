// synth.hip -- device side of the seeded synthetic-input generator, plus two
// data-movement kernels used as bandwidth references.  No optimizer
// arithmetic lives here: these kernels draw numbers and move bytes.
//
// Element i of stream `key` is SplitMix64's output for state
// key + (i + 1) * 0x9E3779B97F4A7C15 (Steele, Lea and Flood, OOPSLA 2014),
// mapped through a host-built lookup table, so the host generator in
// synth/__init__.py produces identical bits for any element.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__device__ __forceinline__ uint16_t grad_at(uint64_t key, int64_t idx, const uint16_t* table,
                                            const uint16_t* tail, uint32_t tail_thresh)
{
    uint64_t z = mix64(key + (uint64_t)(idx + 1) * kGolden);
    uint32_t j = (uint32_t)(z & 0xFFFFu);
    bool heavy = (uint32_t)(z >> 32) < tail_thresh;
    return heavy ? tail[j] : table[j];
}

__device__ __forceinline__ float master_at(uint64_t key, int64_t idx, const uint32_t* table)
{
    uint64_t z = mix64(key + (uint64_t)(idx + 1) * kGolden);
    uint32_t bits = table[z & 0xFFFFu] ^ (uint32_t)((z >> 16) & 0xFFu);
    return __uint_as_float(bits);
}

__global__ __launch_bounds__(256) void fill_grad16_kernel(uint16_t* out, int64_t n, int64_t start,
                                                          uint64_t key, const uint16_t* table,
                                                          const uint16_t* tail, uint32_t tail_thresh)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t n4 = n / 4;
    uint2* out4 = reinterpret_cast<uint2*>(out);
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < n4; q += stride) {
        int64_t e = start + 4 * q;
        uint32_t h0 = grad_at(key, e + 0, table, tail, tail_thresh);
        uint32_t h1 = grad_at(key, e + 1, table, tail, tail_thresh);
        uint32_t h2 = grad_at(key, e + 2, table, tail, tail_thresh);
        uint32_t h3 = grad_at(key, e + 3, table, tail, tail_thresh);
        out4[q] = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
    }
    for (int64_t i = 4 * n4 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        out[i] = grad_at(key, start + i, table, tail, tail_thresh);
}

__global__ __launch_bounds__(256) void fill_grad16_unaligned_kernel(
    uint16_t* out, int64_t n, int64_t start, uint64_t key, const uint16_t* table,
    const uint16_t* tail, uint32_t tail_thresh)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        out[i] = grad_at(key, start + i, table, tail, tail_thresh);
}

__global__ __launch_bounds__(256) void fill_master32_kernel(float* out, int64_t n, int64_t start,
                                                            uint64_t key, const uint32_t* table)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        out[i] = master_at(key, start + i, table);
}

// Plain copy, one 16-byte vector per lane, 64-lane blocks, one block per 64
// vectors (the blocks loop when there are more than 2^25 of them, keeping the
// launch within 2^31 work-items); non-temporal hints.  Of the copy shapes
// measured on MI355X (64-1024 lanes x 1-4 vectors) this one moves the most
// bytes per second.
typedef unsigned copy_u4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(64) void copy_kernel(copy_u4* __restrict__ dst, const copy_u4* __restrict__ src,
                                                  int64_t n16)
{
    const int64_t stride = (int64_t)gridDim.x * 64;
    for (int64_t i = (int64_t)blockIdx.x * 64 + threadIdx.x; i < n16; i += stride)
        __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// Moves the bytes of one optimizer step without computing anything: per
// element it reads a 16-bit value and three fp32 values and writes three fp32
// values (rotated) and the 16-bit value.  Laid out like a streaming optimizer
// kernel: each 256-lane block owns one tile of 4 x 256 quads (4096 elements),
// loads all of it, then stores all of it, with non-temporal hints.
typedef float mix_f4 __attribute__((ext_vector_type(4)));
typedef unsigned mix_u2 __attribute__((ext_vector_type(2)));
// LANES lanes per block, QUADS quads per lane, one tile of LANES x QUADS quads
// per block: 256 x 4 is the optimizer step's tiling, 64 x 1 the plain copy's.
template <int LANES, int QUADS>
__global__ __launch_bounds__(LANES) void stream_mix_kernel(const mix_u2* __restrict__ g,
                                                           mix_f4* __restrict__ a,
                                                           mix_f4* __restrict__ b,
                                                           mix_f4* __restrict__ c,
                                                           mix_u2* __restrict__ h, int64_t n4)
{
    constexpr int kMixLanes = LANES, kMixQuads = QUADS;
    const int64_t first = (int64_t)blockIdx.x * (kMixLanes * kMixQuads) + threadIdx.x;
    mix_u2 gv[kMixQuads];
    mix_f4 av[kMixQuads], bv[kMixQuads], cv[kMixQuads];
#pragma unroll
    for (int u = 0; u < kMixQuads; ++u) {
        const int64_t q = first + (int64_t)u * kMixLanes;
        if (q < n4) {
            gv[u] = __builtin_nontemporal_load(g + q);
            av[u] = __builtin_nontemporal_load(a + q);
            bv[u] = __builtin_nontemporal_load(b + q);
            cv[u] = __builtin_nontemporal_load(c + q);
        }
    }
#pragma unroll
    for (int u = 0; u < kMixQuads; ++u) {
        const int64_t q = first + (int64_t)u * kMixLanes;
        if (q < n4) {
            __builtin_nontemporal_store(bv[u], a + q);
            __builtin_nontemporal_store(cv[u], b + q);
            __builtin_nontemporal_store(av[u], c + q);
            __builtin_nontemporal_store(gv[u], h + q);
        }
    }
}

int grid_for(int64_t work_items)
{
    int64_t blocks = (work_items + 255) / 256;
    if (blocks < 1) blocks = 1;
    if (blocks > 16384) blocks = 16384;
    return (int)blocks;
}

}  // namespace

extern "C" {

// Fill out[0..n) with the fp16 gradient draws of elements [start, start+n) of
// stream `key`.  table/tail: device uint16[65536].  Returns a hipError_t code.
int synth_fill_grad16(uint16_t* out, int64_t n, int64_t start, uint64_t key, const uint16_t* table,
                      const uint16_t* tail, uint32_t tail_thresh, void* stream)
{
    if (n <= 0) return 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((reinterpret_cast<uintptr_t>(out) & 7u) == 0)
        fill_grad16_kernel<<<grid_for(n / 4 > 0 ? n / 4 : 1), 256, 0, s>>>(out, n, start, key, table,
                                                                        tail, tail_thresh);
    else
        fill_grad16_unaligned_kernel<<<grid_for(n), 256, 0, s>>>(out, n, start, key, table, tail,
                                                                 tail_thresh);
    return (int)hipGetLastError();
}

int synth_fill_master32(float* out, int64_t n, int64_t start, uint64_t key, const uint32_t* table,
                        void* stream)
{
    if (n <= 0) return 0;
    fill_master32_kernel<<<grid_for(n), 256, 0, static_cast<hipStream_t>(stream)>>>(out, n, start,
                                                                                   key, table);
    return (int)hipGetLastError();
}

// Copy n16 16-byte vectors; both pointers 16-byte aligned.
int synth_copy(void* dst, const void* src, int64_t n16, void* stream)
{
    if (n16 <= 0) return 0;
    if (((reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(src)) & 15u) != 0)
        return (int)hipErrorInvalidValue;
    int64_t blocks = (n16 + 63) / 64;
    if (blocks > (int64_t(1) << 25)) blocks = int64_t(1) << 25;
    copy_kernel<<<(unsigned)blocks, 64, 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<copy_u4*>(dst), static_cast<const copy_u4*>(src), n16);
    return (int)hipGetLastError();
}

// n elements, n a multiple of 4, all pointers 16-byte aligned (g, h: 8-byte).
int synth_stream_mix_shape(const void* g, void* a, void* b, void* c, void* h, int64_t n, int32_t small_tiles,
                           void* stream);

int synth_stream_mix(const void* g, void* a, void* b, void* c, void* h, int64_t n, void* stream)
{
    return synth_stream_mix_shape(g, a, b, c, h, n, 0, stream);
}

// small_tiles = 0: 256 lanes x 4 quads per block; 1: 64 lanes x 1 quad
int synth_stream_mix_shape(const void* g, void* a, void* b, void* c, void* h, int64_t n, int32_t small_tiles,
                           void* stream)
{
    if (n <= 0) return 0;
    if (n % 4 != 0) return (int)hipErrorInvalidValue;
    if (((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b) |
          reinterpret_cast<uintptr_t>(c)) & 15u) != 0 ||
        ((reinterpret_cast<uintptr_t>(g) | reinterpret_cast<uintptr_t>(h)) & 7u) != 0)
        return (int)hipErrorInvalidValue;
    const int64_t n4 = n / 4;
    const int64_t per = small_tiles ? 64 : 256 * 4;
    const int64_t tiles = (n4 + per - 1) / per;
    if (tiles > 0x7FFFFFFF) return (int)hipErrorInvalidValue;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const mix_u2* gp = static_cast<const mix_u2*>(g);
    if (small_tiles)
        stream_mix_kernel<64, 1><<<(unsigned)tiles, 64, 0, s>>>(gp, static_cast<mix_f4*>(a), static_cast<mix_f4*>(b),
                                                                static_cast<mix_f4*>(c), static_cast<mix_u2*>(h), n4);
    else
        stream_mix_kernel<256, 4><<<(unsigned)tiles, 256, 0, s>>>(gp, static_cast<mix_f4*>(a), static_cast<mix_f4*>(b),
                                                                  static_cast<mix_f4*>(c), static_cast<mix_u2*>(h), n4);
    return (int)hipGetLastError();
}

}  // extern "C"
