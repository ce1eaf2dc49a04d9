/*
 * host_checks.c -- every host-only path of libdszero.so, for a build with the
 * host AddressSanitizer and UndefinedBehaviorSanitizer (device code is built
 * as usual; no GPU is used): argument validation of every entry point (each
 * call below fails before any device work), the layout and partition
 * routines on the ragged Llama-like layout and on random layouts, and the
 * status strings.  Exit status 0 when every expectation holds; the
 * sanitizers abort on any memory or undefined-behaviour error.
 */
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "dszero.h"

static int failures = 0;

/* the header's layout of the state, as the Python binding mirrors it */
_Static_assert(sizeof(ds_scaler) == 128, "ds_scaler is 128 bytes");
_Static_assert(offsetof(ds_scaler, overflow) == 28 && offsetof(ds_scaler, step) == 32, "ds_scaler layout");
_Static_assert(offsetof(ds_scaler, last_overflow) == 60 && offsetof(ds_scaler, grad_sumsq) == 64, "ds_scaler layout");
_Static_assert(offsetof(ds_scaler, blocks_done) == 80 && offsetof(ds_scaler, sumsq_blocks_done) == 84,
               "ds_scaler layout");
_Static_assert(offsetof(ds_scaler, current) == 88 && offsetof(ds_scaler, db_tickets) == 96,
               "ds_scaler layout: the 64-bit ticket is 8-byte aligned");

#define EXPECT(cond)                                                   \
    do {                                                               \
        if (!(cond)) {                                                 \
            fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                \
        }                                                              \
    } while (0)

/* fake device addresses: never dereferenced, every call below is rejected */
#define A ((void*)(uintptr_t)0x10000000u)
#define B ((void*)(uintptr_t)0x20000000u)
#define C ((void*)(uintptr_t)0x30000000u)
#define D ((void*)(uintptr_t)0x40000000u)
#define E ((void*)(uintptr_t)0x50000000u)
#define ST ((ds_scaler*)(uintptr_t)0x60000000u)

static void validation(void)
{
    float* f = (float*)A;
    EXPECT(ds_adam_step(ST, f, (float*)B, (float*)C, (uint16_t*)D, DS_FP16, E, DS_FP16, -1, 1e-4f, 0.9f, 0.999f,
                        1e-8f, 0.0f, 0.0f, 1, NULL) == DS_ERR_SIZE);
    EXPECT(ds_adam_step(ST, f, (float*)B, (float*)C, (uint16_t*)D, DS_FP32, E, DS_FP16, 8, 1e-4f, 0.9f, 0.999f,
                        1e-8f, 0.0f, 0.0f, 1, NULL) == DS_ERR_DTYPE);
    EXPECT(ds_adam_step(ST, f, (float*)B, (float*)C, (uint16_t*)D, DS_FP16, E, DS_FP16, 8, 1e-4f, 1.0f, 0.999f,
                        1e-8f, 0.0f, 0.0f, 1, NULL) == DS_ERR_HPARAM);
    EXPECT(ds_adam_step(NULL, f, (float*)B, (float*)C, (uint16_t*)D, DS_FP16, E, DS_FP16, 8, 1e-4f, 0.9f, 0.999f,
                        1e-8f, 0.0f, 0.0f, 1, NULL) == DS_ERR_NULL);
    EXPECT(ds_adam_step(ST, f + 1, (float*)B, (float*)C, (uint16_t*)D, DS_FP16, E, DS_FP16, 8, 1e-4f, 0.9f,
                        0.999f, 1e-8f, 0.0f, 0.0f, 1, NULL) == DS_ERR_ALIGN);
    EXPECT(ds_adam_step(ST, f, f + 4, (float*)C, (uint16_t*)D, DS_FP16, E, DS_FP16, 8, 1e-4f, 0.9f, 0.999f,
                        1e-8f, 0.0f, 0.0f, 1, NULL) == DS_ERR_ALIAS);
    EXPECT(ds_adam_step(ST, f, (float*)B, (float*)C, (uint16_t*)D, DS_FP16, E, DS_FP16, 0, 1e-4f, 0.9f, 0.999f,
                        1e-8f, 0.0f, 0.0f, 1, NULL) == DS_OK);
    EXPECT(ds_adam_step_fused(ST, f, (float*)B, (float*)C, (uint16_t*)D, DS_FP16, E, DS_FP16, -1, 1e-4f, NULL,
                              0.9f, 0.999f, 1e-8f, 0.0f, 0.0f, 1, NULL) == DS_ERR_SIZE);
    /* beyond any device: refused before a byte count is formed from n */
    EXPECT(ds_adam_step_fused(ST, f, (float*)B, (float*)C, (uint16_t*)D, DS_FP16, E, DS_FP16, INT64_MAX, 1e-4f,
                              NULL, 0.9f, 0.999f, 1e-8f, 0.0f, 0.0f, 1, NULL) == DS_ERR_SIZE);
    EXPECT(ds_accumulate(f, (uint16_t*)B, DS_FP16, ((int64_t)1 << 40) + 1, 1, NULL, NULL) == DS_ERR_SIZE);
    EXPECT(ds_check_overflow(ST, E, DS_FP16, INT64_MAX, NULL) == DS_ERR_SIZE);
    ds_lr_schedule bad = {7, 0, 10, 20, 0.0f, 1e-3f};
    EXPECT(ds_adam_step_sched(ST, f, (float*)B, (float*)C, (uint16_t*)D, DS_FP16, E, DS_FP16, 8, &bad, 0.9f,
                              0.999f, 1e-8f, 0.0f, 0.0f, 1, NULL) == DS_ERR_HPARAM);
    EXPECT(ds_adam_step_sched(ST, f, (float*)B, (float*)C, (uint16_t*)D, DS_FP16, E, DS_FP16, 8, NULL, 0.9f,
                              0.999f, 1e-8f, 0.0f, 0.0f, 1, NULL) == DS_ERR_NULL);
    EXPECT(ds_accumulate(f, (uint16_t*)B, DS_FP32, 8, 1, NULL, NULL) == DS_ERR_DTYPE);
    const uint16_t* list[9] = {(uint16_t*)B, (uint16_t*)C, (uint16_t*)D, (uint16_t*)B, (uint16_t*)C,
                               (uint16_t*)D, (uint16_t*)B, (uint16_t*)C, (uint16_t*)D};
    EXPECT(ds_accumulate_multi(f, list, 9, DS_FP16, 8, 1, NULL, NULL, 0, NULL) == DS_ERR_SIZE);
    EXPECT(ds_accumulate_multi(f, list, 0, DS_FP16, 8, 1, NULL, NULL, 0, NULL) == DS_ERR_SIZE);
    EXPECT(ds_accumulate_multi(f, list, 3, DS_FP16, 8, 1, NULL, E, 8, NULL) == DS_ERR_NULL);
    const uint16_t* inside[2] = {(uint16_t*)B, (uint16_t*)(f + 4)};
    EXPECT(ds_accumulate_multi(f, inside, 2, DS_FP16, 64, 1, NULL, NULL, 0, NULL) == DS_ERR_ALIAS);
    EXPECT(ds_accumulate(f, (uint16_t*)f + 2, DS_FP16, 8, 1, NULL, NULL) == DS_ERR_ALIGN);
    EXPECT(ds_accumulate(f, (uint16_t*)(f + 4), DS_FP16, 64, 1, NULL, NULL) == DS_ERR_ALIAS);
    EXPECT(ds_check_overflow(ST, E, (ds_dtype)9, 8, NULL) == DS_ERR_DTYPE);
    EXPECT(ds_check_overflow(ST, (char*)E + 8, DS_FP16, 8, NULL) == DS_ERR_ALIGN);
    const size_t ws = ds_sumsq_workspace_bytes(100000);
    EXPECT(ws == 8 * (98 + 1));   /* 98 chunks of 1024 elements, one group of chunk sums */
    EXPECT(ds_check_overflow_sumsq(ST, E, DS_FP16, 100000, A, ws - 8, NULL) == DS_ERR_SIZE);
    EXPECT(ds_accumulate_sumsq(f, (uint16_t*)B, DS_FP16, 100000, 1, ST, NULL, ws, NULL) == DS_ERR_NULL);
    EXPECT(ds_state_init(ST, 0.0f, 1.0f, 1000, 1, 0, 1, NULL) == DS_ERR_HPARAM);
    EXPECT(ds_state_init((ds_scaler*)((char*)ST + 4), 65536.0f, 1.0f, 1000, 1, 0, 1, NULL) == DS_ERR_ALIGN);
    EXPECT(ds_update_loss_scale(NULL, NULL) == DS_ERR_NULL);
    EXPECT(ds_adam_bias_scalars(ST, 1e-4f, 0.9f, 1.5f, (float*)A, NULL) == DS_ERR_HPARAM);
    ds_lr_schedule good = {DS_LR_WARMUP_DECAY, 0, 2000, 100000, 0.0f, 3e-4f};
    EXPECT(ds_lr_scalars(ST, &good, 0.9f, 0.999f, (float*)((char*)ST + 8), NULL) == DS_ERR_ALIAS);
    /* the double-buffered step: two copies of every state array, each rejected path */
    float* c_master[2] = {(float*)A, (float*)((char*)A + 0x100000)};
    float* c_m[2] = {(float*)B, (float*)((char*)B + 0x100000)};
    float* c_v[2] = {(float*)C, (float*)((char*)C + 0x100000)};
    uint16_t* c_p16[2] = {(uint16_t*)D, (uint16_t*)((char*)D + 0x100000)};
    float* c_null[2] = {(float*)B, NULL};
    float* c_odd[2] = {(float*)A, (float*)((char*)A + 0x100004)};
    float* c_alias[2] = {(float*)B, (float*)((char*)A + 16)};   /* inside master copy 0 */
    EXPECT(ds_adam_step_double_buffered(ST, c_master, c_m, c_v, c_p16, DS_FP16, E, DS_FP16, -1, 1e-4f, NULL, 0.9f,
                                        0.999f, 1e-8f, 0.0f, 1, NULL) == DS_ERR_SIZE);
    EXPECT(ds_adam_step_double_buffered(ST, c_master, c_m, c_v, c_p16, DS_FP16, E, DS_FP16, INT64_MAX, 1e-4f, NULL,
                                        0.9f, 0.999f, 1e-8f, 0.0f, 1, NULL) == DS_ERR_SIZE);
    EXPECT(ds_adam_step_double_buffered(ST, c_master, c_m, c_v, c_p16, DS_FP32, E, DS_FP16, 8, 1e-4f, NULL, 0.9f,
                                        0.999f, 1e-8f, 0.0f, 1, NULL) == DS_ERR_DTYPE);
    EXPECT(ds_adam_step_double_buffered(ST, c_master, c_m, c_v, c_p16, DS_FP16, E, DS_FP16, 8, 1e-4f, NULL, 1.0f,
                                        0.999f, 1e-8f, 0.0f, 1, NULL) == DS_ERR_HPARAM);
    EXPECT(ds_adam_step_double_buffered(ST, c_master, c_m, c_v, c_p16, DS_FP16, E, DS_FP16, 8, 1e-4f, &bad, 0.9f,
                                        0.999f, 1e-8f, 0.0f, 1, NULL) == DS_ERR_HPARAM);
    EXPECT(ds_adam_step_double_buffered(NULL, c_master, c_m, c_v, c_p16, DS_FP16, E, DS_FP16, 8, 1e-4f, NULL, 0.9f,
                                        0.999f, 1e-8f, 0.0f, 1, NULL) == DS_ERR_NULL);
    EXPECT(ds_adam_step_double_buffered(ST, c_master, NULL, c_v, c_p16, DS_FP16, E, DS_FP16, 8, 1e-4f, NULL, 0.9f,
                                        0.999f, 1e-8f, 0.0f, 1, NULL) == DS_ERR_NULL);
    EXPECT(ds_adam_step_double_buffered(ST, c_master, c_null, c_v, c_p16, DS_FP16, E, DS_FP16, 8, 1e-4f, NULL, 0.9f,
                                        0.999f, 1e-8f, 0.0f, 1, NULL) == DS_ERR_NULL);
    EXPECT(ds_adam_step_double_buffered(ST, c_odd, c_m, c_v, c_p16, DS_FP16, E, DS_FP16, 8, 1e-4f, NULL, 0.9f,
                                        0.999f, 1e-8f, 0.0f, 1, NULL) == DS_ERR_ALIGN);
    EXPECT(ds_adam_step_double_buffered(ST, c_master, c_alias, c_v, c_p16, DS_FP16, E, DS_FP16, 8, 1e-4f, NULL,
                                        0.9f, 0.999f, 1e-8f, 0.0f, 1, NULL) == DS_ERR_ALIAS);
    EXPECT(ds_adam_step_double_buffered(ST, c_master, c_m, c_v, c_p16, DS_FP16, (char*)A + 0x100000 + 16,
                                        DS_FP16, 8, 1e-4f, NULL, 0.9f, 0.999f, 1e-8f, 0.0f, 1, NULL) == DS_ERR_ALIAS);
    /* the last micro-batches folded into the double-buffered pass, and its scaler update */
    const uint16_t* g1[1] = {(const uint16_t*)E};
    const uint16_t* g8[8] = {(const uint16_t*)E, (const uint16_t*)E, (const uint16_t*)E, (const uint16_t*)E,
                             (const uint16_t*)E, (const uint16_t*)E, (const uint16_t*)E, (const uint16_t*)E};
    const float* sum = (const float*)((char*)E + 0x100000);
    EXPECT(ds_accumulate_adam_double_buffered(ST, c_master, c_m, c_v, c_p16, DS_FP16, sum, g1, 0, DS_FP16, 8, 1e-4f,
                                              NULL, 0.9f, 0.999f, 1e-8f, 0.0f, 8, NULL) == DS_ERR_SIZE);
    EXPECT(ds_accumulate_adam_double_buffered(ST, c_master, c_m, c_v, c_p16, DS_FP16, sum, g1, 1, DS_FP32, 8, 1e-4f,
                                              NULL, 0.9f, 0.999f, 1e-8f, 0.0f, 8, NULL) == DS_ERR_DTYPE);
    EXPECT(ds_accumulate_adam_double_buffered(ST, c_master, c_m, c_v, c_p16, DS_FP16, NULL, g1, 1, DS_FP16, 8, 1e-4f,
                                              NULL, 0.9f, 0.999f, 1e-8f, 0.0f, 8, NULL) == DS_ERR_HPARAM);
    EXPECT(ds_accumulate_adam_double_buffered(ST, c_master, c_m, c_v, c_p16, DS_FP16, sum, g8, 8, DS_FP16, 8, 1e-4f,
                                              NULL, 0.9f, 0.999f, 1e-8f, 0.0f, 8, NULL) == DS_ERR_HPARAM);
    EXPECT(ds_accumulate_adam_double_buffered(ST, c_master, c_null, c_v, c_p16, DS_FP16, sum, g1, 1, DS_FP16, 8,
                                              1e-4f, NULL, 0.9f, 0.999f, 1e-8f, 0.0f, 8, NULL) == DS_ERR_NULL);
    EXPECT(ds_accumulate_adam_double_buffered(ST, c_master, c_m, c_v, c_p16, DS_FP16, (const float*)((char*)A + 16),
                                              g1, 1, DS_FP16, 8, 1e-4f, NULL, 0.9f, 0.999f, 1e-8f, 0.0f, 8,
                                              NULL) == DS_ERR_ALIAS);
    EXPECT(ds_accumulate_adam_double_buffered(ST, c_master, c_m, c_v, c_p16, DS_FP16, NULL, g8, 8, DS_FP16, 0, 1e-4f,
                                              NULL, 0.9f, 0.999f, 1e-8f, 0.0f, 8, NULL) == DS_OK);
    EXPECT(ds_update_loss_scale_double_buffered(NULL, NULL) == DS_ERR_NULL);
    /* the allocation-free check: every rejection comes before the scratch array is looked up */
    EXPECT(ds_check_overflow_sumsq_noalloc(ST, E, DS_FP16, DS_NOALLOC_MAX_ELEMS + 1, NULL) == DS_ERR_SIZE);
    EXPECT(ds_check_overflow_sumsq_noalloc(ST, E, (ds_dtype)9, 8, NULL) == DS_ERR_DTYPE);
    EXPECT(ds_check_overflow_sumsq_noalloc(NULL, E, DS_FP16, 8, NULL) == DS_ERR_NULL);
    EXPECT(ds_check_overflow_sumsq_noalloc(ST, (char*)E + 8, DS_FP16, 8, NULL) == DS_ERR_ALIGN);
    EXPECT(ds_check_overflow_sumsq_noalloc(ST, (void*)ST, DS_FP16, 8, NULL) == DS_ERR_ALIAS);
    for (int s = -2; s < 10; ++s)
        EXPECT(ds_status_string((ds_status)s) != NULL && strlen(ds_status_string((ds_status)s)) > 0);
    EXPECT(ds_scaler_size() == 128);
}

/* The layout rule: tensors keep their order, each starts aligned, a bucket
 * holds whole tensors, and the buckets tile [0, total). */
static void check_layout(const int64_t* numels, int32_t count, int64_t cap, int64_t align)
{
    int64_t* offsets = malloc(sizeof(int64_t) * (size_t)(count > 0 ? count : 1));
    int32_t* bucket_of = malloc(sizeof(int32_t) * (size_t)(count > 0 ? count : 1));
    int64_t* bstart = malloc(sizeof(int64_t) * (size_t)(count > 0 ? count : 1));
    int64_t* bsize = malloc(sizeof(int64_t) * (size_t)(count > 0 ? count : 1));
    int32_t nb = -1;
    int64_t total = -1;
    EXPECT(ds_layout_greedy(numels, count, cap, align, offsets, bucket_of, bstart, bsize, &nb, &total) == DS_OK);
    EXPECT(nb >= 0 && nb <= (count > 0 ? count : 0));
    int64_t covered = 0;
    for (int32_t b = 0; b < nb; ++b) {
        EXPECT(bstart[b] == covered);
        covered += bsize[b];
    }
    EXPECT(covered == total);
    for (int32_t i = 0; i < count; ++i) {
        EXPECT(offsets[i] % align == 0);
        EXPECT(i == 0 || offsets[i] >= offsets[i - 1] + numels[i - 1]);
        const int32_t b = bucket_of[i];
        EXPECT(b >= 0 && b < nb);
        if (b >= 0 && b < nb)
            EXPECT(offsets[i] >= bstart[b] && offsets[i] + numels[i] <= bstart[b] + bsize[b]);
    }
    free(offsets);
    free(bucket_of);
    free(bstart);
    free(bsize);
}

static uint64_t rng_state = 20261202u;
static uint64_t next_u64(void)
{
    /* SplitMix64 */
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static void layouts(void)
{
    /* the ragged Llama-like layout: 32 layers of q, k, v, o, gate, up, down, two norms */
    int64_t ragged[32 * 9];
    for (int l = 0; l < 32; ++l) {
        const int64_t h = 4096, f = 11008;
        const int64_t t[9] = {h * h, h * h, h * h, h * h, f * h, f * h, f * h, h, h};
        memcpy(ragged + 9 * l, t, sizeof t);
    }
    check_layout(ragged, 32 * 9, 200000000, 64);
    int32_t nb = 0;
    int64_t total = 0;
    int64_t offsets[32 * 9], bstart[32 * 9], bsize[32 * 9];
    int32_t bof[32 * 9];
    EXPECT(ds_layout_greedy(ragged, 32 * 9, 200000000, 64, offsets, bof, bstart, bsize, &nb, &total) == DS_OK);
    EXPECT(nb == 38 && total == 6476267520ll);
    for (int trial = 0; trial < 300; ++trial) {
        const int32_t count = (int32_t)(next_u64() % 50);
        int64_t numels[50];
        for (int32_t i = 0; i < count; ++i)
            numels[i] = (int64_t)(next_u64() % 5000);
        check_layout(numels, count, 1 + (int64_t)(next_u64() % 9000), 1 + (int64_t)(next_u64() % 128));
    }
    int64_t neg[2] = {5, -1};
    EXPECT(ds_layout_greedy(neg, 2, 100, 8, offsets, bof, bstart, bsize, &nb, &total) == DS_ERR_SIZE);
    EXPECT(ds_layout_greedy(NULL, 0, 100, 8, NULL, NULL, NULL, NULL, &nb, &total) == DS_OK && nb == 0 && total == 0);
    /* partitions tile [0, total) */
    for (int trial = 0; trial < 300; ++trial) {
        const int64_t tot = (int64_t)(next_u64() % 100000);
        const int32_t world = 1 + (int32_t)(next_u64() % 70);
        const int64_t align = 1 + (int64_t)(next_u64() % 64);
        int64_t end = 0;
        for (int32_t r = 0; r < world; ++r) {
            int64_t start = -1, count = -1;
            EXPECT(ds_partition_range(tot, world, r, align, &start, &count) == DS_OK);
            EXPECT(count >= 0 && (count == 0 || start == end));
            if (count > 0)
                end = start + count;
        }
        EXPECT(end == tot);
    }
    int64_t s0, c0;
    /* the extremes the validation admits: no signed overflow (UBSan checks) */
    const int64_t most = (int64_t)1 << 40;
    EXPECT(ds_partition_range(most, INT32_MAX, INT32_MAX - 1, most, &s0, &c0) == DS_OK && s0 == most && c0 == 0);
    EXPECT(ds_partition_range(most, INT32_MAX, 0, 8, &s0, &c0) == DS_OK && s0 == 0 && c0 > 0);
    EXPECT(ds_partition_range(most + 1, 2, 0, 8, &s0, &c0) == DS_ERR_SIZE);
    int64_t huge[2] = {INT64_MAX, INT64_MAX};
    EXPECT(ds_layout_greedy(huge, 2, 100, 8, offsets, bof, bstart, bsize, &nb, &total) == DS_ERR_SIZE);
    int64_t edge[2] = {most / 2 - 64, most / 2 - 64};
    EXPECT(ds_layout_greedy(edge, 2, most, 64, offsets, bof, bstart, bsize, &nb, &total) == DS_OK &&
           total == most - 128 && nb == 1);
    EXPECT(ds_partition_range(10, 0, 0, 8, &s0, &c0) == DS_ERR_SIZE);
    EXPECT(ds_partition_range(10, 4, 4, 8, &s0, &c0) == DS_ERR_SIZE);
}

int main(void)
{
    validation();
    layouts();
    if (failures != 0) {
        fprintf(stderr, "host_checks: %d expectation(s) failed\n", failures);
        return 1;
    }
    printf("host_checks: all host paths ok\n");
    return 0;
}
