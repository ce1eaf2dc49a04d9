/*
 * abi_driver.c -- the optimizer step driven from plain C through the C ABI of
 * libdszero.so (include/dszero.h): no Python and no PyTorch in the process.
 * Test infrastructure: tests/test_gpu_c_abi.py writes the inputs, runs this
 * program as a child process and compares its outputs with the oracle.
 *
 *   abi_driver DIR
 *
 * DIR/params.txt   n K steps init_scale window lr beta1 beta2 eps weight_decay max_grad_norm [double]
 *                  (double = 1: ds_adam_step_double_buffered over two copies of the state in place
 *                  of the check, ds_adam_step and ds_update_loss_scale; double = 2, K > 1: micro-batches
 *                  1..K-1 summed by ds_accumulate, the last one folded into the double-buffered pass by
 *                  ds_accumulate_adam_double_buffered, then ds_update_loss_scale_double_buffered; both
 *                  need max_grad_norm = 0)
 * DIR/master.bin   float32[n]                initial fp32 master copy
 * DIR/grads.bin    uint16[steps][K][n]       fp16 gradients, micro-batch by micro-batch
 * writes
 * DIR/master_out.bin, m_out.bin, v_out.bin (float32[n]), p16_out.bin (uint16[n]) of the copy
 *                  that holds the state
 * DIR/scaler.txt   one line per step: last_overflow scale step iter skipped
 *
 * Device memory comes from hipMalloc, the work runs on a stream created here,
 * and every entry point's status is checked; exit status 0 on success.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "dszero.h"

#define CHECK_HIP(call)                                                                   \
    do {                                                                                  \
        hipError_t e_ = (call);                                                           \
        if (e_ != hipSuccess) {                                                           \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));             \
            exit(2);                                                                      \
        }                                                                                 \
    } while (0)

#define CHECK_DS(call)                                                                    \
    do {                                                                                  \
        ds_status s_ = (call);                                                            \
        if (s_ != DS_OK) {                                                                \
            fprintf(stderr, "%s failed: %s\n", #call, ds_status_string(s_));              \
            exit(3);                                                                      \
        }                                                                                 \
    } while (0)

static void* read_file(const char* dir, const char* name, size_t bytes)
{
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "rb");
    if (f == NULL) {
        perror(path);
        exit(4);
    }
    void* buf = malloc(bytes > 0 ? bytes : 1);
    if (buf == NULL || fread(buf, 1, bytes, f) != bytes) {
        fprintf(stderr, "%s: short read\n", path);
        exit(4);
    }
    fclose(f);
    return buf;
}

static void write_file(const char* dir, const char* name, const void* buf, size_t bytes)
{
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "wb");
    if (f == NULL || fwrite(buf, 1, bytes, f) != bytes) {
        fprintf(stderr, "%s: write failed\n", path);
        exit(4);
    }
    fclose(f);
}

int main(int argc, char** argv)
{
    if (argc != 2) {
        fprintf(stderr, "usage: %s DIR\n", argv[0]);
        return 1;
    }
    const char* dir = argv[1];
    long long n_ll, K_l, steps_l, window_l, double_l = 0;
    float init_scale, lr, b1, b2, eps, wd, clip;
    {
        char path[4096];
        snprintf(path, sizeof path, "%s/params.txt", dir);
        FILE* f = fopen(path, "r");
        int got = f == NULL ? 0 : fscanf(f, "%lld %lld %lld %f %lld %f %f %f %f %f %f %lld", &n_ll, &K_l, &steps_l,
                                         &init_scale, &window_l, &lr, &b1, &b2, &eps, &wd, &clip, &double_l);
        if (got != 11 && got != 12) {
            fprintf(stderr, "%s: bad parameters\n", path);
            return 4;
        }
        fclose(f);
    }
    const int dbl = double_l != 0;
    const int fold_last = double_l == 2;
    if ((dbl && clip > 0.0f) || (fold_last && K_l < 2)) {
        fprintf(stderr, "the double-buffered step takes no clipping; folding the last micro-batch needs K > 1\n");
        return 4;
    }
    const int64_t n = n_ll;
    const int32_t K = (int32_t)K_l, steps = (int32_t)steps_l;
    /* micro-batch slots of the gradient buffer start 16-byte aligned */
    const size_t stride = ((size_t)n + 7) & ~(size_t)7;

    /* a rejected call has no effect and names its error */
    if (ds_adam_step(NULL, NULL, NULL, NULL, NULL, DS_FP16, NULL, DS_FP16, -1, lr, b1, b2, eps, wd, clip, K,
                     NULL) != DS_ERR_SIZE) {
        fprintf(stderr, "negative size not rejected\n");
        return 5;
    }
    printf("rejected as expected: %s\n", ds_status_string(DS_ERR_SIZE));

    float* h_master = read_file(dir, "master.bin", 4 * (size_t)n);
    uint16_t* h_grads = read_file(dir, "grads.bin", 2 * (size_t)n * (size_t)K * (size_t)steps);

    hipStream_t stream;
    CHECK_HIP(hipStreamCreate(&stream));
    float *master, *m, *v, *acc = NULL;
    uint16_t *p16, *g16;
    /* the double-buffered step's two copies: copy 0 is master/m/v/p16 */
    float *master2[2], *m2[2], *v2[2];
    uint16_t* p16_2[2];
    void *state, *ws = NULL;
    const size_t ws_bytes = ds_sumsq_workspace_bytes(n);
    CHECK_HIP(hipMalloc((void**)&master, 4 * (size_t)n));
    CHECK_HIP(hipMalloc((void**)&m, 4 * (size_t)n));
    CHECK_HIP(hipMalloc((void**)&v, 4 * (size_t)n));
    CHECK_HIP(hipMalloc((void**)&p16, 2 * (size_t)n));
    CHECK_HIP(hipMalloc((void**)&g16, 2 * stride * (size_t)K));
    CHECK_HIP(hipMalloc(&state, ds_scaler_size()));
    if (K > 1)
        CHECK_HIP(hipMalloc((void**)&acc, 4 * (size_t)n));
    if (clip > 0.0f)
        CHECK_HIP(hipMalloc(&ws, ws_bytes > 0 ? ws_bytes : 8));
    CHECK_HIP(hipMemcpyAsync(master, h_master, 4 * (size_t)n, hipMemcpyHostToDevice, stream));
    CHECK_HIP(hipMemsetAsync(m, 0, 4 * (size_t)n, stream));
    CHECK_HIP(hipMemsetAsync(v, 0, 4 * (size_t)n, stream));
    CHECK_HIP(hipMemsetAsync(p16, 0, 2 * (size_t)n, stream));
    CHECK_DS(ds_state_init((ds_scaler*)state, init_scale, 1.0f, (int32_t)window_l, 1, 0, 1, stream));
    master2[0] = master;
    m2[0] = m;
    v2[0] = v;
    p16_2[0] = p16;
    if (dbl) {   /* copy 1 holds no state until the first applied step writes it */
        CHECK_HIP(hipMalloc((void**)&master2[1], 4 * (size_t)n));
        CHECK_HIP(hipMalloc((void**)&m2[1], 4 * (size_t)n));
        CHECK_HIP(hipMalloc((void**)&v2[1], 4 * (size_t)n));
        CHECK_HIP(hipMalloc((void**)&p16_2[1], 2 * (size_t)n));
    }

    char path[4096];
    snprintf(path, sizeof path, "%s/scaler.txt", dir);
    FILE* trace = fopen(path, "w");
    if (trace == NULL) {
        perror(path);
        return 4;
    }
    for (int32_t s = 0; s < steps; ++s) {
        for (int32_t k = 0; k < K; ++k) {
            const uint16_t* hg = h_grads + ((size_t)s * (size_t)K + (size_t)k) * (size_t)n;
            CHECK_HIP(hipMemcpyAsync(g16 + (size_t)k * stride, hg, 2 * (size_t)n, hipMemcpyHostToDevice, stream));
        }
        const void* grad = g16;
        ds_dtype gdt = DS_FP16;
        if (K == 1 && dbl) {
            /* the check runs inside the double-buffered pass */
        } else if (fold_last) {
            /* micro-batches 1..K-1 into the running sum; the last one goes into the pass below */
            for (int32_t k = 0; k < K - 1; ++k)
                CHECK_DS(ds_accumulate(acc, g16 + (size_t)k * stride, DS_FP16, n, k == 0, NULL, stream));
        } else if (K == 1) {
            if (clip > 0.0f)
                CHECK_DS(ds_check_overflow_sumsq((ds_scaler*)state, g16, DS_FP16, n, ws, ws_bytes, stream));
            else
                CHECK_DS(ds_check_overflow((ds_scaler*)state, g16, DS_FP16, n, stream));
        } else if (s % 2 == 1 && K <= 8) {
            /* odd steps: the K micro-batches folded in one pass (same result) */
            const uint16_t* list[8];
            for (int32_t k = 0; k < K; ++k)
                list[k] = g16 + (size_t)k * stride;
            CHECK_DS(ds_accumulate_multi(acc, list, K, DS_FP16, n, 1, (ds_scaler*)state, clip > 0.0f ? ws : NULL,
                                         clip > 0.0f ? ws_bytes : 0, stream));
            grad = acc;
            gdt = DS_FP32;
        } else {
            for (int32_t k = 0; k < K; ++k) {
                const uint16_t* gk = g16 + (size_t)k * stride;
                if (k == K - 1 && clip > 0.0f)
                    CHECK_DS(ds_accumulate_sumsq(acc, gk, DS_FP16, n, k == 0, (ds_scaler*)state, ws, ws_bytes,
                                                 stream));
                else
                    CHECK_DS(ds_accumulate(acc, gk, DS_FP16, n, k == 0, k == K - 1 ? (ds_scaler*)state : NULL,
                                           stream));
            }
            grad = acc;
            gdt = DS_FP32;
        }
        if (fold_last) {
            const uint16_t* last[1] = {g16 + (size_t)(K - 1) * stride};
            CHECK_DS(ds_accumulate_adam_double_buffered((ds_scaler*)state, master2, m2, v2, p16_2, DS_FP16, acc, last,
                                                        1, DS_FP16, n, lr, NULL, b1, b2, eps, wd, K, stream));
            CHECK_DS(ds_update_loss_scale_double_buffered((ds_scaler*)state, stream));
        } else if (dbl) {
            CHECK_DS(ds_adam_step_double_buffered((ds_scaler*)state, master2, m2, v2, p16_2, DS_FP16, grad, gdt, n,
                                                  lr, NULL, b1, b2, eps, wd, K, stream));
        } else {
            CHECK_DS(ds_adam_step((const ds_scaler*)state, master, m, v, p16, DS_FP16, grad, gdt, n, lr, b1, b2,
                                  eps, wd, clip, K, stream));
            CHECK_DS(ds_update_loss_scale((ds_scaler*)state, stream));
        }
        ds_scaler sc;
        CHECK_DS(ds_state_read((const ds_scaler*)state, &sc, stream));
        fprintf(trace, "%u %.9g %lld %lld %lld\n", sc.last_overflow, (double)sc.scale, (long long)sc.step,
                (long long)sc.iter, (long long)sc.skipped);
    }
    fclose(trace);

    float* out = malloc(4 * (size_t)n);
    uint16_t* out16 = malloc(2 * (size_t)n);
    if (out == NULL || out16 == NULL)
        return 4;
    int cur = 0;
    if (dbl) {
        ds_scaler sc;
        CHECK_DS(ds_state_read((const ds_scaler*)state, &sc, stream));
        cur = (int)(sc.current & 1u);
        printf("current copy: %d\n", cur);
    }
    CHECK_HIP(hipStreamSynchronize(stream));
    CHECK_HIP(hipMemcpy(out, master2[cur], 4 * (size_t)n, hipMemcpyDeviceToHost));
    write_file(dir, "master_out.bin", out, 4 * (size_t)n);
    CHECK_HIP(hipMemcpy(out, m2[cur], 4 * (size_t)n, hipMemcpyDeviceToHost));
    write_file(dir, "m_out.bin", out, 4 * (size_t)n);
    CHECK_HIP(hipMemcpy(out, v2[cur], 4 * (size_t)n, hipMemcpyDeviceToHost));
    write_file(dir, "v_out.bin", out, 4 * (size_t)n);
    CHECK_HIP(hipMemcpy(out16, p16_2[cur], 2 * (size_t)n, hipMemcpyDeviceToHost));
    write_file(dir, "p16_out.bin", out16, 2 * (size_t)n);
    if (dbl) {
        CHECK_HIP(hipFree(master2[1]));
        CHECK_HIP(hipFree(m2[1]));
        CHECK_HIP(hipFree(v2[1]));
        CHECK_HIP(hipFree(p16_2[1]));
    }

    CHECK_HIP(hipFree(master));
    CHECK_HIP(hipFree(m));
    CHECK_HIP(hipFree(v));
    CHECK_HIP(hipFree(p16));
    CHECK_HIP(hipFree(g16));
    CHECK_HIP(hipFree(state));
    if (acc != NULL)
        CHECK_HIP(hipFree(acc));
    if (ws != NULL)
        CHECK_HIP(hipFree(ws));
    CHECK_HIP(hipStreamDestroy(stream));
    free(out);
    free(out16);
    free(h_master);
    free(h_grads);
    printf("abi_driver: %d steps of %lld elements (K=%d) done\n", steps, (long long)n, K);
    return 0;
}
