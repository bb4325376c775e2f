/*
 * One rank's optimizer step driven from C through libzshard.so on the GPU,
 * checked against the oracle (liboracle.so, linked here as test
 * infrastructure).  Built and run by tests/test_gpu_c_abi.py with gcc
 * -std=c11: the C ABI used the way the header documents it, with device
 * memory from hipMalloc and the default stream.
 *
 * A ragged shard of n elements: three bf16 micro-batches accumulated in fp32
 * (grad_accum twice, grad_accum_norm_sq for the last), the master tiled into
 * the tiled state (state_tile), one clipped AdamW step (adamw_step_tiled) with
 * the bf16 re-cast, then state_untile.  Inputs come from a counter-based
 * generator in this file and feed both sides.  The GPU norm must be within
 * 1e-5 of the oracle's; the step, handed the oracle's norm, must be
 * bit-identical to the oracle's (accumulator, master, moments, bf16 output).
 * The same three accumulations once more with grad_accum_norm_sq_noalloc for
 * the last (no workspace) must give the same accumulator and norm bit for bit.
 * And the one-pass form of the same step: two accumulations, then
 * grad_sum_norm_sq and adamw_step_tiled_sum on accumulator + third gradient:
 * the same norm bit for bit, the same state and bf16 output as the oracle's,
 * the accumulator left holding the first two micro-batches' sum.
 * Run with the argument "contiguous", the streamed buffers (state, master,
 * moments, accumulators, gradients, bf16 outputs) are carved from one
 * hipExtMallocWithFlags(..., hipDeviceMallocContiguous) block, 256-byte
 * aligned, as the header's placement note advises (the norms and the
 * workspace stay hipMalloc'd, and the block is never freed: the process's
 * end releases it); every check is the same.
 * Prints "c gpu step: ok" and exits 0, else the number of the failed check.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "zshard.h"

/* oracle (tests only) */
typedef struct {
    double lr, beta1, beta2, eps, weight_decay, grad_scale, max_norm, extra_norm_sq;
    int64_t step;
} orc_adamw_hp;
int orc_grad_accum(float* acc, const void* grad, int32_t grad_dtype, int64_t n, int32_t overwrite);
double orc_grad_norm_sq(const float* acc, int64_t n, double grad_scale);
int orc_adamw_step(const orc_adamw_hp* hp, float* master, float* exp_avg, float* exp_avg_sq, const float* grad,
                   uint16_t* param_bf16, int64_t n, const double* norm_sq);

#define CHECK(cond, code) do { if (!(cond)) { fprintf(stderr, "check %d failed: %s\n", code, #cond); return code; } } while (0)
#define HIPOK(x, code) CHECK((x) == hipSuccess, code)

/* splitmix64 of a counter: a uniform value in [0, 1) */
static double uniform(uint64_t k)
{
    uint64_t z = k * 0x9E3779B97F4A7C15ull + 0x5EED;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (double)(z >> 11) * (1.0 / 9007199254740992.0);
}

static uint16_t bf16_bits_trunc(float x)   /* an input value: the top half of x */
{
    uint32_t u;
    memcpy(&u, &x, 4);
    return (uint16_t)(u >> 16);
}

/* device memory for a streamed buffer: from the block when one is given (the
 * next 256-byte-aligned bytes), else its own hipMalloc */
static int dev_alloc(void** p, size_t bytes, char* block, size_t* used, size_t cap)
{
    if (block == NULL) return hipMalloc(p, bytes) == hipSuccess ? 0 : -1;
    const size_t at = (*used + 255) / 256 * 256;
    if (at + bytes > cap) return -1;
    *p = block + at;
    *used = at + bytes;
    return 0;
}

int main(int argc, char** argv)
{
    const int contiguous = argc > 1 && strcmp(argv[1], "contiguous") == 0;
    const int64_t n = 100003;
    const int M = 3;
    const double scale = 1.0 / 24;
    float* p_ref = malloc(sizeof(float) * n);
    float* m_ref = calloc((size_t)n, sizeof(float));
    float* v_ref = calloc((size_t)n, sizeof(float));
    float* acc_ref = malloc(sizeof(float) * n);
    uint16_t* b_ref = malloc(sizeof(uint16_t) * n);
    uint16_t* g = malloc(sizeof(uint16_t) * n * M);
    float* back = malloc(sizeof(float) * n);
    uint16_t* back16 = malloc(sizeof(uint16_t) * n);
    CHECK(p_ref && m_ref && v_ref && acc_ref && b_ref && g && back && back16, 1);
    for (int64_t i = 0; i < n; ++i) p_ref[i] = (float)(0.2 * uniform((uint64_t)i) - 0.1);
    for (int64_t i = 0; i < n * M; ++i)
        g[i] = bf16_bits_trunc((float)(0.02 * (uniform((uint64_t)(n + i)) + uniform((uint64_t)(2 * n * M + i)) - 1.0)));

    /* device buffers */
    float *d_master, *d_state, *d_acc, *d_p, *d_m, *d_v;
    uint16_t *d_g, *d_b;
    double *d_norm, *d_norm_ref, *d_norm2;
    float *d_acc2, *d_acc3, *d_state2;
    uint16_t* d_b2;
    double* d_norm3;
    void* d_ws;
    const int64_t ws_bytes = grad_accum_norm_sq_workspace_bytes(n);
    const int64_t st = state_tiled_numel(n);
    CHECK(ws_bytes > 0 && st == 3 * (int64_t)ZS_STATE_TILE * ((n + ZS_STATE_TILE - 1) / ZS_STATE_TILE), 2);
    /* the streamed buffers: 7 fp32 arrays of n, 2 tiled states, M + 2 bf16 arrays, each padded to 256 bytes */
    const size_t cap = 7 * (sizeof(float) * n + 256) + 2 * (sizeof(float) * st + 256) +
                       (size_t)(M + 2) * (sizeof(uint16_t) * n + 256);
    char* block = NULL;
    size_t used = 0;
    if (contiguous) HIPOK(hipExtMallocWithFlags((void**)&block, cap, hipDeviceMallocContiguous), 3);
    CHECK(dev_alloc((void**)&d_master, sizeof(float) * n, block, &used, cap) == 0, 3);
    CHECK(dev_alloc((void**)&d_state, sizeof(float) * st, block, &used, cap) == 0, 3);
    CHECK(dev_alloc((void**)&d_acc, sizeof(float) * n, block, &used, cap) == 0, 3);
    CHECK(dev_alloc((void**)&d_p, sizeof(float) * n, block, &used, cap) == 0, 3);
    CHECK(dev_alloc((void**)&d_m, sizeof(float) * n, block, &used, cap) == 0, 3);
    CHECK(dev_alloc((void**)&d_v, sizeof(float) * n, block, &used, cap) == 0, 3);
    CHECK(dev_alloc((void**)&d_g, sizeof(uint16_t) * n * M, block, &used, cap) == 0, 3);
    CHECK(dev_alloc((void**)&d_b, sizeof(uint16_t) * n, block, &used, cap) == 0, 3);
    HIPOK(hipMalloc((void**)&d_norm, sizeof(double)), 3);
    HIPOK(hipMalloc((void**)&d_norm_ref, sizeof(double)), 3);
    HIPOK(hipMalloc((void**)&d_norm2, sizeof(double)), 3);
    CHECK(dev_alloc((void**)&d_acc2, sizeof(float) * n, block, &used, cap) == 0, 3);
    CHECK(dev_alloc((void**)&d_acc3, sizeof(float) * n, block, &used, cap) == 0, 3);
    CHECK(dev_alloc((void**)&d_state2, sizeof(float) * st, block, &used, cap) == 0, 3);
    CHECK(dev_alloc((void**)&d_b2, sizeof(uint16_t) * n, block, &used, cap) == 0, 3);
    HIPOK(hipMalloc((void**)&d_norm3, sizeof(double)), 3);
    HIPOK(hipMalloc(&d_ws, (size_t)ws_bytes), 3);
    HIPOK(hipMemcpy(d_master, p_ref, sizeof(float) * n, hipMemcpyHostToDevice), 4);
    HIPOK(hipMemcpy(d_g, g, sizeof(uint16_t) * n * M, hipMemcpyHostToDevice), 4);

    /* the library's step */
    CHECK(state_tile(d_master, NULL, NULL, d_state, n, NULL) == ZS_OK, 5);
    for (int k = 0; k < M - 1; ++k)
        CHECK(grad_accum(d_acc, d_g + (size_t)k * n, ZS_BF16, n, k == 0, NULL) == ZS_OK, 6);
    CHECK(grad_accum_norm_sq(d_acc, d_g + (size_t)(M - 1) * n, ZS_BF16, n, 0, scale, d_norm, d_ws, ws_bytes, NULL)
          == ZS_OK, 7);

    /* the oracle's */
    for (int k = 0; k < M; ++k) CHECK(orc_grad_accum(acc_ref, g + (size_t)k * n, 1, n, k == 0) == 0, 8);
    const double S = orc_grad_norm_sq(acc_ref, n, scale);
    double S_gpu = 0.0;
    HIPOK(hipMemcpy(&S_gpu, d_norm, sizeof(double), hipMemcpyDeviceToHost), 9);
    CHECK(fabs(sqrt(S_gpu) - sqrt(S)) <= 1e-5 * sqrt(S), 9);
    HIPOK(hipMemcpy(back, d_acc, sizeof(float) * n, hipMemcpyDeviceToHost), 10);
    CHECK(memcmp(back, acc_ref, sizeof(float) * n) == 0, 10);

    /* the same accumulations with the no-alloc form for the last micro-batch */
    for (int k = 0; k < M - 1; ++k)
        CHECK(grad_accum(d_acc2, d_g + (size_t)k * n, ZS_BF16, n, k == 0, NULL) == ZS_OK, 20);
    CHECK(grad_accum_norm_sq_noalloc(d_acc2, d_g + (size_t)(M - 1) * n, ZS_BF16, n, 0, scale, d_norm2, NULL)
          == ZS_OK, 20);
    CHECK(grad_accum_norm_sq_noalloc(d_acc2, d_g, ZS_BF16, ZS_NOALLOC_MAX_ELEMS + 1, 0, scale, d_norm2, NULL)
          == ZS_EINVAL, 20);
    double S_noalloc = 0.0;
    HIPOK(hipMemcpy(&S_noalloc, d_norm2, sizeof(double), hipMemcpyDeviceToHost), 21);
    CHECK(memcmp(&S_noalloc, &S_gpu, sizeof(double)) == 0, 21);
    HIPOK(hipMemcpy(back, d_acc2, sizeof(float) * n, hipMemcpyDeviceToHost), 22);
    CHECK(memcmp(back, acc_ref, sizeof(float) * n) == 0, 22);

    /* the one-pass form: the third micro-batch folded into the norm and the step */
    CHECK(state_tile(d_master, NULL, NULL, d_state2, n, NULL) == ZS_OK, 23);
    for (int k = 0; k < M - 1; ++k)
        CHECK(grad_accum(d_acc3, d_g + (size_t)k * n, ZS_BF16, n, k == 0, NULL) == ZS_OK, 23);
    CHECK(grad_sum_norm_sq(d_acc3, d_g + (size_t)(M - 1) * n, ZS_BF16, n, 0, scale, d_norm3, d_ws, ws_bytes, NULL)
          == ZS_OK, 23);
    double S_one = 0.0;
    HIPOK(hipMemcpy(&S_one, d_norm3, sizeof(double), hipMemcpyDeviceToHost), 24);
    CHECK(memcmp(&S_one, &S_gpu, sizeof(double)) == 0, 24);

    const double max_norm = 0.5 * sqrt(S), extra = 0.2 * S;   /* the clip applies */
    zs_adamw hp = {3e-4, 0.9, 0.95, 1e-8, 0.1, scale, max_norm, extra, 1};
    orc_adamw_hp ohp = {3e-4, 0.9, 0.95, 1e-8, 0.1, scale, max_norm, extra, 1};
    HIPOK(hipMemcpy(d_norm_ref, &S, sizeof(double), hipMemcpyHostToDevice), 11);
    CHECK(adamw_step_tiled(&hp, d_state, d_acc, d_b, n, d_norm_ref, NULL) == ZS_OK, 11);
    CHECK(orc_adamw_step(&ohp, p_ref, m_ref, v_ref, acc_ref, b_ref, n, &S) == 0, 12);
    CHECK(state_untile(d_state, d_p, d_m, d_v, n, NULL) == ZS_OK, 13);
    HIPOK(hipDeviceSynchronize(), 14);
    HIPOK(hipMemcpy(back, d_p, sizeof(float) * n, hipMemcpyDeviceToHost), 15);
    CHECK(memcmp(back, p_ref, sizeof(float) * n) == 0, 15);
    HIPOK(hipMemcpy(back, d_m, sizeof(float) * n, hipMemcpyDeviceToHost), 16);
    CHECK(memcmp(back, m_ref, sizeof(float) * n) == 0, 16);
    HIPOK(hipMemcpy(back, d_v, sizeof(float) * n, hipMemcpyDeviceToHost), 17);
    CHECK(memcmp(back, v_ref, sizeof(float) * n) == 0, 17);
    HIPOK(hipMemcpy(back16, d_b, sizeof(uint16_t) * n, hipMemcpyDeviceToHost), 18);
    CHECK(memcmp(back16, b_ref, sizeof(uint16_t) * n) == 0, 18);
    CHECK(adamw_step_tiled_sum(&hp, d_state2, d_acc3, d_g + (size_t)(M - 1) * n, ZS_BF16, d_b2, n, d_norm_ref, NULL)
          == ZS_OK, 25);
    CHECK(state_untile(d_state2, d_p, d_m, d_v, n, NULL) == ZS_OK, 25);
    HIPOK(hipDeviceSynchronize(), 25);
    HIPOK(hipMemcpy(back, d_p, sizeof(float) * n, hipMemcpyDeviceToHost), 26);
    CHECK(memcmp(back, p_ref, sizeof(float) * n) == 0, 26);
    HIPOK(hipMemcpy(back, d_m, sizeof(float) * n, hipMemcpyDeviceToHost), 26);
    CHECK(memcmp(back, m_ref, sizeof(float) * n) == 0, 26);
    HIPOK(hipMemcpy(back, d_v, sizeof(float) * n, hipMemcpyDeviceToHost), 26);
    CHECK(memcmp(back, v_ref, sizeof(float) * n) == 0, 26);
    HIPOK(hipMemcpy(back16, d_b2, sizeof(uint16_t) * n, hipMemcpyDeviceToHost), 27);
    CHECK(memcmp(back16, b_ref, sizeof(uint16_t) * n) == 0, 27);
    /* the accumulator holds the first M - 1 micro-batches' sum */
    for (int k = 0; k < M - 1; ++k) CHECK(orc_grad_accum(acc_ref, g + (size_t)k * n, 1, n, k == 0) == 0, 28);
    HIPOK(hipMemcpy(back, d_acc3, sizeof(float) * n, hipMemcpyDeviceToHost), 28);
    CHECK(memcmp(back, acc_ref, sizeof(float) * n) == 0, 28);
    CHECK(zs_last_hip_error() == 0, 19);

    if (!contiguous) {   /* a contiguous block is never freed: the process's end releases it */
        hipFree(d_master); hipFree(d_state); hipFree(d_acc); hipFree(d_p); hipFree(d_m); hipFree(d_v);
        hipFree(d_g); hipFree(d_b); hipFree(d_acc2); hipFree(d_acc3); hipFree(d_state2); hipFree(d_b2);
    }
    hipFree(d_norm); hipFree(d_norm_ref); hipFree(d_ws); hipFree(d_norm2); hipFree(d_norm3);
    free(p_ref); free(m_ref); free(v_ref); free(acc_ref); free(b_ref); free(g); free(back); free(back16);
    printf("c gpu step: ok\n");
    return 0;
}
