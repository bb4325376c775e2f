/*
 * Drives every oracle function under AddressSanitizer and
 * UndefinedBehaviorSanitizer (built and run by tests/test_sanitizers.py).
 * Every buffer is allocated at its exact size, so an access one element past
 * the end is reported; special values (signed zeros, subnormals, huge values,
 * inf, NaN) go through the arithmetic.  Exit status 0: no finding and every
 * return code as documented.
 */
#include "../../oracle/oracle.c"

#include <stdio.h>

static uint32_t rng_state = 12345u;
static float frand(void)   /* uniform in [-1, 1) */
{
    rng_state = rng_state * 1664525u + 1013904223u;
    return (float)(rng_state >> 8) * (1.0f / 8388608.0f) - 1.0f;
}

static float special(int k)
{
    static const float s[] = {0.0f, -0.0f, 1e-45f, -1e-40f, 3e-39f, 1e20f, 3e38f, -3.4e38f, INFINITY, -INFINITY};
    if (k % 13 == 12) return NAN;
    return s[k % 10];
}

static void* xmalloc(size_t bytes)
{
    void* p = malloc(bytes ? bytes : 1);
    if (!p) exit(90);
    return p;
}

#define CHECK(cond, code) do { if (!(cond)) { fprintf(stderr, "check failed: %s\n", #cond); return code; } } while (0)

int main(void)
{
    /* shard ranges, every rank of small worlds, and the rejected arguments */
    for (int64_t T = 0; T <= 70; ++T)
        for (int32_t N = 1; N <= 9; ++N)
            for (int32_t r = 0; r < N; ++r) {
                int64_t o[4];
                CHECK(orc_shard_range(T, N, r, o) == 0, 1);
                CHECK(o[1] <= o[2] && o[2] <= T && o[3] == (int64_t)N * o[0], 2);
            }
    {
        int64_t o[4];
        CHECK(orc_shard_range(10, 0, 0, o) == -1, 3);
        CHECK(orc_shard_range(10, 4, 4, o) == -1, 3);
        CHECK(orc_shard_range(-1, 4, 0, o) == -1, 3);
    }

    /* flatten, unflatten and apply over ragged tensors */
    const int64_t numel[] = {0, 1, 3, 7, 1025, 2};
    const int count = 6;
    int64_t total = 0;
    for (int t = 0; t < count; ++t) total += numel[t];
    const int64_t padded = total + 5;
    float* src32[6];
    uint16_t* src16[6];
    void* dst[6];
    for (int t = 0; t < count; ++t) {
        src32[t] = xmalloc(sizeof(float) * numel[t]);
        src16[t] = xmalloc(sizeof(uint16_t) * numel[t]);
        for (int64_t j = 0; j < numel[t]; ++j) {
            src32[t][j] = frand();
            src16[t][j] = orc_bf16_rne(frand());
        }
    }
    float* flat32 = xmalloc(sizeof(float) * padded);
    uint16_t* flat16 = xmalloc(sizeof(uint16_t) * padded);
    CHECK(orc_flat_pack((const void* const*)src32, numel, count, ORC_F32, flat32, ORC_F32, padded) == 0, 4);
    CHECK(orc_flat_pack((const void* const*)src16, numel, count, ORC_BF16, flat32, ORC_F32, padded) == 0, 4);
    CHECK(orc_flat_pack((const void* const*)src16, numel, count, ORC_BF16, flat16, ORC_BF16, padded) == 0, 4);
    CHECK(orc_flat_pack((const void* const*)src32, numel, count, ORC_F32, flat16, ORC_BF16, padded) == -1, 5);
    CHECK(orc_flat_pack((const void* const*)src32, numel, count, ORC_F32, flat32, ORC_F32, total - 1) == -1, 5);
    for (int t = 0; t < count; ++t) dst[t] = src16[t];
    CHECK(orc_flat_unpack(flat32, ORC_F32, dst, numel, count, ORC_BF16) == 0, 6);
    CHECK(orc_flat_unpack(flat16, ORC_BF16, dst, numel, count, ORC_F32) == -1, 6);
    for (int t = 0; t < count; ++t) dst[t] = src32[t];
    CHECK(orc_flat_unpack(flat32, ORC_F32, dst, numel, count, ORC_F32) == 0, 6);
    float* update = xmalloc(sizeof(float) * total);   /* exactly the tensors: padding never read */
    for (int64_t k = 0; k < total; ++k) update[k] = (k % 17 == 0) ? special((int)k) : 1e-3f * frand();
    CHECK(orc_flat_apply_update(update, dst, numel, count, ORC_F32) == 0, 7);
    for (int t = 0; t < count; ++t) dst[t] = src16[t];
    CHECK(orc_flat_apply_update(update, dst, numel, count, ORC_BF16) == 0, 7);
    CHECK(orc_flat_apply_update(update, dst, numel, count, 9) == -1, 7);

    /* accumulation, norm and the three step forms */
    const int64_t sizes[] = {0, 1, 5, 4099};
    for (int si = 0; si < 4; ++si) {
        const int64_t n = sizes[si];
        float* acc = xmalloc(sizeof(float) * n);
        float* g32 = xmalloc(sizeof(float) * n);
        uint16_t* g16 = xmalloc(sizeof(uint16_t) * n);
        float* p = xmalloc(sizeof(float) * n);
        float* m = xmalloc(sizeof(float) * n);
        float* v = xmalloc(sizeof(float) * n);
        float* u = xmalloc(sizeof(float) * n);
        uint16_t* b = xmalloc(sizeof(uint16_t) * n);
        for (int64_t i = 0; i < n; ++i) {
            g32[i] = (i % 11 == 3) ? special((int)i) : 1e-3f * frand();
            g16[i] = orc_bf16_rne(1e-3f * frand());
            p[i] = 0.1f * frand();
            m[i] = v[i] = 0.0f;
            b[i] = orc_bf16_rne(p[i]);
        }
        orc_bf16_rne_array(p, b, n);
        CHECK(orc_grad_accum(acc, g16, ORC_BF16, n, 1) == 0, 8);
        CHECK(orc_grad_accum(acc, g32, ORC_F32, n, 0) == 0, 8);
        CHECK(orc_grad_accum(acc, g32, 7, n, 0) == -1, 8);
        const double S = orc_grad_norm_sq(acc, n, 1.0 / 8);
        for (int64_t t = 1; t <= 3; ++t) {
            orc_adamw_hp hp = {3e-4, 0.9, 0.95, 1e-8, 0.1, 1.0 / 8, 1.0, 0.5, t};
            orc_adamw_hp h0 = hp;
            h0.weight_decay = 0.0;
            const double finite = 1.0;
            CHECK(orc_adamw_step(&hp, p, m, v, acc, b, n, &finite) == 0, 9);
            CHECK(orc_adamw_step(&hp, p, m, v, acc, NULL, n, NULL) == 0, 9);
            CHECK(orc_adamw_step(&hp, p, m, v, acc, b, n, &S) >= 0, 9);
            CHECK(orc_adamw_step_no_master(&hp, b, m, v, acc, n, NULL) == 0, 10);
            CHECK(orc_adam_update(&h0, m, v, acc, u, n, &finite) == 0, 11);
            CHECK(orc_adam_update(&hp, m, v, acc, u, n, NULL) == -1, 11);   /* decay refused */
        }
        orc_adamw_hp bad = {3e-4, 1.0, 0.95, 1e-8, 0.1, 1.0, 0.0, 0.0, 1};
        CHECK(orc_adamw_step(&bad, p, m, v, acc, b, n, NULL) == -1, 12);
        bad.beta1 = 0.9;
        bad.step = 0;
        CHECK(orc_adamw_step(&bad, p, m, v, acc, b, n, NULL) == -1, 12);
        const double inf = INFINITY;
        CHECK(orc_adamw_step(&bad, p, m, v, acc, b, n, &inf) == -1, 12);
        bad.step = 1;
        CHECK(orc_adamw_step(&bad, p, m, v, acc, b, n, &inf) == 1, 13);   /* non-finite: skipped */
        (void)orc_clip_coef(S, 0.25, 1.0);
        /* tiled state: exact-size buffer, a tile that divides n and one that does not */
        for (int64_t tile = 1; tile <= 8; tile += 7) {
            const int64_t ts = orc_state_tiled_numel(n, tile);
            CHECK(ts >= 3 * n && ts < 3 * (n + tile), 14);
            float* st = xmalloc(sizeof(float) * ts);
            CHECK(orc_state_tile(p, NULL, v, st, n, tile) == 0, 14);
            CHECK(orc_state_untile(st, p, m, NULL, n, tile) == 0, 14);
            CHECK(orc_state_tile(p, m, v, st, -1, tile) == -1, 14);
            CHECK(orc_state_untile(st, p, m, v, n, 0) == -1, 14);
            free(st);
            const int64_t ms = orc_moments_tiled_numel(n, tile);
            CHECK(ms >= 2 * n && ms < 2 * (n + tile), 14);
            float* mo = xmalloc(sizeof(float) * ms);
            CHECK(orc_moments_tile(m, NULL, mo, n, tile) == 0, 14);
            CHECK(orc_moments_untile(mo, NULL, v, n, tile) == 0, 14);
            CHECK(orc_moments_tile(m, v, mo, n, 0) == -1, 14);
            free(mo);
        }
        free(acc); free(g32); free(g16); free(p); free(m); free(v); free(u); free(b);
    }
    for (int t = 0; t < count; ++t) {
        free(src32[t]);
        free(src16[t]);
    }
    free(flat32); free(flat16); free(update);
    printf("oracle sanitizer drive: ok\n");
    return 0;
}
