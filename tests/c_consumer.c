/*
 * A plain C11 consumer of include/zshard.h and libzshard.so (built and run by
 * tests/test_abi.py with gcc -std=c11 -Wall -Wextra -Wpedantic -Werror): the
 * header is valid C, the exported names link from C, and the host-only
 * functions and rejecting paths return what the header documents.  No call
 * reaches a kernel launch (there is no GPU here): every device call either
 * fails validation or is an n == 0 no-op.  Pointers are never dereferenced.
 * Exit status 0 and "c consumer: ok" on success; the failing check's number
 * otherwise.
 */
#include <stdint.h>
#include <stdio.h>

#include "zshard.h"

#define CHECK(cond, code) do { if (!(cond)) { fprintf(stderr, "check failed: %s\n", #cond); return code; } } while (0)

int main(void)
{
    zs_shard s;
    CHECK(zero_shard_range(1000003, 8, 3, &s) == ZS_OK, 1);
    CHECK(s.chunk == 125001 && s.start == 375003 && s.end == 500004 && s.padded_total == 1000008, 1);
    CHECK(zero_shard_range(855654400, 64, 17, &s) == ZS_OK && s.start == 227283200 && s.end == 240652800, 1);
    CHECK(zero_shard_range(10, 0, 0, &s) == ZS_EINVAL, 1);

    CHECK(state_tiled_numel(0) == 0 && state_tiled_numel(1) == 3 * ZS_STATE_TILE, 2);
    CHECK(state_tiled_numel(842301952) == 3 * (int64_t)ZS_STATE_TILE * 102821, 2);
    CHECK(grad_norm_sq_workspace_bytes(-1) == -1, 2);

    zs_adamw hp = {3e-4, 0.9, 0.95, 1e-8, 0.1, 1.0 / 64, 1.0, 0.0, 1};
    zs_adamw_scalars sc;
    CHECK(adamw_scalars(&hp, &sc) == ZS_OK && sc.clip == 1 && sc.beta1 == 0.9f, 3);
    hp.step = 0;
    CHECK(adamw_scalars(&hp, &sc) == ZS_EINVAL, 3);
    hp.step = 1;

    float* f = (float*)(uintptr_t)0x7F0000000000ull;      /* fake device addresses */
    CHECK(adamw_step(&hp, f, f, f, f, NULL, 0, NULL, NULL) == ZS_OK, 4);              /* n == 0: no-op */
    CHECK(adamw_step(&hp, f, f + 1, f + 4096, f + 8192, NULL, 16, NULL, NULL) == ZS_EOVERLAP, 4);
    CHECK(adamw_step_tiled(&hp, f + 1, f + 65536, NULL, 16, NULL, NULL) == ZS_EINVAL, 4);   /* state off 16 B */
    CHECK(state_tile(NULL, NULL, NULL, f, 0, NULL) == ZS_OK, 4);
    CHECK(state_untile(f, f + 8, f + 8, NULL, 16, NULL) == ZS_EOVERLAP, 4);
    CHECK(grad_accum(f, f + 1, ZS_F32, 16, 1, NULL) == ZS_EOVERLAP, 4);
    CHECK(flat_pack(NULL, 0, ZS_BF16, NULL, ZS_BF16, 0, NULL) == ZS_OK, 4);
    CHECK(zs_last_hip_error() == 0, 5);
    CHECK(zs_strerror(ZS_EOVERLAP) != NULL, 5);
    printf("c consumer: ok\n");
    return 0;
}
