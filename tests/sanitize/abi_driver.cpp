// Drives the C ABI's host-side validation under AddressSanitizer and
// UndefinedBehaviorSanitizer (built with hipcc, the sanitizers on the host
// pass only; run by tests/test_sanitizers.py on a machine without a GPU).
// Every call below fails validation or is a no-op, so nothing reaches a
// launch and no pointer is dereferenced; tensor lists and chunk tables are
// allocated at their exact sizes, so reading one entry too many is reported.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../../include/zshard.h"
#include "../../fsdp_sharded_optimizer_amd/csrc/zs_common.h"

#define CHECK(cond, code)                                          \
    do {                                                           \
        if (!(cond)) {                                             \
            std::fprintf(stderr, "check failed: %s\n", #cond);     \
            return code;                                           \
        }                                                          \
    } while (0)

static const uintptr_t FAKE = 0x7F0000000000ull;
static void* fake(uint64_t off) { return reinterpret_cast<void*>(FAKE + off); }

// The norm kernels' partial slots (zs::xcd_slot) are a bijection of [0, nb)
// for every grid size: each partial lands in the workspace, no two share one.
static int check_xcd_slots() {
    std::vector<int64_t> sizes;
    for (int64_t nb = 1; nb <= 2100; ++nb) sizes.push_back(nb);
    for (int64_t nb : {3290242LL, 1645121LL, 205640LL, 397213LL, 8388608LL, 8388607LL}) sizes.push_back(nb);
    for (int64_t nb : sizes) {
        std::vector<unsigned char> seen((size_t)nb, 0);
        for (int64_t b = 0; b < nb; ++b) {
            const int64_t s = zs::xcd_slot(b, nb);
            if (s < 0 || s >= nb || seen[(size_t)s]) return 1;
            seen[(size_t)s] = 1;
        }
    }
    return 0;
}

// The waves of a launch that each take K blocks (zs::xcd_block, grid
// zs::sum_norm_grid) run every block of [0, nb) once, and each block on the
// XCD that would have run it as a one-wave workgroup of its own.
static int check_xcd_blocks() {
    for (int64_t W : {1, 2, 4})
        for (int64_t K : {1, 2, 3, 4, 8})
            for (int64_t nb = 1; nb <= 700; ++nb) {
                std::vector<unsigned char> seen((size_t)nb, 0);
                const int64_t grid = zs::sum_norm_grid(nb, W, K);
                if (grid % 8) return 1;
                for (int64_t B = 0; B < grid; ++B)
                    for (int64_t w = 0; w < W; ++w)
                        for (int64_t k = 0; k < K; ++k) {
                            const int64_t vb = zs::xcd_block(B, w, k, W, K);
                            if (vb < 0) return 2;
                            if (vb >= nb) continue;
                            if (seen[(size_t)vb] || (vb & 7) != (B & 7)) return 3;
                            seen[(size_t)vb] = 1;
                        }
                for (unsigned char c : seen)
                    if (!c) return 4;
            }
    return 0;
}

int main() {
    CHECK(check_xcd_slots() == 0, 30);
    CHECK(check_xcd_blocks() == 0, 32);
    // the no-alloc norm: sizes beyond its scratch and bad arguments, before any device call
    CHECK(grad_accum_norm_sq_noalloc((float*)fake(0), fake(1 << 30), ZS_BF16, ZS_NOALLOC_MAX_ELEMS + 1, 0, 1.0,
                                     (double*)fake(3ull << 30), nullptr) == ZS_EINVAL, 31);
    CHECK(grad_accum_norm_sq_noalloc((float*)fake(0), fake(1 << 30), ZS_BF16, 64, 0, -1.0,
                                     (double*)fake(3ull << 30), nullptr) == ZS_EINVAL, 31);
    CHECK(grad_accum_norm_sq_noalloc(nullptr, fake(1 << 30), ZS_BF16, 64, 0, 1.0, (double*)fake(3ull << 30),
                                     nullptr) == ZS_EINVAL, 31);
    for (int64_t T = 0; T <= 64; ++T)
        for (int32_t N = 1; N <= 9; ++N)
            for (int32_t r = 0; r < N; ++r) {
                zs_shard s;
                CHECK(zero_shard_range(T, N, r, &s) == ZS_OK, 1);
                CHECK(s.start <= s.end && s.end <= T && s.padded_total == (int64_t)N * s.chunk, 2);
            }
    zs_shard s;
    CHECK(zero_shard_range(INT64_MAX, 1, 0, &s) == ZS_OK, 3);
    CHECK(zero_shard_range(INT64_MAX, 3, 2, &s) == ZS_EINVAL, 3);   // 3 * ceil(T/3) overflows
    CHECK(zero_shard_range(INT64_MAX - 1, 3, 2, &s) == ZS_OK && s.end == INT64_MAX - 1, 3);
    CHECK(zero_shard_range(10, 0, 0, &s) == ZS_EINVAL && zero_shard_range(10, 2, 2, nullptr) == ZS_EINVAL, 3);

    CHECK(grad_norm_sq_workspace_bytes(-1) == -1 && grad_accum_norm_sq_workspace_bytes(-5) == -1, 4);
    CHECK(grad_norm_sq_workspace_bytes(INT64_MAX) == -1 && grad_accum_norm_sq_workspace_bytes(INT64_MAX) == -1, 4);
    CHECK(grad_norm_sq_workspace_bytes(int64_t(1) << 39) > 0 && grad_accum_norm_sq_workspace_bytes(int64_t(1) << 39) > 0,
          4);

    zs_adamw hp{3e-4, 0.9, 0.95, 1e-8, 0.1, 1.0, 0.0, 0.0, 1};
    zs_adamw bad = hp;
    bad.beta1 = NAN;
    float* f = static_cast<float*>(fake(0));
    CHECK(adamw_step(&bad, f, f + 1024, f + 2048, f + 4096, nullptr, 16, nullptr, nullptr) == ZS_EINVAL, 5);
    CHECK(adamw_step(&hp, f, f + 2, f + 2048, f + 4096, nullptr, 16, nullptr, nullptr) == ZS_EOVERLAP, 5);
    CHECK(adamw_step(&hp, f, f, f, f, nullptr, 0, nullptr, nullptr) == ZS_OK, 5);
    CHECK(adamw_step(&hp, f, f + 1024, f + 2048, f + 4096, nullptr, int64_t(1) << 40, nullptr, nullptr) ==
              ZS_EINVAL, 5);
    CHECK(adamw_step_no_master(&hp, static_cast<uint16_t*>(fake(1)), f + 1024, f + 2048, f + 4096, 8, nullptr,
                               nullptr) == ZS_EINVAL, 6);
    CHECK(adam_update(&hp, f, f + 1024, f + 2048, f + 4096, 8, nullptr, nullptr) == ZS_EINVAL, 6);   // decay

    // tiled state: sizes near the per-call limit, overlaps with the state's padded end, misalignment
    CHECK(state_tiled_numel(-1) == -1 && state_tiled_numel((int64_t(1) << 39) + 1) == -1, 14);
    CHECK(state_tiled_numel(int64_t(1) << 39) == 3 * (int64_t(1) << 39), 14);
    CHECK(state_tiled_numel(1) == 3 * ZS_STATE_TILE, 14);
    float* st = static_cast<float*>(fake(1ull << 32));
    CHECK(adamw_step_tiled(&bad, st, f, nullptr, 16, nullptr, nullptr) == ZS_EINVAL, 15);
    CHECK(adamw_step_tiled(&hp, st + 1, f, nullptr, 16, nullptr, nullptr) == ZS_EINVAL, 15);   // state off 16 bytes
    CHECK(adamw_step_tiled(&hp, st, st + 3 * ZS_STATE_TILE - 1, nullptr, 16, nullptr, nullptr) == ZS_EOVERLAP, 15);
    CHECK(adamw_step_tiled(&hp, st, f, nullptr, int64_t(1) << 40, nullptr, nullptr) == ZS_EINVAL, 15);
    CHECK(adamw_step_tiled(&hp, st, f, nullptr, 0, nullptr, nullptr) == ZS_OK, 15);
    CHECK(adamw_step_tiled_dev(nullptr, st, f, nullptr, 16, nullptr, nullptr) == ZS_EINVAL, 15);
    CHECK(state_tile(f, nullptr, st + 100, st, 16, nullptr) == ZS_EOVERLAP, 16);
    CHECK(state_tile(f, nullptr, nullptr, st + 2, 16, nullptr) == ZS_EINVAL, 16);
    CHECK(state_untile(st, f, f + 8, nullptr, 16, nullptr) == ZS_EOVERLAP, 16);
    CHECK(state_untile(st, f, nullptr, nullptr, int64_t(1) << 40, nullptr) == ZS_EINVAL, 16);
    CHECK(state_untile(st, nullptr, nullptr, nullptr, 0, nullptr) == ZS_OK, 16);
    CHECK(moments_tiled_numel(1) == 2 * ZS_STATE_TILE && moments_tiled_numel(-1) == -1, 17);
    CHECK(moments_tile(f, nullptr, st + 2, 16, nullptr) == ZS_EINVAL, 17);
    CHECK(moments_untile(st, f, f + 4, 16, nullptr) == ZS_EOVERLAP, 17);
    CHECK(adam_update_tiled(&hp, st, f, f + 4096, 16, nullptr, nullptr) == ZS_EINVAL, 17);   // decay refused
    CHECK(adamw_step_no_master_tiled(&hp, static_cast<uint16_t*>(fake(1)), st, f, 16, nullptr, nullptr) ==
              ZS_EINVAL, 17);

    CHECK(grad_accum(f, f + 1, 3, 8, 0, nullptr) == ZS_EINVAL, 7);
    CHECK(grad_accum(f, f + 1, ZS_F32, 8, 0, nullptr) == ZS_EOVERLAP, 7);
    CHECK(grad_accum(f, f + 1, ZS_F32, 0, 0, nullptr) == ZS_OK, 7);
    double* d = static_cast<double*>(fake(1 << 20));
    CHECK(grad_norm_sq(f, 1 << 20, 1.0, d, d + 1, 8, nullptr) == ZS_EWORKSPACE, 8);   // needs 8 KiB
    CHECK(grad_accum_norm_sq(f, f + 4096, ZS_BF16, 1 << 16, 1, 1.0, d, d + 8, 16, nullptr) == ZS_EWORKSPACE, 8);

    // the one-pass last micro-batch: a missing accumulator only where one is read, overlaps, limits
    uint16_t* gb = static_cast<uint16_t*>(fake(1ull << 28));
    CHECK(grad_sum_norm_sq(nullptr, gb, ZS_BF16, 1 << 16, 0, 1.0, d, d + 8, 1 << 30, nullptr) == ZS_EINVAL, 33);
    CHECK(grad_sum_norm_sq(nullptr, gb, ZS_BF16, 1 << 16, 1, 1.0, d, d + 8, 16, nullptr) == ZS_EWORKSPACE, 33);
    CHECK(grad_sum_norm_sq(f, gb + 1, ZS_F32, 1 << 16, 0, 1.0, d, d + 8, 1 << 30, nullptr) == ZS_EINVAL, 33);
    CHECK(grad_sum_norm_sq(f, gb, ZS_BF16, 1 << 16, 0, 1.0, reinterpret_cast<double*>(f + 64), d + 8, 1 << 30,
                           nullptr) == ZS_EOVERLAP, 33);
    CHECK(grad_sum_norm_sq(f, gb, ZS_BF16, (int64_t(1) << 39) + 1, 0, 1.0, d, d + 8, 1 << 30, nullptr) == ZS_EINVAL,
          33);
    CHECK(adamw_step_tiled_sum(&bad, st, f, gb, ZS_BF16, nullptr, 16, nullptr, nullptr) == ZS_EINVAL, 34);
    CHECK(adamw_step_tiled_sum(&hp, st, f, gb, 9, nullptr, 16, nullptr, nullptr) == ZS_EINVAL, 34);
    char* fb = reinterpret_cast<char*>(f);
    CHECK(adamw_step_tiled_sum(&hp, st, reinterpret_cast<float*>(fb + 2), gb, ZS_BF16, nullptr, 16, nullptr,
                               nullptr) == ZS_EINVAL, 34);   // fp32 accumulator off 4 bytes
    CHECK(adamw_step_tiled_sum(&hp, st, f, reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(gb) + 1), ZS_BF16,
                               nullptr, 16, nullptr, nullptr) == ZS_EINVAL, 34);   // bf16 at an odd address
    CHECK(adamw_step_tiled_sum(&hp, st, st + 8, gb, ZS_BF16, nullptr, 16, nullptr, nullptr) == ZS_EOVERLAP, 34);
    CHECK(adamw_step_tiled_sum(&hp, st, nullptr, st + 3 * ZS_STATE_TILE - 4, ZS_BF16, nullptr, 16, nullptr,
                               nullptr) == ZS_EOVERLAP, 34);
    CHECK(adamw_step_tiled_sum(&hp, st, f, gb, ZS_BF16, nullptr, int64_t(1) << 40, nullptr, nullptr) == ZS_EINVAL, 34);
    CHECK(adamw_step_tiled_sum(&hp, nullptr, nullptr, nullptr, ZS_BF16, nullptr, 0, nullptr, nullptr) == ZS_OK, 34);
    CHECK(adamw_step_tiled_sum_dev(nullptr, st, f, gb, ZS_BF16, nullptr, 16, nullptr, nullptr) == ZS_EINVAL, 34);

    // chunk tables and tensor lists of every length up to 40, exactly sized;
    // the last entry is the one that fails, so every entry is read
    for (int count = 1; count <= 40; ++count) {
        std::vector<const void*> chunks(count);
        for (int k = 0; k < count; ++k) chunks[k] = fake(uint64_t(1 + k) << 24);
        chunks[count - 1] = fake((uint64_t(count) << 24) + 1);   // misaligned bf16
        CHECK(grad_reduce_chunks(f, chunks.data(), count, ZS_BF16, 64, 1, nullptr) == ZS_EINVAL, 9);
        std::vector<zs_tensor> ts(count);
        for (int k = 0; k < count; ++k) ts[k] = zs_tensor{fake(uint64_t(1 + k) << 24), 16};
        ts[count - 1].numel = -1;
        CHECK(flat_pack(ts.data(), count, ZS_F32, fake(1ull << 40), ZS_F32, 16 * count, nullptr) == ZS_EINVAL, 10);
        CHECK(flat_unpack(fake(1ull << 40), ZS_F32, ts.data(), count, ZS_F32, nullptr) == ZS_EINVAL, 10);
        CHECK(flat_apply_update(f, ts.data(), count, ZS_BF16, nullptr) == ZS_EINVAL, 10);
        ts[count - 1].numel = 16;
        if (count > 1) {   // two tensors overlap: the last one starts inside the first
            ts[count - 1].ptr = fake((1ull << 24) + 8);
            CHECK(flat_unpack(fake(1ull << 40), ZS_F32, ts.data(), count, ZS_F32, nullptr) == ZS_EOVERLAP, 11);
        }
    }
    CHECK(zs_last_hip_error() == 0, 12);   // nothing reached a launch
    for (int32_t c = -6; c <= 1; ++c) CHECK(zs_strerror(c) != nullptr, 13);
    std::printf("abi sanitizer drive: ok\n");
    return 0;
}
