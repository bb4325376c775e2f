// Deterministic binary64 reductions shared by the norm kernels (internal).
#pragma once

#include "zs_common.h"

namespace zs {

// Butterfly over the 64 lanes of a wave (fixed order).
__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// Sum over a kBlock-thread workgroup, result valid in thread 0 (fixed order:
// the wave butterflies, then wave 0 + wave 1 + wave 2 + wave 3).
__device__ __forceinline__ double block_sum(double x) {
    __shared__ double wave_part[kBlock / 64];
    x = wave_sum(x);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) wave_part[wave] = x;
    __syncthreads();
    double s = 0.0;
    if (threadIdx.x == 0) {
        s = wave_part[0];
#pragma unroll
        for (int w = 1; w < kBlock / 64; ++w) s += wave_part[w];
    }
    return s;
}

// Accumulates the binary64 squares of g1 = fl32(g * scale) for 4 elements
// into two running sums (elements 0, 2 into s0; 1, 3 into s1).  The binary64
// product of two binary32 values is exact, so the fused form equals
// fl64(s + g1*g1).
__device__ __forceinline__ void add_squares4(const float (&g)[4], float scale, double& s0, double& s1) {
    const double a0 = (double)(g[0] * scale), a1 = (double)(g[1] * scale);
    const double a2 = (double)(g[2] * scale), a3 = (double)(g[3] * scale);
    s0 = __builtin_fma(a0, a0, s0);
    s1 = __builtin_fma(a1, a1, s1);
    s0 = __builtin_fma(a2, a2, s0);
    s1 = __builtin_fma(a3, a3, s1);
}

// Reduce `count` binary64 partials to *out in a fixed tree: up to
// kReduceChunks workgroups each add a contiguous chunk into `stage`
// (kReduceChunks doubles), then one workgroup adds those.  count == 0
// writes 0.  (The fused accumulation leaves one partial per 256 elements:
// 3.3M for an 842M shard, about 1,600 per chunk.)
constexpr int64_t kReduceChunks = 2048;
constexpr int64_t kSumOneGroup = kBlock * 8;   // up to this many partials: one workgroup, no stage
hipError_t launch_sum_partials(const double* partials, int64_t count, double* stage, double* out,
                               hipStream_t stream);

}  // namespace zs
