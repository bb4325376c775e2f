// This shard's share of the squared global gradient norm, in two stages.
//
// Stage 1 (HBM-bound, 4 B/element): a fixed grid of P workgroups, P a
// function of n only, grid-strides over 4-element vectors (one 128-bit
// lane-contiguous load per lane and iteration; P <= 2048 measured best on
// gfx950 against larger grids, deeper unrolls and one-shot tiles).  Each thread
// forms g1 = fl32(g * scale), squares it exactly in binary64 and adds it to
// a binary64 running sum; the 64 lanes of a wave are combined by a fixed
// butterfly of cross-lane shuffles, the 4 waves of a workgroup through LDS,
// and each workgroup writes one binary64 partial to the workspace.
// Stage 2: one workgroup adds the P partials in a fixed tree.
// The association is fixed by n alone, so the result is bit-identical run
// to run, whichever alignment path loaded the data.
#include "zs_common.h"

namespace zs {
namespace {

constexpr int64_t kMaxPartials = 2048;   // 8 workgroups per CU on 256 CUs

__device__ __forceinline__ double wave_sum(double x) {
    // butterfly over the 64 lanes of a wave
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// Sum over the workgroup, result valid in thread 0.
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

template <bool ALIGNED>
__global__ __launch_bounds__(kBlock) void norm_partial_kernel(const float* __restrict__ grad,
                                                              int64_t n, float scale,
                                                              double* __restrict__ partials) {
    const int64_t nvec = (n + 3) / 4;
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    double s0 = 0.0, s1 = 0.0;
    for (int64_t k = (int64_t)blockIdx.x * kBlock + threadIdx.x; k < nvec; k += stride) {
        const int64_t first = k * 4;
        float g[4];
        if (ALIGNED && first + 4 <= n) {
            const f32x4 a = ld_stream(reinterpret_cast<const f32x4*>(grad + first));
            g[0] = a.x; g[1] = a.y; g[2] = a.z; g[3] = a.w;
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) g[j] = first + j < n ? grad[first + j] : 0.0f;
        }
        // the binary64 product of two binary32 values is exact, so the
        // fused form equals fl64(s + g1*g1)
        const double a0 = (double)(g[0] * scale), a1 = (double)(g[1] * scale);
        const double a2 = (double)(g[2] * scale), a3 = (double)(g[3] * scale);
        s0 = __builtin_fma(a0, a0, s0);
        s1 = __builtin_fma(a1, a1, s1);
        s0 = __builtin_fma(a2, a2, s0);
        s1 = __builtin_fma(a3, a3, s1);
    }
    const double total = block_sum(s0 + s1);
    if (threadIdx.x == 0) partials[blockIdx.x] = total;
}

__global__ __launch_bounds__(kBlock) void norm_final_kernel(const double* __restrict__ partials,
                                                            int64_t count, double* __restrict__ out) {
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < count; i += kBlock) s += partials[i];
    const double total = block_sum(s);
    if (threadIdx.x == 0) *out = total;
}

}  // namespace

int64_t norm_partial_blocks(int64_t n) {
    if (n <= 0) return 0;
    const int64_t nvec = (n + 3) / 4;
    const int64_t b = (nvec + kBlock - 1) / kBlock;
    return b < kMaxPartials ? b : kMaxPartials;
}

hipError_t launch_grad_norm_sq(const float* grad, int64_t n, float scale, double* out,
                               double* partials, bool vec_ok, hipStream_t stream) {
    const int64_t blocks = norm_partial_blocks(n);
    if (blocks > 0) {
        if (vec_ok)
            hipLaunchKernelGGL((norm_partial_kernel<true>), dim3((unsigned)blocks), dim3(kBlock), 0,
                               stream, grad, n, scale, partials);
        else
            hipLaunchKernelGGL((norm_partial_kernel<false>), dim3((unsigned)blocks), dim3(kBlock), 0,
                               stream, grad, n, scale, partials);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(norm_final_kernel, dim3(1), dim3(kBlock), 0, stream, partials, blocks, out);
    return hipGetLastError();
}

}  // namespace zs
