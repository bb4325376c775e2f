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
// to run.  The gradient is only read, so any 4-byte-aligned start takes the
// 128-bit path.
#include "reduce.h"

namespace zs {
namespace {

constexpr int64_t kMaxPartials = 2048;   // 8 workgroups per CU on 256 CUs

__global__ __launch_bounds__(kBlock) void norm_partial_kernel(const float* __restrict__ grad,
                                                              int64_t n, float scale,
                                                              double* __restrict__ partials) {
    const int64_t nvec = (n + 3) / 4;
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    double s0 = 0.0, s1 = 0.0;
    for (int64_t k = (int64_t)blockIdx.x * kBlock + threadIdx.x; k < nvec; k += stride) {
        const int64_t first = k * 4;
        float g[4];
        if (first + 4 <= n) {   // read-only: a dword-aligned 128-bit load at any offset
            const f32x4 a = ld_stream_f32x4_a4(grad + first);
            g[0] = a.x; g[1] = a.y; g[2] = a.z; g[3] = a.w;
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) g[j] = first + j < n ? grad[first + j] : 0.0f;
        }
        add_squares4(g, scale, s0, s1);
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

// workgroup c adds partials [c*per, min((c+1)*per, count))
__global__ __launch_bounds__(kBlock) void chunk_sum_kernel(const double* __restrict__ partials,
                                                           int64_t count, int64_t per,
                                                           double* __restrict__ stage) {
    const int64_t lo = (int64_t)blockIdx.x * per;
    const int64_t hi = lo + per < count ? lo + per : count;
    double s = 0.0;
    for (int64_t i = lo + threadIdx.x; i < hi; i += kBlock) s += partials[i];
    const double total = block_sum(s);
    if (threadIdx.x == 0) stage[blockIdx.x] = total;
}

}  // namespace

hipError_t launch_sum_partials(const double* partials, int64_t count, double* stage, double* out,
                               hipStream_t stream) {
    if (count <= kBlock * 8) {   // small: one workgroup
        hipLaunchKernelGGL(norm_final_kernel, dim3(1), dim3(kBlock), 0, stream, partials, count, out);
        return hipGetLastError();
    }
    const int64_t per = (count + kReduceChunks - 1) / kReduceChunks;
    const int64_t chunks = (count + per - 1) / per;
    hipLaunchKernelGGL(chunk_sum_kernel, dim3((unsigned)chunks), dim3(kBlock), 0, stream, partials, count, per,
                       stage);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(norm_final_kernel, dim3(1), dim3(kBlock), 0, stream, stage, chunks, out);
    return hipGetLastError();
}

int64_t norm_partial_blocks(int64_t n) {
    if (n <= 0) return 0;
    const int64_t nvec = (n + 3) / 4;
    const int64_t b = (nvec + kBlock - 1) / kBlock;
    return b < kMaxPartials ? b : kMaxPartials;
}

hipError_t launch_grad_norm_sq(const float* grad, int64_t n, float scale, double* out,
                               double* partials, hipStream_t stream) {
    const int64_t blocks = norm_partial_blocks(n);
    if (blocks > 0) {
        hipLaunchKernelGGL(norm_partial_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, stream, grad, n, scale,
                           partials);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(norm_final_kernel, dim3(1), dim3(kBlock), 0, stream, partials, blocks, out);
    return hipGetLastError();
}

}  // namespace zs
