// fp32 gradient accumulation over micro-batches: acc = widen(g) for the
// first micro-batch, acc = fl(acc + widen(g)) after it.
//
// HBM-bound streaming: bf16 gradients move 6 B/element on the first
// micro-batch (read 2, write 4) and 10 B/element after it (read 2 + 4,
// write 4); fp32 gradients move 8 and 12.
//
// Layout: lane-contiguous groups of 4 elements (a 64-bit bf16 or 128-bit
// fp32 load and a 128-bit fp32 access per lane).  A workgroup covers Q
// groups per lane, the q-th at offset q*1024 in its tile, with every load
// of the tile issued before the first store: Q = 2 for the accumulating
// form and Q = 1 for the overwriting form (the faster shapes on gfx950).
#include "zs_common.h"

namespace zs {
namespace {

template <bool BF16>
__device__ __forceinline__ f32x4 load4(const void* grad, int64_t i) {
    if (BF16) {
        const u32x2 w = ld_stream(reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(grad) + i));
        return f32x4{bf16_to_f32(w.x & 0xFFFFu), bf16_to_f32(w.x >> 16),
                     bf16_to_f32(w.y & 0xFFFFu), bf16_to_f32(w.y >> 16)};
    }
    return ld_stream(reinterpret_cast<const f32x4*>(static_cast<const float*>(grad) + i));
}

template <bool BF16>
__device__ __forceinline__ float load1(const void* grad, int64_t i) {
    if (BF16) return bf16_to_f32(static_cast<const uint16_t*>(grad)[i]);
    return static_cast<const float*>(grad)[i];
}

template <int Q, bool VEC, bool BF16, bool OVERWRITE>
__global__ __launch_bounds__(kBlock) void accum_kernel(float* __restrict__ acc,
                                                       const void* __restrict__ grad, int64_t n) {
    constexpr int64_t kGroup = kBlock * 4;
    const int64_t tile = (int64_t)blockIdx.x * kGroup * Q;
    const int64_t lane0 = tile + threadIdx.x * 4;
    if (VEC && tile + kGroup * Q <= n) {   // whole tile in range
        f32x4 g[Q], a[Q];
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            g[q] = load4<BF16>(grad, lane0 + q * kGroup);
            if (!OVERWRITE) a[q] = ld_stream(reinterpret_cast<const f32x4*>(acc + lane0 + q * kGroup));
        }
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const f32x4 r = OVERWRITE ? g[q]
                                      : f32x4{a[q].x + g[q].x, a[q].y + g[q].y, a[q].z + g[q].z,
                                              a[q].w + g[q].w};
            st_stream(reinterpret_cast<f32x4*>(acc + lane0 + q * kGroup), r);
        }
        return;
    }
    // ragged tile (or a misaligned buffer): element by element
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int64_t first = lane0 + q * kGroup;
        const int64_t last = first + 4 < n ? first + 4 : n;
        for (int64_t i = first; i < last; ++i) {
            const float g = load1<BF16>(grad, i);
            acc[i] = OVERWRITE ? g : acc[i] + g;
        }
    }
}

template <int Q, bool VEC, bool BF16, bool OVERWRITE>
hipError_t launch(float* acc, const void* grad, int64_t n, hipStream_t stream) {
    const int64_t per_block = (int64_t)kBlock * 4 * Q;
    const int64_t blocks = (n + per_block - 1) / per_block;
    hipLaunchKernelGGL((accum_kernel<Q, VEC, BF16, OVERWRITE>), dim3((unsigned)blocks), dim3(kBlock), 0,
                       stream, acc, grad, n);
    return hipGetLastError();
}

template <bool VEC>
hipError_t dispatch(float* acc, const void* grad, int grad_bf16, int64_t n, int overwrite,
                    hipStream_t stream) {
    if (grad_bf16) return overwrite ? launch<1, VEC, true, true>(acc, grad, n, stream)
                                    : launch<2, VEC, true, false>(acc, grad, n, stream);
    return overwrite ? launch<1, VEC, false, true>(acc, grad, n, stream)
                     : launch<2, VEC, false, false>(acc, grad, n, stream);
}

}  // namespace

hipError_t launch_grad_accum(float* acc, const void* grad, int grad_bf16, int64_t n, int overwrite,
                             bool vec_ok, hipStream_t stream) {
    return vec_ok ? dispatch<true>(acc, grad, grad_bf16, n, overwrite, stream)
                  : dispatch<false>(acc, grad, grad_bf16, n, overwrite, stream);
}

}  // namespace zs
