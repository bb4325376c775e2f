// fp32 gradient accumulation over micro-batches: acc = widen(g) for the
// first micro-batch, acc = fl(acc + widen(g)) after it.
//
// HBM-bound streaming: bf16 gradients move 6 B/element on the first
// micro-batch (read 2, write 4) and 10 B/element after it (read 2 + 4,
// write 4); fp32 gradients move 8 and 12.  Thread k owns elements
// [8k, 8k+8): one 128-bit bf16 load (or two fp32 loads) and two 128-bit fp32
// accesses per stream.
#include "zs_common.h"

namespace zs {
namespace {

template <bool BF16>
__device__ __forceinline__ void load8(const void* grad, int64_t first, float (&g)[8]) {
    if (BF16) {
        const u32x4 w = ld_stream(reinterpret_cast<const u32x4*>(
            static_cast<const uint16_t*>(grad) + first));
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            g[2 * j] = bf16_to_f32(ws[j] & 0xFFFFu);
            g[2 * j + 1] = bf16_to_f32(ws[j] >> 16);
        }
    } else {
        const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(grad) + first);
        const f32x4 a = ld_stream(p), b = ld_stream(p + 1);
        g[0] = a.x; g[1] = a.y; g[2] = a.z; g[3] = a.w;
        g[4] = b.x; g[5] = b.y; g[6] = b.z; g[7] = b.w;
    }
}

template <bool BF16>
__device__ __forceinline__ float load1(const void* grad, int64_t i) {
    if (BF16) return bf16_to_f32(static_cast<const uint16_t*>(grad)[i]);
    return static_cast<const float*>(grad)[i];
}

template <int VEC, bool BF16, bool OVERWRITE>
__global__ __launch_bounds__(kBlock) void accum_kernel(float* __restrict__ acc,
                                                       const void* __restrict__ grad, int64_t n) {
    const int64_t first = ((int64_t)blockIdx.x * kBlock + threadIdx.x) * VEC;
    if (first >= n) return;
    if (VEC == 8 && first + 8 <= n) {
        float g[8];
        f32x4* a4 = reinterpret_cast<f32x4*>(acc + first);
        f32x4 a0, a1;
        if (!OVERWRITE) { a0 = ld_stream(a4); a1 = ld_stream(a4 + 1); }
        load8<BF16>(grad, first, g);
        if (OVERWRITE) {
            a0 = f32x4{g[0], g[1], g[2], g[3]};
            a1 = f32x4{g[4], g[5], g[6], g[7]};
        } else {
            a0 = f32x4{a0.x + g[0], a0.y + g[1], a0.z + g[2], a0.w + g[3]};
            a1 = f32x4{a1.x + g[4], a1.y + g[5], a1.z + g[6], a1.w + g[7]};
        }
        st_stream(a4, a0);
        st_stream(a4 + 1, a1);
        return;
    }
    const int64_t last = first + VEC < n ? first + VEC : n;
    for (int64_t i = first; i < last; ++i) {
        const float g = load1<BF16>(grad, i);
        acc[i] = OVERWRITE ? g : acc[i] + g;
    }
}

template <int VEC, bool BF16, bool OVERWRITE>
hipError_t launch(float* acc, const void* grad, int64_t n, hipStream_t stream) {
    const int64_t threads = (n + VEC - 1) / VEC;
    const int64_t blocks = (threads + kBlock - 1) / kBlock;
    hipLaunchKernelGGL((accum_kernel<VEC, BF16, OVERWRITE>), dim3((unsigned)blocks), dim3(kBlock), 0,
                       stream, acc, grad, n);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_grad_accum(float* acc, const void* grad, int grad_bf16, int64_t n, int overwrite,
                             bool vec_ok, hipStream_t stream) {
    if (vec_ok) {
        if (grad_bf16) return overwrite ? launch<8, true, true>(acc, grad, n, stream)
                                        : launch<8, true, false>(acc, grad, n, stream);
        return overwrite ? launch<8, false, true>(acc, grad, n, stream)
                         : launch<8, false, false>(acc, grad, n, stream);
    }
    if (grad_bf16) return overwrite ? launch<1, true, true>(acc, grad, n, stream)
                                    : launch<1, true, false>(acc, grad, n, stream);
    return overwrite ? launch<1, false, true>(acc, grad, n, stream)
                     : launch<1, false, false>(acc, grad, n, stream);
}

}  // namespace zs
