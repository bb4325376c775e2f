// Bandwidth ceiling for the AdamW step's traffic (a measurement aid for the
// benchmark, not part of libzshard's interface).
//
// The kernel moves exactly the AdamW step's bytes with the AdamW kernel's
// launch shape, but replaces the update with one addition per stream:
// reads grad, master, exp_avg, exp_avg_sq (16 B/element) and writes
// master + grad, exp_avg + grad, exp_avg_sq + grad (12 B) and the top half
// of the new master's bits (2 B, when a bf16 buffer is given): 30 B/element.
// Same one-wave workgroups of 4 elements per lane and 128-bit
// non-temporal accesses; the LDS reserved per workgroup (which caps how many
// workgroups a CU holds) is an argument, so the caller can take the best
// residency for this kernel rather than the one tuned for the AdamW
// arithmetic (16 KiB).  Whatever the AdamW kernel loses against this
// kernel's best is lost to its arithmetic; whatever this kernel loses
// against the 8 TB/s peak is lost to the memory system on this mix of four
// read and four written streams.
//
//   int32_t zsc_adamw_traffic(float* master, float* exp_avg, float* exp_avg_sq,
//                             const float* grad, uint16_t* bf16_or_null,
//                             int64_t n, int32_t lds_bytes, void* hip_stream)
// Device buffers of n elements; master, exp_avg, exp_avg_sq and bf16 must be
// 16-byte aligned and grad 4-byte aligned; lds_bytes in [0, 65536].
// Returns 0, -1 for a bad argument (nothing launched), or the hipError_t of
// the launch.
//
//   int32_t zsc_adamw_traffic_tiled(float* state, const float* grad,
//                                   uint16_t* bf16_or_null, int64_t n,
//                                   int32_t lds_bytes, void* hip_stream)
// The same traffic on libzshard's tiled state layout (per tile of 8192
// elements: the masters, then the exp_avgs, then the exp_avg_sqs, 8192 floats
// each), the reference for adamw_step_tiled.  state: 16-byte aligned, at
// least 3 * 8192 * ceil(n / 8192) floats.
//
//   int32_t zsc_adamw_traffic_tiled_sum(float* state, const float* acc_or_null,
//                                       const uint16_t* grad_bf16, uint16_t* bf16_or_null,
//                                       int64_t n, int32_t lds_bytes, void* hip_stream)
// The traffic of adamw_step_tiled_sum: the gradient read as an fp32
// accumulator plus a bf16 micro-batch gradient (32 B/element with the bf16
// output), or the bf16 gradient alone (acc NULL: 28 B/element), summed as the
// step sums them.  acc 4-byte aligned, grad_bf16 4-byte aligned.
#include <hip/hip_runtime.h>
#include <cstdint>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));

constexpr int kBlock = 64;
constexpr int64_t kTile = 8192;   // libzshard's ZS_STATE_TILE

typedef uint32_t u32x2_a4 __attribute__((ext_vector_type(2), aligned(4)));

__device__ inline float widen(uint32_t h) { return __uint_as_float(h << 16); }

// SRC: the gradient is g (0), widen(gb) (1) or g + widen(gb) (2).
template <int SRC>
__device__ inline f32x4 grad4(const float* g, const uint16_t* gb, int64_t first) {
    f32x4 r = {0.0f, 0.0f, 0.0f, 0.0f};
    if (SRC != 1) r = __builtin_nontemporal_load(reinterpret_cast<const f32x4_a4*>(g + first));
    if (SRC != 0) {
        const u32x2 w = __builtin_nontemporal_load(reinterpret_cast<const u32x2_a4*>(gb + first));
        r += f32x4{widen(w.x & 0xFFFFu), widen(w.x >> 16), widen(w.y & 0xFFFFu), widen(w.y >> 16)};
    }
    return r;
}

template <int SRC>
__device__ inline float grad1(const float* g, const uint16_t* gb, int64_t i) {
    return (SRC != 1 ? g[i] : 0.0f) + (SRC != 0 ? widen(gb[i]) : 0.0f);
}

// TILED: p is the tiled state (m and v unused); element i's three values sit
// at tile_base + (i mod kTile) + {0, 1, 2} * kTile.
template <bool BF16, bool TILED, int SRC = 0>
__global__ __launch_bounds__(kBlock) void adamw_traffic_kernel(float* __restrict__ p, float* __restrict__ m,
                                                               float* __restrict__ v, const float* __restrict__ g,
                                                               uint16_t* __restrict__ b, int64_t n,
                                                               const uint16_t* __restrict__ gb = nullptr) {
    const int64_t first = ((int64_t)blockIdx.x * kBlock + threadIdx.x) * 4;
    if (first + 4 <= n) {
        float* pp = p + first;
        float* mp = TILED ? nullptr : m + first;
        float* vp = TILED ? nullptr : v + first;
        if (TILED) {
            pp = p + (first / kTile) * (3 * kTile) + first % kTile;
            mp = pp + kTile;
            vp = pp + 2 * kTile;
        }
        const f32x4 g4 = grad4<SRC>(g, gb, first);
        f32x4 p4 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(pp));
        f32x4 m4 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(mp));
        f32x4 v4 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(vp));
        p4 += g4;
        m4 += g4;
        v4 += g4;
        __builtin_nontemporal_store(p4, reinterpret_cast<f32x4*>(pp));
        __builtin_nontemporal_store(m4, reinterpret_cast<f32x4*>(mp));
        __builtin_nontemporal_store(v4, reinterpret_cast<f32x4*>(vp));
        if (BF16) {
            const uint32_t w0 = (__float_as_uint(p4.x) >> 16) | (__float_as_uint(p4.y) & 0xFFFF0000u);
            const uint32_t w1 = (__float_as_uint(p4.z) >> 16) | (__float_as_uint(p4.w) & 0xFFFF0000u);
            __builtin_nontemporal_store(u32x2{w0, w1}, reinterpret_cast<u32x2*>(b + first));
        }
        return;
    }
    for (int64_t i = first; i < n; ++i) {
        float* pi = p + i;
        float* mi = TILED ? nullptr : m + i;
        float* vi = TILED ? nullptr : v + i;
        if (TILED) {
            pi = p + (i / kTile) * (3 * kTile) + i % kTile;
            mi = pi + kTile;
            vi = pi + 2 * kTile;
        }
        const float gi = grad1<SRC>(g, gb, i);
        *pi += gi;
        *mi += gi;
        *vi += gi;
        if (BF16) b[i] = (uint16_t)(__float_as_uint(*pi) >> 16);
    }
}

bool aligned(const void* q, uintptr_t a) { return ((uintptr_t)q & (a - 1)) == 0; }

}  // namespace

extern "C" __attribute__((visibility("default"))) int32_t zsc_adamw_traffic(
        float* master, float* exp_avg, float* exp_avg_sq, const float* grad, uint16_t* bf16, int64_t n,
        int32_t lds_bytes, void* hip_stream) {
    if (n < 0 || (int64_t)1 << 39 < n || lds_bytes < 0 || lds_bytes > 65536) return -1;
    if (n == 0) return 0;
    if (!master || !exp_avg || !exp_avg_sq || !grad) return -1;
    if (!aligned(master, 16) || !aligned(exp_avg, 16) || !aligned(exp_avg_sq, 16) || !aligned(grad, 4) ||
        (bf16 && !aligned(bf16, 16)))
        return -1;
    const int64_t blocks = (n + 4 * kBlock - 1) / (4 * kBlock);
    if (blocks > (int64_t)UINT32_MAX) return -1;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    if (bf16)
        hipLaunchKernelGGL((adamw_traffic_kernel<true, false>), dim3((unsigned)blocks), dim3(kBlock), (unsigned)lds_bytes,
                           s, master, exp_avg, exp_avg_sq, grad, bf16, n);
    else
        hipLaunchKernelGGL((adamw_traffic_kernel<false, false>), dim3((unsigned)blocks), dim3(kBlock), (unsigned)lds_bytes,
                           s, master, exp_avg, exp_avg_sq, grad, bf16, n);
    return (int32_t)hipGetLastError();
}

extern "C" __attribute__((visibility("default"))) int32_t zsc_adamw_traffic_tiled(
        float* state, const float* grad, uint16_t* bf16, int64_t n, int32_t lds_bytes, void* hip_stream) {
    if (n < 0 || (int64_t)1 << 31 < n || lds_bytes < 0 || lds_bytes > 65536) return -1;
    if (n == 0) return 0;
    if (!state || !grad) return -1;
    if (!aligned(state, 16) || !aligned(grad, 4) || (bf16 && !aligned(bf16, 16))) return -1;
    const int64_t blocks = (n + 4 * kBlock - 1) / (4 * kBlock);
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    if (bf16)
        hipLaunchKernelGGL((adamw_traffic_kernel<true, true>), dim3((unsigned)blocks), dim3(kBlock), (unsigned)lds_bytes,
                           s, state, nullptr, nullptr, grad, bf16, n);
    else
        hipLaunchKernelGGL((adamw_traffic_kernel<false, true>), dim3((unsigned)blocks), dim3(kBlock), (unsigned)lds_bytes,
                           s, state, nullptr, nullptr, grad, bf16, n);
    return (int32_t)hipGetLastError();
}

extern "C" __attribute__((visibility("default"))) int32_t zsc_adamw_traffic_tiled_sum(
        float* state, const float* acc, const uint16_t* grad, uint16_t* bf16, int64_t n, int32_t lds_bytes,
        void* hip_stream) {
    if (n < 0 || (int64_t)1 << 31 < n || lds_bytes < 0 || lds_bytes > 65536) return -1;
    if (n == 0) return 0;
    if (!state || !grad) return -1;
    if (!aligned(state, 16) || !aligned(grad, 4) || (acc && !aligned(acc, 4)) || (bf16 && !aligned(bf16, 16)))
        return -1;
    const int64_t blocks = (n + 4 * kBlock - 1) / (4 * kBlock);
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    const unsigned lds = (unsigned)lds_bytes;
    if (acc && bf16)
        hipLaunchKernelGGL((adamw_traffic_kernel<true, true, 2>), dim3((unsigned)blocks), dim3(kBlock), lds, s, state,
                           nullptr, nullptr, acc, bf16, n, grad);
    else if (acc)
        hipLaunchKernelGGL((adamw_traffic_kernel<false, true, 2>), dim3((unsigned)blocks), dim3(kBlock), lds, s,
                           state, nullptr, nullptr, acc, bf16, n, grad);
    else if (bf16)
        hipLaunchKernelGGL((adamw_traffic_kernel<true, true, 1>), dim3((unsigned)blocks), dim3(kBlock), lds, s, state,
                           nullptr, nullptr, nullptr, bf16, n, grad);
    else
        hipLaunchKernelGGL((adamw_traffic_kernel<false, true, 1>), dim3((unsigned)blocks), dim3(kBlock), lds, s,
                           state, nullptr, nullptr, nullptr, bf16, n, grad);
    return (int32_t)hipGetLastError();
}
