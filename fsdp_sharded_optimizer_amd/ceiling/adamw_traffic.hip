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
#include <hip/hip_runtime.h>
#include <cstdint>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));

constexpr int kBlock = 64;
constexpr int64_t kTile = 8192;   // libzshard's ZS_STATE_TILE

// TILED: p is the tiled state (m and v unused); element i's three values sit
// at tile_base + (i mod kTile) + {0, 1, 2} * kTile.
template <bool BF16, bool TILED>
__global__ __launch_bounds__(kBlock) void adamw_traffic_kernel(float* __restrict__ p, float* __restrict__ m,
                                                               float* __restrict__ v, const float* __restrict__ g,
                                                               uint16_t* __restrict__ b, int64_t n) {
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
        const f32x4 g4 = __builtin_nontemporal_load(reinterpret_cast<const f32x4_a4*>(g + first));
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
        *pi += g[i];
        *mi += g[i];
        *vi += g[i];
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
