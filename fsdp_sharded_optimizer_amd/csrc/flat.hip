// FlatParameter flatten (pack) and unflatten (unpack) as one batched copy.
//
// The tensor table (device pointer, flat offset, numel, first workgroup)
// travels in the kernel arguments, up to kFlatMaxTensors tensors per launch,
// so nothing is allocated on the device.  Workgroups are laid out tensor
// after tensor: workgroup w finds its tensor t with a uniform (scalar) scan
// of the first-workgroup table, then copies the 4096-element tile
// [tile*4096, tile*4096 + 4096) of that tensor.  Every workgroup therefore
// works on a single tensor with uniform base addresses; only a tensor's
// last tile is ragged.  A pack entry with a NULL tensor zero-fills the
// padding [total, padded_total).
//
// HBM-bound: 4 B/element for bf16 copies, 8 for fp32, 6 for the bf16->fp32
// widening and the fp32->bf16 re-cast.
#include "zs_common.h"

namespace zs {
namespace {

constexpr int kTile = 4096;           // elements per workgroup: 2 vectors of 8 per thread
constexpr int kSub = kBlock * 8;      // elements per sweep of the workgroup

// element types per kind: 0 f32->f32, 1 bf16->bf16, 2 bf16->f32, 3 f32->bf16
template <int KIND> struct Kind;
template <> struct Kind<0> { using S = float; using D = float; };
template <> struct Kind<1> { using S = uint16_t; using D = uint16_t; };
template <> struct Kind<2> { using S = uint16_t; using D = float; };
template <> struct Kind<3> { using S = float; using D = uint16_t; };

template <int KIND>
__device__ __forceinline__ typename Kind<KIND>::D convert1(typename Kind<KIND>::S x) {
    if constexpr (KIND == 2) return bf16_to_f32(x);
    else if constexpr (KIND == 3) return (uint16_t)f32_to_bf16_rne(x);
    else return x;
}

// 8 elements in registers as 32-bit words: fp32 -> 8 words, bf16 -> 4 words.
template <typename T> struct Vec8;
template <> struct Vec8<float> { u32x4 lo, hi; };
template <> struct Vec8<uint16_t> { u32x4 w; };

__device__ __forceinline__ Vec8<float> load8(const float* p) {
    const u32x4* q = reinterpret_cast<const u32x4*>(p);
    return {ld_stream(q), ld_stream(q + 1)};
}
__device__ __forceinline__ Vec8<uint16_t> load8(const uint16_t* p) {
    return {ld_stream(reinterpret_cast<const u32x4*>(p))};
}
__device__ __forceinline__ void store8(float* p, const Vec8<float>& v) {
    u32x4* q = reinterpret_cast<u32x4*>(p);
    st_stream(q, v.lo);
    st_stream(q + 1, v.hi);
}
__device__ __forceinline__ void store8(uint16_t* p, const Vec8<uint16_t>& v) {
    st_stream(reinterpret_cast<u32x4*>(p), v.w);
}

template <int KIND>
__device__ __forceinline__ Vec8<typename Kind<KIND>::D> convert8(const Vec8<typename Kind<KIND>::S>& x) {
    if constexpr (KIND == 2) {   // bf16 -> fp32: each 32-bit word holds two elements
        const uint32_t w[4] = {x.w.x, x.w.y, x.w.z, x.w.w};
        return {u32x4{w[0] << 16, w[0] & 0xFFFF0000u, w[1] << 16, w[1] & 0xFFFF0000u},
                u32x4{w[2] << 16, w[2] & 0xFFFF0000u, w[3] << 16, w[3] & 0xFFFF0000u}};
    } else if constexpr (KIND == 3) {   // fp32 -> bf16, round to nearest even
        const float f[8] = {__uint_as_float(x.lo.x), __uint_as_float(x.lo.y),
                            __uint_as_float(x.lo.z), __uint_as_float(x.lo.w),
                            __uint_as_float(x.hi.x), __uint_as_float(x.hi.y),
                            __uint_as_float(x.hi.z), __uint_as_float(x.hi.w)};
        return {u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                      pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7])}};
    } else {
        return x;
    }
}

template <typename T>
__device__ __forceinline__ Vec8<T> zero8() {
    if constexpr (sizeof(T) == 4) return {u32x4{0, 0, 0, 0}, u32x4{0, 0, 0, 0}};
    else return {u32x4{0, 0, 0, 0}};
}

template <int KIND, bool UNPACK>
__global__ __launch_bounds__(kBlock) void flat_kernel(const FlatBatch b) {
    using S = typename Kind<KIND>::S;
    using D = typename Kind<KIND>::D;
    // uniform scan: the tensor this workgroup copies
    const int64_t w = blockIdx.x;
    int t = 0;
    while (t + 1 < b.count && w >= b.tile_start[t + 1]) ++t;
    const int64_t numel = b.numel[t];
    const int64_t base = (w - b.tile_start[t]) * kTile;
    const bool vec = b.vec_ok[t] != 0;
    const S* src;
    D* dst;
    if (UNPACK) {
        src = static_cast<const S*>(b.flat) + b.flat_off[t];
        dst = static_cast<D*>(b.tensor[t]);
    } else {
        src = static_cast<const S*>(b.tensor[t]);   // NULL: zero fill
        dst = static_cast<D*>(b.flat) + b.flat_off[t];
    }
    const bool zero = src == nullptr;

    int64_t j0 = base + threadIdx.x * 8;
    int64_t j1 = j0 + kSub;
    if (vec && j1 + 8 <= numel) {   // both vectors full: loads first, then stores
        Vec8<D> a, c;
        if (zero) {
            a = zero8<D>();
            c = a;
        } else {
            const Vec8<S> x0 = load8(src + j0), x1 = load8(src + j1);
            a = convert8<KIND>(x0);
            c = convert8<KIND>(x1);
        }
        store8(dst + j0, a);
        store8(dst + j1, c);
        return;
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int64_t j = u == 0 ? j0 : j1;
        if (j >= numel) break;
        if (vec && j + 8 <= numel) {
            store8(dst + j, zero ? zero8<D>() : convert8<KIND>(load8(src + j)));
        } else {
            const int64_t last = j + 8 < numel ? j + 8 : numel;
            for (int64_t i = j; i < last; ++i) dst[i] = zero ? D(0) : convert1<KIND>(src[i]);
        }
    }
}

template <int KIND, bool UNPACK>
hipError_t launch(const FlatBatch& b, hipStream_t stream) {
    const int64_t blocks = b.tile_start[b.count];
    if (blocks <= 0) return hipSuccess;
    if (blocks > (int64_t)UINT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL((flat_kernel<KIND, UNPACK>), dim3((unsigned)blocks), dim3(kBlock), 0, stream, b);
    return hipGetLastError();
}

}  // namespace

int64_t flat_tile_elems() { return kTile; }

hipError_t launch_flat(const FlatBatch& b, int kind, int unpack, hipStream_t stream) {
    if (unpack) {
        switch (kind) {
            case 0: return launch<0, true>(b, stream);
            case 1: return launch<1, true>(b, stream);
            case 3: return launch<3, true>(b, stream);
            default: return hipErrorInvalidValue;
        }
    }
    switch (kind) {
        case 0: return launch<0, false>(b, stream);
        case 1: return launch<1, false>(b, stream);
        case 2: return launch<2, false>(b, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace zs
