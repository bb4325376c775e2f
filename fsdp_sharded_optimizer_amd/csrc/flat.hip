// FlatParameter flatten (pack) and unflatten (unpack) as one batched copy.
//
// The tensor table (device pointer, flat offset, numel, first workgroup)
// travels in the kernel arguments, up to kFlatMaxTensors tensors per launch,
// so nothing is allocated on the device.  Workgroups are laid out tensor
// after tensor: workgroup w finds its tensor t with a uniform (scalar) scan
// of the first-workgroup table, then copies one tile of that tensor in
// one-wave workgroups: one 128-bit vector per lane for bit copies (512 bf16
// or 256 fp32 elements), two groups of 4 elements per lane for conversions
// (512 elements; a 64-bit access on the bf16 side).  Every
// workgroup works on a single tensor with uniform base addresses; only a
// tensor's last tile is ragged.  A pack entry with a NULL tensor zero-fills
// the padding [total, padded_total).  (One vector per lane measured 81 % of
// the HBM peak on gfx950 for a bf16 copy, against 74-76 % for two.)
//
// The same walk applies a gathered update (the ZeRO page's _apply_update):
// each tensor adds the next numel elements of an fp32 flat buffer in place,
// in 256-thread workgroups of 1024 (fp32 tensors) or 2048 (bf16) elements,
// residency capped at 6 per CU.
//
// HBM-bound: 4 B/element for bf16 copies, 8 for fp32, 6 for the bf16->fp32
// widening and the fp32->bf16 re-cast; the apply reads the update and the
// tensor and writes the tensor: 12 B/element for fp32 tensors, 8 for bf16.
#include "zs_common.h"

namespace zs {
namespace {

// element types, vector width, groups per lane and workgroup size per kind:
// 0 f32->f32, 1 bf16->bf16, 2 bf16->f32 (widen), 3 f32->bf16 (re-cast),
// 4 f32 += f32, 5 bf16 = RNE(widen(bf16) + f32) (apply; S is the update).
// The copies and conversions run one-wave workgroups (over the 70B block's 9
// tensors, against 256-thread workgroups: the fp32 copy 81 -> 83.5 % of the
// HBM peak, the bf16 copy 81 -> 83 %; 256-thread workgroups with the applies'
// residency caps, 20-28 KiB: copies 69-83 %, conversions 51-82 %).  The applies run 256-thread
// workgroups with 24 KiB of LDS reserved (6 per CU): over the 291 Llama-7B
// tensors in batches of 32, the bf16 apply (8 elements per lane, one 128-bit
// access to the parameter) 81.6 -> 82.2 % and the fp32 apply 81.3 -> 83.0 %
// against one-wave workgroups; the cap is sharp (256 threads at 20 / 28 / 32
// KiB: 80 / 79-81 / 69-75 %; 128 or 512 threads: 71-81 %).  The conversions (one 64-bit access on their bf16 side) take
// Q = 2 groups of 4 elements per lane, a wave's width (256 elements) apart,
// both loads issued before either store: the widening pack 74 -> 81 %, the
// re-casting unpack 76 -> 81 % (Q = 4: 73 / 77 %; one group as 8 contiguous
// elements, so two 128-bit fp32 stores 32 bytes apart per lane: 40 %;
// residency capped by reserved LDS: 35-67 %).  The bit copies and applies
// keep one group: two per lane measured 85 -> 70 % for the fp32 copy and
// 81 -> 76 % for the fp32 apply, and the bf16 apply as groups of 4 elements
// (a 64-bit parameter access) 63 % with one group, 78 % with two, 70 % with
// four, against 82 % for the 8-element shape.
template <int KIND> struct Kind;
template <> struct Kind<0> { using S = float; using D = float; static constexpr int VE = 4, Q = 1, BS = 64; };
template <> struct Kind<1> { using S = uint16_t; using D = uint16_t; static constexpr int VE = 8, Q = 1, BS = 64; };
template <> struct Kind<2> { using S = uint16_t; using D = float; static constexpr int VE = 4, Q = 2, BS = 64; };
template <> struct Kind<3> { using S = float; using D = uint16_t; static constexpr int VE = 4, Q = 2, BS = 64; };
template <> struct Kind<4> { using S = float; using D = float; static constexpr int VE = 4, Q = 1, BS = 256; };
template <> struct Kind<5> { using S = float; using D = uint16_t; static constexpr int VE = 8, Q = 1, BS = 256; };
template <int KIND> constexpr int64_t kGroupElems = (int64_t)Kind<KIND>::BS * Kind<KIND>::VE;
template <int KIND> constexpr int64_t kTileElems = kGroupElems<KIND> * Kind<KIND>::Q;
constexpr bool is_apply(int kind) { return kind >= 4; }
// LDS reserved (never touched) per workgroup to cap residency: the applies
// run 256-thread workgroups, 6 per CU.
template <int KIND> constexpr unsigned kLdsReserve = is_apply(KIND) ? 24576u : 0u;

template <int KIND>
__device__ __forceinline__ typename Kind<KIND>::D convert1(typename Kind<KIND>::S x) {
    if constexpr (KIND == 2) return bf16_to_f32(x);
    else if constexpr (KIND == 3) return (uint16_t)f32_to_bf16_rne(x);
    else return x;
}

// One element of the apply: the tensor's value plus the update, one fp32
// addition, rounded once into the tensor's dtype.
template <int KIND>
__device__ __forceinline__ typename Kind<KIND>::D apply1(typename Kind<KIND>::D p, float u) {
    if constexpr (KIND == 5) return (uint16_t)f32_to_bf16_rne(bf16_to_f32(p) + u);
    else return p + u;
}

// One lane's vector of the apply: VE update elements into VE tensor elements.
template <int KIND>
__device__ __forceinline__ void apply_vec(const float* upd, typename Kind<KIND>::D* dst) {
    if constexpr (KIND == 4) {
        const f32x4 u = ld_stream_f32x4_a4(upd);   // read-only: dword alignment suffices
        const f32x4 p = ld_stream(reinterpret_cast<const f32x4*>(dst));
        st_stream(reinterpret_cast<f32x4*>(dst), f32x4{p.x + u.x, p.y + u.y, p.z + u.z, p.w + u.w});
    } else {
        const f32x4 u = ld_stream_f32x4_a4(upd);
        const f32x4 v = ld_stream_f32x4_a4(upd + 4);
        const u32x4 w = ld_stream(reinterpret_cast<const u32x4*>(dst));
        st_stream(reinterpret_cast<u32x4*>(dst),
                  u32x4{pack_bf16x2(bf16_to_f32(w.x & 0xFFFFu) + u.x, bf16_to_f32(w.x >> 16) + u.y),
                        pack_bf16x2(bf16_to_f32(w.y & 0xFFFFu) + u.z, bf16_to_f32(w.y >> 16) + u.w),
                        pack_bf16x2(bf16_to_f32(w.z & 0xFFFFu) + v.x, bf16_to_f32(w.z >> 16) + v.y),
                        pack_bf16x2(bf16_to_f32(w.w & 0xFFFFu) + v.z, bf16_to_f32(w.w >> 16) + v.w)});
    }
}

// One lane's vector: load VE source elements, convert, store VE destination
// elements (zero fill when src is NULL).
template <int KIND>
__device__ __forceinline__ void copy_vec(const void* src, void* dst, bool zero) {
    if constexpr (KIND == 0 || KIND == 1) {   // 16-byte bit copy
        const u32x4 x = zero ? u32x4{0, 0, 0, 0} : ld_stream_u32x4_a4(src);   // the read side: dword alignment
        st_stream(static_cast<u32x4*>(dst), x);
    } else if constexpr (KIND == 2) {          // 4 bf16 -> 4 fp32
        const u32x2 w = zero ? u32x2{0, 0} : ld_stream_u32x2_a4(src);
        st_stream(static_cast<u32x4*>(dst),
                  u32x4{w.x << 16, w.x & 0xFFFF0000u, w.y << 16, w.y & 0xFFFF0000u});
    } else {                                   // 4 fp32 -> 4 bf16, round to nearest even
        const f32x4 f = zero ? f32x4{0.0f, 0.0f, 0.0f, 0.0f} : ld_stream_f32x4_a4(src);
        st_stream(static_cast<u32x2*>(dst), u32x2{pack_bf16x2(f.x, f.y), pack_bf16x2(f.z, f.w)});
    }
}

// A conversion lane's Q vectors, `stride` elements apart: every load first,
// then every store, so Q loads per lane are in flight together.
template <int KIND>
__device__ __forceinline__ void convert_vecs(const typename Kind<KIND>::S* src, typename Kind<KIND>::D* dst,
                                             bool zero, int64_t stride) {
    constexpr int Q = Kind<KIND>::Q;
    if constexpr (KIND == 2) {
        u32x2 w[Q];
#pragma unroll
        for (int g = 0; g < Q; ++g) w[g] = zero ? u32x2{0, 0} : ld_stream_u32x2_a4(src + g * stride);
#pragma unroll
        for (int g = 0; g < Q; ++g)
            st_stream(reinterpret_cast<u32x4*>(dst + g * stride),
                      u32x4{w[g].x << 16, w[g].x & 0xFFFF0000u, w[g].y << 16, w[g].y & 0xFFFF0000u});
    } else {
        static_assert(KIND == 3, "conversions only");
        f32x4 f[Q];
#pragma unroll
        for (int g = 0; g < Q; ++g)
            f[g] = zero ? f32x4{0.0f, 0.0f, 0.0f, 0.0f} : ld_stream_f32x4_a4(src + g * stride);
#pragma unroll
        for (int g = 0; g < Q; ++g)
            st_stream(reinterpret_cast<u32x2*>(dst + g * stride),
                      u32x2{pack_bf16x2(f[g].x, f[g].y), pack_bf16x2(f[g].z, f[g].w)});
    }
}

template <int KIND, bool UNPACK>
__global__ __launch_bounds__(Kind<KIND>::BS) void flat_kernel(const FlatBatch b) {
    using S = typename Kind<KIND>::S;
    using D = typename Kind<KIND>::D;
    constexpr int VE = Kind<KIND>::VE;
    constexpr int Q = Kind<KIND>::Q;
    constexpr int64_t kGroup = kGroupElems<KIND>;
    // the tensor this workgroup copies: the number of later tensors whose
    // first workgroup is <= w (the table is nondecreasing).  A fixed-length,
    // branch-free count (its second half only for batches of more than 16
    // tensors) lets the table loads issue at once instead of one dependent
    // load per tensor; only the tensor's record is a dependent load.
    const uint32_t w = blockIdx.x;
    int t = 0;
    uint32_t first = 0;   // tile_start[t], tracked in the same pass
#pragma unroll
    for (int k = 1; k <= kFlatMaxTensors / 2; ++k) {
        const bool past = k < b.count && w >= b.tile_start[k];
        t += past ? 1 : 0;
        first = past ? b.tile_start[k] : first;
    }
    if (b.count > kFlatMaxTensors / 2) {
#pragma unroll
        for (int k = kFlatMaxTensors / 2 + 1; k <= kFlatMaxTensors; ++k) {
            const bool past = k < b.count && w >= b.tile_start[k];
            t += past ? 1 : 0;
            first = past ? b.tile_start[k] : first;
        }
    }
    const FlatEntry e = b.e[t];
    const int64_t numel = e.numel;
    const int64_t j = (int64_t)(w - first) * kTileElems<KIND> + threadIdx.x * VE;   // the lane's first group
    if (j >= numel) return;
    const S* src;
    D* dst;
    if (UNPACK) {
        src = static_cast<const S*>(b.flat) + e.flat_off;
        dst = static_cast<D*>(e.tensor);
    } else {
        src = static_cast<const S*>(e.tensor);   // NULL: zero fill
        dst = static_cast<D*>(b.flat) + e.flat_off;
    }
    if constexpr (is_apply(KIND)) {
        if (e.vec_ok && j + VE <= numel) {
            apply_vec<KIND>(src + j, dst + j);
            return;
        }
        const int64_t last = j + VE < numel ? j + VE : numel;
        for (int64_t i = j; i < last; ++i) dst[i] = apply1<KIND>(dst[i], src[i]);
        return;
    }
    const bool zero = src == nullptr;
    if constexpr (Q > 1) {
        if (e.vec_ok && j + (Q - 1) * kGroup + VE <= numel) {   // all of the lane's groups whole
            convert_vecs<KIND>(zero ? nullptr : src + j, dst + j, zero, kGroup);
            return;
        }
    }
    // one group at a time: the tensor's last tile (and unaligned tensors)
#pragma unroll
    for (int g = 0; g < Q; ++g) {
        const int64_t jg = j + g * kGroup;
        if (jg >= numel) return;
        if (e.vec_ok && jg + VE <= numel) {
            copy_vec<KIND>(zero ? nullptr : src + jg, dst + jg, zero);
            continue;
        }
        const int64_t last = jg + VE < numel ? jg + VE : numel;
        for (int64_t i = jg; i < last; ++i) dst[i] = zero ? D(0) : convert1<KIND>(src[i]);
    }
}

template <int KIND, bool UNPACK>
hipError_t launch(const FlatBatch& b, hipStream_t stream) {
    const int64_t blocks = b.tile_start[b.count];
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL((flat_kernel<KIND, UNPACK>), dim3((unsigned)blocks), dim3(Kind<KIND>::BS), kLdsReserve<KIND>,
                       stream, b);
    return hipGetLastError();
}

}  // namespace

int64_t flat_tile_elems(int kind) {
    switch (kind) {
        case 0: return kTileElems<0>;
        case 1: return kTileElems<1>;
        case 2: return kTileElems<2>;
        case 3: return kTileElems<3>;
        case 4: return kTileElems<4>;
        default: return kTileElems<5>;
    }
}

int64_t flat_max_batch_tiles(int kind) {
    static_assert(Kind<4>::BS == Kind<5>::BS && Kind<0>::BS == Kind<1>::BS && Kind<0>::BS == Kind<2>::BS &&
                  Kind<0>::BS == Kind<3>::BS, "one workgroup size for the copies, one for the applies");
    const int64_t bs = is_apply(kind) ? Kind<4>::BS : Kind<0>::BS;
    return (int64_t)UINT32_MAX / bs;   // workgroups x workgroup size < 2^32 work-items
}

hipError_t launch_flat(const FlatBatch& b, int kind, int unpack, hipStream_t stream) {
    if (unpack) {
        switch (kind) {
            case 0: return launch<0, true>(b, stream);
            case 1: return launch<1, true>(b, stream);
            case 3: return launch<3, true>(b, stream);
            case 4: return launch<4, true>(b, stream);
            case 5: return launch<5, true>(b, stream);
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
