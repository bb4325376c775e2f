// Fused AdamW step over one rank's shard, one HBM pass.
//
// Per element the kernel reads grad, master, exp_avg, exp_avg_sq (16 B) and
// writes master, exp_avg, exp_avg_sq (12 B) and, optionally, the bf16
// re-cast of the master (2 B): 30 B of algorithmic traffic, streamed once.
// The arithmetic (the update of the ai6s.net cann-recipes-train ZeRO page,
// §ZeRO-1/2/3 step, with decoupled decay) is ~20 fp32 operations including
// two IEEE divisions and one IEEE square root per element, far below the
// gfx950 vector rate at 8 TB/s, so the kernel is HBM-bound: the design goal
// is deep memory-level parallelism and fully coalesced 128-bit accesses.
//
// The master forms (tiled or split state) also take the gradient as the last
// micro-batch's sum, formed as it is read (GS): fl(acc + widen(g)) from the
// fp32 accumulator and the micro-batch's bf16 or fp32 gradient, or widen(g)
// alone for a step of one micro-batch.  It is the value the accumulation
// would have stored, so the step is bit for bit the one that follows an
// accumulation, and the accumulator is never written: the last micro-batch
// and the step move 32 B/element (bf16 micro-batch; 28 alone) instead of the
// accumulation's 10 (6) plus the step's 30.
//
// Two more forms share the code: the bf16 parameter updated in place with no
// master (the ZeRO page's ZeRO-3 step; 24 B/element), and the ZeRO-1 form
// that writes the update vector -u instead of a parameter (Adam without
// decay; R grad, m, v and W m, v, update: 24 B/element).
//
// Every form also runs on a tiled state (TILED): master, exp_avg and
// exp_avg_sq in one buffer, three runs of kStateTile floats per tile of
// elements (the moments alone, two runs, for the no-master and update forms).  Same bytes and arithmetic; a wave's three state
// accesses then fall in one 96 KiB region instead of three separate
// buffers, which keeps fewer DRAM rows open: on gfx950 the AdamW step runs
// at 85 % of the peak against 80-83 % on split buffers (7B, 70B and 13B
// shard sizes, clipped or not), with residency capped at 11 workgroups per
// CU (14 KiB reserved each; 10, 12 and 13 per CU measure 0.7-1.6 points
// lower).
//
// Layout: every array is a flat 1-D fp32 (bf16) buffer; thread k of the grid
// owns the 4 consecutive elements [4k, 4k+4): one 128-bit access per fp32
// stream and one 64-bit access for the bf16 stream, so each wave64 access
// covers 1 KiB of a stream with no gaps.  One-shot grid of one-wave
// workgroups (256 elements each), with residency capped at 10 workgroups
// per CU: each workgroup reserves 16 KiB of LDS it never touches, out of
// gfx950's 160 KiB per CU (12 KiB, 13 per CU, for the six-stream forms).  Eight concurrent streams per element (4 read,
// 4 written) otherwise keep too many DRAM rows open at once; on gfx950 the
// cap lifts the kernel from 74 % to 83 % of the 8 TB/s peak (fewer waves:
// 64-71 %; more: 73-81 %).  A shard whose master or moments are views at an
// element offset that is not a multiple of 4 takes the VEC = 1 instantiation
// of the same code, in 256-thread workgroups without the cap; the read-only
// gradient may sit at any 4-byte boundary and the write-only output (bf16
// re-cast, ZeRO-1 update) at any element offset on the vector path.
#include "zs_common.h"

namespace zs {
namespace {

// One element: the moments in place and the returned step u, in the order
// and with the roundings the header documents.  Built with
// -ffp-contract=off: no multiply-add fusion; the quotient and square root
// are IEEE round-to-nearest (correctly rounded fp32 division and sqrt are
// requested at compile time).
__device__ __forceinline__ float adam_elem(const AdamwScalars& a, float coef, float gr, float& m, float& v) {
    float g = gr * a.grad_scale;
    g = g * coef;
    const float m_keep = a.beta1 * m;
    const float m_new = a.one_minus_beta1 * g;
    m = m_keep + m_new;
    const float g2 = g * g;
    const float v_keep = a.beta2 * v;
    const float v_new = a.one_minus_beta2 * g2;
    v = v_keep + v_new;
    const float root = sqrtf(v);
    float den = root / a.bias_correction2_sqrt;
    den = den + a.eps;
    const float ratio = m / den;
    return ratio * a.step_size;
}

// the parameter after the step: decoupled decay, then the step
__device__ __forceinline__ float apply_step(const AdamwScalars& a, float p, float u) {
    const float pd = p * a.decay;
    return pd - u;
}

// Four consecutive gradient elements from `first` (vector path; every source
// is read-only, so dword alignment suffices) and one element (scalar path),
// for the gradient source GS; the sums round as the accumulation does.
template <int GS>
__device__ __forceinline__ f32x4 grad4(const AdamwArgs& a, int64_t first) {
    if constexpr (GS == kGradF32) {
        return ld_stream_f32x4_a4(a.grad + first);
    } else if constexpr (GS == kGradSumF32) {
        const f32x4 s = ld_stream_f32x4_a4(a.grad + first);
        const f32x4 g = ld_stream_f32x4_a4(static_cast<const float*>(a.grad_mb) + first);
        return f32x4{s.x + g.x, s.y + g.y, s.z + g.z, s.w + g.w};
    } else {
        const u32x2 w = ld_stream_u32x2_a4(static_cast<const uint16_t*>(a.grad_mb) + first);
        const f32x4 g = {bf16_to_f32(w.x & 0xFFFFu), bf16_to_f32(w.x >> 16), bf16_to_f32(w.y & 0xFFFFu),
                         bf16_to_f32(w.y >> 16)};
        if constexpr (GS == kGradBf16) return g;
        const f32x4 s = ld_stream_f32x4_a4(a.grad + first);
        return f32x4{s.x + g.x, s.y + g.y, s.z + g.z, s.w + g.w};
    }
}

template <int GS>
__device__ __forceinline__ float grad1(const AdamwArgs& a, int64_t i) {
    if constexpr (GS == kGradF32) return a.grad[i];
    else if constexpr (GS == kGradSumF32) return a.grad[i] + static_cast<const float*>(a.grad_mb)[i];
    else {
        const float g = bf16_to_f32(static_cast<const uint16_t*>(a.grad_mb)[i]);
        if constexpr (GS == kGradBf16) return g;
        else return a.grad[i] + g;
    }
}

// Clip coefficient from the squared norm, in binary64 (uniform per wave).
// Returns false when the global squared norm is not finite: the step is
// skipped, no state is written (the update form writes -0.0, see below).
__device__ __forceinline__ bool clip_coef(const AdamwScalars& a, const double* norm_sq, float& coef) {
    coef = 1.0f;
    if (norm_sq == nullptr) return true;
    const double s = *norm_sq + a.extra_norm_sq;
    if (!__builtin_isfinite(s)) return false;
    if (a.clip) {
        const double total = sqrt(s);
        double c = a.max_norm / (total + 1e-6);
        if (c > 1.0) c = 1.0;
        coef = (float)c;
    }
    return true;
}

// A skipped ZeRO-1 step (non-finite global norm) still writes its update
// vector: -0.0, the identity of IEEE addition, so the apply that follows the
// all-gather leaves every parameter bit for bit as it was (the moments are
// not written).  Four consecutive elements from `at`.
template <bool OUT_ALIGNED>
__device__ __forceinline__ void skip_update(float* at) {
    if constexpr (OUT_ALIGNED) {
        st_stream(reinterpret_cast<f32x4*>(at), f32x4{-0.0f, -0.0f, -0.0f, -0.0f});
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) st_stream(at + j, -0.0f);
    }
}

// vector path: one wave per workgroup, with LDS reserved per workgroup to
// cap residency: 16 KiB (10 workgroups per CU) for the eight-stream master
// forms; 12 KiB (13 per CU) for the six-stream no-master and update forms,
// which measured 84-85 % there against 80-82 % at 16 KiB.
constexpr int kVecBlock = 64;
constexpr unsigned kVecLdsReserve = 16384;
constexpr unsigned kVecLdsReserve6 = 12288;
constexpr unsigned kVecLdsReserveTiled = 14336;
// The tiled forms on an accumulator + micro-batch gradient (nine streams):
// 10 per CU.  On buffers carved from one physically contiguous block they
// measured 86.1-86.3 % there against 85.1 % at 11 per CU (86.3-86.4 % at 8);
// on separately allocated buffers 84.1-84.2 % against 84.3-84.6 % (81.7 % at
// 8 per CU).
constexpr unsigned kVecLdsReserveTiledSum = 16384;

// What a step reads and writes besides grad, exp_avg and exp_avg_sq:
//   kMaster      R/W fp32 master                          28 B/element
//   kMasterBf16  R/W fp32 master, W bf16 re-cast          30 B/element
//   kNoMaster    R/W bf16 parameter (no fp32 master)      24 B/element
//   kUpdate      W fp32 update = -u (no parameter, no decay) 24 B/element
enum Form : int { kMaster = 0, kMasterBf16 = 1, kNoMaster = 2, kUpdate = 3 };

// DEV: the scalars come from device memory (one uniform load per wave) instead
// of the kernel arguments, so a captured graph replays any step whose scalars
// the caller copied in beforehand.
// TILED: the state comes from a tiled buffer: master, exp_avg, exp_avg_sq
// (3 runs per tile) for the master forms, exp_avg, exp_avg_sq (2 runs) for
// the no-master and update forms; 4 consecutive elements never straddle a
// tile.
// OUT_ALIGNED = false: the one output stream that is only written, the bf16
// re-cast or the ZeRO-1 update, starts off a 16-byte boundary (a view at
// any element offset of a larger buffer); the vector path then writes it
// element by element (16- or 32-bit stores) and keeps 128-bit accesses for
// everything else: 81 % of the peak against 65 % for the element-wise path.
// GS: where the gradient comes from (GradSource; the master forms only).
template <int VEC, int FORM, int BS, bool DEV, bool TILED = false, bool OUT_ALIGNED = true, int GS = kGradF32>
__global__ __launch_bounds__(BS) void adamw_kernel(const AdamwArgs a) {
    static_assert(OUT_ALIGNED || FORM == kMasterBf16 || FORM == kUpdate, "a write-only output to split");
    static_assert(GS == kGradF32 || FORM == kMaster || FORM == kMasterBf16, "summed gradients: master forms");
    constexpr bool kMasterForm = FORM == kMaster || FORM == kMasterBf16;
    constexpr int kRuns = kMasterForm ? 3 : 2;   // runs per tile of the tiled state
    constexpr bool kReadP = FORM != kUpdate;
    const AdamwScalars sc = DEV ? *a.sc_dev : a.sc;
    const int64_t n = a.n;
    const int64_t first = ((int64_t)blockIdx.x * BS + threadIdx.x) * VEC;
    // No early exit for lanes past the end: they fall through the scalar
    // path's empty loop.  Every path then uses the buffer pointers, so the
    // kernel-argument loads issue together with n's instead of one round
    // trip after it (a second scalar round trip before the first vector load
    // costs every workgroup of this residency-capped launch).
    if (VEC == 4 && first + 4 <= n) {
        // One 128-bit access per fp32 stream, lane-contiguous across the wave.
        // The loads are issued before the clip coefficient is resolved, so
        // the latency of the norm's read overlaps with them.
        const f32x4 g4 = grad4<GS>(a, first);
        // this lane's master (master forms only), exp_avg and exp_avg_sq
        float* p_at = nullptr;
        float* m_at;
        float* v_at;
        if constexpr (TILED) {
            float* const t = a.state + tiled_offset<kRuns>(first);
            if constexpr (kMasterForm) p_at = t;
            m_at = kMasterForm ? t + kStateTile : t;
            v_at = m_at + kStateTile;
        } else {
            if constexpr (FORM == kMaster || FORM == kMasterBf16) p_at = a.master + first;
            m_at = a.exp_avg + first;
            v_at = a.exp_avg_sq + first;
        }
        f32x4 p4 = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (FORM == kNoMaster) {
            const u32x2 w = ld_stream(reinterpret_cast<const u32x2*>(a.param_bf16 + first));
            p4 = f32x4{bf16_to_f32(w.x & 0xFFFFu), bf16_to_f32(w.x >> 16), bf16_to_f32(w.y & 0xFFFFu),
                       bf16_to_f32(w.y >> 16)};
        } else if constexpr (kReadP) {
            p4 = ld_stream(reinterpret_cast<const f32x4*>(p_at));
        }
        const f32x4 m4 = ld_stream(reinterpret_cast<const f32x4*>(m_at));
        const f32x4 v4 = ld_stream(reinterpret_cast<const f32x4*>(v_at));
        float coef;
        if (!clip_coef(sc, a.norm_sq, coef)) {
            if constexpr (FORM == kUpdate) skip_update<OUT_ALIGNED>(a.update + first);
            return;
        }
        float gs[4] = {g4.x, g4.y, g4.z, g4.w};
        float ps[4] = {p4.x, p4.y, p4.z, p4.w};
        float ms[4] = {m4.x, m4.y, m4.z, m4.w};
        float vs[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float u = adam_elem(sc, coef, gs[j], ms[j], vs[j]);
            ps[j] = FORM == kUpdate ? -u : apply_step(sc, ps[j], u);
        }
        if constexpr (FORM == kMaster || FORM == kMasterBf16)
            st_stream(reinterpret_cast<f32x4*>(p_at), f32x4{ps[0], ps[1], ps[2], ps[3]});
        if constexpr (FORM == kUpdate) {
            if constexpr (OUT_ALIGNED) {
                st_stream(reinterpret_cast<f32x4*>(a.update + first), f32x4{ps[0], ps[1], ps[2], ps[3]});
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) st_stream(a.update + first + j, ps[j]);
            }
        }
        st_stream(reinterpret_cast<f32x4*>(m_at), f32x4{ms[0], ms[1], ms[2], ms[3]});
        st_stream(reinterpret_cast<f32x4*>(v_at), f32x4{vs[0], vs[1], vs[2], vs[3]});
        if constexpr (FORM == kMasterBf16 || FORM == kNoMaster) {
            if constexpr (OUT_ALIGNED) {
                st_stream(reinterpret_cast<u32x2*>(a.param_bf16 + first),
                          u32x2{pack_bf16x2(ps[0], ps[1]), pack_bf16x2(ps[2], ps[3])});
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) st_stream(a.param_bf16 + first + j, (uint16_t)f32_to_bf16_rne(ps[j]));
            }
        }
        return;
    }
    // scalar path: VEC == 1, or the ragged tail of the VEC == 4 grid
    const int64_t last = first + VEC < n ? first + VEC : n;
    float coef;
    if (!clip_coef(sc, a.norm_sq, coef)) {
        if constexpr (FORM == kUpdate)
            for (int64_t i = first; i < last; ++i) a.update[i] = -0.0f;
        return;
    }
    for (int64_t i = first; i < last; ++i) {
        float* const ts = TILED ? a.state + tiled_offset<kRuns>(i) : nullptr;   // the element's first run
        float* const m_at = TILED ? (kMasterForm ? ts + kStateTile : ts) : a.exp_avg + i;
        float* const v_at = TILED ? m_at + kStateTile : a.exp_avg_sq + i;
        float m = *m_at, v = *v_at;
        const float u = adam_elem(sc, coef, grad1<GS>(a, i), m, v);
        *m_at = m;
        *v_at = v;
        if constexpr (FORM == kUpdate) {
            a.update[i] = -u;
        } else if constexpr (FORM == kNoMaster) {
            a.param_bf16[i] = (uint16_t)f32_to_bf16_rne(apply_step(sc, bf16_to_f32(a.param_bf16[i]), u));
        } else {
            float* const p_at = TILED ? ts : a.master + i;
            const float p = apply_step(sc, *p_at, u);
            *p_at = p;
            if constexpr (FORM == kMasterBf16) a.param_bf16[i] = (uint16_t)f32_to_bf16_rne(p);
        }
    }
}

template <typename T>
T* advance(T* p, int64_t off) { return p == nullptr ? nullptr : p + off; }

// one launch per kLaunchElems elements, each on its own slice of the buffers
// (a multiple of kStateTile: a piece of the tiled state starts at runs*off)
template <int VEC, int FORM, int BS, bool DEV, bool TILED = false, bool OUT_ALIGNED = true, int GS = kGradF32>
hipError_t launch(const AdamwArgs& a, unsigned lds, hipStream_t stream) {
    static_assert(kLaunchElems % kStateTile == 0, "launch pieces start on a tile");
    constexpr int64_t runs = (FORM == kMaster || FORM == kMasterBf16) ? 3 : 2;
    constexpr int64_t mb_size = GS == kGradSumF32 ? 4 : 2;   // bytes per micro-batch gradient element
    for (int64_t off = 0; off < a.n; off += kLaunchElems) {
        AdamwArgs p = a;
        p.n = launch_piece(a.n, off);
        p.state = advance(a.state, runs * off);
        p.master = advance(a.master, off);
        p.exp_avg = advance(a.exp_avg, off);
        p.exp_avg_sq = advance(a.exp_avg_sq, off);
        p.grad = advance(a.grad, off);
        p.grad_mb = a.grad_mb == nullptr ? nullptr : static_cast<const char*>(a.grad_mb) + off * mb_size;
        p.param_bf16 = advance(a.param_bf16, off);
        p.update = advance(a.update, off);
        const int64_t blocks = ((p.n + VEC - 1) / VEC + BS - 1) / BS;
        hipLaunchKernelGGL((adamw_kernel<VEC, FORM, BS, DEV, TILED, OUT_ALIGNED, GS>), dim3((unsigned)blocks),
                           dim3(BS), lds, stream, p);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// vec_ok: the vector path's alignment holds for every stream but the
// write-only output; out_aligned: that output (bf16 re-cast or update) is
// 16-byte aligned too.  A tiled state is 16-byte aligned by contract, so the
// tiled forms take the vector path, except the no-master form with its bf16
// parameter (read and written) off a 16-byte boundary.  The six-stream forms
// keep the 13-per-CU cap tiled too (tiled moments for the update form: 84.5 %
// there, 83.9 % at 11 per CU).
// The summed-gradient forms take the element-wise path on a tiled state too,
// for a bf16 micro-batch gradient off a 4-byte boundary (split buffers: also
// for state off a 16-byte boundary, as the stored-gradient form).
template <int FORM, bool DEV = false, bool TILED = false, int GS = kGradF32>
hipError_t launch_form(const AdamwArgs& a, bool vec_ok, bool out_aligned, hipStream_t stream) {
    constexpr bool six = FORM == kNoMaster || FORM == kUpdate;
    constexpr bool summed = GS == kGradSumBf16 || GS == kGradSumF32;
    constexpr unsigned lds = six     ? kVecLdsReserve6
                             : TILED ? (summed ? kVecLdsReserveTiledSum : kVecLdsReserveTiled)
                                     : kVecLdsReserve;
    if constexpr (FORM == kMasterBf16 || FORM == kUpdate) {
        if (vec_ok && !out_aligned) return launch<4, FORM, kVecBlock, DEV, TILED, false, GS>(a, lds, stream);
    }
    if (vec_ok) return launch<4, FORM, kVecBlock, DEV, TILED, true, GS>(a, lds, stream);
    if constexpr (TILED && FORM != kNoMaster && GS == kGradF32) return hipErrorInvalidValue;   // always vec_ok
    else return launch<1, FORM, kBlock, DEV, TILED, true, GS>(a, 0, stream);
}

template <int GS, bool TILED>
hipError_t launch_sum(const AdamwArgs& a, bool vec_ok, bool out_aligned, hipStream_t stream) {
    if (a.sc_dev != nullptr)
        return a.param_bf16 != nullptr
                   ? launch_form<kMasterBf16, true, TILED, GS>(a, vec_ok, out_aligned, stream)
                   : launch_form<kMaster, true, TILED, GS>(a, vec_ok, true, stream);
    return a.param_bf16 != nullptr ? launch_form<kMasterBf16, false, TILED, GS>(a, vec_ok, out_aligned, stream)
                                   : launch_form<kMaster, false, TILED, GS>(a, vec_ok, true, stream);
}

template <bool TILED>
hipError_t launch_sum_source(const AdamwArgs& a, int grad_source, bool vec_ok, bool out_aligned,
                             hipStream_t stream) {
    switch (grad_source) {
    case kGradBf16: return launch_sum<kGradBf16, TILED>(a, vec_ok, out_aligned, stream);
    case kGradSumBf16: return launch_sum<kGradSumBf16, TILED>(a, vec_ok, out_aligned, stream);
    case kGradSumF32: return launch_sum<kGradSumF32, TILED>(a, vec_ok, out_aligned, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_adamw(const AdamwArgs& a, bool vec_ok, bool out_aligned, hipStream_t stream) {
    if (a.sc_dev != nullptr)
        return a.param_bf16 != nullptr ? launch_form<kMasterBf16, true>(a, vec_ok, out_aligned, stream)
                                       : launch_form<kMaster, true>(a, vec_ok, true, stream);
    return a.param_bf16 != nullptr ? launch_form<kMasterBf16>(a, vec_ok, out_aligned, stream)
                                   : launch_form<kMaster>(a, vec_ok, true, stream);
}

hipError_t launch_adamw_tiled(const AdamwArgs& a, bool out_aligned, hipStream_t stream) {
    if (a.sc_dev != nullptr)
        return a.param_bf16 != nullptr ? launch_form<kMasterBf16, true, true>(a, true, out_aligned, stream)
                                       : launch_form<kMaster, true, true>(a, true, true, stream);
    return a.param_bf16 != nullptr ? launch_form<kMasterBf16, false, true>(a, true, out_aligned, stream)
                                   : launch_form<kMaster, false, true>(a, true, true, stream);
}

hipError_t launch_adamw_no_master(const AdamwArgs& a, bool vec_ok, hipStream_t stream) {
    return launch_form<kNoMaster>(a, vec_ok, true, stream);
}

hipError_t launch_adam_update(const AdamwArgs& a, bool vec_ok, bool out_aligned, hipStream_t stream) {
    return launch_form<kUpdate>(a, vec_ok, out_aligned, stream);
}

hipError_t launch_adamw_tiled_sum(const AdamwArgs& a, int grad_source, bool vec_ok, bool out_aligned,
                                  hipStream_t stream) {
    return launch_sum_source<true>(a, grad_source, vec_ok, out_aligned, stream);
}

hipError_t launch_adamw_sum(const AdamwArgs& a, int grad_source, bool vec_ok, bool out_aligned,
                            hipStream_t stream) {
    return launch_sum_source<false>(a, grad_source, vec_ok, out_aligned, stream);
}

hipError_t launch_adam_update_tiled(const AdamwArgs& a, bool out_aligned, hipStream_t stream) {
    return launch_form<kUpdate, false, true>(a, true, out_aligned, stream);
}

hipError_t launch_adamw_no_master_tiled(const AdamwArgs& a, bool vec_ok, hipStream_t stream) {
    return launch_form<kNoMaster, false, true>(a, vec_ok, true, stream);
}

}  // namespace zs
