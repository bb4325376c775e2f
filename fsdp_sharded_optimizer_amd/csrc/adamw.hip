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
// Layout: every array is a flat 1-D fp32 (bf16) buffer; thread k of the grid
// owns the 4 consecutive elements [4k, 4k+4): one 128-bit access per fp32
// stream and one 64-bit access for the bf16 stream, so each wave64 access
// covers 1 KiB of a stream with no gaps.  One-shot grid of one-wave
// workgroups (256 elements each), with residency capped at 10 workgroups
// per CU: each workgroup reserves 16 KiB of LDS it never touches, out of
// gfx950's 160 KiB per CU.  Eight concurrent streams per element (4 read,
// 4 written) otherwise keep too many DRAM rows open at once; on gfx950 the
// cap lifts the kernel from 74 % to 83 % of the 8 TB/s peak (fewer waves:
// 64-71 %; more: 73-81 %).  A misaligned shard (a view whose element offset
// is not a multiple of 4) takes the VEC = 1 instantiation of the same code,
// in 256-thread workgroups without the cap.
#include "zs_common.h"

namespace zs {
namespace {

// One element of the update, in the order and with the roundings the
// header documents.  Built with -ffp-contract=off: no multiply-add fusion;
// the quotient and square root are IEEE round-to-nearest (correctly rounded
// fp32 division and sqrt are requested at compile time).
__device__ __forceinline__ void adamw_elem(const AdamwArgs& a, float coef, float gr, float& p,
                                           float& m, float& v) {
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
    const float u = ratio * a.step_size;
    const float pd = p * a.decay;
    p = pd - u;
}

// Clip coefficient from the squared norm, in binary64 (uniform per wave).
// Returns false when the global squared norm is not finite: the step is
// skipped and nothing is written.
__device__ __forceinline__ bool clip_coef(const AdamwArgs& a, float& coef) {
    coef = 1.0f;
    if (a.norm_sq == nullptr) return true;
    const double s = *a.norm_sq + a.extra_norm_sq;
    if (!__builtin_isfinite(s)) return false;
    if (a.clip) {
        const double total = sqrt(s);
        double c = a.max_norm / (total + 1e-6);
        if (c > 1.0) c = 1.0;
        coef = (float)c;
    }
    return true;
}

// vector path: one wave per workgroup, 16 KiB of LDS reserved per workgroup
constexpr int kVecBlock = 64;
constexpr unsigned kVecLdsReserve = 16384;

// NO_MASTER: the bf16 parameter is read, updated and rounded back in place
// (no fp32 master): 24 B/element (R g, m, v 12 + p 2; W m, v 8 + p 2).
template <int VEC, bool BF16, int BS, bool NO_MASTER = false>
__global__ __launch_bounds__(BS) void adamw_kernel(const AdamwArgs a) {
    const int64_t n = a.n;
    const int64_t first = ((int64_t)blockIdx.x * BS + threadIdx.x) * VEC;
    if (first >= n) return;

    if (VEC == 4 && first + 4 <= n) {
        // One 128-bit access per fp32 stream, lane-contiguous across the wave.
        // The loads are issued before the clip coefficient is resolved, so
        // the latency of the norm's read overlaps with them.
        const f32x4 g4 = ld_stream(reinterpret_cast<const f32x4*>(a.grad + first));
        f32x4 p4;
        if (NO_MASTER) {
            const u32x2 w = ld_stream(reinterpret_cast<const u32x2*>(a.param_bf16 + first));
            p4 = f32x4{bf16_to_f32(w.x & 0xFFFFu), bf16_to_f32(w.x >> 16), bf16_to_f32(w.y & 0xFFFFu),
                       bf16_to_f32(w.y >> 16)};
        } else {
            p4 = ld_stream(reinterpret_cast<const f32x4*>(a.master + first));
        }
        const f32x4 m4 = ld_stream(reinterpret_cast<const f32x4*>(a.exp_avg + first));
        const f32x4 v4 = ld_stream(reinterpret_cast<const f32x4*>(a.exp_avg_sq + first));
        float coef;
        if (!clip_coef(a, coef)) return;
        float gs[4] = {g4.x, g4.y, g4.z, g4.w};
        float ps[4] = {p4.x, p4.y, p4.z, p4.w};
        float ms[4] = {m4.x, m4.y, m4.z, m4.w};
        float vs[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) adamw_elem(a, coef, gs[j], ps[j], ms[j], vs[j]);
        if (!NO_MASTER)
            st_stream(reinterpret_cast<f32x4*>(a.master + first), f32x4{ps[0], ps[1], ps[2], ps[3]});
        st_stream(reinterpret_cast<f32x4*>(a.exp_avg + first), f32x4{ms[0], ms[1], ms[2], ms[3]});
        st_stream(reinterpret_cast<f32x4*>(a.exp_avg_sq + first), f32x4{vs[0], vs[1], vs[2], vs[3]});
        if (BF16 || NO_MASTER)
            st_stream(reinterpret_cast<u32x2*>(a.param_bf16 + first),
                      u32x2{pack_bf16x2(ps[0], ps[1]), pack_bf16x2(ps[2], ps[3])});
        return;
    }
    // scalar path: VEC == 1, or the ragged tail of the VEC == 4 grid
    float coef;
    if (!clip_coef(a, coef)) return;
    const int64_t last = first + VEC < n ? first + VEC : n;
    for (int64_t i = first; i < last; ++i) {
        float p = NO_MASTER ? bf16_to_f32(a.param_bf16[i]) : a.master[i];
        float m = a.exp_avg[i], v = a.exp_avg_sq[i];
        adamw_elem(a, coef, a.grad[i], p, m, v);
        if (!NO_MASTER) a.master[i] = p;
        a.exp_avg[i] = m;
        a.exp_avg_sq[i] = v;
        if (BF16 || NO_MASTER) a.param_bf16[i] = (uint16_t)f32_to_bf16_rne(p);
    }
}

template <int VEC, bool BF16, int BS, bool NO_MASTER = false>
hipError_t launch(const AdamwArgs& a, unsigned lds, hipStream_t stream) {
    const int64_t threads = (a.n + VEC - 1) / VEC;
    const int64_t blocks = (threads + BS - 1) / BS;
    if (blocks > (int64_t)UINT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL((adamw_kernel<VEC, BF16, BS, NO_MASTER>), dim3((unsigned)blocks), dim3(BS), lds, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_adamw_no_master(const AdamwArgs& a, bool vec_ok, hipStream_t stream) {
    if (vec_ok) return launch<4, true, kVecBlock, true>(a, kVecLdsReserve, stream);
    return launch<1, true, kBlock, true>(a, 0, stream);
}

hipError_t launch_adamw(const AdamwArgs& a, bool vec_ok, hipStream_t stream) {
    const bool bf16 = a.param_bf16 != nullptr;
    if (vec_ok)
        return bf16 ? launch<4, true, kVecBlock>(a, kVecLdsReserve, stream)
                    : launch<4, false, kVecBlock>(a, kVecLdsReserve, stream);
    return bf16 ? launch<1, true, kBlock>(a, 0, stream) : launch<1, false, kBlock>(a, 0, stream);
}

}  // namespace zs
