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
// owns the 8 consecutive elements [8k, 8k+8) (two 128-bit accesses per fp32
// stream, one per bf16 stream), so a wave64 touches 2 KiB of each fp32
// stream per access pair.  A misaligned shard (a view into a larger buffer
// whose element offset is not a multiple of 4) takes the VEC = 1
// instantiation of the same code.
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

template <int VEC, bool BF16>
__global__ __launch_bounds__(kBlock) void adamw_kernel(const AdamwArgs a) {
    float coef;
    if (!clip_coef(a, coef)) return;
    const int64_t n = a.n;
    const int64_t first = ((int64_t)blockIdx.x * kBlock + threadIdx.x) * VEC;
    if (first >= n) return;

    if (VEC == 8 && first + 8 <= n) {
        const f32x4* g4 = reinterpret_cast<const f32x4*>(a.grad + first);
        f32x4* p4 = reinterpret_cast<f32x4*>(a.master + first);
        f32x4* m4 = reinterpret_cast<f32x4*>(a.exp_avg + first);
        f32x4* v4 = reinterpret_cast<f32x4*>(a.exp_avg_sq + first);
        // issue all eight 128-bit loads before any use
        f32x4 g0 = ld_stream(g4), g1 = ld_stream(g4 + 1);
        f32x4 p0 = ld_stream(p4), p1 = ld_stream(p4 + 1);
        f32x4 m0 = ld_stream(m4), m1 = ld_stream(m4 + 1);
        f32x4 v0 = ld_stream(v4), v1 = ld_stream(v4 + 1);
        float gs[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
        float ps[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
        float ms[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
        float vs[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) adamw_elem(a, coef, gs[j], ps[j], ms[j], vs[j]);
        st_stream(p4, f32x4{ps[0], ps[1], ps[2], ps[3]});
        st_stream(p4 + 1, f32x4{ps[4], ps[5], ps[6], ps[7]});
        st_stream(m4, f32x4{ms[0], ms[1], ms[2], ms[3]});
        st_stream(m4 + 1, f32x4{ms[4], ms[5], ms[6], ms[7]});
        st_stream(v4, f32x4{vs[0], vs[1], vs[2], vs[3]});
        st_stream(v4 + 1, f32x4{vs[4], vs[5], vs[6], vs[7]});
        if (BF16) {
            u32x4 b = {pack_bf16x2(ps[0], ps[1]), pack_bf16x2(ps[2], ps[3]),
                       pack_bf16x2(ps[4], ps[5]), pack_bf16x2(ps[6], ps[7])};
            st_stream(reinterpret_cast<u32x4*>(a.param_bf16 + first), b);
        }
        return;
    }
    // scalar path: VEC == 1, or the ragged tail of the VEC == 8 grid
    const int64_t last = first + VEC < n ? first + VEC : n;
    for (int64_t i = first; i < last; ++i) {
        float p = a.master[i], m = a.exp_avg[i], v = a.exp_avg_sq[i];
        adamw_elem(a, coef, a.grad[i], p, m, v);
        a.master[i] = p;
        a.exp_avg[i] = m;
        a.exp_avg_sq[i] = v;
        if (BF16) a.param_bf16[i] = (uint16_t)f32_to_bf16_rne(p);
    }
}

template <int VEC, bool BF16>
hipError_t launch(const AdamwArgs& a, hipStream_t stream) {
    const int64_t threads = (a.n + VEC - 1) / VEC;
    const int64_t blocks = (threads + kBlock - 1) / kBlock;
    hipLaunchKernelGGL((adamw_kernel<VEC, BF16>), dim3((unsigned)blocks), dim3(kBlock), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_adamw(const AdamwArgs& a, bool vec_ok, hipStream_t stream) {
    const bool bf16 = a.param_bf16 != nullptr;
    if (vec_ok) return bf16 ? launch<8, true>(a, stream) : launch<8, false>(a, stream);
    return bf16 ? launch<1, true>(a, stream) : launch<1, false>(a, stream);
}

}  // namespace zs
