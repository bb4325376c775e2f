/*
 * Oracle for the per-rank ZeRO/FSDP optimizer step — TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU implementation of what the GPU library
 * computes.  Only the test suite, the smoke check and the benchmark's CPU
 * baseline may load it.  It shares no source, header, constant or helper with
 * the GPU library, and the GPU library never calls it.
 *
 * Sources (pages; section / listing named, never line numbers):
 *   [ZeRO page]   ai6s.net "cann-recipes-train" ZeRO 三阶段 page
 *                 (https://ai6s.net/6a2abebd10ee7a33f27b4f16.html)
 *   [Accum page]  ai6s.net LLaMA-13B 梯度累积 + Gradient Checkpoint page
 *                 (https://ai6s.net/6a128b8710ee7a33f274bf75.html)
 *   [Memory page] ybb.press "大模型分布式训练并行与显存工程实战"
 *                 (https://www.ybb.press/ai-applications/14955.html)
 *
 * Arithmetic rules: every floating-point operation below is one IEEE-754
 * binary32 (or binary64 where stated) operation with round-to-nearest-even.
 * Build with -ffp-contract=off -fno-fast-math so that no a*b+c is fused and
 * subnormals are kept.  OpenMP only splits independent elements across
 * threads (and the norm across fixed blocks), so no result depends on the
 * thread count.
 *
 * Pins: every function here is checked by tests/test_oracle_*.py against
 * closed forms, brute force, invariants or an independent library routine.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1

/* Threads of every OpenMP loop below: the count orc_set_num_threads set,
 * else OpenMP's default (no result depends on it). */
#ifdef _OPENMP
#include <omp.h>
#endif
static int g_team = 0;
static int orc_team(void)
{
#ifdef _OPENMP
    return g_team > 0 ? g_team : omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------ */
/* bit helpers                                                          */
/* ------------------------------------------------------------------ */
static uint32_t f32_bits(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }
static float bits_f32(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }

/*
 * bf16 from fp32, round to nearest, ties to even.  The pages keep an fp32
 * master and a bf16 parameter ([ZeRO page] "组合策略" recipe docstring:
 * FP32 master weights; [Memory page] FSDP MixedPrecision param_dtype=bf16)
 * but never write the cast; this is the IEEE round-to-nearest-even reading.
 * Every NaN maps to the single quiet NaN 0x7FC0.
 */
uint16_t orc_bf16_rne(float x)
{
    if (isnan(x)) return (uint16_t)0x7FC0;
    uint32_t u = f32_bits(x);
    uint32_t hi = u >> 16;
    uint32_t lo = u & 0xFFFFu;
    /* round up when the dropped half is above one half, or exactly one half
     * and the kept part is odd */
    if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u))) hi += 1u;
    return (uint16_t)hi;
}

/* bf16 to fp32 is exact: the bf16 pattern is the top half of the fp32 one. */
float orc_bf16_widen(uint16_t b) { return bits_f32((uint32_t)b << 16); }

void orc_bf16_rne_array(const float* x, uint16_t* out, int64_t n)
{
    #pragma omp parallel for schedule(static) num_threads(orc_team())
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_rne(x[i]);
}

/* ------------------------------------------------------------------ */
/* Shard range  ([ZeRO page] §ZeRO-1 ZeRO1Optimizer.__init__: chunk is  */
/* the ceiling of total/world, start = rank*chunk, end clipped to total;*/
/* §ZeRO-2 reduce_gradients recomputes the same chunk)                  */
/* ------------------------------------------------------------------ */
/*
 * out = {chunk, start, end, padded_total}.  Readings where the page leaves a
 * gap: a rank whose start lies past the end gets the empty range
 * [total, total) (the page's size would go negative); padded_total is
 * world*chunk, the length the equal-size all-gather / reduce-scatter of the
 * page need.  Returns 0, or -1 for world < 1, rank outside [0, world) or
 * total < 0.
 */
int orc_shard_range(int64_t total, int32_t world, int32_t rank, int64_t out[4])
{
    if (world < 1 || rank < 0 || rank >= world || total < 0) return -1;
    int64_t chunk = (total + world - 1) / world;
    int64_t start = (int64_t)rank * chunk;
    if (start > total) start = total;
    int64_t end = start + chunk;
    if (end > total) end = total;
    out[0] = chunk;
    out[1] = start;
    out[2] = end;
    out[3] = (int64_t)world * chunk;
    return 0;
}

/* ------------------------------------------------------------------ */
/* Element conversion used by pack / unpack / accumulate               */
/* ------------------------------------------------------------------ */
static float load_as_f32(const void* p, int32_t dtype, int64_t i)
{
    if (dtype == ORC_F32) return ((const float*)p)[i];
    return orc_bf16_widen(((const uint16_t*)p)[i]);
}

/* copy one element from (src,sd)[i] to (dst,dd)[j]; same dtype is a bit copy */
static void convert_one(const void* src, int32_t sd, int64_t i, void* dst, int32_t dd, int64_t j)
{
    if (sd == dd) {
        if (sd == ORC_F32) ((uint32_t*)dst)[j] = ((const uint32_t*)src)[i];
        else ((uint16_t*)dst)[j] = ((const uint16_t*)src)[i];
    } else if (sd == ORC_BF16 && dd == ORC_F32) {
        ((float*)dst)[j] = orc_bf16_widen(((const uint16_t*)src)[i]);
    } else { /* fp32 -> bf16 */
        ((uint16_t*)dst)[j] = orc_bf16_rne(((const float*)src)[i]);
    }
}

static int dtype_ok(int32_t d) { return d == ORC_F32 || d == ORC_BF16; }

/* ------------------------------------------------------------------ */
/* Flatten  ([ZeRO page] §ZeRO-1 _flatten_gradients: each tensor viewed */
/* as 1-D and concatenated in parameter order; [Memory page] "FSDP 的关 */
/* 键抽象：FlatParameter": one 1-D buffer per wrap unit)                */
/* ------------------------------------------------------------------ */
/*
 * flat[o_i + j] = src_i[j] with o_i the running sum of the earlier numels;
 * flat[total, padded_total) = 0.  Allowed dtype pairs: same dtype, or
 * bf16 -> fp32 (the exact widening of the page's .float()).
 * Returns 0, or -1 when a numel is negative, sum(numel) > padded_total or a
 * dtype pair is not allowed.
 */
int orc_flat_pack(const void* const* src, const int64_t* numel, int32_t count, int32_t src_dtype,
                  void* flat, int32_t flat_dtype, int64_t padded_total)
{
    if (count < 0 || !dtype_ok(src_dtype) || !dtype_ok(flat_dtype)) return -1;
    if (src_dtype == ORC_F32 && flat_dtype == ORC_BF16) return -1;
    int64_t total = 0;
    for (int32_t t = 0; t < count; ++t) {
        if (numel[t] < 0) return -1;
        total += numel[t];
    }
    if (total > padded_total) return -1;
    int64_t offset = 0;
    for (int32_t t = 0; t < count; ++t) {
        for (int64_t j = 0; j < numel[t]; ++j)
            convert_one(src[t], src_dtype, j, flat, flat_dtype, offset + j);
        offset += numel[t];
    }
    for (int64_t k = total; k < padded_total; ++k) {
        if (flat_dtype == ORC_F32) ((uint32_t*)flat)[k] = 0u;
        else ((uint16_t*)flat)[k] = 0u;
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Unflatten  ([ZeRO page] §ZeRO-1 _apply_update: walk an offset over   */
/* the parameters, each taking the next numel elements of the flat      */
/* buffer; padding is never read)                                       */
/* ------------------------------------------------------------------ */
/*
 * dst_i[j] = flat[o_i + j].  Allowed dtype pairs: same dtype, or
 * fp32 -> bf16 (round to nearest even, the re-cast above).
 */
int orc_flat_unpack(const void* flat, int32_t flat_dtype, void* const* dst, const int64_t* numel,
                    int32_t count, int32_t dst_dtype)
{
    if (count < 0 || !dtype_ok(flat_dtype) || !dtype_ok(dst_dtype)) return -1;
    if (flat_dtype == ORC_BF16 && dst_dtype == ORC_F32) return -1;
    int64_t offset = 0;
    for (int32_t t = 0; t < count; ++t) {
        if (numel[t] < 0) return -1;
        for (int64_t j = 0; j < numel[t]; ++j)
            convert_one(flat, flat_dtype, offset + j, dst[t], dst_dtype, j);
        offset += numel[t];
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Gradient accumulation  ([ZeRO page] "梯度累积——用计算换通信"          */
/* GradientAccumulator.backward: fp32 buffer += grad.float(), one       */
/* micro-batch after another; [Memory page] FlatParameter section:     */
/* reduce_dtype fp32 because the reduction is a sum)                    */
/* ------------------------------------------------------------------ */
/*
 * overwrite != 0 (first micro-batch): acc_i = widen(g_i) — a copy, so -0.0
 * stays -0.0.  overwrite == 0: acc_i = fl(acc_i + widen(g_i)).
 */
int orc_grad_accum(float* acc, const void* grad, int32_t grad_dtype, int64_t n, int32_t overwrite)
{
    if (n < 0 || !dtype_ok(grad_dtype)) return -1;
    #pragma omp parallel for schedule(static) num_threads(orc_team())
    for (int64_t i = 0; i < n; ++i) {
        float g = load_as_f32(grad, grad_dtype, i);
        if (overwrite) acc[i] = g;
        else acc[i] = acc[i] + g;
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Squared L2 norm of the scaled gradient                              */
/* ([ZeRO page] §ZeRO-1 step and §ZeRO-2 reduce_gradients divide the   */
/* summed gradient by the world size; "组合策略" recipe divides the loss */
/* by the accumulation steps, then clip_grad_norm_(max_norm=1.0) over  */
/* all parameters; [Accum page] "梯度累积" the same clip after the      */
/* micro-batches)                                                       */
/* ------------------------------------------------------------------ */
#define ORC_NORM_BLOCK ((int64_t)1 << 20)

/*
 * g1_i = fl32(acc_i * s32) with s32 = (float)grad_scale; returns
 * S = sum_i (double)g1_i * (double)g1_i.  Each square is exact in binary64.
 * The sum runs in ascending order inside fixed blocks of 2^20 elements,
 * then over the block sums in ascending order, so the value does not depend
 * on the thread count.
 */
double orc_grad_norm_sq(const float* acc, int64_t n, double grad_scale)
{
    if (n <= 0) return 0.0;
    const float s32 = (float)grad_scale;
    int64_t nblocks = (n + ORC_NORM_BLOCK - 1) / ORC_NORM_BLOCK;
    double* part = (double*)malloc((size_t)nblocks * sizeof(double));
    if (!part) return NAN;
    #pragma omp parallel for schedule(static) num_threads(orc_team())
    for (int64_t b = 0; b < nblocks; ++b) {
        int64_t lo = b * ORC_NORM_BLOCK;
        int64_t hi = lo + ORC_NORM_BLOCK < n ? lo + ORC_NORM_BLOCK : n;
        double s = 0.0;
        for (int64_t i = lo; i < hi; ++i) {
            float g1 = acc[i] * s32;
            double gd = (double)g1;
            s = s + gd * gd;
        }
        part[b] = s;
    }
    double total = 0.0;
    for (int64_t b = 0; b < nblocks; ++b) total = total + part[b];
    free(part);
    return total;
}

/* ------------------------------------------------------------------ */
/* AdamW step on one rank's shard                                       */
/* ------------------------------------------------------------------ */
typedef struct {
    double lr, beta1, beta2, eps, weight_decay;
    double grad_scale;     /* 1/(accumulation_steps * world_size) */
    double max_norm;       /* <= 0: no clip */
    double extra_norm_sq;  /* the other ranks' share of the squared norm */
    int64_t step;          /* t >= 1 */
} orc_adamw_hp;

typedef struct {
    float beta1, beta2;       /* (float)beta */
    float one_minus_beta1;    /* (float)(1 - beta1) */
    float one_minus_beta2;    /* (float)(1 - beta2) */
    float step_size;          /* (float)(lr / bias_correction1) */
    float bias_correction2_sqrt; /* (float)sqrt(bias_correction2) */
    float eps;                /* (float)eps */
    float decay;              /* (float)(1 - lr*weight_decay); 1 when wd = 0 */
    float grad_scale;         /* (float)grad_scale */
} orc_adamw_scalars;

/*
 * Host scalars.  [ZeRO page] §ZeRO-1 step: the step counter is incremented
 * before use (first step t = 1); bias_correction1 = 1 - beta1^t,
 * bias_correction2 = 1 - beta2^t as Python floats (binary64);
 * step_size = lr / bias_correction1; the denominator divides sqrt(v) by
 * sqrt(bias_correction2).  Decoupled weight decay (AdamW, named on the
 * [Memory page] "一、显存账本" as the default optimizer, its formula not
 * given) multiplies the master by 1 - lr*wd.  Every scalar is formed in
 * binary64 and rounded to binary32 once.
 * Returns 0, or -1 for out-of-range hyperparameters.
 */
int orc_adamw_scalars_make(const orc_adamw_hp* hp, orc_adamw_scalars* s)
{
    if (hp->step < 1) return -1;
    if (!(hp->beta1 >= 0.0 && hp->beta1 < 1.0)) return -1;
    if (!(hp->beta2 >= 0.0 && hp->beta2 < 1.0)) return -1;
    if (!(hp->eps > 0.0) || !(hp->lr >= 0.0) || !(hp->weight_decay >= 0.0)) return -1;
    if (!(hp->grad_scale > 0.0) || !isfinite(hp->grad_scale)) return -1;
    double bc1 = 1.0 - pow(hp->beta1, (double)hp->step);
    double bc2 = 1.0 - pow(hp->beta2, (double)hp->step);
    s->beta1 = (float)hp->beta1;
    s->beta2 = (float)hp->beta2;
    s->one_minus_beta1 = (float)(1.0 - hp->beta1);
    s->one_minus_beta2 = (float)(1.0 - hp->beta2);
    s->step_size = (float)(hp->lr / bc1);
    s->bias_correction2_sqrt = (float)sqrt(bc2);
    s->eps = (float)hp->eps;
    s->decay = (float)(1.0 - hp->lr * hp->weight_decay);
    s->grad_scale = (float)hp->grad_scale;
    return 0;
}

/*
 * Clip coefficient.  The pages call clip_grad_norm_(max_norm=1.0) with no
 * formula; the reading is the library's: total = sqrt(S) over every rank's
 * squares, coef = max_norm / (total + 1e-6), applied when below 1 (so it
 * applies at total == max_norm).  Computed in binary64, rounded once.
 */
float orc_clip_coef(double norm_sq_local, double extra_norm_sq, double max_norm)
{
    if (!(max_norm > 0.0)) return 1.0f;
    double total = sqrt(norm_sq_local + extra_norm_sq);
    double coef = max_norm / (total + 1e-6);
    if (coef > 1.0) coef = 1.0;
    return (float)coef;
}

/*
 * One AdamW step over n elements, in place on master / exp_avg / exp_avg_sq;
 * param_bf16 (may be NULL) receives bf16_rne(new master).
 *
 * norm_sq: NULL -> no clip and no finiteness check.  Otherwise *norm_sq is
 * this shard's sum of squares (orc_grad_norm_sq); S = *norm_sq +
 * extra_norm_sq.  A non-finite S leaves every buffer untouched and returns 1
 * ([ZeRO page] "组合策略" recipe: a non-finite grad norm skips the update).
 *
 * Per element, in this order, one rounding per operation, no fusion
 * ([ZeRO page] §"ZeRO-1: 切分优化器状态", the optimizer step: first and
 * second moments as exponential moving averages of g and g^2, the second
 * moment's square root divided by the square root of its bias correction
 * before eps is added, the first moment over that denominator scaled by the
 * learning rate over the first bias correction, subtracted from p):
 *   g  = fl(fl(acc*scale) * coef)
 *   m  = fl(fl(beta1*m) + fl((1-beta1)*g))
 *   v  = fl(fl(beta2*v) + fl((1-beta2)*fl(g*g)))
 *   den= fl(fl(sqrt(v) / sqrt(bc2)) + eps)
 *   u  = fl(fl(m/den) * step_size)
 *   p  = fl(fl(p*decay) - u)
 * Returns 0 (updated), 1 (skipped) or -1 (invalid arguments).
 */
int orc_adamw_step(const orc_adamw_hp* hp, float* master, float* exp_avg, float* exp_avg_sq,
                   const float* grad, uint16_t* param_bf16, int64_t n, const double* norm_sq)
{
    orc_adamw_scalars s;
    if (n < 0 || orc_adamw_scalars_make(hp, &s) != 0) return -1;
    float coef = 1.0f;
    if (norm_sq) {
        double S = *norm_sq + hp->extra_norm_sq;
        if (!isfinite(S)) return 1;
        coef = orc_clip_coef(*norm_sq, hp->extra_norm_sq, hp->max_norm);
    }
    #pragma omp parallel for schedule(static) num_threads(orc_team())
    for (int64_t i = 0; i < n; ++i) {
        float g = grad[i] * s.grad_scale;
        g = g * coef;
        float m = exp_avg[i];
        float v = exp_avg_sq[i];
        float p = master[i];
        float m_a = s.beta1 * m;
        float m_b = s.one_minus_beta1 * g;
        m = m_a + m_b;
        float gg = g * g;
        float v_a = s.beta2 * v;
        float v_b = s.one_minus_beta2 * gg;
        v = v_a + v_b;
        float root = sqrtf(v);
        float den = root / s.bias_correction2_sqrt;
        den = den + s.eps;
        float ratio = m / den;
        float u = ratio * s.step_size;
        float pd = p * s.decay;
        p = pd - u;
        exp_avg[i] = m;
        exp_avg_sq[i] = v;
        master[i] = p;
        if (param_bf16) param_bf16[i] = orc_bf16_rne(p);
    }
    return 0;
}

/*
 * The same step with no fp32 master: the bf16 parameter itself is read,
 * updated and rounded back ([ZeRO page] §"ZeRO-3: 切分参数", ZeRO3Optimizer.step
 * adds the update straight into the low-precision parameter chunk).  Per
 * element: p = widen(param_bf16[i]); m, v, den, u as in orc_adamw_step;
 * param_bf16[i] = bf16_rne(fl(fl(p*decay) - u)).  An update smaller than
 * half a bf16 ulp of p leaves the parameter unchanged: the stall an fp32
 * master avoids.  Returns 0 (updated), 1 (skipped) or -1.
 */
int orc_adamw_step_no_master(const orc_adamw_hp* hp, uint16_t* param_bf16, float* exp_avg, float* exp_avg_sq,
                             const float* grad, int64_t n, const double* norm_sq)
{
    orc_adamw_scalars s;
    if (n < 0 || !param_bf16 || orc_adamw_scalars_make(hp, &s) != 0) return -1;
    float coef = 1.0f;
    if (norm_sq) {
        double S = *norm_sq + hp->extra_norm_sq;
        if (!isfinite(S)) return 1;
        coef = orc_clip_coef(*norm_sq, hp->extra_norm_sq, hp->max_norm);
    }
    #pragma omp parallel for schedule(static) num_threads(orc_team())
    for (int64_t i = 0; i < n; ++i) {
        float g = grad[i] * s.grad_scale;
        g = g * coef;
        float m = exp_avg[i];
        float v = exp_avg_sq[i];
        float p = orc_bf16_widen(param_bf16[i]);
        m = s.beta1 * m + s.one_minus_beta1 * g;
        float gg = g * g;
        v = s.beta2 * v + s.one_minus_beta2 * gg;
        float den = sqrtf(v) / s.bias_correction2_sqrt + s.eps;
        float u = (m / den) * s.step_size;
        float pd = p * s.decay;
        exp_avg[i] = m;
        exp_avg_sq[i] = v;
        param_bf16[i] = orc_bf16_rne(pd - u);
    }
    return 0;
}

/*
 * The ZeRO-1 form of the step ([ZeRO page] §"ZeRO-1: 切分优化器状态",
 * ZeRO1Optimizer.step): plain Adam over this rank's slice of the full,
 * averaged gradient, whose result is an update vector rather than a new
 * parameter.  Every rank's update is then gathered into one full-length
 * buffer and added into the parameters (orc_flat_apply_update below).
 * Per element: g, m, v, den as in orc_adamw_step, then
 *   update[i] = fl(fl(m/den) * (-step_size))
 * the page's exp_avg / denom * (-step_size).  The page's ZeRO-1 has no
 * weight decay, and a decoupled decay has no update-vector form that adds
 * to the same bits, so weight_decay must be 0 (else -1).  Adding the update
 * to p gives fl(p - u): the master path of orc_adamw_step with decay 1.
 * A non-finite S skips the step ([ZeRO page] "组合策略" recipe: a
 * non-finite grad norm skips the update): the moments are left untouched and
 * every update[i] is written as -0.0, the identity of IEEE addition
 * (x + -0.0 == x for every x, -0.0 and NaN included), so the apply that
 * follows the all-gather leaves every parameter as it was instead of adding
 * whatever the update buffer held before.
 * Returns 0 (written), 1 (skipped: non-finite norm, update = -0.0) or -1.
 */
int orc_adam_update(const orc_adamw_hp* hp, float* exp_avg, float* exp_avg_sq, const float* grad,
                    float* update, int64_t n, const double* norm_sq)
{
    orc_adamw_scalars s;
    if (n < 0 || hp->weight_decay != 0.0 || orc_adamw_scalars_make(hp, &s) != 0) return -1;
    float coef = 1.0f;
    if (norm_sq) {
        double S = *norm_sq + hp->extra_norm_sq;
        if (!isfinite(S)) {
            for (int64_t i = 0; i < n; ++i) update[i] = -0.0f;
            return 1;
        }
        coef = orc_clip_coef(*norm_sq, hp->extra_norm_sq, hp->max_norm);
    }
    const float neg_step_size = -s.step_size;
    #pragma omp parallel for schedule(static) num_threads(orc_team())
    for (int64_t i = 0; i < n; ++i) {
        float g = grad[i] * s.grad_scale;
        g = g * coef;
        float m = s.beta1 * exp_avg[i] + s.one_minus_beta1 * g;
        float v = s.beta2 * exp_avg_sq[i] + s.one_minus_beta2 * (g * g);
        float denom = sqrtf(v) / s.bias_correction2_sqrt + s.eps;
        exp_avg[i] = m;
        exp_avg_sq[i] = v;
        update[i] = m / denom * neg_step_size;
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Apply a gathered update  ([ZeRO page] §ZeRO-1 _apply_update: walk an */
/* offset over the parameters; each adds the next numel elements of the */
/* full update in place)                                                */
/* ------------------------------------------------------------------ */
/*
 * dst_i[j] += update[o_i + j], o_i the running sum of the earlier numels.
 * fp32 parameters: fl(p + u).  bf16 parameters: bf16_rne(fl(widen(p) + u)),
 * the page's in-place add on a low-precision tensor read as one fp32 add
 * rounded once into the parameter's dtype.  Elements past sum(numel) (the
 * all-gather's padding) are never read.  Returns 0, or -1 for a negative
 * numel or an unknown dtype.
 */
int orc_flat_apply_update(const float* update, void* const* dst, const int64_t* numel, int32_t count,
                          int32_t dst_dtype)
{
    if (count < 0 || !dtype_ok(dst_dtype)) return -1;
    for (int32_t t = 0; t < count; ++t)
        if (numel[t] < 0) return -1;
    int64_t offset = 0;
    for (int32_t t = 0; t < count; ++t) {
        for (int64_t j = 0; j < numel[t]; ++j) {
            float u = update[offset + j];
            if (dst_dtype == ORC_F32) {
                float* p = (float*)dst[t];
                p[j] = p[j] + u;
            } else {
                uint16_t* p = (uint16_t*)dst[t];
                p[j] = orc_bf16_rne(orc_bf16_widen(p[j]) + u);
            }
        }
        offset += numel[t];
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Tiled optimizer state: a storage layout, not arithmetic.  The pages  */
/* keep an fp32 master, exp_avg and exp_avg_sq per parameter ([Memory   */
/* page] "一、显存账本": 4 + 4 + 4 of the 16 B per parameter) and update */
/* every element on its own ([Memory page] same section; [ZeRO page]    */
/* §ZeRO-1/2/3 step), so where the values are stored cannot change any  */
/* result.  The layout groups the shard in tiles of `tile` elements;    */
/* tile t holds, one after the other, a run of each array (master,      */
/* exp_avg, exp_avg_sq; or exp_avg, exp_avg_sq alone) for its elements  */
/* [t*tile, (t+1)*tile).                                                */
/* ------------------------------------------------------------------ */
/* floats a tiled buffer of n elements occupies with `runs` arrays per tile:
 * runs runs of `tile` per started tile.  -1 for n < 0, tile < 1 or runs < 1. */
int64_t orc_tiled_runs_numel(int64_t n, int64_t tile, int runs)
{
    if (n < 0 || tile < 1 || runs < 1) return -1;
    int64_t tiles = n / tile;
    if (n % tile != 0) tiles += 1;
    return (int64_t)runs * tile * tiles;
}

/* buf[(runs*t + k)*tile + j] = src[k][t*tile + j] for t*tile + j < n, and 0
 * past n (the unused end of the last tile).  A NULL src[k] stands for zeros.
 * Returns 0, or -1 for n < 0, tile < 1 or runs < 1. */
int orc_tile_runs(const float* const* src, int runs, float* buf, int64_t n, int64_t tile)
{
    int64_t total = orc_tiled_runs_numel(n, tile, runs);
    if (total < 0) return -1;
    int64_t tiles = total / ((int64_t)runs * tile);
    for (int64_t t = 0; t < tiles; ++t)
        for (int k = 0; k < runs; ++k)
            for (int64_t j = 0; j < tile; ++j) {
                int64_t e = t * tile + j;
                float x = 0.0f;
                if (e < n && src[k] != NULL) x = src[k][e];
                buf[((int64_t)runs * t + k) * tile + j] = x;
            }
    return 0;
}

/* The inverse: dst[k][e] = buf[(runs*(e / tile) + k)*tile + e % tile] for
 * e < n; a NULL dst[k] is skipped.  Returns 0, or -1 for bad arguments. */
int orc_untile_runs(const float* buf, int runs, float* const* dst, int64_t n, int64_t tile)
{
    if (orc_tiled_runs_numel(n, tile, runs) < 0) return -1;
    for (int k = 0; k < runs; ++k) {
        if (dst[k] == NULL) continue;
        for (int64_t e = 0; e < n; ++e) {
            int64_t t = e / tile, j = e % tile;
            dst[k][e] = buf[((int64_t)runs * t + k) * tile + j];
        }
    }
    return 0;
}

/* The optimizer state of a master form: master, exp_avg, exp_avg_sq (three
 * runs per tile). */
int64_t orc_state_tiled_numel(int64_t n, int64_t tile) { return orc_tiled_runs_numel(n, tile, 3); }

int orc_state_tile(const float* master, const float* exp_avg, const float* exp_avg_sq, float* state,
                   int64_t n, int64_t tile)
{
    const float* src[3] = {master, exp_avg, exp_avg_sq};
    return orc_tile_runs(src, 3, state, n, tile);
}

int orc_state_untile(const float* state, float* master, float* exp_avg, float* exp_avg_sq,
                     int64_t n, int64_t tile)
{
    float* dst[3] = {master, exp_avg, exp_avg_sq};
    return orc_untile_runs(state, 3, dst, n, tile);
}

/* The moments alone (the no-master and ZeRO-1 forms hold no fp32 master):
 * exp_avg, exp_avg_sq (two runs per tile). */
int64_t orc_moments_tiled_numel(int64_t n, int64_t tile) { return orc_tiled_runs_numel(n, tile, 2); }

int orc_moments_tile(const float* exp_avg, const float* exp_avg_sq, float* moments, int64_t n, int64_t tile)
{
    const float* src[2] = {exp_avg, exp_avg_sq};
    return orc_tile_runs(src, 2, moments, n, tile);
}

int orc_moments_untile(const float* moments, float* exp_avg, float* exp_avg_sq, int64_t n, int64_t tile)
{
    float* dst[2] = {exp_avg, exp_avg_sq};
    return orc_untile_runs(moments, 2, dst, n, tile);
}

/* Thread count OpenMP will use for the loops above (reported by the
 * CPU-baseline timing). */
int orc_num_threads(void) { return orc_team(); }
void orc_set_num_threads(int n) { if (n > 0) g_team = n; }
