/*
 * zshard.h — C ABI of the MI355X (gfx950) per-rank ZeRO/FSDP optimizer-step
 * library (libzshard.so).
 *
 * The library runs one data-parallel rank's share of a sharded optimizer
 * step over a flattened 1-D parameter buffer: the shard range, flattening
 * and unflattening, fp32 gradient accumulation, the scaled squared gradient
 * norm with the global-norm clip, and the fused AdamW update of the fp32
 * master / exp_avg / exp_avg_sq with the bf16 re-cast.  Collectives are the
 * caller's business; the only cross-rank quantity the library consumes is
 * the other ranks' share of the squared norm (zs_adamw.extra_norm_sq).
 *
 * Sources (pages; section or listing named):
 *   [ZeRO page]   ai6s.net "cann-recipes-train" ZeRO 三阶段 page
 *                 (https://ai6s.net/6a2abebd10ee7a33f27b4f16.html)
 *   [Accum page]  ai6s.net LLaMA-13B 梯度累积 + Gradient Checkpoint page
 *                 (https://ai6s.net/6a128b8710ee7a33f274bf75.html)
 *   [Memory page] ybb.press "大模型分布式训练并行与显存工程实战"
 *                 (https://www.ybb.press/ai-applications/14955.html)
 *
 * Conventions for every entry point:
 *   - extern "C"; no exception crosses the ABI; every function is reentrant
 *     and keeps no state except the thread-local last HIP error.
 *   - Device buffers are owned by the caller (allocated and freed by it);
 *     the library allocates nothing.  Host arrays passed in (zs_tensor
 *     lists, zs_adamw) are read during the call only.
 *   - hip_stream is a hipStream_t (NULL = the default stream) of the current
 *     device, and every device buffer lives on that device.  Device calls
 *     only enqueue work on it and return; nothing blocks, nothing syncs,
 *     nothing is allocated or cleared, so a sequence of calls can be
 *     captured into a HIP graph as is.
 *   - Arguments are validated on the host before anything is enqueued; on
 *     failure the call returns a negative code and launches nothing.
 *     n == 0 (or count == 0 with nothing to pad) is a valid no-op.
 *   - Element counts (n, numel, padded_total, their sums) are at most 2^39
 *     per call; larger counts are ZS_EINVAL.  A call over more than 2^31
 *     elements is enqueued as several launches of at most 2^31 elements
 *     each (HIP grids stay below 2^32 work-items), with the same results as
 *     one; a ZS_EHIP from a later launch leaves the earlier ones enqueued.
 *   - fp32 pointers must be 4-byte aligned, bf16 pointers 2-byte aligned,
 *     fp64 pointers 8-byte aligned.  Any alignment beyond that only selects
 *     a faster code path: 128-bit accesses when every buffer a call writes
 *     is 16-byte aligned and every buffer it only reads is 4-byte aligned
 *     (a view at any element offset of an fp32 buffer, or at an even one of
 *     a bf16 buffer); element-wise accesses otherwise.  The AdamW steps and
 *     adam_update relax this for their one write-only output (param_bf16,
 *     update): at any element offset it is written element by element while
 *     everything else keeps the 128-bit path.  Full speed wants buffers that
 *     are read and written to start on a 128-byte boundary (whole cache lines
 *     per wave); adamw_step, adamw_step_dev and adam_update run the first
 *     1-31 elements of views that share one offset off that boundary element
 *     by element and the rest on the 128-bit path.
 *   - bf16 values are passed as their 16-bit patterns (uint16_t).
 *   - Placement (speed only): on gfx950 the streaming calls ran 1-6 points
 *     of the HBM peak faster with a rank's streamed buffers (tiled state,
 *     accumulator, micro-batch gradients, bf16 parameter) carved from one
 *     hipExtMallocWithFlags(..., hipDeviceMallocContiguous) block allocated
 *     at start-up than as separate allocations made after other processes
 *     had allocated and freed device memory.  Such a block bypasses the L2
 *     for writes, so keep the norm workspaces (sparse 8-byte partials) and
 *     *out_sq_dev out of it, and do not free it before the process ends:
 *     freeing memory of that kind has left later allocations holding stale
 *     values on this hardware.
 */
#ifndef ZSHARD_H
#define ZSHARD_H

#include <stdint.h>

/* Only the functions below are exported from libzshard.so; the library is
 * built with hidden visibility for everything else. */
#if defined(__GNUC__) || defined(__clang__)
#define ZS_API __attribute__((visibility("default")))
#else
#define ZS_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* element types */
enum { ZS_F32 = 0, ZS_BF16 = 1 };

/* return codes */
enum {
    ZS_OK = 0,
    ZS_EINVAL = -1,     /* bad argument: null pointer with work to do, range,
                           dtype, misalignment, size mismatch */
    ZS_EOVERLAP = -2,   /* two buffers that must be disjoint overlap */
    ZS_EWORKSPACE = -3, /* workspace smaller than grad_norm_sq_workspace_bytes */
    ZS_EHIP = -4        /* a HIP launch (or another HIP call) failed; see zs_last_hip_error() */
};

/* One rank's range of the flat buffer. */
typedef struct {
    int64_t chunk;        /* ceil(total / world) */
    int64_t start;        /* min(rank * chunk, total) */
    int64_t end;          /* min(start + chunk, total) */
    int64_t padded_total; /* world * chunk */
} zs_shard;

/* A contiguous device tensor, seen as 1-D in row-major order. */
typedef struct {
    void* ptr;            /* device pointer; may be NULL only when numel == 0 */
    int64_t numel;
} zs_tensor;

/* AdamW hyperparameters and step state, all host values.  Every scalar the
 * kernel uses is formed from these in binary64 and rounded to binary32 once. */
typedef struct {
    double lr;            /* >= 0 */
    double beta1, beta2;  /* in [0, 1) */
    double eps;           /* > 0, added after the bias-corrected sqrt */
    double weight_decay;  /* >= 0; decoupled (master *= 1 - lr*wd); 0 = Adam */
    double grad_scale;    /* > 0; the stored gradient is multiplied by it:
                             1/(accumulation_steps * world_size) */
    double max_norm;      /* > 0: clip to this global L2 norm; <= 0: no clip */
    double extra_norm_sq; /* >= 0 or non-finite: the other ranks' sum of
                             squares of their scaled gradients (the result of
                             the scalar all-reduce); 0 for a single rank, or
                             when *norm_sq_dev was itself all-reduced across
                             ranks on the device (no host synchronisation) */
    int64_t step;         /* t >= 1, caller-owned, incremented before the call */
} zs_adamw;

/*
 * zero_shard_range — the range of the flat buffer that `rank` owns.
 * [ZeRO page] §"ZeRO-1: 切分 Optimizer States", ZeRO1Optimizer.__init__
 * (chunk is the ceiling of total/world, start = rank*chunk, end clipped to
 * total) and §"ZeRO-2" reduce_gradients (same chunk).  padded_total is the
 * length the equal-size all-gather / reduce-scatter of those sections need.
 * A rank that starts past the end gets the empty range [total, total).
 * Host only (no GPU needed).  out: caller-owned host struct.
 * Errors: ZS_EINVAL for out == NULL, world < 1, rank outside [0, world),
 * total < 0, or world*chunk overflowing int64.
 */
ZS_API int32_t zero_shard_range(int64_t total, int32_t world, int32_t rank, zs_shard* out);

/*
 * flat_pack — the FlatParameter flatten.
 * [ZeRO page] §ZeRO-1 _flatten_gradients (each tensor viewed 1-D, in
 * parameter order, concatenated; .float() widening) and [Memory page]
 * §"FSDP 的关键抽象：FlatParameter" (one 1-D buffer per wrap unit).
 * flat[o_i + j] = src[i][j], o_i = sum of the numels before i; the tail
 * [sum(numel), padded_total) is set to zero (the padding to a multiple of
 * the world size).
 * src: host array of `count` device tensors of dtype src_dtype (read).
 * flat: device buffer of padded_total elements of flat_dtype (written).
 * dtype pairs: (F32,F32), (BF16,BF16) bit copies; (BF16,F32) exact widening.
 * Errors: ZS_EINVAL (count < 0, negative numel, sum(numel) > padded_total,
 * dtype pair, null/misaligned pointer), ZS_EOVERLAP (a source overlaps
 * flat), ZS_EHIP.
 */
ZS_API int32_t flat_pack(const zs_tensor* src, int32_t count, int32_t src_dtype,
                         void* flat, int32_t flat_dtype, int64_t padded_total, void* hip_stream);

/*
 * flat_unpack — the inverse of flat_pack, padding dropped.
 * [ZeRO page] §ZeRO-1 _apply_update (an offset walks the parameters, each
 * taking its next numel elements of the flat buffer).
 * dst[i][j] = flat[o_i + j].  flat: device, read; dst: host array of
 * `count` device tensors, written; they must not overlap flat or each other.
 * dtype pairs: (F32,F32), (BF16,BF16) bit copies; (F32,BF16) the bf16
 * round-to-nearest-even re-cast (NaN -> 0x7FC0).
 * Errors: as flat_pack.
 */
ZS_API int32_t flat_unpack(const void* flat, int32_t flat_dtype,
                           const zs_tensor* dst, int32_t count, int32_t dst_dtype, void* hip_stream);

/*
 * flat_apply_update — add a gathered fp32 update into the parameters.
 * [ZeRO page] §ZeRO-1 _apply_update: an offset walks the parameters and each
 * adds its next numel elements of the full (all-gathered) update in place.
 * dst[i][j] += update[o_i + j], o_i = sum of the numels before i; elements
 * of update past sum(numel) (the all-gather's padding) are not read.
 * F32 tensors: fl(p + u).  BF16 tensors: bf16_rne(fl(widen(p) + u)), the
 * in-place add on a low-precision tensor done as one fp32 add rounded once.
 * update: device fp32[sum(numel)] or longer, read; dst: host array of
 * `count` device tensors of dst_dtype, read-write; they must not overlap
 * update or each other.
 * Errors: ZS_EINVAL (count < 0, negative numel, dtype, null/misaligned
 * pointer), ZS_EOVERLAP, ZS_EHIP.
 */
ZS_API int32_t flat_apply_update(const float* update, const zs_tensor* dst, int32_t count, int32_t dst_dtype,
                                 void* hip_stream);

/*
 * grad_accum — fp32 gradient accumulation over micro-batches.
 * [ZeRO page] §"梯度累积——用计算换通信" GradientAccumulator.backward
 * (an fp32 buffer adds each micro-batch's grad.float()) and [Memory page]
 * §FlatParameter (reduce_dtype fp32: the reduction is a sum).
 * overwrite != 0 (first micro-batch): acc[i] = widen(grad[i]) (a copy);
 * overwrite == 0: acc[i] = fl32(acc[i] + widen(grad[i])).
 * acc: device fp32[n], read-write; grad: device [n] of grad_dtype, read.
 * Errors: ZS_EINVAL, ZS_EOVERLAP (acc overlaps grad), ZS_EHIP.
 */
ZS_API int32_t grad_accum(float* acc, const void* grad, int32_t grad_dtype, int64_t n,
                          int32_t overwrite, void* hip_stream);

/*
 * grad_reduce_chunks — the receiving side of a reduce-scatter on one GPU:
 * this rank's fp32 shard is the sum, in rank order, of the N ranks' chunks
 * for it.  [ZeRO page] §"ZeRO-2" reduce_gradients (reduce_scatter_tensor with
 * SUM, then the division by the world size, which this library applies
 * later as part of zs_adamw.grad_scale) and [Memory page] §FlatParameter
 * (the reduce-scatter runs with reduce_dtype fp32).
 * acc = (overwrite ? widen(chunks[0]) : fl32(acc + widen(chunks[0]))), then
 * acc = fl32(acc + widen(chunks[k])) for k = 1 .. count-1: the same left fold,
 * bit for bit, as one grad_accum call per chunk, in one pass per 16 chunks.
 * acc: device fp32[n], read-write; chunks: host array of `count` device
 * pointers, each [n] of grad_dtype, read (they may alias each other, not
 * acc).  count == 0 with overwrite == 0 is a no-op.
 * Errors: ZS_EINVAL (count < 0, count == 0 with overwrite, null/misaligned
 * pointer, dtype), ZS_EOVERLAP (a chunk overlaps acc), ZS_EHIP.
 */
ZS_API int32_t grad_reduce_chunks(float* acc, const void* const* chunks, int32_t count, int32_t grad_dtype, int64_t n,
                                  int32_t overwrite, void* hip_stream);

/*
 * grad_reduce_chunks_norm_sq_workspace_bytes — bytes of device workspace
 * grad_reduce_chunks_norm_sq needs for n elements (0 for n == 0; -1 for
 * n < 0 or n > 2^39).  Host only.
 */
ZS_API int64_t grad_reduce_chunks_norm_sq_workspace_bytes(int64_t n);

/*
 * grad_reduce_chunks_norm_sq — grad_reduce_chunks followed by grad_norm_sq
 * of the result, in one pass over the buffer: for a step whose micro-batch
 * gradients are all held in device memory, [ZeRO page] §"组合策略" recipe
 * (gradient accumulation over micro-batches, then the global-norm clip) with
 * the accumulation taken in one fold.
 * acc: as grad_reduce_chunks, bit for bit the same left fold, in rank (or
 * micro-batch) order.  *out_sq_dev (device binary64) = sum over i of
 * (grad_scale * acc[i])^2 after the fold, summed as grad_accum_norm_sq sums
 * (binary64 partials per 512 elements in a fixed tree: bit-reproducible,
 * within 1e-5 relative of the exact sum).  count >= 1; chunks as in
 * grad_reduce_chunks; workspace: device, 8-byte aligned, at least
 * grad_reduce_chunks_norm_sq_workspace_bytes(n) bytes, scratch owned by the
 * caller for the duration of the call.  n == 0 writes 0.
 * Errors: ZS_EINVAL (count < 1, bad dtype or size, null or misaligned
 * pointers, grad_scale not finite and > 0), ZS_EWORKSPACE (workspace too
 * small), ZS_EOVERLAP (acc, a chunk, the workspace or *out_sq_dev overlap;
 * chunks may alias each other), ZS_EHIP.  On an error nothing is launched,
 * except ZS_EHIP from a launch after the first pass of more than 16 chunks.
 */
ZS_API int32_t grad_reduce_chunks_norm_sq(float* acc, const void* const* chunks, int32_t count, int32_t grad_dtype,
                                          int64_t n, int32_t overwrite, double grad_scale, double* out_sq_dev,
                                          void* workspace, int64_t workspace_bytes, void* hip_stream);

/*
 * grad_norm_sq_workspace_bytes — bytes of device workspace grad_norm_sq
 * needs for n elements (0 for n == 0; -1 for n < 0 or n > 2^39).  Host only.
 */
ZS_API int64_t grad_norm_sq_workspace_bytes(int64_t n);

/*
 * grad_norm_sq — this shard's share of the squared global gradient norm.
 * [ZeRO page] §ZeRO-1 step / §ZeRO-2 reduce_gradients (the summed gradient
 * is divided by the world size), §"组合策略" recipe (the loss is divided by
 * the accumulation steps; clip_grad_norm_(max_norm=1.0) over all
 * parameters) and [Accum page] §"梯度累积：用时间换显存" (the same clip
 * after the micro-batches).
 * *out_sq_dev = sum_i (double)g1_i^2 with g1_i = fl32(grad[i] *
 * (float)grad_scale); squares exact in binary64, summed in binary64 in a
 * fixed order (the result depends only on n and the data, run to run).
 * grad: device fp32[n], read.  out_sq_dev: device double, written (0 when
 * n == 0).  workspace: device, >= grad_norm_sq_workspace_bytes(n) bytes,
 * 8-byte aligned, scratch owned by the caller, may be reused after the
 * stream reaches the end of this call.
 * Errors: ZS_EINVAL, ZS_EWORKSPACE, ZS_EOVERLAP, ZS_EHIP.
 */
ZS_API int32_t grad_norm_sq(const float* grad, int64_t n, double grad_scale, double* out_sq_dev,
                            void* workspace, int64_t workspace_bytes, void* hip_stream);

/*
 * grad_accum_norm_sq_workspace_bytes — bytes of device workspace
 * grad_accum_norm_sq needs for n elements (0 for n == 0; -1 for n < 0 or
 * n > 2^39).
 */
ZS_API int64_t grad_accum_norm_sq_workspace_bytes(int64_t n);

/*
 * grad_accum_norm_sq — grad_accum fused with grad_norm_sq for the last
 * micro-batch: one pass accumulates and forms this shard's squared norm of
 * the scaled result, saving the norm's separate read of the accumulator.
 * Same sources as grad_accum and grad_norm_sq ([ZeRO page] "梯度累积" and
 * §"组合策略"; [Accum page] §"梯度累积：用时间换显存": the clip follows the
 * last micro-batch).
 * acc[i] as grad_accum; then *out_sq_dev = sum_i (double)g1_i^2 with
 * g1_i = fl32(acc[i] * (float)grad_scale), binary64, in a fixed order that
 * depends only on n (not the one grad_norm_sq uses: the two agree to
 * rounding, each is bit-reproducible run to run).
 * acc: device fp32[n], read-write; grad: device [n] of grad_dtype, read;
 * out_sq_dev: device double, written (0 when n == 0); workspace: device,
 * >= grad_accum_norm_sq_workspace_bytes(n) bytes, 8-byte aligned.
 * Errors: ZS_EINVAL, ZS_EWORKSPACE, ZS_EOVERLAP (any two of acc, grad,
 * *out_sq_dev, workspace), ZS_EHIP.
 */
ZS_API int32_t grad_accum_norm_sq(float* acc, const void* grad, int32_t grad_dtype, int64_t n, int32_t overwrite,
                                  double grad_scale, double* out_sq_dev, void* workspace, int64_t workspace_bytes,
                                  void* hip_stream);

/*
 * grad_sum_norm_sq — the squared norm grad_accum_norm_sq forms, without its
 * store: for a step that folds the last micro-batch into the AdamW update
 * (adamw_step_tiled_sum) instead of accumulating it first.  Same sources as
 * grad_accum_norm_sq ([ZeRO page] "梯度累积" and §"组合策略"; [Accum page]
 * §"梯度累积：用时间换显存": the clip follows the last micro-batch).
 * *out_sq_dev receives, bit for bit, the value grad_accum_norm_sq(acc, grad,
 * grad_dtype, n, overwrite, grad_scale, ...) would write (the same
 * association, fixed by n, overwrite and grad_dtype), and acc is left as it
 * is: read when overwrite == 0; not read, and may be NULL, when overwrite !=
 * 0.  Read-only passes: 6 B/element (bf16 gradient onto an accumulator), 2
 * (bf16, overwrite), 8 and 4 for fp32.
 * acc: device fp32[n], 4-byte aligned; grad: device [n] of grad_dtype;
 * out_sq_dev: device double, written (0 when n == 0); workspace: device,
 * >= grad_accum_norm_sq_workspace_bytes(n) bytes, 8-byte aligned.
 * Errors: ZS_EINVAL, ZS_EWORKSPACE, ZS_EOVERLAP (the workspace or
 * *out_sq_dev with any other buffer), ZS_EHIP.
 */
ZS_API int32_t grad_sum_norm_sq(const float* acc, const void* grad, int32_t grad_dtype, int64_t n, int32_t overwrite,
                                double grad_scale, double* out_sq_dev, void* workspace, int64_t workspace_bytes,
                                void* hip_stream);

/*
 * grad_accum_norm_sq_noalloc — grad_accum_norm_sq for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  It takes no workspace and
 * allocates nothing; the norm's partials go to a scratch array the library
 * holds in device memory, ZS_NOALLOC_SCRATCH_BYTES (64 MiB) on each GPU it
 * runs on, kept until the process ends.  n is at most ZS_NOALLOC_MAX_ELEMS
 * (2,146,959,360 elements).  Results are bit for bit those of
 * grad_accum_norm_sq (the same kernels and partial layout).
 * The first call on a device, with that device current, looks up the
 * array's device address (hipGetSymbolAddress); make that call outside a
 * graph capture.  Every call on one GPU uses that GPU's one array: calls
 * that overlap in time (two streams, two threads, two captured graphs
 * replaying at once) race on it and give wrong norms, so order them (one
 * stream, or events).  The array keeps the last call's partials; nothing
 * in it needs to start at zero (every partial a call reads, it wrote).
 * Arguments as grad_accum_norm_sq, without the workspace.
 * Errors: ZS_EINVAL (as grad_accum_norm_sq, or n > ZS_NOALLOC_MAX_ELEMS,
 * both found before any device call), ZS_EOVERLAP, ZS_EHIP (a launch, or
 * the array's address could not be obtained).
 */
#define ZS_NOALLOC_SCRATCH_BYTES (64ll << 20)
#define ZS_NOALLOC_MAX_ELEMS 2146959360ll
ZS_API int32_t grad_accum_norm_sq_noalloc(float* acc, const void* grad, int32_t grad_dtype, int64_t n,
                                          int32_t overwrite, double grad_scale, double* out_sq_dev,
                                          void* hip_stream);

/*
 * adamw_step — the fused AdamW update of one rank's shard.
 * [ZeRO page] §ZeRO-1 step, §ZeRO-2 step, §ZeRO-3 step: step counter
 * incremented before use; bias_correction1 = 1 - beta1^t,
 * bias_correction2 = 1 - beta2^t; exp_avg = beta1*exp_avg + (1-beta1)*g;
 * exp_avg_sq = beta2*exp_avg_sq + (1-beta2)*g*g; denom = sqrt(exp_avg_sq) /
 * sqrt(bias_correction2) + eps; update = -(lr/bias_correction1) * exp_avg /
 * denom.  [Memory page] §"一、显存账本": bf16 params with AdamW and an
 * element-wise, independent update per parameter; decoupled decay is this
 * library's reading (master *= 1 - lr*wd before the update).  The fp32
 * master is updated and param_bf16 (if not NULL) receives its bf16
 * round-to-nearest-even re-cast ([Memory page] FSDP MixedPrecision
 * param_dtype=bf16; [ZeRO page] §"组合策略" FP32 master weights).
 * Per element, one IEEE binary32 rounding per operation, no fusion:
 *   g = fl(fl(grad*scale)*coef); m = fl(fl(b1*m) + fl((1-b1)*g));
 *   v = fl(fl(b2*v) + fl((1-b2)*fl(g*g))); den = fl(fl(sqrt(v)/sqrt(bc2)) + eps);
 *   master = fl(fl(master*(1-lr*wd)) - fl(fl(m/den)*(lr/bc1)))
 * norm_sq_dev: NULL -> coef = 1, no check.  Otherwise a device double
 * holding this shard's squared norm (grad_norm_sq); S = *norm_sq_dev +
 * extra_norm_sq; a non-finite S leaves every buffer unchanged (the recipe
 * skips the update on a non-finite grad norm); else, when max_norm > 0,
 * coef = (float)min(1, max_norm / (sqrt(S) + 1e-6)), all in binary64 on the
 * device ([ZeRO page] §"组合策略" clip_grad_norm_).
 * master, exp_avg, exp_avg_sq: device fp32[n], read-write; grad: device
 * fp32[n], read; param_bf16: device bf16[n] or NULL, written.  No two of
 * them may overlap, nor overlap *norm_sq_dev.
 * Errors: ZS_EINVAL (hp NULL or out of range, pointers), ZS_EOVERLAP, ZS_EHIP.
 */
ZS_API int32_t adamw_step(const zs_adamw* hp, float* master, float* exp_avg, float* exp_avg_sq,
                          const float* grad, uint16_t* param_bf16, int64_t n,
                          const double* norm_sq_dev, void* hip_stream);

/*
 * adamw_step_sum — adamw_step whose gradient is the last micro-batch's
 * accumulation, formed as it is read (the split-buffer form of
 * adamw_step_tiled_sum, below): element i's gradient is fl(acc[i] +
 * widen(grad[i])), or widen(grad[i]) when acc is NULL.  Results are bit for
 * bit those of grad_accum(acc, grad, grad_dtype, n, acc == NULL) followed by
 * adamw_step(hp, master, exp_avg, exp_avg_sq, acc, ...); acc is only read.
 * Same sources as adamw_step_tiled_sum.
 * master, exp_avg, exp_avg_sq, param_bf16, norm_sq_dev: as adamw_step;
 * acc: device fp32[n], 4-byte aligned, read, or NULL; grad: device [n] of
 * grad_dtype (ZS_BF16 or ZS_F32), read.  No two of the six buffers may
 * overlap, nor a written one overlap *norm_sq_dev.
 * Errors: ZS_EINVAL (as adamw_step, or a bad grad_dtype), ZS_EOVERLAP,
 * ZS_EHIP.
 */
ZS_API int32_t adamw_step_sum(const zs_adamw* hp, float* master, float* exp_avg, float* exp_avg_sq, const float* acc,
                              const void* grad, int32_t grad_dtype, uint16_t* param_bf16, int64_t n,
                              const double* norm_sq_dev, void* hip_stream);

/*
 * The per-step scalars of adamw_step, formed on the host from zs_adamw in
 * binary64 and each rounded to binary32 once (beta1, beta2, 1 - beta1,
 * 1 - beta2, lr / (1 - beta1^t), sqrt(1 - beta2^t), eps, 1 - lr*wd,
 * grad_scale), plus the clip switch and the two binary64 clip inputs.
 */
typedef struct {
    float beta1, beta2;
    float one_minus_beta1, one_minus_beta2;
    float step_size;              /* (float)(lr / (1 - beta1^t)) */
    float bias_correction2_sqrt;  /* (float)sqrt(1 - beta2^t) */
    float eps;
    float decay;                  /* (float)(1 - lr * weight_decay) */
    float grad_scale;
    int32_t clip;                 /* max_norm > 0 */
    double max_norm;
    double extra_norm_sq;
} zs_adamw_scalars;

/*
 * adamw_scalars — the scalars adamw_step forms from hp, on the host.
 * Validates hp as adamw_step does (ZS_EINVAL; also for out == NULL).
 */
ZS_API int32_t adamw_scalars(const zs_adamw* hp, zs_adamw_scalars* out);

/*
 * adamw_step_dev — adamw_step with its scalars read from device memory.
 * The kernels read *scalars_dev (adamw_scalars' output, copied to the
 * device by the caller) when they run, not when the call is made: a step
 * captured once in a HIP graph, behind a copy of the next step's scalars
 * into scalars_dev, replays every later step (step counter, learning-rate
 * schedule, clip inputs) without re-capture.  Results are those of
 * adamw_step with the same hyperparameters, bit for bit.  scalars_dev:
 * device, 8-byte aligned, read; it must not overlap any written buffer.
 * The values are not validated (they are not on the host).  Other
 * arguments, layout and errors as adamw_step.
 */
ZS_API int32_t adamw_step_dev(const zs_adamw_scalars* scalars_dev, float* master, float* exp_avg,
                              float* exp_avg_sq, const float* grad, uint16_t* param_bf16, int64_t n,
                              const double* norm_sq_dev, void* hip_stream);

/*
 * adamw_step_sum_dev — adamw_step_sum with its scalars read from device
 * memory when the kernels run (as adamw_step_dev).  scalars_dev: device,
 * 8-byte aligned, read; it must not overlap a written buffer.  Other
 * arguments, results and errors as adamw_step_sum.
 */
ZS_API int32_t adamw_step_sum_dev(const zs_adamw_scalars* scalars_dev, float* master, float* exp_avg,
                                  float* exp_avg_sq, const float* acc, const void* grad, int32_t grad_dtype,
                                  uint16_t* param_bf16, int64_t n, const double* norm_sq_dev, void* hip_stream);

/*
 * Tiled optimizer state — a storage layout of this library, not of the
 * pages.  The pages keep an fp32 master, exp_avg and exp_avg_sq per
 * parameter ([Memory page] §"一、显存账本": 4 + 4 + 4 of the 16 B per
 * parameter) and update each element independently, so where the three
 * values sit changes no result.  The tiled layout keeps them in one fp32
 * buffer: the shard's elements are grouped in tiles of ZS_STATE_TILE; tile t
 * holds the masters of its elements [t*ZS_STATE_TILE, (t+1)*ZS_STATE_TILE),
 * then their exp_avgs, then their exp_avg_sqs, each a run of ZS_STATE_TILE
 * floats:
 *   state[(3*t + 0)*ZS_STATE_TILE + j]  master     of element t*ZS_STATE_TILE + j
 *   state[(3*t + 1)*ZS_STATE_TILE + j]  exp_avg    of that element
 *   state[(3*t + 2)*ZS_STATE_TILE + j]  exp_avg_sq of that element
 * The last tile keeps full-length runs; positions past n are padding, never
 * read by the step.  The AdamW step streams this layout faster than three
 * separate buffers on gfx950 (its three state accesses per element fall in
 * one region, so fewer DRAM rows are open at once); bytes and results are
 * the same.  A tiled state buffer must be 16-byte aligned (every hipMalloc
 * allocation is) and hold state_tiled_numel(n) floats.
 */
#define ZS_STATE_TILE 8192

/* Floats in the tiled state of n elements: 3 * ZS_STATE_TILE * ceil(n /
 * ZS_STATE_TILE).  -1 for n < 0 or n above the per-call limit.  Host only. */
ZS_API int64_t state_tiled_numel(int64_t n);

/*
 * state_tile — split arrays into the tiled layout.  master, exp_avg,
 * exp_avg_sq: device fp32[n], read; each may be NULL, which stands for zeros
 * (a fresh optimizer's moments).  state: device fp32[state_tiled_numel(n)],
 * written in full, the last tile's padding as zeros.  Bit-exact copies.
 * state must not overlap a source; the sources may overlap one another.
 * Errors: ZS_EINVAL (state NULL or not 16-byte aligned with n > 0, a source
 * not 4-byte aligned, n out of range), ZS_EOVERLAP, ZS_EHIP.
 */
ZS_API int32_t state_tile(const float* master, const float* exp_avg, const float* exp_avg_sq, float* state,
                          int64_t n, void* hip_stream);

/*
 * state_untile — the inverse: master, exp_avg, exp_avg_sq (device fp32[n],
 * written; each may be NULL: that stream is skipped) from the tiled state
 * (device fp32[state_tiled_numel(n)], read).  Bit-exact copies; checkpoints
 * and state_dicts use the split arrays.  The destinations must not overlap
 * the state or one another.  Errors: as state_tile.
 */
ZS_API int32_t state_untile(const float* state, float* master, float* exp_avg, float* exp_avg_sq, int64_t n,
                            void* hip_stream);

/*
 * adamw_step_tiled — adamw_step on a tiled state: the same update, order of
 * operations, clip and non-finite skip ([ZeRO page] §ZeRO-1/2/3 step;
 * decoupled decay as in adamw_step), with master, exp_avg and exp_avg_sq
 * read from and written back to their places in `state`.  Results are bit
 * for bit those of adamw_step on the untiled arrays; 30 B per element (28
 * without param_bf16), as adamw_step.
 * state: device fp32[state_tiled_numel(n)], 16-byte aligned, read-write
 * (padding untouched); grad: device fp32[n], read; param_bf16: device
 * bf16[n] or NULL, written; norm_sq_dev as in adamw_step.  No two of them
 * may overlap, nor overlap *norm_sq_dev.
 * Errors: ZS_EINVAL (as adamw_step, or state not 16-byte aligned),
 * ZS_EOVERLAP, ZS_EHIP.
 */
ZS_API int32_t adamw_step_tiled(const zs_adamw* hp, float* state, const float* grad, uint16_t* param_bf16,
                                int64_t n, const double* norm_sq_dev, void* hip_stream);

/*
 * adamw_step_tiled_dev — adamw_step_tiled with its scalars read from device
 * memory when the kernels run, as adamw_step_dev does for adamw_step (one
 * captured HIP graph replays every step).  scalars_dev: device, 8-byte
 * aligned, read; it must not overlap a written buffer.  Other arguments,
 * results and errors as adamw_step_tiled.
 */
ZS_API int32_t adamw_step_tiled_dev(const zs_adamw_scalars* scalars_dev, float* state, const float* grad,
                                    uint16_t* param_bf16, int64_t n, const double* norm_sq_dev, void* hip_stream);

/*
 * adamw_step_tiled_sum — adamw_step_tiled whose gradient is the last
 * micro-batch's accumulation, formed as it is read instead of stored first:
 * element i's gradient is the value grad_accum would leave in acc[i] for
 * this micro-batch, fl(acc[i] + widen(grad[i])), or widen(grad[i]) when acc
 * is NULL (a step of one micro-batch: grad_accum with overwrite).  The
 * accumulation and the step are the pages' ([ZeRO page] "梯度累积" and
 * §ZeRO-1/2/3 step; [Accum page] §"梯度累积：用时间换显存"); doing them in one
 * pass is this library's schedule.  Results are bit for bit those of
 * grad_accum(acc, grad, grad_dtype, n, acc == NULL) followed by
 * adamw_step_tiled(hp, state, acc, ...), but acc is only read, never
 * written: it does not hold the final gradient afterwards.  With the norm
 * from grad_sum_norm_sq, the last micro-batch and the step move 32 B per
 * element (bf16 gradient onto an accumulator; 28 with acc NULL) plus the
 * norm's read-only pass (6; 2), against grad_accum_norm_sq's 10 (6) and
 * adamw_step_tiled's 30.
 * state: as adamw_step_tiled; acc: device fp32[n], 4-byte aligned, read, or
 * NULL; grad: device [n] of grad_dtype (ZS_BF16 or ZS_F32), read;
 * param_bf16, norm_sq_dev as adamw_step_tiled.  No two of state, acc, grad,
 * param_bf16 may overlap, nor a written one overlap *norm_sq_dev.
 * Errors: ZS_EINVAL (as adamw_step_tiled, or a bad grad_dtype), ZS_EOVERLAP,
 * ZS_EHIP.
 */
ZS_API int32_t adamw_step_tiled_sum(const zs_adamw* hp, float* state, const float* acc, const void* grad,
                                    int32_t grad_dtype, uint16_t* param_bf16, int64_t n, const double* norm_sq_dev,
                                    void* hip_stream);

/*
 * adamw_step_tiled_sum_dev — adamw_step_tiled_sum with its scalars read from
 * device memory when the kernels run (as adamw_step_tiled_dev).
 * scalars_dev: device, 8-byte aligned, read; it must not overlap a written
 * buffer.  Other arguments, results and errors as adamw_step_tiled_sum.
 */
ZS_API int32_t adamw_step_tiled_sum_dev(const zs_adamw_scalars* scalars_dev, float* state, const float* acc,
                                        const void* grad, int32_t grad_dtype, uint16_t* param_bf16, int64_t n,
                                        const double* norm_sq_dev, void* hip_stream);

/*
 * Tiled moments — the same layout for the forms that keep no fp32 master
 * (adamw_step_no_master, adam_update): per tile of ZS_STATE_TILE elements,
 * the tile's exp_avgs, then its exp_avg_sqs, two runs of ZS_STATE_TILE floats:
 *   moments[(2*t + 0)*ZS_STATE_TILE + j]  exp_avg    of element t*ZS_STATE_TILE + j
 *   moments[(2*t + 1)*ZS_STATE_TILE + j]  exp_avg_sq of that element
 * moments_tiled_numel(n) floats (2 * ZS_STATE_TILE * ceil(n / ZS_STATE_TILE),
 * -1 for an invalid n; host only), 16-byte aligned.  moments_tile and
 * moments_untile convert as state_tile and state_untile do (NULL source:
 * zeros; NULL destination: skipped; same rules and errors).
 */
ZS_API int64_t moments_tiled_numel(int64_t n);
ZS_API int32_t moments_tile(const float* exp_avg, const float* exp_avg_sq, float* moments, int64_t n,
                            void* hip_stream);
ZS_API int32_t moments_untile(const float* moments, float* exp_avg, float* exp_avg_sq, int64_t n,
                              void* hip_stream);

/*
 * adamw_step_no_master — the same update with no fp32 master: the bf16
 * parameter shard is read, updated and rounded back in place.
 * [ZeRO page] §"ZeRO-3: 切分参数", ZeRO3Optimizer.step (the update is added
 * straight into the low-precision parameter chunk).  Per element:
 * p = widen(param_bf16); m, v, den and the update as in adamw_step;
 * param_bf16 = bf16_rne(fl(fl(p*(1-lr*wd)) - update)).  Saves 4 B of state
 * and 6 B of traffic per element, but an update smaller than half a bf16
 * ulp of the parameter is lost every step (the stall an fp32 master avoids).
 * param_bf16: device bf16[n], read-write; exp_avg, exp_avg_sq: device
 * fp32[n], read-write; grad: device fp32[n], read; norm_sq_dev as in
 * adamw_step.  Errors: as adamw_step.
 */
ZS_API int32_t adamw_step_no_master(const zs_adamw* hp, uint16_t* param_bf16, float* exp_avg, float* exp_avg_sq,
                                    const float* grad, int64_t n, const double* norm_sq_dev, void* hip_stream);

/*
 * adam_update — the ZeRO-1 form of the step: the update as a vector.
 * [ZeRO page] §"ZeRO-1: 切分优化器状态", ZeRO1Optimizer.step: plain Adam on
 * this rank's slice of the full averaged gradient (often a view at any
 * element offset of one resident flat buffer), producing
 * update = exp_avg / denom * (-lr/bias_correction1), which the caller
 * all-gathers and adds into the parameters (flat_apply_update).  m, v, den
 * and the clip as in adamw_step; update = fl(fl(m/den) * -(lr/bc1)).  The
 * page's ZeRO-1 has no weight decay, and decoupled decay has no
 * update-vector form with the same bits, so hp->weight_decay must be 0.
 * Adding the update to an fp32 parameter gives the bits adamw_step gives.
 * exp_avg, exp_avg_sq: device fp32[n], read-write; grad: device fp32[n],
 * read; update: device fp32[n], written.  No two may overlap, nor overlap
 * *norm_sq_dev.  A non-finite S skips the step ([ZeRO page] §"组合策略"
 * recipe): exp_avg and exp_avg_sq are left unchanged and every update[i] is
 * written as -0.0, the identity of IEEE addition, so flat_apply_update of the
 * gathered update leaves every parameter as it was (fp32 bit for bit; bf16
 * too, except that a NaN parameter is rewritten as the quiet NaN 0x7FC0).
 * Errors: ZS_EINVAL (as adamw_step, or weight_decay != 0), ZS_EOVERLAP,
 * ZS_EHIP.
 */
ZS_API int32_t adam_update(const zs_adamw* hp, float* exp_avg, float* exp_avg_sq, const float* grad, float* update,
                           int64_t n, const double* norm_sq_dev, void* hip_stream);

/*
 * adam_update_tiled, adamw_step_no_master_tiled — adam_update and
 * adamw_step_no_master with exp_avg and exp_avg_sq read from and written
 * back to tiled moments: the same arithmetic, results bit for bit, bytes per
 * element and rules (adam_update_tiled requires weight_decay = 0).
 * moments: device fp32[moments_tiled_numel(n)], 16-byte aligned, read-write
 * (padding untouched); grad: device fp32[n], read; update: device fp32[n],
 * written, at any element offset; param_bf16: device bf16[n], read-write.  No
 * two may overlap, nor overlap *norm_sq_dev.  Errors: as the split forms, or
 * ZS_EINVAL for moments not 16-byte aligned.
 */
ZS_API int32_t adam_update_tiled(const zs_adamw* hp, float* moments, const float* grad, float* update, int64_t n,
                                 const double* norm_sq_dev, void* hip_stream);
ZS_API int32_t adamw_step_no_master_tiled(const zs_adamw* hp, uint16_t* param_bf16, float* moments,
                                          const float* grad, int64_t n, const double* norm_sq_dev,
                                          void* hip_stream);

/* Static description of a return code. */
ZS_API const char* zs_strerror(int32_t code);

/* The hipError_t of the last ZS_EHIP on this thread (0 if none). */
ZS_API int32_t zs_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ZSHARD_H */
