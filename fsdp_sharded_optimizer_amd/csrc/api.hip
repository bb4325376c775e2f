// C-ABI entry points of libzshard (declared in include/zshard.h).
//
// Every call validates its arguments on the host first (null pointers,
// ranges, dtypes, alignment, overlap) and returns an error code without
// launching anything when they are wrong.  Valid calls only enqueue kernels
// on the caller's stream.  Host scalars are formed in binary64 and rounded
// to binary32 once.
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstddef>
#include <cstring>

#include "../../include/zshard.h"
#include "reduce.h"

namespace {

thread_local int32_t g_last_hip_error = 0;

int32_t hip_status(hipError_t e) {
    if (e == hipSuccess) return ZS_OK;
    g_last_hip_error = (int32_t)e;
    return ZS_EHIP;
}

inline uintptr_t addr(const void* p) { return reinterpret_cast<uintptr_t>(p); }
inline bool aligned(const void* p, uintptr_t a) { return (addr(p) & (a - 1)) == 0; }

// [p, p+bytes) and [q, q+qbytes) share a byte (empty ranges never overlap)
inline bool overlap(const void* p, int64_t bytes, const void* q, int64_t qbytes) {
    if (bytes <= 0 || qbytes <= 0) return false;
    const uintptr_t a = addr(p), b = addr(q);
    return a < b + (uintptr_t)qbytes && b < a + (uintptr_t)bytes;
}

inline int64_t elem_size(int32_t dtype) { return dtype == ZS_F32 ? 4 : 2; }
inline bool dtype_ok(int32_t d) { return d == ZS_F32 || d == ZS_BF16; }
inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// At most 2^39 elements per call (2 TiB of fp32, beyond any one GPU's
// memory): byte sizes stay far inside int64.  The launchers split a call
// into launches of at most 2^31 elements, so every grid stays below 2^32
// work-items.
constexpr int64_t kMaxElems = int64_t(1) << 39;
inline bool size_ok(int64_t n) { return n >= 0 && n <= kMaxElems; }

}  // namespace

// The scratch of grad_accum_norm_sq_noalloc: one array per GPU (each device
// holds its own copy of a __device__ variable), sized for the partials and
// chunk stage of ZS_NOALLOC_MAX_ELEMS elements.  In host code `scratch`
// names a host-side stand-in, not device memory: kernels get the address
// hipGetSymbolAddress returns for the current device, looked up once per
// device and kept in g_scratch_ptr.
constexpr int64_t kScratchBytes = ZS_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) double scratch[kScratchBytes / 8];
constexpr int kScratchDevices = 64;
static std::atomic<void*> g_scratch_ptr[kScratchDevices];

static_assert(ZS_NOALLOC_MAX_ELEMS % 256 == 0 &&
                  (ZS_NOALLOC_MAX_ELEMS / 256 + zs::kReduceChunks) * 8 == kScratchBytes,
              "the largest call's partials and chunk stage fill the scratch exactly");

// Device address of the current device's scratch (ZS_OK), looked up on the
// first call on that device.  Two threads racing on the first call look it
// up twice and store the same address.
static int32_t current_scratch(void** out) {
    int dev = -1;
    int32_t rc = hip_status(hipGetDevice(&dev));
    if (rc != ZS_OK) return rc;
    if (dev >= 0 && dev < kScratchDevices) {
        void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
        if (p != nullptr) {
            *out = p;
            return ZS_OK;
        }
    }
    void* p = nullptr;
    rc = hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (rc != ZS_OK) return rc;
    if (p == nullptr) return hip_status(hipErrorInvalidSymbol);
    if (dev >= 0 && dev < kScratchDevices) g_scratch_ptr[dev].store(p, std::memory_order_release);
    *out = p;
    return ZS_OK;
}

extern "C" {

const char* zs_strerror(int32_t code) {
    switch (code) {
        case ZS_OK: return "ok";
        case ZS_EINVAL: return "invalid argument";
        case ZS_EOVERLAP: return "buffers overlap";
        case ZS_EWORKSPACE: return "workspace too small";
        case ZS_EHIP: return "HIP call failed";
        default: return "unknown error code";
    }
}

int32_t zs_last_hip_error(void) { return g_last_hip_error; }

int32_t zero_shard_range(int64_t total, int32_t world, int32_t rank, zs_shard* out) {
    if (out == nullptr || world < 1 || rank < 0 || rank >= world || total < 0) return ZS_EINVAL;
    // ceil(total / world) without forming total + world - 1
    const int64_t chunk = total / world + (total % world != 0 ? 1 : 0);
    if (chunk > INT64_MAX / world) return ZS_EINVAL;
    int64_t start = (int64_t)rank * chunk;
    if (start > total) start = total;   // a rank past the end owns nothing
    const int64_t end = total - start < chunk ? total : start + chunk;
    out->chunk = chunk;
    out->start = start;
    out->end = end;
    out->padded_total = (int64_t)world * chunk;
    return ZS_OK;
}

int32_t grad_accum(float* acc, const void* grad, int32_t grad_dtype, int64_t n, int32_t overwrite,
                   void* hip_stream) {
    if (!dtype_ok(grad_dtype) || !size_ok(n)) return ZS_EINVAL;
    if (n == 0) return ZS_OK;
    const int64_t gsz = elem_size(grad_dtype);
    if (acc == nullptr || grad == nullptr) return ZS_EINVAL;
    if (!aligned(acc, 4) || !aligned(grad, (uintptr_t)gsz)) return ZS_EINVAL;
    if (overlap(acc, n * 4, grad, n * gsz)) return ZS_EOVERLAP;
    // written streams 16-byte aligned; the read-only gradient dword aligned
    const bool vec = aligned(acc, 16) && aligned(grad, 4);
    return hip_status(zs::launch_grad_accum(acc, grad, grad_dtype == ZS_BF16, n, overwrite != 0, vec,
                                            as_stream(hip_stream)));
}

int32_t grad_reduce_chunks(float* acc, const void* const* chunks, int32_t count, int32_t grad_dtype, int64_t n,
                           int32_t overwrite, void* hip_stream) {
    if (!dtype_ok(grad_dtype) || !size_ok(n) || count < 0) return ZS_EINVAL;
    if (n == 0) return ZS_OK;
    if (count == 0) return overwrite ? ZS_EINVAL : ZS_OK;
    if (acc == nullptr || chunks == nullptr || !aligned(acc, 4)) return ZS_EINVAL;
    const int64_t gsz = elem_size(grad_dtype);
    bool vec = aligned(acc, 16);
    for (int32_t k = 0; k < count; ++k) {
        if (chunks[k] == nullptr || !aligned(chunks[k], (uintptr_t)gsz)) return ZS_EINVAL;
        if (overlap(acc, n * 4, chunks[k], n * gsz)) return ZS_EOVERLAP;
        vec = vec && aligned(chunks[k], 4);   // read-only: dword alignment suffices
    }
    for (int32_t k0 = 0; k0 < count; k0 += zs::kReduceMaxChunks) {
        zs::ChunkBatch b;
        std::memset(&b, 0, sizeof(b));
        b.count = count - k0 < zs::kReduceMaxChunks ? count - k0 : zs::kReduceMaxChunks;
        for (int32_t k = 0; k < b.count; ++k) b.chunk[k] = chunks[k0 + k];
        const int32_t rc = hip_status(zs::launch_reduce_chunks(acc, b, grad_dtype == ZS_BF16, n,
                                                               (k0 == 0 && overwrite) ? 1 : 0, vec,
                                                               as_stream(hip_stream)));
        if (rc != ZS_OK) return rc;
    }
    return ZS_OK;
}

int64_t grad_reduce_chunks_norm_sq_workspace_bytes(int64_t n) {
    if (!size_ok(n)) return -1;
    const int64_t parts = zs::reduce_norm_partials(n);
    return parts == 0 ? 0 : (parts + zs::kReduceChunks) * (int64_t)sizeof(double);
}

int32_t grad_reduce_chunks_norm_sq(float* acc, const void* const* chunks, int32_t count, int32_t grad_dtype,
                                   int64_t n, int32_t overwrite, double grad_scale, double* out_sq_dev,
                                   void* workspace, int64_t workspace_bytes, void* hip_stream) {
    if (!dtype_ok(grad_dtype) || !size_ok(n) || count < 1) return ZS_EINVAL;
    if (out_sq_dev == nullptr || !aligned(out_sq_dev, 8)) return ZS_EINVAL;
    if (!(grad_scale > 0.0) || !std::isfinite(grad_scale)) return ZS_EINVAL;
    if (chunks == nullptr) return ZS_EINVAL;
    const int64_t gsz = elem_size(grad_dtype);
    if (n > 0 && (acc == nullptr || !aligned(acc, 4))) return ZS_EINVAL;
    const int64_t need = grad_reduce_chunks_norm_sq_workspace_bytes(n);
    if (need > 0 && (workspace == nullptr || !aligned(workspace, 8))) return ZS_EINVAL;
    if (workspace_bytes < need) return ZS_EWORKSPACE;
    if (overlap(acc, n * 4, out_sq_dev, 8) || overlap(workspace, need, out_sq_dev, 8) ||
        overlap(workspace, need, acc, n * 4))
        return ZS_EOVERLAP;
    bool vec = aligned(acc, 16);
    for (int32_t k = 0; k < count && n > 0; ++k) {
        if (chunks[k] == nullptr || !aligned(chunks[k], (uintptr_t)gsz)) return ZS_EINVAL;
        if (overlap(acc, n * 4, chunks[k], n * gsz) || overlap(chunks[k], n * gsz, out_sq_dev, 8) ||
            overlap(workspace, need, chunks[k], n * gsz))
            return ZS_EOVERLAP;
        vec = vec && aligned(chunks[k], 4);   // read-only: dword alignment suffices
    }
    hipStream_t stream = as_stream(hip_stream);
    // every pass but the last folds up to 16 chunks; the last also forms the norm
    int32_t k0 = 0;
    for (;;) {
        zs::ChunkBatch b;
        std::memset(&b, 0, sizeof(b));
        b.count = count - k0 < zs::kReduceMaxChunks ? count - k0 : zs::kReduceMaxChunks;
        for (int32_t k = 0; k < b.count; ++k) b.chunk[k] = chunks[k0 + k];
        const int ow = (k0 == 0 && overwrite) ? 1 : 0;
        if (k0 + b.count == count)
            return hip_status(zs::launch_reduce_chunks_norm_sq(acc, b, grad_dtype == ZS_BF16, n, ow, vec,
                                                               (float)grad_scale, out_sq_dev,
                                                               static_cast<double*>(workspace), stream));
        if (n > 0) {
            const int32_t rc =
                hip_status(zs::launch_reduce_chunks(acc, b, grad_dtype == ZS_BF16, n, ow, vec, stream));
            if (rc != ZS_OK) return rc;
        }
        k0 += b.count;
    }
}

int64_t grad_norm_sq_workspace_bytes(int64_t n) {
    if (!size_ok(n)) return -1;
    // one partial per 4096-element tile, then (beyond one workgroup's share)
    // the chunk stage of the partials' reduction
    const int64_t parts = zs::norm_partials(n);
    return (parts <= zs::kSumOneGroup ? parts : parts + zs::kReduceChunks) * (int64_t)sizeof(double);
}

int32_t grad_norm_sq(const float* grad, int64_t n, double grad_scale, double* out_sq_dev,
                     void* workspace, int64_t workspace_bytes, void* hip_stream) {
    if (!size_ok(n) || out_sq_dev == nullptr || !aligned(out_sq_dev, 8)) return ZS_EINVAL;
    if (!(grad_scale > 0.0) || !std::isfinite(grad_scale)) return ZS_EINVAL;
    const int64_t need = grad_norm_sq_workspace_bytes(n);
    if (n > 0 && (grad == nullptr || !aligned(grad, 4))) return ZS_EINVAL;
    if (need > 0 && (workspace == nullptr || !aligned(workspace, 8))) return ZS_EINVAL;
    if (workspace_bytes < need) return ZS_EWORKSPACE;
    if (overlap(grad, n * 4, out_sq_dev, 8) || overlap(workspace, need, out_sq_dev, 8) ||
        overlap(workspace, need, grad, n * 4))
        return ZS_EOVERLAP;
    return hip_status(zs::launch_grad_norm_sq(grad, n, (float)grad_scale, out_sq_dev,
                                              static_cast<double*>(workspace), as_stream(hip_stream)));
}

int64_t grad_accum_norm_sq_workspace_bytes(int64_t n) {
    if (!size_ok(n)) return -1;
    const int64_t parts = zs::accum_norm_partials(n);
    return parts == 0 ? 0 : (parts + zs::kReduceChunks) * (int64_t)sizeof(double);
}

int32_t grad_accum_norm_sq(float* acc, const void* grad, int32_t grad_dtype, int64_t n, int32_t overwrite,
                           double grad_scale, double* out_sq_dev, void* workspace, int64_t workspace_bytes,
                           void* hip_stream) {
    if (!dtype_ok(grad_dtype) || !size_ok(n)) return ZS_EINVAL;
    if (out_sq_dev == nullptr || !aligned(out_sq_dev, 8)) return ZS_EINVAL;
    if (!(grad_scale > 0.0) || !std::isfinite(grad_scale)) return ZS_EINVAL;
    const int64_t gsz = elem_size(grad_dtype);
    if (n > 0 && (acc == nullptr || grad == nullptr || !aligned(acc, 4) || !aligned(grad, (uintptr_t)gsz)))
        return ZS_EINVAL;
    const int64_t need = grad_accum_norm_sq_workspace_bytes(n);
    if (need > 0 && (workspace == nullptr || !aligned(workspace, 8))) return ZS_EINVAL;
    if (workspace_bytes < need) return ZS_EWORKSPACE;
    if (overlap(acc, n * 4, grad, n * gsz) || overlap(acc, n * 4, out_sq_dev, 8) ||
        overlap(grad, n * gsz, out_sq_dev, 8) || overlap(workspace, need, out_sq_dev, 8) ||
        overlap(workspace, need, acc, n * 4) || overlap(workspace, need, grad, n * gsz))
        return ZS_EOVERLAP;
    const bool vec = aligned(acc, 16) && aligned(grad, 4);
    return hip_status(zs::launch_grad_accum_norm_sq(acc, grad, grad_dtype == ZS_BF16, n, overwrite != 0,
                                                    (float)grad_scale, out_sq_dev,
                                                    static_cast<double*>(workspace), vec,
                                                    as_stream(hip_stream)));
}

int32_t grad_sum_norm_sq(const float* acc, const void* grad, int32_t grad_dtype, int64_t n, int32_t overwrite,
                         double grad_scale, double* out_sq_dev, void* workspace, int64_t workspace_bytes,
                         void* hip_stream) {
    if (!dtype_ok(grad_dtype) || !size_ok(n)) return ZS_EINVAL;
    if (out_sq_dev == nullptr || !aligned(out_sq_dev, 8)) return ZS_EINVAL;
    if (!(grad_scale > 0.0) || !std::isfinite(grad_scale)) return ZS_EINVAL;
    const int64_t gsz = elem_size(grad_dtype);
    if (overwrite) acc = nullptr;   // not read
    if (n > 0 && (grad == nullptr || !aligned(grad, (uintptr_t)gsz))) return ZS_EINVAL;
    if (n > 0 && !overwrite && (acc == nullptr || !aligned(acc, 4))) return ZS_EINVAL;
    const int64_t need = grad_accum_norm_sq_workspace_bytes(n);
    if (need > 0 && (workspace == nullptr || !aligned(workspace, 8))) return ZS_EINVAL;
    if (workspace_bytes < need) return ZS_EWORKSPACE;
    const int64_t acc_bytes = acc == nullptr ? 0 : n * 4;
    // only the workspace and *out_sq_dev are written
    if (overlap(acc, acc_bytes, out_sq_dev, 8) || overlap(grad, n * gsz, out_sq_dev, 8) ||
        overlap(workspace, need, out_sq_dev, 8) || overlap(workspace, need, acc, acc_bytes) ||
        overlap(workspace, need, grad, n * gsz))
        return ZS_EOVERLAP;
    return hip_status(zs::launch_grad_sum_norm_sq(acc, grad, grad_dtype == ZS_BF16, n, overwrite != 0,
                                                  (float)grad_scale, out_sq_dev, static_cast<double*>(workspace),
                                                  aligned(grad, 4), as_stream(hip_stream)));
}

// ---------------------------------------------------------------------------
// grad_accum_norm_sq with its partials in a static device array
// ---------------------------------------------------------------------------

int32_t grad_accum_norm_sq_noalloc(float* acc, const void* grad, int32_t grad_dtype, int64_t n, int32_t overwrite,
                                   double grad_scale, double* out_sq_dev, void* hip_stream) {
    // the size limit and the argument checks come before any device call
    if (n < 0 || n > ZS_NOALLOC_MAX_ELEMS) return ZS_EINVAL;
    const int64_t need = grad_accum_norm_sq_workspace_bytes(n);
    if (need < 0 || need > kScratchBytes) return ZS_EINVAL;
    if (!dtype_ok(grad_dtype) || out_sq_dev == nullptr || !aligned(out_sq_dev, 8)) return ZS_EINVAL;
    if (!(grad_scale > 0.0) || !std::isfinite(grad_scale)) return ZS_EINVAL;
    if (n > 0 && (acc == nullptr || grad == nullptr || !aligned(acc, 4) ||
                  !aligned(grad, (uintptr_t)elem_size(grad_dtype))))
        return ZS_EINVAL;
    void* ws = nullptr;
    const int32_t rc = current_scratch(&ws);
    if (rc != ZS_OK) return rc;
    // the workspace entry point's checks (overlap with the scratch included)
    // and launches, on the scratch
    return grad_accum_norm_sq(acc, grad, grad_dtype, n, overwrite, grad_scale, out_sq_dev, ws, kScratchBytes,
                              hip_stream);
}

// Elements to run element by element before the vector path when every
// buffer of `bufs` (fp32, read and written by the step) sits at the same
// offset off a 128-byte boundary: advancing all of them by that many elements
// (1-31, at most n) puts each wave's 1 KiB accesses on whole cache lines.
// A read-modify-write stream that is 16-byte aligned but not line aligned
// runs the vector path at 59-64 % of the HBM peak on gfx950 (waves share
// partly written lines), below the element-wise path's 65 %; peeled, 78-80 %.
// 0 when the buffers are line aligned already or their offsets differ.
constexpr uintptr_t kLineBytes = 128;
static int64_t shared_head(float* const* bufs, int count, int64_t n) {
    const uintptr_t off = addr(bufs[0]) & (kLineBytes - 1);
    if (off == 0) return 0;
    for (int i = 1; i < count; ++i)
        if ((addr(bufs[i]) & (kLineBytes - 1)) != off) return 0;
    const int64_t head = (int64_t)((kLineBytes - off) / 4);   // off is a multiple of 4 (fp32 alignment)
    return head < n ? head : n;
}

static int32_t adamw_check_hp(const zs_adamw* hp, int64_t n, const double* norm_sq_dev) {
    if (hp == nullptr || !size_ok(n)) return ZS_EINVAL;
    if (hp->step < 1) return ZS_EINVAL;
    if (!(hp->beta1 >= 0.0 && hp->beta1 < 1.0) || !(hp->beta2 >= 0.0 && hp->beta2 < 1.0))
        return ZS_EINVAL;
    if (!(hp->eps > 0.0) || !std::isfinite(hp->eps)) return ZS_EINVAL;
    if (!(hp->lr >= 0.0) || !std::isfinite(hp->lr)) return ZS_EINVAL;
    if (!(hp->weight_decay >= 0.0) || !std::isfinite(hp->weight_decay)) return ZS_EINVAL;
    if (!(hp->grad_scale > 0.0) || !std::isfinite(hp->grad_scale)) return ZS_EINVAL;
    if (std::isnan(hp->max_norm) || hp->extra_norm_sq < 0.0) return ZS_EINVAL;
    if (norm_sq_dev != nullptr && !aligned(norm_sq_dev, 8)) return ZS_EINVAL;
    return ZS_OK;
}

// host scalars: binary64, each rounded to binary32 once
static zs::AdamwScalars make_scalars(const zs_adamw* hp) {
    const double t = (double)hp->step;
    const double bias_correction1 = 1.0 - std::pow(hp->beta1, t);
    const double bias_correction2 = 1.0 - std::pow(hp->beta2, t);
    zs::AdamwScalars c;
    std::memset(&c, 0, sizeof(c));
    c.beta1 = (float)hp->beta1;
    c.beta2 = (float)hp->beta2;
    c.one_minus_beta1 = (float)(1.0 - hp->beta1);
    c.one_minus_beta2 = (float)(1.0 - hp->beta2);
    c.step_size = (float)(hp->lr / bias_correction1);
    c.bias_correction2_sqrt = (float)std::sqrt(bias_correction2);
    c.eps = (float)hp->eps;
    c.decay = (float)(1.0 - hp->lr * hp->weight_decay);
    c.grad_scale = (float)hp->grad_scale;
    c.clip = hp->max_norm > 0.0 ? 1 : 0;
    c.max_norm = hp->max_norm;
    c.extra_norm_sq = hp->extra_norm_sq;
    return c;
}

static zs::AdamwArgs make_args(const zs_adamw* hp, const double* norm_sq_dev) {
    zs::AdamwArgs a;
    std::memset(&a, 0, sizeof(a));
    a.sc = make_scalars(hp);
    a.norm_sq = norm_sq_dev;
    return a;
}

// the public struct and the kernels' one are the same bytes
static_assert(sizeof(zs_adamw_scalars) == sizeof(zs::AdamwScalars), "scalar layout");
static_assert(offsetof(zs_adamw_scalars, grad_scale) == offsetof(zs::AdamwScalars, grad_scale), "scalar layout");
static_assert(offsetof(zs_adamw_scalars, clip) == offsetof(zs::AdamwScalars, clip), "scalar layout");
static_assert(offsetof(zs_adamw_scalars, max_norm) == offsetof(zs::AdamwScalars, max_norm), "scalar layout");
static_assert(offsetof(zs_adamw_scalars, extra_norm_sq) == offsetof(zs::AdamwScalars, extra_norm_sq),
              "scalar layout");

// The scalars of a master-form step: host hyperparameters (hp, validated
// here) or a device copy of adamw_scalars' output (sc_dev: only its
// alignment can be checked); and the kernels' arguments for either.
static int32_t check_scalars(const zs_adamw* hp, const zs_adamw_scalars* sc_dev, int64_t n,
                             const double* norm_sq_dev) {
    if (sc_dev == nullptr) return adamw_check_hp(hp, n, norm_sq_dev);
    if (!size_ok(n) || !aligned(sc_dev, 8)) return ZS_EINVAL;
    if (norm_sq_dev != nullptr && !aligned(norm_sq_dev, 8)) return ZS_EINVAL;
    return ZS_OK;
}

static zs::AdamwArgs step_args(const zs_adamw* hp, const zs_adamw_scalars* sc_dev, const double* norm_sq_dev) {
    if (sc_dev == nullptr) return make_args(hp, norm_sq_dev);
    zs::AdamwArgs a;
    std::memset(&a, 0, sizeof(a));
    a.sc_dev = reinterpret_cast<const zs::AdamwScalars*>(sc_dev);
    a.norm_sq = norm_sq_dev;
    return a;
}

// the five buffers (any may be absent: bytes 0) pairwise disjoint, and none
// that is written overlapping the norm
static int32_t adamw_check_overlap(const void* const* bufs, const int64_t* bytes, const bool* written,
                                   const double* norm_sq_dev) {
    for (int i = 0; i < 5; ++i) {
        for (int j = i + 1; j < 5; ++j)
            if (overlap(bufs[i], bytes[i], bufs[j], bytes[j])) return ZS_EOVERLAP;
        if (norm_sq_dev != nullptr && written[i] && overlap(bufs[i], bytes[i], norm_sq_dev, 8))
            return ZS_EOVERLAP;
    }
    return ZS_OK;
}

// the master-form step: host scalars (hp) or a device copy of them (sc_dev)
static int32_t adamw_master(const zs_adamw* hp, const zs_adamw_scalars* sc_dev, float* master, float* exp_avg,
                            float* exp_avg_sq, const float* grad, uint16_t* param_bf16, int64_t n,
                            const double* norm_sq_dev, void* hip_stream) {
    int32_t rc = check_scalars(hp, sc_dev, n, norm_sq_dev);
    if (rc != ZS_OK) return rc;
    if (n == 0) return ZS_OK;
    if (master == nullptr || exp_avg == nullptr || exp_avg_sq == nullptr || grad == nullptr)
        return ZS_EINVAL;
    if (!aligned(master, 4) || !aligned(exp_avg, 4) || !aligned(exp_avg_sq, 4) || !aligned(grad, 4) ||
        (param_bf16 != nullptr && !aligned(param_bf16, 2)))
        return ZS_EINVAL;
    const void* bufs[5] = {master, exp_avg, exp_avg_sq, grad, param_bf16};
    const int64_t bytes[5] = {n * 4, n * 4, n * 4, n * 4, param_bf16 ? n * 2 : 0};
    const bool written[5] = {true, true, true, false, true};
    rc = adamw_check_overlap(bufs, bytes, written, norm_sq_dev);
    if (rc != ZS_OK) return rc;
    if (sc_dev != nullptr)   // the scalars are read while the buffers are written
        for (int i = 0; i < 5; ++i)
            if (written[i] && overlap(bufs[i], bytes[i], sc_dev, (int64_t)sizeof(zs_adamw_scalars)))
                return ZS_EOVERLAP;
    zs::AdamwArgs a = step_args(hp, sc_dev, norm_sq_dev);
    a.master = master;
    a.exp_avg = exp_avg;
    a.exp_avg_sq = exp_avg_sq;
    a.grad = grad;
    a.param_bf16 = param_bf16;
    a.n = n;
    // the read-write state 16-byte aligned (the read-only gradient is 4-byte
    // aligned already); the write-only bf16 output may sit at any element
    // offset.  Views sharing one offset off a 128-byte boundary run their
    // first 1-31 elements element by element and the rest on the vector path.
    float* const state[3] = {master, exp_avg, exp_avg_sq};
    const int64_t head = shared_head(state, 3, n);
    if (head > 0) {
        zs::AdamwArgs h = a;
        h.n = head;
        rc = hip_status(zs::launch_adamw(h, false, true, as_stream(hip_stream)));
        if (rc != ZS_OK) return rc;
        a.master += head;
        a.exp_avg += head;
        a.exp_avg_sq += head;
        a.grad += head;
        if (a.param_bf16 != nullptr) a.param_bf16 += head;
        a.n -= head;
    }
    const bool vec = aligned(a.master, 16) && aligned(a.exp_avg, 16) && aligned(a.exp_avg_sq, 16);
    const bool out_aligned = a.param_bf16 == nullptr || aligned(a.param_bf16, 16);
    if (a.n == 0) return ZS_OK;
    return hip_status(zs::launch_adamw(a, vec, out_aligned, as_stream(hip_stream)));
}

// the split master-form step on the last micro-batch's sum (acc, nullable, +
// grad of grad_dtype): host scalars (hp) or a device copy of them (sc_dev)
static int32_t adamw_master_sum(const zs_adamw* hp, const zs_adamw_scalars* sc_dev, float* master, float* exp_avg,
                                float* exp_avg_sq, const float* acc, const void* grad, int32_t grad_dtype,
                                uint16_t* param_bf16, int64_t n, const double* norm_sq_dev, void* hip_stream) {
    int32_t rc = check_scalars(hp, sc_dev, n, norm_sq_dev);
    if (rc != ZS_OK) return rc;
    if (!dtype_ok(grad_dtype)) return ZS_EINVAL;
    if (n == 0) return ZS_OK;
    const int64_t gsz = elem_size(grad_dtype);
    if (master == nullptr || exp_avg == nullptr || exp_avg_sq == nullptr || grad == nullptr) return ZS_EINVAL;
    if (!aligned(master, 4) || !aligned(exp_avg, 4) || !aligned(exp_avg_sq, 4) || !aligned(grad, (uintptr_t)gsz) ||
        (acc != nullptr && !aligned(acc, 4)) || (param_bf16 != nullptr && !aligned(param_bf16, 2)))
        return ZS_EINVAL;
    const void* bufs[6] = {master, exp_avg, exp_avg_sq, acc, grad, param_bf16};
    const int64_t bytes[6] = {n * 4, n * 4, n * 4, acc ? n * 4 : 0, n * gsz, param_bf16 ? n * 2 : 0};
    const bool written[6] = {true, true, true, false, false, true};
    for (int i = 0; i < 6; ++i) {
        for (int j = i + 1; j < 6; ++j)
            if (overlap(bufs[i], bytes[i], bufs[j], bytes[j])) return ZS_EOVERLAP;
        if (norm_sq_dev != nullptr && written[i] && overlap(bufs[i], bytes[i], norm_sq_dev, 8)) return ZS_EOVERLAP;
        if (sc_dev != nullptr && written[i] && overlap(bufs[i], bytes[i], sc_dev, (int64_t)sizeof(zs_adamw_scalars)))
            return ZS_EOVERLAP;
    }
    zs::AdamwArgs a = step_args(hp, sc_dev, norm_sq_dev);
    a.master = master;
    a.exp_avg = exp_avg;
    a.exp_avg_sq = exp_avg_sq;
    a.grad = acc;
    a.grad_mb = grad;
    a.param_bf16 = param_bf16;
    a.n = n;
    const int source = grad_dtype == ZS_F32 ? (acc != nullptr ? zs::kGradSumF32 : zs::kGradF32)
                                            : (acc != nullptr ? zs::kGradSumBf16 : zs::kGradBf16);
    if (source == zs::kGradF32) {   // one fp32 micro-batch: the stored-gradient step on it
        a.grad = static_cast<const float*>(grad);
        a.grad_mb = nullptr;
    }
    auto launch = [&](const zs::AdamwArgs& x, bool vec, bool out_aligned) {
        return source == zs::kGradF32 ? zs::launch_adamw(x, vec, out_aligned, as_stream(hip_stream))
                                      : zs::launch_adamw_sum(x, source, vec, out_aligned, as_stream(hip_stream));
    };
    // as adamw_step: views sharing one offset off a 128-byte boundary run
    // their first 1-31 elements element by element, the rest on the vector
    // path when the state is 16-byte aligned and the gradient's micro-batch
    // part 4-byte aligned
    float* const state[3] = {master, exp_avg, exp_avg_sq};
    const int64_t head = shared_head(state, 3, n);
    if (head > 0) {
        zs::AdamwArgs h = a;
        h.n = head;
        rc = hip_status(launch(h, false, true));
        if (rc != ZS_OK) return rc;
        a.master += head;
        a.exp_avg += head;
        a.exp_avg_sq += head;
        if (a.grad != nullptr) a.grad += head;
        if (a.grad_mb != nullptr) a.grad_mb = static_cast<const char*>(a.grad_mb) + head * gsz;
        if (a.param_bf16 != nullptr) a.param_bf16 += head;
        a.n -= head;
    }
    const bool vec = aligned(a.master, 16) && aligned(a.exp_avg, 16) && aligned(a.exp_avg_sq, 16) &&
                     (a.grad_mb == nullptr || aligned(a.grad_mb, 4));
    const bool out_aligned = a.param_bf16 == nullptr || aligned(a.param_bf16, 16);
    if (a.n == 0) return ZS_OK;
    return hip_status(launch(a, vec, out_aligned));
}

int32_t adamw_step_sum(const zs_adamw* hp, float* master, float* exp_avg, float* exp_avg_sq, const float* acc,
                       const void* grad, int32_t grad_dtype, uint16_t* param_bf16, int64_t n,
                       const double* norm_sq_dev, void* hip_stream) {
    if (hp == nullptr) return ZS_EINVAL;
    return adamw_master_sum(hp, nullptr, master, exp_avg, exp_avg_sq, acc, grad, grad_dtype, param_bf16, n,
                            norm_sq_dev, hip_stream);
}

int32_t adamw_step_sum_dev(const zs_adamw_scalars* scalars_dev, float* master, float* exp_avg, float* exp_avg_sq,
                           const float* acc, const void* grad, int32_t grad_dtype, uint16_t* param_bf16,
                           int64_t n, const double* norm_sq_dev, void* hip_stream) {
    if (scalars_dev == nullptr) return ZS_EINVAL;
    return adamw_master_sum(nullptr, scalars_dev, master, exp_avg, exp_avg_sq, acc, grad, grad_dtype, param_bf16, n,
                            norm_sq_dev, hip_stream);
}

int32_t adamw_step(const zs_adamw* hp, float* master, float* exp_avg, float* exp_avg_sq,
                   const float* grad, uint16_t* param_bf16, int64_t n, const double* norm_sq_dev,
                   void* hip_stream) {
    if (hp == nullptr) return ZS_EINVAL;
    return adamw_master(hp, nullptr, master, exp_avg, exp_avg_sq, grad, param_bf16, n, norm_sq_dev, hip_stream);
}

int32_t adamw_scalars(const zs_adamw* hp, zs_adamw_scalars* out) {
    if (out == nullptr) return ZS_EINVAL;
    const int32_t rc = adamw_check_hp(hp, 0, nullptr);
    if (rc != ZS_OK) return rc;
    const zs::AdamwScalars c = make_scalars(hp);
    std::memcpy(out, &c, sizeof(c));
    return ZS_OK;
}

int32_t adamw_step_dev(const zs_adamw_scalars* scalars_dev, float* master, float* exp_avg, float* exp_avg_sq,
                       const float* grad, uint16_t* param_bf16, int64_t n, const double* norm_sq_dev,
                       void* hip_stream) {
    if (scalars_dev == nullptr) return ZS_EINVAL;
    return adamw_master(nullptr, scalars_dev, master, exp_avg, exp_avg_sq, grad, param_bf16, n, norm_sq_dev,
                        hip_stream);
}

// ---------------------------------------------------------------------------
// tiled optimizer state
// ---------------------------------------------------------------------------

static_assert(ZS_STATE_TILE == zs::kStateTile, "tile length of the header and the kernels");

static int64_t tiled_runs_numel(int64_t n, int runs) {
    if (!size_ok(n)) return -1;
    return runs * ((n + zs::kStateTile - 1) / zs::kStateTile) * zs::kStateTile;
}

int64_t state_tiled_numel(int64_t n) { return tiled_runs_numel(n, 3); }
int64_t moments_tiled_numel(int64_t n) { return tiled_runs_numel(n, 2); }

// split arrays (each nullable: zeros) into a tiled buffer of `runs` runs per tile
static int32_t tile_runs(const float* const* src, int runs, float* buf, int64_t n, void* hip_stream) {
    if (!size_ok(n)) return ZS_EINVAL;
    if (n == 0) return ZS_OK;
    if (buf == nullptr || !aligned(buf, 16)) return ZS_EINVAL;
    const int64_t buf_bytes = tiled_runs_numel(n, runs) * 4;
    for (int k = 0; k < runs; ++k) {
        if (src[k] != nullptr && !aligned(src[k], 4)) return ZS_EINVAL;
        if (overlap(src[k], src[k] ? n * 4 : 0, buf, buf_bytes)) return ZS_EOVERLAP;
    }
    return hip_status(zs::launch_tile_runs(src, runs, buf, n, as_stream(hip_stream)));
}

// a tiled buffer of `runs` runs per tile into split arrays (each nullable: skipped)
static int32_t untile_runs(const float* buf, int runs, float* const* dst, int64_t n, void* hip_stream) {
    if (!size_ok(n)) return ZS_EINVAL;
    if (n == 0) return ZS_OK;
    if (buf == nullptr || !aligned(buf, 16)) return ZS_EINVAL;
    const int64_t buf_bytes = tiled_runs_numel(n, runs) * 4;
    bool vec = true;
    for (int k = 0; k < runs; ++k) {
        if (dst[k] == nullptr) continue;
        if (!aligned(dst[k], 4)) return ZS_EINVAL;
        if (overlap(dst[k], n * 4, buf, buf_bytes)) return ZS_EOVERLAP;
        for (int j = k + 1; j < runs; ++j)
            if (dst[j] != nullptr && overlap(dst[k], n * 4, dst[j], n * 4)) return ZS_EOVERLAP;
        vec = vec && aligned(dst[k], 16);
    }
    return hip_status(zs::launch_untile_runs(buf, runs, dst, n, vec, as_stream(hip_stream)));
}

int32_t state_tile(const float* master, const float* exp_avg, const float* exp_avg_sq, float* state, int64_t n,
                   void* hip_stream) {
    const float* src[3] = {master, exp_avg, exp_avg_sq};
    return tile_runs(src, 3, state, n, hip_stream);
}

int32_t state_untile(const float* state, float* master, float* exp_avg, float* exp_avg_sq, int64_t n,
                     void* hip_stream) {
    float* dst[3] = {master, exp_avg, exp_avg_sq};
    return untile_runs(state, 3, dst, n, hip_stream);
}

int32_t moments_tile(const float* exp_avg, const float* exp_avg_sq, float* moments, int64_t n, void* hip_stream) {
    const float* src[2] = {exp_avg, exp_avg_sq};
    return tile_runs(src, 2, moments, n, hip_stream);
}

int32_t moments_untile(const float* moments, float* exp_avg, float* exp_avg_sq, int64_t n, void* hip_stream) {
    float* dst[2] = {exp_avg, exp_avg_sq};
    return untile_runs(moments, 2, dst, n, hip_stream);
}

// the tiled master-form step: host scalars (hp) or a device copy of them (sc_dev)
static int32_t adamw_tiled(const zs_adamw* hp, const zs_adamw_scalars* sc_dev, float* state, const float* grad,
                           uint16_t* param_bf16, int64_t n, const double* norm_sq_dev, void* hip_stream) {
    int32_t rc = check_scalars(hp, sc_dev, n, norm_sq_dev);
    if (rc != ZS_OK) return rc;
    if (n == 0) return ZS_OK;
    if (state == nullptr || grad == nullptr) return ZS_EINVAL;
    if (!aligned(state, 16) || !aligned(grad, 4) || (param_bf16 != nullptr && !aligned(param_bf16, 2)))
        return ZS_EINVAL;
    const void* bufs[5] = {state, grad, param_bf16, nullptr, nullptr};
    const int64_t bytes[5] = {state_tiled_numel(n) * 4, n * 4, param_bf16 ? n * 2 : 0, 0, 0};
    const bool written[5] = {true, false, true, false, false};
    rc = adamw_check_overlap(bufs, bytes, written, norm_sq_dev);
    if (rc != ZS_OK) return rc;
    if (sc_dev != nullptr)   // the scalars are read while the buffers are written
        for (int i = 0; i < 5; ++i)
            if (written[i] && overlap(bufs[i], bytes[i], sc_dev, (int64_t)sizeof(zs_adamw_scalars)))
                return ZS_EOVERLAP;
    zs::AdamwArgs a = step_args(hp, sc_dev, norm_sq_dev);
    a.state = state;
    a.grad = grad;
    a.param_bf16 = param_bf16;
    a.n = n;
    // the state is 16-byte aligned by contract, so the vector path always
    // applies; a bf16 output off a 16-byte boundary is written element by element
    const bool out_aligned = param_bf16 == nullptr || aligned(param_bf16, 16);
    return hip_status(zs::launch_adamw_tiled(a, out_aligned, as_stream(hip_stream)));
}

int32_t adamw_step_tiled(const zs_adamw* hp, float* state, const float* grad, uint16_t* param_bf16, int64_t n,
                         const double* norm_sq_dev, void* hip_stream) {
    if (hp == nullptr) return ZS_EINVAL;
    return adamw_tiled(hp, nullptr, state, grad, param_bf16, n, norm_sq_dev, hip_stream);
}

int32_t adamw_step_tiled_dev(const zs_adamw_scalars* scalars_dev, float* state, const float* grad,
                             uint16_t* param_bf16, int64_t n, const double* norm_sq_dev, void* hip_stream) {
    if (scalars_dev == nullptr) return ZS_EINVAL;
    return adamw_tiled(nullptr, scalars_dev, state, grad, param_bf16, n, norm_sq_dev, hip_stream);
}

// the tiled step on the last micro-batch's sum: host scalars (hp) or a device copy (sc_dev)
static int32_t adamw_tiled_sum(const zs_adamw* hp, const zs_adamw_scalars* sc_dev, float* state, const float* acc,
                               const void* grad, int32_t grad_dtype, uint16_t* param_bf16, int64_t n,
                               const double* norm_sq_dev, void* hip_stream) {
    int32_t rc = check_scalars(hp, sc_dev, n, norm_sq_dev);
    if (rc != ZS_OK) return rc;
    if (!dtype_ok(grad_dtype)) return ZS_EINVAL;
    if (n == 0) return ZS_OK;
    const int64_t gsz = elem_size(grad_dtype);
    if (state == nullptr || grad == nullptr) return ZS_EINVAL;
    if (!aligned(state, 16) || !aligned(grad, (uintptr_t)gsz) || (acc != nullptr && !aligned(acc, 4)) ||
        (param_bf16 != nullptr && !aligned(param_bf16, 2)))
        return ZS_EINVAL;
    const void* bufs[5] = {state, acc, grad, param_bf16, nullptr};
    const int64_t bytes[5] = {state_tiled_numel(n) * 4, acc ? n * 4 : 0, n * gsz, param_bf16 ? n * 2 : 0, 0};
    const bool written[5] = {true, false, false, true, false};
    rc = adamw_check_overlap(bufs, bytes, written, norm_sq_dev);
    if (rc != ZS_OK) return rc;
    if (sc_dev != nullptr)   // the scalars are read while the buffers are written
        for (int i = 0; i < 5; ++i)
            if (written[i] && overlap(bufs[i], bytes[i], sc_dev, (int64_t)sizeof(zs_adamw_scalars)))
                return ZS_EOVERLAP;
    zs::AdamwArgs a = step_args(hp, sc_dev, norm_sq_dev);
    a.state = state;
    a.grad = acc;
    a.grad_mb = grad;
    a.param_bf16 = param_bf16;
    a.n = n;
    const int source = grad_dtype == ZS_F32 ? (acc != nullptr ? zs::kGradSumF32 : zs::kGradF32)
                                            : (acc != nullptr ? zs::kGradSumBf16 : zs::kGradBf16);
    const bool out_aligned = param_bf16 == nullptr || aligned(param_bf16, 16);
    if (source == zs::kGradF32) {   // one fp32 micro-batch: the plain tiled step on it
        a.grad = static_cast<const float*>(grad);
        a.grad_mb = nullptr;
        return hip_status(zs::launch_adamw_tiled(a, out_aligned, as_stream(hip_stream)));
    }
    return hip_status(zs::launch_adamw_tiled_sum(a, source, aligned(grad, 4), out_aligned, as_stream(hip_stream)));
}

int32_t adamw_step_tiled_sum(const zs_adamw* hp, float* state, const float* acc, const void* grad,
                             int32_t grad_dtype, uint16_t* param_bf16, int64_t n, const double* norm_sq_dev,
                             void* hip_stream) {
    if (hp == nullptr) return ZS_EINVAL;
    return adamw_tiled_sum(hp, nullptr, state, acc, grad, grad_dtype, param_bf16, n, norm_sq_dev, hip_stream);
}

int32_t adamw_step_tiled_sum_dev(const zs_adamw_scalars* scalars_dev, float* state, const float* acc,
                                 const void* grad, int32_t grad_dtype, uint16_t* param_bf16, int64_t n,
                                 const double* norm_sq_dev, void* hip_stream) {
    if (scalars_dev == nullptr) return ZS_EINVAL;
    return adamw_tiled_sum(nullptr, scalars_dev, state, acc, grad, grad_dtype, param_bf16, n, norm_sq_dev,
                           hip_stream);
}

int32_t adam_update_tiled(const zs_adamw* hp, float* moments, const float* grad, float* update, int64_t n,
                          const double* norm_sq_dev, void* hip_stream) {
    int32_t rc = adamw_check_hp(hp, n, norm_sq_dev);
    if (rc != ZS_OK) return rc;
    if (hp->weight_decay != 0.0) return ZS_EINVAL;
    if (n == 0) return ZS_OK;
    if (moments == nullptr || grad == nullptr || update == nullptr) return ZS_EINVAL;
    if (!aligned(moments, 16) || !aligned(grad, 4) || !aligned(update, 4)) return ZS_EINVAL;
    const void* bufs[5] = {moments, grad, update, nullptr, nullptr};
    const int64_t bytes[5] = {moments_tiled_numel(n) * 4, n * 4, n * 4, 0, 0};
    const bool written[5] = {true, false, true, false, false};
    rc = adamw_check_overlap(bufs, bytes, written, norm_sq_dev);
    if (rc != ZS_OK) return rc;
    zs::AdamwArgs a = make_args(hp, norm_sq_dev);
    a.state = moments;
    a.grad = grad;
    a.update = update;
    a.n = n;
    // the moments are 16-byte aligned by contract; the update may sit at any element offset
    return hip_status(zs::launch_adam_update_tiled(a, aligned(update, 16), as_stream(hip_stream)));
}

int32_t adamw_step_no_master_tiled(const zs_adamw* hp, uint16_t* param_bf16, float* moments, const float* grad,
                                   int64_t n, const double* norm_sq_dev, void* hip_stream) {
    int32_t rc = adamw_check_hp(hp, n, norm_sq_dev);
    if (rc != ZS_OK) return rc;
    if (n == 0) return ZS_OK;
    if (param_bf16 == nullptr || moments == nullptr || grad == nullptr) return ZS_EINVAL;
    if (!aligned(param_bf16, 2) || !aligned(moments, 16) || !aligned(grad, 4)) return ZS_EINVAL;
    const void* bufs[5] = {param_bf16, moments, grad, nullptr, nullptr};
    const int64_t bytes[5] = {n * 2, moments_tiled_numel(n) * 4, n * 4, 0, 0};
    const bool written[5] = {true, true, false, false, false};
    rc = adamw_check_overlap(bufs, bytes, written, norm_sq_dev);
    if (rc != ZS_OK) return rc;
    zs::AdamwArgs a = make_args(hp, norm_sq_dev);
    a.state = moments;
    a.grad = grad;
    a.param_bf16 = param_bf16;
    a.n = n;
    // the bf16 parameter is read and written: the vector path needs it 16-byte aligned
    return hip_status(zs::launch_adamw_no_master_tiled(a, aligned(param_bf16, 16), as_stream(hip_stream)));
}

int32_t adamw_step_no_master(const zs_adamw* hp, uint16_t* param_bf16, float* exp_avg, float* exp_avg_sq,
                             const float* grad, int64_t n, const double* norm_sq_dev, void* hip_stream) {
    int32_t rc = adamw_check_hp(hp, n, norm_sq_dev);
    if (rc != ZS_OK) return rc;
    if (n == 0) return ZS_OK;
    if (param_bf16 == nullptr || exp_avg == nullptr || exp_avg_sq == nullptr || grad == nullptr)
        return ZS_EINVAL;
    if (!aligned(param_bf16, 2) || !aligned(exp_avg, 4) || !aligned(exp_avg_sq, 4) || !aligned(grad, 4))
        return ZS_EINVAL;
    const void* bufs[5] = {param_bf16, exp_avg, exp_avg_sq, grad, nullptr};
    const int64_t bytes[5] = {n * 2, n * 4, n * 4, n * 4, 0};
    const bool written[5] = {true, true, true, false, false};
    rc = adamw_check_overlap(bufs, bytes, written, norm_sq_dev);
    if (rc != ZS_OK) return rc;
    zs::AdamwArgs a = make_args(hp, norm_sq_dev);
    a.exp_avg = exp_avg;
    a.exp_avg_sq = exp_avg_sq;
    a.grad = grad;
    a.param_bf16 = param_bf16;
    a.n = n;
    const bool vec = aligned(param_bf16, 16) && aligned(exp_avg, 16) && aligned(exp_avg_sq, 16);
    return hip_status(zs::launch_adamw_no_master(a, vec, as_stream(hip_stream)));
}

int32_t adam_update(const zs_adamw* hp, float* exp_avg, float* exp_avg_sq, const float* grad, float* update,
                    int64_t n, const double* norm_sq_dev, void* hip_stream) {
    int32_t rc = adamw_check_hp(hp, n, norm_sq_dev);
    if (rc != ZS_OK) return rc;
    if (hp->weight_decay != 0.0) return ZS_EINVAL;
    if (n == 0) return ZS_OK;
    if (exp_avg == nullptr || exp_avg_sq == nullptr || grad == nullptr || update == nullptr) return ZS_EINVAL;
    if (!aligned(exp_avg, 4) || !aligned(exp_avg_sq, 4) || !aligned(grad, 4) || !aligned(update, 4))
        return ZS_EINVAL;
    const void* bufs[5] = {update, exp_avg, exp_avg_sq, grad, nullptr};
    const int64_t bytes[5] = {n * 4, n * 4, n * 4, n * 4, 0};
    const bool written[5] = {true, true, true, false, false};
    rc = adamw_check_overlap(bufs, bytes, written, norm_sq_dev);
    if (rc != ZS_OK) return rc;
    zs::AdamwArgs a = make_args(hp, norm_sq_dev);
    a.exp_avg = exp_avg;
    a.exp_avg_sq = exp_avg_sq;
    a.grad = grad;
    a.update = update;
    a.n = n;
    // the moments 16-byte aligned; the write-only update may sit at any element
    // offset (a rank's chunk of the gathered buffer).  Moments sharing one
    // offset off a 128-byte boundary run their first 1-31 elements element by
    // element and the rest on the vector path.
    float* const moments[2] = {exp_avg, exp_avg_sq};
    const int64_t head = shared_head(moments, 2, n);
    if (head > 0) {
        zs::AdamwArgs h = a;
        h.n = head;
        rc = hip_status(zs::launch_adam_update(h, false, true, as_stream(hip_stream)));
        if (rc != ZS_OK) return rc;
        a.exp_avg += head;
        a.exp_avg_sq += head;
        a.grad += head;
        a.update += head;
        a.n -= head;
    }
    const bool vec = aligned(a.exp_avg, 16) && aligned(a.exp_avg_sq, 16);
    const bool out_aligned = aligned(a.update, 16);
    if (a.n == 0) return ZS_OK;
    return hip_status(zs::launch_adam_update(a, vec, out_aligned, as_stream(hip_stream)));
}

// ---------------------------------------------------------------------------
// flatten / unflatten / apply
// ---------------------------------------------------------------------------

// apply: the tensors take += of the (fp32) flat buffer instead of a copy
static int32_t flat_common(const zs_tensor* tensors, int32_t count, void* flat, int32_t flat_dtype,
                           int32_t tensor_dtype, int64_t padded_total, bool unpack,
                           hipStream_t stream, bool apply = false) {
    if (count < 0 || (count > 0 && tensors == nullptr)) return ZS_EINVAL;
    if (!dtype_ok(flat_dtype) || !dtype_ok(tensor_dtype)) return ZS_EINVAL;
    int kind;
    if (apply) {
        if (!unpack || flat_dtype != ZS_F32) return ZS_EINVAL;
        kind = tensor_dtype == ZS_F32 ? 4 : 5;
    } else if (flat_dtype == tensor_dtype) kind = flat_dtype == ZS_F32 ? 0 : 1;
    else if (!unpack && tensor_dtype == ZS_BF16 && flat_dtype == ZS_F32) kind = 2;
    else if (unpack && flat_dtype == ZS_F32 && tensor_dtype == ZS_BF16) kind = 3;
    else return ZS_EINVAL;
    const int64_t fsz = elem_size(flat_dtype), tsz = elem_size(tensor_dtype);
    int64_t total = 0;
    for (int32_t i = 0; i < count; ++i) {
        const int64_t k = tensors[i].numel;
        if (!size_ok(k) || total > kMaxElems - k) return ZS_EINVAL;
        if (k > 0 && (tensors[i].ptr == nullptr || !aligned(tensors[i].ptr, (uintptr_t)tsz)))
            return ZS_EINVAL;
        total += k;
    }
    if (unpack) padded_total = total;
    if (!size_ok(padded_total) || total > padded_total) return ZS_EINVAL;
    if (padded_total == 0) return ZS_OK;
    if (flat == nullptr || !aligned(flat, (uintptr_t)fsz)) return ZS_EINVAL;
    for (int32_t i = 0; i < count; ++i) {
        const int64_t bi = tensors[i].numel * tsz;
        if (overlap(tensors[i].ptr, bi, flat, padded_total * fsz)) return ZS_EOVERLAP;
        if (unpack)   // written tensors must be pairwise disjoint
            for (int32_t j = i + 1; j < count; ++j)
                if (overlap(tensors[i].ptr, bi, tensors[j].ptr, tensors[j].numel * tsz))
                    return ZS_EOVERLAP;
    }

    // batches of up to kFlatMaxTensors entries and fewer than 2^32
    // work-items; a tensor longer than kLaunchElems takes one entry per
    // kLaunchElems elements (a multiple of every tile: each piece keeps the
    // tensor's alignment); the pack padding is one more entry with a NULL
    // tensor
    const int64_t tile = zs::flat_tile_elems(kind);
    const int64_t max_tiles = zs::flat_max_batch_tiles(kind);
    const int64_t tsz_bytes = tsz;
    zs::FlatBatch b;
    std::memset(&b, 0, sizeof(b));
    b.flat = flat;
    int64_t offset = 0;
    auto flush = [&]() -> int32_t {
        if (b.count == 0) return ZS_OK;
        const int32_t rc = hip_status(zs::launch_flat(b, kind, unpack ? 1 : 0, stream));
        std::memset(&b, 0, sizeof(b));
        b.flat = flat;
        return rc;
    };
    auto add_piece = [&](void* ptr, int64_t flat_off, int64_t numel) -> int32_t {
        const int64_t tiles = (numel + tile - 1) / tile;   // numel <= kLaunchElems: tiles << max_tiles
        if (b.count == zs::kFlatMaxTensors || (int64_t)b.tile_start[b.count] + tiles > max_tiles) {
            const int32_t rc = flush();
            if (rc != ZS_OK) return rc;
        }
        const int c = b.count;
        b.e[c].tensor = ptr;
        b.e[c].flat_off = flat_off;
        b.e[c].numel = numel;
        // the vector path writes 16-byte aligned vectors and reads dword-aligned ones
        const void* flat_at = static_cast<const char*>(flat) + flat_off * fsz;
        const void* written = unpack ? ptr : flat_at;
        const void* read = unpack ? flat_at : ptr;   // NULL: the zero fill reads nothing
        b.e[c].vec_ok = aligned(written, 16) && (read == nullptr || aligned(read, 4));
        b.tile_start[c + 1] = b.tile_start[c] + (uint32_t)tiles;
        b.count = c + 1;
        return ZS_OK;
    };
    auto add = [&](void* ptr, int64_t flat_off, int64_t numel) -> int32_t {
        for (int64_t off = 0; off < numel; off += zs::kLaunchElems) {
            void* piece = ptr == nullptr ? nullptr : static_cast<char*>(ptr) + off * tsz_bytes;
            const int32_t rc = add_piece(piece, flat_off + off, zs::launch_piece(numel, off));
            if (rc != ZS_OK) return rc;
        }
        return ZS_OK;
    };
    for (int32_t i = 0; i < count; ++i) {
        const int64_t k = tensors[i].numel;
        if (k > 0) {
            const int32_t rc = add(tensors[i].ptr, offset, k);
            if (rc != ZS_OK) return rc;
        }
        offset += k;
    }
    if (!unpack && padded_total > total) {
        const int32_t rc = add(nullptr, total, padded_total - total);
        if (rc != ZS_OK) return rc;
    }
    return flush();
}

int32_t flat_pack(const zs_tensor* src, int32_t count, int32_t src_dtype, void* flat,
                  int32_t flat_dtype, int64_t padded_total, void* hip_stream) {
    return flat_common(src, count, flat, flat_dtype, src_dtype, padded_total, false,
                       as_stream(hip_stream));
}

int32_t flat_unpack(const void* flat, int32_t flat_dtype, const zs_tensor* dst, int32_t count,
                    int32_t dst_dtype, void* hip_stream) {
    return flat_common(dst, count, const_cast<void*>(flat), flat_dtype, dst_dtype, 0, true,
                       as_stream(hip_stream));
}

int32_t flat_apply_update(const float* update, const zs_tensor* dst, int32_t count, int32_t dst_dtype,
                          void* hip_stream) {
    return flat_common(dst, count, const_cast<float*>(update), ZS_F32, dst_dtype, 0, true,
                       as_stream(hip_stream), true);
}

}  // extern "C"
