// Internal declarations shared by the libzshard sources (not installed).
//
// Device helpers for gfx950 (wave64, 128-bit global accesses) and the
// launchers each kernel file provides to the C-ABI layer in api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace zs {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 256;   // threads per workgroup: 4 wave64s

// --- bf16 <-> fp32 ---------------------------------------------------------
// Widening is exact: the bf16 pattern is the upper half of the fp32 one.
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round to nearest, ties to even, by adding 0x7FFF plus the lowest kept bit
// and truncating; the carry walks into the exponent (and to +-inf) as IEEE
// rounding does.  Every NaN becomes the quiet NaN 0x7FC0.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
    uint32_t u = __float_as_uint(x);
    uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    return ((u & 0x7FFFFFFFu) > 0x7F800000u) ? 0x7FC0u : r;
}

// Two bf16 patterns in one 32-bit word, element 0 in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// --- streaming loads / stores ---------------------------------------------
// Every byte of the streamed buffers is touched exactly once per call, so
// the accesses carry the non-temporal hint (no reuse to keep in L2/MALL).
template <typename T>
__device__ __forceinline__ T ld_stream(const T* p) { return __builtin_nontemporal_load(p); }
template <typename T>
__device__ __forceinline__ void st_stream(T* p, T v) { __builtin_nontemporal_store(v, p); }

// Read-only streams need only dword (4-byte) alignment on the vector path:
// gfx950 serves a dword-aligned 128- or 64-bit global load at full speed (an
// AdamW gradient 4 bytes off a 16-byte boundary streams at 80.3 % of the HBM
// peak against 80.6 % aligned), while a misaligned written stream drops the
// kernel to 61 %, so written streams stay 16-byte aligned.  The _a4 types
// tell the compiler the weaker alignment of such a load.
typedef float f32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x2_a4 __attribute__((ext_vector_type(2), aligned(4)));
__device__ __forceinline__ f32x4 ld_stream_f32x4_a4(const void* p) {
    return __builtin_nontemporal_load(static_cast<const f32x4_a4*>(p));
}
__device__ __forceinline__ u32x4 ld_stream_u32x4_a4(const void* p) {
    return __builtin_nontemporal_load(static_cast<const u32x4_a4*>(p));
}
__device__ __forceinline__ u32x2 ld_stream_u32x2_a4(const void* p) {
    return __builtin_nontemporal_load(static_cast<const u32x2_a4*>(p));
}

// --- scalars of one AdamW step, formed on the host ------------------------
// Binary64 on the host, each rounded to binary32 once; the same layout as
// zs_adamw_scalars in zshard.h (checked in api.hip).
struct AdamwScalars {
    float beta1, beta2;
    float one_minus_beta1, one_minus_beta2;
    float step_size;            // (float)(lr / bias_correction1)
    float bias_correction2_sqrt;// (float)sqrt(bias_correction2)
    float eps;
    float decay;                // (float)(1 - lr*wd)
    float grad_scale;           // (float)grad_scale
    int32_t clip;               // max_norm > 0
    double max_norm;
    double extra_norm_sq;
};

// --- tiled optimizer state ------------------------------------------------
// R fp32 arrays of a shard in one buffer: for each tile of kStateTile
// elements, a run of kStateTile floats of each array, one after the other
// (the last tile keeps full-length runs; its unused ends are padding).  The
// state of the master forms has R = 3 runs (master, exp_avg, exp_avg_sq), the
// moments of the no-master and update forms R = 2 (exp_avg, exp_avg_sq).
// Element i's first value sits at tiled_offset<R>(i), its k-th k*kStateTile
// floats later.  kStateTile equals ZS_STATE_TILE in zshard.h (checked in
// api.hip).
constexpr int64_t kStateTile = 8192;
template <int R = 3>
__host__ __device__ __forceinline__ int64_t tiled_offset(int64_t i) {
    const uint64_t u = (uint64_t)i;
    return (int64_t)((u / kStateTile) * (R * kStateTile) + (u % kStateTile));
}

struct AdamwArgs {
    AdamwScalars sc;            // in the kernel arguments, unless sc_dev is set
    const AdamwScalars* sc_dev; // device copy of the scalars (a step replayable from a graph), nullable
    const double* norm_sq;      // device, nullable
    float* state;               // tiled forms: master, exp_avg, exp_avg_sq (or the moments alone) tiled
    float* master;
    float* exp_avg;
    float* exp_avg_sq;
    const float* grad;          // the fp32 gradient; the fp32 accumulator for the summed-gradient forms
    const void* grad_mb;        // summed-gradient forms: the last micro-batch's gradient (bf16 or fp32)
    uint16_t* param_bf16;       // nullable
    float* update;              // the ZeRO-1 form's output
    int64_t n;
};

// One launch covers at most kLaunchElems elements.  A HIP launch must keep
// gridDim.x * blockDim.x below 2^32 work-items, and the scalar AdamW path
// runs one element per work-item (2^31 of them at most, then), so a longer
// call is split into launches
// at multiples of kLaunchElems: a multiple of every tile, workgroup partial
// and vector width, so the pieces keep the tiles, partial indices (results
// bit-identical to one launch) and 16-byte alignment of a single launch.
constexpr int64_t kLaunchElems = int64_t(1) << 31;
inline int64_t launch_piece(int64_t n, int64_t off) { return n - off < kLaunchElems ? n - off : kLaunchElems; }

// Where workgroup b of a launch of nb workgroups writes its binary64 norm
// partial.  gfx950 deals a launch's workgroups to its 8 XCDs round-robin
// (workgroup b on XCD b mod 8), and each XCD has its own L2.  Partials
// written in workgroup order put the 16 of a 128-byte line on 8 different
// XCDs, and every L2 writes its two 8-byte values back as its own partly
// filled 32-byte sector: the HBM write counter reads 4x the partials' bytes,
// and the stream of small write-backs costs the standalone norm 5 points of
// its bandwidth (86.7 % of the peak against 91.4 %).  Here the workgroups of
// one XCD write one contiguous run of slots instead (XCD x's workgroups
// x, x+8, x+16, ... fill the run after XCD 0..x-1's), so lines are written
// whole and the partials cost their 8 bytes each.  A bijection of [0, nb)
// onto itself; the norm's association is still fixed by n alone.
__host__ __device__ constexpr int64_t xcd_slot(int64_t b, int64_t nb) {
    const int64_t x = b & 7, j = b >> 3, q = nb >> 3, r = nb & 7;
    return x * q + (x < r ? x : r) + j;
}

// The block a wave runs when one launch's waves each take K of the blocks a
// grid of one-wave workgroups would have run, and the workgroups W waves
// each: the k-th block of wave w of workgroup B is one its XCD (B mod 8)
// would have run, 8j + B mod 8 for K consecutive j, so what the wave writes
// per block at xcd_slot stays in that XCD's run of slots.  A grid of
// 8 * ceil(ceil(nb / 8) / (W * K)) workgroups covers every block of [0, nb)
// once (the blocks at or past nb are skipped).
__host__ __device__ constexpr int64_t xcd_block(int64_t B, int64_t w, int64_t k, int64_t W, int64_t K) {
    return 8 * (((B >> 3) * W + w) * K + k) + (B & 7);
}
__host__ __device__ constexpr int64_t sum_norm_grid(int64_t nb, int64_t W, int64_t K) {
    return 8 * (((nb + 7) / 8 + W * K - 1) / (W * K));
}

// Launchers: enqueue on `stream`, return the hipError_t of the (first failed) launch.
// vec_ok: every stream but the write-only output (bf16 re-cast, ZeRO-1
// update) allows the 128-bit path; out_aligned: that output is 16-byte
// aligned as well (else it is written element by element on the same path).
hipError_t launch_adamw(const AdamwArgs& a, bool vec_ok, bool out_aligned, hipStream_t stream);
hipError_t launch_adamw_no_master(const AdamwArgs& a, bool vec_ok, hipStream_t stream);
hipError_t launch_adam_update(const AdamwArgs& a, bool vec_ok, bool out_aligned, hipStream_t stream);
hipError_t launch_adamw_tiled(const AdamwArgs& a, bool out_aligned, hipStream_t stream);
hipError_t launch_adam_update_tiled(const AdamwArgs& a, bool out_aligned, hipStream_t stream);
hipError_t launch_adamw_no_master_tiled(const AdamwArgs& a, bool vec_ok, hipStream_t stream);
// The master-form step whose gradient is the last micro-batch's sum,
// formed as it is read: grad_source 1 = widen(bf16 grad_mb) (no accumulator),
// 2 = fl(grad + widen(bf16 grad_mb)), 3 = fl(grad + fp32 grad_mb).  vec_ok:
// grad_mb is 4-byte aligned (else the element-wise path).
enum GradSource : int { kGradF32 = 0, kGradBf16 = 1, kGradSumBf16 = 2, kGradSumF32 = 3 };
hipError_t launch_adamw_tiled_sum(const AdamwArgs& a, int grad_source, bool vec_ok, bool out_aligned,
                                  hipStream_t stream);
// the same on split master, exp_avg and exp_avg_sq (vec_ok: the state 16-byte
// aligned and grad_mb 4-byte aligned)
hipError_t launch_adamw_sum(const AdamwArgs& a, int grad_source, bool vec_ok, bool out_aligned,
                            hipStream_t stream);
// runs (2 or 3) split fp32 arrays (each nullable: zeros) -> tiled buffer,
// padding zeroed; and back (each destination nullable: skipped)
hipError_t launch_tile_runs(const float* const* src, int runs, float* buf, int64_t n, hipStream_t stream);
hipError_t launch_untile_runs(const float* buf, int runs, float* const* dst, int64_t n, bool vec_ok,
                              hipStream_t stream);
hipError_t launch_grad_accum(float* acc, const void* grad, int grad_bf16, int64_t n,
                             int overwrite, bool vec_ok, hipStream_t stream);
int64_t norm_partials(int64_t n);   // grad_norm_sq's stage-1 partials for n elements
int64_t accum_norm_partials(int64_t n);
hipError_t launch_grad_accum_norm_sq(float* acc, const void* grad, int grad_bf16, int64_t n, int overwrite,
                                     float scale, double* out, double* workspace, bool vec_ok,
                                     hipStream_t stream);
hipError_t launch_grad_norm_sq(const float* grad, int64_t n, float scale, double* out,
                               double* workspace, hipStream_t stream);
// launch_grad_accum_norm_sq's norm, bit for bit, without its store (acc is
// read, not written; not read when overwrite is set)
hipError_t launch_grad_sum_norm_sq(const float* acc, const void* grad, int grad_bf16, int64_t n, int overwrite,
                                   float scale, double* out, double* workspace, bool vec_ok,
                                   hipStream_t stream);

// Up to kReduceMaxChunks rank chunks summed per launch (pointers travel in
// the kernel arguments).
constexpr int kReduceMaxChunks = 16;
struct ChunkBatch {
    const void* chunk[kReduceMaxChunks];
    int32_t count;
};
hipError_t launch_reduce_chunks(float* acc, const ChunkBatch& b, int grad_bf16, int64_t n, int overwrite,
                                bool vec_ok, hipStream_t stream);
// the same pass also forming the squared norm (partials, then their sum)
int64_t reduce_norm_partials(int64_t n);
hipError_t launch_reduce_chunks_norm_sq(float* acc, const ChunkBatch& b, int grad_bf16, int64_t n, int overwrite,
                                        bool vec_ok, float scale, double* out, double* workspace,
                                        hipStream_t stream);

// One launch of the flatten/unflatten copy covers up to kFlatMaxTensors
// tensors (the table travels in the kernel arguments; no device allocation).
// The workgroup table is 32-bit so a workgroup finds its tensor from two
// scalar loads; each tensor's record is then one more 32-byte load.
constexpr int kFlatMaxTensors = 32;
struct FlatEntry {
    void* tensor;        // src (pack) / dst (unpack); NULL = zero fill
    int64_t flat_off;    // element offset of the tensor in the flat buffer
    int64_t numel;
    int32_t vec_ok;      // vector path allowed for this tensor
    int32_t pad_;
};
struct FlatBatch {
    uint32_t tile_start[kFlatMaxTensors + 1];   // first workgroup of each tensor; [count] = total
    int32_t count;                             // tensors in this batch (incl. a zero-fill entry)
    void* flat;
    FlatEntry e[kFlatMaxTensors];
};
// kind: 0 = f32->f32, 1 = bf16->bf16, 2 = bf16->f32 (pack widen), 3 = f32->bf16 (unpack RNE),
// 4 = f32 tensor += f32 flat, 5 = bf16 tensor = RNE(widen(tensor) + f32 flat) (apply, unpack side)
hipError_t launch_flat(const FlatBatch& b, int kind, int unpack, hipStream_t stream);
int64_t flat_tile_elems(int kind);        // elements per workgroup
int64_t flat_max_batch_tiles(int kind);   // workgroups one launch may hold (< 2^32 work-items)

}  // namespace zs
