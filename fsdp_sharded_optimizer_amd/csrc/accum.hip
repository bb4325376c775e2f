// fp32 gradient accumulation over micro-batches: acc = widen(g) for the
// first micro-batch, acc = fl(acc + widen(g)) after it; optionally fused
// with this shard's squared norm of the scaled result (the last micro-batch).
//
// HBM-bound streaming: bf16 gradients move 6 B/element on the first
// micro-batch (read 2, write 4) and 10 B/element after it (read 2 + 4,
// write 4); fp32 gradients move 8 and 12.  The fused norm adds no traffic
// beyond one binary64 partial per workgroup.
//
// Layout: lane-contiguous groups of 4 elements (a 64-bit bf16 or 128-bit
// fp32 load and a 128-bit fp32 access per lane).  A workgroup of BS threads
// covers Q groups per lane, the q-th at offset q*BS*4 in its tile, every
// load of the tile issued before the first store.  The plain forms and the
// accumulating fused form run Q = 1 in one-wave workgroups: the fastest
// shape on gfx950 (84 % of peak for the accumulating form, 85 % for the
// overwriting one, 84.5 % with the norm partials, against 82 %, 83 % and
// 79.8 % in 256-thread workgroups with the best Q and residency cap), the
// plain accumulating form with residency capped by reserved LDS (kAddLds*,
// 86 % on contiguous buffers), the others uncapped; the overwriting fused
// form runs Q = 4 (see launch_grad_accum_norm_sq).
//
// Fused norm association (fixed by n, the overwrite flag and the gradient
// dtype): each lane adds the squares of its Q groups of 4 elements, 0 and 2
// into one running sum, 1 and 3 into the other; the 64 lanes combine in a
// fixed butterfly into one binary64 partial per 256*Q elements, stored at
// the workgroup's XCD-contiguous slot (xcd_slot: each partial written once,
// as a whole line with its neighbours); the partials are reduced in fixed
// contiguous chunks of slots (at most kReduceChunks), then by one workgroup.
// Two groups per lane (one partial per 512 elements) measured 79 % against
// 85 % for one; four with residency capped, 82 %.
#include "reduce.h"

namespace zs {
namespace {

template <bool BF16>
__device__ __forceinline__ f32x4 load4(const void* grad, int64_t i) {
    if (BF16) {   // read-only: dword alignment suffices
        const u32x2 w = ld_stream_u32x2_a4(static_cast<const uint16_t*>(grad) + i);
        return f32x4{bf16_to_f32(w.x & 0xFFFFu), bf16_to_f32(w.x >> 16),
                     bf16_to_f32(w.y & 0xFFFFu), bf16_to_f32(w.y >> 16)};
    }
    return ld_stream_f32x4_a4(static_cast<const float*>(grad) + i);
}

template <bool BF16>
__device__ __forceinline__ float load1(const void* grad, int64_t i) {
    if (BF16) return bf16_to_f32(static_cast<const uint16_t*>(grad)[i]);
    return static_cast<const float*>(grad)[i];
}

template <int Q, int BS, bool VEC, bool BF16, bool OVERWRITE, bool NORM>
__global__ __launch_bounds__(BS) void accum_kernel(float* __restrict__ acc, const void* __restrict__ grad,
                                                   int64_t n, float scale, double* __restrict__ partials) {
    static_assert(!NORM || BS == 64, "the fused norm's partial is one wave's butterfly");
    constexpr int64_t kGroup = BS * 4;
    const int64_t tile = (int64_t)blockIdx.x * kGroup * Q;
    const int64_t lane0 = tile + threadIdx.x * 4;
    double s0 = 0.0, s1 = 0.0;
    if (VEC && tile + kGroup * Q <= n) {   // whole tile in range
        f32x4 g[Q], a[Q];
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            g[q] = load4<BF16>(grad, lane0 + q * kGroup);
            if (!OVERWRITE) a[q] = ld_stream(reinterpret_cast<const f32x4*>(acc + lane0 + q * kGroup));
        }
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const f32x4 r = OVERWRITE ? g[q]
                                      : f32x4{a[q].x + g[q].x, a[q].y + g[q].y, a[q].z + g[q].z,
                                              a[q].w + g[q].w};
            st_stream(reinterpret_cast<f32x4*>(acc + lane0 + q * kGroup), r);
            if (NORM) {
                const float rv[4] = {r.x, r.y, r.z, r.w};
                add_squares4(rv, scale, s0, s1);
            }
        }
    } else {
        // ragged tile (or a misaligned buffer): element by element, the same
        // association for the norm (out-of-range elements add +0)
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int64_t first = lane0 + q * kGroup;
            float rv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t i = first + j;
                if (i < n) {
                    const float g = load1<BF16>(grad, i);
                    const float r = OVERWRITE ? g : acc[i] + g;
                    acc[i] = r;
                    rv[j] = r;
                }
            }
            if (NORM) add_squares4(rv, scale, s0, s1);
        }
    }
    if (NORM) {
        const double total = wave_sum(s0 + s1);
        if (threadIdx.x == 0) partials[xcd_slot(blockIdx.x, gridDim.x)] = total;
    }
}

constexpr int kAccumBlock = 64;   // one wave per workgroup

template <int Q>
constexpr int64_t per_block() { return (int64_t)kAccumBlock * 4 * Q; }

// The fused forms run Q = 1 uncapped (84.5 % of the HBM peak accumulating a
// bf16 gradient, 83.5 % overwriting with an fp32 one), except the overwriting
// form with a bf16 gradient: it moves only 6 B per element, so its waves are
// short and the norm's tail weighs more, and Q = 4 (1024 elements and one
// partial per workgroup) with residency capped at 13 workgroups per CU
// measured 82.7 % on gfx950 against 76-78 % for Q = 1 (for an fp32 gradient
// that shape gives 80 %).
constexpr int kFusedQAdd = 1;
// The plain accumulating form caps residency with reserved LDS: 6 KiB per
// one-wave workgroup (26 per CU) for a bf16 gradient, 7 KiB (22) for an fp32
// one.  On buffers carved from one physically contiguous block they measured
// 86.2-86.3 % and 85.7-85.9 % of the peak against 84.2-84.3 % and 84.6-84.8 %
// uncapped (bf16 at 7 / 8 KiB: 86.6 / 85.1-85.5 %); on an ordinary
// allocation 84.1-84.2 % and 84.0-84.2 % against 83.9-84.0 % and 84.1 %.
// The overwriting and fused forms run uncapped (a cap measured no better).
constexpr unsigned kAddLdsBf16 = 6144;
constexpr unsigned kAddLdsF32 = 7168;
constexpr int kFusedQOverwrite = 4;
constexpr unsigned kFusedOverwriteLds = 12288;

static_assert(kLaunchElems % per_block<kFusedQOverwrite>() == 0, "pieces keep the partials' positions");

// one launch per kLaunchElems elements; piece k's partials follow piece
// k-1's, so the partials (and the norm) are those of a single launch
template <int Q, bool VEC, bool BF16, bool OVERWRITE, bool NORM>
hipError_t launch(float* acc, const void* grad, int64_t n, float scale, double* partials, unsigned lds,
                  hipStream_t stream) {
    const int64_t gsz = BF16 ? 2 : 4;
    for (int64_t off = 0; off < n; off += kLaunchElems) {
        const int64_t m = launch_piece(n, off);
        const int64_t blocks = (m + per_block<Q>() - 1) / per_block<Q>();
        hipLaunchKernelGGL((accum_kernel<Q, kAccumBlock, VEC, BF16, OVERWRITE, NORM>), dim3((unsigned)blocks),
                           dim3(kAccumBlock), lds, stream, acc + off,
                           static_cast<const char*>(grad) + off * gsz, m, scale,
                           NORM ? partials + off / per_block<Q>() : nullptr);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int Q, bool NORM, bool OVERWRITE>
hipError_t dispatch(float* acc, const void* grad, int grad_bf16, int64_t n, bool vec, float scale,
                    double* partials, unsigned lds, hipStream_t stream) {
    if (vec)
        return grad_bf16 ? launch<Q, true, true, OVERWRITE, NORM>(acc, grad, n, scale, partials, lds, stream)
                         : launch<Q, true, false, OVERWRITE, NORM>(acc, grad, n, scale, partials, lds, stream);
    return grad_bf16 ? launch<Q, false, true, OVERWRITE, NORM>(acc, grad, n, scale, partials, 0, stream)
                     : launch<Q, false, false, OVERWRITE, NORM>(acc, grad, n, scale, partials, 0, stream);
}

// The squared norm of the fused pass without its store, for a step that
// forms the last micro-batch's sum again as it reads it (the AdamW step's
// summed-gradient forms).  Each wave runs, for K of the one-wave workgroups
// of accum_kernel<Q, 64, ...> (virtual blocks of nvb), exactly what each
// computes for its partial: the same Q groups per lane, sums, butterfly
// and slot, so the partials, and the norm formed from them, are bit for bit
// the fused pass's.  The K blocks of a wave are those its XCD would have run
// (workgroup B runs on XCD B mod 8; its blocks are 8j + B mod 8 for K
// consecutive j), so its partials fall in its XCD's run of slots and every
// line of partials is still written by one XCD.  Read-only: acc (unless
// OVERWRITE) and grad, dword alignment suffices for both; on the vector path
// every load of the wave's K blocks is issued before the first square.
template <int Q, int W, int K, bool VEC, bool BF16, bool OVERWRITE>
__global__ __launch_bounds__(W * 64) void sum_norm_kernel(const float* __restrict__ acc,
                                                          const void* __restrict__ grad, int64_t n, int64_t nvb,
                                                          float scale, double* __restrict__ partials) {
    constexpr int64_t kGroup = 256;   // one wave's 64 lanes x 4 elements
    constexpr int64_t kSpan = kGroup * Q;   // elements per virtual block
    const int64_t wave = threadIdx.x >> 6;
    if (xcd_block(blockIdx.x, wave, 0, W, K) >= nvb) return;   // no block for this wave (whole waves)
    const int lane = threadIdx.x & 63;
    const int64_t vb_last = xcd_block(blockIdx.x, wave, K - 1, W, K);
    if (VEC && (vb_last + 1) * kSpan <= n) {   // all K blocks exist and are whole
        f32x4 g[K * Q], a[K * Q];
#pragma unroll
        for (int k = 0; k < K; ++k) {
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const int64_t at = xcd_block(blockIdx.x, wave, k, W, K) * kSpan + q * kGroup + lane * 4;
                g[k * Q + q] = load4<BF16>(grad, at);
                if (!OVERWRITE) a[k * Q + q] = ld_stream_f32x4_a4(acc + at);
            }
        }
#pragma unroll
        for (int k = 0; k < K; ++k) {
            double s0 = 0.0, s1 = 0.0;
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const int i = k * Q + q;
                const f32x4 r = OVERWRITE ? g[i]
                                          : f32x4{a[i].x + g[i].x, a[i].y + g[i].y, a[i].z + g[i].z,
                                                  a[i].w + g[i].w};
                const float rv[4] = {r.x, r.y, r.z, r.w};
                add_squares4(rv, scale, s0, s1);
            }
            const double total = wave_sum(s0 + s1);
            if (lane == 0) partials[xcd_slot(xcd_block(blockIdx.x, wave, k, W, K), nvb)] = total;
        }
        return;
    }
    // the ragged end: block by block, element by element (out-of-range
    // elements add +0), as the fused kernel's ragged tile
    for (int k = 0; k < K && xcd_block(blockIdx.x, wave, k, W, K) < nvb; ++k) {
        const int64_t vb = xcd_block(blockIdx.x, wave, k, W, K);
        double s0 = 0.0, s1 = 0.0;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int64_t first = vb * kSpan + q * kGroup + lane * 4;
            float rv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t i = first + j;
                if (i < n) {
                    const float g = load1<BF16>(grad, i);
                    rv[j] = OVERWRITE ? g : acc[i] + g;
                }
            }
            add_squares4(rv, scale, s0, s1);
        }
        const double total = wave_sum(s0 + s1);
        if (lane == 0) partials[xcd_slot(vb, nvb)] = total;
    }
}

// One-wave workgroups, uncapped, as the fused kernel; each wave takes two
// blocks of the accumulating shape (Q = 1: 89.3 % of the HBM peak on gfx950
// for a bf16 gradient onto the accumulator, against 81.4 % for one and 85.5 %
// for four; two blocks that are neighbours in memory instead of in their
// XCD's run measured 82.6 %, their partials written 2x) and one of the
// overwriting bf16 shape (Q = 4: 92.5 %, against 91.8 % for two).
constexpr int kSumNormWaves = 1;   // waves per workgroup of sum_norm_kernel
template <int Q>
constexpr int sum_norm_blocks() { return Q == 1 ? 2 : 1; }   // virtual blocks per wave

// launch pieces and partial positions as launch() gives the fused kernel
template <int Q, bool VEC, bool BF16, bool OVERWRITE>
hipError_t launch_sum_norm(const float* acc, const void* grad, int64_t n, float scale, double* partials,
                           hipStream_t stream) {
    const int64_t gsz = BF16 ? 2 : 4;
    for (int64_t off = 0; off < n; off += kLaunchElems) {
        const int64_t m = launch_piece(n, off);
        const int64_t nvb = (m + per_block<Q>() - 1) / per_block<Q>();
        constexpr int K = sum_norm_blocks<Q>();
        const int64_t blocks = sum_norm_grid(nvb, kSumNormWaves, K);
        hipLaunchKernelGGL((sum_norm_kernel<Q, kSumNormWaves, K, VEC, BF16, OVERWRITE>),
                           dim3((unsigned)blocks),
                           dim3(kSumNormWaves * 64), 0, stream, OVERWRITE ? nullptr : acc + off,
                           static_cast<const char*>(grad) + off * gsz, m, nvb, scale, partials + off / per_block<Q>());
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int Q, bool OVERWRITE>
hipError_t dispatch_sum_norm(const float* acc, const void* grad, int grad_bf16, int64_t n, bool vec, float scale,
                             double* partials, hipStream_t stream) {
    if (vec)
        return grad_bf16 ? launch_sum_norm<Q, true, true, OVERWRITE>(acc, grad, n, scale, partials, stream)
                         : launch_sum_norm<Q, true, false, OVERWRITE>(acc, grad, n, scale, partials, stream);
    return grad_bf16 ? launch_sum_norm<Q, false, true, OVERWRITE>(acc, grad, n, scale, partials, stream)
                     : launch_sum_norm<Q, false, false, OVERWRITE>(acc, grad, n, scale, partials, stream);
}

}  // namespace

hipError_t launch_grad_sum_norm_sq(const float* acc, const void* grad, int grad_bf16, int64_t n, int overwrite,
                                   float scale, double* out, double* workspace, bool vec_ok,
                                   hipStream_t stream) {
    int64_t parts = 0;
    if (n > 0) {
        hipError_t e;
        // the fused pass's shapes: Q = 4 for an overwriting bf16 gradient, else 1
        if (overwrite && grad_bf16) {
            parts = (n + per_block<kFusedQOverwrite>() - 1) / per_block<kFusedQOverwrite>();
            e = dispatch_sum_norm<kFusedQOverwrite, true>(acc, grad, grad_bf16, n, vec_ok, scale, workspace,
                                                          stream);
        } else {
            parts = (n + per_block<kFusedQAdd>() - 1) / per_block<kFusedQAdd>();
            e = overwrite ? dispatch_sum_norm<kFusedQAdd, true>(acc, grad, grad_bf16, n, vec_ok, scale, workspace,
                                                                stream)
                          : dispatch_sum_norm<kFusedQAdd, false>(acc, grad, grad_bf16, n, vec_ok, scale,
                                                                 workspace, stream);
        }
        if (e != hipSuccess) return e;
    }
    return launch_sum_partials(workspace, parts, workspace + accum_norm_partials(n), out, stream);
}

hipError_t launch_grad_accum(float* acc, const void* grad, int grad_bf16, int64_t n, int overwrite,
                             bool vec_ok, hipStream_t stream) {
    if (overwrite) return dispatch<1, false, true>(acc, grad, grad_bf16, n, vec_ok, 0.0f, nullptr, 0, stream);
    return dispatch<1, false, false>(acc, grad, grad_bf16, n, vec_ok, 0.0f, nullptr,
                                     grad_bf16 ? kAddLdsBf16 : kAddLdsF32, stream);
}

// workspace partials: the larger count of the two fused shapes
int64_t accum_norm_partials(int64_t n) {
    return n <= 0 ? 0 : (n + per_block<kFusedQAdd>() - 1) / per_block<kFusedQAdd>();
}

hipError_t launch_grad_accum_norm_sq(float* acc, const void* grad, int grad_bf16, int64_t n, int overwrite,
                                     float scale, double* out, double* workspace, bool vec_ok,
                                     hipStream_t stream) {
    int64_t parts = 0;
    if (n > 0) {
        hipError_t e;
        if (overwrite && grad_bf16) {
            parts = (n + per_block<kFusedQOverwrite>() - 1) / per_block<kFusedQOverwrite>();
            e = dispatch<kFusedQOverwrite, true, true>(acc, grad, grad_bf16, n, vec_ok, scale, workspace,
                                                       kFusedOverwriteLds, stream);
        } else {
            parts = (n + per_block<kFusedQAdd>() - 1) / per_block<kFusedQAdd>();
            e = overwrite ? dispatch<kFusedQAdd, true, true>(acc, grad, grad_bf16, n, vec_ok, scale, workspace, 0,
                                                             stream)
                          : dispatch<kFusedQAdd, true, false>(acc, grad, grad_bf16, n, vec_ok, scale, workspace, 0,
                                                              stream);
        }
        if (e != hipSuccess) return e;
    }
    // the stage buffer follows the largest partial count the workspace is sized for
    return launch_sum_partials(workspace, parts, workspace + accum_norm_partials(n), out, stream);
}

}  // namespace zs

// ---------------------------------------------------------------------------
// Sum of N rank chunks into this rank's fp32 shard, in rank order: the
// arithmetic of a reduce-scatter's receiving side.  One pass per launch of up
// to kReduceMaxChunks chunks: acc = ((acc + widen(c0)) + widen(c1)) + ...,
// the same left fold, rounding for rounding, as one grad_accum call per
// chunk, at 2 B (bf16) or 4 B (fp32) per chunk element plus 8 B of acc
// traffic per element instead of ~10 B per chunk element.
// ---------------------------------------------------------------------------
namespace zs {
namespace {

// Layout: one-wave workgroups, two groups of 4 elements per lane, 256
// elements apart (every chunk's loads for both groups issued before the
// fold): 76 % of the HBM peak on gfx950 for 8 bf16 chunks, against 68 % for
// one group per lane in 256-thread workgroups (with the residency caps
// below, 82 % against 74-77 % for 256-thread workgroups of two or four groups
// under caps of 0-40 KiB, and 63-72 % for one-wave workgroups of four).
constexpr int kReduceBlock = 64;
constexpr int kReduceGroups = 2;

// LDS reserved (never touched) per workgroup to cap residency, by chunk
// dtype and count, whether the pass overwrites the accumulator or adds into
// it (one more stream: the accumulator read), and whether it forms the norm,
// as measured on gfx950 over the 842M-element shard (% of the HBM peak at the
// cap taken / uncapped):
//   bf16 chunks   overwrite          add                overwrite + norm   add + norm
//   2             8 KiB  84 / 81     12 KiB 83.5 / 77   none 83            8 KiB  81.5 / 78
//   3-4           12 KiB 83 / 77     16 KiB 83 / 73     8 KiB  81.5 / 78   12 KiB 83 / 73
//   5-8           20 KiB 82 / 72     20 KiB 80 / -      14.5 KiB 81 / 72   18 KiB 81 / -
// (14.5 KiB is 11 workgroups per CU, 18 KiB 9).  The pass that forms the
// norm keeps each wave longer (the binary64 squares and the butterfly at
// its end) and mostly wants one step more residency.  More chunks, or fp32
// chunks beyond two, run best uncapped.
unsigned reduce_lds_reserve(bool bf16, int count, bool overwrite, bool norm) {
    if (bf16) {
        if (count > 8) return 0u;
        const int c = count <= 2 ? 0 : count <= 4 ? 1 : 2;
        static constexpr unsigned kCap[2][2][3] = {
            {{12288u, 16384u, 20480u}, {8192u, 12288u, 18176u}},   // add: plain, norm
            {{8192u, 12288u, 20480u}, {0u, 8192u, 14848u}},        // overwrite: plain, norm
        };
        return kCap[overwrite ? 1 : 0][norm ? 1 : 0][c];
    }
    return count <= 2 ? 12288u : 0u;
}

// The loaded words stay in their storage width (2 VGPRs per bf16 group, not
// 4) until the fold widens them: with 16 chunks x 2 groups in flight this
// keeps the kernel at 6+ waves per SIMD instead of 3.
template <bool BF16> struct Raw4;
template <> struct Raw4<true> {
    using T = u32x2;
    static __device__ __forceinline__ T load(const void* p, int64_t i) {
        return ld_stream_u32x2_a4(static_cast<const uint16_t*>(p) + i);   // read-only: dword alignment
    }
    static __device__ __forceinline__ f32x4 widen(T w) {
        return f32x4{bf16_to_f32(w.x & 0xFFFFu), bf16_to_f32(w.x >> 16), bf16_to_f32(w.y & 0xFFFFu),
                     bf16_to_f32(w.y >> 16)};
    }
};
template <> struct Raw4<false> {
    using T = f32x4;
    static __device__ __forceinline__ T load(const void* p, int64_t i) {
        return ld_stream_f32x4_a4(static_cast<const float*>(p) + i);
    }
    static __device__ __forceinline__ f32x4 widen(T w) { return w; }
};

// NORM: the pass that folds the last chunks also adds the squares of the
// scaled sums, one binary64 partial per wave (512 elements), as the fused
// accumulation does for one micro-batch.
template <bool VEC, bool BF16, bool OVERWRITE, bool NORM>
__global__ __launch_bounds__(kReduceBlock) void reduce_chunks_kernel(float* __restrict__ acc, const ChunkBatch b,
                                                                     int64_t n, float scale,
                                                                     double* __restrict__ partials) {
    static_assert(kReduceBlock == 64, "the norm's partial is one wave's butterfly");
    constexpr int64_t kGroup = kReduceBlock * 4;
    const int64_t tile = (int64_t)blockIdx.x * kGroup * kReduceGroups;
    const int64_t lane0 = tile + threadIdx.x * 4;
    const int count = b.count;
    double s0 = 0.0, s1 = 0.0;
    if (VEC && tile + kGroup * kReduceGroups <= n) {   // whole tile in range
        using R = Raw4<BF16>;
        f32x4 r[kReduceGroups];
        typename R::T g[kReduceGroups][kReduceMaxChunks];
#pragma unroll
        for (int q = 0; q < kReduceGroups; ++q) {
            r[q] = OVERWRITE ? f32x4{0.0f, 0.0f, 0.0f, 0.0f}
                             : ld_stream(reinterpret_cast<const f32x4*>(acc + lane0 + q * kGroup));
#pragma unroll
            for (int k = 0; k < kReduceMaxChunks; ++k)
                if (k < count) g[q][k] = R::load(b.chunk[k], lane0 + q * kGroup);
        }
#pragma unroll
        for (int q = 0; q < kReduceGroups; ++q) {
#pragma unroll
            for (int k = 0; k < kReduceMaxChunks; ++k) {
                if (k < count) {
                    const f32x4 x = R::widen(g[q][k]);
                    // the first chunk of an overwriting batch is a copy (keeps -0.0)
                    r[q] = (OVERWRITE && k == 0) ? x
                                                 : f32x4{r[q].x + x.x, r[q].y + x.y, r[q].z + x.z, r[q].w + x.w};
                }
            }
            st_stream(reinterpret_cast<f32x4*>(acc + lane0 + q * kGroup), r[q]);
            if (NORM) {
                const float rv[4] = {r[q].x, r[q].y, r[q].z, r[q].w};
                add_squares4(rv, scale, s0, s1);
            }
        }
    } else {
        // ragged tile (or a misaligned buffer): element by element, the same
        // association for the norm (out-of-range elements add +0)
#pragma unroll
        for (int q = 0; q < kReduceGroups; ++q) {
            const int64_t first = lane0 + q * kGroup;
            float rv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t i = first + j;
                if (i < n) {
                    float r = OVERWRITE ? 0.0f : acc[i];
                    for (int k = 0; k < count; ++k) {
                        const float g = load1<BF16>(b.chunk[k], i);
                        r = (OVERWRITE && k == 0) ? g : r + g;
                    }
                    acc[i] = r;
                    rv[j] = r;
                }
            }
            if (NORM) add_squares4(rv, scale, s0, s1);
        }
    }
    if (NORM) {
        const double total = wave_sum(s0 + s1);
        if (threadIdx.x == 0) partials[xcd_slot(blockIdx.x, gridDim.x)] = total;
    }
}

constexpr int64_t kReducePerBlock = (int64_t)kReduceBlock * 4 * kReduceGroups;
static_assert(kLaunchElems % kReducePerBlock == 0, "pieces keep the partials' positions");

// one launch per kLaunchElems elements, the chunk pointers advanced with acc;
// piece k's partials follow piece k-1's
template <bool VEC, bool BF16, bool OVERWRITE, bool NORM>
hipError_t launch_reduce(float* acc, const ChunkBatch& b, int64_t n, float scale, double* partials,
                         hipStream_t stream) {
    const int64_t per = kReducePerBlock;
    const int64_t gsz = BF16 ? 2 : 4;
    const unsigned lds = VEC ? reduce_lds_reserve(BF16, b.count, OVERWRITE, NORM) : 0u;
    for (int64_t off = 0; off < n; off += kLaunchElems) {
        const int64_t m = launch_piece(n, off);
        ChunkBatch p = b;
        for (int k = 0; k < b.count; ++k) p.chunk[k] = static_cast<const char*>(b.chunk[k]) + off * gsz;
        const int64_t blocks = (m + per - 1) / per;
        hipLaunchKernelGGL((reduce_chunks_kernel<VEC, BF16, OVERWRITE, NORM>), dim3((unsigned)blocks),
                           dim3(kReduceBlock), lds, stream, acc + off, p, m, scale,
                           NORM ? partials + off / per : nullptr);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <bool NORM>
hipError_t dispatch_reduce(float* acc, const ChunkBatch& b, bool bf16, int64_t n, bool overwrite, bool vec,
                           float scale, double* partials, hipStream_t stream) {
    if (vec) {
        if (bf16) return overwrite ? launch_reduce<true, true, true, NORM>(acc, b, n, scale, partials, stream)
                                   : launch_reduce<true, true, false, NORM>(acc, b, n, scale, partials, stream);
        return overwrite ? launch_reduce<true, false, true, NORM>(acc, b, n, scale, partials, stream)
                         : launch_reduce<true, false, false, NORM>(acc, b, n, scale, partials, stream);
    }
    if (bf16) return overwrite ? launch_reduce<false, true, true, NORM>(acc, b, n, scale, partials, stream)
                               : launch_reduce<false, true, false, NORM>(acc, b, n, scale, partials, stream);
    return overwrite ? launch_reduce<false, false, true, NORM>(acc, b, n, scale, partials, stream)
                     : launch_reduce<false, false, false, NORM>(acc, b, n, scale, partials, stream);
}

}  // namespace

hipError_t launch_reduce_chunks(float* acc, const ChunkBatch& b, int grad_bf16, int64_t n, int overwrite,
                                bool vec_ok, hipStream_t stream) {
    return dispatch_reduce<false>(acc, b, grad_bf16 != 0, n, overwrite != 0, vec_ok, 0.0f, nullptr, stream);
}

int64_t reduce_norm_partials(int64_t n) { return n <= 0 ? 0 : (n + kReducePerBlock - 1) / kReducePerBlock; }

hipError_t launch_reduce_chunks_norm_sq(float* acc, const ChunkBatch& b, int grad_bf16, int64_t n, int overwrite,
                                        bool vec_ok, float scale, double* out, double* workspace,
                                        hipStream_t stream) {
    const int64_t parts = reduce_norm_partials(n);
    if (n > 0) {
        const hipError_t e = dispatch_reduce<true>(acc, b, grad_bf16 != 0, n, overwrite != 0, vec_ok, scale,
                                                   workspace, stream);
        if (e != hipSuccess) return e;
    }
    return launch_sum_partials(workspace, parts, workspace + parts, out, stream);
}

}  // namespace zs
