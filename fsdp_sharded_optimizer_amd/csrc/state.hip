// Conversions between split fp32 optimizer-state arrays (one buffer each) and
// the tiled layouts the tiled AdamW steps stream (zs_common.h: per tile of
// kStateTile elements, a run of each array: master, exp_avg, exp_avg_sq for
// the master forms; exp_avg, exp_avg_sq for the no-master and update forms).
//
// A layout change, not arithmetic: each value is copied bit for bit.  These
// run when a shard's state is set up, checkpointed or restored, not in the
// step, so they are plain streaming copies: 256-thread workgroups, 4
// consecutive elements per lane per stream (128-bit accesses), one-shot grid.
// Tile direction: reads and writes 4 B per element per array (4 B read less
// per missing source); the last tile's unused ends are written as zeros so
// the whole buffer is defined.  Untile direction: the same bytes the other way;
// a missing destination is neither read nor written.
#include "zs_common.h"

namespace zs {
namespace {

constexpr int kStateBlock = 256;
constexpr int64_t kStateGroupElems = 4;   // elements per lane per stream

struct TileArgs {
    const float* src[3];   // the R arrays (nullable: zeros)
    float* state;
    int64_t n;             // elements of this piece
    int64_t n_padded;      // whole tiles: every float of them is written
};

// 4 consecutive tiled positions [i, i+4) (never straddling a tile) of each
// of the R streams: element values below n, zeros from n on.  Sources are
// read-only, so a dword-aligned 128-bit load serves them on gfx950; the
// tiled side is 16-byte aligned by the entry point's contract.
template <int R>
__global__ __launch_bounds__(kStateBlock) void state_tile_kernel(const TileArgs a) {
    const int64_t i = ((int64_t)blockIdx.x * kStateBlock + threadIdx.x) * kStateGroupElems;
    if (i >= a.n_padded) return;
    float* const dst = a.state + tiled_offset<R>(i);
#pragma unroll
    for (int k = 0; k < R; ++k) {
        f32x4 x = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        const float* s = a.src[k];
        if (s != nullptr) {
            if (i + 4 <= a.n) {
                x = ld_stream_f32x4_a4(s + i);
            } else {
                if (i + 0 < a.n) x.x = s[i + 0];
                if (i + 1 < a.n) x.y = s[i + 1];
                if (i + 2 < a.n) x.z = s[i + 2];
            }
        }
        st_stream(reinterpret_cast<f32x4*>(dst + k * kStateTile), x);
    }
}

struct UntileArgs {
    const float* state;
    float* dst[3];         // the R arrays (nullable: skipped)
    int64_t n;
};

// VEC: every destination is 16-byte aligned, so a full group is one 128-bit
// store; otherwise element stores.
template <int R, bool VEC>
__global__ __launch_bounds__(kStateBlock) void state_untile_kernel(const UntileArgs a) {
    const int64_t i = ((int64_t)blockIdx.x * kStateBlock + threadIdx.x) * kStateGroupElems;
    if (i >= a.n) return;
    const float* const src = a.state + tiled_offset<R>(i);
#pragma unroll
    for (int k = 0; k < R; ++k) {
        float* const d = a.dst[k];
        if (d == nullptr) continue;
        const f32x4 x = ld_stream(reinterpret_cast<const f32x4*>(src + k * kStateTile));
        if (VEC && i + 4 <= a.n) {
            st_stream(reinterpret_cast<f32x4*>(d + i), x);
        } else {
            d[i] = x.x;
            if (i + 1 < a.n) d[i + 1] = x.y;
            if (i + 2 < a.n) d[i + 2] = x.z;
            if (i + 3 < a.n) d[i + 3] = x.w;
        }
    }
}

const float* advance_c(const float* p, int64_t off) { return p == nullptr ? nullptr : p + off; }
float* advance_m(float* p, int64_t off) { return p == nullptr ? nullptr : p + off; }

int64_t whole_tiles(int64_t n) { return (n + kStateTile - 1) / kStateTile * kStateTile; }

}  // namespace

hipError_t launch_tile_runs(const float* const* src, int runs, float* buf, int64_t n, hipStream_t stream) {
    static_assert(kLaunchElems % kStateTile == 0, "launch pieces start on a tile");
    for (int64_t off = 0; off < n; off += kLaunchElems) {
        TileArgs a;
        a.n = launch_piece(n, off);
        a.n_padded = whole_tiles(a.n);
        for (int k = 0; k < 3; ++k) a.src[k] = k < runs ? advance_c(src[k], off) : nullptr;
        a.state = buf + runs * off;
        const int64_t blocks = (a.n_padded / kStateGroupElems + kStateBlock - 1) / kStateBlock;
        if (runs == 3)
            hipLaunchKernelGGL(state_tile_kernel<3>, dim3((unsigned)blocks), dim3(kStateBlock), 0, stream, a);
        else
            hipLaunchKernelGGL(state_tile_kernel<2>, dim3((unsigned)blocks), dim3(kStateBlock), 0, stream, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_untile_runs(const float* buf, int runs, float* const* dst, int64_t n, bool vec_ok,
                              hipStream_t stream) {
    for (int64_t off = 0; off < n; off += kLaunchElems) {
        UntileArgs a;
        a.n = launch_piece(n, off);
        a.state = buf + runs * off;
        for (int k = 0; k < 3; ++k) a.dst[k] = k < runs ? advance_m(dst[k], off) : nullptr;
        const int64_t blocks = ((a.n + kStateGroupElems - 1) / kStateGroupElems + kStateBlock - 1) / kStateBlock;
        const dim3 grid((unsigned)blocks), block(kStateBlock);
        if (runs == 3) {
            if (vec_ok) hipLaunchKernelGGL((state_untile_kernel<3, true>), grid, block, 0, stream, a);
            else hipLaunchKernelGGL((state_untile_kernel<3, false>), grid, block, 0, stream, a);
        } else {
            if (vec_ok) hipLaunchKernelGGL((state_untile_kernel<2, true>), grid, block, 0, stream, a);
            else hipLaunchKernelGGL((state_untile_kernel<2, false>), grid, block, 0, stream, a);
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace zs
