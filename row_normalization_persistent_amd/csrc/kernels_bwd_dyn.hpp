// Backward kernels of the run-time-hidden path: the combined inner + outer
// reduction of "Llu/ln bwd" (author note and review thread) for LayerNorm and,
// with the same structure, RMSNorm and the fused residual-add + RMSNorm, with
// hidden, the row strides and 1/hidden as kernel arguments.  Arithmetic per
// row is that of the compiled-hidden backward kernels; the layout of a row in
// registers and the masking of accesses past the row's end are those of
// dyn_common.hpp.
//
// A workgroup of dyn_block<T>() lanes runs R = block / T row "walkers" (one
// per lane group); walker w of P = grid * R walks the rows w, w + P, w + 2P, ...
// with a ring of D rows in flight and accumulates the column sums of its
// lanes' columns in registers.  At the end the workgroup adds its R walkers'
// sums in LDS (walker order) and writes one slab of the workspace:
// [grid][outs][padded] fp32, padded = hidden rounded up to 64.  The shared
// column-reduce kernel then sums the grid slabs in a fixed order.
//
// Every walker of a workgroup runs as many ring steps as the workgroup's
// first walker (which has the most rows); the extra rows are past the end,
// load zeros from no memory, store nothing and add exactly zero to the sums
// (their dy is zero and their statistics are forced to zero), so the loop has
// no per-walker branch and every barrier is reached by the whole workgroup.
#pragma once

#include <type_traits>
#include <utility>

#include "dyn_common.hpp"
#include "launch.hpp"

namespace rownorm {

template <int W, int T>
__device__ __forceinline__ int dyn_boff(int b, int lane) { return (b * T + lane) * (2 * W); }

template <int W, int V, bool LN, bool DRES>
struct DynRow {
    raw_t<W> x[V];
    raw_t<W> dy[V];
    raw_t<W> dres[DRES ? V : 1];
    float mean, rstd;  // LayerNorm only
};

// The rows one ring step of a workgroup touches: for rows of >= 64 lanes each
// lane group's own row (one descriptor per row, uniform over its waves); for
// narrower rows the R consecutive rows of all the workgroup's groups (one
// descriptor, each lane at its row's offset).  See rows_rsrc / set_off.
struct WalkRows {
    int64_t first;  // first row of the set
    int span;       // rows in the set
    int local;      // this lane group's row within the set
    __device__ __forceinline__ int64_t row() const { return first + local; }
};

template <int T>
__device__ __forceinline__ WalkRows walk_rows(int64_t wg_first, int g, int64_t step) {
    if constexpr (T < kWave) return WalkRows{opaque_row(wg_first + step), dyn_block<T>() / T, g};
    else return WalkRows{opaque_row(wg_first + g + step), 1, 0};
}

template <int W, int T>
__device__ __forceinline__ int walk_off(const WalkRows& w, int b, int lane, int64_t ld, int h) {
    return set_off<T>(w.local, (b * T + lane) * W, ld, h, 2);
}

template <int W, int T, int V, bool LN, bool DRES>
__device__ __forceinline__ void dyn_load_row(DynRow<W, V, LN, DRES>& r, const DynBwdArgs& a,
                                             const WalkRows& w, int lane) {
    const int h = a.hidden;
    const rsrc_t rx = rows_rsrc<T>(a.x, w.first, w.span, a.rows, a.ld_x, h, 2);
    const rsrc_t rd = rows_rsrc<T>(a.dy, w.first, w.span, a.rows, a.ld_dy, h, 2);
#pragma unroll
    for (int b = 0; b < V; ++b)
        r.x[b] = aload<W, kCachePolicyNT>(rx, walk_off<W, T>(w, b, lane, a.ld_x, h));
#pragma unroll
    for (int b = 0; b < V; ++b)
        r.dy[b] = aload<W, kCachePolicyNT>(rd, walk_off<W, T>(w, b, lane, a.ld_dy, h));
    if constexpr (DRES) {
        const rsrc_t rr = rows_rsrc<T>(a.dres, w.first, w.span, a.rows, a.ld_dres, h, 2);
#pragma unroll
        for (int b = 0; b < V; ++b)
            r.dres[b] = aload<W, kCachePolicyNT>(rr, walk_off<W, T>(w, b, lane, a.ld_dres, h));
    }
    if constexpr (LN) {
        if constexpr (T >= kWave) {
            // one row per lane group: its mean and rstd are wave-uniform, so
            // scalar loads (through the constant address space: the kernel
            // never writes them) from a clamped row index replace a buffer
            // load in every lane (rows >= 1 whenever the kernel runs)
            typedef const __attribute__((address_space(4))) float cfloat;
            const int64_t row = w.first;
            const int64_t rc = row < a.rows ? row : a.rows - 1;
            const float m = ((const cfloat*)(uintptr_t)a.mean)[rc];
            const float q = ((const cfloat*)(uintptr_t)a.rstd)[rc];
            r.mean = row < a.rows ? m : 0.0f;
            r.rstd = row < a.rows ? q : 0.0f;
        } else {
            const int off = set_off<T>(w.local, 0, 1, 1, 4);
            r.mean = rload_f32(rows_rsrc<T>(a.mean, w.first, w.span, a.rows, 1, 1, 4), off);
            r.rstd = rload_f32(rows_rsrc<T>(a.rstd, w.first, w.span, a.rows, 1, 1, 4), off);
        }
    }
}

// LayerNorm row: c1 = mean_j g, c2 = mean_j g * xhat, dx = rstd (g - c1 - xhat c2);
// pw += dy * xhat, pb += dy.  Past the row's end dy = w = 0, so g = 0 and
// the accesses there add nothing.
template <int W, int T, int V>
__device__ __forceinline__ void dyn_ln_row(const DynRow<W, V, true, false>& cur,
                                           const float (&wf)[V][W], float (&pw)[V][W],
                                           float (&pb)[V][W], const DynBwdArgs& a, float inv_h,
                                           float* slot, const WalkRows& w, int lane) {
    float xh[V][W], g[V][W];
    float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
    for (int b = 0; b < V; ++b) {
        float xf[W], df[W];
        aunpack<W>(cur.x[b], xf);
        aunpack<W>(cur.dy[b], df);
#pragma unroll
        for (int k = 0; k < W; ++k) {
            xh[b][k] = (xf[k] - cur.mean) * cur.rstd;
            g[b][k] = df[k] * wf[b][k];
            s1 += g[b][k];
            s2 += g[b][k] * xh[b][k];
            pw[b][k] += df[k] * xh[b][k];
            pb[b][k] += df[k];
        }
    }
    dyn_row_sum2<T>(s1, s2, slot, lane);
    const float c1 = s1 * inv_h;
    const float c2 = s2 * inv_h;
    const rsrc_t rdx = rows_rsrc<T>(a.dx, w.first, w.span, a.rows, a.ld_dx, a.hidden, 2);
#pragma unroll
    for (int b = 0; b < V; ++b) {
        float o[W];
#pragma unroll
        for (int k = 0; k < W; ++k) o[k] = cur.rstd * (g[b][k] - c1 - xh[b][k] * c2);
        astore<W, kCachePolicyNT>(rdx, walk_off<W, T>(w, b, lane, a.ld_dx, a.hidden),
                                  apack<W>(o));
    }
}

// RMSNorm row: rstd = rsqrt(mean_j x^2 + eps), dx = rstd g - rstd^3 mean_j(g x) x
// [+ dres]; pw += dy * x * rstd.
template <int W, int T, int V, bool DRES>
__device__ __forceinline__ void dyn_rms_row(const DynRow<W, V, false, DRES>& cur,
                                            const float (&wf)[V][W], float (&pw)[V][W],
                                            const DynBwdArgs& a, float inv_h, float* slot,
                                            const WalkRows& w, int lane) {
    float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
    for (int b = 0; b < V; ++b) {
        float xf[W], df[W];
        aunpack<W>(cur.x[b], xf);
        aunpack<W>(cur.dy[b], df);
#pragma unroll
        for (int k = 0; k < W; ++k) {
            s1 += xf[k] * xf[k];
            s2 += df[k] * wf[b][k] * xf[k];
        }
    }
    dyn_row_sum2<T>(s1, s2, slot, lane);
    // a row past the end must add exactly nothing, also at eps = 0
    const float rstd = w.row() < a.rows ? fast_rsqrt(s1 * inv_h + a.eps) : 0.0f;
    const float coef = rstd * rstd * rstd * s2 * inv_h;
    const rsrc_t rdx = rows_rsrc<T>(a.dx, w.first, w.span, a.rows, a.ld_dx, a.hidden, 2);
#pragma unroll
    for (int b = 0; b < V; ++b) {
        float xf[W], df[W], o[W];
        aunpack<W>(cur.x[b], xf);
        aunpack<W>(cur.dy[b], df);
#pragma unroll
        for (int k = 0; k < W; ++k) {
            o[k] = rstd * (df[k] * wf[b][k]) - coef * xf[k];
            pw[b][k] += df[k] * (xf[k] * rstd);
        }
        if constexpr (DRES) {
            float rf[W];
            aunpack<W>(cur.dres[b], rf);
#pragma unroll
            for (int k = 0; k < W; ++k) o[k] += rf[k];
        }
        astore<W, kCachePolicyNT>(rdx, walk_off<W, T>(w, b, lane, a.ld_dx, a.hidden),
                                  apack<W>(o));
    }
}

// Writes the workgroup's column sums to its slab (columns past hidden are
// skipped; they hold zeros anyway).  One walker (R == 1): each lane stores its
// own.  Several: per access b, every lane puts its W sums in LDS, then the
// workgroup's lanes take the access's T * W columns in turn, add each over
// the R walkers in walker order and store it; `stage` holds R * T * W floats.
// Uniform control flow required.
template <int W, int T, int V>
__device__ __forceinline__ void dyn_store_partials(float* slab, const float (&p)[V][W],
                                                   int hidden, int lane, int g, float* stage) {
    constexpr int R = dyn_block<T>() / T;
    if constexpr (R == 1) {
#pragma unroll
        for (int b = 0; b < V; ++b) {
            const int col = (b * T + lane) * W;
            if (col < hidden) {
#pragma unroll
                for (int k = 0; k < W; ++k) slab[col + k] = p[b][k];
            }
        }
    } else {
        constexpr int kCols = T * W;  // columns of one access
        constexpr int kBlock = dyn_block<T>();
#pragma unroll
        for (int b = 0; b < V; ++b) {
#pragma unroll
            for (int k = 0; k < W; ++k) stage[(g * T + lane) * W + k] = p[b][k];
            __syncthreads();
#pragma unroll
            for (int c0 = 0; c0 < kCols; c0 += kBlock) {
                const int c = c0 + (int)threadIdx.x;
                if (c < kCols && b * kCols + c < hidden) {
                    float s = stage[c];
#pragma unroll
                    for (int r = 1; r < R; ++r) s += stage[r * kCols + c];
                    slab[b * kCols + c] = s;
                }
            }
            __syncthreads();
        }
    }
}

template <int W, int T, int V, int D, bool LN, bool DRES>
__global__ __launch_bounds__(dyn_block<T>()) void norm_bwd_dyn_rows_kernel(DynBwdArgs a) {
    constexpr int R = dyn_block<T>() / T;
    constexpr int kSlot = 2 * dyn_red_floats<T>();  // one two-value reduction of the workgroup
    __shared__ float red[2 * kSlot];
    const int lane = threadIdx.x % T;
    const int g = uniform_group<T>(threadIdx.x / T);
    const float inv_h = 1.0f / (float)a.hidden;

    float wf[V][W];
    {
        const rsrc_t rw = row_rsrc_ld(a.weight, 0, 1, 0, a.hidden * 2);
#pragma unroll
        for (int b = 0; b < V; ++b) aunpack<W>(aload<W, 0>(rw, dyn_boff<W, T>(b, lane)), wf[b]);
    }
    float pw[V][W], pb[LN ? V : 1][W];
#pragma unroll
    for (int b = 0; b < V; ++b)
#pragma unroll
        for (int k = 0; k < W; ++k) pw[b][k] = 0.0f;
    if constexpr (LN) {
#pragma unroll
        for (int b = 0; b < V; ++b)
#pragma unroll
            for (int k = 0; k < W; ++k) pb[b][k] = 0.0f;
    }

    const int64_t P = (int64_t)gridDim.x * R;
    const int64_t first = (int64_t)blockIdx.x * R;  // the workgroup's first walker
    const int64_t n = first < a.rows ? (a.rows - 1 - first) / P + 1 : 0;
    DynRow<W, V, LN, DRES> buf[D];
    // fences keep each slot's loads in slot order (precise memory-counter waits)
#pragma unroll
    for (int d = 0; d < D; ++d) {
        dyn_load_row<W, T, V, LN, DRES>(buf[d], a, walk_rows<T>(first, g, d * P), lane);
        issue_fence();
    }
    int parity = 0;
    for (int64_t i = 0; i < n; i += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const WalkRows w = walk_rows<T>(first, g, (i + d) * P);
            float* slot = red + parity * kSlot + g * (2 * (T / kWave));
            if constexpr (LN)
                dyn_ln_row<W, T, V>(buf[d], wf, pw, pb, a, inv_h, slot, w, lane);
            else
                dyn_rms_row<W, T, V, DRES>(buf[d], wf, pw, a, inv_h, slot, w, lane);
            parity ^= 1;
            issue_fence();
            dyn_load_row<W, T, V, LN, DRES>(buf[d], a, walk_rows<T>(first, g, (i + d + D) * P),
                                            lane);
            issue_fence();
        }
    }

    const int64_t padded = dyn_padded_hidden(a.hidden);
    float* slab = a.workspace + (int64_t)blockIdx.x * (LN ? 2 : 1) * padded;
    __shared__ float stage[R > 1 ? dyn_block<T>() * W : 1];
    dyn_store_partials<W, T, V>(slab, pw, a.hidden, lane, g, stage);
    if constexpr (LN) dyn_store_partials<W, T, V>(slab + padded, pb, a.hidden, lane, g, stage);
}

// Ring depth: as deep as the register budget allows without spills (the
// compiler's resource report on gfx950), counted in 16-byte accesses per lane.
// A lane may use 256 VGPRs in workgroups of up to 512 lanes and 128 in
// 1024-lane workgroups; more than 2 16-byte accesses a lane do not fit there.
template <int W, int T, int V>
constexpr int dyn_bwd_depth() {
    constexpr int U = (V * W + 7) / 8;
    if constexpr (T >= 1024) return U > 1 ? 1 : (W == 1 ? 2 : 3);
    if constexpr (U <= 1) return 4;
    if constexpr (U == 2) return 3;
    if constexpr (U == 3) return 2;
    return T >= 512 ? 1 : 2;
}

template <int W, int T, int V>
constexpr bool dyn_bwd_fits() {
    return T < 1024 || V * W <= 8 || (W == 8 && V == 2);
}

template <int W, int T, int V, bool LN>
hipError_t launch_bwd_dyn(const DynBwdArgs& a, hipStream_t stream) {
    constexpr int D = dyn_bwd_depth<W, T, V>();
    const int outs = LN ? 2 : 1;
    if (a.rows > 0) {
        if constexpr (LN) {
            hipLaunchKernelGGL((norm_bwd_dyn_rows_kernel<W, T, V, D, true, false>), dim3(a.grid),
                               dim3(dyn_block<T>()), 0, stream, a);
        } else {
            if (a.dres)
                hipLaunchKernelGGL((norm_bwd_dyn_rows_kernel<W, T, V, D, false, true>),
                                   dim3(a.grid), dim3(dyn_block<T>()), 0, stream, a);
            else
                hipLaunchKernelGGL((norm_bwd_dyn_rows_kernel<W, T, V, D, false, false>),
                                   dim3(a.grid), dim3(dyn_block<T>()), 0, stream, a);
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return launch_norm_colreduce(a.workspace, a.rows > 0 ? a.grid : 0, a.hidden,
                                 (int32_t)dyn_padded_hidden(a.hidden), outs, a.dweight, a.dbias,
                                 stream);
}

// Accesses per lane compiled for each width (the backward keeps column sums
// as well as the row ring in registers, so at most 4 16-byte accesses' worth
// of row data a lane).
template <int W>
using DynBwdVecs = std::conditional_t<W == 8, std::integer_sequence<int, 1, 2, 3, 4>,
                                      std::integer_sequence<int, 1, 2, 4, 8>>;

template <bool LN, int W, int T, int V>
void add_dyn_bwd_one(std::vector<DynBwdEntry>& v) {
    if constexpr (dyn_bwd_fits<W, T, V>())
        v.push_back({W, T, V, dyn_bwd_depth<W, T, V>(), &launch_bwd_dyn<W, T, V, LN>});
}

template <bool LN, int W, int T, int... Vs>
void add_dyn_bwd(std::vector<DynBwdEntry>& v, std::integer_sequence<int, Vs...>) {
    (add_dyn_bwd_one<LN, W, T, Vs>(v), ...);
}

template <bool LN, int W>
void add_dyn_bwd_w(std::vector<DynBwdEntry>& v) {
    add_dyn_bwd<LN, W, 8>(v, DynBwdVecs<W>{});
    add_dyn_bwd<LN, W, 16>(v, DynBwdVecs<W>{});
    add_dyn_bwd<LN, W, 32>(v, DynBwdVecs<W>{});
    add_dyn_bwd<LN, W, 64>(v, DynBwdVecs<W>{});
    add_dyn_bwd<LN, W, 128>(v, DynBwdVecs<W>{});
    add_dyn_bwd<LN, W, 256>(v, DynBwdVecs<W>{});
    add_dyn_bwd<LN, W, 512>(v, DynBwdVecs<W>{});
    add_dyn_bwd<LN, W, 1024>(v, DynBwdVecs<W>{});
}

template <bool LN>
std::vector<DynBwdEntry> build_dyn_bwd_table() {
    std::vector<DynBwdEntry> v;
    add_dyn_bwd_w<LN, 8>(v);
    add_dyn_bwd_w<LN, 4>(v);
    add_dyn_bwd_w<LN, 2>(v);
    add_dyn_bwd_w<LN, 1>(v);
    return v;
}

}  // namespace rownorm
