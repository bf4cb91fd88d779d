// Backward kernels for rows too wide for the register-resident layout
// (hidden above 16384): the LDS-staged persistent buffer of "TMA inner
// persistent scheduler" (description summary: rows staged in shared memory
// when registers cannot hold them), on gfx950's buffer-to-LDS loads instead of
// TMA.  Arithmetic per row is that of the other backward kernels ("Llu/ln
// bwd", author note: the combined inner + outer reduction):
//   LayerNorm: xhat = (x - mean) rstd, g = dy w, c1 = mean_j g, c2 = mean_j g xhat,
//              dx = rstd (g - c1 - xhat c2); pw += dy xhat, pb += dy;
//   RMSNorm:   rstd = rsqrt(mean_j x^2 + eps), dx = rstd g - rstd^3 mean_j(g x) x
//              [+ dres]; pw += dy x rstd.
//
// A workgroup of 512 lanes (8 waves) walks rows blockIdx.x, + G, ... one at a
// time.  Lane t holds accesses b*512 + t (16 bytes, 8 columns each) for b < V,
// hidden <= 4096 V (V = 5 ... 8: hidden above 16384, up to 32768).  What
// bounds the width is the column sums: every lane keeps pw (and pb) for its
// columns in registers across all its rows, 8 V (16 V) floats; 512-lane
// workgroups get 256 registers a lane (1024-lane ones 128, too few for
// LayerNorm's 64 sums a lane at 32768).  So the row itself lives in LDS
// (2 V x 8 KiB, 128 KiB at 32768): x and dy go from
// HBM straight into LDS (buffer loads with the LDS bit: each wave's 64 lanes
// write 64 consecutive 16-byte slots, which are exactly the slots those lanes
// read back, so no barrier is needed) and never occupy registers; the weights
// stay in registers packed as bf16 (4 per access); dres (fused op) is loaded
// after the reduction.  One two-value reduction over the 16 waves (LDS, one
// barrier) per row.  A single wide row keeps 2 V x 8 KiB of loads in flight
// per workgroup, enough to cover the memory latency without a ring of rows.
// At the end each workgroup writes one slab of [G][outs][padded] column sums
// for the shared column-reduce kernel.
#pragma once

#include <type_traits>
#include <utility>

#include "dyn_common.hpp"
#include "launch.hpp"

namespace rownorm {

constexpr int kWideLanes = kWideBwdLanes;
// s_waitcnt operand (gfx9 encoding: vmcnt bits 15:14 and 3:0, expcnt 6:4,
// lgkmcnt 11:8) waiting for LDS operations only: vmcnt 63, expcnt 7, lgkmcnt 0.
constexpr int kWaitLdsOnly = 0xC07F;

// The value of v, opaque to the optimizer (emits no instruction).
__device__ __forceinline__ int opaque_lane(int v) {
    asm volatile("" : "+v"(v));
    return v;
}

template <int V, bool LN, bool DRES>
__global__ __launch_bounds__(kWideLanes) void norm_bwd_wide_kernel(DynBwdArgs a) {
    constexpr int T = kWideLanes;
    __shared__ u32x4 xs[V * T], ds[V * T];      // the row's x and dy, 16 bytes per slot
    __shared__ float red[2 * 2 * (T / kWave)];  // two alternating two-value slots
    const int lane = threadIdx.x;
    const int wave_base = lane & ~(kWave - 1);
    const int h = a.hidden;
    const float inv_h = 1.0f / (float)h;
    // the weights stay in registers for the whole walk, packed (4 per access)
    const rsrc_t rw = row_rsrc_ld(a.weight, 0, 1, 0, h * 2);
    u32x4 wv[V];
#pragma unroll
    for (int b = 0; b < V; ++b) wv[b] = aload<8, 0>(rw, (b * T + lane) * 16);

    float pw[V][8], pb[LN ? V : 1][8];
#pragma unroll
    for (int b = 0; b < V; ++b)
#pragma unroll
        for (int k = 0; k < 8; ++k) pw[b][k] = 0.0f;
    if constexpr (LN) {
#pragma unroll
        for (int b = 0; b < V; ++b)
#pragma unroll
            for (int k = 0; k < 8; ++k) pb[b][k] = 0.0f;
    }

    const int64_t G = gridDim.x;
    const int64_t first = blockIdx.x;
    const int64_t n = first < a.rows ? (a.rows - 1 - first) / G + 1 : 0;
    int parity = 0;
    for (int64_t i = 0; i < n; ++i) {
        const int64_t row = opaque_row(first + i * G);
        // lane offsets recomputed every row (an opaque lane index), not hoisted
        // out of the loop into registers held for the whole walk
        const int l = opaque_lane(lane);
        const rsrc_t rx = row_rsrc_ld(a.x, row, a.rows, a.ld_x * 2, h * 2);
        const rsrc_t rd = row_rsrc_ld(a.dy, row, a.rows, a.ld_dy * 2, h * 2);
        // x, dy -> LDS (lane t's slot b is [b*T + t]; the wave writes its 64 slots)
#pragma unroll
        for (int b = 0; b < V; ++b) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rx, (__attribute__((address_space(3))) void*)&xs[b * T + wave_base], 16,
                (b * T + l) * 16, 0, 0, kCachePolicyNT);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rd, (__attribute__((address_space(3))) void*)&ds[b * T + wave_base], 16,
                (b * T + l) * 16, 0, 0, kCachePolicyNT);
        }
        float mean = 0.0f, rstd_in = 0.0f;
        if constexpr (LN) {
            mean = rload_f32(row_rsrc_ld(a.mean, row, a.rows, 4, 4), 0);
            rstd_in = rload_f32(row_rsrc_ld(a.rstd, row, a.rows, 4, 4), 0);
        }
        __builtin_amdgcn_s_waitcnt(0);  // the row's loads, the LDS writes included

        // the row's two sums (an access past the row's end, in the last b, is
        // left out whatever its LDS slot holds; hidden is a multiple of 8, so
        // an access is wholly inside the row or wholly past it)
        float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
        for (int b = 0; b < V; ++b) {
            const bool in_row = (b * T + l) * 8 < h;
            float xf[8], df[8], wf[8];
            unpack8(xs[b * T + l], xf);
            unpack8(ds[b * T + l], df);
            unpack8(wv[b], wf);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                xf[k] = in_row ? xf[k] : 0.0f;
                df[k] = in_row ? df[k] : 0.0f;
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                if constexpr (LN) {
                    const float xh = (xf[k] - mean) * rstd_in;
                    const float g = df[k] * wf[k];
                    s1 += g;
                    s2 += g * xh;
                } else {
                    s1 += xf[k] * xf[k];
                    s2 += df[k] * wf[k] * xf[k];
                }
            }
        }
        row_sum2<T>(s1, s2, red + parity * (2 * (T / kWave)), lane);
        parity ^= 1;
        // the second pass re-reads x, dy (LDS) and the weights (cache) instead
        // of keeping the first pass's values live across the reduction: an
        // opaque copy of the lane index keeps the compiler from merging them
        const int t = opaque_lane(lane);

        const rsrc_t rdx = row_rsrc_ld(a.dx, row, a.rows, a.ld_dx * 2, h * 2);
        rsrc_t rr = rdx;
        if constexpr (DRES) rr = row_rsrc_ld(a.dres, row, a.rows, a.ld_dres * 2, h * 2);
        if constexpr (LN) {
            const float c1 = s1 * inv_h, c2 = s2 * inv_h;
#pragma unroll
            for (int b = 0; b < V; ++b) {
                float xf[8], df[8], wf[8], o[8];
                unpack8(xs[b * T + t], xf);
                unpack8(ds[b * T + t], df);
                unpack8(wv[b], wf);
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const float xh = (xf[k] - mean) * rstd_in;
                    o[k] = rstd_in * (df[k] * wf[k] - c1 - xh * c2);
                    pw[b][k] += df[k] * xh;
                    pb[b][k] += df[k];
                }
                astore<8, kCachePolicyNT>(rdx, (b * T + lane) * 16, pack8(o));
            }
        } else {
            // a row past the end must add exactly nothing, also at eps = 0
            const float rstd = row < a.rows ? fast_rsqrt(s1 * inv_h + a.eps) : 0.0f;
            const float coef = rstd * rstd * rstd * s2 * inv_h;
            u32x4 dr[DRES ? V : 1];
            if constexpr (DRES) {
#pragma unroll
                for (int b = 0; b < V; ++b) dr[b] = aload<8, kCachePolicyNT>(rr, (b * T + lane) * 16);
            }
#pragma unroll
            for (int b = 0; b < V; ++b) {
                float xf[8], df[8], wf[8], o[8];
                unpack8(xs[b * T + t], xf);
                unpack8(ds[b * T + t], df);
                unpack8(wv[b], wf);
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    o[k] = rstd * (df[k] * wf[k]) - coef * xf[k];
                    pw[b][k] += df[k] * (xf[k] * rstd);
                }
                if constexpr (DRES) {
                    float rf[8];
                    unpack8(dr[b], rf);
#pragma unroll
                    for (int k = 0; k < 8; ++k) o[k] += rf[k];
                }
                astore<8, kCachePolicyNT>(rdx, (b * T + lane) * 16, pack8(o));
            }
        }
        // the next row's x may land in LDS only after this row's reads of it
        // are done (the dx stores may still be in flight)
        __builtin_amdgcn_s_waitcnt(kWaitLdsOnly);
    }

    const int64_t padded = dyn_padded_hidden(h);
    float* slab = a.workspace + (int64_t)blockIdx.x * (LN ? 2 : 1) * padded;
#pragma unroll
    for (int b = 0; b < V; ++b) {
        const int col = (b * T + lane) * 8;
        if (col < h) {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                slab[col + k] = pw[b][k];
                if constexpr (LN) slab[padded + col + k] = pb[b][k];
            }
        }
    }
}

template <int V, bool LN>
hipError_t launch_bwd_wide(const DynBwdArgs& a, hipStream_t stream) {
    const int outs = LN ? 2 : 1;
    if (a.rows > 0) {
        if constexpr (LN) {
            hipLaunchKernelGGL((norm_bwd_wide_kernel<V, true, false>), dim3(a.grid),
                               dim3(kWideLanes), 0, stream, a);
        } else {
            if (a.dres)
                hipLaunchKernelGGL((norm_bwd_wide_kernel<V, false, true>), dim3(a.grid),
                                   dim3(kWideLanes), 0, stream, a);
            else
                hipLaunchKernelGGL((norm_bwd_wide_kernel<V, false, false>), dim3(a.grid),
                                   dim3(kWideLanes), 0, stream, a);
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return launch_norm_colreduce(a.workspace, a.rows > 0 ? a.grid : 0, a.hidden,
                                 (int32_t)dyn_padded_hidden(a.hidden), outs, a.dweight, a.dbias,
                                 stream);
}

}  // namespace rownorm
