// Forward row-normalization kernels: fused residual-add + RMSNorm, RMSNorm,
// LayerNorm.  One row per T lanes, R rows per workgroup; the whole row stays
// in registers between the reduction and the normalize step, so every input
// byte is read from HBM once and every output byte written once ("inner
// persistent" normalization in "optimize inner persistent scheduler for
// static fusion", author description).
#pragma once

#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"

namespace rownorm {

// Sum of 8 per-element accumulators in a fixed tree.
__device__ __forceinline__ float tree8(const float (&a)[8]) {
    return ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
}

// The lane's V 16-byte vectors of a per-column parameter (weight or bias).
template <int V, int T>
__device__ __forceinline__ void load_params(u32x4 (&v)[V], const u32x4* __restrict__ p,
                                            int lane) {
#pragma unroll
    for (int b = 0; b < V; ++b) v[b] = p[lane + b * T];
}

// Each of the three kernels below comes in two variants that differ only in
// when the lanes load the weight (and bias): `*_kernel` issues them right
// after the row, before any arithmetic; `*_lw_kernel` ("late weights") only
// once the row's statistics are known, so the row's HBM loads are the only
// loads in flight until then.  Which one is faster depends on the shape and
// the batch (measured on MI355X: from 20 % faster to 8 % slower), so both are
// compiled and the launch choice picks one per shape and row count.

// ---------------------------------------------------------------------------
// Fused residual-add + RMSNorm ("optimize inner persistent scheduler for
// static fusion", changes walkthrough: the benchmarked op updates its residual
// input in place).  s = x + r in fp32; residual <- bf16(s);
// out <- bf16(s * rsqrt(mean(s^2) + eps) * w), with s re-derived from the
// x and r registers (the same fp32 sum) instead of re-read.
// ---------------------------------------------------------------------------
template <int H, int T, int R, bool LATE>
__device__ __forceinline__ void fused_add_rmsnorm_body(u32x4* out, u32x4* residual,
                                                       const u32x4* x,
                                                       const u32x4* __restrict__ weight,
                                                       int64_t rows, float eps) {
    using S = Shape<H, T, R>;
    constexpr int V = S::kVecs;
    __shared__ float red[S::kWaves > 1 ? R * S::kWaves : 1];

    const int lane = threadIdx.x % T;
    const int rib = threadIdx.x / T;
    const int64_t row = (int64_t)blockIdx.x * R + rib;
    const bool valid = row < rows;
    if constexpr (S::kWaves == 1) {
        if (!valid) return;  // whole wave, no barrier follows
    }
    const int64_t base = row * S::kRowVecs + lane;

    // Issue the whole row (x and r interleaved, in the order they are
    // consumed), then (early variant) the weight, before any arithmetic.
    u32x4 xv[V], rv[V], wv[V];
    if (valid) {
#pragma unroll
        for (int b = 0; b < V; ++b) {
            xv[b] = load_stream(x + base + b * T);
            rv[b] = load_stream(residual + base + b * T);
        }
    } else {
#pragma unroll
        for (int b = 0; b < V; ++b) xv[b] = rv[b] = u32x4{0, 0, 0, 0};
    }
    if constexpr (!LATE) load_params<V, T>(wv, weight, lane);
    issue_fence();

    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int b = 0; b < V; ++b) {
        float xf[8], rf[8], s[8];
        unpack8(xv[b], xf);
        unpack8(rv[b], rf);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            s[k] = xf[k] + rf[k];
            acc[k] += s[k] * s[k];
        }
        if (valid) store_stream(residual + base + b * T, pack8(s));
    }
    const float ss = row_sum<T>(tree8(acc), red + rib * S::kWaves, lane);
    const float rstd = fast_rsqrt(ss * (1.0f / H) + eps);
    if (!valid) return;
    if constexpr (LATE) load_params<V, T>(wv, weight, lane);
#pragma unroll
    for (int b = 0; b < V; ++b) {
        float xf[8], rf[8], wf[8], o[8];
        unpack8(xv[b], xf);
        unpack8(rv[b], rf);
        unpack8(wv[b], wf);
#pragma unroll
        for (int k = 0; k < 8; ++k) o[k] = (xf[k] + rf[k]) * rstd * wf[k];
        store_stream(out + base + b * T, pack8(o));
    }
}

// ---------------------------------------------------------------------------
// RMSNorm forward ("TMA inner persistent scheduler", description summary).
// ---------------------------------------------------------------------------
template <int H, int T, int R, bool LATE>
__device__ __forceinline__ void rmsnorm_fwd_body(u32x4* out, const u32x4* x,
                                                 const u32x4* __restrict__ weight, int64_t rows,
                                                 float eps) {
    using S = Shape<H, T, R>;
    constexpr int V = S::kVecs;
    __shared__ float red[S::kWaves > 1 ? R * S::kWaves : 1];

    const int lane = threadIdx.x % T;
    const int rib = threadIdx.x / T;
    const int64_t row = (int64_t)blockIdx.x * R + rib;
    const bool valid = row < rows;
    if constexpr (S::kWaves == 1) {
        if (!valid) return;
    }
    const int64_t base = row * S::kRowVecs + lane;

    u32x4 xv[V], wv[V];
    if (valid) {
#pragma unroll
        for (int b = 0; b < V; ++b) xv[b] = load_stream(x + base + b * T);
    } else {
#pragma unroll
        for (int b = 0; b < V; ++b) xv[b] = u32x4{0, 0, 0, 0};
    }
    if constexpr (!LATE) load_params<V, T>(wv, weight, lane);
    issue_fence();

    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int b = 0; b < V; ++b) {
        float xf[8];
        unpack8(xv[b], xf);
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] += xf[k] * xf[k];
    }
    const float ss = row_sum<T>(tree8(acc), red + rib * S::kWaves, lane);
    const float rstd = fast_rsqrt(ss * (1.0f / H) + eps);
    if (!valid) return;
    if constexpr (LATE) load_params<V, T>(wv, weight, lane);
#pragma unroll
    for (int b = 0; b < V; ++b) {
        float xf[8], wf[8], o[8];
        unpack8(xv[b], xf);
        unpack8(wv[b], wf);
#pragma unroll
        for (int k = 0; k < 8; ++k) o[k] = xf[k] * rstd * wf[k];
        store_stream(out + base + b * T, pack8(o));
    }
}

// ---------------------------------------------------------------------------
// LayerNorm forward with affine weight/bias ("TMA inner persistent
// scheduler", description summary).  Two-pass statistics: the mean first,
// then the sum of squared deviations from it, both over the row held in
// registers (the second pass costs no memory traffic).
// ---------------------------------------------------------------------------
template <int H, int T, int R, bool LATE>
__device__ __forceinline__ void layernorm_fwd_body(u32x4* y, float* mean_out, float* rstd_out,
                                                   const u32x4* x,
                                                   const u32x4* __restrict__ weight,
                                                   const u32x4* __restrict__ bias, int64_t rows,
                                                   float eps) {
    using S = Shape<H, T, R>;
    constexpr int V = S::kVecs;
    constexpr int kSlot = S::kWaves > 1 ? R * S::kWaves : 1;
    __shared__ float red[2 * kSlot];

    const int lane = threadIdx.x % T;
    const int rib = threadIdx.x / T;
    const int64_t row = (int64_t)blockIdx.x * R + rib;
    const bool valid = row < rows;
    if constexpr (S::kWaves == 1) {
        if (!valid) return;
    }
    const int64_t base = row * S::kRowVecs + lane;

    u32x4 xv[V], wv[V], bv[V];
    if (valid) {
#pragma unroll
        for (int b = 0; b < V; ++b) xv[b] = load_stream(x + base + b * T);
    } else {
#pragma unroll
        for (int b = 0; b < V; ++b) xv[b] = u32x4{0, 0, 0, 0};
    }
    if constexpr (!LATE) {
        load_params<V, T>(wv, weight, lane);
        load_params<V, T>(bv, bias, lane);
    }
    issue_fence();

    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int b = 0; b < V; ++b) {
        float xf[8];
        unpack8(xv[b], xf);
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] += xf[k];
    }
    const float mu = row_sum<T>(tree8(acc), red + rib * S::kWaves, lane) * (1.0f / H);

    float acc2[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int b = 0; b < V; ++b) {
        float xf[8];
        unpack8(xv[b], xf);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float d = xf[k] - mu;
            acc2[k] += d * d;
        }
    }
    const float var = row_sum<T>(tree8(acc2), red + kSlot + rib * S::kWaves, lane) * (1.0f / H);
    const float rstd = fast_rsqrt(var + eps);
    if (!valid) return;
    if constexpr (LATE) {
        load_params<V, T>(wv, weight, lane);
        load_params<V, T>(bv, bias, lane);
    }
    if (mean_out != nullptr && lane == 0) {
        mean_out[row] = mu;
        rstd_out[row] = rstd;
    }
#pragma unroll
    for (int b = 0; b < V; ++b) {
        float xf[8], wf[8], bf[8], o[8];
        unpack8(xv[b], xf);
        unpack8(wv[b], wf);
        unpack8(bv[b], bf);
#pragma unroll
        for (int k = 0; k < 8; ++k) o[k] = (xf[k] - mu) * rstd * wf[k] + bf[k];
        store_stream(y + base + b * T, pack8(o));
    }
}

#define ROWNORM_FWD_KERNELS(name, body, params, args)                                  \
    template <int H, int T, int R>                                                      \
    __global__ __launch_bounds__(T * R) void name##_kernel params {                      \
        body<H, T, R, false> args;                                                     \
    }                                                                                   \
    template <int H, int T, int R>                                                      \
    __global__ __launch_bounds__(T * R) void name##_lw_kernel params {                   \
        body<H, T, R, true> args;                                                      \
    }
ROWNORM_FWD_KERNELS(fused_add_rmsnorm, fused_add_rmsnorm_body,
                    (u32x4 * out, u32x4* residual, const u32x4* x,
                     const u32x4* __restrict__ weight, int64_t rows, float eps),
                    (out, residual, x, weight, rows, eps))
ROWNORM_FWD_KERNELS(rmsnorm_fwd, rmsnorm_fwd_body,
                    (u32x4 * out, const u32x4* x, const u32x4* __restrict__ weight,
                     int64_t rows, float eps),
                    (out, x, weight, rows, eps))
ROWNORM_FWD_KERNELS(layernorm_fwd, layernorm_fwd_body,
                    (u32x4 * y, float* mean_out, float* rstd_out, const u32x4* x,
                     const u32x4* __restrict__ weight, const u32x4* __restrict__ bias,
                     int64_t rows, float eps),
                    (y, mean_out, rstd_out, x, weight, bias, rows, eps))
#undef ROWNORM_FWD_KERNELS

// ---------------------------------------------------------------------------
// LayerNorm forward on a persistent grid: G workgroups of T lanes walk the
// rows blockIdx.x + i*G with a ring of D rows whose loads are in flight while
// the current row is reduced and stored, and keep the weight and bias in
// registers for the whole walk.  Same arithmetic as layernorm_fwd_kernel;
// measured 6-7 % faster on MI355X at 2048 rows of 4096-16384 (the two
// dependent reductions of a row no longer stall its workgroup's memory
// stream).  Rows past the end of a partial ring step go through zero-size
// buffer descriptors (zeros loaded, stores dropped), so the loop has no
// per-row branch around a memory access.
// ---------------------------------------------------------------------------
template <int H, int T, int D>
__global__ __launch_bounds__(T) void layernorm_fwd_ring_kernel(
    u32x4* y, float* mean_out, float* rstd_out, const u32x4* x,
    const u32x4* __restrict__ weight, const u32x4* __restrict__ bias, int64_t rows, float eps) {
    using S = Shape<H, T, 1>;
    constexpr int V = S::kVecs;
    __shared__ float red[2][S::kWaves];  // alternating slots: one barrier per reduction
    const int lane = threadIdx.x;
    u32x4 wv[V], bv[V];
#pragma unroll
    for (int b = 0; b < V; ++b) {
        wv[b] = weight[lane + b * T];
        bv[b] = bias[lane + b * T];
    }
    const int64_t G = gridDim.x;
    const int64_t first = blockIdx.x;
    const int64_t n = first < rows ? (rows - 1 - first) / G + 1 : 0;
    u32x4 ring[D][V];
#pragma unroll
    for (int d = 0; d < D; ++d) {
        const rsrc_t rx = row_rsrc(x, first + d * G, rows, H * 2);
#pragma unroll
        for (int b = 0; b < V; ++b) ring[d][b] = rload_stream(rx, (b * T + lane) * 16);
        issue_fence();
    }
    int slot = 0;
    for (int64_t i = 0; i < n; i += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int64_t r = first + (i + d) * G;
            float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
            for (int b = 0; b < V; ++b) {
                float xf[8];
                unpack8(ring[d][b], xf);
#pragma unroll
                for (int k = 0; k < 8; ++k) acc[k] += xf[k];
            }
            const float mu = row_sum<T>(tree8(acc), red[slot], lane) * (1.0f / H);
            slot ^= 1;
            float acc2[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
            for (int b = 0; b < V; ++b) {
                float xf[8];
                unpack8(ring[d][b], xf);
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const float dd = xf[k] - mu;
                    acc2[k] += dd * dd;
                }
            }
            const float var = row_sum<T>(tree8(acc2), red[slot], lane) * (1.0f / H);
            slot ^= 1;
            const float rstd = fast_rsqrt(var + eps);
            if (mean_out != nullptr && lane == 0 && r < rows) {
                mean_out[r] = mu;
                rstd_out[r] = rstd;
            }
            const rsrc_t ry = row_rsrc(y, r, rows, H * 2);
#pragma unroll
            for (int b = 0; b < V; ++b) {
                float xf[8], wf[8], bf[8], o[8];
                unpack8(ring[d][b], xf);
                unpack8(wv[b], wf);
                unpack8(bv[b], bf);
#pragma unroll
                for (int k = 0; k < 8; ++k) o[k] = (xf[k] - mu) * rstd * wf[k] + bf[k];
                rstore_stream(ry, (b * T + lane) * 16, pack8(o));
            }
            issue_fence();
            const rsrc_t rx = row_rsrc(x, r + D * G, rows, H * 2);
#pragma unroll
            for (int b = 0; b < V; ++b) ring[d][b] = rload_stream(rx, (b * T + lane) * 16);
            issue_fence();
        }
    }
}

// ---------------------------------------------------------------------------
// RMSNorm forward on the same persistent grid: the LayerNorm ring above with
// one reduction (the mean square) and no bias.  Same arithmetic as
// rmsnorm_fwd_kernel, so bitwise equal to it at the same lane count.  With the
// ring depth covering a workgroup's walk it measured 5-18 % faster than the
// one-row-per-lane-group kernels at hidden 12288-16384 from 512 rows and at
// hidden 8192 from 2048 rows (MI355X, 256 workgroups).
// ---------------------------------------------------------------------------
template <int H, int T, int D>
__global__ __launch_bounds__(T) void rmsnorm_fwd_ring_kernel(u32x4* y, const u32x4* x,
                                                             const u32x4* __restrict__ weight,
                                                             int64_t rows, float eps) {
    using S = Shape<H, T, 1>;
    constexpr int V = S::kVecs;
    __shared__ float red[2][S::kWaves];  // alternating slots: one barrier per reduction
    const int lane = threadIdx.x;
    u32x4 wv[V];
#pragma unroll
    for (int b = 0; b < V; ++b) wv[b] = weight[lane + b * T];
    const int64_t G = gridDim.x;
    const int64_t first = blockIdx.x;
    const int64_t n = first < rows ? (rows - 1 - first) / G + 1 : 0;
    u32x4 ring[D][V];
#pragma unroll
    for (int d = 0; d < D; ++d) {
        const rsrc_t rx = row_rsrc(x, first + d * G, rows, H * 2);
#pragma unroll
        for (int b = 0; b < V; ++b) ring[d][b] = rload_stream(rx, (b * T + lane) * 16);
        issue_fence();
    }
    int slot = 0;
    for (int64_t i = 0; i < n; i += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int64_t r = first + (i + d) * G;
            float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
            for (int b = 0; b < V; ++b) {
                float xf[8];
                unpack8(ring[d][b], xf);
#pragma unroll
                for (int k = 0; k < 8; ++k) acc[k] += xf[k] * xf[k];
            }
            const float ss = row_sum<T>(tree8(acc), red[slot], lane);
            slot ^= 1;
            const float rstd = fast_rsqrt(ss * (1.0f / H) + eps);
            const rsrc_t ry = row_rsrc(y, r, rows, H * 2);
#pragma unroll
            for (int b = 0; b < V; ++b) {
                float xf[8], wf[8], o[8];
                unpack8(ring[d][b], xf);
                unpack8(wv[b], wf);
#pragma unroll
                for (int k = 0; k < 8; ++k) o[k] = xf[k] * rstd * wf[k];
                rstore_stream(ry, (b * T + lane) * 16, pack8(o));
            }
            issue_fence();
            const rsrc_t rx = row_rsrc(x, r + D * G, rows, H * 2);
#pragma unroll
            for (int b = 0; b < V; ++b) ring[d][b] = rload_stream(rx, (b * T + lane) * 16);
            issue_fence();
        }
    }
}

// ---------------------------------------------------------------------------
// Launchers and the compile-time shape lists.
// ---------------------------------------------------------------------------
// Widest per-lane row buffer compiled: what stays within a lane's 256 VGPRs
// without spills on gfx950 (row vectors plus the weight, and bias, vectors).
struct OpFused {
    static constexpr int kMaxVecs = 16;  // x, r, w: 12 VGPRs per vector
};
struct OpRms {
    static constexpr int kMaxVecs = 16;  // x, w: 8 VGPRs per vector
};
struct OpLnFwd {
    static constexpr int kMaxVecs = 12;  // x, w, b: 12 VGPRs per vector
};

template <class Op, int H, int T, int R>
constexpr bool shape_ok() {
    return T % kWave == 0 && H % (8 * T) == 0 && H / (8 * T) <= Op::kMaxVecs &&
           T * R <= 1024;
}

template <class Op, int H, int T, int R, bool LATE>
hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)((a.rows + R - 1) / R));
    const dim3 block(T * R);
    u32x4* out = (u32x4*)a.out;
    const u32x4* x = (const u32x4*)a.x;
    const u32x4* w = (const u32x4*)a.weight;
    if constexpr (std::is_same_v<Op, OpFused>) {
        u32x4* res = (u32x4*)a.residual;
        if constexpr (LATE)
            hipLaunchKernelGGL((fused_add_rmsnorm_lw_kernel<H, T, R>), grid, block, 0, stream, out,
                               res, x, w, a.rows, a.eps);
        else
            hipLaunchKernelGGL((fused_add_rmsnorm_kernel<H, T, R>), grid, block, 0, stream, out,
                               res, x, w, a.rows, a.eps);
    } else if constexpr (std::is_same_v<Op, OpRms>) {
        if constexpr (LATE)
            hipLaunchKernelGGL((rmsnorm_fwd_lw_kernel<H, T, R>), grid, block, 0, stream, out, x, w,
                               a.rows, a.eps);
        else
            hipLaunchKernelGGL((rmsnorm_fwd_kernel<H, T, R>), grid, block, 0, stream, out, x, w,
                               a.rows, a.eps);
    } else {
        const u32x4* b = (const u32x4*)a.bias;
        if constexpr (LATE)
            hipLaunchKernelGGL((layernorm_fwd_lw_kernel<H, T, R>), grid, block, 0, stream, out,
                               a.mean, a.rstd, x, w, b, a.rows, a.eps);
        else
            hipLaunchKernelGGL((layernorm_fwd_kernel<H, T, R>), grid, block, 0, stream, out,
                               a.mean, a.rstd, x, w, b, a.rows, a.eps);
    }
    return hipGetLastError();
}

template <int H, int T, int D>
hipError_t launch_rms_ring(const FwdArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((rmsnorm_fwd_ring_kernel<H, T, D>), dim3(a.grid), dim3(T), 0, stream,
                       (u32x4*)a.out, (const u32x4*)a.x, (const u32x4*)a.weight, a.rows, a.eps);
    return hipGetLastError();
}

template <int H, int T, int D>
hipError_t launch_ln_ring(const FwdArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((layernorm_fwd_ring_kernel<H, T, D>), dim3(a.grid), dim3(T), 0, stream,
                       (u32x4*)a.out, a.mean, a.rstd, (const u32x4*)a.x, (const u32x4*)a.weight,
                       (const u32x4*)a.bias, a.rows, a.eps);
    return hipGetLastError();
}

// Ring depths of the LayerNorm ring kernels: each ring shape is compiled at
// depths 2, 4 and 8, where the lane's registers hold that depth without
// spills (from gfx950's resource report: about 20 VGPRs per 16-byte vector
// for the held weight and bias and the arithmetic, 4 per vector for each ring
// row, 24 besides; 128 VGPRs a lane in 1024-lane workgroups, 256 otherwise).
// The launch picks a depth per call from the length of a workgroup's walk.
template <int H, int T, int D>
constexpr bool ln_ring_fits() {
    constexpr int V = H / (8 * T);
    return 20 * V + 4 * V * D + 24 <= (T >= 1024 ? 128 : 256);
}
// RMSNorm's ring holds the weight only (about 12 VGPRs per vector besides the
// ring rows).  Compiled from hidden 8192 and 256 lanes, where it is used.
template <int H, int T, int D>
constexpr bool rms_ring_fits() {
    constexpr int V = H / (8 * T);
    return H >= 8192 && T >= 256 && 12 * V + 4 * V * D + 24 <= (T >= 1024 ? 128 : 256);
}

// (lanes per row, rows per workgroup) pairs tried for every hidden size;
// pairs that do not divide the row or exceed the register budget are skipped
// at compile time.
template <int T, int R>
struct LR {};
using FwdShapeList = std::tuple<LR<64, 1>, LR<64, 2>, LR<64, 4>, LR<64, 8>, LR<128, 1>,
                                LR<128, 2>, LR<128, 4>, LR<256, 1>, LR<256, 2>, LR<512, 1>,
                                LR<512, 2>, LR<1024, 1>>;

template <class Op, int H, int T, int R>
void add_fwd_entry(std::vector<FwdEntry>& v, LR<T, R>) {
    if constexpr (shape_ok<Op, H, T, R>())
        v.push_back({H, T, R, &launch_fwd<Op, H, T, R, false>, 0, &launch_fwd<Op, H, T, R, true>});
    // LayerNorm also gets persistent ring kernels per lane count, one per depth
    if constexpr (std::is_same_v<Op, OpLnFwd> && R == 1 && H % (8 * T) == 0 && T % kWave == 0 &&
                  H >= 2048) {
        if constexpr (ln_ring_fits<H, T, 2>())
            v.push_back({H, T, 1, &launch_ln_ring<H, T, 2>, 2, nullptr});
        if constexpr (ln_ring_fits<H, T, 4>())
            v.push_back({H, T, 1, &launch_ln_ring<H, T, 4>, 4, nullptr});
        if constexpr (ln_ring_fits<H, T, 8>())
            v.push_back({H, T, 1, &launch_ln_ring<H, T, 8>, 8, nullptr});
    }
    // RMSNorm: the same per-depth ring kernels where rms_ring_fits
    if constexpr (std::is_same_v<Op, OpRms> && R == 1 && H % (8 * T) == 0 && T % kWave == 0) {
        if constexpr (rms_ring_fits<H, T, 2>())
            v.push_back({H, T, 1, &launch_rms_ring<H, T, 2>, 2, nullptr});
        if constexpr (rms_ring_fits<H, T, 4>())
            v.push_back({H, T, 1, &launch_rms_ring<H, T, 4>, 4, nullptr});
        if constexpr (rms_ring_fits<H, T, 8>())
            v.push_back({H, T, 1, &launch_rms_ring<H, T, 8>, 8, nullptr});
    }
}

template <class Op, int H, class... Ls>
void add_fwd_entries_h(std::vector<FwdEntry>& v, std::tuple<Ls...>) {
    (add_fwd_entry<Op, H>(v, Ls{}), ...);
}

template <class Op>
std::vector<FwdEntry> build_fwd_table() {
    std::vector<FwdEntry> v;
    add_fwd_entries_h<Op, 1024>(v, FwdShapeList{});
    add_fwd_entries_h<Op, 2048>(v, FwdShapeList{});
    add_fwd_entries_h<Op, 4096>(v, FwdShapeList{});
    add_fwd_entries_h<Op, 8192>(v, FwdShapeList{});
    add_fwd_entries_h<Op, 12288>(v, FwdShapeList{});
    add_fwd_entries_h<Op, 16384>(v, FwdShapeList{});
    return v;
}

}  // namespace rownorm
