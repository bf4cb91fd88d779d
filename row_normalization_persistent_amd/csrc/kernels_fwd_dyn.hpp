// Forward kernels of the run-time-hidden path (layout and masking rules in
// dyn_common.hpp).  Same arithmetic as the compiled-hidden kernels: the fused
// residual-add + RMSNorm ("optimize inner persistent scheduler for static
// fusion", author description and changes walkthrough), RMSNorm and LayerNorm
// ("TMA inner persistent scheduler", description summary); hidden, the row
// strides and 1/hidden are kernel arguments instead of constants.
//
// Template parameters: W elements per access, T lanes per row, V accesses per
// lane, K rows per lane group.  A workgroup of dyn_block<T>() lanes holds
// R = block / T lane groups and R*K rows.
#pragma once

#include <type_traits>
#include <utility>

#include "dyn_common.hpp"
#include "launch.hpp"

namespace rownorm {

template <int W, int T>
__device__ __forceinline__ int dyn_off(int b, int lane) { return (b * T + lane) * (2 * W); }

// The lane's V accesses of a per-column parameter (weight or bias).
template <int W, int T, int V>
__device__ __forceinline__ void dyn_load_params(raw_t<W> (&v)[V], rsrc_t r, int lane) {
#pragma unroll
    for (int b = 0; b < V; ++b) v[b] = aload<W, 0>(r, dyn_off<W, T>(b, lane));
}

// K rows per lane group (K > 1 only for rows narrower than a wave, which
// reduce without LDS): the group issues the loads of all K rows before the
// first reduction.  Rows of workgroup k: k*R*K + j*R + g for j < K
// (consecutive groups take consecutive rows).  Addressing: one descriptor per
// row for rows of >= 64 lanes, one per workgroup for narrower rows
// (dyn_common.hpp, rows_rsrc / set_off).
template <int T, int K>
struct RowSet {
    static constexpr int R = dyn_block<T>() / T;
    static_assert(K == 1 || T < kWave, "several rows per lane group only without LDS");
    int64_t first, span;
    __device__ __forceinline__ explicit RowSet(int g) {
        if constexpr (T < kWave) {
            first = (int64_t)blockIdx.x * (R * K);
            span = R * K;
        } else {
            first = (int64_t)blockIdx.x * R + g;
            span = 1;
        }
    }
    __device__ __forceinline__ int local(int j, int g) const {
        if constexpr (T < kWave) return j * R + g;
        else return 0;
    }
    __device__ __forceinline__ int64_t row(int j, int g) const { return first + local(j, g); }
    __device__ __forceinline__ rsrc_t rsrc(const void* base, int64_t rows, int64_t ld,
                                           int hidden) const {
        return rows_rsrc<T>(base, first, span, rows, ld, hidden, 2);
    }
};

template <int W, int T>
__device__ __forceinline__ int acc_off(int local, int b, int lane, int64_t ld, int hidden) {
    return set_off<T>(local, (b * T + lane) * W, ld, hidden, 2);
}

// LATE: the weight (and bias) loads are issued once the first row's
// statistics are known instead of right behind the rows' loads (the
// `*_lw_kernel` variants; kernels_fwd.hpp describes the trade-off).
template <int W, int T, int V, int K, bool LATE>
__device__ __forceinline__ void fused_add_rmsnorm_dyn_body(const DynFwdArgs& a) {
    __shared__ float red[dyn_red_floats<T>()];
    const int lane = threadIdx.x % T;
    const int g = uniform_group<T>(threadIdx.x / T);
    const RowSet<T, K> set(g);
    const int h = a.hidden;
    const rsrc_t rx = set.rsrc(a.x, a.rows, a.ld_x, h);
    const rsrc_t rr = set.rsrc(a.residual, a.rows, a.ld_res, h);
    const rsrc_t ro = set.rsrc(a.out, a.rows, a.ld_out, h);
    const rsrc_t rw = row_rsrc_ld(a.weight, 0, 1, 0, h * 2);
    raw_t<W> xv[K][V], rv[K][V], wv[V];
#pragma unroll
    for (int j = 0; j < K; ++j) {
        const int l = set.local(j, g);
#pragma unroll
        for (int b = 0; b < V; ++b) {
            xv[j][b] = aload<W, kCachePolicyNT>(rx, acc_off<W, T>(l, b, lane, a.ld_x, h));
            rv[j][b] = aload<W, kCachePolicyNT>(rr, acc_off<W, T>(l, b, lane, a.ld_res, h));
        }
    }
    if constexpr (!LATE) dyn_load_params<W, T, V>(wv, rw, lane);
    issue_fence();
#pragma unroll
    for (int j = 0; j < K; ++j) {
        const int l = set.local(j, g);
        float acc = 0.0f;
#pragma unroll
        for (int b = 0; b < V; ++b) {
            float xf[W], rf[W], sv[W];
            aunpack<W>(xv[j][b], xf);
            aunpack<W>(rv[j][b], rf);
#pragma unroll
            for (int k = 0; k < W; ++k) {
                sv[k] = xf[k] + rf[k];
                acc += sv[k] * sv[k];  // accesses past the row's end are 0 + 0
            }
            astore<W, kCachePolicyNT>(rr, acc_off<W, T>(l, b, lane, a.ld_res, h), apack<W>(sv));
        }
        const float ss = dyn_row_sum<T>(acc, red + g * (T / kWave), lane);
        const float rstd = fast_rsqrt(ss / (float)h + a.eps);
        if (LATE && j == 0) dyn_load_params<W, T, V>(wv, rw, lane);
#pragma unroll
        for (int b = 0; b < V; ++b) {
            float xf[W], rf[W], wf[W], o[W];
            aunpack<W>(xv[j][b], xf);
            aunpack<W>(rv[j][b], rf);
            aunpack<W>(wv[b], wf);
#pragma unroll
            for (int k = 0; k < W; ++k) o[k] = (xf[k] + rf[k]) * rstd * wf[k];
            astore<W, kCachePolicyNT>(ro, acc_off<W, T>(l, b, lane, a.ld_out, h), apack<W>(o));
        }
    }
}

template <int W, int T, int V, int K, bool LATE>
__device__ __forceinline__ void rmsnorm_fwd_dyn_body(const DynFwdArgs& a) {
    __shared__ float red[dyn_red_floats<T>()];
    const int lane = threadIdx.x % T;
    const int g = uniform_group<T>(threadIdx.x / T);
    const RowSet<T, K> set(g);
    const int h = a.hidden;
    const rsrc_t rx = set.rsrc(a.x, a.rows, a.ld_x, h);
    const rsrc_t ro = set.rsrc(a.out, a.rows, a.ld_out, h);
    const rsrc_t rw = row_rsrc_ld(a.weight, 0, 1, 0, h * 2);
    raw_t<W> xv[K][V], wv[V];
#pragma unroll
    for (int j = 0; j < K; ++j) {
        const int l = set.local(j, g);
#pragma unroll
        for (int b = 0; b < V; ++b)
            xv[j][b] = aload<W, kCachePolicyNT>(rx, acc_off<W, T>(l, b, lane, a.ld_x, h));
    }
    if constexpr (!LATE) dyn_load_params<W, T, V>(wv, rw, lane);
    issue_fence();
#pragma unroll
    for (int j = 0; j < K; ++j) {
        const int l = set.local(j, g);
        float acc = 0.0f;
#pragma unroll
        for (int b = 0; b < V; ++b) {
            float xf[W];
            aunpack<W>(xv[j][b], xf);
#pragma unroll
            for (int k = 0; k < W; ++k) acc += xf[k] * xf[k];
        }
        const float ss = dyn_row_sum<T>(acc, red + g * (T / kWave), lane);
        const float rstd = fast_rsqrt(ss / (float)h + a.eps);
        if (LATE && j == 0) dyn_load_params<W, T, V>(wv, rw, lane);
#pragma unroll
        for (int b = 0; b < V; ++b) {
            float xf[W], wf[W], o[W];
            aunpack<W>(xv[j][b], xf);
            aunpack<W>(wv[b], wf);
#pragma unroll
            for (int k = 0; k < W; ++k) o[k] = xf[k] * rstd * wf[k];
            astore<W, kCachePolicyNT>(ro, acc_off<W, T>(l, b, lane, a.ld_out, h), apack<W>(o));
        }
    }
}

template <int W, int T, int V, int K, bool LATE>
__device__ __forceinline__ void layernorm_fwd_dyn_body(const DynFwdArgs& a) {
    constexpr int kRed = dyn_red_floats<T>();
    __shared__ float red[2 * kRed];  // mean and variance use different slots: one barrier each
    const int lane = threadIdx.x % T;
    const int g = uniform_group<T>(threadIdx.x / T);
    const RowSet<T, K> set(g);
    const int h = a.hidden;
    const rsrc_t rx = set.rsrc(a.x, a.rows, a.ld_x, h);
    const rsrc_t ry = set.rsrc(a.out, a.rows, a.ld_out, h);
    const rsrc_t rw = row_rsrc_ld(a.weight, 0, 1, 0, h * 2);
    const rsrc_t rbias = row_rsrc_ld(a.bias, 0, 1, 0, h * 2);
    raw_t<W> xv[K][V], wv[V], bv[V];
#pragma unroll
    for (int j = 0; j < K; ++j) {
        const int l = set.local(j, g);
#pragma unroll
        for (int b = 0; b < V; ++b)
            xv[j][b] = aload<W, kCachePolicyNT>(rx, acc_off<W, T>(l, b, lane, a.ld_x, h));
    }
    if constexpr (!LATE) {
        dyn_load_params<W, T, V>(wv, rw, lane);
        dyn_load_params<W, T, V>(bv, rbias, lane);
    }
    issue_fence();
    const float inv_h = 1.0f / (float)h;
#pragma unroll
    for (int j = 0; j < K; ++j) {
        const int l = set.local(j, g);
        const int64_t row = set.row(j, g);
        float acc = 0.0f;
#pragma unroll
        for (int b = 0; b < V; ++b) {
            float xf[W];
            aunpack<W>(xv[j][b], xf);
#pragma unroll
            for (int k = 0; k < W; ++k) acc += xf[k];
        }
        const float mu = dyn_row_sum<T>(acc, red + g * (T / kWave), lane) * inv_h;
        float acc2 = 0.0f;
#pragma unroll
        for (int b = 0; b < V; ++b) {
            // an access past the row's end holds zeros, but (0 - mu)^2 must not count
            const bool in_row = (b * T + lane) * W < h;
            float xf[W];
            aunpack<W>(xv[j][b], xf);
#pragma unroll
            for (int k = 0; k < W; ++k) {
                const float d = in_row ? xf[k] - mu : 0.0f;
                acc2 += d * d;
            }
        }
        const float var = dyn_row_sum<T>(acc2, red + kRed + g * (T / kWave), lane) * inv_h;
        const float rstd = fast_rsqrt(var + a.eps);
        if (LATE && j == 0) {
            dyn_load_params<W, T, V>(wv, rw, lane);
            dyn_load_params<W, T, V>(bv, rbias, lane);
        }
        if (a.mean != nullptr && lane == 0 && row < a.rows) {
            a.mean[row] = mu;
            a.rstd[row] = rstd;
        }
#pragma unroll
        for (int b = 0; b < V; ++b) {
            float xf[W], wf[W], bf[W], o[W];
            aunpack<W>(xv[j][b], xf);
            aunpack<W>(wv[b], wf);
            aunpack<W>(bv[b], bf);
#pragma unroll
            for (int k = 0; k < W; ++k) o[k] = (xf[k] - mu) * rstd * wf[k] + bf[k];
            astore<W, kCachePolicyNT>(ry, acc_off<W, T>(l, b, lane, a.ld_out, h), apack<W>(o));
        }
    }
}

#define ROWNORM_DYN_FWD_KERNELS(name)                                                  \
    template <int W, int T, int V, int K>                                               \
    __global__ __launch_bounds__(dyn_block<T>()) void name##_dyn_kernel(DynFwdArgs a) {   \
        name##_dyn_body<W, T, V, K, false>(a);                                          \
    }                                                                                   \
    template <int W, int T, int V, int K>                                               \
    __global__ __launch_bounds__(dyn_block<T>()) void name##_dyn_lw_kernel(DynFwdArgs a) { \
        name##_dyn_body<W, T, V, K, true>(a);                                           \
    }
ROWNORM_DYN_FWD_KERNELS(fused_add_rmsnorm)
ROWNORM_DYN_FWD_KERNELS(rmsnorm_fwd)
ROWNORM_DYN_FWD_KERNELS(layernorm_fwd)
#undef ROWNORM_DYN_FWD_KERNELS

struct OpFusedDyn {};
struct OpRmsDyn {};
struct OpLnFwdDyn {};

template <class Op, int W, int T, int V, int K, bool LATE>
hipError_t launch_fwd_dyn(const DynFwdArgs& a, hipStream_t stream) {
    constexpr int RK = dyn_block<T>() / T * K;
    const dim3 grid((unsigned)((a.rows + RK - 1) / RK));
    const dim3 block(dyn_block<T>());
    if constexpr (std::is_same_v<Op, OpFusedDyn>) {
        if constexpr (LATE)
            hipLaunchKernelGGL((fused_add_rmsnorm_dyn_lw_kernel<W, T, V, K>), grid, block, 0,
                               stream, a);
        else
            hipLaunchKernelGGL((fused_add_rmsnorm_dyn_kernel<W, T, V, K>), grid, block, 0, stream,
                               a);
    } else if constexpr (std::is_same_v<Op, OpRmsDyn>) {
        if constexpr (LATE)
            hipLaunchKernelGGL((rmsnorm_fwd_dyn_lw_kernel<W, T, V, K>), grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL((rmsnorm_fwd_dyn_kernel<W, T, V, K>), grid, block, 0, stream, a);
    } else {
        if constexpr (LATE)
            hipLaunchKernelGGL((layernorm_fwd_dyn_lw_kernel<W, T, V, K>), grid, block, 0, stream,
                               a);
        else
            hipLaunchKernelGGL((layernorm_fwd_dyn_kernel<W, T, V, K>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

// Accesses per lane compiled for each width: every count up to 8 for 16-byte
// accesses, powers of two for the narrower ones (rarer layouts, where the
// host rounds the count up and the extra accesses fall past the row's end).
template <int W>
using DynVecs = std::conditional_t<W == 8, std::integer_sequence<int, 1, 2, 3, 4, 5, 6, 7, 8>,
                                   std::integer_sequence<int, 1, 2, 4, 8>>;

// LayerNorm keeps x, weight and bias in registers; at 1024 lanes (128 VGPRs a
// lane) more than 6 16-byte accesses per lane would spill.
template <class Op, int W, int T, int V>
constexpr bool dyn_fwd_fits() {
    return !(std::is_same_v<Op, OpLnFwdDyn> && T == 1024 && V * W > 48);
}

// Rows per lane group compiled: 1 everywhere; also 2 and 4 for rows of at
// most two accesses a lane on fewer than 64 lanes (small rows, whose workgroups
// would otherwise keep too few bytes in flight).
template <class Op, int W, int T, int V>
void add_dyn_fwd_one(std::vector<DynFwdEntry>& v) {
    if constexpr (dyn_fwd_fits<Op, W, T, V>()) {
        v.push_back({W, T, V, &launch_fwd_dyn<Op, W, T, V, 1, false>, 1,
                     &launch_fwd_dyn<Op, W, T, V, 1, true>});
        if constexpr (T < kWave && V <= 2) {
            v.push_back({W, T, V, &launch_fwd_dyn<Op, W, T, V, 2, false>, 2,
                         &launch_fwd_dyn<Op, W, T, V, 2, true>});
            v.push_back({W, T, V, &launch_fwd_dyn<Op, W, T, V, 4, false>, 4,
                         &launch_fwd_dyn<Op, W, T, V, 4, true>});
        }
    }
}

template <class Op, int W, int T, int... Vs>
void add_dyn_fwd(std::vector<DynFwdEntry>& v, std::integer_sequence<int, Vs...>) {
    (add_dyn_fwd_one<Op, W, T, Vs>(v), ...);
}

template <class Op, int W>
void add_dyn_fwd_w(std::vector<DynFwdEntry>& v) {
    add_dyn_fwd<Op, W, 8>(v, DynVecs<W>{});
    add_dyn_fwd<Op, W, 16>(v, DynVecs<W>{});
    add_dyn_fwd<Op, W, 32>(v, DynVecs<W>{});
    add_dyn_fwd<Op, W, 64>(v, DynVecs<W>{});
    add_dyn_fwd<Op, W, 128>(v, DynVecs<W>{});
    add_dyn_fwd<Op, W, 256>(v, DynVecs<W>{});
    add_dyn_fwd<Op, W, 512>(v, DynVecs<W>{});
    add_dyn_fwd<Op, W, 1024>(v, DynVecs<W>{});
}

template <class Op>
std::vector<DynFwdEntry> build_dyn_fwd_table() {
    std::vector<DynFwdEntry> v;
    add_dyn_fwd_w<Op, 8>(v);
    add_dyn_fwd_w<Op, 4>(v);
    add_dyn_fwd_w<Op, 2>(v);
    add_dyn_fwd_w<Op, 1>(v);
    return v;
}

}  // namespace rownorm
