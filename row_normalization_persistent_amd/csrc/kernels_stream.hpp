// Rows too wide for one workgroup's registers and LDS: the streamed fallback
// of the persistent buffer.  "TMA inner persistent scheduler" (description
// summary) keeps the row in shared memory when registers cannot hold it; a row
// of more than 65536 bf16 values (fused add + RMSNorm, RMSNorm), 49152
// (LayerNorm forward) or 32768 (the backward operations, whose per-column
// sums also live on chip) fits neither, so these kernels read it twice: once
// for the row's reduction and once more, from the Infinity Cache while the
// rows in flight fit there, for the normalized output.  16-byte accesses
// only (hidden a multiple of 8, every row stride too, 16-byte-aligned
// pointers), any such hidden up to 2^20.
//
// Forward (stream_fwd_kernel, 1024 lanes, workgroups walk the rows g, g + G,
// ...): pass 1 streams the row for its statistic -- sum s^2 (s = x + r for
// the fused op), or for LayerNorm each lane's count, sum and centered sum of
// squares, merged access by access with the pairwise update of a sum of
// squared deviations (Chan, Golub & LeVeque), then combined over the lanes
// exactly as the row split combines its chunks:
//   mean = sum_l S_l / H,  M2 = sum_l M2_l + n_l (S_l / n_l - mean)^2;
// pass 2 re-reads the row, normalizes and stores it (and the fused op's
// residual, which pass 1 leaves untouched so that pass 2 still reads the
// caller's residual).
//
// Backward, two kernels before the shared column reduce:
//  * stream_bwd_stats_kernel (1024 lanes, workgroups walk the rows): the
//    row's two reductions -- LayerNorm c1 = mean_j g, c2 = mean_j g * xhat;
//    RMSNorm rstd = rsqrt(mean_j x^2 + eps) and coef = rstd^3 mean_j g x --
//    stored as two floats per row after the workspace's partial-sum slabs;
//  * stream_bwd_tile_kernel (512 lanes): the columns are cut into tiles of
//    512 * V * 8; workgroup (walker w, tile t) walks the rows w, w + P, ...
//    of its tile with a ring of D rows in flight, writes dx of its columns
//    and accumulates their column sums in registers (no reduction over the
//    row, so no barrier in the loop), then writes them into slab w, columns
//    of tile t: the same [P][outs][padded] layout as the other backward
//    kernels.
#pragma once

#include "dyn_common.hpp"
#include "launch.hpp"

namespace rownorm {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// The first read of a row (the forward's statistic pass, the backward's
// reduction kernel) takes the default cache policy, so the row stays in the
// Infinity Cache for the second read, which is the row's last use and
// streams (non-temporal).  Measured on MI355X against non-temporal first reads
// (graph-timed over cold buffers, A/B in one process): fused add + RMSNorm
// 2048 x 131072 560 -> 477 us, LayerNorm forward 2048 x 65536 155 -> 114 us,
// LayerNorm backward 512 x 65536 78 -> 70 us and 4096 x 65536 468 -> 455 us;
// 8 accesses in flight instead of 4 moved each by -5 .. +1 %.  Build-time
// switches for measurement.
#ifndef ROWNORM_STREAM_UNROLL
#define ROWNORM_STREAM_UNROLL 4
#endif
#ifndef ROWNORM_STREAM_P1_POLICY
#define ROWNORM_STREAM_P1_POLICY 0
#endif
constexpr int kStreamUnroll = ROWNORM_STREAM_UNROLL;  // 16-byte accesses in flight per lane and matrix
constexpr int kStreamPass1 = ROWNORM_STREAM_P1_POLICY;  // cache policy of the first read

// ---- forward -------------------------------------------------------------------
template <int OP>
__global__ __launch_bounds__(kStreamFwdLanes) void stream_fwd_kernel(DynFwdArgs a) {
    constexpr int T = kStreamFwdLanes;
    constexpr int U = kStreamUnroll;
    constexpr bool kFused = OP == kSplitFused, kLn = OP == kSplitLn;
    __shared__ float red[4 * (T / kWave)];
    const int lane = threadIdx.x;
    const int h = a.hidden;
    const int n_acc = h / 8;
    const float inv_h = 1.0f / (float)h;
    const rsrc_t rw = row_rsrc_ld(a.weight, 0, 1, 0, h * 2);
    rsrc_t rb = rw;
    if constexpr (kLn) rb = row_rsrc_ld(a.bias, 0, 1, 0, h * 2);

    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
        const int64_t r = opaque_row(row);
        const rsrc_t rx = row_rsrc_ld(a.x, r, a.rows, a.ld_x * 2, h * 2);
        const rsrc_t ro = row_rsrc_ld(a.out, r, a.rows, a.ld_out * 2, h * 2);
        rsrc_t rr = rx;
        if constexpr (kFused) rr = row_rsrc_ld(a.residual, r, a.rows, a.ld_res * 2, h * 2);

        // pass 1: the row's statistic
        float p0 = 0.0f, p1 = 0.0f, n_l = 0.0f;
        for (int base = lane; base < n_acc; base += U * T) {
            u32x4 xv[U], rv[kFused ? U : 1];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                xv[u] = aload<8, kStreamPass1>(rx, (base + u * T) * 16);
                if constexpr (kFused) rv[u] = aload<8, kStreamPass1>(rr, (base + u * T) * 16);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float s[8];
                unpack8(xv[u], s);
                if constexpr (kFused) {
                    float rf[8];
                    unpack8(rv[u], rf);
#pragma unroll
                    for (int e = 0; e < 8; ++e) s[e] += rf[e];
                }
                if constexpr (kLn) {
                    if (base + u * T < n_acc) {  // an access past the row's end holds no data
                        float sg = 0.0f;
#pragma unroll
                        for (int e = 0; e < 8; ++e) sg += s[e];
                        const float mg = sg * 0.125f;
                        float m2g = 0.0f;
#pragma unroll
                        for (int e = 0; e < 8; ++e) m2g += (s[e] - mg) * (s[e] - mg);
                        if (n_l == 0.0f) {
                            p0 = sg;
                            p1 = m2g;
                        } else {
                            const float d = mg - p0 / n_l;
                            p1 += m2g + d * d * (n_l * 8.0f / (n_l + 8.0f));
                            p0 += sg;
                        }
                        n_l += 8.0f;
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) p0 += s[e] * s[e];  // past the end: zeros
                }
            }
        }
        float mu = 0.0f, rstd;
        if constexpr (kLn) {
            const float tot = row_sum<T>(p0, red, lane);
            mu = tot * inv_h;
            const float d = n_l > 0.0f ? p0 / n_l - mu : 0.0f;
            const float m2 = row_sum<T>(p1 + n_l * d * d, red + (T / kWave), lane);
            rstd = fast_rsqrt(m2 * inv_h + a.eps);
            if (lane == 0 && a.mean != nullptr) {
                a.mean[r] = mu;
                a.rstd[r] = rstd;
            }
        } else {
            rstd = fast_rsqrt(row_sum<T>(p0, red, lane) * inv_h + a.eps);
        }

        // pass 2: normalize (the row comes back from the caches while the rows
        // in flight fit there)
        for (int base = lane; base < n_acc; base += U * T) {
            u32x4 xv[U], rv[kFused ? U : 1], wv[U], bv[kLn ? U : 1];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int off = (base + u * T) * 16;
                xv[u] = aload<8, kCachePolicyNT>(rx, off);
                if constexpr (kFused) rv[u] = aload<8, kCachePolicyNT>(rr, off);
                wv[u] = aload<8, 0>(rw, off);
                if constexpr (kLn) bv[u] = aload<8, 0>(rb, off);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int off = (base + u * T) * 16;
                float s[8], wf[8], o[8];
                unpack8(xv[u], s);
                unpack8(wv[u], wf);
                if constexpr (kFused) {
                    float rf[8];
                    unpack8(rv[u], rf);
#pragma unroll
                    for (int e = 0; e < 8; ++e) s[e] += rf[e];
                    astore<8, kCachePolicyNT>(rr, off, pack8(s));
                }
                if constexpr (kLn) {
                    float bf[8];
                    unpack8(bv[u], bf);
#pragma unroll
                    for (int e = 0; e < 8; ++e) o[e] = (s[e] - mu) * rstd * wf[e] + bf[e];
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) o[e] = s[e] * rstd * wf[e];
                }
                astore<8, kCachePolicyNT>(ro, off, pack8(o));
            }
        }
        // the next row's first reduction must not overwrite slots still being read
        __syncthreads();
    }
}

template <int OP>
hipError_t launch_stream_fwd_op(const DynFwdArgs& a, hipStream_t stream) {
    const int64_t grid = a.rows < kStreamMaxGrid ? a.rows : kStreamMaxGrid;
    hipLaunchKernelGGL((stream_fwd_kernel<OP>), dim3((unsigned)grid), dim3(kStreamFwdLanes), 0,
                       stream, a);
    return hipGetLastError();
}

// ---- backward: the rows' two reductions ------------------------------------------
template <bool LN>
__global__ __launch_bounds__(kStreamFwdLanes) void stream_bwd_stats_kernel(DynBwdArgs a,
                                                                           float* stats) {
    constexpr int T = kStreamFwdLanes;
    constexpr int U = kStreamUnroll;
    __shared__ float red[2 * 2 * (T / kWave)];
    const int lane = threadIdx.x;
    const int h = a.hidden;
    const int n_acc = h / 8;
    const float inv_h = 1.0f / (float)h;
    const rsrc_t rw = row_rsrc_ld(a.weight, 0, 1, 0, h * 2);
    int parity = 0;
    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
        const int64_t r = opaque_row(row);
        const rsrc_t rx = row_rsrc_ld(a.x, r, a.rows, a.ld_x * 2, h * 2);
        const rsrc_t rd = row_rsrc_ld(a.dy, r, a.rows, a.ld_dy * 2, h * 2);
        float mean = 0.0f, q = 0.0f;
        if constexpr (LN) {
            mean = a.mean[r];
            q = a.rstd[r];
        }
        float s1 = 0.0f, s2 = 0.0f;
        for (int base = lane; base < n_acc; base += U * T) {
            u32x4 xv[U], dv[U], wv[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int off = (base + u * T) * 16;
                xv[u] = aload<8, kStreamPass1>(rx, off);
                dv[u] = aload<8, kStreamPass1>(rd, off);
                wv[u] = aload<8, 0>(rw, off);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float xf[8], df[8], wf[8];
                unpack8(xv[u], xf);
                unpack8(dv[u], df);
                unpack8(wv[u], wf);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float g = df[e] * wf[e];
                    if constexpr (LN) {
                        s1 += g;
                        s2 += g * ((xf[e] - mean) * q);
                    } else {
                        s1 += xf[e] * xf[e];
                        s2 += g * xf[e];
                    }
                }
            }
        }
        row_sum2<T>(s1, s2, red + parity * 2 * (T / kWave), lane);
        parity ^= 1;
        if (lane == 0) {
            if constexpr (LN) {
                stats[2 * r] = s1 * inv_h;
                stats[2 * r + 1] = s2 * inv_h;
            } else {
                const float rstd = fast_rsqrt(s1 * inv_h + a.eps);
                stats[2 * r] = rstd;
                stats[2 * r + 1] = rstd * rstd * rstd * s2 * inv_h;
            }
        }
    }
}

// ---- backward: dx and the column sums, one tile of columns per workgroup ------------
template <int V, bool DRES>
struct TileRow {
    u32x4 x[V];
    u32x4 dy[V];
    u32x4 dres[DRES ? V : 1];
    float s0, s1;                  // LayerNorm: c1, c2; RMSNorm: rstd, coef
    float mean, rstd;              // LayerNorm only
};

// Loads row `row` of tile columns [col0, ...) (a row past the end loads
// zeros from no memory and statistics of zero, so it adds nothing).
template <int V, bool LN, bool DRES>
__device__ __forceinline__ void load_tile_row(TileRow<V, DRES>& t, const DynBwdArgs& a,
                                              const float* stats, int64_t row, int col0,
                                              int lane) {
    constexpr int T = kStreamTileLanes;
    const int h = a.hidden;
    const rsrc_t rx = row_rsrc_ld(a.x, row, a.rows, a.ld_x * 2, h * 2);
    const rsrc_t rd = row_rsrc_ld(a.dy, row, a.rows, a.ld_dy * 2, h * 2);
#pragma unroll
    for (int b = 0; b < V; ++b) t.x[b] = aload<8, kCachePolicyNT>(rx, (col0 + (b * T + lane) * 8) * 2);
#pragma unroll
    for (int b = 0; b < V; ++b) t.dy[b] = aload<8, kCachePolicyNT>(rd, (col0 + (b * T + lane) * 8) * 2);
    if constexpr (DRES) {
        const rsrc_t rr = row_rsrc_ld(a.dres, row, a.rows, a.ld_dres * 2, h * 2);
#pragma unroll
        for (int b = 0; b < V; ++b)
            t.dres[b] = aload<8, kCachePolicyNT>(rr, (col0 + (b * T + lane) * 8) * 2);
    }
    const bool in = row < a.rows;
    const int64_t rc = in ? row : a.rows - 1;
    const float s0 = stats[2 * rc], s1 = stats[2 * rc + 1];
    t.s0 = in ? s0 : 0.0f;
    t.s1 = in ? s1 : 0.0f;
    if constexpr (LN) {
        const float m = a.mean[rc], q = a.rstd[rc];
        t.mean = in ? m : 0.0f;
        t.rstd = in ? q : 0.0f;
    }
}

template <int V, bool LN, bool DRES>
__device__ __forceinline__ void tile_row(const TileRow<V, DRES>& t, const u32x4 (&wv)[V],
                                         float (&pw)[V][8], float (&pb)[LN ? V : 1][8],
                                         const DynBwdArgs& a, int64_t row, int col0, int lane) {
    constexpr int T = kStreamTileLanes;
    const rsrc_t rdx = row_rsrc_ld(a.dx, row, a.rows, a.ld_dx * 2, a.hidden * 2);
#pragma unroll
    for (int b = 0; b < V; ++b) {
        float xf[8], df[8], wf[8], o[8];
        unpack8(t.x[b], xf);
        unpack8(t.dy[b], df);
        unpack8(wv[b], wf);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float g = df[e] * wf[e];
            if constexpr (LN) {
                const float xh = (xf[e] - t.mean) * t.rstd;
                o[e] = t.rstd * (g - t.s0 - xh * t.s1);
                pw[b][e] += df[e] * xh;
                pb[b][e] += df[e];
            } else {
                o[e] = t.s0 * g - t.s1 * xf[e];
                pw[b][e] += df[e] * (xf[e] * t.s0);
            }
        }
        if constexpr (DRES) {
            float rf[8];
            unpack8(t.dres[b], rf);
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] += rf[e];
        }
        astore<8, kCachePolicyNT>(rdx, (col0 + (b * T + lane) * 8) * 2, pack8(o));
    }
}

// Grid: walkers * tiles workgroups; workgroup i is tile i % tiles of walker
// i / tiles.  The stats of every row are complete (stream_bwd_stats_kernel
// ran before on the same stream).
template <int V, bool LN, bool DRES, int D>
__global__ __launch_bounds__(kStreamTileLanes) void stream_bwd_tile_kernel(DynBwdArgs a,
                                                                           const float* stats,
                                                                           int tiles) {
    constexpr int T = kStreamTileLanes;
    const int lane = threadIdx.x;
    const int tile = blockIdx.x % tiles;
    const int64_t walker = blockIdx.x / tiles;
    const int64_t P = gridDim.x / tiles;
    const int col0 = tile * (T * V * 8);
    const int h = a.hidden;
    const rsrc_t rw = row_rsrc_ld(a.weight, 0, 1, 0, h * 2);
    u32x4 wv[V];
#pragma unroll
    for (int b = 0; b < V; ++b) wv[b] = aload<8, 0>(rw, (col0 + (b * T + lane) * 8) * 2);
    float pw[V][8], pb[LN ? V : 1][8];
#pragma unroll
    for (int b = 0; b < V; ++b)
#pragma unroll
        for (int e = 0; e < 8; ++e) pw[b][e] = 0.0f;
#pragma unroll
    for (int b = 0; b < (LN ? V : 1); ++b)
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[b][e] = 0.0f;

    const int64_t n = walker < a.rows ? (a.rows - 1 - walker) / P + 1 : 0;
    TileRow<V, DRES> buf[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
        load_tile_row<V, LN, DRES>(buf[d], a, stats, opaque_row(walker + d * P), col0, lane);
        issue_fence();
    }
    for (int64_t i = 0; i < n; i += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int64_t r = opaque_row(walker + (i + d) * P);
            tile_row<V, LN, DRES>(buf[d], wv, pw, pb, a, r, col0, lane);
            issue_fence();
            load_tile_row<V, LN, DRES>(buf[d], a, stats, r + D * P, col0, lane);
            issue_fence();
        }
    }

    // this tile's columns of slab `walker`: [outs][padded]; columns past the
    // padded width are dropped by the descriptors' range
    const int padded = (h + 63) / 64 * 64;
    const int outs = LN ? 2 : 1;
    float* slab = a.workspace + walker * outs * (int64_t)padded;
    const rsrc_t sw = __builtin_amdgcn_make_buffer_rsrc(slab, (short)0, padded * 4, kRsrcWord3);
    const rsrc_t sb = __builtin_amdgcn_make_buffer_rsrc(slab + padded, (short)0,
                                                        LN ? padded * 4 : 0, kRsrcWord3);
#pragma unroll
    for (int b = 0; b < V; ++b) {
        const int off = (col0 + (b * T + lane) * 8) * 4;
        const f32x4 w0 = {pw[b][0], pw[b][1], pw[b][2], pw[b][3]};
        const f32x4 w1 = {pw[b][4], pw[b][5], pw[b][6], pw[b][7]};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, w0), sw, off, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, w1), sw, off + 16, 0, 0);
        if constexpr (LN) {
            const f32x4 b0 = {pb[b][0], pb[b][1], pb[b][2], pb[b][3]};
            const f32x4 b1 = {pb[b][4], pb[b][5], pb[b][6], pb[b][7]};
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, b0), sb, off, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, b1), sb, off + 16, 0,
                                                   0);
        }
    }
}

}  // namespace rownorm
