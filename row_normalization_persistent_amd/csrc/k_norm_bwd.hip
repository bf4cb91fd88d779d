// Normalization backward passes as a combined inner + outer reduction ("Llu/ln
// bwd", author note and review thread: the grid-parallel inner-and-outer
// normalization, the special case for LayerNorm backward), for LayerNorm and,
// with the same structure, for RMSNorm and the fused residual-add + RMSNorm.
//
// Kernel 1 (rows, persistent): G workgroups, each of T lanes, walk the rows
// g, g + G, g + 2G, ...  Per row (the inner reduction), LayerNorm:
//     xhat = (x - mean) * rstd,  g = dy * w,
//     c1 = mean_j g,  c2 = mean_j g * xhat   (one fused two-value reduction)
//     dx = bf16(rstd * (g - c1 - xhat * c2))
// RMSNorm (rstd recomputed from the row in registers):
//     sum_j x^2 and sum_j g * x               (one fused two-value reduction)
//     rstd = rsqrt(mean_j x^2 + eps),  dx = bf16(rstd * g - rstd^3 * mean_j(g x) * x [+ dres])
// Because every row maps the same columns to the same lane, each lane
// accumulates its columns' outer sums in registers across all the rows the
// workgroup visits (pw_j += dy * xhat, and for LayerNorm pb_j += dy).  Several
// rows' inputs are in flight behind the arithmetic (a ring of register
// buffers).  At the end each workgroup writes its partial sums to its slab of
// the workspace: [G][outs][H] fp32, outs = 2 (LayerNorm) or 1 (RMSNorm).
//
// Kernel 2 (column reduce): dweight_j = sum_g slab_g[0][j] (and dbias_j =
// sum_g slab_g[1][j]) in a fixed order, so results are reproducible bit for bit.
#include "device_common.hpp"
#include "launch.hpp"

namespace rownorm {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int V>
struct BwdRow {
    u32x4 x[V];
    u32x4 dy[V];
    float mean, rstd;
};

// Loads one row (predicated: a row index past the end loads zeros, from no
// memory, and its mean/rstd are 0, so it contributes nothing below).  The
// row's mean and rstd are the same for every lane of the workgroup, so they
// come in by scalar loads from a clamped row index (rows >= 1 whenever the
// kernel runs) instead of a buffer load in every lane: at one 16-byte access
// per lane that halves a row's vector memory instructions.  Measured on
// MI355X: 8192 x 2048 / 4096 / 8192 rows kernel 5 / 2 / 1 % faster, output
// bitwise unchanged.  The LDS waits of the row's reduction also wait for the
// next row's scalar loads (one counter covers both); fetching a walk's 64
// next pairs by one vector load instead and reading each with readlane was
// 3-5 % slower still (8192 x 4096 / 8192, 16384 x 4096), and so were per-row
// vector loads zeroed at the use rather than the load (8192 x 4096 41.3 ->
// 42.6 us, 8192 x 8192 78 -> 82).
template <int H, int T, int V>
__device__ __forceinline__ void load_bwd_row(BwdRow<V>& r, const u32x4* x, const u32x4* dy,
                                             const float* __restrict__ mean,
                                             const float* __restrict__ rstd, int64_t row,
                                             int64_t rows, int lane) {
    const rsrc_t rx = row_rsrc(x, row, rows, H * 2);
    const rsrc_t rd = row_rsrc(dy, row, rows, H * 2);
#pragma unroll
    for (int b = 0; b < V; ++b) r.x[b] = rload_stream(rx, (b * T + lane) * 16);
#pragma unroll
    for (int b = 0; b < V; ++b) r.dy[b] = rload_stream(rd, (b * T + lane) * 16);
    const int64_t rc = row < rows ? row : rows - 1;
    const float m = __builtin_nontemporal_load(mean + rc);
    const float q = __builtin_nontemporal_load(rstd + rc);
    r.mean = row < rows ? m : 0.0f;
    r.rstd = row < rows ? q : 0.0f;
}

// RMSNorm row: x, dy and (fused op) the residual-output gradient dres.
template <int V, bool DRES>
struct RmsRow {
    u32x4 x[V];
    u32x4 dy[V];
    u32x4 dres[DRES ? V : 1];
};

template <int H, int T, int V, bool DRES>
__device__ __forceinline__ void load_rms_row(RmsRow<V, DRES>& r, const u32x4* x, const u32x4* dy,
                                             const u32x4* dres, int64_t row, int64_t rows,
                                             int lane) {
    const rsrc_t rx = row_rsrc(x, row, rows, H * 2);
    const rsrc_t rd = row_rsrc(dy, row, rows, H * 2);
#pragma unroll
    for (int b = 0; b < V; ++b) r.x[b] = rload_stream(rx, (b * T + lane) * 16);
#pragma unroll
    for (int b = 0; b < V; ++b) r.dy[b] = rload_stream(rd, (b * T + lane) * 16);
    if constexpr (DRES) {
        const rsrc_t rr = row_rsrc(dres, row, rows, H * 2);
#pragma unroll
        for (int b = 0; b < V; ++b) r.dres[b] = rload_stream(rr, (b * T + lane) * 16);
    }
}

template <int H, int T, int V>
__device__ __forceinline__ void bwd_row(const BwdRow<V>& cur, const float (&wf)[V][8],
                                        float (&pw)[V][8], float (&pb)[V][8], u32x4* dx,
                                        float* red, int64_t row, int64_t rows, int lane) {
    float xh[V][8], g[V][8];
    float a1[8] = {0, 0, 0, 0, 0, 0, 0, 0}, a2[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int b = 0; b < V; ++b) {
        float xf[8], df[8];
        unpack8(cur.x[b], xf);
        unpack8(cur.dy[b], df);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            xh[b][k] = (xf[k] - cur.mean) * cur.rstd;
            g[b][k] = df[k] * wf[b][k];
            a1[k] += g[b][k];
            a2[k] += g[b][k] * xh[b][k];
            pw[b][k] += df[k] * xh[b][k];
            pb[b][k] += df[k];
        }
    }
    float s1 = ((a1[0] + a1[1]) + (a1[2] + a1[3])) + ((a1[4] + a1[5]) + (a1[6] + a1[7]));
    float s2 = ((a2[0] + a2[1]) + (a2[2] + a2[3])) + ((a2[4] + a2[5]) + (a2[6] + a2[7]));
    row_sum2<T>(s1, s2, red, lane);
    const float c1 = s1 * (1.0f / H);
    const float c2 = s2 * (1.0f / H);
    const rsrc_t rdx = row_rsrc(dx, row, rows, H * 2);  // drops the stores of rows >= rows
#pragma unroll
    for (int b = 0; b < V; ++b) {
        float o[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) o[k] = cur.rstd * (g[b][k] - c1 - xh[b][k] * c2);
        rstore_stream(rdx, (b * T + lane) * 16, pack8(o));
    }
}

template <int H, int T, int V, bool DRES>
__device__ __forceinline__ void rms_bwd_row(const RmsRow<V, DRES>& cur, const float (&wf)[V][8],
                                            float (&pw)[V][8], u32x4* dx, float* red,
                                            int64_t row, int64_t rows, int lane, float eps) {
    float a1[8] = {0, 0, 0, 0, 0, 0, 0, 0}, a2[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int b = 0; b < V; ++b) {
        float xf[8], df[8];
        unpack8(cur.x[b], xf);
        unpack8(cur.dy[b], df);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            a1[k] += xf[k] * xf[k];
            a2[k] += df[k] * wf[b][k] * xf[k];
        }
    }
    float s1 = ((a1[0] + a1[1]) + (a1[2] + a1[3])) + ((a1[4] + a1[5]) + (a1[6] + a1[7]));
    float s2 = ((a2[0] + a2[1]) + (a2[2] + a2[3])) + ((a2[4] + a2[5]) + (a2[6] + a2[7]));
    row_sum2<T>(s1, s2, red, lane);
    // a row past the end (all zeros) must add exactly nothing to the column
    // sums, also at eps = 0, where rsqrt(0) is inf and 0 * inf is NaN
    const float rstd = row < rows ? fast_rsqrt(s1 * (1.0f / H) + eps) : 0.0f;
    const float coef = rstd * rstd * rstd * s2 * (1.0f / H);  // rstd * mean_j(g * xhat) * rstd
    const rsrc_t rdx = row_rsrc(dx, row, rows, H * 2);  // drops the stores of rows >= rows
#pragma unroll
    for (int b = 0; b < V; ++b) {
        float xf[8], df[8], o[8];
        unpack8(cur.x[b], xf);
        unpack8(cur.dy[b], df);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            o[k] = rstd * (df[k] * wf[b][k]) - coef * xf[k];
            pw[b][k] += df[k] * (xf[k] * rstd);
        }
        if constexpr (DRES) {
            float rf[8];
            unpack8(cur.dres[b], rf);
#pragma unroll
            for (int k = 0; k < 8; ++k) o[k] += rf[k];
        }
        rstore_stream(rdx, (b * T + lane) * 16, pack8(o));
    }
}

// D rows are kept in flight per workgroup: a ring of D register buffers, the
// loop unrolled by D so each buffer index is a compile-time constant.  After
// row i is finished its buffer is refilled with row i + D*G, so while one row
// is reduced the loads of the next D - 1 rows are outstanding.
template <int H, int T, int D>
__global__ __launch_bounds__(T) void layernorm_bwd_rows_kernel(
    u32x4* dx, const u32x4* dy, const u32x4* x, const float* __restrict__ mean,
    const float* __restrict__ rstd, const u32x4* __restrict__ weight, float* workspace,
    int64_t rows) {
    using S = Shape<H, T, 1>;
    constexpr int V = S::kVecs;
    constexpr int kSlot = 2 * S::kWaves;
    __shared__ float red[2 * kSlot];

    const int lane = threadIdx.x;
    float wf[V][8];
#pragma unroll
    for (int b = 0; b < V; ++b) unpack8(weight[lane + b * T], wf[b]);

    float pw[V][8], pb[V][8];
#pragma unroll
    for (int b = 0; b < V; ++b)
#pragma unroll
        for (int k = 0; k < 8; ++k) pw[b][k] = pb[b][k] = 0.0f;

    // This workgroup owns rows blockIdx.x + i * G, i = 0 .. n - 1.  They are
    // walked in groups of D; the last group may run past the end, and those
    // slots load zeros and store nothing (see row_rsrc), so the loop body has
    // no branch and every barrier is reached by the whole workgroup.
    const int64_t G = gridDim.x;
    const int64_t first = blockIdx.x;
    const int64_t n = first < rows ? (rows - 1 - first) / G + 1 : 0;
    BwdRow<V> buf[D];
    // The fences keep the slots' loads in slot order on both paths into the
    // loop (prologue and back edge), so the memory-counter wait before slot d
    // only covers slot d's own loads, not the younger slots'.
#pragma unroll
    for (int d = 0; d < D; ++d) {
        load_bwd_row<H, T, V>(buf[d], x, dy, mean, rstd, first + d * G, rows, lane);
        issue_fence();
    }
    int parity = 0;
    for (int64_t i = 0; i < n; i += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int64_t r = first + (i + d) * G;
            bwd_row<H, T, V>(buf[d], wf, pw, pb, dx, red + parity * kSlot, r, rows, lane);
            parity ^= 1;
            issue_fence();
            load_bwd_row<H, T, V>(buf[d], x, dy, mean, rstd, r + D * G, rows, lane);
            issue_fence();
        }
    }

    float* slab = workspace + (int64_t)blockIdx.x * 2 * H;
#pragma unroll
    for (int b = 0; b < V; ++b) {
        const int col = (b * T + lane) * 8;
        f32x4* pwv = (f32x4*)(slab + col);
        f32x4* pbv = (f32x4*)(slab + H + col);
        pwv[0] = f32x4{pw[b][0], pw[b][1], pw[b][2], pw[b][3]};
        pwv[1] = f32x4{pw[b][4], pw[b][5], pw[b][6], pw[b][7]};
        pbv[0] = f32x4{pb[b][0], pb[b][1], pb[b][2], pb[b][3]};
        pbv[1] = f32x4{pb[b][4], pb[b][5], pb[b][6], pb[b][7]};
    }
}

template <int H, int T, int D, bool DRES>
__global__ __launch_bounds__(T) void rmsnorm_bwd_rows_kernel(
    u32x4* dx, const u32x4* dy, const u32x4* x, const u32x4* dres,
    const u32x4* __restrict__ weight, float* workspace, int64_t rows, float eps) {
    using S = Shape<H, T, 1>;
    constexpr int V = S::kVecs;
    constexpr int kSlot = 2 * S::kWaves;
    __shared__ float red[2 * kSlot];

    const int lane = threadIdx.x;
    float wf[V][8];
#pragma unroll
    for (int b = 0; b < V; ++b) unpack8(weight[lane + b * T], wf[b]);
    float pw[V][8];
#pragma unroll
    for (int b = 0; b < V; ++b)
#pragma unroll
        for (int k = 0; k < 8; ++k) pw[b][k] = 0.0f;

    // same ring walk as the LayerNorm kernel above
    const int64_t G = gridDim.x;
    const int64_t first = blockIdx.x;
    const int64_t n = first < rows ? (rows - 1 - first) / G + 1 : 0;
    RmsRow<V, DRES> buf[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
        load_rms_row<H, T, V, DRES>(buf[d], x, dy, dres, first + d * G, rows, lane);
        issue_fence();
    }
    int parity = 0;
    for (int64_t i = 0; i < n; i += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int64_t r = first + (i + d) * G;
            rms_bwd_row<H, T, V, DRES>(buf[d], wf, pw, dx, red + parity * kSlot, r, rows, lane,
                                       eps);
            parity ^= 1;
            issue_fence();
            load_rms_row<H, T, V, DRES>(buf[d], x, dy, dres, r + D * G, rows, lane);
            issue_fence();
        }
    }

    float* slab = workspace + (int64_t)blockIdx.x * H;
#pragma unroll
    for (int b = 0; b < V; ++b) {
        f32x4* pwv = (f32x4*)(slab + (b * T + lane) * 8);
        pwv[0] = f32x4{pw[b][0], pw[b][1], pw[b][2], pw[b][3]};
        pwv[1] = f32x4{pw[b][4], pw[b][5], pw[b][6], pw[b][7]};
    }
}

// Column reduce.  A workgroup owns C consecutive columns of the flat
// [outs][padded] slab (dweight columns, then dbias columns; padded is a
// multiple of 64, so a workgroup never straddles two outputs); its 256 lanes
// form C/4 column groups of 4 columns x 1024/C slab streams.  Stream s adds
// the slabs s, s + S, s + 2S, ... (S streams, 16 independent loads in flight
// per pass; a slab index past the last is clamped to the slab count, whose
// offset the workspace descriptor range-checks to zero), then the S stream
// sums of each column are added as a fixed pairwise tree.  C = 64 for up to
// 256 slabs (one pass), 16 beyond, so many slabs spread over more workgroups.
// The summation order is fixed for a given (slabs, hidden), so the result is
// bit-reproducible.  Columns in the padding (hidden <= j < padded) are
// summed but not stored.
template <int C>
__global__ __launch_bounds__(kColReduceThreads) void norm_bwd_colreduce_kernel(
    const float* __restrict__ workspace, int32_t grid_slabs, int32_t hidden, int32_t padded,
    int32_t outs, float* __restrict__ dweight, float* __restrict__ dbias) {
    constexpr int kGroups = C / 4;                              // column groups of 4
    constexpr int kStreams = kColReduceThreads / kGroups;       // slab streams
    constexpr int kUnroll = 16;
    const int cg = threadIdx.x % kGroups;
    const int stream = threadIdx.x / kGroups;
    const int flat = blockIdx.x * C + cg * 4;                   // < outs * padded
    const int slab_bytes = outs * padded * 4;
    const rsrc_t ws = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(workspace), (short)0, grid_slabs * slab_bytes, kRsrcWord3);
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int g0 = 0; g0 < grid_slabs; g0 += kStreams * kUnroll) {
        f32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int g = min(g0 + stream + u * kStreams, grid_slabs);
            v[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 ws, g * slab_bytes + flat * 4, 0, 0));
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc += v[u];
    }
    // the S stream sums of each column, added as a fixed pairwise tree
    __shared__ f32x4 part[kStreams][kGroups];
    part[stream][cg] = acc;
    __syncthreads();
#pragma unroll
    for (int half = kStreams / 2; half >= 1; half /= 2) {
        if (stream < half) part[stream][cg] += part[stream + half][cg];
        __syncthreads();
    }
    if (threadIdx.x < kGroups) {
        const f32x4 s = part[0][cg];
        const int o = flat / padded;
        const int col = flat - o * padded;
        float* dst = (o == 0 ? dweight : dbias) + col;
        if (col + 0 < hidden) dst[0] = s.x;
        if (col + 1 < hidden) dst[1] = s.y;
        if (col + 2 < hidden) dst[2] = s.z;
        if (col + 3 < hidden) dst[3] = s.w;
    }
}

hipError_t launch_norm_colreduce(const float* workspace, int32_t slabs, int32_t hidden,
                                 int32_t padded, int32_t outs, float* dweight, float* dbias,
                                 hipStream_t stream) {
    const int cols = colreduce_cols(slabs);
    const dim3 grid(outs * padded / cols), block(kColReduceThreads);
    if (cols == 64)
        hipLaunchKernelGGL(norm_bwd_colreduce_kernel<64>, grid, block, 0, stream, workspace,
                           slabs, hidden, padded, outs, dweight, dbias);
    else
        hipLaunchKernelGGL(norm_bwd_colreduce_kernel<16>, grid, block, 0, stream, workspace,
                           slabs, hidden, padded, outs, dweight, dbias);
    return hipGetLastError();
}

// Rows in flight per workgroup (the register ring depth): the deepest ring
// that compiles without register spills for both LayerNorm and RMSNorm (with
// the residual gradient), from the compiler's resource report on gfx950.  A
// lane may use 256 VGPRs in workgroups of up to 512 lanes and 128 in 1024-lane
// workgroups, and each ring slot costs about 26-30 VGPRs per 16-byte vector.
// Depth 4 at one vector per lane (512 lanes at hidden 4096) and depth 3 at
// 1024 lanes measured fastest.
#ifndef ROWNORM_BWD_DEPTH
#define ROWNORM_BWD_DEPTH 0
#endif
template <int H, int T>
constexpr int bwd_depth() {
    constexpr int V = H / (8 * T);
    if constexpr (ROWNORM_BWD_DEPTH > 0) return ROWNORM_BWD_DEPTH;
    if constexpr (T >= 1024) return V == 1 ? 3 : 1;
    if constexpr (V == 1) return 4;
    if constexpr (V == 2) return T >= 512 ? 3 : 4;
    if constexpr (V == 3) return 2;
    return T >= 512 ? 1 : 3;
}

template <int H, int T>
hipError_t launch_colreduce(const BwdArgs& a, int outs, hipStream_t stream) {
    static_assert(H % kColReduceCols == 0, "compiled hidden sizes need no padding");
    return launch_norm_colreduce(a.workspace, a.rows > 0 ? a.grid : 0, H, H, outs, a.dweight,
                                 a.dbias, stream);
}

template <int H, int T>
hipError_t launch_ln_bwd(const BwdArgs& a, hipStream_t stream) {
    if (a.rows > 0) {
        hipLaunchKernelGGL((layernorm_bwd_rows_kernel<H, T, bwd_depth<H, T>()>), dim3(a.grid),
                           dim3(T), 0, stream, (u32x4*)a.dx, (const u32x4*)a.dy,
                           (const u32x4*)a.x, a.mean, a.rstd, (const u32x4*)a.weight, a.workspace,
                           a.rows);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return launch_colreduce<H, T>(a, 2, stream);
}

template <int H, int T>
hipError_t launch_rms_bwd(const BwdArgs& a, hipStream_t stream) {
    if (a.rows > 0) {
        if (a.dres) {
            hipLaunchKernelGGL((rmsnorm_bwd_rows_kernel<H, T, bwd_depth<H, T>(), true>),
                               dim3(a.grid), dim3(T), 0, stream, (u32x4*)a.dx, (const u32x4*)a.dy,
                               (const u32x4*)a.x, (const u32x4*)a.dres, (const u32x4*)a.weight,
                               a.workspace, a.rows, a.eps);
        } else {
            hipLaunchKernelGGL((rmsnorm_bwd_rows_kernel<H, T, bwd_depth<H, T>(), false>),
                               dim3(a.grid), dim3(T), 0, stream, (u32x4*)a.dx, (const u32x4*)a.dy,
                               (const u32x4*)a.x, (const u32x4*)nullptr, (const u32x4*)a.weight,
                               a.workspace, a.rows, a.eps);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return launch_colreduce<H, T>(a, 1, stream);
}

// Lanes per row: at most 4 vectors per lane, since each lane also keeps
// fp32 column accumulators (16 per vector for LayerNorm, 8 for RMSNorm).
template <int T>
struct Lanes {};
using BwdShapeList = std::tuple<Lanes<64>, Lanes<128>, Lanes<256>, Lanes<512>, Lanes<1024>>;

template <bool RMS, int H, int T>
void add_bwd_entry(std::vector<BwdEntry>& v, Lanes<T>) {
    if constexpr (H % (8 * T) == 0 && H / (8 * T) <= 4) {
        if constexpr (RMS)
            v.push_back({H, T, bwd_depth<H, T>(), &launch_rms_bwd<H, T>});
        else
            v.push_back({H, T, bwd_depth<H, T>(), &launch_ln_bwd<H, T>});
    }
}

template <bool RMS, int H, class... Ls>
void add_bwd_entries_h(std::vector<BwdEntry>& v, std::tuple<Ls...>) {
    (add_bwd_entry<RMS, H>(v, Ls{}), ...);
}

template <bool RMS>
std::vector<BwdEntry> build_bwd_table() {
    std::vector<BwdEntry> v;
    add_bwd_entries_h<RMS, 1024>(v, BwdShapeList{});
    add_bwd_entries_h<RMS, 2048>(v, BwdShapeList{});
    add_bwd_entries_h<RMS, 4096>(v, BwdShapeList{});
    add_bwd_entries_h<RMS, 8192>(v, BwdShapeList{});
    add_bwd_entries_h<RMS, 12288>(v, BwdShapeList{});
    add_bwd_entries_h<RMS, 16384>(v, BwdShapeList{});
    return v;
}

const std::vector<BwdEntry>& layernorm_bwd_table() {
    static const std::vector<BwdEntry> table = build_bwd_table<false>();
    return table;
}

const std::vector<BwdEntry>& rmsnorm_bwd_table() {
    static const std::vector<BwdEntry> table = build_bwd_table<true>();
    return table;
}

}  // namespace rownorm
