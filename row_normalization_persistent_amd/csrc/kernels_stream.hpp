// Streamed rows: the rows of a [rows, hidden] matrix walked by workgroups that
// read each row from memory twice instead of holding it on chip.  "TMA inner
// persistent scheduler" (description summary) keeps the row in shared memory
// when registers cannot hold it; a bf16 row of more than 65536 values (fused
// add + RMSNorm, RMSNorm), 49152 (LayerNorm forward) or 32768 (the backward
// operations, whose per-column sums also live on chip) fits neither, so
// these kernels read it twice: once for the row's reduction and once more,
// from the Infinity Cache while the rows in flight fit there, for the
// normalized output.  The same kernels serve fp32 activations (at every
// width but the backward's 8196 ... 16384 columns, which the LDS-staged
// kernel reads once; forward rows of up to 1024 fp32 values go several to a
// wave in group_fwd_kernel).  16-byte accesses only: E = uint16_t (bf16 patterns, 8 a 16-byte
// access) or float (4), hidden a multiple of the access's element count,
// every row stride too, 16-byte-aligned pointers, hidden up to 2^20.
//
// Forward (stream_fwd_kernel, T lanes a row -- 1024 for bf16; for fp32 as
// many as give each lane at most 4 accesses of a row of up to 16384 values,
// 1024 beyond -- workgroups walk the rows g, g + G, ...): pass 1 streams the
// row for its statistic -- sum s^2 (s = x + r for
// the fused op), or for LayerNorm each lane's count, sum and centered sum of
// squares, merged access by access with the pairwise update of a sum of
// squared deviations (Chan, Golub & LeVeque), then combined over the lanes
// exactly as the row split combines its chunks:
//   mean = sum_l S_l / H,  M2 = sum_l M2_l + n_l (S_l / n_l - mean)^2;
// pass 2 normalizes and stores the row (and the fused op's residual, which
// pass 1 leaves untouched so that pass 2 still reads the caller's residual).
// The row's first kStreamUnroll accesses a lane stay in registers from pass
// 1 to pass 2; only the rest is read again (a row of up to 4 x T accesses is
// read once: every fp32 row of up to 16384 values).
//
// Backward, before the shared column reduce: stream_bwd_tile_kernel (512
// lanes) cuts the columns into tiles of 512 * V accesses; workgroup (walker
// w, tile t) walks the rows w, w + P, ... of its tile with a ring of D rows in
// flight, writes dx of its columns and accumulates their column sums in
// registers, then writes them into slab w, columns of tile t: the same
// [P][outs][padded] layout as the other backward kernels.  The row's two
// reductions -- LayerNorm sum_j g and sum_j g * xhat; RMSNorm sum_j x^2 and
// sum_j g x, giving rstd = rsqrt(mean_j x^2 + eps) and coef = rstd^3 mean_j
// g x -- come from one of:
//  * XCH (2 to kXchMaxTiles tiles a row): the tiles of a row exchange their
//    partial sums through 64-bit slots in the workspace, a group of D rows
//    per round trip (bf16: two rings, one group published ahead), with a
//    bounded wait and a fallback that reads the other tiles' columns itself;
//    each row is read once (stream_zero_kernel clears the slots first);
//  * INROW (fp32 up to 8192 columns, one tile holds the row, V = 1, 2 or 4):
//    the tile kernel reduces the row itself, one barrier a row;
//  * stream_bwd_stats_kernel (1024 lanes; rows of more than kXchMaxTiles
//    tiles, whose all-to-all exchange would cost more than a second read):
//    the two reductions of every row as two floats a row after the slabs,
//    before the tile kernel, which then reads x and dy a second time.
#pragma once

#include "dyn_common.hpp"
#include "launch.hpp"
#include "lds_stage.hpp"
#include "stream_select.hpp"

namespace rownorm {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// The first read of the part of a row that is read twice (the forward's
// statistic pass past the accesses it keeps in registers, the backward's
// reduction kernel) takes the default cache policy, so that part stays in
// the Infinity Cache for the second read, which is its last use and streams
// (non-temporal).  Measured on MI355X against non-temporal first reads
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
// The forward's accesses kept in registers from the first pass to the second
// are never read again: non-temporal, so that they do not take Infinity Cache
// lines from the rest of the row (measured on MI355X against the default
// policy, graph-timed over cold buffers, alternating processes: fp32 fused
// 8192 x 4096 100.8 -> 91.5 us and 4096 x 8192 107.6 -> 96.6, fp32 RMSNorm
// 4096 x 16384 92.4 -> 87.9, fp32 LayerNorm 2048 x 16384 51.5 -> 49.2; bf16
// fused 2048 x 131072 441 -> 432, LayerNorm 2048 x 65536 110.3 -> 106.9).
#ifndef ROWNORM_STREAM_KEPT_NT
#define ROWNORM_STREAM_KEPT_NT 1
#endif
constexpr int kStreamKept = ROWNORM_STREAM_KEPT_NT ? kCachePolicyNT : kStreamPass1;

template <int Aux>
__device__ __forceinline__ u32x4 load16(rsrc_t r, int byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, Aux);
}
__device__ __forceinline__ void store16(rsrc_t r, int byte_off, const u32x4& v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_off, 0, kCachePolicyNT);
}

// ---- forward -------------------------------------------------------------------
// One pass-1 step over accesses base + u * T (u < U) of the loaded chunk.
template <typename E, int OP, int U, int T>
__device__ __forceinline__ void stream_stat_step(const u32x4 (&xv)[U],
                                                 const u32x4 (&rv)[OP == kSplitFused ? U : 1],
                                                 int base, int n_acc, float& p0, float& p1,
                                                 float& n_l) {
    constexpr int EP = Elems<E>::kPer;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float s[EP];
        unpack16<E>(xv[u], s);
        if constexpr (OP == kSplitFused) {
            float rf[EP];
            unpack16<E>(rv[u], rf);
#pragma unroll
            for (int e = 0; e < EP; ++e) s[e] += rf[e];
        }
        if constexpr (OP == kSplitLn) {
            if (base + u * T < n_acc) {  // an access past the row's end holds no data
                float sg = 0.0f;
#pragma unroll
                for (int e = 0; e < EP; ++e) sg += s[e];
                const float mg = sg * (1.0f / EP);
                float m2g = 0.0f;
#pragma unroll
                for (int e = 0; e < EP; ++e) m2g += (s[e] - mg) * (s[e] - mg);
                if (n_l == 0.0f) {
                    p0 = sg;
                    p1 = m2g;
                } else {
                    const float d = mg - p0 / n_l;
                    p1 += m2g + d * d * (n_l * (float)EP / (n_l + (float)EP));
                    p0 += sg;
                }
                n_l += (float)EP;
            }
        } else {
#pragma unroll
            for (int e = 0; e < EP; ++e) p0 += s[e] * s[e];  // past the end: zeros
        }
    }
}

// One pass-2 step: normalize and store the U accesses base + u * T.
template <typename E, int OP, int U, int T>
__device__ __forceinline__ void stream_norm_step(const u32x4 (&xv)[U],
                                                 const u32x4 (&rv)[OP == kSplitFused ? U : 1],
                                                 rsrc_t rw, rsrc_t rb, rsrc_t rr, rsrc_t ro,
                                                 int base, float mu, float rstd) {
    constexpr int EP = Elems<E>::kPer;
    u32x4 wv[U], bv[OP == kSplitLn ? U : 1];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        wv[u] = load16<0>(rw, (base + u * T) * 16);
        if constexpr (OP == kSplitLn) bv[u] = load16<0>(rb, (base + u * T) * 16);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int off = (base + u * T) * 16;
        float s[EP], wf[EP], o[EP];
        unpack16<E>(xv[u], s);
        unpack16<E>(wv[u], wf);
        if constexpr (OP == kSplitFused) {
            float rf[EP];
            unpack16<E>(rv[u], rf);
#pragma unroll
            for (int e = 0; e < EP; ++e) s[e] += rf[e];
            store16(rr, off, pack16<E>(s));
        }
        if constexpr (OP == kSplitLn) {
            float bf[EP];
            unpack16<E>(bv[u], bf);
#pragma unroll
            for (int e = 0; e < EP; ++e) o[e] = (s[e] - mu) * rstd * wf[e] + bf[e];
        } else {
#pragma unroll
            for (int e = 0; e < EP; ++e) o[e] = s[e] * rstd * wf[e];
        }
        store16(ro, off, pack16<E>(o));
    }
}

template <typename E, int OP, int T, int U = kStreamUnroll>
__global__ __launch_bounds__(T) void stream_fwd_kernel(DynFwdArgs a) {
    constexpr int EP = Elems<E>::kPer;
    constexpr int ES = (int)sizeof(E);
    constexpr bool kFused = OP == kSplitFused, kLn = OP == kSplitLn;
    __shared__ float red[4 * (T / kWave)];
    const int lane = threadIdx.x;
    const int h = a.hidden;
    const int n_acc = h / EP;
    const float inv_h = 1.0f / (float)h;
    const rsrc_t rw = row_rsrc_ld(a.weight, 0, 1, 0, h * ES);
    rsrc_t rb = rw;
    if constexpr (kLn) rb = row_rsrc_ld(a.bias, 0, 1, 0, h * ES);

    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
        const int64_t r = opaque_row(row);
        const rsrc_t rx = row_rsrc_ld(a.x, r, a.rows, a.ld_x * ES, h * ES);
        const rsrc_t ro = row_rsrc_ld(a.out, r, a.rows, a.ld_out * ES, h * ES);
        rsrc_t rr = rx;
        if constexpr (kFused) rr = row_rsrc_ld(a.residual, r, a.rows, a.ld_res * ES, h * ES);

        // pass 1: the row's statistic; the first U accesses a lane are kept
        float p0 = 0.0f, p1 = 0.0f, n_l = 0.0f;
        u32x4 x0[U], r0[kFused ? U : 1];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            x0[u] = load16<kStreamKept>(rx, (lane + u * T) * 16);
            if constexpr (kFused) r0[u] = load16<kStreamKept>(rr, (lane + u * T) * 16);
        }
        stream_stat_step<E, OP, U, T>(x0, r0, lane, n_acc, p0, p1, n_l);
        for (int base = lane + U * T; base < n_acc; base += U * T) {
            u32x4 xv[U], rv[kFused ? U : 1];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                xv[u] = load16<kStreamPass1>(rx, (base + u * T) * 16);
                if constexpr (kFused) rv[u] = load16<kStreamPass1>(rr, (base + u * T) * 16);
            }
            stream_stat_step<E, OP, U, T>(xv, rv, base, n_acc, p0, p1, n_l);
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

        // pass 2: normalize; the rest of the row comes back from the caches
        // while the rows in flight fit there
        stream_norm_step<E, OP, U, T>(x0, r0, rw, rb, rr, ro, lane, mu, rstd);
        for (int base = lane + U * T; base < n_acc; base += U * T) {
            u32x4 xv[U], rv[kFused ? U : 1];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                xv[u] = load16<kCachePolicyNT>(rx, (base + u * T) * 16);
                if constexpr (kFused) rv[u] = load16<kCachePolicyNT>(rr, (base + u * T) * 16);
            }
            stream_norm_step<E, OP, U, T>(xv, rv, rw, rb, rr, ro, base, mu, rstd);
        }
        // the next row's first reduction must not overwrite slots still being read
        __syncthreads();
    }
}

template <typename E, int OP, int T, int U = kStreamUnroll>
hipError_t launch_stream_fwd_op(const DynFwdArgs& a, hipStream_t stream) {
    const int64_t grid = a.rows < kStreamMaxGrid ? a.rows : kStreamMaxGrid;
    hipLaunchKernelGGL((stream_fwd_kernel<E, OP, T, U>), dim3((unsigned)grid), dim3(T), 0, stream,
                       a);
    return hipGetLastError();
}

// ---- forward, rows held in registers and LDS ----------------------------------------
// For rows a little too wide for the registers (the LDS-staged persistent
// buffer of "TMA inner persistent scheduler", description summary): lane t of
// the 1024 holds accesses b*1024 + t, the first U in registers (as in
// stream_fwd_kernel) and the next L in LDS slots, which buffer loads with the
// LDS bit fill straight from HBM (x, and r for the fused op: 16 KiB a slot and
// matrix); rows of up to (U + L) * 1024 accesses are read once.  One row at a
// time (the LDS holds one): its slot loads, then its register loads, go out
// at the start; the first pass reads slot k once at most as many loads are
// outstanding as were issued after k's (the later slots' and the register
// accesses; the buffer-to-LDS loads are invisible to the compiler, whose own
// waits for the register accesses are exact because those go out last); the
// weights (and LayerNorm's bias) of the whole row go out before the row's
// reduction and land during it.  Measured against handing each slot to the
// next row's load during the second pass (the walk pipelined by access, as
// the LDS-staged backward does): that was 2-18 % slower at every shape.  The
// launcher takes this kernel for the fused op and RMSNorm only (the rows it
// takes: stage_fwd_holds); LayerNorm's rows stream.  A lane's slots past the
// row's end are zeroed once for the walk.
template <typename E, int OP>
__device__ __forceinline__ void stage_norm_access(const u32x4& xv, const u32x4& rv,
                                                  const u32x4& wv, const u32x4& bv, rsrc_t rr,
                                                  rsrc_t ro, int off, float mu, float rstd) {
    constexpr int EP = Elems<E>::kPer;
    float s[EP], wf[EP], o[EP];
    unpack16<E>(xv, s);
    unpack16<E>(wv, wf);
    if constexpr (OP == kSplitFused) {
        float rf[EP];
        unpack16<E>(rv, rf);
#pragma unroll
        for (int e = 0; e < EP; ++e) s[e] += rf[e];
        store16(rr, off, pack16<E>(s));
    }
    if constexpr (OP == kSplitLn) {
        float bf[EP];
        unpack16<E>(bv, bf);
#pragma unroll
        for (int e = 0; e < EP; ++e) o[e] = (s[e] - mu) * rstd * wf[e] + bf[e];
    } else {
#pragma unroll
        for (int e = 0; e < EP; ++e) o[e] = s[e] * rstd * wf[e];
    }
    store16(ro, off, pack16<E>(o));
}

template <typename E, int OP, int U, int L>
__global__ __launch_bounds__(kStreamFwdLanes) void stage_fwd_kernel(DynFwdArgs a) {
    constexpr int T = kStreamFwdLanes;
    constexpr int EP = Elems<E>::kPer;
    constexpr int ES = (int)sizeof(E);
    constexpr bool kFused = OP == kSplitFused, kLn = OP == kSplitLn;
    constexpr int M = kFused ? 2 : 1;  // matrices staged an access: x (and r)
    constexpr int NB = U + L;          // accesses a lane
    static_assert(M * L * T * 16 + 4 * (T / kWave) * 4 <= 160 * 1024, "LDS of one workgroup");
    __shared__ u32x4 st[L * M * T];  // slot (k, m) of lane t: st[(k M + m) T + t]
    __shared__ float red[4 * (T / kWave)];
    const int lane = threadIdx.x;
    const int h = a.hidden;
    const int n_acc = h / EP;
    const float inv_h = 1.0f / (float)h;
    const rsrc_t rw = row_rsrc_ld(a.weight, 0, 1, 0, h * ES);
    rsrc_t rb = rw;
    if constexpr (kLn) rb = row_rsrc_ld(a.bias, 0, 1, 0, h * ES);
    // LDS byte address of this wave's 64 slots of slot (0, 0), wave uniform
    const uint32_t st_lds =
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)st +
        (uint32_t)__builtin_amdgcn_readfirstlane(lane & ~(kWave - 1)) * 16u;
    // A lane's slots past the row's end (the same for every row) hold zeros
    // for the whole walk, so that they add nothing to the row's sums: a
    // buffer load past its range returns zeros, whether or not it then writes
    // its LDS slot.
#pragma unroll
    for (int k = 0; k < L; ++k) {
        if ((U + k) * T + lane >= n_acc) {
            const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int m = 0; m < M; ++m) st[(k * M + m) * T + lane] = zero;
        }
    }

    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
        const int64_t r = opaque_row(row);
        const int t = opaque_lane(lane);
        const rsrc_t rx = row_rsrc_ld(a.x, r, a.rows, a.ld_x * ES, h * ES);
        const rsrc_t ro = row_rsrc_ld(a.out, r, a.rows, a.ld_out * ES, h * ES);
        rsrc_t rr = rx;
        if constexpr (kFused) rr = row_rsrc_ld(a.residual, r, a.rows, a.ld_res * ES, h * ES);
        // the row's staged accesses, slot by slot, then its register accesses
        {
            const desc4 dx = row_desc(a.x, r, a.rows, a.ld_x * ES, h * ES);
            desc4 dr = dx;
            if constexpr (kFused) dr = row_desc(a.residual, r, a.rows, a.ld_res * ES, h * ES);
#pragma unroll
            for (int k = 0; k < L; ++k) {
                lds_load16(dx, ((U + k) * T + t) * 16, st_lds + (uint32_t)(k * M) * T * 16u);
                if constexpr (kFused)
                    lds_load16(dr, ((U + k) * T + t) * 16,
                               st_lds + (uint32_t)(k * M + 1) * T * 16u);
            }
        }
        u32x4 x0[U], r0[kFused ? U : 1];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            x0[u] = load16<kCachePolicyNT>(rx, (u * T + t) * 16);
            if constexpr (kFused) r0[u] = load16<kCachePolicyNT>(rr, (u * T + t) * 16);
        }

        // pass 1: the staged accesses as they land (each slot's M loads are
        // followed by M per later slot and the M U register loads), then the
        // registers, pinned below the slots so that no use of them, and so no
        // wait for them, moves above
        float p0 = 0.0f, p1 = 0.0f, n_l = 0.0f;
#pragma unroll
        for (int k = 0; k < L; ++k) {
            wait_vm_at_most(M * (L - 1 - k) + M * U);
            u32x4 xv[1] = {st[(k * M) * T + t]};
            u32x4 rv[1] = {kFused ? st[(k * M + 1) * T + t] : xv[0]};
            stream_stat_step<E, OP, 1, T>(xv, rv, (U + k) * T + t, n_acc, p0, p1, n_l);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            asm volatile("" : "+v"(x0[u]));
            if constexpr (kFused) asm volatile("" : "+v"(r0[u]));
        }
        stream_stat_step<E, OP, U, T>(x0, r0, t, n_acc, p0, p1, n_l);
        // the weights (and bias) of the whole row, packed, landing during the
        // reduction
        u32x4 wv[NB], bv[kLn ? NB : 1];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            wv[b] = load16<0>(rw, (b * T + t) * 16);
            if constexpr (kLn) bv[b] = load16<0>(rb, (b * T + t) * 16);
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

        // pass 2: the register accesses, then the slots
#pragma unroll
        for (int u = 0; u < U; ++u)
            stage_norm_access<E, OP>(x0[u], r0[kFused ? u : 0], wv[u], bv[kLn ? u : 0], rr, ro,
                                     (u * T + t) * 16, mu, rstd);
#pragma unroll
        for (int k = 0; k < L; ++k) {
            const u32x4 xv = st[(k * M) * T + t];
            const u32x4 rv = kFused ? st[(k * M + 1) * T + t] : xv;
            stage_norm_access<E, OP>(xv, rv, wv[U + k], bv[kLn ? U + k : 0], rr, ro,
                                     ((U + k) * T + t) * 16, mu, rstd);
        }
        // this wave's reads of its slots are done before the next row's loads
        // overwrite them; the next row's first reduction must not overwrite
        // slots still being read
        wait_lds();
        __syncthreads();
    }
}

template <typename E, int OP, int U, int L>
hipError_t launch_stage_fwd(const DynFwdArgs& a, hipStream_t stream) {
    const int64_t grid = a.rows < kStageGridRows ? a.rows : kStageGridRows;
    if (grid > 0)
        hipLaunchKernelGGL((stage_fwd_kernel<E, OP, U, L>), dim3((unsigned)grid),
                           dim3(kStreamFwdLanes), 0, stream, a);
    return hipGetLastError();
}

// ---- forward, short fp32 rows: several rows a wave ---------------------------------
// A row of up to 4 G U values (G lanes x U 16-byte accesses, G = 8, 16 or 32)
// is held by a lane group of G lanes; a 256-lane workgroup holds 256 / G rows,
// walking the row sets blockIdx.x, + gridDim.x, ...  One buffer descriptor
// covers a workgroup's set of rows and each lane adds its row's offset (an
// access past its row's end gets an offset past the descriptor's range: it
// loads zeros and stores nothing).  The row's reductions stay inside its lane
// group (DPP and one cross-lane swap, no LDS, no barrier).  LayerNorm takes
// the two passes over the row in registers: mean, then the centered sum of
// squares of the row's values (accesses past the end left out).
constexpr int kGroupBlock = 256;

template <int OP, int G, int U>
__global__ __launch_bounds__(kGroupBlock) void group_fwd_kernel(DynFwdArgs a) {
    static_assert(G == 8 || G == 16 || G == 32, "rows narrower than a wave");
    constexpr int R = kGroupBlock / G;  // rows a workgroup
    constexpr bool kFused = OP == kSplitFused, kLn = OP == kSplitLn;
    const int lane = threadIdx.x;
    const int g = lane / G, gl = lane % G;
    const int h = a.hidden;
    const float inv_h = 1.0f / (float)h;
    const rsrc_t rw = row_rsrc_ld(a.weight, 0, 1, 0, h * 4);
    rsrc_t rb = rw;
    if constexpr (kLn) rb = row_rsrc_ld(a.bias, 0, 1, 0, h * 4);
    u32x4 wv[U], bv[kLn ? U : 1];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int col = (gl + u * G) * 4;
        const int off = col < h ? col * 4 : kOutOfRange;
        wv[u] = load16<0>(rw, off);
        if constexpr (kLn) bv[u] = load16<0>(rb, off);
    }
    for (int64_t first = (int64_t)blockIdx.x * R; first < a.rows;
         first += (int64_t)gridDim.x * R) {
        const int64_t r0 = opaque_row(first);
        const rsrc_t rx = rows_rsrc<G>(a.x, r0, R, a.rows, a.ld_x, h, 4);
        const rsrc_t ro = rows_rsrc<G>(a.out, r0, R, a.rows, a.ld_out, h, 4);
        rsrc_t rr = rx;
        if constexpr (kFused) rr = rows_rsrc<G>(a.residual, r0, R, a.rows, a.ld_res, h, 4);
        int off_x[U], off_o[U], off_r[U];
        float s[U][4];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int col = (gl + u * G) * 4;
            off_x[u] = set_off<G>(g, col, a.ld_x, h, 4);
            off_o[u] = set_off<G>(g, col, a.ld_out, h, 4);
            off_r[u] = kFused ? set_off<G>(g, col, a.ld_res, h, 4) : 0;
        }
        u32x4 xv[U], rv[kFused ? U : 1];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            xv[u] = load16<kCachePolicyNT>(rx, off_x[u]);
            if constexpr (kFused) rv[u] = load16<kCachePolicyNT>(rr, off_r[u]);
        }
        float p0 = 0.0f;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            unpack16<float>(xv[u], s[u]);
            if constexpr (kFused) {
                float rf[4];
                unpack16<float>(rv[u], rf);
#pragma unroll
                for (int e = 0; e < 4; ++e) s[u][e] += rf[e];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) p0 += kLn ? s[u][e] : s[u][e] * s[u][e];
        }
        p0 = group_sum<G>(p0);  // past the end: zeros, add nothing
        float mu = 0.0f, rstd;
        if constexpr (kLn) {
            mu = p0 * inv_h;
            float p1 = 0.0f;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const bool in = (gl + u * G) * 4 < h;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float d = s[u][e] - mu;
                    p1 += in ? d * d : 0.0f;
                }
            }
            rstd = fast_rsqrt(group_sum<G>(p1) * inv_h + a.eps);
            const int64_t row = r0 + g;
            if (gl == 0 && row < a.rows && a.mean != nullptr) {
                a.mean[row] = mu;
                a.rstd[row] = rstd;
            }
        } else {
            rstd = fast_rsqrt(p0 * inv_h + a.eps);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float wf[4], o[4];
            unpack16<float>(wv[u], wf);
            if constexpr (kFused) store16(rr, off_r[u], pack16<float>(s[u]));
            if constexpr (kLn) {
                float bf[4];
                unpack16<float>(bv[u], bf);
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = (s[u][e] - mu) * rstd * wf[e] + bf[e];
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = s[u][e] * rstd * wf[e];
            }
            store16(ro, off_o[u], pack16<float>(o));
        }
    }
}

template <int OP, int G, int U>
hipError_t launch_group_fwd(const DynFwdArgs& a, hipStream_t stream) {
    constexpr int R = kGroupBlock / G;
    const int64_t sets = (a.rows + R - 1) / R;
    const int64_t grid = sets < kStreamMaxGrid ? sets : kStreamMaxGrid;
    hipLaunchKernelGGL((group_fwd_kernel<OP, G, U>), dim3((unsigned)grid), dim3(kGroupBlock), 0,
                       stream, a);
    return hipGetLastError();
}

// ---- backward: the rows' two reductions ------------------------------------------
template <typename E, bool LN>
__global__ __launch_bounds__(kStreamFwdLanes) void stream_bwd_stats_kernel(DynBwdArgs a,
                                                                           float* stats) {
    constexpr int T = kStreamFwdLanes;
    constexpr int U = kStreamUnroll;
    constexpr int EP = Elems<E>::kPer;
    constexpr int ES = (int)sizeof(E);
    __shared__ float red[2 * 2 * (T / kWave)];
    const int lane = threadIdx.x;
    const int h = a.hidden;
    const int n_acc = h / EP;
    const float inv_h = 1.0f / (float)h;
    const rsrc_t rw = row_rsrc_ld(a.weight, 0, 1, 0, h * ES);
    int parity = 0;
    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
        const int64_t r = opaque_row(row);
        const rsrc_t rx = row_rsrc_ld(a.x, r, a.rows, a.ld_x * ES, h * ES);
        const rsrc_t rd = row_rsrc_ld(a.dy, r, a.rows, a.ld_dy * ES, h * ES);
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
                xv[u] = load16<kStreamPass1>(rx, off);
                dv[u] = load16<kStreamPass1>(rd, off);
                wv[u] = load16<0>(rw, off);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float xf[EP], df[EP], wf[EP];
                unpack16<E>(xv[u], xf);
                unpack16<E>(dv[u], df);
                unpack16<E>(wv[u], wf);
#pragma unroll
                for (int e = 0; e < EP; ++e) {
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
    bool in;                       // a row of the matrix (not past its end)
};

// Loads row `row` of the tile whose first access is acc0 (a row past the end
// loads zeros from no memory and statistics of zero, so it adds nothing).
// INROW: the tile is the whole row and its statistics are reduced from the
// loaded row (tile_row), not read from the stats kernel's output.
template <typename E, int V, bool LN, bool DRES, bool INROW, bool XCH, int T>
__device__ __forceinline__ void load_tile_row(TileRow<V, DRES>& t, const DynBwdArgs& a,
                                              const float* stats, int64_t row, int acc0,
                                              int lane) {
    constexpr int ES = (int)sizeof(E);
    const int h = a.hidden;
    const rsrc_t rx = row_rsrc_ld(a.x, row, a.rows, a.ld_x * ES, h * ES);
    const rsrc_t rd = row_rsrc_ld(a.dy, row, a.rows, a.ld_dy * ES, h * ES);
#pragma unroll
    for (int b = 0; b < V; ++b) t.x[b] = load16<kCachePolicyNT>(rx, (acc0 + b * T + lane) * 16);
#pragma unroll
    for (int b = 0; b < V; ++b) t.dy[b] = load16<kCachePolicyNT>(rd, (acc0 + b * T + lane) * 16);
    if constexpr (DRES) {
        const rsrc_t rr = row_rsrc_ld(a.dres, row, a.rows, a.ld_dres * ES, h * ES);
#pragma unroll
        for (int b = 0; b < V; ++b)
            t.dres[b] = load16<kCachePolicyNT>(rr, (acc0 + b * T + lane) * 16);
    }
    const bool in = row < a.rows;
    const int64_t rc = in ? row : a.rows - 1;
    t.in = in;
    if constexpr (!INROW && !XCH) {
        const float s0 = stats[2 * rc], s1 = stats[2 * rc + 1];
        t.s0 = in ? s0 : 0.0f;
        t.s1 = in ? s1 : 0.0f;
    }
    if constexpr (LN) {
        if constexpr ((XCH && kXchVecStats) || (INROW && kInrowVecStats)) {
            // vector loads (the row index made opaque in vector registers):
            // counted with the row's own loads, not with the LDS reductions'
            // scalar counter; the uses zero a past-end row's values, a select
            // here would wait.  32 bits where the host keeps rows below 2^31
            // (the exchange), 64 for the one-tile kernel (any row count).
            if constexpr (XCH) {
                const int ri = opaque_lane((int)rc);
                t.mean = a.mean[ri];
                t.rstd = a.rstd[ri];
            } else {
                int64_t ri = rc;
                asm volatile("" : "+v"(ri));
                t.mean = a.mean[ri];
                t.rstd = a.rstd[ri];
            }
        } else {
            const float m = a.mean[rc], q = a.rstd[rc];
            t.mean = in ? m : 0.0f;
            t.rstd = in ? q : 0.0f;
        }
    }
}

// The two per-lane sums of the row's backward over V accesses a lane (the
// stats kernel's and INROW's terms: LayerNorm sum g and sum g xhat, RMSNorm
// sum x^2 and sum g x; g = dy w).
template <typename E, bool LN>
__device__ __forceinline__ void accumulate_access(const u32x4& x, const u32x4& dy,
                                                  const u32x4& w, float mean, float rstd,
                                                  float& s1, float& s2) {
    constexpr int EP = Elems<E>::kPer;
    float xf[EP], df[EP], wf[EP];
    unpack16<E>(x, xf);
    unpack16<E>(dy, df);
    unpack16<E>(w, wf);
#pragma unroll
    for (int e = 0; e < EP; ++e) {
        const float g = df[e] * wf[e];
        if constexpr (LN) {
            s1 += g;
            s2 += g * ((xf[e] - mean) * rstd);
        } else {
            s1 += xf[e] * xf[e];
            s2 += g * xf[e];
        }
    }
}

template <typename E, int V, bool LN>
__device__ __forceinline__ void tile_sums(const u32x4 (&x)[V], const u32x4 (&dy)[V],
                                          const u32x4 (&wv)[V], float mean, float rstd,
                                          float& s1, float& s2) {
    s1 = 0.0f;
    s2 = 0.0f;
#pragma unroll
    for (int b = 0; b < V; ++b) accumulate_access<E, LN>(x[b], dy[b], wv[b], mean, rstd, s1, s2);
}

// ---- the column tiles of a row exchange their partial sums ---------------------------
// Each (walker, tile) workgroup forms its tile's two sums for the D rows of
// its ring at once (one reduction over the workgroup for all 2 D values) and
// publishes them; a row's sums are the tiles' partials added in tile order,
// so every tile of the row, and every run, gets the same bits.  A partial
// goes out as one device-coherent 64-bit word (value bits << 32 | row + 1),
// the tag naming the row, in slot (walk step mod kXchRing, tile, which) of
// the walker's part of the exchange area, which the host zero-fills before
// the launch (a tag of 0 names no row).  One round trip of polls covers the
// group's D rows.  A tile publishes group g + 1 only after it has read every
// partial of group g, and a partner publishes group g + 2 only after this
// tile has published group g + 1, so slots of steps k and k + 2 D may share:
// kXchRing >= 2 D.  Waits are bounded: a tile that runs out of polls (a
// partner not resident, or the host's spin limit) stops waiting for the rest
// of its walk and reads the other tiles of each row itself, forming their
// partials exactly as their own workgroups do (same lanes, same order): the
// same bits, from a second read of the row.

// Sum over the workgroup of N values a lane (wave sums, then the waves' totals
// added in wave order, as row_sum2 does for two): one barrier for all N.
template <int T, int N>
__device__ __forceinline__ void row_sum_n(float (&v)[N], float* slot, int lane) {
    constexpr int kWaves = T / kWave;
#pragma unroll
    for (int j = 0; j < N; ++j) v[j] = wave_sum(v[j]);
    const int w = lane / kWave;
    if ((lane & (kWave - 1)) == 0) {
#pragma unroll
        for (int j = 0; j < N; ++j) slot[N * w + j] = v[j];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < N; ++j) {
        float t = slot[j];
#pragma unroll
        for (int i = 1; i < kWaves; ++i) t += slot[N * i + j];
        v[j] = t;
    }
}

__device__ __forceinline__ uint64_t xch_word(float v, int64_t row) {
    return ((uint64_t)__float_as_uint(v) << 32) | ((uint64_t)(row + 1) & 0xffffffffu);
}

// The row's sums from a re-read of the other tiles (this tile's own partials
// s1, s2 as formed): tile by tile, each formed as its own workgroup forms it,
// then added in tile order.  Plain loads (no buffer descriptors held in
// scalar registers on this rare path).  Uniform control flow.
template <typename E, int V, bool LN, int T>
__device__ __forceinline__ void xch_reread_row(const DynBwdArgs& a, int64_t row, int tiles,
                                               int tile, float s1, float s2, float mean,
                                               float rstd, float* redf, int lane, float& S1,
                                               float& S2) {
    constexpr int EP = Elems<E>::kPer;
    constexpr int ES = (int)sizeof(E);
    const int h = a.hidden;
    // the row's byte offsets in vector registers (this path holds no more
    // scalar registers than the walk around it)
    int64_t xo = row * a.ld_x * ES, dyo = row * a.ld_dy * ES;
    asm volatile("" : "+v"(xo));
    asm volatile("" : "+v"(dyo));
    const char* xr = static_cast<const char*>(a.x) + xo;
    const char* dr = static_cast<const char*>(a.dy) + dyo;
    const char* wr = static_cast<const char*>(a.weight);
    const u32x4 zero = {0u, 0u, 0u, 0u};
    for (int tp = 0; tp < tiles; ++tp) {
        float p1 = s1, p2 = s2;  // this tile's own partials: the same bits
        if (tp != tile) {
            const int acc0 = tp * (T * V);
            p1 = 0.0f;
            p2 = 0.0f;
#pragma unroll 1
            for (int b = 0; b < V; ++b) {  // in the order tile_sums adds them
                const int idx = acc0 + b * T + lane;
                const bool in = idx * EP < h;  // past the row's end: zeros, as a buffer load
                const int64_t off = (int64_t)idx * 16;
                const u32x4 xv = in ? *reinterpret_cast<const u32x4*>(xr + off) : zero;
                const u32x4 dv = in ? *reinterpret_cast<const u32x4*>(dr + off) : zero;
                const u32x4 wv = in ? *reinterpret_cast<const u32x4*>(wr + off) : zero;
                accumulate_access<E, LN>(xv, dv, wv, mean, rstd, p1, p2);
            }
            row_sum2<T>(p1, p2, redf, lane);
            __syncthreads();  // the slots serve the next tile's reduction
        }
        if (tp == 0) {
            S1 = p1;
            S2 = p2;
        } else {
            S1 += p1;
            S2 += p2;
        }
    }
}

template <typename E, int V, bool LN, bool DRES, bool INROW, int T>
__device__ __forceinline__ void tile_row(TileRow<V, DRES>& t, const u32x4 (&wv)[V],
                                         float (&pw)[V][Elems<E>::kPer],
                                         float (&pb)[LN ? V : 1][Elems<E>::kPer],
                                         const DynBwdArgs& a, int64_t row, int acc0, int lane,
                                         float* red) {
    constexpr int EP = Elems<E>::kPer;
    constexpr int ES = (int)sizeof(E);
    if constexpr (INROW) {
        // the row's two reductions, as stream_bwd_stats_kernel forms them
        const float tmi = LN && t.in ? t.mean : 0.0f, tri = LN && t.in ? t.rstd : 0.0f;
        float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
        for (int b = 0; b < V; ++b) {
            float xf[EP], df[EP], wf[EP];
            unpack16<E>(t.x[b], xf);
            unpack16<E>(t.dy[b], df);
            unpack16<E>(wv[b], wf);
#pragma unroll
            for (int e = 0; e < EP; ++e) {
                const float g = df[e] * wf[e];
                if constexpr (LN) {
                    s1 += g;
                    s2 += g * ((xf[e] - tmi) * tri);
                } else {
                    s1 += xf[e] * xf[e];
                    s2 += g * xf[e];
                }
            }
        }
        row_sum2<T>(s1, s2, red, lane);
        const float inv_h = 1.0f / (float)a.hidden;
        if constexpr (LN) {
            t.s0 = s1 * inv_h;
            t.s1 = s2 * inv_h;
        } else {
            const float rstd = fast_rsqrt(s1 * inv_h + a.eps);
            t.s0 = rstd;
            t.s1 = rstd * rstd * rstd * s2 * inv_h;
        }
        if (!t.in) {  // a row past the end adds nothing (rsqrt(eps) may be infinite)
            t.s0 = 0.0f;
            t.s1 = 0.0f;
        }
    }
    const rsrc_t rdx = row_rsrc_ld(a.dx, row, a.rows, a.ld_dx * ES, a.hidden * ES);
    // LayerNorm: a past-end row's statistics are zero (loads may leave them raw)
    const float tm = LN && t.in ? t.mean : 0.0f, tr = LN && t.in ? t.rstd : 0.0f;
#pragma unroll
    for (int b = 0; b < V; ++b) {
        float xf[EP], df[EP], wf[EP], o[EP];
        unpack16<E>(t.x[b], xf);
        unpack16<E>(t.dy[b], df);
        unpack16<E>(wv[b], wf);
#pragma unroll
        for (int e = 0; e < EP; ++e) {
            const float g = df[e] * wf[e];
            if constexpr (LN) {
                const float xh = (xf[e] - tm) * tr;
                o[e] = tr * (g - t.s0 - xh * t.s1);
                pw[b][e] += df[e] * xh;
                pb[b][e] += df[e];
            } else {
                o[e] = t.s0 * g - t.s1 * xf[e];
                pw[b][e] += df[e] * (xf[e] * t.s0);
            }
        }
        if constexpr (DRES) {
            float rf[EP];
            unpack16<E>(t.dres[b], rf);
#pragma unroll
            for (int e = 0; e < EP; ++e) o[e] += rf[e];
        }
        store16(rdx, (acc0 + b * T + lane) * 16, pack16<E>(o));
    }
}

// Zero-fills n 16-byte words (the exchange area before an XCH launch).  A
// kernel, not a memset, so that graphs capturing the call record no memset
// node.
__global__ __launch_bounds__(256) void stream_zero_kernel(u32x4* p, int64_t n) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        p[i] = z;
}

// Grid: walkers * tiles workgroups; workgroup i is tile i % tiles of walker
// i / tiles.  The row's two reductions: with XCH, exchanged between the row's
// tiles through `xch` (zeroed before the launch; kXchRing walk steps of
// `tiles` slot pairs per walker; a wait gives up after spin_limit polls);
// with INROW (one tile holds the whole row), reduced here from the row in
// registers; else read from `stats` (stream_bwd_stats_kernel ran before on
// the same stream).
template <typename E, int V, bool LN, bool DRES, int D, bool INROW = false, bool XCH = false>
__global__ __launch_bounds__(kStreamTileLanes) void stream_bwd_tile_kernel(
    DynBwdArgs a, const float* stats, int tiles, uint64_t* xch, uint32_t spin_limit) {
    // lanes: the exchange's kXchLanesBf16 / kXchLanesF32, else kStreamTileLanes
    constexpr int T = !XCH ? kStreamTileLanes : sizeof(E) == 2 ? kXchLanesBf16 : kXchLanesF32;
    constexpr int EP = Elems<E>::kPer;
    constexpr int ES = (int)sizeof(E);
    static_assert(!(INROW && XCH), "one way to form the row's sums");
    // two sums per wave, two sets used alternately so that a row's reduction
    // never overwrites slots the previous row's lanes may still be reading
    __shared__ float red[INROW ? 2 * 2 * (T / kWave) : XCH ? 2 * 2 * D * (T / kWave) : 1];
    // XCH: the group's partials, row d of tile tp at [d * kXchMaxTiles + tp]
    __shared__ float xq1[XCH ? D * kXchMaxTiles : 1], xq2[XCH ? D * kXchMaxTiles : 1];
    __shared__ float redf[XCH ? 2 * (T / kWave) : 1];
    // XCH: the workgroup's own partials of each ring's group (for a re-read)
    __shared__ float xown[XCH ? 2 * 2 * D : 1];
    __shared__ int xflag[XCH ? T / kWave : 1];
    int parity = 0;
    const int lane = threadIdx.x;
    const int tile = blockIdx.x % tiles;
    const int64_t walker = blockIdx.x / tiles;
    // XCH: the workspace pointer waits in VGPRs through the walk (it is used
    // once, at the end), leaving the scalar registers to the walk
    uint32_t ws_lo = (uint32_t)(uintptr_t)a.workspace;
    uint32_t ws_hi = (uint32_t)((uintptr_t)a.workspace >> 32);
    if constexpr (XCH) asm volatile("" : "+v"(ws_lo), "+v"(ws_hi));
    const int64_t P = gridDim.x / tiles;
    const int acc0 = tile * (T * V);  // the tile's first 16-byte access
    const int h = a.hidden;
    const rsrc_t rw = row_rsrc_ld(a.weight, 0, 1, 0, h * ES);
    u32x4 wv[V];
#pragma unroll
    for (int b = 0; b < V; ++b) wv[b] = load16<0>(rw, (acc0 + b * T + lane) * 16);
    float pw[V][EP], pb[LN ? V : 1][EP];
#pragma unroll
    for (int b = 0; b < V; ++b)
#pragma unroll
        for (int e = 0; e < EP; ++e) pw[b][e] = 0.0f;
#pragma unroll
    for (int b = 0; b < (LN ? V : 1); ++b)
#pragma unroll
        for (int e = 0; e < EP; ++e) pb[b][e] = 0.0f;

    const int64_t n = walker < a.rows ? (a.rows - 1 - walker) / P + 1 : 0;
    TileRow<V, DRES> buf[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
        load_tile_row<E, V, LN, DRES, INROW, XCH, T>(buf[d], a, stats, opaque_row(walker + d * P),
                                                  acc0, lane);
        issue_fence();
    }
    if constexpr (XCH) {
        // The ring's D rows are one group: their partials in one reduction,
        // their exchange in one round trip of polls, then dx row by row.
        // AHEAD (bf16; fp32 with two rings of 2 rows, the fused op of 1): two
        // rings, the group at i + D published before the group at i is waited
        // on, so the round trip overlaps a group's loads and sums.
        constexpr bool AHEAD =
            kXchAhead && (ES == 2 || (kXchAheadF32 && (!DRES || kXchAheadF32Dres)));
        constexpr int kStep = AHEAD ? 2 * D : D;  // walk steps between a ring's groups
        static_assert(AHEAD ? 4 * D <= kXchRing : 2 * D <= kXchRing,
                      "slots of the groups other tiles may still read");
        uint64_t* mine = xch + walker * kXchRing * tiles * 2;
        bool sticky = false;  // a wait ran out: re-read rows for the rest of the walk
        const float inv_h = 1.0f / (float)h;
        const int nw = (int)n;  // a walker's rows: the host keeps rows below 2^31

        // the group at walk step i in ring k: partials of its rows (past the
        // walk's end: zeros) reduced over the workgroup, rows < nw published
        // and kept in xown; returns the group's first row
        auto sums_publish = [&](TileRow<V, DRES>(&rb)[D], int k, int i)
                                __attribute__((always_inline)) {
            float v[2 * D];
#pragma unroll
            for (int d = 0; d < D; ++d)
                tile_sums<E, V, LN>(rb[d].x, rb[d].dy, wv, rb[d].in ? rb[d].mean : 0.0f,
                                    rb[d].in ? rb[d].rstd : 0.0f, v[2 * d], v[2 * d + 1]);
            row_sum_n<T, 2 * D>(v, red + parity * 2 * D * (T / kWave), lane);
            parity ^= 1;
            const int64_t r0 = opaque_row(walker + i * P);
            const int nd = nw - i < D ? nw - i : D;
            if (lane < nd) {  // lane d (of wave 0) publishes row d
                // an opaque lane: the lane == d masks are formed here, not
                // hoisted to live across the walk
                const int ld = opaque_lane(lane);
                float p1 = v[0], p2 = v[1];
#pragma unroll
                for (int d = 1; d < D; ++d) {
                    p1 = ld == d ? v[2 * d] : p1;
                    p2 = ld == d ? v[2 * d + 1] : p2;
                }
                const int64_t row = r0 + lane * P;
                xown[k * 2 * D + 2 * lane] = p1;
                xown[k * 2 * D + 2 * lane + 1] = p2;
                uint64_t* me = mine + (((i + lane) % kXchRing) * tiles + tile) * 2;
                __hip_atomic_store(&me[0], xch_word(p1, row), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(&me[1], xch_word(p2, row), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            }
            return r0;
        };

        // the group at walk step i (i < nw, published): its row sums, dx of
        // its rows, the ring reloaded with the rows kStep steps on
        auto poll_finish = [&](TileRow<V, DRES>(&rb)[D], int k, int i, int64_t r0)
                               __attribute__((always_inline)) {
            const int nd = nw - i < D ? nw - i : D;
            // every lane of the workgroup waits on its own slot pair (one pair
            // a lane while nd * tiles <= T), so the group's polls are in
            // flight together rather than one after another in one wave
            bool seen = true;
            if (!sticky) {
                for (int p = lane; p < nd * tiles; p += T) {
                    const int d = p / tiles, tp = p - d * tiles;
                    const int64_t row = r0 + d * P;
                    const uint64_t tag = (uint64_t)(row + 1) & 0xffffffffu;
                    const uint64_t* slot = mine + (((i + d) % kXchRing) * tiles + tp) * 2;
                    uint64_t u = 0, w = 0;
                    bool ok = false;
                    for (uint32_t polls = 0; polls < spin_limit; ++polls) {
                        if ((u & 0xffffffffu) != tag)
                            u = __hip_atomic_load(&slot[0], __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
                        if ((w & 0xffffffffu) != tag)
                            w = __hip_atomic_load(&slot[1], __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
                        if ((u & 0xffffffffu) == tag && (w & 0xffffffffu) == tag) {
                            ok = true;
                            break;
                        }
                        __builtin_amdgcn_s_sleep(1);
                    }
                    xq1[d * kXchMaxTiles + tp] = __uint_as_float((uint32_t)(u >> 32));
                    xq2[d * kXchMaxTiles + tp] = __uint_as_float((uint32_t)(w >> 32));
                    seen = seen && ok;
                }
            }
            const bool wave_seen = __builtin_amdgcn_ballot_w64(!seen) == 0;
            if ((lane & (kWave - 1)) == 0) xflag[lane / kWave] = wave_seen ? 1 : 0;
            __syncthreads();
            bool all = !sticky;
#pragma unroll
            for (int k = 0; k < T / kWave; ++k) all = all && xflag[k] != 0;
            sticky = !all;
#pragma unroll
            for (int d = 0; d < D; ++d) {
                float S1 = 0.0f, S2 = 0.0f;
                if (d < nd) {
                    if (all) {
                        // opaque here, so that the unrolled loop's trip-count
                        // values are not hoisted to live across the whole walk
                        int nt = tiles;
                        asm volatile("" : "+s"(nt));
                        S1 = xq1[d * kXchMaxTiles];
                        S2 = xq2[d * kXchMaxTiles];
                        for (int tp = 1; tp < nt; ++tp) {
                            S1 += xq1[d * kXchMaxTiles + tp];
                            S2 += xq2[d * kXchMaxTiles + tp];
                        }
                    } else {
                        xch_reread_row<E, V, LN, T>(a, r0 + d * P, tiles, tile,
                                                 xown[k * 2 * D + 2 * d],
                                                 xown[k * 2 * D + 2 * d + 1],
                                                 rb[d].in ? rb[d].mean : 0.0f,
                                                 rb[d].in ? rb[d].rstd : 0.0f, redf, lane, S1,
                                                 S2);
                    }
                }
                TileRow<V, DRES>& t = rb[d];
                if constexpr (LN) {
                    t.s0 = S1 * inv_h;
                    t.s1 = S2 * inv_h;
                } else {
                    const float rs = fast_rsqrt(S1 * inv_h + a.eps);
                    t.s0 = rs;
                    t.s1 = rs * rs * rs * S2 * inv_h;
                }
                if (!t.in) {  // a row past the end adds nothing
                    t.s0 = 0.0f;
                    t.s1 = 0.0f;
                }
                // dx unpacks the row again rather than keep the sums' unpacked
                // values live across the exchange
#pragma unroll
                for (int b = 0; b < V; ++b) {
                    asm volatile("" : "+v"(t.x[b]));
                    asm volatile("" : "+v"(t.dy[b]));
                }
            }
#pragma unroll
            for (int d = 0; d < D; ++d) {
                const int64_t r = opaque_row(walker + (i + d) * P);
                tile_row<E, V, LN, DRES, false, T>(rb[d], wv, pw, pb, a, r, acc0, lane, nullptr);
                issue_fence();
                load_tile_row<E, V, LN, DRES, INROW, XCH, T>(rb[d], a, stats, r + kStep * P, acc0,
                                                          lane);
                issue_fence();
            }
        };

        if constexpr (AHEAD) {
            TileRow<V, DRES> buf2[D];
#pragma unroll
            for (int d = 0; d < D; ++d) {
                load_tile_row<E, V, LN, DRES, INROW, XCH, T>(
                    buf2[d], a, stats, opaque_row(walker + (D + d) * P), acc0, lane);
                issue_fence();
            }
            sums_publish(buf, 0, 0);
            for (int i = 0; i < nw; i += 2 * D) {
                sums_publish(buf2, 1, i + D);
                poll_finish(buf, 0, i, opaque_row(walker + i * P));
                if (i + D >= nw) break;
                sums_publish(buf, 0, i + 2 * D);
                poll_finish(buf2, 1, i + D, opaque_row(walker + (i + D) * P));
            }
        } else {
            for (int i = 0; i < nw; i += D) {
                poll_finish(buf, 0, i, sums_publish(buf, 0, i));
            }
        }
    } else {
        for (int64_t i = 0; i < n; i += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                const int64_t r = opaque_row(walker + (i + d) * P);
                tile_row<E, V, LN, DRES, INROW, T>(buf[d], wv, pw, pb, a, r, acc0, lane,
                                                red + parity * 2 * (T / kWave));
                parity ^= 1;
                issue_fence();
                load_tile_row<E, V, LN, DRES, INROW, XCH, T>(buf[d], a, stats, r + D * P, acc0,
                                                          lane);
                issue_fence();
            }
        }
    }

    // this tile's columns of slab `walker`: [outs][padded]; columns past the
    // padded width are dropped by the descriptors' range
    const int padded = (h + 63) / 64 * 64;
    const int outs = LN ? 2 : 1;
    float* ws = a.workspace;
    if constexpr (XCH)
        ws = (float*)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)ws_hi) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)ws_lo));
    float* slab = ws + walker * outs * (int64_t)padded;
    const rsrc_t sw = __builtin_amdgcn_make_buffer_rsrc(slab, (short)0, padded * 4, kRsrcWord3);
    const rsrc_t sb = __builtin_amdgcn_make_buffer_rsrc(slab + padded, (short)0,
                                                        LN ? padded * 4 : 0, kRsrcWord3);
#pragma unroll
    for (int b = 0; b < V; ++b) {
        const int off = (acc0 + b * T + lane) * EP * 4;  // byte offset of the access's first column
#pragma unroll
        for (int q = 0; q < EP / 4; ++q) {
            const f32x4 w4 = {pw[b][4 * q], pw[b][4 * q + 1], pw[b][4 * q + 2], pw[b][4 * q + 3]};
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, w4), sw,
                                                   off + 16 * q, 0, 0);
            if constexpr (LN) {
                const f32x4 b4 = {pb[b][4 * q], pb[b][4 * q + 1], pb[b][4 * q + 2],
                                  pb[b][4 * q + 3]};
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, b4), sb,
                                                       off + 16 * q, 0, 0);
            }
        }
    }
}

}  // namespace rownorm
