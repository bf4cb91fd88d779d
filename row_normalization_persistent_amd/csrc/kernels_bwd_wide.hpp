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
// after the reduction.  One two-value reduction over the 8 waves (LDS, one
// barrier) per row.  There is room in LDS for one row only, so the walk is
// pipelined by access instead of by row: in the second pass over row i each
// lane, once it has read access b of x and dy, issues row i+1's loads into
// the same two slots, and row i+1 streams in while row i is finished and
// stored (without this the memory pipe idled through every row's two passes
// and reduction).
// At the end each workgroup writes one slab of [G][outs][padded] column sums
// for the shared column-reduce kernel.
// The element type E is uint16_t (bf16 patterns, 8 a 16-byte access: hidden
// 16392 ... 32768) or float (4 an access: fp32 rows of 8196 ... 16384, whose
// column sums take half the registers and whose LDS footprint is that of a
// bf16 row twice as wide).
#pragma once

#include <type_traits>
#include <utility>

#include "dyn_common.hpp"
#include "launch.hpp"
#include "lds_stage.hpp"

namespace rownorm {

constexpr int kWideLanes = kWideBwdLanes;
// Waits until an access's x and dy have landed, `later` accesses (two loads
// each) having been issued after it (a constant once the caller's loop over
// the accesses is unrolled: one wait instruction).
__device__ __forceinline__ void wait_access_landed(int later) {
    switch (later) {
        case 0: wait_vm<0>(); break;
        case 1: wait_vm<2>(); break;
        case 2: wait_vm<4>(); break;
        case 3: wait_vm<6>(); break;
        case 4: wait_vm<8>(); break;
        case 5: wait_vm<10>(); break;
        case 6: wait_vm<12>(); break;
        case 7: wait_vm<14>(); break;
        default: wait_vm<16>(); break;
    }
}

// LDS access slots of the staged rows (LayerNorm): a ring of kWideSlots slots
// (x and dy of one access of all 512 lanes each, 16 KiB), of which a row
// takes V; row i's access b sits in slot (i V + b) mod kWideSlots, so the
// kWideSlots - V slots a row leaves free take the next row's first accesses
// before this row's first pass even starts.  Measured on MI355X (A/B in
// alternating processes, bitwise-equal outputs): LayerNorm bwd 8192 x 20480
// (4 accesses ahead) 191-196 -> 185-187 us, 8192 x 24576 223-229 -> 220-225
// us, 4096 x 32768 (1 ahead) level; RMSNorm level (+-0.5 %); the fused op's
// backward 2-2.5 % slower (its dres loads, issued after the head start, wait
// for it), so RMSNorm keeps V slots.  Build-time switch: 0 = V slots always.
#ifndef ROWNORM_WIDE_RING
#define ROWNORM_WIDE_RING 1
#endif
constexpr int kWideSlots = 9;  // 9 x 16 KiB + the reduction slots fit the 160 KiB of LDS

// The first pass over a row starts on access b as soon as b's two loads have
// landed instead of after the whole row (build-time switch for measurement).
#ifndef ROWNORM_WIDE_STAGED
#define ROWNORM_WIDE_STAGED 1
#endif

template <typename E, int V, bool LN, bool DRES>
__global__ __launch_bounds__(kWideLanes) void norm_bwd_wide_kernel(DynBwdArgs a) {
    constexpr int T = kWideLanes;
    constexpr int EP = Elems<E>::kPer;     // values a 16-byte access
    constexpr int ES = (int)sizeof(E);     // bytes a value
    constexpr int S = ROWNORM_WIDE_RING && LN ? kWideSlots : V;  // access slots in LDS
    constexpr int HS = S - V;                               // next-row accesses issued early
    static_assert(HS >= 0, "a row needs V slots");
    __shared__ u32x4 xs[S * T], ds[S * T];      // x and dy of the slots, 16 bytes per lane
    __shared__ float red[2 * 2 * (T / kWave)];  // two alternating two-value slots
    const int lane = threadIdx.x;
    const int wave_base = lane & ~(kWave - 1);
    const int h = a.hidden;
    const float inv_h = 1.0f / (float)h;
    // the weights stay in registers for the whole walk, packed (4 per access)
    const rsrc_t rw = row_rsrc_ld(a.weight, 0, 1, 0, h * ES);
    u32x4 wv[V];
#pragma unroll
    for (int b = 0; b < V; ++b) wv[b] = aload<8, 0>(rw, (b * T + lane) * 16);

    float pw[V][EP], pb[LN ? V : 1][EP];
#pragma unroll
    for (int b = 0; b < V; ++b)
#pragma unroll
        for (int k = 0; k < EP; ++k) pw[b][k] = 0.0f;
    if constexpr (LN) {
#pragma unroll
        for (int b = 0; b < V; ++b)
#pragma unroll
            for (int k = 0; k < EP; ++k) pb[b][k] = 0.0f;
    }

    // access b of lane t of a row: x and dy from HBM into their LDS slots
    // (slot b*T + t; the wave's 64 lanes write its 64 consecutive slots)
    // LDS byte addresses of the wave's first slot of access 0, wave uniform
    const uint32_t wave_slot = (uint32_t)__builtin_amdgcn_readfirstlane(wave_base) * 16u;
    const uint32_t xs_lds =
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)xs + wave_slot;
    const uint32_t ds_lds =
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)ds + wave_slot;
    // access b of a row into slot `slot`
    auto stage = [&](desc4 rx, desc4 rd, int b, int t, int slot) {
        lds_load16(rx, (b * T + t) * 16, xs_lds + slot * T * 16);
        lds_load16(rd, (b * T + t) * 16, ds_lds + slot * T * 16);
    };
    auto slot_of = [&](int base, int b) {  // (base + b) mod S, base < S, b < S
        const int sl = base + b;
        return sl >= S ? sl - S : sl;
    };
    auto x_rsrc = [&](int64_t row) { return row_desc(a.x, row, a.rows, a.ld_x * ES, h * ES); };
    auto dy_rsrc = [&](int64_t row) {
        return row_desc(a.dy, row, a.rows, a.ld_dy * ES, h * ES);
    };

    const int64_t G = gridDim.x;
    const int64_t first = blockIdx.x;
    const int64_t n = first < a.rows ? (a.rows - 1 - first) / G + 1 : 0;
    // The walk is software-pipelined by access: the second pass over a row
    // hands each access's LDS slots, once read, to the next row's loads, so
    // the next row streams in while this one is finished and stored.
    float mean_nx = 0.0f, rstd_nx = 0.0f;
    if (n > 0) {
        const desc4 rx = x_rsrc(first), rd = dy_rsrc(first);
#pragma unroll
        for (int b = 0; b < V; ++b) stage(rx, rd, b, lane, b);
        if constexpr (LN) {
            mean_nx = uniform_load_f32(a.mean, first, a.rows);
            rstd_nx = uniform_load_f32(a.rstd, first, a.rows);
        }
    }
    int parity = 0;
    int base = 0;  // slot of the row's access 0: (i V) mod S
    for (int64_t i = 0; i < n; ++i) {
        const int64_t row = opaque_row(first + i * G);
        const int64_t next = row + G;  // past the end (size-0 descriptors) after the last
        const float mean = mean_nx, rstd_in = rstd_nx;
        const desc4 nrx = x_rsrc(next), nrd = dy_rsrc(next);
        const int nbase = slot_of(base, V % S);  // the next row's access 0
        if constexpr (HS > 0) {
            // the next row's first HS accesses, into the slots the previous
            // row's last HS accesses left (this wave's reads of them are done)
            wait_lds();
#pragma unroll
            for (int b = 0; b < HS; ++b) stage(nrx, nrd, b, lane, slot_of(nbase, b));
        }
        // the row's loads (its LDS writes included); no LDS read may move above.
        // Staged: access b is read once b's x and dy have landed.  The row's
        // loads went out in access order (x then dy of each access; stores of
        // the previous row's dx and its dres loads between them), and after
        // them the next row's first HS accesses: 2 (V - 1 - b + HS) = 2 (S - 1
        // - b) loads follow b's dy.  Vector-memory operations retire in issue
        // order, so once no more than that many are outstanding, b's two loads
        // have landed whether or not the stores are counted.
        if constexpr (!ROWNORM_WIDE_STAGED) wait_all_counters();
        // lane offsets recomputed every row (an opaque lane index), not hoisted
        // out of the loop into registers held for the whole walk
        const int l = opaque_lane(lane);

        // the row's two sums (an access past the row's end, in the last b, is
        // left out whatever its LDS slot holds; hidden is a multiple of EP, so
        // an access is wholly inside the row or wholly past it)
        float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
        for (int b = 0; b < V; ++b) {
            if constexpr (ROWNORM_WIDE_STAGED) wait_access_landed(S - 1 - b);
            const bool in_row = (b * T + l) * EP < h;
            const int sl = slot_of(base, b);
            float xf[EP], df[EP], wf[EP];
            unpack16<E>(xs[sl * T + l], xf);
            unpack16<E>(ds[sl * T + l], df);
            unpack16<E>(wv[b], wf);
#pragma unroll
            for (int k = 0; k < EP; ++k) {
                xf[k] = in_row ? xf[k] : 0.0f;
                df[k] = in_row ? df[k] : 0.0f;
            }
#pragma unroll
            for (int k = 0; k < EP; ++k) {
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
        // (scalar loads, which the row's LDS waits also wait for: a 64-row
        // vector load per walk, read by readlane, measured level to 7 %
        // slower, 4096 x 32768 / 8192 x 32768 / 16384 x 16392)
        if constexpr (LN) {  // past the walk's last row: zeros, never used
            mean_nx = uniform_load_f32(a.mean, next, a.rows);
            rstd_nx = uniform_load_f32(a.rstd, next, a.rows);
        }
        // the second pass re-reads x, dy (LDS) and the weights (registers)
        // instead of keeping the first pass's values live across the
        // reduction: an opaque copy of the lane index keeps the compiler from
        // merging them
        const int t = opaque_lane(lane);

        const rsrc_t rdx = row_rsrc_ld(a.dx, row, a.rows, a.ld_dx * ES, h * ES);
        rsrc_t rr = rdx;
        if constexpr (DRES) rr = row_rsrc_ld(a.dres, row, a.rows, a.ld_dres * ES, h * ES);
        float c1 = 0.0f, c2 = 0.0f, rstd = 0.0f, coef = 0.0f;
        if constexpr (LN) {
            c1 = s1 * inv_h;
            c2 = s2 * inv_h;
        } else {
            // a row past the end must add exactly nothing, also at eps = 0
            rstd = row < a.rows ? fast_rsqrt(s1 * inv_h + a.eps) : 0.0f;
            coef = rstd * rstd * rstd * s2 * inv_h;
        }
        u32x4 dr[DRES ? V : 1];
        if constexpr (DRES) {
#pragma unroll
            for (int b = 0; b < V; ++b) dr[b] = aload<8, kCachePolicyNT>(rr, (b * T + lane) * 16);
        }
#pragma unroll
        for (int b = 0; b < V; ++b) {
            float xf[EP], df[EP], wf[EP], o[EP];
            const int sl = slot_of(base, b);
            unpack16<E>(xs[sl * T + t], xf);
            unpack16<E>(ds[sl * T + t], df);
            // this access's slot is read: hand it to the next row's access b +
            // HS (past the walk's last row the descriptors are empty: nothing
            // is read); the last HS slots wait for the row after next
            if (b + HS < V) {
                wait_lds();
                stage(nrx, nrd, b + HS, t, sl);
            }
            unpack16<E>(wv[b], wf);
#pragma unroll
            for (int k = 0; k < EP; ++k) {
                if constexpr (LN) {
                    const float xh = (xf[k] - mean) * rstd_in;
                    o[k] = rstd_in * (df[k] * wf[k] - c1 - xh * c2);
                    pw[b][k] += df[k] * xh;
                    pb[b][k] += df[k];
                } else {
                    o[k] = rstd * (df[k] * wf[k]) - coef * xf[k];
                    pw[b][k] += df[k] * (xf[k] * rstd);
                }
            }
            if constexpr (DRES) {
                float rf[EP];
                unpack16<E>(dr[b], rf);
#pragma unroll
                for (int k = 0; k < EP; ++k) o[k] += rf[k];
            }
            astore<8, kCachePolicyNT>(rdx, (b * T + lane) * 16, pack16<E>(o));
        }
        base = nbase;
    }

    const int64_t padded = dyn_padded_hidden(h);
    float* slab = a.workspace + (int64_t)blockIdx.x * (LN ? 2 : 1) * padded;
#pragma unroll
    for (int b = 0; b < V; ++b) {
        const int col = (b * T + lane) * EP;
        if (col < h) {
#pragma unroll
            for (int k = 0; k < EP; ++k) {
                slab[col + k] = pw[b][k];
                if constexpr (LN) slab[padded + col + k] = pb[b][k];
            }
        }
    }
}

template <int V, bool LN, typename E = uint16_t>
hipError_t launch_bwd_wide(const DynBwdArgs& a, hipStream_t stream) {
    const int outs = LN ? 2 : 1;
    if (a.rows > 0) {
        if constexpr (LN) {
            hipLaunchKernelGGL((norm_bwd_wide_kernel<E, V, true, false>), dim3(a.grid),
                               dim3(kWideLanes), 0, stream, a);
        } else {
            if (a.dres)
                hipLaunchKernelGGL((norm_bwd_wide_kernel<E, V, false, true>), dim3(a.grid),
                                   dim3(kWideLanes), 0, stream, a);
            else
                hipLaunchKernelGGL((norm_bwd_wide_kernel<E, V, false, false>), dim3(a.grid),
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
