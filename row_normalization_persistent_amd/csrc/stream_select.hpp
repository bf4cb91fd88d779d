// Which streamed-row forward kernel takes a row (host side, shared by the
// launcher and the launch description).
#pragma once

#include <cstdint>

#include "launch.hpp"

namespace rownorm {

// Rows that the LDS-staged forward (stage_fwd_kernel) holds: U register and
// L LDS accesses a lane of 1024 (16 KiB of LDS a slot and staged matrix, x
// and for the fused op r; the weights of all U + L accesses sit in registers
// during the second pass, which bounds U + L: bf16 RMSNorm spills at 6 + 9).
// LayerNorm has none: staged (2 + 9 accesses) it ran 5-20 % slower than the
// streamed kernel's second read from the Infinity Cache.
struct StageShape {
    int u, l;
};
constexpr StageShape stage_fwd_shape(int op, bool f32) {
    if (op == kSplitFused) return {6, 4};
    if (op == kSplitRms) return {f32 ? 8 : 5, 9};
    return {0, 0};
}

// Workgroups of the staged kernel: one a compute unit of the largest part (its
// LDS holds one row), each walking rows blockIdx.x, + 256, ...
constexpr int64_t kStageGridRows = 256;

#ifndef ROWNORM_STAGE_FWD
#define ROWNORM_STAGE_FWD 1
#endif

// The staged kernel takes the rows of which the streamed kernel would read
// at least 1/16 twice (the accesses past those its lanes keep in registers)
// and that registers and LDS hold whole.  Measured on MI355X (graph-timed,
// cold buffers, alternating processes): bf16 fused 2048 x 73736 252.5 ->
// 249.5 us, 2048 x 81920 255.2 -> 252.5; bf16 RMSNorm 4096 x 73728 227.3 ->
// 217.4, 2048 x 98312 165.6 -> 159.1, 2048 x 114688 179.9 -> 170.9; fp32
// fused 4096 x 40960 493.2 -> 475.3, fp32 RMSNorm 2048 x 65536 202.4 -> 191.4;
// level where the second read is short (bf16 RMSNorm 4096 x 69632, 11 of
// 12 accesses a lane in registers), 6 % slower where it is one access in 9
// (4096 x 65544).  op: kSplitFused / kSplitRms / kSplitLn.
constexpr bool stage_fwd_holds(int op, bool f32, int64_t hidden) {
    const StreamFwdShape sh = stream_fwd_shape(f32, op == kSplitLn, op == kSplitRms, hidden);
    const StageShape st = stage_fwd_shape(op, f32);
    const int64_t n_acc = hidden / (f32 ? 4 : 8);
    const int64_t twice = n_acc - (int64_t)sh.lanes * sh.unroll;
    return ROWNORM_STAGE_FWD && st.l > 0 && 16 * twice >= n_acc &&
           n_acc <= (int64_t)kStreamFwdLanes * (st.u + st.l);
}

// ---- streamed backward: the tiles of a row exchange their partial sums --------------
// Exchange area after the walkers' slabs: per walker kXchRing walk steps of
// `tiles` slots of two 64-bit words (16 bytes a slot), zero-filled by a
// kernel before each launch.
// bf16 walks keep two rings of D rows and publish one group ahead: a slot
// is written again only after every tile has read the three groups before
// it, so the ring covers 4D walk steps (D = 3: 12).
#ifndef ROWNORM_XCH_RING
#define ROWNORM_XCH_RING 12
#endif
constexpr int kXchRing = ROWNORM_XCH_RING;
#ifndef ROWNORM_XCH_AHEAD
#define ROWNORM_XCH_AHEAD 1
#endif
constexpr bool kXchAhead = ROWNORM_XCH_AHEAD != 0;
// fp32 LayerNorm / RMSNorm walks with two rings of 2 rows, one group published
// ahead (the fused op's dres rows would spill): against one ring of 3,
// 512 x 131072 LayerNorm 198.6 -> 162.6 us, 2048 x 65536 RMSNorm 312.5 -> 284,
// 1024 x 49152 RMSNorm 123.5 -> 117.3; level at 32768 / 20480 columns;
// 8192 x 16388 RMSNorm 322.5 -> 330.3 (2.4 % slower)
#ifndef ROWNORM_XCH_AHEAD_F32
#define ROWNORM_XCH_AHEAD_F32 1
#endif
constexpr bool kXchAheadF32 = ROWNORM_XCH_AHEAD_F32 != 0;
// the fp32 fused op, whose dres rows leave room for two rings of one row:
// against one ring of 2, 512 x 131072 207.5 -> 175.5 us, 2048 x 65536 333 ->
// 315, 1024 x 49152 127.4 -> 122.2, level at 20480, 8192 x 16388 2 % slower
#ifndef ROWNORM_XCH_AHEAD_F32_DRES
#define ROWNORM_XCH_AHEAD_F32_DRES 1
#endif
constexpr bool kXchAheadF32Dres = ROWNORM_XCH_AHEAD_F32_DRES != 0;
// LayerNorm's per-row mean and rstd by vector loads in the exchanging kernel:
// scalar loads share their counter with LDS, so each group's reductions
// waited for the statistics of the rows just reloaded.  Against scalar
// loads: bf16 4096 x 65536 350 -> 322 us, 2048 x 98304 267 -> 247,
// 1024 x 131072 200 -> 187, 8192 x 40000 397 -> 375; fp32 1-2 %.
#ifndef ROWNORM_XCH_VEC_STATS
#define ROWNORM_XCH_VEC_STATS 1
#endif
constexpr bool kXchVecStats = ROWNORM_XCH_VEC_STATS != 0;
// the same for the fp32 one-tile kernel, which reduces each row in LDS:
// 8192 x 1024 33.5 -> 30.3 us, 8192 x 4096 75.8 -> 73.8, level at 4096 x 8192
// and 16384 x 4096, 16384 x 2048 80.7 -> 82 (2 % slower)
#ifndef ROWNORM_INROW_VEC_STATS
#define ROWNORM_INROW_VEC_STATS 1
#endif
constexpr bool kInrowVecStats = ROWNORM_INROW_VEC_STATS != 0;
// bf16 tiles of the exchanging kernel: 256 lanes x 2 accesses (4096 columns;
// at 4 accesses the exchange's registers push the kernel into spills).  Two
// such workgroups fit a CU (at most 256 VGPRs a lane, the kernel's launch
// bound), so one's barriers and waits overlap the other's loads: against one
// 512-lane workgroup a CU, 4096 x 65536 fused 357 -> 322 us, RMSNorm
// 324 -> 302, LayerNorm 360 -> 349, 8192 x 40000 416 -> 396.
constexpr int kXchVecsBf16 = 2;
#ifndef ROWNORM_XCH_LANES
#define ROWNORM_XCH_LANES 256
#endif
constexpr int kXchLanesBf16 = ROWNORM_XCH_LANES;
constexpr int kXchTileColsBf16 = kXchLanesBf16 * kXchVecsBf16 * 8;
// fp32 exchange tiles (rows past one 8192-column tile): 256 lanes x 4
// accesses (4096 columns), two workgroups a CU as for bf16: against 512
// lanes, 4096 x 20480 LayerNorm 207.7 -> 188.5 us, 8192 x 16388 RMSNorm
// 355 -> 322, 2048 x 65536 fused 345 -> 330, 2048 x 32768 LayerNorm 163 ->
// 158.5; 1.5-5 % slower at 131072 / 262144 columns (512 / 128 rows).
#ifndef ROWNORM_XCH_LANES_F32
#define ROWNORM_XCH_LANES_F32 256
#endif
constexpr int kXchLanesF32 = ROWNORM_XCH_LANES_F32;
constexpr int kXchTileColsF32 = kXchLanesF32 * 4 * 4;
// workgroups of a bf16 streamed backward with the exchange: two a CU, all
// co-resident on 256 CUs
#ifndef ROWNORM_XCH_WG_CAP
#define ROWNORM_XCH_WG_CAP 511
#endif
constexpr int kXchWgCap = ROWNORM_XCH_WG_CAP;
static_assert(kXchWgCap <= 255 || kXchLanesBf16 <= kStreamTileLanes / 2,
              "more than one exchange workgroup a CU needs tiles of at most half the lanes");
#ifndef ROWNORM_XCH_DEPTH
#define ROWNORM_XCH_DEPTH 3
#endif
constexpr int kXchDepthBf16 = ROWNORM_XCH_DEPTH;  // ring rows
// The tiles exchange partial row sums up to kXchMaxTiles bf16 tiles a row
// (262144 columns; fp32 tiles are 8192 columns, so fp32 rows stop at 64
// tiles' worth too): every tile polls every other tile's slots, so the
// exchange's traffic grows with the square of the tiles, and past 262144
// columns the two-kernel path (row sums, then tiles reading the row again)
// was faster (256 x 2^19 / 2^20: 262 / 530 us against 312 / 1058 us).
#ifndef ROWNORM_XCH_MAX_TILES
#define ROWNORM_XCH_MAX_TILES 64
#endif
constexpr int kXchMaxTiles = ROWNORM_XCH_MAX_TILES;
inline int64_t xch_bytes(int64_t walkers, int64_t tiles) {
    return tiles > 1 ? walkers * kXchRing * tiles * 16 : 0;
}
#ifndef ROWNORM_STREAM_BWD_XCH
#define ROWNORM_STREAM_BWD_XCH 1
#endif
inline bool stream_bwd_xch(int64_t hidden) {
    return ROWNORM_STREAM_BWD_XCH &&
           (hidden + kXchTileColsBf16 - 1) / kXchTileColsBf16 <= kXchMaxTiles;
}
// Polls a tile's wait for its partners makes before it re-reads the row
// itself (norm_bwd_set_spin_limit): by default about 16 ms, which a tile
// whose partners run beside it never needs.
constexpr uint32_t kBwdSpinLimit = 1u << 14;
uint32_t stream_bwd_spin_limit();

}  // namespace rownorm
