// Host-side launch tables shared by the kernel translation units and the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>
#include <vector>

namespace rownorm {

// Hidden sizes every operation is compiled for (the hidden size of a given
// model is fixed, so it is a template constant: "optimize inner persistent
// scheduler for static fusion", author description).
constexpr int kHiddenSizes[] = {1024, 2048, 4096, 8192, 12288, 16384};

struct FwdArgs {
    void* out;             // fused/rms: out; layernorm: y
    void* residual;        // fused only (in/out)
    const void* x;
    const void* weight;
    const void* bias;      // layernorm only
    float* mean;           // layernorm only (may be null together with rstd)
    float* rstd;
    int64_t rows;
    float eps;
    int32_t grid;          // ring kernels: persistent workgroups; 0 otherwise
};

struct BwdArgs {
    void* dx;              // RMSNorm-fused: the gradient of x and of the residual input
    const void* dy;        // RMSNorm-fused: the gradient of out
    const void* x;         // RMSNorm-fused: s, the residual output of the forward
    const float* mean;     // LayerNorm only
    const float* rstd;     // LayerNorm only
    const void* dres;      // RMSNorm-fused only: gradient of the residual output, or null
    const void* weight;
    float* workspace;      // [grid][outs][hidden] fp32 partial column sums
    float* dweight;
    float* dbias;          // LayerNorm only
    int64_t rows;
    int32_t grid;
    float eps;             // RMSNorm only (the statistic is recomputed)
};

using FwdLauncher = hipError_t (*)(const FwdArgs&, hipStream_t);
using BwdLauncher = hipError_t (*)(const BwdArgs&, hipStream_t);

struct FwdEntry {
    int hidden, lanes, rows_per_block;
    FwdLauncher launch;
    int depth;  // 0: one row per lane group; > 0: persistent ring of that many rows
    FwdLauncher launch_late;  // the late-weights variant (one row per lane group only)
};

// Default persistent grid of the forward ring kernels (one workgroup per CU of
// the largest part).
constexpr int kFwdRingGrid = 256;

struct BwdEntry {
    int hidden, lanes, depth;  // depth: rows kept in flight per workgroup
    BwdLauncher launch;
};

// Compiled shapes, one table per operation (defined in the kernel units).
const std::vector<FwdEntry>& fused_add_rmsnorm_table();
const std::vector<FwdEntry>& rmsnorm_fwd_table();
const std::vector<FwdEntry>& layernorm_fwd_table();
const std::vector<BwdEntry>& layernorm_bwd_table();
const std::vector<BwdEntry>& rmsnorm_bwd_table();

// ---- run-time-hidden path -------------------------------------------------------
// Leading dimensions (row strides) are in elements; every pointer is aligned
// to the access width (2*elems bytes) and hidden % elems == 0.
struct DynFwdArgs {
    void* out;             // fused/rms: out; layernorm: y
    void* residual;        // fused only (in/out)
    const void* x;
    const void* weight;
    const void* bias;      // layernorm only
    float* mean;           // layernorm only (may be null together with rstd)
    float* rstd;
    int64_t ld_out, ld_res, ld_x;
    int64_t rows;
    int32_t hidden;
    float eps;
};

struct DynBwdArgs {
    void* dx;
    const void* dy;
    const void* x;
    const float* mean;     // LayerNorm only
    const float* rstd;     // LayerNorm only
    const void* dres;      // RMSNorm-fused only, or null
    const void* weight;
    float* workspace;      // [grid * walkers per workgroup][outs][padded hidden] fp32
    float* dweight;
    float* dbias;          // LayerNorm only
    int64_t ld_dx, ld_dy, ld_x, ld_dres;
    int64_t rows;
    int32_t hidden;
    int32_t grid;
    float eps;             // RMSNorm only
};

using DynFwdLauncher = hipError_t (*)(const DynFwdArgs&, hipStream_t);
using DynBwdLauncher = hipError_t (*)(const DynBwdArgs&, hipStream_t);

struct DynFwdEntry {
    int elems, lanes, vecs;  // access width W, lanes per row T, accesses per lane V
    DynFwdLauncher launch;
    int rows_per_group;        // K rows per lane group (workgroup rows = R * K)
    DynFwdLauncher launch_late;  // the late-weights variant
};

struct DynBwdEntry {
    int elems, lanes, vecs, depth;
    DynBwdLauncher launch;
};

const std::vector<DynFwdEntry>& fused_add_rmsnorm_dyn_table();
const std::vector<DynFwdEntry>& rmsnorm_fwd_dyn_table();
const std::vector<DynFwdEntry>& layernorm_fwd_dyn_table();
const std::vector<DynBwdEntry>& layernorm_bwd_dyn_table();
const std::vector<DynBwdEntry>& rmsnorm_bwd_dyn_table();

// ---- backward for rows wider than the registers hold (x staged in LDS) ---------
// 512 lanes, 16-byte accesses, V accesses a lane: hidden <= 4096 V.
constexpr int kWideBwdLanes = 512;
struct WideBwdEntry {
    int vecs;
    DynBwdLauncher launch;
};
using WideVecsLn = std::integer_sequence<int, 5, 6, 7, 8>;
using WideVecsRms = std::integer_sequence<int, 5, 6, 7, 8>;
const std::vector<WideBwdEntry>& layernorm_bwd_wide_table();
const std::vector<WideBwdEntry>& rmsnorm_bwd_wide_table();
// fp32 rows of kWideF32MinHidden ... kWideF32MaxHidden columns (4 values an
// access, V = ceil(hidden / 2048) = 5 ... 8): the same kernel, read once
// instead of the streamed pair's twice.  Grid a.grid, workspace a.grid slabs.
constexpr int64_t kWideF32MinHidden = 8196;
constexpr int64_t kWideF32MaxHidden = 16384;
constexpr int wide_vecs_f32(int64_t hidden) { return (int)((hidden + 2047) / 2048); }
hipError_t launch_bwd_wide_f32(bool ln, const DynBwdArgs& a, hipStream_t stream);

// ---- row-split forward (few rows: one row over k workgroups) ------------------
// Workspace: kSplitHeaderWords 32-bit words (word 0: error bits), then per
// row kSplitRowQwords 64-bit words: [kSplitDepart] the count of workgroups
// done with the row, [kSplitP0 + j] and [kSplitP1 + j] chunk j's two partial
// sums (fp32 bits in the high half, 1 in the low half once written).  Zero
// at rest.
constexpr int kSplitLanes = 256;        // lanes per workgroup
constexpr int kSplitMax = 64;           // workgroups per row at most (one wave polls them)
constexpr int kSplitMaxVecs = 8;        // 16-byte accesses per lane at most
constexpr int kSplitHeaderWords = 64;
constexpr int kSplitDepart = 0;
constexpr int kSplitP0 = 1;
constexpr int kSplitP1 = kSplitP0 + kSplitMax;
constexpr int kSplitRowQwords = 144;    // >= kSplitP1 + kSplitMax, 128-byte multiple
constexpr uint32_t kSplitSpinLimit = 1u << 20;  // default polls per wait (about a second)
enum SplitOp : int { kSplitFused = 0, kSplitRms = 1, kSplitLn = 2 };

struct SplitArgs {
    void* out;             // fused/rms: out; layernorm: y
    void* residual;        // fused only (in/out)
    const void* x;
    const void* weight;
    const void* bias;      // layernorm only
    float* mean;           // layernorm only (may be null together with rstd)
    float* rstd;
    uint32_t* ws;
    int64_t ld_out, ld_res, ld_x;
    int64_t rows;
    int32_t hidden;
    int32_t split;         // k workgroups per row
    float eps;
    uint32_t spin_limit;   // polls a partner wait makes before giving up
};

using SplitLauncher = hipError_t (*)(const SplitArgs&, hipStream_t);

struct SplitEntry {
    int op;    // kSplitFused / kSplitRms / kSplitLn
    int vecs;  // V 16-byte accesses per lane: a chunk is kSplitLanes * V * 8 columns
    SplitLauncher launch;
};

const std::vector<SplitEntry>& split_table();

// ---- streamed rows (wider than registers and LDS hold; kernels_stream.hpp) ------
// Forward: 1024-lane workgroups walk the rows, each row read twice.  Backward:
// a 1024-lane per-row reduction kernel, then 512-lane workgroups over tiles of
// kStreamTileVecs * 512 16-byte accesses (16384 bf16 or 8192 fp32 columns).
// 16-byte accesses only.  The same kernels run fp32 activations (the `_f32`
// entry points; their backward rows of 8196 ... 16384 columns go to the
// LDS-staged kernel instead); the DynFwdArgs / DynBwdArgs pointers then
// point at fp32 matrices and vectors, row strides in fp32 elements.
constexpr int kStreamFwdLanes = 1024;
constexpr int kStreamTileLanes = 512;
constexpr int kStreamTileVecs = 4;
constexpr int kStreamTileCols = kStreamTileLanes * kStreamTileVecs * 8;  // bf16 columns: 16384
constexpr int kStreamTileColsF32 = kStreamTileLanes * kStreamTileVecs * 4;  // fp32: 8192
constexpr int64_t kStreamMaxGrid = 65536;  // workgroups of the row-walking kernels
constexpr int64_t kStreamMaxHidden = int64_t(1) << 20;

// Streamed forward launch shape: lanes a row and 16-byte accesses a lane
// kept in registers from the statistic pass to the normalize pass (a row of
// up to lanes x unroll accesses is read once, the rest twice).  Measured on
// MI355X (graph-timed over cold buffers):
//  * fp32 fused and RMSNorm: 64 .. 1024 lanes x 4 accesses up to 16384
//    columns, 1024 x 8 beyond (2048 x 32768: fused 202 -> 190 us, RMSNorm
//    97 -> 93 us; 1024 x 65536 4-5 % faster; 256 x 262144 even);
//  * fp32 LayerNorm, whose two reductions cost a barrier each: half the lanes
//    with 8 accesses from 1025 to 16384 columns (2048 x 16384 57.3 -> 51.6 us,
//    2048 x 4096 16.3 -> 14.9 us; 4096 x 8192, 8192 x 4096, 16384 x 2048
//    0.5-1.5 % faster, 8192 x 1536 1 % slower), 1024 x 4 beyond (8 accesses
//    were 0-4 % slower there);
//  * bf16 (rows past the on-chip kernels): 1024 x 4; RMSNorm 1024 x 8 up to
//    73728 columns, where 8 accesses hold nearly the whole row (4096 x 65544
//    214 -> 202 us; at 131072 and 262144 columns 1-6 % slower); the fused op
//    1024 x 6 up to 98304 columns (4096 x 65544 454 -> 440 us, 2048 x 81920
//    263 -> 256 us, level at 98304); LayerNorm keeps 4 (6 was 4-12 % slower
//    at 53248-65536 columns); the fused and LayerNorm forms spill at 8.
#ifndef ROWNORM_STREAM_U8
#define ROWNORM_STREAM_U8 1  // build-time switch for measurement: 0 = never 8 accesses past 16384 fp32 columns
#endif
struct StreamFwdShape {
    int lanes, unroll;
};
#ifndef ROWNORM_STREAM_U6
#define ROWNORM_STREAM_U6 1
#endif
constexpr StreamFwdShape stream_fwd_shape(bool f32, bool ln, bool rms, int64_t hidden) {
    if (!f32) {
        if (rms) return {kStreamFwdLanes, ROWNORM_STREAM_U8 && hidden <= 73728 ? 8 : 4};
        if (!ln) return {kStreamFwdLanes, ROWNORM_STREAM_U6 && hidden <= 98304 ? 6 : 4};
        return {kStreamFwdLanes, 4};
    }
    if (hidden <= 1024) return {64, 4};
    if (ln) {
        if (hidden <= 2048) return {64, 8};
        if (hidden <= 4096) return {128, 8};
        if (hidden <= 8192) return {256, 8};
        if (hidden <= 16384) return {512, 8};
        return {kStreamFwdLanes, 4};
    }
    if (hidden <= 2048) return {128, 4};
    if (hidden <= 4096) return {256, 4};
    if (hidden <= 8192) return {512, 4};
    if (hidden <= 16384) return {kStreamFwdLanes, 4};
    return {kStreamFwdLanes, ROWNORM_STREAM_U8 ? 8 : 4};
}
// fp32 backward with one tile (hidden <= kStreamTileColsF32): accesses a lane
// of the 512-lane tile that hold the row (1, 2 or 4).
constexpr int stream_inrow_vecs_f32(int64_t hidden) {
    return hidden <= 2048 ? 1 : hidden <= 4096 ? 2 : 4;
}

// op: kSplitFused / kSplitRms / kSplitLn (the row-split numbering)
hipError_t launch_stream_fwd(int op, bool f32, const DynFwdArgs& a, hipStream_t stream);
// Stats kernel, tile kernel and column reduce.  ln: LayerNorm, else RMSNorm
// (with a.dres: the fused op).  The workspace holds `walkers` slabs of
// [outs][padded] fp32, then two fp32 per row.  fp32 rows of one tile skip the
// stats kernel (the tile kernel reduces each row itself; the per-row floats
// stay unused).
hipError_t launch_stream_bwd(bool ln, bool f32, const DynBwdArgs& a, int32_t tiles,
                             int32_t walkers, hipStream_t stream);

// Workgroup size of the run-time path for T lanes per row: rows narrower than
// 256 lanes are packed 256 / T to a workgroup.
constexpr int dyn_block_size(int lanes) { return lanes < 256 ? 256 : lanes; }
constexpr int dyn_rows_per_block(int lanes) { return dyn_block_size(lanes) / lanes; }
// Partial-sum slabs pad each output's hidden columns to a multiple of the
// column reduce's 64-column tile.
constexpr int64_t dyn_padded_hidden(int64_t hidden) { return (hidden + 63) / 64 * 64; }

// Column reduce shared by both paths: out[o][j] = sum over slabs s of
// ws[s][o][j] for j < hidden, o < outs (dweight, then dbias); slabs hold
// `padded` floats per output.  Defined with the backward kernels.
hipError_t launch_norm_colreduce(const float* workspace, int32_t slabs, int32_t hidden,
                                 int32_t padded, int32_t outs, float* dweight, float* dbias,
                                 hipStream_t stream);

// Column-reduce geometry of the backward ops: 256 lanes a workgroup, 64
// columns a workgroup for up to 256 partial-sum slabs (one pass), 16 for up
// to 1024 and 4 beyond (more workgroups instead of more passes).
constexpr int kColReduceThreads = 256;
constexpr int kColReduceCols = 64;
// Columns per column-reduce workgroup: 64 (16 slab streams, one pass of 256
// slabs) up to 256 slabs, else 16 (64 streams, passes of 1024 slabs).
// Narrower workgroups read 16 bytes of each 128-byte line of a slab row, so
// the line is fetched once per workgroup; measured slower at every slab count.
#ifndef ROWNORM_COLREDUCE_COLS
#define ROWNORM_COLREDUCE_COLS 0  // build-time override of the choice below (64 or 16)
#endif
static_assert(ROWNORM_COLREDUCE_COLS == 0 || ROWNORM_COLREDUCE_COLS == 16 ||
                  ROWNORM_COLREDUCE_COLS == 64,
              "the column reduce is compiled for 64 and 16 columns per workgroup");
constexpr int colreduce_cols(int64_t slabs) {
    if constexpr (ROWNORM_COLREDUCE_COLS > 0) return ROWNORM_COLREDUCE_COLS;
    return slabs <= 256 ? 64 : 16;
}
// Largest persistent grid for a hidden size: the workspace ([grid][2][hidden]
// fp32) must stay addressable by one 32-bit buffer descriptor, with room for
// the column reduce's clamped, range-checked reads one slab past the last.
constexpr int64_t max_bwd_grid(int64_t hidden) {
    return ((int64_t(1) << 31) - 1) / (8 * hidden) - 128;
}

}  // namespace rownorm
