// C ABI of the row-normalization library: argument validation, the choice
// between the compiled-hidden kernels and the run-time-hidden kernels, the
// launch-shape choice, and dispatch.  Declared in norm.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <type_traits>

#include "launch.hpp"
#include "norm.h"
#include "stream_select.hpp"

using namespace rownorm;

namespace rownorm {
// Polls a streamed-backward tile makes while it waits for its row's other
// tiles; process-wide, changed only by norm_bwd_set_spin_limit.
std::atomic<uint32_t> g_bwd_spin_limit{kBwdSpinLimit};
uint32_t stream_bwd_spin_limit() { return g_bwd_spin_limit.load(std::memory_order_relaxed); }
}  // namespace rownorm

// Partial-sum slabs of norm_layernorm_bwd_noalloc (see current_scratch).
static __device__ __align__(256) unsigned char scratch[NORM_NOALLOC_SCRATCH_BYTES];

namespace {

bool hidden_compiled(int64_t hidden) {
    for (int h : kHiddenSizes)
        if (h == hidden) return true;
    return false;
}

uintptr_t addr(const void* p) { return reinterpret_cast<uintptr_t>(p); }
bool aligned(const void* p, uintptr_t a) { return addr(p) % a == 0; }

bool eps_ok(float eps) { return std::isfinite(eps) && eps >= 0.0f; }

// Sanity bounds; each launch also checks that its grid and total work-item
// count fit HIP's 32-bit launch limits.
constexpr int64_t kMaxRows = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxLd = int64_t(1) << 40;  // elements
// Largest hidden any kernel family can hold in registers (the run-time path,
// 16-byte accesses, 1024 lanes x 8 accesses); the exact limit depends on the
// operation and the access width (see the tables).
constexpr int64_t kMaxHidden = kStreamMaxHidden;  // 2^20: the streamed kernels' limit

bool valid_elems(int32_t w) { return w == 0 || w == 1 || w == 2 || w == 4 || w == 8; }

// A strided matrix may span at most 2^47 bytes, far past any device
// allocation: with it, (rows - 1) * ld + cols and every row offset a kernel
// forms stay inside int64.  `ld` >= 1.
constexpr int64_t kMaxSpanBytes = int64_t(1) << 47;
bool span_ok(int64_t rows, int64_t ld, int64_t cols, int elem) {
    if (rows <= 0) return true;
    const int64_t lim = kMaxSpanBytes / elem;  // elements
    return cols <= lim && rows - 1 <= (lim - cols) / ld;
}

// ---- memory regions and overlap ---------------------------------------------------
// A [rows, cols] matrix of `elem`-byte values whose rows start `ld` elements
// apart (a vector is one row).
struct Region {
    const void* p;
    int64_t rows, ld, cols;
    int elem;
    uint64_t bytes() const {
        if (!p || rows <= 0 || cols <= 0) return 0;
        return (uint64_t)((rows - 1) * ld + cols) * (uint64_t)elem;
    }
};

Region vec_region(const void* p, int64_t n, int elem) { return Region{p, 1, n, n, elem}; }

// True if two regions share a byte.  An exact alias (same base, stride and
// width) is allowed when `exact_ok`; two matrices with the same row stride
// whose rows interleave without touching (column windows disjoint modulo the
// stride, e.g. two slices of one wider matrix) never conflict.
bool conflict(const Region& a, const Region& b, bool exact_ok) {
    const uint64_t na = a.bytes(), nb = b.bytes();
    if (na == 0 || nb == 0) return false;
    const uintptr_t a0 = addr(a.p), b0 = addr(b.p);
    if (a0 + na <= b0 || b0 + nb <= a0) return false;
    if (exact_ok && a0 == b0 && a.ld == b.ld && a.cols == b.cols && a.elem == b.elem)
        return false;
    if (a.elem == b.elem && a.ld == b.ld && a.ld > 0) {
        const int64_t d = (int64_t)(b0 - a0);  // two's complement difference
        if (d % a.elem == 0) {
            const int64_t m = ((d / a.elem) % a.ld + a.ld) % a.ld;
            if (m >= a.cols && m + b.cols <= a.ld) return false;
        }
    }
    return true;
}

// ---- compute-unit count, cached per device ---------------------------------
constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

norm_status current_cu_count(int* cu) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return NORM_ERROR_DEVICE;
    if (dev < kMaxDevices) {
        const int c = g_cu_count[dev].load(std::memory_order_relaxed);
        if (c > 0) {
            *cu = c;
            return NORM_SUCCESS;
        }
    }
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        c <= 0)
        return NORM_ERROR_DEVICE;
    if (dev < kMaxDevices) g_cu_count[dev].store(c, std::memory_order_relaxed);
    *cu = c;
    return NORM_SUCCESS;
}

// ---- scratch of the allocation-free backward entry -------------------------
// norm_layernorm_bwd_noalloc keeps its partial-sum slabs here instead of in a
// caller-given workspace.  Each device that runs it holds its own copy of this
// array for the life of the process; host code never uses the array's name
// (a host-side stand-in, not a device address) but the address that
// hipGetSymbolAddress returns for the current device, looked up once per
// device and kept in g_scratch.
constexpr size_t kScratchBytes = NORM_NOALLOC_SCRATCH_BYTES;
std::atomic<void*> g_scratch[kMaxDevices];

norm_status current_scratch(void** ptr) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return NORM_ERROR_DEVICE;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return NORM_ERROR_DEVICE;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return NORM_SUCCESS;
}

// ---- tables ----------------------------------------------------------------
bool is_bwd(norm_op op) {
    return op == NORM_OP_LAYERNORM_BWD || op == NORM_OP_RMSNORM_BWD ||
           op == NORM_OP_FUSED_ADD_RMSNORM_BWD;
}

const std::vector<FwdEntry>& fwd_table(norm_op op) {
    switch (op) {
        case NORM_OP_FUSED_ADD_RMSNORM: return fused_add_rmsnorm_table();
        case NORM_OP_RMSNORM_FWD: return rmsnorm_fwd_table();
        default: return layernorm_fwd_table();
    }
}

const std::vector<DynFwdEntry>& dyn_fwd_table(norm_op op) {
    switch (op) {
        case NORM_OP_FUSED_ADD_RMSNORM: return fused_add_rmsnorm_dyn_table();
        case NORM_OP_RMSNORM_FWD: return rmsnorm_fwd_dyn_table();
        default: return layernorm_fwd_dyn_table();
    }
}

const std::vector<BwdEntry>& bwd_table(norm_op op) {
    return op == NORM_OP_LAYERNORM_BWD ? layernorm_bwd_table() : rmsnorm_bwd_table();
}

const std::vector<DynBwdEntry>& dyn_bwd_table(norm_op op) {
    return op == NORM_OP_LAYERNORM_BWD ? layernorm_bwd_dyn_table() : rmsnorm_bwd_dyn_table();
}

// The LDS-staged backward for rows wider than the register-resident run-time
// kernels hold: 512 lanes, 16-byte accesses, V = ceil(hidden / 4096).
const WideBwdEntry* find_wide(norm_op op, int64_t hidden, int lanes, int w);

// A compiled forward shape: one row per lane group (ring false) or the
// persistent ring kernel (ring true, LayerNorm only).
const FwdEntry* find_fwd(norm_op op, int64_t hidden, int lanes, int rpb, bool ring = false) {
    for (const FwdEntry& e : fwd_table(op))
        if (e.hidden == hidden && e.lanes == lanes && e.rows_per_block == rpb &&
            (e.depth > 0) == ring)
            return &e;
    return nullptr;
}

// The ring kernel (LayerNorm or RMSNorm) a call runs: the shallowest compiled
// depth that holds a workgroup's whole walk (ceil(rows / grid) rows), else the
// deepest compiled.  Measured on MI355X (2048 rows at hidden 8192 / 12288 /
// 16384, one workgroup per CU): loading the whole walk at once beats a
// shallower ring by 6-16 %; with walks longer than the deepest ring the depths
// are within 1-2 % of each other.
const FwdEntry* ring_entry(norm_op op, int64_t hidden, int lanes, int64_t rows, int64_t grid) {
    const int64_t walk = grid > 0 ? std::max<int64_t>(1, (rows + grid - 1) / grid) : 1;
    const FwdEntry *fit = nullptr, *deepest = nullptr;
    for (const FwdEntry& e : fwd_table(op)) {
        if (e.hidden != hidden || e.lanes != lanes || e.rows_per_block != 1 || e.depth == 0)
            continue;
        if (!deepest || e.depth > deepest->depth) deepest = &e;
        if (e.depth >= walk && (!fit || e.depth < fit->depth)) fit = &e;
    }
    return fit ? fit : deepest;
}

// Largest persistent grid of a forward ring kernel (a sanity bound; the ring
// kernels handle any grid from 1 up, idle workgroups included).
constexpr int32_t kMaxFwdRingGrid = 1 << 20;

const BwdEntry* find_bwd(norm_op op, int64_t hidden, int lanes) {
    for (const BwdEntry& e : bwd_table(op))
        if (e.hidden == hidden && e.lanes == lanes) return &e;
    return nullptr;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// The run-time-hidden instantiation with access width w and `lanes` lanes
// whose per-lane access count is the smallest compiled one covering the row.
// Forward entries also match K, the rows per lane group.
template <class Entry>
const Entry* find_dyn(const std::vector<Entry>& table, int64_t hidden, int w, int lanes,
                      int k = 1) {
    const int64_t need = ceil_div(hidden / w, lanes);
    const Entry* best = nullptr;
    for (const Entry& e : table) {
        if constexpr (std::is_same_v<Entry, DynFwdEntry>) {
            if (e.rows_per_group != k) continue;
        }
        if (e.elems == w && e.lanes == lanes && e.vecs >= need && (!best || e.vecs < best->vecs))
            best = &e;
    }
    return best;
}

// Widest row the run-time-hidden instantiations of a table hold at access width w.
template <class Entry>
int64_t max_dyn_hidden(const std::vector<Entry>& table, int w) {
    int64_t m = 0;
    for (const Entry& e : table)
        if (e.elems == w) m = std::max<int64_t>(m, (int64_t)e.lanes * e.vecs * w);
    return m;
}

// The fused op's LDS-staged backward stops at 7 accesses a lane: at 8 (rows of
// 28680 ... 32768 columns) the streamed tiles were faster, 4096 x 32768
// 199 -> 178 us, 8192 x 32768 398 -> 340 us (at 7, 4096 x 28672, 165 against
// 175 us streamed).
constexpr int kWideFusedMaxVecs = 7;
bool wide_serves(norm_op op, int vecs) {
    return op != NORM_OP_FUSED_ADD_RMSNORM_BWD || vecs <= kWideFusedMaxVecs;
}

const WideBwdEntry* find_wide(norm_op op, int64_t hidden, int lanes, int w) {
    if (lanes != kWideBwdLanes || w != 8 || hidden % 8 ||
        hidden <= max_dyn_hidden(dyn_bwd_table(op), 8))
        return nullptr;
    const int64_t v = ceil_div(hidden, (int64_t)8 * kWideBwdLanes);
    if (!wide_serves(op, (int)v)) return nullptr;
    const auto& t = op == NORM_OP_LAYERNORM_BWD ? layernorm_bwd_wide_table()
                                                : rmsnorm_bwd_wide_table();
    for (const WideBwdEntry& e : t)
        if (e.vecs == v) return &e;
    return nullptr;
}

// Widest backward row one workgroup holds on chip for accesses of w elements
// (the LDS-staged kernels take over above the run-time kernels' widest row at
// 16-byte accesses).
int64_t max_bwd_resident(norm_op op, int w) {
    int64_t m = max_dyn_hidden(dyn_bwd_table(op), w);
    if (w == 8) {
        const auto& t = op == NORM_OP_LAYERNORM_BWD ? layernorm_bwd_wide_table()
                                                    : rmsnorm_bwd_wide_table();
        for (const WideBwdEntry& e : t)
            if (wide_serves(op, e.vecs))
                m = std::max<int64_t>(m, (int64_t)e.vecs * 8 * kWideBwdLanes);
    }
    return m;
}

// Streamed rows (kernels_stream.hpp): wider than every on-chip kernel holds,
// 16-byte accesses, up to kStreamMaxHidden.
bool stream_fwd_ok(norm_op op, int64_t hidden, int w) {
    return w == 8 && hidden % 8 == 0 && hidden <= kStreamMaxHidden &&
           hidden > max_dyn_hidden(dyn_fwd_table(op), 8);
}

bool stream_bwd_ok(norm_op op, int64_t hidden, int w) {
    return w == 8 && hidden % 8 == 0 && hidden <= kStreamMaxHidden &&
           hidden > max_bwd_resident(op, 8);
}

// Widest backward row for accesses of w elements.
int64_t max_bwd_hidden(norm_op op, int w) {
    return w == 8 ? kStreamMaxHidden : max_bwd_resident(op, w);
}

// Column tiles of a streamed backward row, and its default row walkers: one
// 512-lane workgroup per (walker, tile), at most 255 in all (one per CU,
// leaving the partial sums of any width under 32 MiB).
int32_t stream_tiles(int64_t hidden) {
    return (int32_t)ceil_div(hidden, stream_bwd_xch(hidden) ? kXchTileColsBf16 : kStreamTileCols);
}
int32_t stream_walkers(int64_t rows, int64_t hidden) {
    const int cap = stream_bwd_xch(hidden) ? kXchWgCap : 255;
    return (int32_t)std::max<int64_t>(1, std::min<int64_t>(rows, cap / stream_tiles(hidden)));
}

// Exchanging tiles wait for each other, so the library's own walker count is
// kept to what the device holds at once (two workgroups a CU at half the
// tile lanes, else one): on a part with fewer CUs than the 256 the caps
// assume (a partition), its waits would otherwise run to their limit.  Never
// raises the count, so the workspace sized for the cap still holds.
int32_t resident_walkers_on(int32_t walkers, int32_t tiles, int lanes, int cu) {
    if (tiles < 2 || cu <= 0) return walkers;
    const int64_t slots = (int64_t)cu * (lanes <= kStreamTileLanes / 2 ? 2 : 1);
    return (int32_t)std::max<int64_t>(1, std::min<int64_t>(walkers, slots / tiles));
}
int32_t resident_walkers(int32_t walkers, int32_t tiles, int lanes) {
    int cu = 0;
    if (tiles < 2 || current_cu_count(&cu) != NORM_SUCCESS) return walkers;
    return resident_walkers_on(walkers, tiles, lanes, cu);
}

// partial-sum slabs per walker: dweight and dbias for LayerNorm, dweight for RMSNorm
int bwd_outs(norm_op op) { return op == NORM_OP_LAYERNORM_BWD ? 2 : 1; }

// ---- access width ---------------------------------------------------------------
// Widest access (elements: 8, 4, 2, 1) that divides hidden and every leading
// dimension, and that every bf16 pointer is aligned to.
int shape_width(int64_t hidden, std::initializer_list<int64_t> lds) {
    int w = 8;
    for (;;) {
        bool ok = hidden % w == 0;
        for (int64_t ld : lds) ok = ok && ld % w == 0;
        if (ok || w == 1) return w;
        w /= 2;
    }
}

int pointer_width(std::initializer_list<const void*> ptrs) {
    int w = 8;
    for (const void* p : ptrs)
        while (w > 1 && p && !aligned(p, 2 * (uintptr_t)w)) w /= 2;
    return w;
}

// ---- launch-shape choice ----------------------------------------------------
// Forward ops, chosen from steady-state measurements on MI355X (graph-replayed
// launches over cold buffers):
//  * Small batches: when rows alone cannot give every SIMD of every CU a wave,
//    each row is spread over more lanes (the small-batch rule of "optimize
//    inner persistent scheduler for static fusion", author description), so
//    the machine still issues enough parallel 16-byte loads; beyond 64 lanes
//    the row's waves meet in LDS.
//  * Large batches: a lane holds at most 8 16-byte vectors of the row (wider
//    per-lane buffers plus the weight/bias vectors cost occupancy), and from
//    4096 rows up the RMS kernels run best at 4 vectors per lane.
//  * Rows per workgroup: 4 for one-wave rows, 2 for two-wave rows, else 1.
// LayerNorm forward from 512 rows (320 at hidden 16384, 4096 at hidden 4096)
// runs on the persistent ring kernel (measured on MI355X, 2048 rows: 6-8 %
// faster at hidden 8192-16384 with a fixed ring depth, 12-16 % with the depth
// picked per walk; at 384 / 511 rows of hidden 16384 0.97 / 0.94 of the plain
// kernel's time, but 1.05-1.09 at hidden 8192 and 12288; with walks of one row
// the launch is latency-bound and the plain kernels win): lanes and grid per
// hidden size from the same sweeps (512 lanes beat 1024 at hidden 16384 and
// 256 at 12288 by 2-10 % at 512-8192 rows).
norm_launch_cfg choose_ln_ring(int64_t rows, int64_t hidden) {
    int lanes = 0, grid = 0;
    if (hidden == 16384 && rows >= 320) lanes = 512, grid = 256;
    if (hidden == 12288 && rows >= 512) lanes = 512, grid = 256;
    if (hidden == 8192 && rows >= 512) lanes = 512, grid = 256;
    if (hidden == 4096 && rows >= 4096) lanes = 64, grid = 1024;
    if (lanes == 0 || !find_fwd(NORM_OP_LAYERNORM_FWD, hidden, lanes, 1, true))
        return norm_launch_cfg{0, 0, 0, 0};
    return norm_launch_cfg{lanes, 1, (int32_t)std::min<int64_t>(grid, rows), 0};
}

// Launch shapes measured faster than the rules below on one MI355X (256 CUs):
// every compiled and run-time shape of each (op, compiled hidden) at 1, 16, 64,
// 256, 1024, 2048, 4096 and 8192 rows, back-to-back launches from a graph over
// cold buffer sets, kept where the best shape beat the rules' choice by >= 4 %
// and >= 0.1 us, then timed again against the rules' shape, interleaved (the
// figures below; kept where >= 3 % faster), and at row counts between the
// measured ones (entries that lost there were dropped or narrowed: shapes that
// win at 1024-4096 rows only by giving exactly one workgroup per CU lose 6-19 %
// at 600, 1200 or 3000 rows, since their gain comes from a whole number of
// workgroup waves).  An entry measured at R < 1024 rows covers the rows between
// the geometric midpoints of its neighbours, one measured at R >= 1024 the rows
// from the midpoint below up to R; counted on a 256-CU part (rows * 256 / CUs).
// A run-time shape (vector_elems 8) here runs the run-time kernel on rows the
// compiled kernels also hold.
#ifndef ROWNORM_NO_TUNED_TABLE
#define ROWNORM_NO_TUNED_TABLE 0  // build-time switch: 1 = the rules alone
#endif
struct TunedFwd {
    norm_op op;
    int32_t hidden;
    int64_t rows_lo, rows_hi;  // [lo, hi) rows on a 256-CU part
    norm_launch_cfg cfg;
};
constexpr TunedFwd kTunedFwd[] = {
    {NORM_OP_RMSNORM_FWD, 1024, 128, 512, {64, 1, 0, 0}},  // 256 rows: 2.50 -> 1.97 us (21 %)
    {NORM_OP_RMSNORM_FWD, 2048, 128, 512, {256, 1, 0, 8}},  // 256 rows: 2.62 -> 2.27 us (13 %)
    {NORM_OP_RMSNORM_FWD, 2048, 1449, 2049, {256, 1, 0, 8}},  // 2048 rows: 4.64 -> 3.88 us (16 %)
    {NORM_OP_RMSNORM_FWD, 4096, 32, 128, {256, 1, 0, 0}},  // 64 rows: 2.59 -> 2.24 us (14 %)
    {NORM_OP_RMSNORM_FWD, 8192, 32, 128, {256, 1, 0, 0}},  // 64 rows: 3.07 -> 2.54 us (17 %)
    {NORM_OP_RMSNORM_FWD, 12288, 32, 128, {256, 1, 0, 0}},  // 64 rows: 3.08 -> 2.79 us (9 %)
    {NORM_OP_RMSNORM_FWD, 16384, 16, 32, {256, 1, 0, 0}},  // 16 rows: 3.21 -> 3.05 us (5 %)
    {NORM_OP_RMSNORM_FWD, 16384, 32, 128, {256, 1, 0, 0}},  // 64 rows: 3.46 -> 3.28 us (5 %)
    {NORM_OP_LAYERNORM_FWD, 1024, 4, 32, {64, 4, 0, 0}},  // 16 rows: 2.52 -> 2.29 us (9 %)
    {NORM_OP_LAYERNORM_FWD, 1024, 32, 128, {64, 4, 0, 0}},  // 64 rows: 2.56 -> 2.32 us (9 %)
    {NORM_OP_LAYERNORM_FWD, 1024, 128, 512, {64, 1, 0, 0}},  // 256 rows: 2.97 -> 2.28 us (23 %)
    {NORM_OP_LAYERNORM_FWD, 1024, 2897, 4097, {64, 1, 0, 0}},  // 4096 rows: 4.97 -> 4.26 us (14 %)
    {NORM_OP_LAYERNORM_FWD, 2048, 128, 512, {64, 1, 0, 0}},  // 256 rows: 3.09 -> 2.58 us (17 %)
    {NORM_OP_LAYERNORM_FWD, 2048, 1449, 2049, {64, 1, 0, 0}},  // 2048 rows: 4.81 -> 4.25 us (12 %)
    {NORM_OP_LAYERNORM_FWD, 2048, 5793, 8193, {128, 1, 0, 0}},  // 8192 rows: 13.81 -> 13.38 us (3 %)
    {NORM_OP_LAYERNORM_FWD, 4096, 32, 128, {256, 1, 0, 0}},  // 64 rows: 3.09 -> 2.64 us (15 %)
    {NORM_OP_LAYERNORM_FWD, 8192, 1, 4, {512, 1, 0, 0}},  // 1 rows: 2.76 -> 2.64 us (4 %)
    {NORM_OP_LAYERNORM_FWD, 8192, 32, 128, {256, 1, 0, 0}},  // 64 rows: 3.88 -> 3.03 us (22 %)
    {NORM_OP_LAYERNORM_FWD, 12288, 32, 128, {256, 1, 0, 0}},  // 64 rows: 3.70 -> 3.44 us (7 %)
    {NORM_OP_LAYERNORM_FWD, 16384, 4, 32, {512, 1, 0, 0}},  // 16 rows: 4.13 -> 3.83 us (7 %)
    {NORM_OP_LAYERNORM_FWD, 16384, 32, 128, {512, 1, 0, 0}},  // 64 rows: 4.31 -> 4.06 us (6 %)
    {NORM_OP_FUSED_ADD_RMSNORM, 1024, 128, 512, {64, 1, 0, 0}},  // 256 rows: 2.58 -> 2.19 us (15 %)
    {NORM_OP_FUSED_ADD_RMSNORM, 2048, 32, 128, {256, 1, 0, 8}},  // 64 rows: 2.47 -> 2.25 us (9 %)
    {NORM_OP_FUSED_ADD_RMSNORM, 2048, 128, 512, {256, 1, 0, 8}},  // 256 rows: 2.88 -> 2.57 us (11 %)
    {NORM_OP_FUSED_ADD_RMSNORM, 2048, 512, 1025, {64, 4, 0, 8}},  // 1024 rows: 4.15 -> 3.84 us (7 %)
    {NORM_OP_FUSED_ADD_RMSNORM, 2048, 1449, 2049, {64, 1, 0, 0}},  // 2048 rows: 6.84 -> 6.38 us (7 %)
    {NORM_OP_FUSED_ADD_RMSNORM, 4096, 32, 128, {512, 1, 0, 8}},  // 64 rows: 2.71 -> 2.50 us (8 %)
    {NORM_OP_FUSED_ADD_RMSNORM, 8192, 16, 32, {256, 1, 0, 0}},  // 16 rows: 3.17 -> 2.93 us (8 %)
    {NORM_OP_FUSED_ADD_RMSNORM, 8192, 32, 128, {256, 1, 0, 0}},  // 64 rows: 3.38 -> 3.16 us (7 %)
    {NORM_OP_FUSED_ADD_RMSNORM, 8192, 512, 1025, {64, 1, 0, 0}},  // 1024 rows: 12.23 -> 11.25 us (8 %)
    {NORM_OP_FUSED_ADD_RMSNORM, 8192, 1449, 2049, {512, 2, 0, 0}},  // 2048 rows: 24.76 -> 23.38 us (6 %)
    {NORM_OP_FUSED_ADD_RMSNORM, 12288, 1, 4, {512, 1, 0, 8}},  // 1 rows: 3.20 -> 3.09 us (3 %)
};

norm_launch_cfg tuned_fwd(norm_op op, int64_t rows, int64_t hidden, int cu) {
    if (ROWNORM_NO_TUNED_TABLE || cu <= 0) return norm_launch_cfg{0, 0, 0, 0};
    const int64_t r = std::max<int64_t>(1, rows * 256 / cu);
    for (const TunedFwd& t : kTunedFwd)
        if (t.op == op && t.hidden == hidden && r >= t.rows_lo && r < t.rows_hi) return t.cfg;
    return norm_launch_cfg{0, 0, 0, 0};
}

// Weight-load variant of the one-row-per-lane-group forward kernels
// (kernels_fwd.hpp: `*_kernel` loads the weight, and bias, with the row;
// `*_lw_kernel` after the row's statistics).  The early variant is the
// default; the late one runs for the shapes and row ranges below, where it
// measured faster (graph-timed, cold buffers, A/B in one process).  Rows are
// counted on a 256-CU part as in the table above.  Build-time switch for
// measurement: 1 = early everywhere, 2 = late everywhere.
#ifndef ROWNORM_FWD_LATE_WEIGHTS
#define ROWNORM_FWD_LATE_WEIGHTS 0
#endif
struct LateFwd {
    norm_op op;
    int32_t hidden, lanes, rows_per_block;
    int64_t rows_lo, rows_hi;  // [lo, hi) rows on a 256-CU part
};
constexpr LateFwd kLateFwd[] = {
    {NORM_OP_LAYERNORM_FWD, 4096, 64, 4, 1449, 2897},       // 2048 rows: 8.22 -> 6.52 us (26 %)
    {NORM_OP_RMSNORM_FWD, 1024, 64, 4, 2897, 5793},         // 4096 rows: 3.93 -> 3.77 us (4 %)
    {NORM_OP_RMSNORM_FWD, 2048, 64, 4, 2897, 5793},         // 4096 rows: 7.35 -> 6.25 us (18 %)
    {NORM_OP_RMSNORM_FWD, 8192, 128, 2, 725, 2897},         // 1024 / 2048 rows: 4 % / 21 %
    {NORM_OP_FUSED_ADD_RMSNORM, 1024, 64, 4, 1449, 5793},   // 2048 / 4096 rows: 8 % / 9 %
    {NORM_OP_FUSED_ADD_RMSNORM, 4096, 64, 4, 1449, 2897},   // 2048 rows: 12.11 -> 11.74 us (3 %)
    {NORM_OP_FUSED_ADD_RMSNORM, 8192, 1024, 1, 1, 8},       // 1 / 4 rows: 5 % / 5 %
    {NORM_OP_FUSED_ADD_RMSNORM, 12288, 256, 1, 363, 725},   // 512 rows: 9.38 -> 8.97 us (5 %)
    {NORM_OP_FUSED_ADD_RMSNORM, 16384, 1024, 1, 1, 91},     // 1-64 rows: 4-7 %
    {NORM_OP_FUSED_ADD_RMSNORM, 16384, 256, 1, 363, 725},   // 512 rows: 12.45 -> 11.47 us (9 %)
};

bool late_listed(norm_op op, int64_t hidden, int lanes, int rpb) {
    if (ROWNORM_FWD_LATE_WEIGHTS != 0) return ROWNORM_FWD_LATE_WEIGHTS == 2;
    for (const LateFwd& t : kLateFwd)
        if (t.op == op && t.hidden == hidden && t.lanes == lanes && t.rows_per_block == rpb)
            return true;
    return false;
}

bool late_weights(norm_op op, int64_t rows, int64_t hidden, int lanes, int rpb, int cu) {
    if (ROWNORM_FWD_LATE_WEIGHTS != 0) return ROWNORM_FWD_LATE_WEIGHTS == 2;
    if (cu <= 0) return false;
    const int64_t r = std::max<int64_t>(1, rows * 256 / cu);
    for (const LateFwd& t : kLateFwd)
        if (t.op == op && t.hidden == hidden && t.lanes == lanes && t.rows_per_block == rpb &&
            r >= t.rows_lo && r < t.rows_hi)
            return true;
    return false;
}

// The run-time-hidden forward kernels (hidden is not a compile-time constant,
// so no per-hidden table): late weights when the grid is one wave of 2 to 4
// workgroups per CU that all start together, for rows of at least one wave.
// Measured (fused, RMSNorm and LayerNorm at hidden 2560 ... 7168, 16 ... 8192
// rows): late was 3-25 % faster at every such grid, e.g. RMSNorm 2048 x 6144
// 10.7 -> 8.6 us, LayerNorm 1024 x 7168 7.8 -> 6.3 us; with one workgroup per
// CU it lost up to 4 %, and from 8 per CU on it was level (+-2 %).
bool late_weights_dyn(int64_t groups, int lanes, int cu) {
    if (ROWNORM_FWD_LATE_WEIGHTS != 0) return ROWNORM_FWD_LATE_WEIGHTS == 2;
    return cu > 0 && lanes >= 64 && groups >= 2 * (int64_t)cu && groups <= 4 * (int64_t)cu;
}

// RMSNorm forward on the persistent ring kernel: 512 lanes, 256 workgroups,
// from 320 rows at hidden 12288 and 16384; at hidden 8192 for 320-511 rows
// and from 2048 rows.  Measured on MI355X against the one-row-per-lane-group
// choice (ring depth picked per walk): hidden 16384 at 384 / 512 / 1024 / 2048
// / 4096 / 8192 rows 0.85 / 0.82 / 0.90 / 0.88 / 0.94 / 0.99 of its time,
// hidden 12288 at 384 / 1024 / 2048 / 4096 rows 0.87 / 0.89 / 0.85 / 0.94,
// hidden 8192 at 384 / 511 / 2048 / 4096 / 8192 rows 0.95 / 0.90 / 0.97 / 0.95
// / 0.98 (at 1024 rows 1.04, where the late-weights kernel runs; at 256 rows
// and fewer, a walk of one row, 1.14-1.21).
norm_launch_cfg choose_rms_ring(int64_t rows, int64_t hidden) {
    const bool on = ((hidden == 16384 || hidden == 12288) && rows >= 320) ||
                    (hidden == 8192 && ((rows >= 320 && rows < 512) || rows >= 2048));
    if (!on || !find_fwd(NORM_OP_RMSNORM_FWD, hidden, 512, 1, true))
        return norm_launch_cfg{0, 0, 0, 0};
    return norm_launch_cfg{512, 1, (int32_t)std::min<int64_t>(256, rows), 0};
}

norm_launch_cfg choose_fwd(norm_op op, int64_t rows, int64_t hidden, int cu) {
    if (const norm_launch_cfg t = tuned_fwd(op, rows, hidden, cu); t.threads_per_row) return t;
    if (op == NORM_OP_LAYERNORM_FWD || op == NORM_OP_RMSNORM_FWD) {
        const norm_launch_cfg ring = op == NORM_OP_LAYERNORM_FWD ? choose_ln_ring(rows, hidden)
                                                                 : choose_rms_ring(rows, hidden);
        if (ring.threads_per_row) return ring;
    }
    const int64_t target_waves = 4 * (int64_t)cu;
    auto valid = [&](int l) {
        for (const FwdEntry& e : fwd_table(op))
            if (e.hidden == hidden && e.lanes == l && e.depth == 0) return true;
        return false;
    };
    const int max_vecs = (op != NORM_OP_LAYERNORM_FWD && rows >= 16 * (int64_t)cu) ? 4 : 8;
    int lanes = 64;
    while (lanes < 1024 && (hidden / (8 * lanes) > max_vecs || !valid(lanes))) lanes *= 2;
    while (lanes < 1024 && rows * (lanes / 64) < target_waves && valid(lanes * 2)) lanes *= 2;
    int rpb = lanes == 64 ? 4 : (lanes == 128 ? 2 : 1);
    while (rpb > 1 && !find_fwd(op, hidden, lanes, rpb)) rpb /= 2;
    return norm_launch_cfg{lanes, rpb, 0, 0};
}

// Run-time-hidden forward: the same two rules in units of accesses of w
// elements, and never more lanes than the row has accesses.  Rows of at most
// 64 accesses get one access per lane (rows narrower than a wave share it),
// so each load instruction of a wave covers whole rows: measured 1.5x faster
// than two accesses per lane for 128-wide rows.  Returns lanes 0 when no
// compiled instantiation holds the row.
// Rows narrower than a wave are addressed through one descriptor per set of
// `rows_per_set` rows; its byte extent must stay below the out-of-range
// offset used for masked accesses.
bool row_set_fits(int lanes, int64_t rows_per_set, int64_t ld_max, int64_t hidden) {
    return lanes >= 64 || ((rows_per_set - 1) * ld_max + hidden) * 2 < 0x7ffffff0;
}

norm_launch_cfg choose_dyn_fwd(norm_op op, int64_t rows, int64_t hidden, int w, int cu,
                               int64_t ld_max) {
    const int64_t nacc = hidden / w;
    const int64_t target_lanes = 4 * (int64_t)cu * 64;
    const int64_t vcap = (op != NORM_OP_LAYERNORM_FWD && rows >= 16 * (int64_t)cu) ? 4 : 8;
    // LayerNorm holds its row for two passes; below a wave, about three
    // accesses a lane (rows of 128-768 bf16 values on 8-32 lanes) ran 3-15 %
    // faster than one access a lane on as many lanes as accesses
    const bool ln = op == NORM_OP_LAYERNORM_FWD;
    int lanes = 8;
    while (lanes < 64 && (ln ? 3 * (int64_t)lanes < nacc : lanes < nacc)) lanes *= 2;
    while (lanes < 1024 && ceil_div(nacc, lanes) > vcap) lanes *= 2;
    while (lanes < 1024 && lanes < nacc && rows * lanes < target_lanes) lanes *= 2;
    while (lanes < 64 && !row_set_fits(lanes, dyn_rows_per_block(lanes), ld_max, hidden))
        lanes *= 2;
    for (; lanes <= 1024; lanes *= 2) {
        if (!find_dyn(dyn_fwd_table(op), hidden, w, lanes)) continue;
        const int r = dyn_rows_per_block(lanes);
        // LayerNorm: four rows per lane group while that leaves 4 workgroups
        // per CU (rows of 64-512 on 8-32 lanes: 3-15 % over one and two)
        if (ln && lanes < 64 && ceil_div(rows, 4 * r) >= 4 * (int64_t)cu &&
            row_set_fits(lanes, 4 * r, ld_max, hidden) &&
            find_dyn(dyn_fwd_table(op), hidden, w, lanes, 4))
            return norm_launch_cfg{lanes, 4 * r, 0, w};
        // rows narrower than a wave: two rows per lane group while that still
        // leaves 8 workgroups per CU (3-6 % faster at 64k-256k rows of 64-256)
        if (lanes < 64 && ceil_div(rows, 2 * r) >= 8 * (int64_t)cu &&
            row_set_fits(lanes, 2 * r, ld_max, hidden) &&
            find_dyn(dyn_fwd_table(op), hidden, w, lanes, 2))
            return norm_launch_cfg{lanes, 2 * r, 0, w};
        return norm_launch_cfg{lanes, r, 0, w};
    }
    if (stream_fwd_ok(op, hidden, w)) return norm_launch_cfg{kStreamFwdLanes, 1, 0, 8};
    return norm_launch_cfg{0, 0, 0, w};
}

// LayerNorm backward: one persistent workgroup per compute unit of the
// largest part (256 on MI355X) made the best trade-off between rows in flight
// and partial-sum slabs to reduce; the grid is a constant, not a device query,
// so the workspace size is pure host arithmetic.
int32_t default_bwd_grid(int64_t rows, int rows_per_block = 1) {
    constexpr int64_t kGroups = 256;
    const int64_t g = ceil_div(std::max<int64_t>(rows, 1), rows_per_block);
    return (int32_t)std::min(g, kGroups);
}

norm_launch_cfg choose_bwd(norm_op op, int64_t rows, int64_t hidden) {
    // one 16-byte vector of x and of dy per lane when compiled (512 lanes at
    // hidden 4096, 1024 at 8192), else the shape with the fewest vectors per lane
    int best = 0;
    for (const BwdEntry& e : bwd_table(op)) {
        if (e.hidden != hidden) continue;
        if (best == 0 || e.lanes > best) best = e.lanes;
    }
    return norm_launch_cfg{best, 1, default_bwd_grid(rows), 0};
}

// Run-time-hidden backward: one access per lane up to 256 lanes, then up to
// 4 accesses per lane on 256 lanes before going wider (measured at hidden
// 5120: 256 lanes x 3 accesses 13-16 % faster than 1024 lanes x 1, which
// leaves lanes idle and caps a lane at 128 VGPRs, a shallower ring).
norm_launch_cfg choose_dyn_bwd(norm_op op, int64_t rows, int64_t hidden, int w,
                               int64_t ld_max) {
    const int64_t nacc = hidden / w;
    int lanes = 8;
    while (lanes < 256 && lanes < nacc) lanes *= 2;
    while (lanes < 64 && !row_set_fits(lanes, dyn_rows_per_block(lanes), ld_max, hidden))
        lanes *= 2;
    for (; lanes <= 1024; lanes *= 2)
        if (row_set_fits(lanes, dyn_rows_per_block(lanes), ld_max, hidden) &&
            find_dyn(dyn_bwd_table(op), hidden, w, lanes)) {
            const int r = dyn_rows_per_block(lanes);
            return norm_launch_cfg{lanes, r, default_bwd_grid(rows, r), w};
        }
    if (find_wide(op, hidden, kWideBwdLanes, w))
        return norm_launch_cfg{kWideBwdLanes, 1, default_bwd_grid(rows), w};
    if (stream_bwd_ok(op, hidden, w))
        return norm_launch_cfg{kStreamTileLanes, 1, stream_walkers(rows, hidden), 8};
    return norm_launch_cfg{0, 0, 0, w};
}

size_t static_ws_bytes(norm_op op, int64_t hidden, int64_t grid) {
    return (size_t)grid * (size_t)bwd_outs(op) * (size_t)hidden * sizeof(float);
}

size_t dyn_ws_bytes(norm_op op, int64_t hidden, int64_t slabs) {
    return (size_t)slabs * (size_t)bwd_outs(op) * (size_t)dyn_padded_hidden(hidden) *
           sizeof(float);
}

// Streamed backward: the walkers' slabs, then the exchange area of the
// tiles' partial sums (per walker kXchRing rows of `tiles` 16-byte slots;
// none with one tile, which reduces its rows itself), or past kXchMaxTiles
// tiles two floats a row (the row sums kernel's output).
size_t stream_ws_bytes(norm_op op, int64_t hidden, int64_t walkers, int64_t rows,
                       int64_t tiles) {
    if (!stream_bwd_xch(hidden))
        return dyn_ws_bytes(op, hidden, walkers) + (size_t)std::max<int64_t>(rows, 0) * 8;
    return dyn_ws_bytes(op, hidden, walkers) + (size_t)(rows > 0 ? xch_bytes(walkers, tiles) : 0);
}

// The column reduce addresses the workspace with 32-bit byte offsets and
// reads at most one slab past the last one (clamped, range-checked to zero).
bool dyn_slabs_fit(norm_op op, int64_t hidden, int64_t slabs) {
    return (slabs + 1) * bwd_outs(op) * dyn_padded_hidden(hidden) * 4 <= INT32_MAX;
}

norm_status from_hip(hipError_t e) { return e == hipSuccess ? NORM_SUCCESS : NORM_ERROR_LAUNCH; }

// ---- forward entry -------------------------------------------------------------
struct FwdCall {
    void* out;
    int64_t ld_out;
    void* residual;
    int64_t ld_res;
    const void* x;
    int64_t ld_x;
    const void* weight;
    const void* bias;
    float* mean;
    float* rstd;
    int64_t rows, hidden;
    float eps;
};

// What the checks of a forward call found out about its layout.
struct FwdLayout {
    int64_t ld_res;    // the residual's stride (hidden for the unfused ops)
    int ws, wp;        // widest access the shape / the pointers allow
    int w_max;         // min(ws, wp)
    bool contiguous;   // every matrix has ld == hidden
    bool compiled_ok;  // a compiled-hidden kernel can run it
};

// Argument checks every forward entry shares (cfg aside).  NORM_SUCCESS with
// rows == 0 means: nothing to launch.
norm_status check_fwd(norm_op op, const FwdCall& c, FwdLayout* L) {
    const bool fused = op == NORM_OP_FUSED_ADD_RMSNORM;
    const bool ln = op == NORM_OP_LAYERNORM_FWD;
    if (c.rows < 0 || c.rows > kMaxRows || !eps_ok(c.eps)) return NORM_ERROR_INVALID_VALUE;
    if (c.rows == 0) return NORM_SUCCESS;
    if (c.hidden < 1 || c.hidden > kMaxHidden) return NORM_ERROR_UNSUPPORTED_HIDDEN;
    if (!c.out || !c.x || !c.weight || (fused && !c.residual) || (ln && !c.bias))
        return NORM_ERROR_INVALID_VALUE;
    if (ln && ((c.mean == nullptr) != (c.rstd == nullptr))) return NORM_ERROR_INVALID_VALUE;
    const int64_t ld_res = fused ? c.ld_res : c.hidden;
    for (int64_t ld : {c.ld_out, c.ld_x, ld_res})
        if (ld < c.hidden || ld > kMaxLd || !span_ok(c.rows, ld, c.hidden, 2))
            return NORM_ERROR_INVALID_VALUE;
    if (!aligned(c.out, 2) || !aligned(c.x, 2) || !aligned(c.weight, 2) ||
        (fused && !aligned(c.residual, 2)) || (ln && !aligned(c.bias, 2)) ||
        (ln && c.mean && (!aligned(c.mean, 4) || !aligned(c.rstd, 4))))
        return NORM_ERROR_MISALIGNED;

    const Region out{c.out, c.rows, c.ld_out, c.hidden, 2}, x{c.x, c.rows, c.ld_x, c.hidden, 2};
    const Region res{fused ? c.residual : nullptr, c.rows, ld_res, c.hidden, 2};
    const Region w = vec_region(c.weight, c.hidden, 2);
    const Region b = vec_region(ln ? c.bias : nullptr, c.hidden, 2);
    const Region mean = vec_region(ln ? c.mean : nullptr, c.rows, 4);
    const Region rstd = vec_region(ln ? c.rstd : nullptr, c.rows, 4);
    // outputs must not overlap anything, except out == x exactly
    if (conflict(out, x, true) || conflict(out, w, false) || conflict(out, res, false) ||
        conflict(out, b, false) || conflict(out, mean, false) || conflict(out, rstd, false) ||
        conflict(res, x, false) || conflict(res, w, false) || conflict(res, b, false) ||
        conflict(mean, x, false) || conflict(mean, w, false) || conflict(mean, b, false) ||
        conflict(mean, rstd, false) || conflict(rstd, x, false) || conflict(rstd, w, false) ||
        conflict(rstd, b, false))
        return NORM_ERROR_INVALID_VALUE;

    L->ld_res = ld_res;
    L->ws = shape_width(c.hidden, {c.ld_out, c.ld_x, ld_res});
    L->wp = pointer_width({c.out, c.x, c.weight, fused ? c.residual : nullptr,
                           ln ? c.bias : nullptr});
    L->w_max = std::min(L->ws, L->wp);
    L->contiguous = c.ld_out == c.hidden && c.ld_x == c.hidden && ld_res == c.hidden;
    L->compiled_ok = hidden_compiled(c.hidden) && L->contiguous && L->w_max == 8;
    return NORM_SUCCESS;
}

norm_status run_fwd(norm_op op, const FwdCall& c, const norm_launch_cfg* cfg,
                    hipStream_t stream) {
    const bool has_ring = op == NORM_OP_LAYERNORM_FWD || op == NORM_OP_RMSNORM_FWD;
    if (c.rows < 0 || c.rows > kMaxRows || !eps_ok(c.eps)) return NORM_ERROR_INVALID_VALUE;
    // grid > 0 names a persistent ring shape: LayerNorm's and RMSNorm's
    // compiled kernels only
    if (cfg && (cfg->grid < 0 || cfg->grid > kMaxFwdRingGrid ||
                (cfg->grid > 0 &&
                 (!has_ring || cfg->vector_elems != 0 || cfg->rows_per_block != 1)) ||
                cfg->threads_per_row <= 0 || cfg->rows_per_block <= 0 ||
                !valid_elems(cfg->vector_elems)))
        return NORM_ERROR_INVALID_VALUE;
    FwdLayout L;
    const norm_status chk = check_fwd(op, c, &L);
    if (chk != NORM_SUCCESS || c.rows == 0) return chk;
    const int64_t ld_res = L.ld_res;
    const int ws = L.ws, wp = L.wp, w_max = L.w_max;
    const bool contiguous = L.contiguous, compiled_ok = L.compiled_ok;

    if (!compiled_ok && !(cfg && cfg->vector_elems == 0) &&
        c.hidden > max_dyn_hidden(dyn_fwd_table(op), cfg ? cfg->vector_elems : w_max) &&
        !stream_fwd_ok(op, c.hidden, cfg ? cfg->vector_elems : w_max))
        return NORM_ERROR_UNSUPPORTED_HIDDEN;

    norm_launch_cfg k;
    int cu = 0;  // queried only where a choice needs it
    if (cfg && cfg->vector_elems == 0) {  // a compiled-hidden shape was asked for
        if (!hidden_compiled(c.hidden)) return NORM_ERROR_UNSUPPORTED_HIDDEN;
        if (!contiguous) return NORM_ERROR_INVALID_VALUE;
        if (wp < 8) return NORM_ERROR_MISALIGNED;
        k = *cfg;
    } else if (cfg) {  // a run-time-hidden shape was asked for
        if (cfg->vector_elems > ws) return NORM_ERROR_INVALID_VALUE;
        if (cfg->vector_elems > wp) return NORM_ERROR_MISALIGNED;
        k = *cfg;
    } else {
        const norm_status st = current_cu_count(&cu);
        if (st != NORM_SUCCESS) return st;
        k = compiled_ok ? choose_fwd(op, c.rows, c.hidden, cu)
                        : choose_dyn_fwd(op, c.rows, c.hidden, w_max, cu,
                                         std::max({c.ld_out, c.ld_x, ld_res}));
        if (k.threads_per_row == 0) return NORM_ERROR_UNSUPPORTED_HIDDEN;
    }

    if (k.vector_elems == 0) {
        const FwdEntry* e =
            k.grid > 0 ? (k.rows_per_block == 1 ? ring_entry(op, c.hidden, k.threads_per_row,
                                                             c.rows, k.grid)
                                                : nullptr)
                       : find_fwd(op, c.hidden, k.threads_per_row, k.rows_per_block);
        if (!e) return NORM_ERROR_INVALID_VALUE;
        const int64_t groups = k.grid > 0 ? k.grid : ceil_div(c.rows, k.rows_per_block);
        if (groups > INT32_MAX ||
            groups * k.threads_per_row * k.rows_per_block > (int64_t)UINT32_MAX)
            return NORM_ERROR_INVALID_VALUE;
        const FwdArgs a{c.out, c.residual, c.x,    c.weight, c.bias,
                        c.mean, c.rstd,    c.rows, c.eps,    k.grid};
        FwdLauncher launch = e->launch;
        if (e->launch_late && late_listed(op, c.hidden, k.threads_per_row, k.rows_per_block)) {
            if (cu == 0) {
                const norm_status st = current_cu_count(&cu);
                if (st != NORM_SUCCESS) return st;
            }
            if (late_weights(op, c.rows, c.hidden, k.threads_per_row, k.rows_per_block, cu))
                launch = e->launch_late;
        }
        return from_hip(launch(a, stream));
    }
    // rows per workgroup = R lane groups x K rows per group
    const int r = dyn_rows_per_block(k.threads_per_row);
    if (k.rows_per_block % r != 0 ||
        !row_set_fits(k.threads_per_row, k.rows_per_block, std::max({c.ld_out, c.ld_x, ld_res}),
                      c.hidden))
        return NORM_ERROR_INVALID_VALUE;
    const DynFwdEntry* e = find_dyn(dyn_fwd_table(op), c.hidden, k.vector_elems,
                                    k.threads_per_row, k.rows_per_block / r);
    if (!e && k.vector_elems == 8 && k.threads_per_row == kStreamFwdLanes &&
        k.rows_per_block == 1 && stream_fwd_ok(op, c.hidden, 8)) {
        // a row no workgroup holds on chip: the streamed two-pass kernel
        const DynFwdArgs a{c.out,     c.residual, c.x,   c.weight, c.bias,   c.mean,
                           c.rstd,    c.ld_out,   ld_res, c.ld_x,  c.rows,   (int32_t)c.hidden,
                           c.eps};
        const int sop = op == NORM_OP_FUSED_ADD_RMSNORM ? kSplitFused
                        : op == NORM_OP_LAYERNORM_FWD   ? kSplitLn
                                                        : kSplitRms;
        return from_hip(launch_stream_fwd(sop, false, a, stream));
    }
    if (!e) return cfg ? NORM_ERROR_INVALID_VALUE : NORM_ERROR_UNSUPPORTED_HIDDEN;
    const int64_t groups = ceil_div(c.rows, k.rows_per_block);
    if (groups > INT32_MAX || groups * dyn_block_size(k.threads_per_row) > (int64_t)UINT32_MAX)
        return NORM_ERROR_INVALID_VALUE;
    const DynFwdArgs a{c.out,     c.residual, c.x,   c.weight, c.bias,   c.mean,
                       c.rstd,    c.ld_out,   ld_res, c.ld_x,  c.rows,   (int32_t)c.hidden,
                       c.eps};
    if (cu == 0) {
        const norm_status st = current_cu_count(&cu);
        if (st != NORM_SUCCESS) return st;
    }
    return from_hip((late_weights_dyn(groups, k.threads_per_row, cu) ? e->launch_late
                                                                      : e->launch)(a, stream));
}

// ---- row-split forward entry ---------------------------------------------------
// Splitting costs ~1 us (the partners' round trip through the workspace) and
// pays only where one workgroup is slow to move its row.  Measured (one MI355X,
// graph-timed, us; "plain" = one workgroup per row):
//   fused 1 x 16384 (128 KiB a row): plain 3.0, best split 3.3   -> not split
//   fused 8 x 24576 (192 KiB):       plain 4.7, k = 3 4.8         -> not split
//   fused 1 x 32768 (256 KiB):       plain 5.4, k = 4 3.7
//   RMSNorm 1 x 49152 (192 KiB):     plain 4.4, k = 4 3.7
//   fused 16 x 49152 (384 KiB):      plain 9.2, k = 4 7.1; 16 x 32768: 6.6 vs 6.4
//   fused 32 x 65536:                plain 12.3, k = 4 10.2; 64 rows: plain wins
// So: up to 8 rows, rows moving >= 256 KiB (fused) or 192 KiB (the others);
// 9-32 rows, >= 384 KiB; chunks of
// ~64 KiB of traffic (8192 columns fused, 16384 RMSNorm, 12288 LayerNorm);
// at most max(4, 64 / rows) chunks a row (16 x 65536 fused: k = 4 7.7 us,
// k = 8 9.0 us).  Rows that no one-workgroup-per-row kernel holds (LayerNorm
// above 49152) are split whenever a shape exists, up to 64 rows.
constexpr int64_t kSplitMaxRows = 512;

// Polls a partner wait makes before it gives up; process-wide, changed only by
// norm_split_set_spin_limit (tests and diagnostics force a give-up with 0).
std::atomic<uint32_t> g_split_spin_limit{kSplitSpinLimit};

size_t split_ws_bytes(int64_t rows) {
    if (rows <= 0) return 0;
    return (size_t)kSplitHeaderWords * 4 +
           (size_t)std::min(rows, kSplitMaxRows) * kSplitRowQwords * 8;
}

struct SplitShape {
    int k;     // workgroups per row (1: no split)
    int vecs;  // 16-byte accesses per lane
};

// The (k, V) of an explicit request of `split` workgroups per row: V is the
// fewest accesses a lane that covers the row in `split` chunks, k the chunks
// that V then needs (no empty chunk).  vecs = 0 when no such shape exists.
SplitShape split_shape(int64_t hidden, int64_t split) {
    if (split < 1) return {1, 0};
    const int64_t acc = hidden / 8;
    const int64_t v = ceil_div(acc, (int64_t)kSplitLanes * split);
    if (v < 1 || v > kSplitMaxVecs) return {1, 0};
    return {(int)ceil_div(acc, (int64_t)kSplitLanes * v), (int)v};
}

// Whether a one-workgroup-per-row kernel holds contiguous 16-byte rows of
// this hidden size.
bool fwd_plain_holds(norm_op op, int64_t hidden) {
    return hidden_compiled(hidden) || hidden <= max_dyn_hidden(dyn_fwd_table(op), 8);
}

SplitShape choose_split(norm_op op, int64_t rows, int64_t hidden, int cu) {
    if (rows < 1 || rows > kSplitMaxRows || hidden % 8) return {1, 0};
    const bool plain = fwd_plain_holds(op, hidden);
    const bool fused = op == NORM_OP_FUSED_ADD_RMSNORM;
    if (plain) {
        const int64_t row_bytes = (fused ? 8 : 4) * hidden;
        const int64_t min_bytes = rows > 8 ? (384 << 10) : (fused ? (256 << 10) : (192 << 10));
        if (rows > 32 || row_bytes < min_bytes) return {1, 0};
    }
    const int64_t kcap = std::min<int64_t>({(int64_t)kSplitMax, std::max<int64_t>(4, 64 / rows),
                                            cu / rows});
    if (kcap < 2) return {1, 0};
    const int64_t target = fused ? 8192 : (op == NORM_OP_LAYERNORM_FWD ? 12288 : 16384);
    const int64_t want = std::max<int64_t>(2, ceil_div(hidden, target));
    SplitShape sh = split_shape(hidden, std::min(kcap, want));
    if (sh.vecs == 0 && !plain) sh = split_shape(hidden, kcap);  // needs more, smaller chunks
    return sh.vecs == 0 || sh.k < 2 ? SplitShape{1, 0} : sh;
}

// The workspace of a row-split call: big enough, 16-byte aligned, apart from
// every other argument.
norm_status check_split_ws(norm_op op, const FwdCall& c, const FwdLayout& L, void* workspace,
                           size_t ws_bytes) {
    if (!workspace || ws_bytes < split_ws_bytes(c.rows)) return NORM_ERROR_WORKSPACE;
    if (!aligned(workspace, 16)) return NORM_ERROR_MISALIGNED;
    const bool fused = op == NORM_OP_FUSED_ADD_RMSNORM;
    const bool ln = op == NORM_OP_LAYERNORM_FWD;
    const Region wsr = vec_region(workspace, (int64_t)split_ws_bytes(c.rows), 1);
    for (const Region& r : {Region{c.out, c.rows, c.ld_out, c.hidden, 2},
                            Region{c.x, c.rows, c.ld_x, c.hidden, 2},
                            Region{fused ? c.residual : nullptr, c.rows, L.ld_res, c.hidden, 2},
                            vec_region(c.weight, c.hidden, 2),
                            vec_region(ln ? c.bias : nullptr, c.hidden, 2),
                            vec_region(ln ? c.mean : nullptr, c.rows, 4),
                            vec_region(ln ? c.rstd : nullptr, c.rows, 4)})
        if (conflict(wsr, r, false)) return NORM_ERROR_INVALID_VALUE;
    return NORM_SUCCESS;
}

norm_status run_fwd_split(norm_op op, const FwdCall& c, void* workspace, size_t ws_bytes,
                          int32_t split, hipStream_t stream) {
    if (split < 0 || split > kSplitMax) return NORM_ERROR_INVALID_VALUE;
    if (split == 1) return run_fwd(op, c, nullptr, stream);
    FwdLayout L;
    norm_status st = check_fwd(op, c, &L);
    if (st != NORM_SUCCESS || c.rows == 0) return st;
    SplitShape sh;
    int cu = 0;
    if (split >= 2) {  // everything but the CU count is checked before any HIP call
        if (!L.contiguous || L.ws < 8 || c.rows > kSplitMaxRows) return NORM_ERROR_INVALID_VALUE;
        if (L.wp < 8) return NORM_ERROR_MISALIGNED;
        sh = split_shape(c.hidden, split);
        if (sh.vecs == 0) return NORM_ERROR_INVALID_VALUE;
        if ((st = check_split_ws(op, c, L, workspace, ws_bytes)) != NORM_SUCCESS) return st;
        if ((st = current_cu_count(&cu)) != NORM_SUCCESS) return st;
        if (c.rows * sh.k > cu) return NORM_ERROR_INVALID_VALUE;
    } else {
        if (!L.contiguous || L.w_max < 8) return run_fwd(op, c, nullptr, stream);
        if ((st = current_cu_count(&cu)) != NORM_SUCCESS) return st;
        sh = choose_split(op, c.rows, c.hidden, cu);
        if (sh.k == 1) return run_fwd(op, c, nullptr, stream);
        if ((st = check_split_ws(op, c, L, workspace, ws_bytes)) != NORM_SUCCESS) return st;
    }

    const int sop = op == NORM_OP_FUSED_ADD_RMSNORM ? kSplitFused
                    : op == NORM_OP_LAYERNORM_FWD   ? kSplitLn
                                                    : kSplitRms;
    for (const SplitEntry& e : split_table())
        if (e.op == sop && e.vecs == sh.vecs) {
            const SplitArgs a{c.out,     c.residual, c.x,      c.weight, c.bias,
                              c.mean,    c.rstd,     static_cast<uint32_t*>(workspace),
                              c.ld_out,  L.ld_res,   c.ld_x,   c.rows,   (int32_t)c.hidden,
                              sh.k,      c.eps,      g_split_spin_limit.load()};
            return from_hip(e.launch(a, stream));
        }
    return NORM_ERROR_INVALID_VALUE;
}

// ---- backward entry ------------------------------------------------------------
struct BwdCall {
    void* dx;
    int64_t ld_dx;
    const void* dy;
    int64_t ld_dy;
    const void* x;
    int64_t ld_x;
    const float* mean;
    const float* rstd;
    const void* dres;
    int64_t ld_dres;
    const void* weight;
    void* workspace;
    size_t workspace_bytes;
    float* dweight;
    float* dbias;
    int64_t rows, hidden;
    float eps;
    // workspace == NULL and workspace_bytes == kScratchBytes: the slabs go to
    // this device's scratch array, looked up after every argument check
    bool use_scratch = false;
};

norm_status run_bwd(norm_op op, const BwdCall& c, const norm_launch_cfg* cfg,
                    hipStream_t stream) {
    const bool ln = op == NORM_OP_LAYERNORM_BWD;
    if (c.rows < 0 || c.rows > kMaxRows || !eps_ok(c.eps)) return NORM_ERROR_INVALID_VALUE;
    if (cfg && (cfg->threads_per_row <= 0 || cfg->rows_per_block <= 0 || cfg->grid < 0 ||
                !valid_elems(cfg->vector_elems)))
        return NORM_ERROR_INVALID_VALUE;
    if (c.hidden < 1 || c.hidden > kMaxHidden) return NORM_ERROR_UNSUPPORTED_HIDDEN;
    const bool any = c.rows > 0;
    if (!c.dweight || (ln && !c.dbias) || (!c.workspace && !c.use_scratch))
        return NORM_ERROR_INVALID_VALUE;
    if (any && (!c.dx || !c.dy || !c.x || !c.weight || (ln && (!c.mean || !c.rstd))))
        return NORM_ERROR_INVALID_VALUE;
    const int64_t ld_dres = c.dres ? c.ld_dres : c.hidden;
    for (int64_t ld : {c.ld_dx, c.ld_dy, c.ld_x, ld_dres})
        if (ld < c.hidden || ld > kMaxLd || !span_ok(c.rows, ld, c.hidden, 2))
            return NORM_ERROR_INVALID_VALUE;
    if (!aligned(c.dweight, 4) || (ln && !aligned(c.dbias, 4)) ||
        (!c.use_scratch && !aligned(c.workspace, 16)))
        return NORM_ERROR_MISALIGNED;
    if (any && (!aligned(c.dx, 2) || !aligned(c.dy, 2) || !aligned(c.x, 2) ||
                !aligned(c.weight, 2) || (c.dres && !aligned(c.dres, 2)) ||
                (ln && (!aligned(c.mean, 4) || !aligned(c.rstd, 4)))))
        return NORM_ERROR_MISALIGNED;

    const int ws_w = shape_width(c.hidden, {c.ld_dx, c.ld_dy, c.ld_x, ld_dres});
    const int wp = any ? pointer_width({c.dx, c.dy, c.x, c.weight, c.dres}) : 8;
    const int w_max = std::min(ws_w, wp);
    const bool contiguous = c.ld_dx == c.hidden && c.ld_dy == c.hidden && c.ld_x == c.hidden &&
                            ld_dres == c.hidden;
    const bool compiled_ok = hidden_compiled(c.hidden) && contiguous && w_max == 8;

    if (!compiled_ok && !(cfg && cfg->vector_elems == 0) &&
        c.hidden > max_bwd_hidden(op, cfg ? cfg->vector_elems : w_max))
        return NORM_ERROR_UNSUPPORTED_HIDDEN;

    norm_launch_cfg k;
    if (cfg && cfg->vector_elems == 0) {
        if (!hidden_compiled(c.hidden)) return NORM_ERROR_UNSUPPORTED_HIDDEN;
        if (!contiguous || cfg->rows_per_block != 1) return NORM_ERROR_INVALID_VALUE;
        if (wp < 8) return NORM_ERROR_MISALIGNED;
        k = *cfg;
        if (k.grid == 0) k.grid = default_bwd_grid(c.rows);
        if (k.grid > max_bwd_grid(c.hidden)) return NORM_ERROR_INVALID_VALUE;
    } else if (cfg) {
        if (cfg->vector_elems > ws_w) return NORM_ERROR_INVALID_VALUE;
        if (cfg->vector_elems > wp) return NORM_ERROR_MISALIGNED;
        k = *cfg;
        if (k.rows_per_block != dyn_rows_per_block(k.threads_per_row) ||
            !row_set_fits(k.threads_per_row, k.rows_per_block,
                          std::max({c.ld_dx, c.ld_dy, c.ld_x, ld_dres}), c.hidden))
            return NORM_ERROR_INVALID_VALUE;
        if (k.grid == 0)
            k.grid = k.vector_elems == 8 && k.threads_per_row == kStreamTileLanes &&
                             stream_bwd_ok(op, c.hidden, 8)
                         ? stream_walkers(c.rows, c.hidden)
                         : default_bwd_grid(c.rows, k.rows_per_block);
    } else {
        k = compiled_ok ? choose_bwd(op, c.rows, c.hidden)
                        : choose_dyn_bwd(op, c.rows, c.hidden, w_max,
                                         std::max({c.ld_dx, c.ld_dy, c.ld_x, ld_dres}));
        if (k.threads_per_row == 0) return NORM_ERROR_UNSUPPORTED_HIDDEN;
    }

    const BwdEntry* se = nullptr;
    DynBwdLauncher dyn_launch = nullptr;
    bool streamed = false;
    size_t ws_need = 0;
    if (k.vector_elems == 0) {
        se = find_bwd(op, c.hidden, k.threads_per_row);
        if (!se) return NORM_ERROR_INVALID_VALUE;
        ws_need = static_ws_bytes(op, c.hidden, any ? k.grid : 0);
    } else {
        if (const DynBwdEntry* de =
                find_dyn(dyn_bwd_table(op), c.hidden, k.vector_elems, k.threads_per_row))
            dyn_launch = de->launch;
        else if (const WideBwdEntry* we =
                     find_wide(op, c.hidden, k.threads_per_row, k.vector_elems))
            dyn_launch = we->launch;
        else if (k.vector_elems == 8 && k.threads_per_row == kStreamTileLanes &&
                 stream_bwd_ok(op, c.hidden, 8))
            streamed = true;  // row statistics, then column tiles (kernels_stream.hpp)
        if (!dyn_launch && !streamed)
            return cfg ? NORM_ERROR_INVALID_VALUE : NORM_ERROR_UNSUPPORTED_HIDDEN;
        if (streamed && !cfg && stream_bwd_xch(c.hidden))
            k.grid = resident_walkers(k.grid, stream_tiles(c.hidden), kXchLanesBf16);
        const int64_t slabs = k.grid;  // one slab per workgroup (streamed: per walker)
        if (!dyn_slabs_fit(op, c.hidden, slabs) ||
            (streamed && slabs * stream_tiles(c.hidden) > INT32_MAX))
            return NORM_ERROR_INVALID_VALUE;
        ws_need = streamed ? stream_ws_bytes(op, c.hidden, any ? slabs : 0, any ? c.rows : 0,
                                             stream_tiles(c.hidden))
                           : dyn_ws_bytes(op, c.hidden, any ? slabs : 0);
    }

    const int64_t mrows = any ? c.rows : 0;
    const Region dx{c.dx, mrows, c.ld_dx, c.hidden, 2}, dy{c.dy, mrows, c.ld_dy, c.hidden, 2},
        x{c.x, mrows, c.ld_x, c.hidden, 2}, dres{c.dres, mrows, ld_dres, c.hidden, 2};
    const Region mean = vec_region(ln ? c.mean : nullptr, mrows, 4),
                 rstd = vec_region(ln ? c.rstd : nullptr, mrows, 4),
                 w = vec_region(any ? c.weight : nullptr, c.hidden, 2),
                 dw = vec_region(c.dweight, c.hidden, 4),
                 db = vec_region(ln ? c.dbias : nullptr, c.hidden, 4),
                 wsr = vec_region(c.workspace, (int64_t)ws_need, 1);
    // outputs overlap no input, except dx == dy (or dx == dres) exactly
    for (const Region* in : {&dy, &x, &mean, &rstd, &dres, &w}) {
        const bool alias_ok = in == &dy || in == &dres;
        if (conflict(dx, *in, alias_ok) || conflict(dw, *in, false) ||
            conflict(db, *in, false) || conflict(wsr, *in, false))
            return NORM_ERROR_INVALID_VALUE;
    }
    if (conflict(dx, dw, false) || conflict(dx, db, false) || conflict(dx, wsr, false) ||
        conflict(dw, db, false) || conflict(dw, wsr, false) || conflict(db, wsr, false))
        return NORM_ERROR_INVALID_VALUE;
    if (c.workspace_bytes < ws_need) return NORM_ERROR_WORKSPACE;

    void* ws = c.workspace;
    if (c.use_scratch) {
        const norm_status st = current_scratch(&ws);
        if (st != NORM_SUCCESS) return st;
    }
    if (se) {
        const BwdArgs a{c.dx,     c.dy,      c.x,    c.mean, c.rstd,    c.dres, c.weight,
                        (float*)ws, c.dweight, c.dbias, c.rows, k.grid, c.eps};
        return from_hip(se->launch(a, stream));
    }
    const DynBwdArgs a{c.dx,    c.dy,     c.x,       c.mean,  c.rstd,
                       c.dres,  c.weight, (float*)ws, c.dweight, c.dbias,
                       c.ld_dx, c.ld_dy,  c.ld_x,    ld_dres, c.rows,
                       (int32_t)c.hidden, k.grid, c.eps};
    if (streamed)
        return from_hip(launch_stream_bwd(op == NORM_OP_LAYERNORM_BWD, false, a,
                                          stream_tiles(c.hidden), k.grid, stream));
    return from_hip(dyn_launch(a, stream));
}

// Workspace for (op, rows, hidden): the given shape's, or with cfg == NULL the
// largest the library's choice can need for any layout of this hidden size
// (the compiled kernels, or the run-time kernels at any access width).
size_t ws_query(norm_op op, int64_t rows, int64_t hidden, const norm_launch_cfg* cfg) {
    if (rows <= 0 || hidden < 1 || hidden > kMaxHidden) return 0;
    if (cfg) {
        if (cfg->vector_elems == 0) {
            if (!hidden_compiled(hidden)) return 0;
            return static_ws_bytes(op, hidden, cfg->grid > 0 ? cfg->grid : default_bwd_grid(rows));
        }
        if (!valid_elems(cfg->vector_elems) || cfg->threads_per_row <= 0) return 0;
        const int r = dyn_rows_per_block(cfg->threads_per_row);
        if (cfg->vector_elems == 8 && cfg->threads_per_row == kStreamTileLanes &&
            stream_bwd_ok(op, hidden, 8))
            return stream_ws_bytes(op, hidden,
                                   cfg->grid > 0 ? cfg->grid : stream_walkers(rows, hidden), rows,
                                   stream_tiles(hidden));
        const int64_t g = cfg->grid > 0 ? cfg->grid : default_bwd_grid(rows, r);
        return dyn_ws_bytes(op, hidden, g);
    }
    size_t need = 0;
    if (hidden_compiled(hidden))
        need = static_ws_bytes(op, hidden, choose_bwd(op, rows, hidden).grid);
    for (int w : {8, 4, 2, 1}) {
        if (hidden % w) continue;
        const norm_launch_cfg k = choose_dyn_bwd(op, rows, hidden, w, hidden);
        if (k.threads_per_row)
            need = std::max(need, stream_bwd_ok(op, hidden, w) && w == 8
                                      ? stream_ws_bytes(op, hidden, k.grid, rows,
                                                        stream_tiles(hidden))
                                      : dyn_ws_bytes(op, hidden, k.grid));
    }
    return need;
}

// The library's choice for contiguous, 16-byte-aligned buffers.
norm_status select(norm_op op, int64_t rows, int64_t hidden, int32_t cu_count,
                   norm_launch_cfg* cfg) {
    if (hidden < 1 || hidden > kMaxHidden) return NORM_ERROR_UNSUPPORTED_HIDDEN;
    const int w = shape_width(hidden, {});
    norm_launch_cfg k;
    if (is_bwd(op)) {
        k = hidden_compiled(hidden) ? choose_bwd(op, rows, hidden)
                                    : choose_dyn_bwd(op, rows, hidden, w, hidden);
        // the exchange's walkers as the launch caps them to the CUs (given, or
        // the current device's; with neither, the 256-CU default)
        if (k.vector_elems == 8 && k.threads_per_row == kStreamTileLanes &&
            stream_bwd_ok(op, hidden, 8) && stream_bwd_xch(hidden) &&
            !find_wide(op, hidden, k.threads_per_row, 8)) {
            int cu = cu_count;
            if (cu <= 0 && current_cu_count(&cu) != NORM_SUCCESS) cu = 0;
            k.grid = resident_walkers_on(k.grid, stream_tiles(hidden), kXchLanesBf16, cu);
        }
    } else {
        int cu = cu_count;
        if (cu <= 0) {
            const norm_status st = current_cu_count(&cu);
            if (st != NORM_SUCCESS) return st;
        }
        k = hidden_compiled(hidden) ? choose_fwd(op, rows, hidden, cu)
                                    : choose_dyn_fwd(op, rows, hidden, w, cu, hidden);
    }
    if (k.threads_per_row == 0) return NORM_ERROR_UNSUPPORTED_HIDDEN;
    *cfg = k;
    return NORM_SUCCESS;
}

// ---- fp32 activations ------------------------------------------------------------
// fp32 calls run the streamed kernels (kernels_stream.hpp) with four fp32
// values a 16-byte access, and the backward's rows of 8196 ... 16384 columns
// the LDS-staged kernel (kernels_bwd_wide.hpp): contiguous rows, hidden a
// multiple of 4 up to kStreamMaxHidden, the matrices and weight / bias
// vectors 16-byte aligned, mean / rstd 4-byte aligned.  The forward reads a
// row of up to 16384 values (32768 for fused / RMSNorm) once and a wider one
// twice; the backward reads a row of up to 16384 values once (one tile of the
// tile kernel up to 8192, LDS above) and a wider one twice (the streamed
// pair), then the column reduce.
// One 512-lane tile holds a row of up to kStreamTileColsF32 (reduced in the
// tile); wider rows: exchange tiles of kXchTileColsF32 up to the exchange's
// width, else the row sums kernel's 8192-column tiles.
int32_t stream_tiles_f32(int64_t hidden) {
    if (hidden <= kStreamTileColsF32) return 1;
    return (int32_t)ceil_div(hidden, stream_bwd_xch(hidden) ? kXchTileColsF32 : kStreamTileColsF32);
}
int32_t stream_walkers_f32(int64_t rows, int64_t hidden) {
    const int32_t tiles = stream_tiles_f32(hidden);
    const int cap = tiles > 1 && stream_bwd_xch(hidden) && kXchLanesF32 < kStreamTileLanes
                        ? kXchWgCap
                        : 255;
    return (int32_t)std::max<int64_t>(1, std::min<int64_t>(rows, cap / tiles));
}
bool f32_hidden_ok(int64_t hidden) {
    return hidden >= 4 && hidden % 4 == 0 && hidden <= kStreamMaxHidden;
}
// fp32 backward rows the LDS-staged kernel holds (read once; one workgroup
// per row walker, up to 256).  Build-time switch for measurement: 0 sends
// them to the streamed pair.
#ifndef ROWNORM_F32_WIDE_BWD
#define ROWNORM_F32_WIDE_BWD 1
#endif
bool f32_wide(int64_t hidden) {
    return ROWNORM_F32_WIDE_BWD && hidden >= kWideF32MinHidden && hidden <= kWideF32MaxHidden;
}
int32_t bwd_walkers_f32(int64_t rows, int64_t hidden) {
    return f32_wide(hidden) ? default_bwd_grid(rows) : stream_walkers_f32(rows, hidden);
}
size_t bwd_ws_bytes_f32(norm_op op, int64_t hidden, int64_t walkers, int64_t rows) {
    return f32_wide(hidden) ? dyn_ws_bytes(op, hidden, walkers)
                            : stream_ws_bytes(op, hidden, walkers, rows, stream_tiles_f32(hidden));
}

norm_status run_fwd_f32(norm_op op, const FwdCall& c, hipStream_t stream) {
    const bool fused = op == NORM_OP_FUSED_ADD_RMSNORM;
    const bool ln = op == NORM_OP_LAYERNORM_FWD;
    if (c.rows < 0 || c.rows > kMaxRows || !eps_ok(c.eps)) return NORM_ERROR_INVALID_VALUE;
    if (c.rows == 0) return NORM_SUCCESS;
    if (!f32_hidden_ok(c.hidden)) return NORM_ERROR_UNSUPPORTED_HIDDEN;
    if (!c.out || !c.x || !c.weight || (fused && !c.residual) || (ln && !c.bias))
        return NORM_ERROR_INVALID_VALUE;
    if (ln && ((c.mean == nullptr) != (c.rstd == nullptr))) return NORM_ERROR_INVALID_VALUE;
    if (!span_ok(c.rows, c.hidden, c.hidden, 4)) return NORM_ERROR_INVALID_VALUE;
    if (!aligned(c.out, 16) || !aligned(c.x, 16) || !aligned(c.weight, 16) ||
        (fused && !aligned(c.residual, 16)) || (ln && !aligned(c.bias, 16)) ||
        (ln && c.mean && (!aligned(c.mean, 4) || !aligned(c.rstd, 4))))
        return NORM_ERROR_MISALIGNED;
    const Region out{c.out, c.rows, c.hidden, c.hidden, 4}, x{c.x, c.rows, c.hidden, c.hidden, 4};
    const Region res{fused ? c.residual : nullptr, c.rows, c.hidden, c.hidden, 4};
    const Region w = vec_region(c.weight, c.hidden, 4);
    const Region b = vec_region(ln ? c.bias : nullptr, c.hidden, 4);
    const Region mean = vec_region(ln ? c.mean : nullptr, c.rows, 4);
    const Region rstd = vec_region(ln ? c.rstd : nullptr, c.rows, 4);
    // outputs must not overlap anything, except out == x exactly
    if (conflict(out, x, true) || conflict(out, w, false) || conflict(out, res, false) ||
        conflict(out, b, false) || conflict(out, mean, false) || conflict(out, rstd, false) ||
        conflict(res, x, false) || conflict(res, w, false) || conflict(res, b, false) ||
        conflict(mean, x, false) || conflict(mean, w, false) || conflict(mean, b, false) ||
        conflict(mean, rstd, false) || conflict(rstd, x, false) || conflict(rstd, w, false) ||
        conflict(rstd, b, false))
        return NORM_ERROR_INVALID_VALUE;
    const DynFwdArgs a{c.out,    c.residual, c.x,      c.weight, c.bias,
                       c.mean,   c.rstd,     c.hidden, c.hidden, c.hidden,
                       c.rows,   (int32_t)c.hidden,   c.eps};
    const int sop = fused ? kSplitFused : ln ? kSplitLn : kSplitRms;
    return from_hip(launch_stream_fwd(sop, true, a, stream));
}

size_t ws_query_f32(norm_op op, int64_t rows, int64_t hidden) {
    if (rows <= 0 || !f32_hidden_ok(hidden)) return 0;
    return bwd_ws_bytes_f32(op, hidden, bwd_walkers_f32(rows, hidden), rows);
}

norm_status run_bwd_f32(norm_op op, const BwdCall& c, hipStream_t stream) {
    const bool ln = op == NORM_OP_LAYERNORM_BWD;
    if (c.rows < 0 || c.rows > kMaxRows || !eps_ok(c.eps)) return NORM_ERROR_INVALID_VALUE;
    if (!f32_hidden_ok(c.hidden)) return NORM_ERROR_UNSUPPORTED_HIDDEN;
    const bool any = c.rows > 0;
    if (!c.dweight || (ln && !c.dbias) || !c.workspace) return NORM_ERROR_INVALID_VALUE;
    if (any && (!c.dx || !c.dy || !c.x || !c.weight || (ln && (!c.mean || !c.rstd))))
        return NORM_ERROR_INVALID_VALUE;
    if (!span_ok(c.rows, c.hidden, c.hidden, 4)) return NORM_ERROR_INVALID_VALUE;
    if (!aligned(c.dweight, 4) || (ln && !aligned(c.dbias, 4)) || !aligned(c.workspace, 16))
        return NORM_ERROR_MISALIGNED;
    if (any && (!aligned(c.dx, 16) || !aligned(c.dy, 16) || !aligned(c.x, 16) ||
                !aligned(c.weight, 16) || (c.dres && !aligned(c.dres, 16)) ||
                (ln && (!aligned(c.mean, 4) || !aligned(c.rstd, 4)))))
        return NORM_ERROR_MISALIGNED;
    const int32_t tiles = stream_tiles_f32(c.hidden);
    int32_t walkers = bwd_walkers_f32(c.rows, c.hidden);
    if (!f32_wide(c.hidden) && stream_bwd_xch(c.hidden))
        walkers = resident_walkers(walkers, tiles, kXchLanesF32);
    const size_t ws_need = bwd_ws_bytes_f32(op, c.hidden, any ? walkers : 0, any ? c.rows : 0);

    const int64_t mrows = any ? c.rows : 0;
    const int64_t h = c.hidden;
    const Region dx{c.dx, mrows, h, h, 4}, dy{c.dy, mrows, h, h, 4}, x{c.x, mrows, h, h, 4},
        dres{c.dres, mrows, h, h, 4};
    const Region mean = vec_region(ln ? c.mean : nullptr, mrows, 4),
                 rstd = vec_region(ln ? c.rstd : nullptr, mrows, 4),
                 w = vec_region(any ? c.weight : nullptr, h, 4),
                 dw = vec_region(c.dweight, h, 4),
                 db = vec_region(ln ? c.dbias : nullptr, h, 4),
                 wsr = vec_region(c.workspace, (int64_t)ws_need, 1);
    // outputs overlap no input, except dx == dy (or dx == dres) exactly
    for (const Region* in : {&dy, &x, &mean, &rstd, &dres, &w}) {
        const bool alias_ok = in == &dy || in == &dres;
        if (conflict(dx, *in, alias_ok) || conflict(dw, *in, false) ||
            conflict(db, *in, false) || conflict(wsr, *in, false))
            return NORM_ERROR_INVALID_VALUE;
    }
    if (conflict(dx, dw, false) || conflict(dx, db, false) || conflict(dx, wsr, false) ||
        conflict(dw, db, false) || conflict(dw, wsr, false) || conflict(db, wsr, false))
        return NORM_ERROR_INVALID_VALUE;
    if (c.workspace_bytes < ws_need) return NORM_ERROR_WORKSPACE;

    const DynBwdArgs a{c.dx,    c.dy,     c.x,       c.mean,    c.rstd,
                       c.dres,  c.weight, (float*)c.workspace, c.dweight, c.dbias,
                       h,       h,        h,         h,         c.rows,
                       (int32_t)h, walkers, c.eps};
    if (f32_wide(h)) return from_hip(launch_bwd_wide_f32(ln, a, stream));
    return from_hip(launch_stream_bwd(ln, true, a, tiles, walkers, stream));
}

}  // namespace

extern "C" {

const char* norm_status_string(norm_status status) {
    switch (status) {
        case NORM_SUCCESS: return "NORM_SUCCESS";
        case NORM_ERROR_INVALID_VALUE: return "NORM_ERROR_INVALID_VALUE: invalid argument";
        case NORM_ERROR_UNSUPPORTED_HIDDEN:
            return "NORM_ERROR_UNSUPPORTED_HIDDEN: no kernel holds a row of this hidden size "
                   "(forward: up to 65536, LayerNorm 49152; backward: up to 32768 with 16-byte "
                   "accesses, 16384 with 8-byte, less for narrower ones)";
        case NORM_ERROR_MISALIGNED:
            return "NORM_ERROR_MISALIGNED: bf16 pointers need 2-byte (compiled shapes: 16-byte) "
                   "alignment, fp32 pointers 4-byte, the workspace 16-byte";
        case NORM_ERROR_WORKSPACE: return "NORM_ERROR_WORKSPACE: workspace too small";
        case NORM_ERROR_LAUNCH: return "NORM_ERROR_LAUNCH: HIP reported a launch error";
        case NORM_ERROR_DEVICE: return "NORM_ERROR_DEVICE: could not query the current device";
    }
    return "unknown norm_status";
}

// ---- forward ------------------------------------------------------------------------
norm_status norm_fused_add_rmsnorm_ex(void* out, int64_t ld_out, void* residual,
                                      int64_t ld_residual, const void* x, int64_t ld_x,
                                      const void* weight, int64_t rows, int64_t hidden,
                                      float eps, const norm_launch_cfg* cfg,
                                      hipStream_t stream) {
    const FwdCall c{out,    ld_out,  residual, ld_residual, x,      ld_x, weight,
                    nullptr, nullptr, nullptr, rows,        hidden, eps};
    return run_fwd(NORM_OP_FUSED_ADD_RMSNORM, c, cfg, stream);
}

norm_status norm_fused_add_rmsnorm_cfg(void* out, void* residual, const void* x,
                                       const void* weight, int64_t rows, int64_t hidden,
                                       float eps, const norm_launch_cfg* cfg,
                                       hipStream_t stream) {
    return norm_fused_add_rmsnorm_ex(out, hidden, residual, hidden, x, hidden, weight, rows,
                                     hidden, eps, cfg, stream);
}

norm_status norm_fused_add_rmsnorm(void* out, void* residual, const void* x, const void* weight,
                                   int64_t rows, int64_t hidden, float eps, hipStream_t stream) {
    return norm_fused_add_rmsnorm_cfg(out, residual, x, weight, rows, hidden, eps, nullptr, stream);
}

norm_status norm_rmsnorm_fwd_ex(void* out, int64_t ld_out, const void* x, int64_t ld_x,
                                const void* weight, int64_t rows, int64_t hidden, float eps,
                                const norm_launch_cfg* cfg, hipStream_t stream) {
    const FwdCall c{out,    ld_out,  nullptr, hidden, x,      ld_x, weight,
                    nullptr, nullptr, nullptr, rows,  hidden, eps};
    return run_fwd(NORM_OP_RMSNORM_FWD, c, cfg, stream);
}

norm_status norm_rmsnorm_fwd_cfg(void* out, const void* x, const void* weight, int64_t rows,
                                 int64_t hidden, float eps, const norm_launch_cfg* cfg,
                                 hipStream_t stream) {
    return norm_rmsnorm_fwd_ex(out, hidden, x, hidden, weight, rows, hidden, eps, cfg, stream);
}

norm_status norm_rmsnorm_fwd(void* out, const void* x, const void* weight, int64_t rows,
                             int64_t hidden, float eps, hipStream_t stream) {
    return norm_rmsnorm_fwd_cfg(out, x, weight, rows, hidden, eps, nullptr, stream);
}

norm_status norm_layernorm_fwd_ex(void* y, int64_t ld_y, float* mean, float* rstd,
                                  const void* x, int64_t ld_x, const void* weight,
                                  const void* bias, int64_t rows, int64_t hidden, float eps,
                                  const norm_launch_cfg* cfg, hipStream_t stream) {
    const FwdCall c{y, ld_y, nullptr, hidden, x, ld_x, weight, bias, mean, rstd, rows, hidden,
                    eps};
    return run_fwd(NORM_OP_LAYERNORM_FWD, c, cfg, stream);
}

norm_status norm_layernorm_fwd_cfg(void* y, float* mean, float* rstd, const void* x,
                                   const void* weight, const void* bias, int64_t rows,
                                   int64_t hidden, float eps, const norm_launch_cfg* cfg,
                                   hipStream_t stream) {
    return norm_layernorm_fwd_ex(y, hidden, mean, rstd, x, hidden, weight, bias, rows, hidden,
                                 eps, cfg, stream);
}

norm_status norm_layernorm_fwd(void* y, float* mean, float* rstd, const void* x,
                               const void* weight, const void* bias, int64_t rows, int64_t hidden,
                               float eps, hipStream_t stream) {
    return norm_layernorm_fwd_cfg(y, mean, rstd, x, weight, bias, rows, hidden, eps, nullptr,
                                  stream);
}

// ---- row-split forward --------------------------------------------------------------
norm_status norm_fused_add_rmsnorm_split(void* out, void* residual, const void* x,
                                         const void* weight, int64_t rows, int64_t hidden,
                                         float eps, void* workspace, size_t workspace_bytes,
                                         int32_t split, hipStream_t stream) {
    const FwdCall c{out,    hidden,  residual, hidden, x,      hidden, weight,
                    nullptr, nullptr, nullptr, rows,   hidden, eps};
    return run_fwd_split(NORM_OP_FUSED_ADD_RMSNORM, c, workspace, workspace_bytes, split,
                         stream);
}

norm_status norm_rmsnorm_fwd_split(void* out, const void* x, const void* weight, int64_t rows,
                                   int64_t hidden, float eps, void* workspace,
                                   size_t workspace_bytes, int32_t split, hipStream_t stream) {
    const FwdCall c{out,    hidden,  nullptr, hidden, x,      hidden, weight,
                    nullptr, nullptr, nullptr, rows,  hidden, eps};
    return run_fwd_split(NORM_OP_RMSNORM_FWD, c, workspace, workspace_bytes, split, stream);
}

norm_status norm_layernorm_fwd_split(void* y, float* mean, float* rstd, const void* x,
                                     const void* weight, const void* bias, int64_t rows,
                                     int64_t hidden, float eps, void* workspace,
                                     size_t workspace_bytes, int32_t split, hipStream_t stream) {
    const FwdCall c{y, hidden, nullptr, hidden, x, hidden, weight, bias, mean, rstd, rows,
                    hidden, eps};
    return run_fwd_split(NORM_OP_LAYERNORM_FWD, c, workspace, workspace_bytes, split, stream);
}

size_t norm_split_workspace_bytes(int64_t rows) { return split_ws_bytes(rows); }

norm_status norm_split_status(void* workspace, int32_t clear, uint32_t* status,
                              hipStream_t stream) {
    if (!workspace || !status) return NORM_ERROR_INVALID_VALUE;
    if (!aligned(workspace, 16)) return NORM_ERROR_MISALIGNED;
    uint32_t word = 0;
    if (hipMemcpyAsync(&word, workspace, sizeof word, hipMemcpyDeviceToHost, stream) !=
            hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return NORM_ERROR_LAUNCH;
    if (word != 0 && clear) {
        static const uint32_t zero = 0;
        if (hipMemcpyAsync(workspace, &zero, sizeof zero, hipMemcpyHostToDevice, stream) !=
                hipSuccess ||
            hipStreamSynchronize(stream) != hipSuccess)
            return NORM_ERROR_LAUNCH;
    }
    *status = word;
    return NORM_SUCCESS;
}

uint32_t norm_split_set_spin_limit(uint32_t polls) { return g_split_spin_limit.exchange(polls); }

uint32_t norm_bwd_set_spin_limit(uint32_t polls) { return rownorm::g_bwd_spin_limit.exchange(polls); }

norm_status norm_select_split(norm_op op, int64_t rows, int64_t hidden, int32_t cu_count,
                              int32_t* split, int32_t* vecs) {
    if (!split || !vecs || rows < 0 || hidden < 1 ||
        (op != NORM_OP_FUSED_ADD_RMSNORM && op != NORM_OP_RMSNORM_FWD &&
         op != NORM_OP_LAYERNORM_FWD))
        return NORM_ERROR_INVALID_VALUE;
    int cu = cu_count;
    if (cu <= 0) {
        const norm_status st = current_cu_count(&cu);
        if (st != NORM_SUCCESS) return st;
    }
    const SplitShape sh = choose_split(op, rows, hidden, cu);
    *split = sh.k;
    *vecs = sh.vecs;
    return NORM_SUCCESS;
}

// ---- backward -----------------------------------------------------------------------
norm_status norm_layernorm_bwd_ex(void* dx, int64_t ld_dx, float* dweight, float* dbias,
                                  const void* dy, int64_t ld_dy, const void* x, int64_t ld_x,
                                  const float* mean, const float* rstd, const void* weight,
                                  void* workspace, size_t workspace_bytes, int64_t rows,
                                  int64_t hidden, float eps, const norm_launch_cfg* cfg,
                                  hipStream_t stream) {
    const BwdCall c{dx,     ld_dx,  dy,        ld_dy,           x,       ld_x,  mean,
                    rstd,   nullptr, hidden,   weight,          workspace, workspace_bytes,
                    dweight, dbias, rows,      hidden,          eps};
    return run_bwd(NORM_OP_LAYERNORM_BWD, c, cfg, stream);
}

norm_status norm_layernorm_bwd_cfg(void* dx, float* dweight, float* dbias, const void* dy,
                                   const void* x, const float* mean, const float* rstd,
                                   const void* weight, void* workspace, size_t workspace_bytes,
                                   int64_t rows, int64_t hidden, float eps,
                                   const norm_launch_cfg* cfg, hipStream_t stream) {
    return norm_layernorm_bwd_ex(dx, hidden, dweight, dbias, dy, hidden, x, hidden, mean, rstd,
                                 weight, workspace, workspace_bytes, rows, hidden, eps, cfg,
                                 stream);
}

norm_status norm_layernorm_bwd(void* dx, float* dweight, float* dbias, const void* dy,
                               const void* x, const float* mean, const float* rstd,
                               const void* weight, void* workspace, size_t workspace_bytes,
                               int64_t rows, int64_t hidden, float eps, hipStream_t stream) {
    return norm_layernorm_bwd_cfg(dx, dweight, dbias, dy, x, mean, rstd, weight, workspace,
                                  workspace_bytes, rows, hidden, eps, nullptr, stream);
}

norm_status norm_layernorm_bwd_noalloc(void* dx, float* dweight, float* dbias, const void* dy,
                                       const void* x, const float* mean, const float* rstd,
                                       const void* weight, int64_t rows, int64_t hidden,
                                       float eps, hipStream_t stream) {
    BwdCall c{dx,     hidden,  dy,      hidden, x,       hidden,       mean,
              rstd,   nullptr, hidden,  weight, nullptr, kScratchBytes, dweight,
              dbias,  rows,    hidden,  eps};
    c.use_scratch = true;
    return run_bwd(NORM_OP_LAYERNORM_BWD, c, nullptr, stream);
}

norm_status norm_rmsnorm_bwd_ex(void* dx, int64_t ld_dx, float* dweight, const void* dy,
                                int64_t ld_dy, const void* x, int64_t ld_x, const void* weight,
                                void* workspace, size_t workspace_bytes, int64_t rows,
                                int64_t hidden, float eps, const norm_launch_cfg* cfg,
                                hipStream_t stream) {
    const BwdCall c{dx,      ld_dx,   dy,      ld_dy,  x,         ld_x,  nullptr,
                    nullptr, nullptr, hidden,  weight, workspace, workspace_bytes,
                    dweight, nullptr, rows,    hidden, eps};
    return run_bwd(NORM_OP_RMSNORM_BWD, c, cfg, stream);
}

norm_status norm_rmsnorm_bwd_cfg(void* dx, float* dweight, const void* dy, const void* x,
                                 const void* weight, void* workspace, size_t workspace_bytes,
                                 int64_t rows, int64_t hidden, float eps,
                                 const norm_launch_cfg* cfg, hipStream_t stream) {
    return norm_rmsnorm_bwd_ex(dx, hidden, dweight, dy, hidden, x, hidden, weight, workspace,
                               workspace_bytes, rows, hidden, eps, cfg, stream);
}

norm_status norm_rmsnorm_bwd(void* dx, float* dweight, const void* dy, const void* x,
                             const void* weight, void* workspace, size_t workspace_bytes,
                             int64_t rows, int64_t hidden, float eps, hipStream_t stream) {
    return norm_rmsnorm_bwd_cfg(dx, dweight, dy, x, weight, workspace, workspace_bytes, rows,
                                hidden, eps, nullptr, stream);
}

norm_status norm_fused_add_rmsnorm_bwd_ex(void* ds, int64_t ld_ds, float* dweight,
                                          const void* dout, int64_t ld_dout, const void* dres,
                                          int64_t ld_dres, const void* s, int64_t ld_s,
                                          const void* weight, void* workspace,
                                          size_t workspace_bytes, int64_t rows, int64_t hidden,
                                          float eps, const norm_launch_cfg* cfg,
                                          hipStream_t stream) {
    const BwdCall c{ds,      ld_ds,   dout,   ld_dout, s,         ld_s,  nullptr,
                    nullptr, dres,    ld_dres, weight, workspace, workspace_bytes,
                    dweight, nullptr, rows,    hidden, eps};
    return run_bwd(NORM_OP_FUSED_ADD_RMSNORM_BWD, c, cfg, stream);
}

norm_status norm_fused_add_rmsnorm_bwd_cfg(void* ds, float* dweight, const void* dout,
                                           const void* dres, const void* s, const void* weight,
                                           void* workspace, size_t workspace_bytes, int64_t rows,
                                           int64_t hidden, float eps, const norm_launch_cfg* cfg,
                                           hipStream_t stream) {
    return norm_fused_add_rmsnorm_bwd_ex(ds, hidden, dweight, dout, hidden, dres, hidden, s,
                                         hidden, weight, workspace, workspace_bytes, rows, hidden,
                                         eps, cfg, stream);
}

norm_status norm_fused_add_rmsnorm_bwd(void* ds, float* dweight, const void* dout,
                                       const void* dres, const void* s, const void* weight,
                                       void* workspace, size_t workspace_bytes, int64_t rows,
                                       int64_t hidden, float eps, hipStream_t stream) {
    return norm_fused_add_rmsnorm_bwd_cfg(ds, dweight, dout, dres, s, weight, workspace,
                                          workspace_bytes, rows, hidden, eps, nullptr, stream);
}

// ---- fp32 activations ---------------------------------------------------------------
norm_status norm_fused_add_rmsnorm_f32(float* out, float* residual, const float* x,
                                       const float* weight, int64_t rows, int64_t hidden,
                                       float eps, hipStream_t stream) {
    const FwdCall c{out,    hidden,  residual, hidden, x,      hidden, weight,
                    nullptr, nullptr, nullptr, rows,   hidden, eps};
    return run_fwd_f32(NORM_OP_FUSED_ADD_RMSNORM, c, stream);
}

norm_status norm_rmsnorm_fwd_f32(float* out, const float* x, const float* weight, int64_t rows,
                                 int64_t hidden, float eps, hipStream_t stream) {
    const FwdCall c{out,    hidden,  nullptr, hidden, x,      hidden, weight,
                    nullptr, nullptr, nullptr, rows,  hidden, eps};
    return run_fwd_f32(NORM_OP_RMSNORM_FWD, c, stream);
}

norm_status norm_layernorm_fwd_f32(float* y, float* mean, float* rstd, const float* x,
                                   const float* weight, const float* bias, int64_t rows,
                                   int64_t hidden, float eps, hipStream_t stream) {
    const FwdCall c{y, hidden, nullptr, hidden, x, hidden, weight, bias, mean, rstd, rows,
                    hidden, eps};
    return run_fwd_f32(NORM_OP_LAYERNORM_FWD, c, stream);
}

norm_status norm_layernorm_bwd_f32(float* dx, float* dweight, float* dbias, const float* dy,
                                   const float* x, const float* mean, const float* rstd,
                                   const float* weight, void* workspace, size_t workspace_bytes,
                                   int64_t rows, int64_t hidden, float eps, hipStream_t stream) {
    const BwdCall c{dx,     hidden,  dy,        hidden, x,         hidden, mean,
                    rstd,   nullptr, hidden,    weight, workspace, workspace_bytes,
                    dweight, dbias,  rows,      hidden, eps};
    return run_bwd_f32(NORM_OP_LAYERNORM_BWD, c, stream);
}

norm_status norm_rmsnorm_bwd_f32(float* dx, float* dweight, const float* dy, const float* x,
                                 const float* weight, void* workspace, size_t workspace_bytes,
                                 int64_t rows, int64_t hidden, float eps, hipStream_t stream) {
    const BwdCall c{dx,      hidden,  dy,      hidden, x,         hidden, nullptr,
                    nullptr, nullptr, hidden,  weight, workspace, workspace_bytes,
                    dweight, nullptr, rows,    hidden, eps};
    return run_bwd_f32(NORM_OP_RMSNORM_BWD, c, stream);
}

norm_status norm_fused_add_rmsnorm_bwd_f32(float* ds, float* dweight, const float* dout,
                                           const float* dres, const float* s,
                                           const float* weight, void* workspace,
                                           size_t workspace_bytes, int64_t rows, int64_t hidden,
                                           float eps, hipStream_t stream) {
    const BwdCall c{ds,      hidden,  dout,   hidden, s,         hidden, nullptr,
                    nullptr, dres,    hidden, weight, workspace, workspace_bytes,
                    dweight, nullptr, rows,   hidden, eps};
    return run_bwd_f32(NORM_OP_FUSED_ADD_RMSNORM_BWD, c, stream);
}

size_t norm_bwd_workspace_bytes_f32(norm_op op, int64_t rows, int64_t hidden) {
    if (!is_bwd(op)) return 0;
    return ws_query_f32(op, rows, hidden);
}

// ---- queries ---------------------------------------------------------------------------
size_t norm_layernorm_bwd_workspace_bytes(int64_t rows, int64_t hidden) {
    return ws_query(NORM_OP_LAYERNORM_BWD, rows, hidden, nullptr);
}

size_t norm_layernorm_bwd_workspace_bytes_cfg(int64_t rows, int64_t hidden,
                                              const norm_launch_cfg* cfg) {
    return ws_query(NORM_OP_LAYERNORM_BWD, rows, hidden, cfg);
}

// Shared by the two RMSNorm backward ops, whose kernel choice differs where
// the fused op streams rows the plain op stages in LDS: enough for either.
size_t norm_rmsnorm_bwd_workspace_bytes(int64_t rows, int64_t hidden) {
    return std::max(ws_query(NORM_OP_RMSNORM_BWD, rows, hidden, nullptr),
                    ws_query(NORM_OP_FUSED_ADD_RMSNORM_BWD, rows, hidden, nullptr));
}

size_t norm_rmsnorm_bwd_workspace_bytes_cfg(int64_t rows, int64_t hidden,
                                            const norm_launch_cfg* cfg) {
    return std::max(ws_query(NORM_OP_RMSNORM_BWD, rows, hidden, cfg),
                    ws_query(NORM_OP_FUSED_ADD_RMSNORM_BWD, rows, hidden, cfg));
}

norm_status norm_select_config(norm_op op, int64_t rows, int64_t hidden, int32_t cu_count,
                               norm_launch_cfg* cfg) {
    if (!cfg || rows < 0 || (int)op < 0 || (int)op > 5) return NORM_ERROR_INVALID_VALUE;
    return select(op, rows, hidden, cu_count, cfg);
}

int32_t norm_describe_config(norm_op op, int64_t rows, int64_t hidden, int32_t cu_count,
                             char* buf, size_t len) {
    static const char* const kNames[] = {"fused_add_rmsnorm", "rmsnorm_fwd",  "layernorm_fwd",
                                         "layernorm_bwd",     "rmsnorm_bwd", "fused_add_rmsnorm_bwd"};
    norm_launch_cfg c;
    if (norm_select_config(op, rows, hidden, cu_count, &c) != NORM_SUCCESS) return -1;
    const bool dyn = c.vector_elems != 0;
    const int w = dyn ? c.vector_elems : 8;
    int vecs = (int)(hidden / (w * c.threads_per_row));
    int depth = 0;
    const WideBwdEntry* wide = dyn && is_bwd(op) ? find_wide(op, hidden, c.threads_per_row, w)
                                                  : nullptr;
    const bool streamed = dyn && (is_bwd(op) ? !wide && stream_bwd_ok(op, hidden, w)
                                             : stream_fwd_ok(op, hidden, w));
    if (streamed) {
        vecs = !is_bwd(op) ? 0 : stream_bwd_xch(hidden) ? kXchVecsBf16 : kStreamTileVecs;
        depth = !is_bwd(op)                          ? 0
                : stream_bwd_xch(hidden)             ? kXchDepthBf16
                : op == NORM_OP_FUSED_ADD_RMSNORM_BWD ? 2
                                                     : 3;
    } else if (wide) {
        vecs = wide->vecs;
        depth = 1;
    } else if (dyn && is_bwd(op)) {
        const DynBwdEntry* e = find_dyn(dyn_bwd_table(op), hidden, w, c.threads_per_row);
        vecs = e->vecs;
        depth = e->depth;
    } else if (dyn) {
        vecs = find_dyn(dyn_fwd_table(op), hidden, w, c.threads_per_row,
                        c.rows_per_block / dyn_rows_per_block(c.threads_per_row))
                   ->vecs;
    } else if (is_bwd(op)) {
        depth = find_bwd(op, hidden, c.threads_per_row)->depth;
    }
    char tmp[640];
    int n;
    if (is_bwd(op)) {
        const int64_t slabs = c.grid;
        const int64_t padded = dyn ? dyn_padded_hidden(hidden) : hidden;
        char grid_text[64];
        if (streamed)
            std::snprintf(grid_text, sizeof grid_text, "%d row walkers x %d column tiles = %lld",
                          c.grid, stream_tiles(hidden),
                          (long long)c.grid * stream_tiles(hidden));
        else
            std::snprintf(grid_text, sizeof grid_text, "%d", c.grid);
        char kern[256];
        if (streamed && stream_bwd_xch(hidden))
            std::snprintf(kern, sizeof kern,
                          "stream_zero_kernel (the exchange area), then "
                          "stream_bwd_tile_kernel<%d,%s,%d,exchange> over %d column tiles of %d "
                          "exchanging partial row sums",
                          vecs, op == NORM_OP_LAYERNORM_BWD ? "layernorm" : "rmsnorm,dres?",
                          depth, stream_tiles(hidden), kXchTileColsBf16);
        else if (streamed)
            std::snprintf(kern, sizeof kern,
                          "stream_bwd_stats_kernel<%s> (1024 lanes a row), then "
                          "stream_bwd_tile_kernel<%d,%s,%d> over %d column tiles of %d",
                          op == NORM_OP_LAYERNORM_BWD ? "layernorm" : "rmsnorm", vecs,
                          op == NORM_OP_LAYERNORM_BWD ? "layernorm" : "rmsnorm,dres?", depth,
                          stream_tiles(hidden), kStreamTileCols);
        else if (wide)
            std::snprintf(kern, sizeof kern, "norm_bwd_wide_kernel<%d,%s> (x, dy staged in LDS)",
                          vecs, op == NORM_OP_LAYERNORM_BWD ? "layernorm" : "rmsnorm,dres?");
        else if (dyn)
            std::snprintf(kern, sizeof kern, "norm_bwd_dyn_rows_kernel<%d,%d,%d,%d,%s>", w,
                          c.threads_per_row, vecs, depth,
                          op == NORM_OP_LAYERNORM_BWD ? "layernorm" : "rmsnorm,dres?");
        else
            std::snprintf(kern, sizeof kern, "%s_bwd_rows_kernel<%lld,%d,%d%s>",
                          op == NORM_OP_LAYERNORM_BWD ? "layernorm" : "rmsnorm",
                          (long long)hidden, c.threads_per_row, depth,
                          op == NORM_OP_LAYERNORM_BWD ? "" : ",dres?");
        // a streamed row spans its tiles: the text gives a tile's workgroup
        const bool xch = streamed && stream_bwd_xch(hidden);
        n = std::snprintf(tmp, sizeof tmp,
                          "%s rows=%lld hidden=%lld: %s (%d lanes per %s, %d rows per "
                          "workgroup, %d %d-byte accesses per lane, ring of %d rows) on a "
                          "persistent grid of %s workgroups, then norm_bwd_colreduce_kernel "
                          "(%lld workgroups of %d) over %lld slabs; workspace %zu bytes",
                          kNames[op], (long long)rows, (long long)hidden, kern,
                          xch ? kXchLanesBf16 : c.threads_per_row,
                          streamed ? "workgroup" : "row", c.rows_per_block, vecs, 2 * w,
                          xch ? 2 * depth : depth, grid_text,
                          (long long)(bwd_outs(op) * padded / colreduce_cols(slabs)),
                          kColReduceThreads,
                          (long long)slabs,
                          streamed ? stream_ws_bytes(op, hidden, rows > 0 ? slabs : 0, rows,
                                                     stream_tiles(hidden))
                          : dyn    ? dyn_ws_bytes(op, hidden, rows > 0 ? slabs : 0)
                                   : static_ws_bytes(op, hidden, rows > 0 ? c.grid : 0));
    } else {
        const char* kern = op == NORM_OP_FUSED_ADD_RMSNORM ? "fused_add_rmsnorm"
                           : op == NORM_OP_RMSNORM_FWD     ? "rmsnorm_fwd"
                                                           : "layernorm_fwd";
        char inst[96];
        const FwdEntry* ring =
            c.grid > 0 ? ring_entry(op, hidden, c.threads_per_row, rows, c.grid) : nullptr;
        const int sop = op == NORM_OP_FUSED_ADD_RMSNORM ? kSplitFused
                        : op == NORM_OP_LAYERNORM_FWD   ? kSplitLn
                                                        : kSplitRms;
        if (streamed && stage_fwd_holds(sop, false, hidden)) {
            std::snprintf(inst, sizeof inst,
                          "stage_fwd_kernel<%s> (registers and LDS, the row read once)", kern);
        } else if (streamed) {
            std::snprintf(inst, sizeof inst, "stream_fwd_kernel<%s> (two passes over the row)",
                          kern);
        } else if (dyn) {
            int cu = cu_count;
            if (cu <= 0 && current_cu_count(&cu) != NORM_SUCCESS) return -1;
            const bool late =
                late_weights_dyn(ceil_div(rows, c.rows_per_block), c.threads_per_row, cu);
            std::snprintf(inst, sizeof inst, "%s%s<%d,%d,%d,%d>", kern,
                          late ? "_dyn_lw_kernel" : "_dyn_kernel", w, c.threads_per_row, vecs,
                          c.rows_per_block / dyn_rows_per_block(c.threads_per_row));
        }
        else if (ring)
            std::snprintf(inst, sizeof inst, "%s_ring_kernel<%lld,%d,%d>", kern,
                          (long long)hidden, c.threads_per_row, ring->depth);
        else {
            int cu = cu_count;
            if (cu <= 0 && late_listed(op, hidden, c.threads_per_row, c.rows_per_block) &&
                current_cu_count(&cu) != NORM_SUCCESS)
                return -1;
            const bool late =
                late_weights(op, rows, hidden, c.threads_per_row, c.rows_per_block, cu);
            std::snprintf(inst, sizeof inst, "%s%s<%lld,%d,%d>", kern,
                          late ? "_lw_kernel" : "_kernel", (long long)hidden, c.threads_per_row,
                          c.rows_per_block);
        }
        const int block = dyn ? dyn_block_size(c.threads_per_row)
                              : c.threads_per_row * c.rows_per_block;
        if (streamed && stage_fwd_holds(sop, false, hidden)) {
            const StageShape st = stage_fwd_shape(sop, false);
            n = std::snprintf(tmp, sizeof tmp,
                              "%s rows=%lld hidden=%lld: %s (%d lanes per row, 1 rows per "
                              "workgroup of %d, %lld 16-byte accesses per lane: up to %d in "
                              "registers, up to %d in LDS), grid %lld",
                              kNames[op], (long long)rows, (long long)hidden, inst,
                              c.threads_per_row, c.threads_per_row,
                              (long long)ceil_div(hidden / 8, c.threads_per_row), st.u, st.l,
                              (long long)std::min<int64_t>(rows, kStageGridRows));
        } else if (streamed) {
            const StreamFwdShape sh = stream_fwd_shape(false, sop == kSplitLn, sop == kSplitRms,
                                                       hidden);
            n = std::snprintf(tmp, sizeof tmp,
                              "%s rows=%lld hidden=%lld: %s (%d lanes per row, 1 rows per "
                              "workgroup of %d, %lld 16-byte accesses per lane, the first %d "
                              "kept in registers), grid %lld",
                              kNames[op], (long long)rows, (long long)hidden, inst,
                              c.threads_per_row, c.threads_per_row,
                              (long long)ceil_div(hidden / 8, c.threads_per_row), sh.unroll,
                              (long long)std::min<int64_t>(rows, kStreamMaxGrid));
        }
        else if (ring)
            n = std::snprintf(tmp, sizeof tmp,
                              "%s rows=%lld hidden=%lld: %s (%d lanes per row, %d 16-byte "
                              "accesses per lane, ring of %d rows) on a persistent grid of %d "
                              "workgroups",
                              kNames[op], (long long)rows, (long long)hidden, inst,
                              c.threads_per_row, vecs, ring->depth, c.grid);
        else
            n = std::snprintf(tmp, sizeof tmp,
                              "%s rows=%lld hidden=%lld: %s (%d lanes per row, %d rows per "
                              "workgroup of %d, %d %d-byte accesses per lane), grid %lld",
                              kNames[op], (long long)rows, (long long)hidden, inst,
                              c.threads_per_row, c.rows_per_block, block, vecs, 2 * w,
                              (long long)ceil_div(rows, c.rows_per_block));
    }
    if (n < 0) return -1;
    if (buf && len > 0) {
        const size_t k = (size_t)n < len - 1 ? (size_t)n : len - 1;
        std::memcpy(buf, tmp, k);
        buf[k] = '\0';
    }
    return n;
}

int32_t norm_list_configs(norm_op op, int64_t hidden, norm_launch_cfg* out, int32_t capacity) {
    int32_t n = 0;
    if ((int)op < 0 || (int)op > 5 || hidden < 1 || hidden > kMaxHidden) return 0;
    auto put = [&](norm_launch_cfg c) {
        if (out && n < capacity) out[n] = c;
        ++n;
    };
    if (is_bwd(op)) {
        for (const BwdEntry& e : bwd_table(op))
            if (e.hidden == hidden) put(norm_launch_cfg{e.lanes, 1, 0, 0});
    } else {
        int ring_lanes_seen = 0;  // bit k: a ring shape of 64 << k lanes listed already
        for (const FwdEntry& e : fwd_table(op)) {
            if (e.hidden != hidden) continue;
            if (e.depth > 0) {  // one shape per lane count (the depth follows the walk)
                const int bit = 1 << __builtin_ctz((unsigned)(e.lanes / 64));
                if (ring_lanes_seen & bit) continue;
                ring_lanes_seen |= bit;
            }
            put(norm_launch_cfg{e.lanes, e.rows_per_block, e.depth > 0 ? kFwdRingGrid : 0, 0});
        }
    }
    // run-time-hidden shapes at the widest access a contiguous row allows
    const int w = shape_width(hidden, {});
    for (int lanes = 8; lanes <= 1024; lanes *= 2) {
        if (lanes > 8 && lanes / 2 >= hidden / w) break;
        const int r = dyn_rows_per_block(lanes);
        if (is_bwd(op)) {
            if (find_dyn(dyn_bwd_table(op), hidden, w, lanes) || find_wide(op, hidden, lanes, w))
                put(norm_launch_cfg{lanes, r, 0, w});
            continue;
        }
        for (int k : {1, 2, 4})
            if (find_dyn(dyn_fwd_table(op), hidden, w, lanes, k))
                put(norm_launch_cfg{lanes, r * k, 0, w});
    }
    // streamed rows (wider than the on-chip kernels hold)
    if (is_bwd(op) ? stream_bwd_ok(op, hidden, w) : stream_fwd_ok(op, hidden, w))
        put(is_bwd(op) ? norm_launch_cfg{kStreamTileLanes, 1, 0, 8}
                       : norm_launch_cfg{kStreamFwdLanes, 1, 0, 8});
    return n;
}

}  // extern "C"
