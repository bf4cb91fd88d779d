// C ABI of the row-normalization library: argument validation, launch-shape
// choice and dispatch to the compiled kernel shapes.  Declared in norm.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "launch.hpp"
#include "norm.h"

using namespace rownorm;

namespace {

bool hidden_supported(int64_t hidden) {
    for (int h : kHiddenSizes)
        if (h == hidden) return true;
    return false;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Span {
    const void* p;
    uint64_t bytes;
};

// True if the spans share a byte, unless they are the same span and that
// exact alias is allowed.
bool bad_overlap(Span a, Span b, bool exact_alias_ok) {
    if (a.bytes == 0 || b.bytes == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    const uintptr_t a1 = a0 + a.bytes, b1 = b0 + b.bytes;
    if (a1 <= b0 || b1 <= a0) return false;
    return !(exact_alias_ok && a0 == b0 && a.bytes == b.bytes);
}

bool eps_ok(float eps) { return std::isfinite(eps) && eps >= 0.0f; }

// Sanity bound on rows; each launch also checks that its grid and total
// work-item count fit HIP's 32-bit launch limits.
constexpr int64_t kMaxRows = (int64_t(1) << 31) - 1;

bool launch_fits(int64_t rows, int lanes, int rpb) {
    const int64_t groups = (rows + rpb - 1) / rpb;
    return groups <= INT32_MAX && groups * lanes * rpb <= (int64_t)UINT32_MAX;
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

// ---- tables ----------------------------------------------------------------
const std::vector<FwdEntry>& fwd_table(norm_op op) {
    switch (op) {
        case NORM_OP_FUSED_ADD_RMSNORM: return fused_add_rmsnorm_table();
        case NORM_OP_RMSNORM_FWD: return rmsnorm_fwd_table();
        default: return layernorm_fwd_table();
    }
}

const FwdEntry* find_fwd(norm_op op, int64_t hidden, int lanes, int rpb) {
    for (const FwdEntry& e : fwd_table(op))
        if (e.hidden == hidden && e.lanes == lanes && e.rows_per_block == rpb) return &e;
    return nullptr;
}

bool is_bwd(norm_op op) {
    return op == NORM_OP_LAYERNORM_BWD || op == NORM_OP_RMSNORM_BWD ||
           op == NORM_OP_FUSED_ADD_RMSNORM_BWD;
}

const std::vector<BwdEntry>& bwd_table(norm_op op) {
    return op == NORM_OP_LAYERNORM_BWD ? layernorm_bwd_table() : rmsnorm_bwd_table();
}

// partial-sum slabs per workgroup: dweight and dbias for LayerNorm, dweight for RMSNorm
int bwd_outs(norm_op op) { return op == NORM_OP_LAYERNORM_BWD ? 2 : 1; }

const BwdEntry* find_bwd(norm_op op, int64_t hidden, int lanes) {
    for (const BwdEntry& e : bwd_table(op))
        if (e.hidden == hidden && e.lanes == lanes) return &e;
    return nullptr;
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
norm_launch_cfg choose_fwd(norm_op op, int64_t rows, int64_t hidden, int cu) {
    const int64_t target_waves = 4 * (int64_t)cu;
    auto valid = [&](int l) {
        for (const FwdEntry& e : fwd_table(op))
            if (e.hidden == hidden && e.lanes == l) return true;
        return false;
    };
    const int max_vecs = (op != NORM_OP_LAYERNORM_FWD && rows >= 16 * (int64_t)cu) ? 4 : 8;
    int lanes = 64;
    while (lanes < 1024 && (hidden / (8 * lanes) > max_vecs || !valid(lanes))) lanes *= 2;
    while (lanes < 1024 && rows * (lanes / 64) < target_waves && valid(lanes * 2)) lanes *= 2;
    int rpb = lanes == 64 ? 4 : (lanes == 128 ? 2 : 1);
    while (rpb > 1 && !find_fwd(op, hidden, lanes, rpb)) rpb /= 2;
    return norm_launch_cfg{lanes, rpb, 0};
}

// LayerNorm backward: one persistent workgroup per compute unit of the
// largest part (256 on MI355X) made the best trade-off between rows in flight
// and partial-sum slabs to reduce; the grid is a constant, not a device query,
// so the workspace size is pure host arithmetic.
int32_t default_bwd_grid(int64_t rows) {
    constexpr int64_t kSlabs = 256;
    return (int32_t)(rows < kSlabs ? (rows > 0 ? rows : 1) : kSlabs);
}

norm_launch_cfg choose_bwd(norm_op op, int64_t rows, int64_t hidden) {
    // one 16-byte vector of x and of dy per lane when compiled (512 lanes at
    // hidden 4096, 1024 at 8192), else the shape with the fewest vectors per lane
    int best = 0;
    for (const BwdEntry& e : bwd_table(op)) {
        if (e.hidden != hidden) continue;
        if (best == 0 || e.lanes > best) best = e.lanes;
    }
    return norm_launch_cfg{best, 1, default_bwd_grid(rows)};
}

int bwd_depth_of(norm_op op, int64_t hidden, int lanes) {
    const BwdEntry* e = find_bwd(op, hidden, lanes);
    return e ? e->depth : 0;
}

size_t bwd_workspace_bytes(norm_op op, int64_t hidden, int32_t grid) {
    return (size_t)grid * (size_t)bwd_outs(op) * (size_t)hidden * sizeof(float);
}

norm_status from_hip(hipError_t e) { return e == hipSuccess ? NORM_SUCCESS : NORM_ERROR_LAUNCH; }

// ---- forward entry -------------------------------------------------------------
norm_status run_fwd(norm_op op, const FwdArgs& a, int64_t hidden, const norm_launch_cfg* cfg,
                    hipStream_t stream) {
    if (a.rows < 0 || a.rows > kMaxRows || !eps_ok(a.eps)) return NORM_ERROR_INVALID_VALUE;
    if (cfg && (cfg->grid != 0 || cfg->threads_per_row <= 0 || cfg->rows_per_block <= 0))
        return NORM_ERROR_INVALID_VALUE;
    if (a.rows == 0) return NORM_SUCCESS;
    if (!hidden_supported(hidden)) return NORM_ERROR_UNSUPPORTED_HIDDEN;

    const bool fused = op == NORM_OP_FUSED_ADD_RMSNORM;
    const bool ln = op == NORM_OP_LAYERNORM_FWD;
    if (!a.out || !a.x || !a.weight || (fused && !a.residual) || (ln && !a.bias))
        return NORM_ERROR_INVALID_VALUE;
    if (ln && ((a.mean == nullptr) != (a.rstd == nullptr))) return NORM_ERROR_INVALID_VALUE;
    if (!aligned(a.out, 16) || !aligned(a.x, 16) || !aligned(a.weight, 16) ||
        (fused && !aligned(a.residual, 16)) || (ln && !aligned(a.bias, 16)) ||
        (ln && a.mean && (!aligned(a.mean, 4) || !aligned(a.rstd, 4))))
        return NORM_ERROR_MISALIGNED;

    const uint64_t mat = (uint64_t)a.rows * (uint64_t)hidden * 2;
    const uint64_t vec = (uint64_t)hidden * 2;
    const uint64_t stat = (uint64_t)a.rows * 4;
    const Span out{a.out, mat}, x{a.x, mat}, w{a.weight, vec};
    const Span res{fused ? a.residual : nullptr, fused ? mat : 0};
    const Span b{ln ? a.bias : nullptr, ln ? vec : 0};
    const Span mean{ln ? a.mean : nullptr, (ln && a.mean) ? stat : 0};
    const Span rstd{ln ? a.rstd : nullptr, (ln && a.rstd) ? stat : 0};
    // outputs must not overlap anything, except out == x exactly
    if (bad_overlap(out, x, true) || bad_overlap(out, w, false) || bad_overlap(out, res, false) ||
        bad_overlap(out, b, false) || bad_overlap(out, mean, false) ||
        bad_overlap(out, rstd, false) || bad_overlap(res, x, false) ||
        bad_overlap(res, w, false) || bad_overlap(res, b, false) || bad_overlap(mean, x, false) ||
        bad_overlap(mean, w, false) || bad_overlap(mean, b, false) ||
        bad_overlap(mean, rstd, false) || bad_overlap(rstd, x, false) ||
        bad_overlap(rstd, w, false) || bad_overlap(rstd, b, false))
        return NORM_ERROR_INVALID_VALUE;

    norm_launch_cfg c;
    if (cfg) {
        c = *cfg;
    } else {
        int cu = 0;
        const norm_status st = current_cu_count(&cu);
        if (st != NORM_SUCCESS) return st;
        c = choose_fwd(op, a.rows, hidden, cu);
    }
    const FwdEntry* e = find_fwd(op, hidden, c.threads_per_row, c.rows_per_block);
    if (!e || !launch_fits(a.rows, c.threads_per_row, c.rows_per_block))
        return NORM_ERROR_INVALID_VALUE;
    return from_hip(e->launch(a, stream));
}

norm_status run_bwd(norm_op op, BwdArgs a, int64_t hidden, float eps, size_t workspace_bytes,
                    const norm_launch_cfg* cfg, hipStream_t stream) {
    const bool ln = op == NORM_OP_LAYERNORM_BWD;
    if (a.rows < 0 || a.rows > kMaxRows || !eps_ok(eps)) return NORM_ERROR_INVALID_VALUE;
    if (cfg && (cfg->threads_per_row <= 0 || cfg->rows_per_block != 1 || cfg->grid < 0))
        return NORM_ERROR_INVALID_VALUE;
    if (!hidden_supported(hidden)) return NORM_ERROR_UNSUPPORTED_HIDDEN;
    if (cfg && cfg->grid > max_bwd_grid(hidden)) return NORM_ERROR_INVALID_VALUE;
    const bool any = a.rows > 0;
    if (!a.dweight || (ln && !a.dbias) || !a.workspace) return NORM_ERROR_INVALID_VALUE;
    if (any && (!a.dx || !a.dy || !a.x || !a.weight || (ln && (!a.mean || !a.rstd))))
        return NORM_ERROR_INVALID_VALUE;
    if (!aligned(a.dweight, 4) || (ln && !aligned(a.dbias, 4)) || !aligned(a.workspace, 16))
        return NORM_ERROR_MISALIGNED;
    if (any && (!aligned(a.dx, 16) || !aligned(a.dy, 16) || !aligned(a.x, 16) ||
                !aligned(a.weight, 16) || (a.dres && !aligned(a.dres, 16)) ||
                (ln && (!aligned(a.mean, 4) || !aligned(a.rstd, 4)))))
        return NORM_ERROR_MISALIGNED;

    norm_launch_cfg c = cfg ? *cfg : choose_bwd(op, a.rows, hidden);
    if (c.grid == 0) c.grid = default_bwd_grid(a.rows);
    const BwdEntry* e = find_bwd(op, hidden, c.threads_per_row);
    if (!e) return NORM_ERROR_INVALID_VALUE;
    a.grid = c.grid;
    a.eps = eps;
    const size_t ws_need = bwd_workspace_bytes(op, hidden, any ? c.grid : 0);

    const uint64_t mat = any ? (uint64_t)a.rows * (uint64_t)hidden * 2 : 0;
    const uint64_t vec = any ? (uint64_t)hidden * 2 : 0;
    const uint64_t stat = ln ? (uint64_t)a.rows * 4 : 0;
    const uint64_t col = (uint64_t)hidden * 4;
    const Span dx{a.dx, mat}, dy{a.dy, mat}, x{a.x, mat}, mean{a.mean, stat},
        rstd{a.rstd, stat}, dres{a.dres, a.dres ? mat : 0}, w{a.weight, vec},
        dw{a.dweight, col}, db{a.dbias, ln ? col : 0}, ws{a.workspace, ws_need};
    // outputs overlap no input, except dx == dy (or dx == dres) exactly
    const Span ins[] = {dy, x, mean, rstd, dres, w};
    for (const Span& in : ins) {
        if (bad_overlap(dx, in, in.p == a.dy || (a.dres && in.p == a.dres)))
            return NORM_ERROR_INVALID_VALUE;
        if (bad_overlap(dw, in, false) || bad_overlap(db, in, false) || bad_overlap(ws, in, false))
            return NORM_ERROR_INVALID_VALUE;
    }
    if (bad_overlap(dx, dw, false) || bad_overlap(dx, db, false) || bad_overlap(dx, ws, false) ||
        bad_overlap(dw, db, false) || bad_overlap(dw, ws, false) || bad_overlap(db, ws, false))
        return NORM_ERROR_INVALID_VALUE;
    if (workspace_bytes < ws_need) return NORM_ERROR_WORKSPACE;
    return from_hip(e->launch(a, stream));
}

}  // namespace

extern "C" {

const char* norm_status_string(norm_status status) {
    switch (status) {
        case NORM_SUCCESS: return "NORM_SUCCESS";
        case NORM_ERROR_INVALID_VALUE: return "NORM_ERROR_INVALID_VALUE: invalid argument";
        case NORM_ERROR_UNSUPPORTED_HIDDEN:
            return "NORM_ERROR_UNSUPPORTED_HIDDEN: hidden must be one of 1024, 2048, 4096, 8192, "
                   "12288, 16384";
        case NORM_ERROR_MISALIGNED:
            return "NORM_ERROR_MISALIGNED: bf16 pointers need 16-byte, fp32 pointers 4-byte "
                   "alignment";
        case NORM_ERROR_WORKSPACE: return "NORM_ERROR_WORKSPACE: workspace too small";
        case NORM_ERROR_LAUNCH: return "NORM_ERROR_LAUNCH: HIP reported a launch error";
        case NORM_ERROR_DEVICE: return "NORM_ERROR_DEVICE: could not query the current device";
    }
    return "unknown norm_status";
}

norm_status norm_fused_add_rmsnorm_cfg(void* out, void* residual, const void* x,
                                       const void* weight, int64_t rows, int64_t hidden,
                                       float eps, const norm_launch_cfg* cfg,
                                       hipStream_t stream) {
    FwdArgs a{out, residual, x, weight, nullptr, nullptr, nullptr, rows, eps};
    return run_fwd(NORM_OP_FUSED_ADD_RMSNORM, a, hidden, cfg, stream);
}

norm_status norm_fused_add_rmsnorm(void* out, void* residual, const void* x, const void* weight,
                                   int64_t rows, int64_t hidden, float eps, hipStream_t stream) {
    return norm_fused_add_rmsnorm_cfg(out, residual, x, weight, rows, hidden, eps, nullptr, stream);
}

norm_status norm_rmsnorm_fwd_cfg(void* out, const void* x, const void* weight, int64_t rows,
                                 int64_t hidden, float eps, const norm_launch_cfg* cfg,
                                 hipStream_t stream) {
    FwdArgs a{out, nullptr, x, weight, nullptr, nullptr, nullptr, rows, eps};
    return run_fwd(NORM_OP_RMSNORM_FWD, a, hidden, cfg, stream);
}

norm_status norm_rmsnorm_fwd(void* out, const void* x, const void* weight, int64_t rows,
                             int64_t hidden, float eps, hipStream_t stream) {
    return norm_rmsnorm_fwd_cfg(out, x, weight, rows, hidden, eps, nullptr, stream);
}

norm_status norm_layernorm_fwd_cfg(void* y, float* mean, float* rstd, const void* x,
                                   const void* weight, const void* bias, int64_t rows,
                                   int64_t hidden, float eps, const norm_launch_cfg* cfg,
                                   hipStream_t stream) {
    FwdArgs a{y, nullptr, x, weight, bias, mean, rstd, rows, eps};
    return run_fwd(NORM_OP_LAYERNORM_FWD, a, hidden, cfg, stream);
}

norm_status norm_layernorm_fwd(void* y, float* mean, float* rstd, const void* x,
                               const void* weight, const void* bias, int64_t rows, int64_t hidden,
                               float eps, hipStream_t stream) {
    return norm_layernorm_fwd_cfg(y, mean, rstd, x, weight, bias, rows, hidden, eps, nullptr,
                                  stream);
}

norm_status norm_layernorm_bwd_cfg(void* dx, float* dweight, float* dbias, const void* dy,
                                   const void* x, const float* mean, const float* rstd,
                                   const void* weight, void* workspace, size_t workspace_bytes,
                                   int64_t rows, int64_t hidden, float eps,
                                   const norm_launch_cfg* cfg, hipStream_t stream) {
    BwdArgs a{dx, dy, x, mean, rstd, nullptr, weight, (float*)workspace, dweight, dbias, rows, 0,
              0.0f};
    return run_bwd(NORM_OP_LAYERNORM_BWD, a, hidden, eps, workspace_bytes, cfg, stream);
}

norm_status norm_layernorm_bwd(void* dx, float* dweight, float* dbias, const void* dy,
                               const void* x, const float* mean, const float* rstd,
                               const void* weight, void* workspace, size_t workspace_bytes,
                               int64_t rows, int64_t hidden, float eps, hipStream_t stream) {
    return norm_layernorm_bwd_cfg(dx, dweight, dbias, dy, x, mean, rstd, weight, workspace,
                                  workspace_bytes, rows, hidden, eps, nullptr, stream);
}

norm_status norm_rmsnorm_bwd_cfg(void* dx, float* dweight, const void* dy, const void* x,
                                 const void* weight, void* workspace, size_t workspace_bytes,
                                 int64_t rows, int64_t hidden, float eps,
                                 const norm_launch_cfg* cfg, hipStream_t stream) {
    BwdArgs a{dx, dy, x, nullptr, nullptr, nullptr, weight, (float*)workspace, dweight, nullptr,
              rows, 0, 0.0f};
    return run_bwd(NORM_OP_RMSNORM_BWD, a, hidden, eps, workspace_bytes, cfg, stream);
}

norm_status norm_rmsnorm_bwd(void* dx, float* dweight, const void* dy, const void* x,
                             const void* weight, void* workspace, size_t workspace_bytes,
                             int64_t rows, int64_t hidden, float eps, hipStream_t stream) {
    return norm_rmsnorm_bwd_cfg(dx, dweight, dy, x, weight, workspace, workspace_bytes, rows,
                                hidden, eps, nullptr, stream);
}

norm_status norm_fused_add_rmsnorm_bwd_cfg(void* ds, float* dweight, const void* dout,
                                           const void* dres, const void* s, const void* weight,
                                           void* workspace, size_t workspace_bytes, int64_t rows,
                                           int64_t hidden, float eps, const norm_launch_cfg* cfg,
                                           hipStream_t stream) {
    BwdArgs a{ds, dout, s, nullptr, nullptr, dres, weight, (float*)workspace, dweight, nullptr,
              rows, 0, 0.0f};
    return run_bwd(NORM_OP_FUSED_ADD_RMSNORM_BWD, a, hidden, eps, workspace_bytes, cfg, stream);
}

norm_status norm_fused_add_rmsnorm_bwd(void* ds, float* dweight, const void* dout,
                                       const void* dres, const void* s, const void* weight,
                                       void* workspace, size_t workspace_bytes, int64_t rows,
                                       int64_t hidden, float eps, hipStream_t stream) {
    return norm_fused_add_rmsnorm_bwd_cfg(ds, dweight, dout, dres, s, weight, workspace,
                                          workspace_bytes, rows, hidden, eps, nullptr, stream);
}

static size_t ws_bytes_for(norm_op op, int64_t rows, int64_t hidden, const norm_launch_cfg* cfg) {
    if (rows <= 0 || !hidden_supported(hidden)) return 0;
    const int32_t g = (cfg && cfg->grid > 0) ? cfg->grid : default_bwd_grid(rows);
    return bwd_workspace_bytes(op, hidden, g);
}

size_t norm_layernorm_bwd_workspace_bytes(int64_t rows, int64_t hidden) {
    return ws_bytes_for(NORM_OP_LAYERNORM_BWD, rows, hidden, nullptr);
}

size_t norm_layernorm_bwd_workspace_bytes_cfg(int64_t rows, int64_t hidden,
                                              const norm_launch_cfg* cfg) {
    return ws_bytes_for(NORM_OP_LAYERNORM_BWD, rows, hidden, cfg);
}

size_t norm_rmsnorm_bwd_workspace_bytes(int64_t rows, int64_t hidden) {
    return ws_bytes_for(NORM_OP_RMSNORM_BWD, rows, hidden, nullptr);
}

size_t norm_rmsnorm_bwd_workspace_bytes_cfg(int64_t rows, int64_t hidden,
                                            const norm_launch_cfg* cfg) {
    return ws_bytes_for(NORM_OP_RMSNORM_BWD, rows, hidden, cfg);
}

norm_status norm_select_config(norm_op op, int64_t rows, int64_t hidden, int32_t cu_count,
                               norm_launch_cfg* cfg) {
    if (!cfg || rows < 0 || (int)op < 0 || (int)op > 5) return NORM_ERROR_INVALID_VALUE;
    if (!hidden_supported(hidden)) return NORM_ERROR_UNSUPPORTED_HIDDEN;
    if (is_bwd(op)) {
        *cfg = choose_bwd(op, rows, hidden);
        return NORM_SUCCESS;
    }
    int cu = cu_count;
    if (cu <= 0) {
        const norm_status st = current_cu_count(&cu);
        if (st != NORM_SUCCESS) return st;
    }
    *cfg = choose_fwd(op, rows, hidden, cu);
    return NORM_SUCCESS;
}

int32_t norm_describe_config(norm_op op, int64_t rows, int64_t hidden, int32_t cu_count,
                             char* buf, size_t len) {
    static const char* const kNames[] = {"fused_add_rmsnorm", "rmsnorm_fwd",  "layernorm_fwd",
                                         "layernorm_bwd",     "rmsnorm_bwd", "fused_add_rmsnorm_bwd"};
    norm_launch_cfg c;
    if (norm_select_config(op, rows, hidden, cu_count, &c) != NORM_SUCCESS) return -1;
    const int vecs = (int)(hidden / (8 * c.threads_per_row));
    char tmp[512];
    int n;
    if (is_bwd(op)) {
        const int depth = bwd_depth_of(op, hidden, c.threads_per_row);
        n = std::snprintf(tmp, sizeof tmp,
                          "%s rows=%lld hidden=%lld: %s_bwd_rows_kernel<%lld,%d,%d%s> "
                          "(%d lanes per row, %d vectors per lane, ring of %d rows) on a "
                          "persistent grid of %d workgroups, then norm_bwd_colreduce_kernel "
                          "(%lld workgroups of %d); workspace %zu bytes",
                          kNames[op], (long long)rows, (long long)hidden,
                          op == NORM_OP_LAYERNORM_BWD ? "layernorm" : "rmsnorm",
                          (long long)hidden, c.threads_per_row, depth,
                          op == NORM_OP_LAYERNORM_BWD ? "" : ",dres?", c.threads_per_row, vecs,
                          depth, c.grid,
                          (long long)(bwd_outs(op) * hidden / kColReduceCols), kColReduceThreads,
                          bwd_workspace_bytes(op, hidden, rows > 0 ? c.grid : 0));
    } else {
        const char* kern = op == NORM_OP_FUSED_ADD_RMSNORM ? "fused_add_rmsnorm_kernel"
                           : op == NORM_OP_RMSNORM_FWD     ? "rmsnorm_fwd_kernel"
                                                           : "layernorm_fwd_kernel";
        n = std::snprintf(tmp, sizeof tmp,
                          "%s rows=%lld hidden=%lld: %s<%lld,%d,%d> (%d lanes per row, %d rows "
                          "per workgroup of %d, %d vectors per lane), grid %lld",
                          kNames[op], (long long)rows, (long long)hidden, kern,
                          (long long)hidden, c.threads_per_row, c.rows_per_block,
                          c.threads_per_row, c.rows_per_block,
                          c.threads_per_row * c.rows_per_block, vecs,
                          (long long)((rows + c.rows_per_block - 1) / c.rows_per_block));
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
    if ((int)op < 0 || (int)op > 5) return 0;
    if (is_bwd(op)) {
        for (const BwdEntry& e : bwd_table(op)) {
            if (e.hidden != hidden) continue;
            if (out && n < capacity) out[n] = norm_launch_cfg{e.lanes, 1, 0};
            ++n;
        }
        return n;
    }
    for (const FwdEntry& e : fwd_table(op)) {
        if (e.hidden != hidden) continue;
        if (out && n < capacity) out[n] = norm_launch_cfg{e.lanes, e.rows_per_block, 0};
        ++n;
    }
    return n;
}

}  // extern "C"
