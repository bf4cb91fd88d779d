/*
 * norm.h -- C ABI of the MI355X (gfx950) inner-persistent row-normalization
 * library (librownorm.so).
 *
 * Every operation normalizes the rows of a row-major [rows, hidden] bf16
 * matrix.  Each row is read from HBM once into registers, reduced there, and
 * written once ("inner persistent": the row stays on-chip between the
 * reduction and the normalize step).  Two kernel families do the work:
 *   - compiled-hidden kernels, where hidden is a template constant ("optimize
 *     inner persistent scheduler for static fusion", author description: the
 *     hidden size of a model is static), for hidden in
 *         {1024, 2048, 4096, 8192, 12288, 16384}
 *     with contiguous rows and 16-byte-aligned bf16 pointers;
 *   - run-time-hidden kernels for everything else (the non-static path of the
 *     same page, reviewer guide, split logic): any hidden >= 1, row strides,
 *     and bf16 pointers aligned to 2 bytes or more.  Rows are read with the
 *     widest access (16, 8, 4 or 2 bytes) that hidden, every row stride and
 *     every bf16 pointer allow.  One workgroup holds the row on chip up to
 *     hidden 65536 forward (LayerNorm 49152) with 16-byte accesses, 8192 *
 *     (access elements) otherwise; backward 32768 with 16-byte accesses
 *     (above 16384 the row is staged in LDS: "TMA inner persistent
 *     scheduler", description summary, the shared-memory persistent
 *     buffer; the fused op's backward up to 28672, wider rows streamed),
 *     16384 with 8-byte accesses, 8192 otherwise.  Wider rows with
 *     16-byte accesses (hidden a multiple of 8, up to 2^20) run on streamed
 *     kernels: forward, one pass for the statistic and one, mostly from the
 *     Infinity Cache, to normalize (the row read twice); backward,
 *     workgroups over 4096-column tiles that exchange each row's partial
 *     sums through the workspace, so the row is read once (up to 262144
 *     columns; wider rows: a row-sums kernel, then 16384-column tiles that
 *     read the row again).  Forward rows that
 *     registers and LDS hold together are read once instead (the fused op
 *     up to 81920, RMSNorm from 69912 up to 114688: the rest of the row
 *     past the registers staged in LDS).  Wider rows with narrower accesses
 *     are unsupported.  The row-split forward entry
 *     points below spread few wide rows over several workgroups instead.
 * The library picks the family; the arithmetic and results (within rounding)
 * are the same.  The `_f32` entry points take fp32 activations, weights and
 * gradients instead (contiguous rows, hidden a multiple of 4 up to 2^20):
 * rows of up to 1024 columns several to a wave, fused and RMSNorm forward
 * rows of 34956 ... 40960 / 69632 columns staged partly in LDS, backward
 * rows of 8196 ... 16384 columns staged in LDS, the streamed kernels
 * everywhere else.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors are DEVICE pointers into memory of the calling thread's current
 *   HIP device.  Matrices are row-major with unit column stride: element
 *   (i, j) of a [rows, hidden] matrix sits at index i * ld + j, where ld (the
 *   leading dimension, in elements, ld >= hidden) is `hidden` for the entry
 *   points without an ld argument and given explicitly to the `_ex` entry
 *   points.  bf16 tensors are passed as void* / const void* holding IEEE bf16
 *   bit patterns and must be 2-byte aligned (16-byte aligned for a
 *   `norm_launch_cfg` that names a compiled-hidden shape); fp32 tensors must
 *   be 4-byte aligned; the backward workspace 16-byte aligned.
 * - Ownership: the caller allocates and frees every buffer (workspace
 *   included).  The library never allocates, frees, or keeps a pointer past
 *   the call.  Its only state is a per-device cache of the compute-unit count.
 * - Execution is asynchronous on `stream` (0 = the null stream).  A
 *   NORM_SUCCESS return means the work was enqueued; faults inside a kernel
 *   surface at the caller's next synchronization.  The library never sets or
 *   switches the current device.
 * - Errors are reported synchronously through the return code; nothing is
 *   enqueued when the code is not NORM_SUCCESS.  Argument checks run before
 *   any HIP call, in this order: rows < 0 / bad eps / bad config ->
 *   INVALID_VALUE; then, for the forward ops, rows == 0 -> SUCCESS with
 *   nothing enqueued; hidden < 1 or beyond every kernel -> UNSUPPORTED_HIDDEN;
 *   null pointer, ld < hidden, ld > 2^40 or a matrix spanning more than
 *   2^47 bytes ((rows - 1) * ld + hidden elements) -> INVALID_VALUE;
 *   misaligned pointer ->
 *   MISALIGNED; buffers that overlap other than by an allowed exact alias ->
 *   INVALID_VALUE (two matrices with the same ld whose rows interleave
 *   without sharing an element, such as two column slices of one wider
 *   matrix, do not overlap); workspace too small -> WORKSPACE.  The backward
 *   ops with rows == 0 enqueue only the zero-fill of dweight (and dbias).
 *   Choosing a launch shape may query the current device once (DEVICE on
 *   failure).  A launch failure reported by HIP returns LAUNCH.
 * - Arithmetic: bf16 inputs are widened exactly to fp32, every sum and product
 *   is fp32, every bf16 store rounds to nearest-even, rstd uses the hardware
 *   reciprocal square root.
 *
 * Sources (the pages name the operations; the formulas are the textbook ones):
 *   "optimize inner persistent scheduler for static fusion" (nvFuser PR 5281),
 *     author description: static hidden size, larger blocks for small batches;
 *     changes walkthrough: fused add + RMSNorm benchmarked with in-place update.
 *   "TMA inner persistent scheduler" (nvFuser PR 5587), description summary:
 *     RMSNorm and LayerNorm forward.
 *   "Llu/ln bwd" (nvFuser PR 207), author note and review thread: LayerNorm
 *     backward as a combined inner (per-row) and outer (per-column) reduction.
 *   RMSNorm: Zhang & Sennrich (2019), eq. 4.  LayerNorm: Ba, Kiros & Hinton
 *   (2016), eq. 4, with eps inside the square root and biased variance.
 */
#ifndef ROWNORM_NORM_H
#define ROWNORM_NORM_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifndef NORM_API
#define NORM_API __attribute__((visibility("default")))
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    NORM_SUCCESS = 0,
    NORM_ERROR_INVALID_VALUE = 1,      /* bad rows/eps/pointer/overlap/config */
    NORM_ERROR_UNSUPPORTED_HIDDEN = 2, /* no kernel holds a row this wide      */
    NORM_ERROR_MISALIGNED = 3,         /* pointer alignment too small           */
    NORM_ERROR_WORKSPACE = 4,          /* LayerNorm-backward workspace too small */
    NORM_ERROR_LAUNCH = 5,             /* HIP reported an error at launch       */
    NORM_ERROR_DEVICE = 6              /* the current device could not be queried */
} norm_status;

typedef enum {
    NORM_OP_FUSED_ADD_RMSNORM = 0,
    NORM_OP_RMSNORM_FWD = 1,
    NORM_OP_LAYERNORM_FWD = 2,
    NORM_OP_LAYERNORM_BWD = 3,
    NORM_OP_RMSNORM_BWD = 4,
    NORM_OP_FUSED_ADD_RMSNORM_BWD = 5
} norm_op;

/* Launch shape of one kernel instantiation.
 *   threads_per_row : lanes that share one row.  Compiled-hidden shapes: a
 *                     multiple of 64 (the wave size); hidden / (8 * lanes)
 *                     16-byte vectors of the row live in each lane's
 *                     registers.  Run-time-hidden shapes: 8, 16, ..., 1024
 *                     (rows narrower than a wave share it).
 *   rows_per_block  : rows handled side by side by one workgroup.  Run-time
 *                     shapes: max(1, 256 / threads_per_row), workgroups of
 *                     max(256, threads_per_row) lanes.
 *   grid            : number of persistent workgroups that walk the rows.
 *                     Backward ops: 0 lets the library choose; each
 *                     workgroup writes one partial column-sum slab.
 *                     LayerNorm and RMSNorm forward: 0 runs one row per lane
 *                     group, > 0 runs the persistent ring kernel of that lane
 *                     count (compiled-hidden shapes, rows_per_block 1) on that
 *                     many workgroups; the library picks the ring depth (rows
 *                     in flight per workgroup) from the walk, ceil(rows /
 *                     grid) rows.  Must be 0 for the fused op.
 *   vector_elems    : 0 for a compiled-hidden shape; 1, 2, 4 or 8 for a
 *                     run-time-hidden shape whose accesses move that many
 *                     bf16 elements (hidden, every ld and every bf16 pointer
 *                     must allow it). */
typedef struct {
    int32_t threads_per_row;
    int32_t rows_per_block;
    int32_t grid;
    int32_t vector_elems;
} norm_launch_cfg;

/* Human-readable name of a status code (static storage, never NULL). */
NORM_API const char* norm_status_string(norm_status status);

/* Fused residual-add + RMSNorm forward ("optimize inner persistent scheduler
 * for static fusion", author description and changes walkthrough):
 *   s        = x + residual                        (fp32)
 *   residual = bf16(s)                             (in place)
 *   out      = bf16(s * rsqrt(mean_j(s^2) + eps) * weight)
 * out, residual, x: [rows, hidden] bf16; weight: [hidden] bf16.
 * out may equal x exactly (in-place normalize); residual may alias nothing.
 * eps must be finite and >= 0. */
NORM_API norm_status norm_fused_add_rmsnorm(void* out, void* residual, const void* x,
                                   const void* weight, int64_t rows, int64_t hidden,
                                   float eps, hipStream_t stream);

/* RMSNorm forward ("TMA inner persistent scheduler", description summary):
 *   out = bf16(x * rsqrt(mean_j(x^2) + eps) * weight)
 * out, x: [rows, hidden] bf16 (out may equal x exactly); weight: [hidden] bf16. */
NORM_API norm_status norm_rmsnorm_fwd(void* out, const void* x, const void* weight,
                             int64_t rows, int64_t hidden, float eps,
                             hipStream_t stream);

/* LayerNorm forward with affine weight and bias ("TMA inner persistent
 * scheduler", description summary), two-pass statistics on the row held in
 * registers:
 *   mu = mean_j x,  var = mean_j (x - mu)^2,  rstd = rsqrt(var + eps)
 *   y  = bf16((x - mu) * rstd * weight + bias)
 * y, x: [rows, hidden] bf16 (y may equal x exactly); weight, bias: [hidden]
 * bf16; mean, rstd: [rows] fp32 outputs, or both NULL to skip storing them. */
NORM_API norm_status norm_layernorm_fwd(void* y, float* mean, float* rstd, const void* x,
                               const void* weight, const void* bias,
                               int64_t rows, int64_t hidden, float eps,
                               hipStream_t stream);

/* LayerNorm backward as one combined inner + outer reduction ("Llu/ln bwd",
 * author note and review thread), with the forward statistics given:
 *   xhat = (x - mean) * rstd,  g = dy * weight
 *   dx   = bf16(rstd * (g - mean_j g - xhat * mean_j(g * xhat)))   (per row)
 *   dweight_j = sum_i dy_ij * xhat_ij,  dbias_j = sum_i dy_ij        (per column)
 * dx, dy, x: [rows, hidden] bf16 (dx may equal dy exactly); mean, rstd: [rows]
 * fp32; weight: [hidden] bf16; dweight, dbias: [hidden] fp32, overwritten (not
 * accumulated).  The column sums are formed in two kernels: per-workgroup
 * partial sums into `workspace`, then a fixed-order column reduce, so results
 * are bitwise reproducible run to run for a given (rows, hidden, device).
 * workspace: device scratch of at least
 * norm_layernorm_bwd_workspace_bytes(rows, hidden) bytes, 16-byte aligned; its
 * contents on entry are ignored and on exit are unspecified.
 * eps is validated like the forward ops' but unused (mean and rstd are given). */
NORM_API norm_status norm_layernorm_bwd(void* dx, float* dweight, float* dbias,
                               const void* dy, const void* x, const float* mean,
                               const float* rstd, const void* weight,
                               void* workspace, size_t workspace_bytes,
                               int64_t rows, int64_t hidden, float eps,
                               hipStream_t stream);

/* norm_layernorm_bwd for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same operation, arguments, launch choice, kernels and
 * errors, with the per-workgroup partial sums kept in a scratch array the
 * library holds in every device's memory (NORM_NOALLOC_SCRATCH_BYTES per
 * device, set up on the first call on a device and kept until the process
 * ends) instead of a caller-given workspace.  Allocates nothing: no
 * hipMalloc, no hipFree, no allocating library call.  Returns
 * NORM_ERROR_WORKSPACE when the launch's workspace
 * (norm_layernorm_bwd_workspace_bytes for contiguous rows: 2 * 4 * hidden
 * bytes, hidden rounded up to 64 off the compiled sizes, for each of its up
 * to 256 workgroups; rows past 32768 columns: the same for each of its up to
 * 511 / ceil(hidden / 4096) row walkers, each with 192 bytes of partial-sum
 * exchange slots per 4096-column tile; past 262144 columns for each of up to
 * 255 / ceil(hidden / 16384) walkers, plus 8 bytes a row) would exceed
 * NORM_NOALLOC_SCRATCH_BYTES: every hidden up to 16384 fits, rows of
 * 16392-32768 columns fit only with fewer rows (32768: up to 128 rows),
 * rows of 32776-262144 columns fit at every row count, and wider rows fit
 * up to at least 16384 rows.
 * NORM_ERROR_DEVICE when the
 * scratch array's address cannot be found on the current device.  All calls
 * on one device share its scratch array: calls that overlap in time on that
 * device (different streams, or different host threads, without ordering
 * between them) race and give wrong column sums; calls in one stream's order
 * are safe.  Nothing in the array needs to start at any value (every slab a
 * launch reads it writes first).  Results are bitwise those of
 * norm_layernorm_bwd. */
#define NORM_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
NORM_API norm_status norm_layernorm_bwd_noalloc(void* dx, float* dweight, float* dbias,
                                                const void* dy, const void* x,
                                                const float* mean, const float* rstd,
                                                const void* weight, int64_t rows,
                                                int64_t hidden, float eps, hipStream_t stream);

/* RMSNorm backward with the same combined inner + outer reduction ("Llu/ln
 * bwd", author note and review thread, applied to RMSNorm), the per-row
 * statistic recomputed from x with `eps` (no saved statistic is needed):
 *   rstd = rsqrt(mean_j x^2 + eps),  xhat = x * rstd,  g = dy * weight
 *   dx   = bf16(rstd * (g - xhat * mean_j(g * xhat)))   (per row)
 *   dweight_j = sum_i dy_ij * xhat_ij                    (per column)
 * dx, dy, x: [rows, hidden] bf16 (dx may equal dy exactly); weight: [hidden]
 * bf16; dweight: [hidden] fp32, overwritten.  workspace: at least
 * norm_rmsnorm_bwd_workspace_bytes(rows, hidden) bytes, 16-byte aligned,
 * contents ignored on entry.  Column sums are bitwise reproducible run to run. */
NORM_API norm_status norm_rmsnorm_bwd(void* dx, float* dweight, const void* dy, const void* x,
                                      const void* weight, void* workspace,
                                      size_t workspace_bytes, int64_t rows, int64_t hidden,
                                      float eps, hipStream_t stream);

/* Backward of norm_fused_add_rmsnorm ("optimize inner persistent scheduler
 * for static fusion", changes walkthrough: the fused residual-add + RMSNorm).
 * The forward's s = x + residual feeds both out = RMSNorm(s) * weight and the
 * residual output, so x and the residual input receive the same gradient:
 *   ds = bf16(RMSNormBackward(dout; s, weight, eps) + dres)
 * s: the residual output of the forward (bf16 [rows, hidden]); dout: gradient
 * of out; dres: gradient of the residual output, or NULL for none.  ds may
 * equal dout or dres exactly.  dweight and workspace as for norm_rmsnorm_bwd. */
NORM_API norm_status norm_fused_add_rmsnorm_bwd(void* ds, float* dweight, const void* dout,
                                                const void* dres, const void* s,
                                                const void* weight, void* workspace,
                                                size_t workspace_bytes, int64_t rows,
                                                int64_t hidden, float eps, hipStream_t stream);

/* Bytes of workspace the two RMSNorm backward ops need: with the library's
 * choice, enough for any layout (strides, alignment) of this hidden size; or
 * for a given shape.  Enough for either op (their kernels differ at 28680 ...
 * 32768 columns, where the fused op streams its rows).  Pure host
 * arithmetic; 0 for an unsupported hidden or rows <= 0. */
NORM_API size_t norm_rmsnorm_bwd_workspace_bytes(int64_t rows, int64_t hidden);
NORM_API size_t norm_rmsnorm_bwd_workspace_bytes_cfg(int64_t rows, int64_t hidden,
                                                     const norm_launch_cfg* cfg);

/* Bytes of workspace norm_layernorm_bwd needs for (rows, hidden) with the
 * library's own launch choice, for any layout (strides, alignment) of this
 * hidden size.  Pure host arithmetic (no HIP call); returns 0 for an
 * unsupported hidden or rows <= 0. */
NORM_API size_t norm_layernorm_bwd_workspace_bytes(int64_t rows, int64_t hidden);

/* Bytes of workspace a given LayerNorm-backward launch shape needs. */
NORM_API size_t norm_layernorm_bwd_workspace_bytes_cfg(int64_t rows, int64_t hidden,
                                              const norm_launch_cfg* cfg);

/* Variants of the operations that run a given launch shape instead of the
 * library's choice (cfg == NULL means the library's choice).  A shape that
 * was not compiled for (op, hidden) returns INVALID_VALUE. */
NORM_API norm_status norm_fused_add_rmsnorm_cfg(void* out, void* residual, const void* x,
                                       const void* weight, int64_t rows, int64_t hidden,
                                       float eps, const norm_launch_cfg* cfg,
                                       hipStream_t stream);
NORM_API norm_status norm_rmsnorm_fwd_cfg(void* out, const void* x, const void* weight,
                                 int64_t rows, int64_t hidden, float eps,
                                 const norm_launch_cfg* cfg, hipStream_t stream);
NORM_API norm_status norm_layernorm_fwd_cfg(void* y, float* mean, float* rstd, const void* x,
                                   const void* weight, const void* bias,
                                   int64_t rows, int64_t hidden, float eps,
                                   const norm_launch_cfg* cfg, hipStream_t stream);
NORM_API norm_status norm_rmsnorm_bwd_cfg(void* dx, float* dweight, const void* dy,
                                          const void* x, const void* weight, void* workspace,
                                          size_t workspace_bytes, int64_t rows, int64_t hidden,
                                          float eps, const norm_launch_cfg* cfg,
                                          hipStream_t stream);
NORM_API norm_status norm_fused_add_rmsnorm_bwd_cfg(void* ds, float* dweight, const void* dout,
                                                    const void* dres, const void* s,
                                                    const void* weight, void* workspace,
                                                    size_t workspace_bytes, int64_t rows,
                                                    int64_t hidden, float eps,
                                                    const norm_launch_cfg* cfg,
                                                    hipStream_t stream);
NORM_API norm_status norm_layernorm_bwd_cfg(void* dx, float* dweight, float* dbias,
                                   const void* dy, const void* x, const float* mean,
                                   const float* rstd, const void* weight,
                                   void* workspace, size_t workspace_bytes,
                                   int64_t rows, int64_t hidden, float eps,
                                   const norm_launch_cfg* cfg, hipStream_t stream);

/* Strided variants ("_ex"): every matrix argument is followed by its leading
 * dimension (row stride in elements, >= hidden), so rows may be slices of
 * wider matrices (for instance the query or key part of a fused projection
 * output); `cfg` as for the "_cfg" variants (NULL: the library's choice).
 * Semantics, aliasing rules and errors are those of the operation without
 * the suffix; an exact alias also needs equal leading dimensions. */
NORM_API norm_status norm_fused_add_rmsnorm_ex(void* out, int64_t ld_out, void* residual,
                                               int64_t ld_residual, const void* x, int64_t ld_x,
                                               const void* weight, int64_t rows, int64_t hidden,
                                               float eps, const norm_launch_cfg* cfg,
                                               hipStream_t stream);
NORM_API norm_status norm_rmsnorm_fwd_ex(void* out, int64_t ld_out, const void* x, int64_t ld_x,
                                         const void* weight, int64_t rows, int64_t hidden,
                                         float eps, const norm_launch_cfg* cfg,
                                         hipStream_t stream);
NORM_API norm_status norm_layernorm_fwd_ex(void* y, int64_t ld_y, float* mean, float* rstd,
                                           const void* x, int64_t ld_x, const void* weight,
                                           const void* bias, int64_t rows, int64_t hidden,
                                           float eps, const norm_launch_cfg* cfg,
                                           hipStream_t stream);
NORM_API norm_status norm_layernorm_bwd_ex(void* dx, int64_t ld_dx, float* dweight, float* dbias,
                                           const void* dy, int64_t ld_dy, const void* x,
                                           int64_t ld_x, const float* mean, const float* rstd,
                                           const void* weight, void* workspace,
                                           size_t workspace_bytes, int64_t rows, int64_t hidden,
                                           float eps, const norm_launch_cfg* cfg,
                                           hipStream_t stream);
NORM_API norm_status norm_rmsnorm_bwd_ex(void* dx, int64_t ld_dx, float* dweight, const void* dy,
                                         int64_t ld_dy, const void* x, int64_t ld_x,
                                         const void* weight, void* workspace,
                                         size_t workspace_bytes, int64_t rows, int64_t hidden,
                                         float eps, const norm_launch_cfg* cfg,
                                         hipStream_t stream);
/* ld_dres is ignored when dres is NULL. */
NORM_API norm_status norm_fused_add_rmsnorm_bwd_ex(void* ds, int64_t ld_ds, float* dweight,
                                                   const void* dout, int64_t ld_dout,
                                                   const void* dres, int64_t ld_dres,
                                                   const void* s, int64_t ld_s,
                                                   const void* weight, void* workspace,
                                                   size_t workspace_bytes, int64_t rows,
                                                   int64_t hidden, float eps,
                                                   const norm_launch_cfg* cfg,
                                                   hipStream_t stream);

/* Row-split forward ("Llu/ln bwd", author note: the grid-parallel inner
 * normalization the pages list as missing).  With few rows one workgroup per
 * row leaves most CUs idle and moves a wide row at the rate of one CU; these
 * entry points may instead cut each row into `k` contiguous chunks, one
 * workgroup each, whose partial sums meet in `workspace` (the workgroups of
 * a row wait for each other there; LayerNorm combines the chunks' sums and
 * centered sums of squares exactly).  Results equal the operation's
 * definition within the same tolerances as the other entry points, with a
 * different summation order, and are bitwise reproducible run to run.
 *   split = 0: the library's choice (norm_select_split; rows it does not
 *              split run the operation's usual kernels and leave the
 *              workspace untouched, which may then be NULL);
 *   split = 1: never split;
 *   split = k >= 2: about k workgroups per row (the chunk count that covers
 *              the row with the fewest 16-byte accesses per lane, at most 8);
 *              needs 16-byte-aligned pointers (else MISALIGNED), hidden a
 *              multiple of 8, rows <= 512 and rows * k <= the device's CU
 *              count (else INVALID_VALUE).
 * Through these entry points LayerNorm forward also takes rows of up to 65536
 * (wider than its one-workgroup-per-row kernels hold) when they are split.
 * Arguments, aliasing rules and errors are otherwise the operation's own;
 * rows are contiguous.  workspace: device memory of at least
 * norm_split_workspace_bytes(rows) bytes, 16-byte aligned, overlapping no
 * other argument, ZERO-FILLED before its first use; every call that finishes
 * leaves it zero-filled again, so one workspace serves any number of calls
 * in stream order (calls that overlap in time on one workspace race).  Its
 * first 32-bit word stays 0 unless a workgroup gave up waiting for its row's
 * partners (about a second, see norm_split_set_spin_limit; only possible
 * when other work keeps the launch from being resident at once): then bit 0
 * is set, and every chunk whose workgroup gave up is written as NaN (its
 * out or y elements, and for a row's first chunk that row's mean and rstd),
 * never as wrong finite values; the fused op's residual is still correct.
 * The bit stays set until norm_split_status clears it; the rest of the
 * workspace is zero-filled again as after any call.  Ownership: the
 * caller's. */
NORM_API norm_status norm_fused_add_rmsnorm_split(void* out, void* residual, const void* x,
                                                  const void* weight, int64_t rows,
                                                  int64_t hidden, float eps, void* workspace,
                                                  size_t workspace_bytes, int32_t split,
                                                  hipStream_t stream);
NORM_API norm_status norm_rmsnorm_fwd_split(void* out, const void* x, const void* weight,
                                            int64_t rows, int64_t hidden, float eps,
                                            void* workspace, size_t workspace_bytes,
                                            int32_t split, hipStream_t stream);
NORM_API norm_status norm_layernorm_fwd_split(void* y, float* mean, float* rstd, const void* x,
                                              const void* weight, const void* bias,
                                              int64_t rows, int64_t hidden, float eps,
                                              void* workspace, size_t workspace_bytes,
                                              int32_t split, hipStream_t stream);

/* Workspace bytes the row-split entry points need for `rows` rows (0 for
 * rows <= 0; constant above 512 rows, which are never split). */
NORM_API size_t norm_split_workspace_bytes(int64_t rows);

/* Error word of a row-split workspace: waits for `stream` (every call
 * enqueued on it so far has finished), then stores the workspace's first
 * 32-bit word in *status (0: no workgroup of any call since the word was
 * last cleared gave up; bit 0 set: at least one did, and that call's NaN
 * chunks mark the rows affected).  clear != 0 resets a nonzero word to 0.
 * Synchronizes the host with `stream`, so it cannot be called while the
 * stream is being captured into a graph.  Errors: INVALID_VALUE for a NULL
 * workspace or status, MISALIGNED for a workspace not 16-byte aligned,
 * LAUNCH when the copy or the synchronization fails. */
NORM_API norm_status norm_split_status(void* workspace, int32_t clear, uint32_t* status,
                                       hipStream_t stream);

/* Polls a row-split partner wait makes before it gives up (default 2^20,
 * about a second; 0: give up at once without polling, which makes every
 * split workgroup write NaN and set the error bit).  Process-wide, read
 * when a split call is enqueued; returns the previous value.  For tests and
 * diagnostics of the give-up path. */
NORM_API uint32_t norm_split_set_spin_limit(uint32_t polls);

/* Polls a streamed-backward tile makes while it waits for the partial row
 * sums of its row's other column tiles (default 2^14, about 16 ms; 0: never
 * wait).  A tile that runs out stops waiting for the rest of its walk and
 * reads the other tiles of each row itself instead, forming their partial
 * sums exactly as their own workgroups do: the results are bitwise the same,
 * only slower (two reads of those rows).  Process-wide, read when a call is
 * enqueued; returns the previous value.  For tests and diagnostics of that
 * path ("Llu/ln bwd", review thread: the grid-parallel inner reduction of
 * the backward, here across a row's column tiles). */
NORM_API uint32_t norm_bwd_set_spin_limit(uint32_t polls);

/* The row split the library would choose for a forward op (fused, RMSNorm or
 * LayerNorm forward) on contiguous 16-byte-aligned rows with `cu_count` CUs
 * (<= 0: the current device): *split = workgroups per row (1: no split) and
 * *vecs = 16-byte accesses per lane (0 when not split).  Rows are split when
 * hidden is a multiple of 8 and either up to 8 rows move >= 256 KiB each
 * (fused op: 8 * hidden bytes) or >= 192 KiB each (the others: 4 * hidden
 * bytes), 9 to 32 rows
 * move >= 384 KiB each, or no one-workgroup-per-row kernel holds the row on
 * chip (above 65536, LayerNorm above 49152; up to 64 rows).  Chunks aim at about 64 KiB of
 * traffic (8192 columns fused, 16384 RMSNorm, 12288 LayerNorm), at most
 * max(4, 64 / rows) a row and rows * k <= cu_count.  Pure host logic when
 * cu_count > 0. */
NORM_API norm_status norm_select_split(norm_op op, int64_t rows, int64_t hidden,
                                       int32_t cu_count, int32_t* split, int32_t* vecs);

/* The library's launch choice for (op, rows, hidden) on a device with
 * `cu_count` compute units (the small-batch rule of "optimize inner
 * persistent scheduler for static fusion", author description: when the
 * batch cannot fill the machine, spread each row over more lanes).
 * cu_count <= 0 queries the current device.  Pure host logic otherwise.
 * Backward rows past 32768 columns that exchange partial sums between
 * column tiles get at most 2 * cu_count / tiles row walkers, so that all of
 * the launch's workgroups are resident at once (the launch applies the same
 * cap with the current device's CUs).
 * The choice assumes contiguous rows and 16-byte-aligned pointers; a call
 * with strides or smaller alignment may run a run-time-hidden shape with
 * narrower accesses instead. */
NORM_API norm_status norm_select_config(norm_op op, int64_t rows, int64_t hidden,
                               int32_t cu_count, norm_launch_cfg* cfg);

/* Human-readable description of the launch the library would make for
 * (op, rows, hidden) through the bf16 entry points (the `_f32` ones choose
 * by hidden alone, as their section below states) on a device with
 * `cu_count` compute units (<= 0: the current device): kernel
 * instantiation, lanes per row, rows per workgroup, 16-byte vectors per lane,
 * workgroup size, grid, ring depth and workspace.
 * Writes a NUL-terminated string of at most `len` bytes to `buf` (which may be
 * NULL when len is 0) and returns the full length without the NUL, or -1 for
 * invalid arguments or an unsupported hidden.  Host logic only when
 * cu_count > 0. */
NORM_API int32_t norm_describe_config(norm_op op, int64_t rows, int64_t hidden,
                                      int32_t cu_count, char* buf, size_t len);

/* Enumerate the launch shapes that can run (op, hidden): the compiled-hidden
 * shapes (when hidden is compiled), then the run-time-hidden shapes at the
 * widest access width hidden allows.  Writes up to `capacity` entries to
 * `out` (which may be NULL when capacity is 0) and returns the total count;
 * 0 for an unsupported hidden. */
NORM_API int32_t norm_list_configs(norm_op op, int64_t hidden, norm_launch_cfg* out,
                          int32_t capacity);

/* ---- fp32 activations ----------------------------------------------------
 * The six operations above on fp32 matrices and fp32 weight / bias vectors:
 * the same formulas, arguments and errors, with every bf16 store replaced by
 * an fp32 store of the fp32 result (norm_fused_add_rmsnorm_f32's residual is
 * the fp32 sum x + residual, rounded once).  The pages fix no activation
 * precision ("TMA inner persistent scheduler" and "optimize inner persistent
 * scheduler for static fusion" benchmark bf16); fp32 is the other activation
 * type their schedulers take.  Restrictions: contiguous rows (ld = hidden),
 * hidden a multiple of 4 from 4 up to 2^20 (else UNSUPPORTED_HIDDEN), the
 * matrices and the weight / bias vectors 16-byte aligned, mean / rstd /
 * dweight / dbias 4-byte aligned, the workspace 16-byte aligned (else
 * MISALIGNED).  Aliasing as for the bf16 entry points: out (y) may equal x,
 * dx (ds) may equal dy (dout) or dres, nothing else overlaps.
 * Forward: rows of up to 1024 values take 8 to 32 lanes each, 256 / lanes
 * rows to a workgroup; wider rows take one workgroup each (64 to 1024
 * lanes), which holds up to 16384 values of the row in registers between
 * the statistic and the normalize step (32768 for the fused op and RMSNorm)
 * and reads any rest again, except fused rows of 34956 ... 40960 and
 * RMSNorm rows of 34956 ... 69632, whose rest is staged in LDS (read once).
 * Backward: rows of up to 8192 columns are held by one 512-lane workgroup
 * that reduces the row itself; 8196 ... 16384 columns are staged in LDS
 * (read once); wider rows take 256-lane workgroups over 4096-column tiles
 * that exchange each row's partial sums (read once; up to 262144 columns,
 * wider rows: a row-sums kernel first, then 512-lane workgroups over
 * 8192-column tiles read the row again);
 * then the fixed-order column reduce (column sums bitwise reproducible run
 * to run).  workspace: at least
 * norm_bwd_workspace_bytes_f32(op, rows, hidden) bytes, contents ignored on
 * entry. */
NORM_API norm_status norm_fused_add_rmsnorm_f32(float* out, float* residual, const float* x,
                                                const float* weight, int64_t rows,
                                                int64_t hidden, float eps, hipStream_t stream);
NORM_API norm_status norm_rmsnorm_fwd_f32(float* out, const float* x, const float* weight,
                                          int64_t rows, int64_t hidden, float eps,
                                          hipStream_t stream);
NORM_API norm_status norm_layernorm_fwd_f32(float* y, float* mean, float* rstd, const float* x,
                                            const float* weight, const float* bias,
                                            int64_t rows, int64_t hidden, float eps,
                                            hipStream_t stream);
NORM_API norm_status norm_layernorm_bwd_f32(float* dx, float* dweight, float* dbias,
                                            const float* dy, const float* x, const float* mean,
                                            const float* rstd, const float* weight,
                                            void* workspace, size_t workspace_bytes,
                                            int64_t rows, int64_t hidden, float eps,
                                            hipStream_t stream);
NORM_API norm_status norm_rmsnorm_bwd_f32(float* dx, float* dweight, const float* dy,
                                          const float* x, const float* weight, void* workspace,
                                          size_t workspace_bytes, int64_t rows, int64_t hidden,
                                          float eps, hipStream_t stream);
NORM_API norm_status norm_fused_add_rmsnorm_bwd_f32(float* ds, float* dweight, const float* dout,
                                                    const float* dres, const float* s,
                                                    const float* weight, void* workspace,
                                                    size_t workspace_bytes, int64_t rows,
                                                    int64_t hidden, float eps,
                                                    hipStream_t stream);
/* Workspace bytes of an fp32 backward op (NORM_OP_LAYERNORM_BWD,
 * NORM_OP_RMSNORM_BWD or NORM_OP_FUSED_ADD_RMSNORM_BWD): 4 * padded hidden
 * (hidden rounded up to 64) per partial-sum slab and output column sum, for
 * each row walker: min(rows, 255) of them up to 8192 columns, min(rows,
 * 256) at 8196 ... 16384, max(1, min(rows, 511 / ceil(hidden / 4096))) at
 * 16388 ... 262144, each with 192 bytes of partial-sum exchange slots per
 * 4096-column tile, and past that max(1, min(rows, 255 / ceil(hidden /
 * 8192))) plus 8 bytes a row.  Pure
 * host arithmetic; 0 for another op, an unsupported hidden or rows <= 0. */
NORM_API size_t norm_bwd_workspace_bytes_f32(norm_op op, int64_t rows, int64_t hidden);

#ifdef __cplusplus
}
#endif

#endif /* ROWNORM_NORM_H */
