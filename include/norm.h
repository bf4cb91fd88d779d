/*
 * norm.h -- C ABI of the MI355X (gfx950) inner-persistent row-normalization
 * library (librownorm.so).
 *
 * Every operation normalizes the rows of a row-major [rows, hidden] bf16
 * matrix.  Each row is read from HBM once into registers, reduced there, and
 * written once ("inner persistent": the row stays on-chip between the
 * reduction and the normalize step).  The hidden size is a compile-time
 * constant of the kernel that runs; the supported set is
 *     {1024, 2048, 4096, 8192, 12288, 16384}.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors are DEVICE pointers into memory of the calling thread's current
 *   HIP device, row-major and contiguous: element (i, j) of a [rows, hidden]
 *   matrix sits at index i * hidden + j.  bf16 tensors are passed as
 *   void* / const void* holding IEEE bf16 bit patterns and must be 16-byte
 *   aligned; fp32 tensors must be 4-byte aligned.
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
 *   nothing enqueued; hidden not supported -> UNSUPPORTED_HIDDEN; null
 *   pointer -> INVALID_VALUE; misaligned pointer -> MISALIGNED; buffers that
 *   overlap other than by an allowed exact alias -> INVALID_VALUE; workspace
 *   too small -> WORKSPACE.  LayerNorm backward with rows == 0 enqueues only
 *   the zero-fill of dweight and dbias.  Choosing a launch shape may query
 *   the current device once (DEVICE on failure).  A launch failure reported
 *   by HIP returns LAUNCH.
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
    NORM_ERROR_UNSUPPORTED_HIDDEN = 2, /* hidden not in the compiled set       */
    NORM_ERROR_MISALIGNED = 3,         /* bf16 ptr not 16 B, fp32 ptr not 4 B  */
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
 *   threads_per_row : lanes that share one row (a multiple of 64, the wave
 *                     size); hidden / (8 * threads_per_row) 16-byte vectors
 *                     of the row live in each lane's registers.
 *   rows_per_block  : rows handled side by side by one workgroup
 *                     (workgroup size = threads_per_row * rows_per_block).
 *   grid            : backward ops only: number of persistent workgroups (one
 *                     partial column-sum slab each); 0 lets the library
 *                     choose.  Must be 0 for the forward ops. */
typedef struct {
    int32_t threads_per_row;
    int32_t rows_per_block;
    int32_t grid;
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

/* Bytes of workspace the two RMSNorm backward ops need (library's launch
 * choice, or a given shape).  Pure host arithmetic; 0 for an unsupported
 * hidden or rows <= 0. */
NORM_API size_t norm_rmsnorm_bwd_workspace_bytes(int64_t rows, int64_t hidden);
NORM_API size_t norm_rmsnorm_bwd_workspace_bytes_cfg(int64_t rows, int64_t hidden,
                                                     const norm_launch_cfg* cfg);

/* Bytes of workspace norm_layernorm_bwd needs for (rows, hidden) with the
 * library's own launch choice.  Pure host arithmetic (no HIP call); returns 0
 * for an unsupported hidden or rows < 0. */
NORM_API size_t norm_layernorm_bwd_workspace_bytes(int64_t rows, int64_t hidden);

/* Bytes of workspace a given LayerNorm-backward launch shape needs. */
NORM_API size_t norm_layernorm_bwd_workspace_bytes_cfg(int64_t rows, int64_t hidden,
                                              const norm_launch_cfg* cfg);

/* Variants of the four operations that run a given compiled launch shape
 * instead of the library's choice (cfg == NULL means the library's choice).
 * A shape that was not compiled for (op, hidden) returns INVALID_VALUE. */
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

/* The library's launch choice for (op, rows, hidden) on a device with
 * `cu_count` compute units (the small-batch rule of "optimize inner
 * persistent scheduler for static fusion", author description: when the
 * batch cannot fill the machine, spread each row over more lanes).
 * cu_count <= 0 queries the current device.  Pure host logic otherwise. */
NORM_API norm_status norm_select_config(norm_op op, int64_t rows, int64_t hidden,
                               int32_t cu_count, norm_launch_cfg* cfg);

/* Human-readable description of the launch the library would make for
 * (op, rows, hidden) on a device with `cu_count` compute units (<= 0: the
 * current device): kernel instantiation, lanes per row, rows per workgroup,
 * 16-byte vectors per lane, workgroup size, grid, ring depth and workspace.
 * Writes a NUL-terminated string of at most `len` bytes to `buf` (which may be
 * NULL when len is 0) and returns the full length without the NUL, or -1 for
 * invalid arguments or an unsupported hidden.  Host logic only when
 * cu_count > 0. */
NORM_API int32_t norm_describe_config(norm_op op, int64_t rows, int64_t hidden,
                                      int32_t cu_count, char* buf, size_t len);

/* Enumerate the compiled launch shapes of (op, hidden): writes up to
 * `capacity` entries to `out` (which may be NULL when capacity is 0) and
 * returns the total count; 0 for an unsupported hidden. */
NORM_API int32_t norm_list_configs(norm_op op, int64_t hidden, norm_launch_cfg* out,
                          int32_t capacity);

#ifdef __cplusplus
}
#endif

#endif /* ROWNORM_NORM_H */
