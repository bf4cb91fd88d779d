/*
 * CPU oracle for inner-persistent row normalization -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, obviously-correct double-precision loops.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load this library.
 * It shares no code, header, table or helper with the HIP library; the two are
 * compared against each other, never composed.
 *
 * Sources of the definitions (the pages name the operations, not formulas):
 *   - "optimize inner persistent scheduler for static fusion" (nvFuser PR 5281),
 *     author description and changes walkthrough: the fused residual-add +
 *     RMSNorm forward whose residual input is updated in place.
 *   - "TMA inner persistent scheduler" (nvFuser PR 5587), description summary:
 *     RMSNorm and LayerNorm forward.
 *   - "Llu/ln bwd" (nvFuser PR 207), author note and review thread: LayerNorm
 *     backward as a combined inner (per-row) + outer (per-column) reduction.
 *   - Textbook formulas: RMSNorm (Zhang & Sennrich, 2019, eq. 4) and LayerNorm
 *     (Ba, Kiros & Hinton, 2016, eq. 4) with the usual affine weight/bias,
 *     eps inside the square root, biased (divide-by-H) variance.
 *   - bf16 = IEEE-754 binary32 truncated to 8 significant bits (1 sign,
 *     8 exponent, 7 fraction bits); rounding is round-to-nearest, ties-to-even.
 *
 * Layout: every matrix is row-major [rows][hidden]; bf16 values are passed as
 * their 16-bit patterns (uint16_t).  Normalized outputs are returned UNROUNDED
 * in double so a caller can measure the error of a bf16 result in ulps.
 * Every function returns 0 on success and -1 on invalid arguments.
 * `nthreads` only splits independent rows (or, for column sums, independent
 * columns); each output is computed by the same sequential loop whatever the
 * thread count, so results do not depend on it.
 */
#ifndef ROWNORM_ORACLE_H
#define ROWNORM_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* bf16 pattern -> exact double value (IEEE-754 field decoding). */
double orc_bf16_decode(uint16_t bits);
/* double -> nearest bf16 pattern, ties to even; overflow -> +-inf; keeps the
 * sign of zero; NaN -> quiet NaN. */
uint16_t orc_bf16_encode(double v);
/* Bulk helpers over n elements. */
void orc_bf16_decode_n(const uint16_t* in, double* out, int64_t n);
void orc_bf16_encode_n(const double* in, uint16_t* out, int64_t n);

/* Fused residual-add + RMSNorm forward.
 *   s = x + r (exact in double),  res_out = bf16(s)  (one rounding),
 *   out = s / sqrt(mean_j(s^2) + eps) * w  (unrounded).
 * rstd_out (may be NULL) receives 1/sqrt(mean(s^2)+eps) per row. */
int orc_fused_add_rmsnorm(const uint16_t* x, const uint16_t* r, const uint16_t* w,
                          int64_t rows, int64_t hidden, double eps,
                          double* out, uint16_t* res_out, double* rstd_out,
                          int nthreads);

/* RMSNorm forward: out = x / sqrt(mean_j(x^2) + eps) * w. */
int orc_rmsnorm_fwd(const uint16_t* x, const uint16_t* w,
                    int64_t rows, int64_t hidden, double eps,
                    double* out, double* rstd_out, int nthreads);

/* LayerNorm forward (two-pass):
 *   mu = mean_j x,  var = mean_j (x - mu)^2,  rstd = 1/sqrt(var + eps),
 *   y = (x - mu) * rstd * w + b. */
int orc_layernorm_fwd(const uint16_t* x, const uint16_t* w, const uint16_t* b,
                      int64_t rows, int64_t hidden, double eps,
                      double* y, double* mean, double* rstd, int nthreads);

/* LayerNorm backward with the per-row statistics given (not recomputed):
 *   xhat = (x - mean) * rstd,  g = dy * w,
 *   c1 = mean_j g,  c2 = mean_j (g * xhat),
 *   dx = rstd * (g - c1 - xhat * c2)                 (inner, per row)
 *   dweight_j = sum_i dy_ij * xhat_ij,  dbias_j = sum_i dy_ij   (outer, per column)
 * Outputs are overwritten.  Column sums run over rows in index order. */
int orc_layernorm_bwd(const uint16_t* dy, const uint16_t* x,
                      const double* mean, const double* rstd, const uint16_t* w,
                      int64_t rows, int64_t hidden,
                      double* dx, double* dweight, double* dbias, int nthreads);

/* RMSNorm backward (and the fused residual-add + RMSNorm backward), with the
 * per-row statistic recomputed from x:
 *   rstd = 1/sqrt(mean_j(x^2) + eps),  xhat = x * rstd,  g = dy * w,
 *   c = mean_j (g * xhat),  dx = rstd * (g - xhat * c)  [+ dres]   (per row)
 *   dweight_j = sum_i dy_ij * xhat_ij                               (per column)
 * dres (may be NULL) is the gradient arriving at the fused op's residual
 * output; the fused op's x and residual inputs both receive dx. */
int orc_rmsnorm_bwd(const uint16_t* dy, const uint16_t* x, const uint16_t* w,
                    const uint16_t* dres, int64_t rows, int64_t hidden, double eps,
                    double* dx, double* dweight, double* rstd_out, int nthreads);

/* fp32 activations (oracle_f32.c): the same five definitions with every
 * operand an IEEE-754 binary32 value, widened to double exactly.  The fused
 * op's res_out is the exact sum x + r rounded once to binary32. */
int orc_fused_add_rmsnorm_f32(const float* x, const float* r, const float* w, int64_t rows,
                              int64_t hidden, double eps, double* out, float* res_out,
                              double* rstd_out, int nthreads);
int orc_rmsnorm_fwd_f32(const float* x, const float* w, int64_t rows, int64_t hidden,
                        double eps, double* out, double* rstd_out, int nthreads);
int orc_layernorm_fwd_f32(const float* x, const float* w, const float* b, int64_t rows,
                          int64_t hidden, double eps, double* y, double* mean, double* rstd,
                          int nthreads);
int orc_layernorm_bwd_f32(const float* dy, const float* x, const double* mean,
                          const double* rstd, const float* w, int64_t rows, int64_t hidden,
                          double* dx, double* dweight, double* dbias, int nthreads);
int orc_rmsnorm_bwd_f32(const float* dy, const float* x, const float* w, const float* dres,
                        int64_t rows, int64_t hidden, double eps, double* dx, double* dweight,
                        double* rstd_out, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
