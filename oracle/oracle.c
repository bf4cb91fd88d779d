/*
 * CPU oracle for inner-persistent row normalization -- TEST INFRASTRUCTURE ONLY.
 * Definitions and sources are listed in oracle.h.  Build: gcc -O2 (never
 * -ffast-math: every sum below must be evaluated exactly as written, in order).
 */
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>

/* ------------------------------------------------------------------------ */
/* bf16 <-> double, written from the IEEE-754 field definitions.             */
/* bf16: sign bit, 8-bit biased exponent (bias 127), 7-bit fraction.         */
/*   E == 0   : subnormal, value = F * 2^-133   (2^-133 = 2^(1-127-7))       */
/*   E == 255 : inf (F == 0) or NaN                                          */
/*   else     : value = (128 + F) * 2^(E - 127 - 7)                          */
/* ------------------------------------------------------------------------ */

double orc_bf16_decode(uint16_t bits) {
    int sign = (bits >> 15) & 1;
    int e = (bits >> 7) & 0xFF;
    int f = bits & 0x7F;
    double mag;
    if (e == 0) {
        mag = ldexp((double)f, -133);
    } else if (e == 255) {
        mag = (f == 0) ? INFINITY : NAN;
    } else {
        mag = ldexp((double)(128 + f), e - 127 - 7);
    }
    return sign ? -mag : mag;
}

/* Round a non-negative double holding an integer-plus-fraction to the
 * nearest integer, ties to the even neighbour. */
static double round_half_even(double s) {
    double fl = floor(s);
    double frac = s - fl; /* exact: s < 2^53 here */
    if (frac > 0.5) return fl + 1.0;
    if (frac < 0.5) return fl;
    return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

uint16_t orc_bf16_encode(double v) {
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    if (isnan(v)) return (uint16_t)(sign | 0x7FC0);
    double a = fabs(v);
    if (isinf(a)) return (uint16_t)(sign | 0x7F80);
    if (a == 0.0) return sign;

    /* a = m * 2^e2 with m in [0.5, 1): the leading bit has weight 2^(e2-1).
     * With 8 significant bits the quantum (ulp) is 2^(e2-1-7), but never
     * smaller than the subnormal quantum 2^-133. */
    int e2;
    (void)frexp(a, &e2);
    int q = e2 - 1 - 7;
    if (q < -133) q = -133;
    double n = round_half_even(ldexp(a, -q)); /* scaling by 2^-q is exact */

    if (q == -133 && n <= 128.0) {
        /* subnormal (n < 128) or rounded up to the smallest normal (n == 128):
         * in both cases the pattern is n itself (fraction field n, or
         * exponent field 1 with fraction 0 when n == 128). */
        return (uint16_t)(sign | (uint16_t)n);
    }
    if (n == 256.0) { /* rounding carried into the next binade */
        n = 128.0;
        q += 1;
    }
    int e = q + 7 + 127; /* biased exponent of n * 2^q, n in [128, 256) */
    if (e >= 255) return (uint16_t)(sign | 0x7F80);
    return (uint16_t)(sign | (uint16_t)(e << 7) | (uint16_t)((int)n - 128));
}

void orc_bf16_decode_n(const uint16_t* in, double* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_decode(in[i]);
}

void orc_bf16_encode_n(const double* in, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_encode(in[i]);
}

/* ------------------------------------------------------------------------ */
/* A plain "run f over [0, n) in nthreads contiguous blocks" helper.         */
/* ------------------------------------------------------------------------ */

typedef void (*range_fn)(const void* ctx, int64_t begin, int64_t end);

typedef struct {
    range_fn fn;
    const void* ctx;
    int64_t begin, end;
} range_job;

static void* range_job_main(void* p) {
    const range_job* j = (const range_job*)p;
    j->fn(j->ctx, j->begin, j->end);
    return NULL;
}

static void parallel_ranges(range_fn fn, const void* ctx, int64_t n, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > n) nthreads = (int)(n > 0 ? n : 1);
    if (nthreads == 1) {
        fn(ctx, 0, n);
        return;
    }
    pthread_t tid[256];
    range_job jobs[256];
    int started[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t].fn = fn;
        jobs[t].ctx = ctx;
        jobs[t].begin = n * t / nthreads;
        jobs[t].end = n * (t + 1) / nthreads;
        started[t] = pthread_create(&tid[t], NULL, range_job_main, &jobs[t]) == 0;
        if (!started[t]) range_job_main(&jobs[t]); /* run inline if no thread */
    }
    for (int t = 0; t < nthreads; ++t)
        if (started[t]) pthread_join(tid[t], NULL);
}

/* ------------------------------------------------------------------------ */
/* RMSNorm forward, with and without the fused residual add.                 */
/* ------------------------------------------------------------------------ */

typedef struct {
    const uint16_t *x, *r, *w; /* r == NULL: plain RMSNorm */
    int64_t hidden;
    double eps;
    double* out;
    uint16_t* res_out;
    double* rstd_out;
} rms_ctx;

static void rms_rows(const void* p, int64_t begin, int64_t end) {
    const rms_ctx* c = (const rms_ctx*)p;
    const int64_t H = c->hidden;
    double* s = (double*)malloc((size_t)H * sizeof(double));
    for (int64_t i = begin; i < end; ++i) {
        const int64_t base = i * H;
        /* s = x + r: both operands carry 8 significant bits, so the double
         * sum is exact unless their exponents are more than 44 apart, and
         * then the smaller one cannot move a bf16 rounding of the sum. */
        for (int64_t j = 0; j < H; ++j) {
            double v = orc_bf16_decode(c->x[base + j]);
            if (c->r) v += orc_bf16_decode(c->r[base + j]);
            s[j] = v;
        }
        if (c->res_out)
            for (int64_t j = 0; j < H; ++j) c->res_out[base + j] = orc_bf16_encode(s[j]);

        double ss = 0.0;
        for (int64_t j = 0; j < H; ++j) ss += s[j] * s[j];
        const double rstd = 1.0 / sqrt(ss / (double)H + c->eps);
        if (c->rstd_out) c->rstd_out[i] = rstd;
        for (int64_t j = 0; j < H; ++j)
            c->out[base + j] = s[j] * rstd * orc_bf16_decode(c->w[j]);
    }
    free(s);
}

static int bad_common(int64_t rows, int64_t hidden, double eps) {
    return rows < 0 || hidden <= 0 || !(eps >= 0.0) || isinf(eps);
}

int orc_fused_add_rmsnorm(const uint16_t* x, const uint16_t* r, const uint16_t* w,
                          int64_t rows, int64_t hidden, double eps,
                          double* out, uint16_t* res_out, double* rstd_out,
                          int nthreads) {
    if (bad_common(rows, hidden, eps)) return -1;
    if (rows == 0) return 0;
    if (!x || !r || !w || !out || !res_out) return -1;
    rms_ctx c = {x, r, w, hidden, eps, out, res_out, rstd_out};
    parallel_ranges(rms_rows, &c, rows, nthreads);
    return 0;
}

int orc_rmsnorm_fwd(const uint16_t* x, const uint16_t* w,
                    int64_t rows, int64_t hidden, double eps,
                    double* out, double* rstd_out, int nthreads) {
    if (bad_common(rows, hidden, eps)) return -1;
    if (rows == 0) return 0;
    if (!x || !w || !out) return -1;
    rms_ctx c = {x, NULL, w, hidden, eps, out, NULL, rstd_out};
    parallel_ranges(rms_rows, &c, rows, nthreads);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* LayerNorm forward.                                                        */
/* ------------------------------------------------------------------------ */

typedef struct {
    const uint16_t *x, *w, *b;
    int64_t hidden;
    double eps;
    double *y, *mean, *rstd;
} lnf_ctx;

static void lnf_rows(const void* p, int64_t begin, int64_t end) {
    const lnf_ctx* c = (const lnf_ctx*)p;
    const int64_t H = c->hidden;
    for (int64_t i = begin; i < end; ++i) {
        const uint16_t* xr = c->x + i * H;
        double sum = 0.0;
        for (int64_t j = 0; j < H; ++j) sum += orc_bf16_decode(xr[j]);
        const double mu = sum / (double)H;
        double sq = 0.0;
        for (int64_t j = 0; j < H; ++j) {
            const double d = orc_bf16_decode(xr[j]) - mu;
            sq += d * d;
        }
        const double var = sq / (double)H;
        const double rstd = 1.0 / sqrt(var + c->eps);
        c->mean[i] = mu;
        c->rstd[i] = rstd;
        for (int64_t j = 0; j < H; ++j)
            c->y[i * H + j] = (orc_bf16_decode(xr[j]) - mu) * rstd * orc_bf16_decode(c->w[j]) +
                              orc_bf16_decode(c->b[j]);
    }
}

int orc_layernorm_fwd(const uint16_t* x, const uint16_t* w, const uint16_t* b,
                      int64_t rows, int64_t hidden, double eps,
                      double* y, double* mean, double* rstd, int nthreads) {
    if (bad_common(rows, hidden, eps)) return -1;
    if (rows == 0) return 0;
    if (!x || !w || !b || !y || !mean || !rstd) return -1;
    lnf_ctx c = {x, w, b, hidden, eps, y, mean, rstd};
    parallel_ranges(lnf_rows, &c, rows, nthreads);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* LayerNorm backward: inner (per-row dx) and outer (per-column) sums.       */
/* ------------------------------------------------------------------------ */

typedef struct {
    const uint16_t *dy, *x, *w;
    const double *mean, *rstd;
    int64_t rows, hidden;
    double *dx, *dweight, *dbias;
} lnb_ctx;

static double lnb_xhat(const lnb_ctx* c, int64_t i, int64_t j) {
    return (orc_bf16_decode(c->x[i * c->hidden + j]) - c->mean[i]) * c->rstd[i];
}

static void lnb_rows(const void* p, int64_t begin, int64_t end) {
    const lnb_ctx* c = (const lnb_ctx*)p;
    const int64_t H = c->hidden;
    for (int64_t i = begin; i < end; ++i) {
        double sum_g = 0.0, sum_gx = 0.0;
        for (int64_t j = 0; j < H; ++j) {
            const double g = orc_bf16_decode(c->dy[i * H + j]) * orc_bf16_decode(c->w[j]);
            sum_g += g;
            sum_gx += g * lnb_xhat(c, i, j);
        }
        const double c1 = sum_g / (double)H;
        const double c2 = sum_gx / (double)H;
        for (int64_t j = 0; j < H; ++j) {
            const double g = orc_bf16_decode(c->dy[i * H + j]) * orc_bf16_decode(c->w[j]);
            c->dx[i * H + j] = c->rstd[i] * (g - c1 - lnb_xhat(c, i, j) * c2);
        }
    }
}

static void lnb_cols(const void* p, int64_t begin, int64_t end) {
    const lnb_ctx* c = (const lnb_ctx*)p;
    for (int64_t j = begin; j < end; ++j) {
        double dw = 0.0, db = 0.0;
        for (int64_t i = 0; i < c->rows; ++i) {
            const double d = orc_bf16_decode(c->dy[i * c->hidden + j]);
            dw += d * lnb_xhat(c, i, j);
            db += d;
        }
        c->dweight[j] = dw;
        c->dbias[j] = db;
    }
}

int orc_layernorm_bwd(const uint16_t* dy, const uint16_t* x,
                      const double* mean, const double* rstd, const uint16_t* w,
                      int64_t rows, int64_t hidden,
                      double* dx, double* dweight, double* dbias, int nthreads) {
    if (rows < 0 || hidden <= 0) return -1;
    if (!dweight || !dbias) return -1;
    if (rows == 0) {
        for (int64_t j = 0; j < hidden; ++j) dweight[j] = dbias[j] = 0.0;
        return 0;
    }
    if (!dy || !x || !mean || !rstd || !w || !dx) return -1;
    lnb_ctx c = {dy, x, w, mean, rstd, rows, hidden, dx, dweight, dbias};
    parallel_ranges(lnb_rows, &c, rows, nthreads);
    parallel_ranges(lnb_cols, &c, hidden, nthreads);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* RMSNorm backward: inner (per-row dx) and outer (per-column dweight) sums. */
/* ------------------------------------------------------------------------ */

typedef struct {
    const uint16_t *dy, *x, *w, *dres;
    int64_t rows, hidden;
    double eps;
    double *dx, *dweight, *rstd;
} rmsb_ctx;

static double rmsb_rstd(const rmsb_ctx* c, int64_t i) {
    double ss = 0.0;
    for (int64_t j = 0; j < c->hidden; ++j) {
        const double v = orc_bf16_decode(c->x[i * c->hidden + j]);
        ss += v * v;
    }
    return 1.0 / sqrt(ss / (double)c->hidden + c->eps);
}

static void rmsb_rows(const void* p, int64_t begin, int64_t end) {
    const rmsb_ctx* c = (const rmsb_ctx*)p;
    const int64_t H = c->hidden;
    for (int64_t i = begin; i < end; ++i) {
        const double rstd = rmsb_rstd(c, i);
        c->rstd[i] = rstd;
        double sum_gx = 0.0;
        for (int64_t j = 0; j < H; ++j) {
            const double g = orc_bf16_decode(c->dy[i * H + j]) * orc_bf16_decode(c->w[j]);
            sum_gx += g * orc_bf16_decode(c->x[i * H + j]) * rstd;
        }
        const double cc = sum_gx / (double)H;
        for (int64_t j = 0; j < H; ++j) {
            const double g = orc_bf16_decode(c->dy[i * H + j]) * orc_bf16_decode(c->w[j]);
            const double xhat = orc_bf16_decode(c->x[i * H + j]) * rstd;
            double v = rstd * (g - xhat * cc);
            if (c->dres) v += orc_bf16_decode(c->dres[i * H + j]);
            c->dx[i * H + j] = v;
        }
    }
}

static void rmsb_cols(const void* p, int64_t begin, int64_t end) {
    const rmsb_ctx* c = (const rmsb_ctx*)p;
    for (int64_t j = begin; j < end; ++j) {
        double dw = 0.0;
        for (int64_t i = 0; i < c->rows; ++i)
            dw += orc_bf16_decode(c->dy[i * c->hidden + j]) *
                  (orc_bf16_decode(c->x[i * c->hidden + j]) * c->rstd[i]);
        c->dweight[j] = dw;
    }
}

int orc_rmsnorm_bwd(const uint16_t* dy, const uint16_t* x, const uint16_t* w,
                    const uint16_t* dres, int64_t rows, int64_t hidden, double eps,
                    double* dx, double* dweight, double* rstd_out, int nthreads) {
    if (bad_common(rows, hidden, eps) || !dweight) return -1;
    if (rows == 0) {
        for (int64_t j = 0; j < hidden; ++j) dweight[j] = 0.0;
        return 0;
    }
    if (!dy || !x || !w || !dx) return -1;
    double* rstd = rstd_out ? rstd_out : (double*)malloc((size_t)rows * sizeof(double));
    if (!rstd) return -1;
    rmsb_ctx c = {dy, x, w, dres, rows, hidden, eps, dx, dweight, rstd};
    parallel_ranges(rmsb_rows, &c, rows, nthreads);
    parallel_ranges(rmsb_cols, &c, hidden, nthreads);
    if (!rstd_out) free(rstd);
    return 0;
}
