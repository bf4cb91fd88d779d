/*
 * CPU oracle, fp32 activations -- TEST INFRASTRUCTURE ONLY.
 * The same definitions as oracle.c (see oracle.h) for operands given as
 * IEEE-754 binary32 values instead of bf16 patterns: every input is widened
 * to double exactly, every sum and product runs in double in the written
 * order, and normalized outputs are returned unrounded.  The fused op's
 * residual output is the exact sum x + r rounded once to binary32 (ties to
 * even): the double sum of two binary32 values is exact unless their
 * exponents differ by more than 29, and then the smaller one lies below a
 * quarter of a binary32 ulp of the larger, so both the exact and the double
 * sum round to the larger operand.  Build: gcc -O2, no fast-math, no
 * contraction (as oracle.c).
 */
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>

typedef void (*range_fn32)(const void* ctx, int64_t begin, int64_t end);

typedef struct {
    range_fn32 fn;
    const void* ctx;
    int64_t begin, end;
} range_job32;

static void* range_main32(void* p) {
    const range_job32* j = (const range_job32*)p;
    j->fn(j->ctx, j->begin, j->end);
    return NULL;
}

/* run fn over [0, n) in nthreads contiguous blocks */
static void ranges32(range_fn32 fn, const void* ctx, int64_t n, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > n) nthreads = (int)(n > 0 ? n : 1);
    if (nthreads == 1) {
        fn(ctx, 0, n);
        return;
    }
    pthread_t tid[256];
    range_job32 jobs[256];
    int started[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t].fn = fn;
        jobs[t].ctx = ctx;
        jobs[t].begin = n * t / nthreads;
        jobs[t].end = n * (t + 1) / nthreads;
        started[t] = pthread_create(&tid[t], NULL, range_main32, &jobs[t]) == 0;
        if (!started[t]) range_main32(&jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t)
        if (started[t]) pthread_join(tid[t], NULL);
}

static int bad_args32(int64_t rows, int64_t hidden, double eps) {
    return rows < 0 || hidden <= 0 || !(eps >= 0.0) || isinf(eps);
}

/* ---- RMSNorm forward, with and without the fused residual add ------------ */

typedef struct {
    const float *x, *r, *w; /* r == NULL: plain RMSNorm */
    int64_t hidden;
    double eps;
    double* out;
    float* res_out;
    double* rstd_out;
} rms32_ctx;

static void rms32_rows(const void* p, int64_t begin, int64_t end) {
    const rms32_ctx* c = (const rms32_ctx*)p;
    const int64_t H = c->hidden;
    double* s = (double*)malloc((size_t)H * sizeof(double));
    for (int64_t i = begin; i < end; ++i) {
        const int64_t base = i * H;
        for (int64_t j = 0; j < H; ++j) {
            double v = (double)c->x[base + j];
            if (c->r) v += (double)c->r[base + j];
            s[j] = v;
        }
        if (c->res_out)
            for (int64_t j = 0; j < H; ++j) c->res_out[base + j] = (float)s[j];
        double ss = 0.0;
        for (int64_t j = 0; j < H; ++j) ss += s[j] * s[j];
        const double rstd = 1.0 / sqrt(ss / (double)H + c->eps);
        if (c->rstd_out) c->rstd_out[i] = rstd;
        for (int64_t j = 0; j < H; ++j) c->out[base + j] = s[j] * rstd * (double)c->w[j];
    }
    free(s);
}

int orc_fused_add_rmsnorm_f32(const float* x, const float* r, const float* w, int64_t rows,
                              int64_t hidden, double eps, double* out, float* res_out,
                              double* rstd_out, int nthreads) {
    if (bad_args32(rows, hidden, eps)) return -1;
    if (rows == 0) return 0;
    if (!x || !r || !w || !out || !res_out) return -1;
    rms32_ctx c = {x, r, w, hidden, eps, out, res_out, rstd_out};
    ranges32(rms32_rows, &c, rows, nthreads);
    return 0;
}

int orc_rmsnorm_fwd_f32(const float* x, const float* w, int64_t rows, int64_t hidden,
                        double eps, double* out, double* rstd_out, int nthreads) {
    if (bad_args32(rows, hidden, eps)) return -1;
    if (rows == 0) return 0;
    if (!x || !w || !out) return -1;
    rms32_ctx c = {x, NULL, w, hidden, eps, out, NULL, rstd_out};
    ranges32(rms32_rows, &c, rows, nthreads);
    return 0;
}

/* ---- LayerNorm forward (two-pass statistics) ----------------------------- */

typedef struct {
    const float *x, *w, *b;
    int64_t hidden;
    double eps;
    double *y, *mean, *rstd;
} lnf32_ctx;

static void lnf32_rows(const void* p, int64_t begin, int64_t end) {
    const lnf32_ctx* c = (const lnf32_ctx*)p;
    const int64_t H = c->hidden;
    for (int64_t i = begin; i < end; ++i) {
        const float* xr = c->x + i * H;
        double sum = 0.0;
        for (int64_t j = 0; j < H; ++j) sum += (double)xr[j];
        const double mu = sum / (double)H;
        double sq = 0.0;
        for (int64_t j = 0; j < H; ++j) {
            const double d = (double)xr[j] - mu;
            sq += d * d;
        }
        const double rstd = 1.0 / sqrt(sq / (double)H + c->eps);
        c->mean[i] = mu;
        c->rstd[i] = rstd;
        for (int64_t j = 0; j < H; ++j)
            c->y[i * H + j] = ((double)xr[j] - mu) * rstd * (double)c->w[j] + (double)c->b[j];
    }
}

int orc_layernorm_fwd_f32(const float* x, const float* w, const float* b, int64_t rows,
                          int64_t hidden, double eps, double* y, double* mean, double* rstd,
                          int nthreads) {
    if (bad_args32(rows, hidden, eps)) return -1;
    if (rows == 0) return 0;
    if (!x || !w || !b || !y || !mean || !rstd) return -1;
    lnf32_ctx c = {x, w, b, hidden, eps, y, mean, rstd};
    ranges32(lnf32_rows, &c, rows, nthreads);
    return 0;
}

/* ---- LayerNorm backward, statistics given --------------------------------- */

typedef struct {
    const float *dy, *x, *w;
    const double *mean, *rstd;
    int64_t rows, hidden;
    double *dx, *dweight, *dbias;
} lnb32_ctx;

static double lnb32_xhat(const lnb32_ctx* c, int64_t i, int64_t j) {
    return ((double)c->x[i * c->hidden + j] - c->mean[i]) * c->rstd[i];
}

static void lnb32_rows(const void* p, int64_t begin, int64_t end) {
    const lnb32_ctx* c = (const lnb32_ctx*)p;
    const int64_t H = c->hidden;
    for (int64_t i = begin; i < end; ++i) {
        double sum_g = 0.0, sum_gx = 0.0;
        for (int64_t j = 0; j < H; ++j) {
            const double g = (double)c->dy[i * H + j] * (double)c->w[j];
            sum_g += g;
            sum_gx += g * lnb32_xhat(c, i, j);
        }
        const double c1 = sum_g / (double)H;
        const double c2 = sum_gx / (double)H;
        for (int64_t j = 0; j < H; ++j) {
            const double g = (double)c->dy[i * H + j] * (double)c->w[j];
            c->dx[i * H + j] = c->rstd[i] * (g - c1 - lnb32_xhat(c, i, j) * c2);
        }
    }
}

static void lnb32_cols(const void* p, int64_t begin, int64_t end) {
    const lnb32_ctx* c = (const lnb32_ctx*)p;
    for (int64_t j = begin; j < end; ++j) {
        double dw = 0.0, db = 0.0;
        for (int64_t i = 0; i < c->rows; ++i) {
            const double d = (double)c->dy[i * c->hidden + j];
            dw += d * lnb32_xhat(c, i, j);
            db += d;
        }
        c->dweight[j] = dw;
        c->dbias[j] = db;
    }
}

int orc_layernorm_bwd_f32(const float* dy, const float* x, const double* mean,
                          const double* rstd, const float* w, int64_t rows, int64_t hidden,
                          double* dx, double* dweight, double* dbias, int nthreads) {
    if (rows < 0 || hidden <= 0) return -1;
    if (!dweight || !dbias) return -1;
    if (rows == 0) {
        for (int64_t j = 0; j < hidden; ++j) dweight[j] = dbias[j] = 0.0;
        return 0;
    }
    if (!dy || !x || !mean || !rstd || !w || !dx) return -1;
    lnb32_ctx c = {dy, x, w, mean, rstd, rows, hidden, dx, dweight, dbias};
    ranges32(lnb32_rows, &c, rows, nthreads);
    ranges32(lnb32_cols, &c, hidden, nthreads);
    return 0;
}

/* ---- RMSNorm backward (and the fused op's), statistic recomputed ----------- */

typedef struct {
    const float *dy, *x, *w, *dres;
    int64_t rows, hidden;
    double eps;
    double *dx, *dweight, *rstd;
} rmsb32_ctx;

static void rmsb32_rows(const void* p, int64_t begin, int64_t end) {
    const rmsb32_ctx* c = (const rmsb32_ctx*)p;
    const int64_t H = c->hidden;
    for (int64_t i = begin; i < end; ++i) {
        double ss = 0.0;
        for (int64_t j = 0; j < H; ++j) {
            const double v = (double)c->x[i * H + j];
            ss += v * v;
        }
        const double rstd = 1.0 / sqrt(ss / (double)H + c->eps);
        c->rstd[i] = rstd;
        double sum_gx = 0.0;
        for (int64_t j = 0; j < H; ++j) {
            const double g = (double)c->dy[i * H + j] * (double)c->w[j];
            sum_gx += g * (double)c->x[i * H + j] * rstd;
        }
        const double cc = sum_gx / (double)H;
        for (int64_t j = 0; j < H; ++j) {
            const double g = (double)c->dy[i * H + j] * (double)c->w[j];
            const double xhat = (double)c->x[i * H + j] * rstd;
            double v = rstd * (g - xhat * cc);
            if (c->dres) v += (double)c->dres[i * H + j];
            c->dx[i * H + j] = v;
        }
    }
}

static void rmsb32_cols(const void* p, int64_t begin, int64_t end) {
    const rmsb32_ctx* c = (const rmsb32_ctx*)p;
    for (int64_t j = begin; j < end; ++j) {
        double dw = 0.0;
        for (int64_t i = 0; i < c->rows; ++i)
            dw += (double)c->dy[i * c->hidden + j] * ((double)c->x[i * c->hidden + j] * c->rstd[i]);
        c->dweight[j] = dw;
    }
}

int orc_rmsnorm_bwd_f32(const float* dy, const float* x, const float* w, const float* dres,
                        int64_t rows, int64_t hidden, double eps, double* dx, double* dweight,
                        double* rstd_out, int nthreads) {
    if (bad_args32(rows, hidden, eps) || !dweight) return -1;
    if (rows == 0) {
        for (int64_t j = 0; j < hidden; ++j) dweight[j] = 0.0;
        return 0;
    }
    if (!dy || !x || !w || !dx) return -1;
    double* rstd = rstd_out ? rstd_out : (double*)malloc((size_t)rows * sizeof(double));
    if (!rstd) return -1;
    rmsb32_ctx c = {dy, x, w, dres, rows, hidden, eps, dx, dweight, rstd};
    ranges32(rmsb32_rows, &c, rows, nthreads);
    ranges32(rmsb32_cols, &c, hidden, nthreads);
    if (!rstd_out) free(rstd);
    return 0;
}
