/*
 * Row-by-row comparison of a device result with the oracle.  TEST
 * INFRASTRUCTURE ONLY: the parity tests call it to compare every token row of
 * the large workloads, which the comparison in Python (float64 arrays of the
 * whole output) cannot do in seconds.
 *
 * It holds none of the method's arithmetic: every reference value comes from
 * oracle_fwd and oracle_bwd (adaln_oracle.c), called on one token row at a
 * time.  What it adds is the bookkeeping of the tolerances the tests state:
 * per element it forms the error |g - r| of a device value g against the
 * oracle's r and folds it into a few running maxima and sums, from which the
 * caller decides pass or fail:
 *
 *   max_ratio   max of err / (atol + rtol * |r|)          (a bound per element)
 *   max_excess  max of err - rel * |r|                    (compare with a
 *                                                          floor times the rms)
 *   max_above   max of err over elements with err > rel * |r|, else 0
 *   sum_sq_err, sum_sq_ref                                (normwise error, rms)
 *
 * For mean the per-element bound is rtol_stat * max(|r|, rms of the row's
 * x); for rstd it is rtol_stat * |r|.  Inputs and device outputs are passed
 * in their storage type (float32, or bfloat16 as raw 16-bit words); each value
 * is widened to double exactly.
 *
 * Build: compiled into liboracle.so with adaln_oracle.c (gcc -O2 -fopenmp).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

void oracle_fwd(const double *x, const double *scale, const double *shift,
                int64_t B, int64_t N, int64_t D, double eps,
                double *y, double *mean, double *rstd);
void oracle_bwd(const double *dy, const double *x, const double *scale,
                int64_t B, int64_t N, int64_t D, double eps,
                double *dx, double *dscale, double *dshift);

typedef struct {
    int64_t n;          /* elements compared */
    int64_t nonfinite;  /* device values that are NaN or infinite */
    int64_t over_atol;  /* elements with err > atol */
    double max_err;
    double max_ratio;
    double max_excess;
    double max_above;
    double sum_sq_err;
    double sum_sq_ref;
} check_stat;

/* Storage codes: 0 = float32, 1 = bfloat16.  Widens n values starting at
 * element i of `base` into out. */
static void widen(const void *base, int dtype, int64_t i, int64_t n,
                  double *out)
{
    if (dtype == 1) {
        const uint16_t *h = (const uint16_t *)base + i;
        for (int64_t k = 0; k < n; ++k) {
            uint32_t w = (uint32_t)h[k] << 16;
            float f;
            memcpy(&f, &w, sizeof f);
            out[k] = (double)f;
        }
    } else {
        const float *f = (const float *)base + i;
        for (int64_t k = 0; k < n; ++k)
            out[k] = (double)f[k];
    }
}

static void stat_init(check_stat *s)
{
    memset(s, 0, sizeof *s);
    s->max_excess = -INFINITY;
}

static void stat_merge(check_stat *into, const check_stat *s)
{
    into->n += s->n;
    into->nonfinite += s->nonfinite;
    into->over_atol += s->over_atol;
    if (s->max_err > into->max_err) into->max_err = s->max_err;
    if (s->max_ratio > into->max_ratio) into->max_ratio = s->max_ratio;
    if (s->max_excess > into->max_excess) into->max_excess = s->max_excess;
    if (s->max_above > into->max_above) into->max_above = s->max_above;
    into->sum_sq_err += s->sum_sq_err;
    into->sum_sq_ref += s->sum_sq_ref;
}

/* Folds one element: device value g, oracle value r, per-element bound
 * `allowed` (for max_ratio) and relative part `rel` (for max_excess and
 * max_above). */
static void fold(check_stat *s, double g, double r, double allowed,
                 double rel, double atol)
{
    s->n += 1;
    if (!isfinite(g)) {
        s->nonfinite += 1;
        return;
    }
    double err = fabs(g - r);
    if (err > s->max_err) s->max_err = err;
    if (err > atol) s->over_atol += 1;
    double ratio = allowed > 0.0 ? err / allowed : (err > 0.0 ? INFINITY : 0.0);
    if (ratio > s->max_ratio) s->max_ratio = ratio;
    double ex = err - rel * fabs(r);
    if (ex > s->max_excess) s->max_excess = ex;
    if (ex > 0.0 && err > s->max_above) s->max_above = err;
    s->sum_sq_err += (g - r) * (g - r);
    s->sum_sq_ref += r * r;
}

/*
 * Compares rows [row0, row0 + nrows) of a [T, D] result with the oracle.
 *   dtype          storage of x, dy, scale, shift, y, dx (0 f32, 1 bf16)
 *   x, dy          [T, D] inputs
 *   scale, shift   [nmod, D] modulation vectors
 *   row_mod        int64 [T]: vector of each row, or NULL: vector row / N
 *   N              rows per sample when row_mod is NULL
 *   y, dx          [T, D] device outputs (either may be NULL: not compared)
 *   mean, rstd     [T] float32 device outputs (either may be NULL)
 *   tol            {atol, rtol, rel, rtol_stat}
 *   out            check_stat[4]: y, dx, mean, rstd
 * Returns 0, or -1 when host memory runs out.
 */
int check_rows(int dtype, const void *x, const void *dy, const void *scale,
               const void *shift, const int64_t *row_mod, int64_t N,
               int64_t D, int64_t row0, int64_t nrows, const void *y,
               const void *dx, const float *mean, const float *rstd,
               const double *tol, double eps, check_stat *out)
{
    const double atol = tol[0], rtol = tol[1], rel = tol[2],
                 rtol_stat = tol[3];
    int failed = 0;
    for (int k = 0; k < 4; ++k)
        stat_init(&out[k]);

#pragma omp parallel
    {
        double *buf = (double *)malloc(sizeof(double) * (size_t)D * 8);
        check_stat loc[4];
        for (int k = 0; k < 4; ++k)
            stat_init(&loc[k]);
        if (!buf) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t row = row0; row < row0 + nrows; ++row) {
            if (!buf)
                continue;
            double *xr = buf, *gr = buf + D, *sr = buf + 2 * D,
                   *hr = buf + 3 * D, *yr = buf + 4 * D, *dxr = buf + 5 * D,
                   *yg = buf + 6 * D, *dxg = buf + 7 * D;
            const int64_t m = row_mod ? row_mod[row] : row / N;
            widen(x, dtype, row * D, D, xr);
            widen(scale, dtype, m * D, D, sr);
            widen(shift, dtype, m * D, D, hr);
            double sq = 0.0;
            for (int64_t d = 0; d < D; ++d)
                sq += xr[d] * xr[d];
            double mu, r;
            oracle_fwd(xr, sr, hr, 1, 1, D, eps, yr, &mu, &r);
            if (y) {
                widen(y, dtype, row * D, D, yg);
                for (int64_t d = 0; d < D; ++d)
                    fold(&loc[0], yg[d], yr[d], atol + rtol * fabs(yr[d]),
                         rel, atol);
            }
            if (dx && dy) {
                widen(dy, dtype, row * D, D, gr);
                oracle_bwd(gr, xr, sr, 1, 1, D, eps, dxr, NULL, NULL);
                widen(dx, dtype, row * D, D, dxg);
                for (int64_t d = 0; d < D; ++d)
                    fold(&loc[1], dxg[d], dxr[d],
                         atol + rtol * fabs(dxr[d]), rel, atol);
            }
            if (mean) {
                double row_rms = sqrt(sq / (double)D);
                double floor_ = fabs(mu) > row_rms ? fabs(mu) : row_rms;
                fold(&loc[2], (double)mean[row], mu, rtol_stat * floor_,
                     rtol_stat, INFINITY);
            }
            if (rstd)
                fold(&loc[3], (double)rstd[row], r, rtol_stat * fabs(r),
                     rtol_stat, INFINITY);
        }
#pragma omp critical
        for (int k = 0; k < 4; ++k)
            stat_merge(&out[k], &loc[k]);
        free(buf);
    }
    return failed ? -1 : 0;
}
