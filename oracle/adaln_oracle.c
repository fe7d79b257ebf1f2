/*
 * Oracle for the fused AdaLN (LayerNorm-Modulate) operator and for the
 * dual-constraint bucket sizing rule.  TEST INFRASTRUCTURE ONLY: the parity
 * tests, the smoke check and the CPU-baseline leg of the benchmark call it;
 * the GPU path never does.  It shares no code, header or constant with the
 * HIP library.
 *
 * Source: the AdaptiveLoad technical summary pages (gist.science, arXiv
 * 2605.17923), "Methodology" section:
 *   - part A (dual-constraint adaptive load balancing): the bucket batch is
 *     the larger of 1 and the smaller of the memory bound floor(M_mem / S)
 *     and the compute bound floor(M_comp / S^p);
 *   - part B (fused LayerNorm-Modulate kernels): the forward pass normalises
 *     each token row over the feature dimension D with its mean and variance
 *     and then applies the modulation; in the backward pass the gradients of
 *     the modulation parameters are reductions along the sequence dimension N.
 *
 * The pages do not print the formula.  This file takes the plainest reading
 * that the rest of the pages supports (LayerNorm without affine, biased
 * variance, eps inside the square root, per-sample modulation vectors):
 *
 *     mu    = (1/D) sum_d x[d]
 *     var   = (1/D) sum_d (x[d] - mu)^2
 *     rstd  = 1 / sqrt(var + eps)
 *     xhat  = (x - mu) * rstd
 *     y     = xhat * (1 + scale[b]) + shift[b]
 *
 * and its exact gradient for a loss L with dL/dy = dy:
 *
 *     g       = dy * (1 + scale[b])
 *     dx      = rstd * (g - mean_d(g) - xhat * mean_d(g * xhat))
 *     dscale  = sum_n dy * xhat          (per sample b and feature d)
 *     dshift  = sum_n dy
 *
 * All arithmetic, inputs and outputs are IEEE double precision (every
 * bfloat16 and float32 input value converts to double exactly).
 * Rows are independent; OpenMP only splits independent rows (or independent
 * features for the sums over N), so every sum is taken in its natural index
 * order and the results do not depend on the thread count.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC (no -ffast-math: no reassociation).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Dual-constraint bucket batch size (section 2.A, the intersection of the
 * linear memory constraint B*S <= M_mem and the polynomial compute constraint
 * B*S^p <= M_comp, floored, at least 1).  Integer arithmetic throughout.
 * Returns -1 for S <= 0 or negative bounds / exponent.  When S^p exceeds the
 * int64 range the compute bound is 0, so the result is 1. */
int64_t oracle_bshape(int64_t S, int64_t m_mem, int64_t m_comp, int32_t p)
{
    if (S <= 0 || m_mem < 0 || m_comp < 0 || p < 0)
        return -1;
    int64_t mem_bound = m_mem / S;

    int64_t s_pow_p = 1;
    int overflow = 0;
    for (int32_t i = 0; i < p; ++i) {
        if (s_pow_p > INT64_MAX / S) {
            overflow = 1;
            break;
        }
        s_pow_p *= S;
    }
    int64_t comp_bound = overflow ? 0 : m_comp / s_pow_p;

    int64_t b = mem_bound < comp_bound ? mem_bound : comp_bound;
    return b > 1 ? b : 1;
}

/* Mean and reciprocal standard deviation of one token row (section 2.B,
 * forward pass: the row's mean and variance over the feature dimension).
 * Two passes: the mean first, then the centred sum of squares. */
static void row_stats(const double *xr, int64_t D, double eps,
                      double *mean_out, double *rstd_out)
{
    double sum = 0.0;
    for (int64_t d = 0; d < D; ++d)
        sum += xr[d];
    double mu = sum / (double)D;

    double sq = 0.0;
    for (int64_t d = 0; d < D; ++d) {
        double c = xr[d] - mu;
        sq += c * c;
    }
    double var = sq / (double)D;

    *mean_out = mu;
    *rstd_out = 1.0 / sqrt(var + eps);
}

/* Forward: y = xhat * (1 + scale[b]) + shift[b] for every token row.
 * x: [B, N, D]; scale, shift: [B, D]; y: [B, N, D] (may be NULL);
 * mean, rstd: [B, N] (each may be NULL). */
void oracle_fwd(const double *x, const double *scale, const double *shift,
                int64_t B, int64_t N, int64_t D, double eps,
                double *y, double *mean, double *rstd)
{
    int64_t rows = B * N;
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < rows; ++row) {
        int64_t b = row / N;
        const double *xr = x + row * D;
        double mu, r;
        row_stats(xr, D, eps, &mu, &r);
        if (mean)
            mean[row] = mu;
        if (rstd)
            rstd[row] = r;
        if (y) {
            for (int64_t d = 0; d < D; ++d) {
                double xhat = (xr[d] - mu) * r;
                y[row * D + d] = xhat * (1.0 + scale[b * D + d])
                                 + shift[b * D + d];
            }
        }
    }
}

/* Backward of the forward above, for upstream gradient dy: [B, N, D].
 * dx: [B, N, D] (may be NULL); dscale, dshift: [B, D] (each may be NULL).
 * The statistics are recomputed from x in double precision. */
void oracle_bwd(const double *dy, const double *x, const double *scale,
                int64_t B, int64_t N, int64_t D, double eps,
                double *dx, double *dscale, double *dshift)
{
    int64_t rows = B * N;
    double *mu = (double *)malloc(sizeof(double) * (size_t)(rows > 0 ? rows : 1));
    double *r = (double *)malloc(sizeof(double) * (size_t)(rows > 0 ? rows : 1));
    if (!mu || !r)
        abort(); /* out of host memory: no result is better than a wrong one */

#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < rows; ++row)
        row_stats(x + row * D, D, eps, &mu[row], &r[row]);

    /* dx: the gradient of the normalisation, row by row. */
    if (dx) {
#pragma omp parallel for schedule(static)
        for (int64_t row = 0; row < rows; ++row) {
            int64_t b = row / N;
            const double *xr = x + row * D;
            const double *gr = dy + row * D;
            double sum_g = 0.0, sum_gx = 0.0;
            for (int64_t d = 0; d < D; ++d) {
                double g = gr[d] * (1.0 + scale[b * D + d]);
                double xhat = (xr[d] - mu[row]) * r[row];
                sum_g += g;
                sum_gx += g * xhat;
            }
            double c1 = sum_g / (double)D;
            double c2 = sum_gx / (double)D;
            for (int64_t d = 0; d < D; ++d) {
                double g = gr[d] * (1.0 + scale[b * D + d]);
                double xhat = (xr[d] - mu[row]) * r[row];
                dx[row * D + d] = r[row] * (g - c1 - xhat * c2);
            }
        }
    }

    /* dscale, dshift: per (sample, feature), sums over the N tokens of the
     * sample in order n = 0, 1, ..., N-1.  Threads split the features; each
     * walks the rows and keeps one running sum per feature it owns. */
    if (dscale || dshift) {
        const int64_t FB = 64; /* features per work item */
        int64_t nfb = (D + FB - 1) / FB;
#pragma omp parallel for schedule(static) collapse(2)
        for (int64_t b = 0; b < B; ++b) {
            for (int64_t fb = 0; fb < nfb; ++fb) {
                double acc_s[64], acc_h[64];
                int64_t d0 = fb * FB;
                int64_t nd = (D - d0) < FB ? (D - d0) : FB;
                for (int64_t j = 0; j < nd; ++j) {
                    acc_s[j] = 0.0;
                    acc_h[j] = 0.0;
                }
                for (int64_t n = 0; n < N; ++n) {
                    int64_t row = b * N + n;
                    for (int64_t j = 0; j < nd; ++j) {
                        int64_t d = d0 + j;
                        double g = dy[row * D + d];
                        double xhat = (x[row * D + d] - mu[row]) * r[row];
                        acc_s[j] += g * xhat;
                        acc_h[j] += g;
                    }
                }
                for (int64_t j = 0; j < nd; ++j) {
                    if (dscale)
                        dscale[b * D + d0 + j] = acc_s[j];
                    if (dshift)
                        dshift[b * D + d0 + j] = acc_h[j];
                }
            }
        }
    }

    free(mu);
    free(r);
}

/* Packed variable-length layout (the unpadded mixed-length batches of
 * section 2.A, and the separately modulated text and video token segments of
 * MMDiT samples): the token rows of nseg segments lie back to back in one
 * [T, D] array, segment s being rows off[s] .. off[s+1]-1 with off[0] = 0 and
 * T = off[nseg], and segment s is modulated by vector mod[s] of scale, shift:
 * [nmod, D] (mod == NULL: vector s).  Each row is normalised and modulated
 * exactly as in oracle_fwd; the caller guarantees a valid table. */
static int64_t seg_mod_of(const int32_t *mod, int64_t s)
{
    return mod ? (int64_t)mod[s] : s;
}

void oracle_fwd_segments(const double *x, const double *scale,
                         const double *shift, const int64_t *off,
                         const int32_t *mod, int64_t nseg, int64_t D,
                         double eps, double *y, double *mean, double *rstd)
{
    for (int64_t s = 0; s < nseg; ++s) {
        int64_t m = seg_mod_of(mod, s);
#pragma omp parallel for schedule(static)
        for (int64_t row = off[s]; row < off[s + 1]; ++row) {
            const double *xr = x + row * D;
            double mu, r;
            row_stats(xr, D, eps, &mu, &r);
            if (mean)
                mean[row] = mu;
            if (rstd)
                rstd[row] = r;
            if (y) {
                for (int64_t d = 0; d < D; ++d) {
                    double xhat = (xr[d] - mu) * r;
                    y[row * D + d] = xhat * (1.0 + scale[m * D + d])
                                     + shift[m * D + d];
                }
            }
        }
    }
}

/* Backward of oracle_fwd_segments.  dx as in oracle_bwd, row by row with the
 * row's segment's scale; dscale[m] and dshift[m] sum dy * xhat and dy over
 * the rows of every segment s with mod[s] == m, segments in index order and
 * rows in order within each (zero where no segment uses m). */
void oracle_bwd_segments(const double *dy, const double *x,
                         const double *scale, const int64_t *off,
                         const int32_t *mod, int64_t nseg, int64_t nmod,
                         int64_t D, double eps, double *dx, double *dscale,
                         double *dshift)
{
    int64_t rows = nseg > 0 ? off[nseg] : 0;
    double *mu = (double *)malloc(sizeof(double) * (size_t)(rows > 0 ? rows : 1));
    double *r = (double *)malloc(sizeof(double) * (size_t)(rows > 0 ? rows : 1));
    if (!mu || !r)
        abort();

#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < rows; ++row)
        row_stats(x + row * D, D, eps, &mu[row], &r[row]);

    if (dx) {
        for (int64_t s = 0; s < nseg; ++s) {
            int64_t m = seg_mod_of(mod, s);
#pragma omp parallel for schedule(static)
            for (int64_t row = off[s]; row < off[s + 1]; ++row) {
                const double *xr = x + row * D;
                const double *gr = dy + row * D;
                double sum_g = 0.0, sum_gx = 0.0;
                for (int64_t d = 0; d < D; ++d) {
                    double g = gr[d] * (1.0 + scale[m * D + d]);
                    double xhat = (xr[d] - mu[row]) * r[row];
                    sum_g += g;
                    sum_gx += g * xhat;
                }
                double c1 = sum_g / (double)D;
                double c2 = sum_gx / (double)D;
                for (int64_t d = 0; d < D; ++d) {
                    double g = gr[d] * (1.0 + scale[m * D + d]);
                    double xhat = (xr[d] - mu[row]) * r[row];
                    dx[row * D + d] = r[row] * (g - c1 - xhat * c2);
                }
            }
        }
    }

    if (dscale || dshift) {
        /* one (modulation vector, block of 64 features) pair per work item;
         * each walks the rows of the segments that use the vector and keeps
         * one running sum per feature it owns */
        const int64_t FB = 64;
        int64_t nfb = (D + FB - 1) / FB;
#pragma omp parallel for schedule(static) collapse(2)
        for (int64_t m = 0; m < nmod; ++m) {
            for (int64_t fb = 0; fb < nfb; ++fb) {
                double acc_s[64], acc_h[64];
                int64_t d0 = fb * FB;
                int64_t nd = (D - d0) < FB ? (D - d0) : FB;
                for (int64_t j = 0; j < nd; ++j) {
                    acc_s[j] = 0.0;
                    acc_h[j] = 0.0;
                }
                for (int64_t s = 0; s < nseg; ++s) {
                    if (seg_mod_of(mod, s) != m)
                        continue;
                    for (int64_t row = off[s]; row < off[s + 1]; ++row) {
                        for (int64_t j = 0; j < nd; ++j) {
                            int64_t d = d0 + j;
                            double g = dy[row * D + d];
                            double xhat = (x[row * D + d] - mu[row]) * r[row];
                            acc_s[j] += g * xhat;
                            acc_h[j] += g;
                        }
                    }
                }
                for (int64_t j = 0; j < nd; ++j) {
                    if (dscale)
                        dscale[m * D + d0 + j] = acc_s[j];
                    if (dshift)
                        dshift[m * D + d0 + j] = acc_h[j];
                }
            }
        }
    }

    free(mu);
    free(r);
}

/* Number of threads an OpenMP parallel region of this library uses. */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Set the thread count for the following calls (n <= 0 leaves it alone). */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}
