// Host side of the dual-constraint bucket scheduler (AdaptiveLoad technical
// summary, section 2.A, cost-fitting system): the step-time model
// t = a + b * B * S^p fitted to measured (B, S, t) samples by least squares,
// and the bucket batch size with a real exponent and compute bound.  No HIP
// call is made here.
//
// The fit is a variable projection: for a fixed exponent p the model is
// linear in (a, b), whose least-squares values have a closed form; what is
// left is a one-dimensional search of the residual over p -- a scan of a
// uniform grid to bracket the global minimum, then golden-section search
// inside the bracket.
#include <math.h>
#include <stdint.h>

#include "adaln.h"
#include "launch.hpp"

#define ADALN_API extern "C" __attribute__((visibility("default")))

namespace adaln {
namespace {

struct LinFit {
  double a, b, rss;
};

// Least-squares (a, b) of t = a + b * x for x_i = B_i * S_i^p.  The x are
// divided by their largest value first so that the centred sums stay well
// scaled for any p.
LinFit fit_at(const double *B, const double *S, const double *t, int64_t n,
              double p) {
  double xmax = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    const double x = B[i] * pow(S[i], p);
    if (x > xmax) xmax = x;
  }
  double xm = 0.0, tm = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    xm += B[i] * pow(S[i], p) / xmax;
    tm += t[i];
  }
  xm /= (double)n;
  tm /= (double)n;
  double sxx = 0.0, sxt = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    const double dx = B[i] * pow(S[i], p) / xmax - xm;
    sxx += dx * dx;
    sxt += dx * (t[i] - tm);
  }
  LinFit f;
  const double bs = sxx > 0.0 ? sxt / sxx : 0.0;  // slope in scaled units
  f.b = bs / xmax;
  f.a = tm - bs * xm;
  f.rss = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    const double r = t[i] - (f.a + bs * (B[i] * pow(S[i], p) / xmax));
    f.rss += r * r;
  }
  return f;
}

constexpr int kGrid = 400;  // grid intervals of the bracketing scan

}  // namespace

}  // namespace adaln

using namespace adaln;

ADALN_API int adaln_costfit(const double *B, const double *S, const double *t,
                            int64_t n, double p_lo, double p_hi, double *out) {
  if (B == nullptr || S == nullptr || t == nullptr || out == nullptr)
    return fail(ADALN_ERR_INVALID, "costfit: NULL array");
  if (n < 3) return fail(ADALN_ERR_INVALID, "costfit needs at least 3 samples");
  if (!(isfinite(p_lo) && isfinite(p_hi) && p_lo < p_hi))
    return fail(ADALN_ERR_INVALID, "costfit needs finite p_lo < p_hi");
  for (int64_t i = 0; i < n; ++i)
    if (!(B[i] > 0.0 && S[i] > 0.0 && isfinite(B[i]) && isfinite(S[i]) &&
          isfinite(t[i])))
      return fail(ADALN_ERR_INVALID,
                  "costfit sample %lld: B and S must be positive, t finite",
                  (long long)i);
  // bracket: the best grid point and its two neighbours
  const double h = (p_hi - p_lo) / kGrid;
  int best = 0;
  double best_rss = INFINITY;
  for (int k = 0; k <= kGrid; ++k) {
    const double r = fit_at(B, S, t, n, p_lo + k * h).rss;
    if (r < best_rss) {
      best_rss = r;
      best = k;
    }
  }
  double lo = p_lo + (best > 0 ? best - 1 : 0) * h;
  double hi = p_lo + (best < kGrid ? best + 1 : kGrid) * h;
  // golden-section search inside the bracket
  const double g = 0.5 * (sqrt(5.0) - 1.0);
  double c = hi - g * (hi - lo), d = lo + g * (hi - lo);
  double fc = fit_at(B, S, t, n, c).rss, fd = fit_at(B, S, t, n, d).rss;
  for (int it = 0; it < 200 && hi - lo > 1e-13 * (1.0 + fabs(lo)); ++it) {
    if (fc <= fd) {
      hi = d;
      d = c;
      fd = fc;
      c = hi - g * (hi - lo);
      fc = fit_at(B, S, t, n, c).rss;
    } else {
      lo = c;
      c = d;
      fc = fd;
      d = lo + g * (hi - lo);
      fd = fit_at(B, S, t, n, d).rss;
    }
  }
  double p = 0.5 * (lo + hi);
  LinFit f = fit_at(B, S, t, n, p);
  // keep the grid point if the refinement did not improve on it (a minimum
  // at an end of the range)
  if (best_rss < f.rss) {
    p = p_lo + best * h;
    f = fit_at(B, S, t, n, p);
  }
  out[0] = f.a;
  out[1] = f.b;
  out[2] = p;
  out[3] = f.rss;
  return ok();
}

ADALN_API int64_t adaln_bshape_real(int64_t S, int64_t m_mem, double m_comp,
                                    double p) {
  if (S <= 0 || m_mem < 0 || !(m_comp >= 0.0) || !(p >= 0.0) ||
      !isfinite(m_comp) || !isfinite(p))
    return fail(ADALN_ERR_INVALID,
                "bshape_real needs S > 0, non-negative bounds and exponent");
  const double q = floor(m_comp / pow((double)S, p));
  const int64_t by_memory = m_mem / S;
  const int64_t by_compute =
      q >= (double)INT64_MAX ? INT64_MAX : (int64_t)q;
  const int64_t b = by_memory < by_compute ? by_memory : by_compute;
  ok();
  return b < 1 ? 1 : b;
}

ADALN_API double adaln_mcomp(double p, int64_t m_mem, int64_t s_ref) {
  if (s_ref <= 0 || m_mem < 0 || !(p >= 0.0) || !isfinite(p)) {
    fail(ADALN_ERR_INVALID,
         "mcomp needs s_ref > 0, m_mem >= 0 and a finite exponent >= 0");
    return -1.0;
  }
  // the memory-bound batch of the reference length, times its S^p
  const int64_t b_mem = m_mem / s_ref;
  ok();
  return (double)b_mem * pow((double)s_ref, p);
}
