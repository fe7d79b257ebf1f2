"""Oracle of the scheduler's host-side arithmetic (AdaptiveLoad technical
summary pages, section 2.A "dual-constraint adaptive load balancing", the
cost-fitting system): the step-time model t = a + b * B * S^p fitted to
measured (B, S, t) samples by nonlinear least squares, and the bucket batch
size with a real exponent and compute bound.

TEST INFRASTRUCTURE ONLY: the tests call it; the library never does, and it
imports nothing from the library.

The fit minimises sum_i (t_i - a - b * B_i * S_i^p)^2 over (a, b, p) with
p in [p_lo, p_hi], in two library steps: a dense grid over p, where each
point's (a, b) is a linear least-squares solve (numpy.linalg.lstsq), picks a
start; scipy.optimize.least_squares then refines all three parameters
together (trust-region reflective, bounds on p).  B * S^p is divided by its
value at the start's p so that the slope is of order one.
"""

from __future__ import annotations

import math

import numpy as np


def model(a: float, b: float, p: float, B, S) -> np.ndarray:
    """Predicted step time a + b * B * S^p."""
    return a + b * np.asarray(B, float) * np.asarray(S, float) ** p


def rss(a: float, b: float, p: float, B, S, t) -> float:
    """Residual sum of squares of the model on the samples."""
    r = np.asarray(t, float) - model(a, b, p, B, S)
    return float(r @ r)


def linear_fit(B, S, t, p: float):
    """Least-squares (a, b) for a fixed exponent p, and its residual."""
    x = np.asarray(B, float) * np.asarray(S, float) ** p
    t = np.asarray(t, float)
    A = np.stack([np.ones_like(x), x / x.max()], axis=1)
    coef, *_ = np.linalg.lstsq(A, t, rcond=None)
    a, bs = coef
    b = bs / x.max()
    return float(a), float(b), rss(a, b, p, B, S, t)


def fit(B, S, t, p_lo: float = 0.5, p_hi: float = 3.0, grid: int = 2000):
    """Returns (a, b, p, rss) of the least-squares fit with p in
    [p_lo, p_hi]."""
    from scipy.optimize import least_squares
    B = np.asarray(B, float)
    S = np.asarray(S, float)
    t = np.asarray(t, float)
    ps = np.linspace(p_lo, p_hi, grid + 1)
    fits = [linear_fit(B, S, t, p) for p in ps]
    k = int(np.argmin([f[2] for f in fits]))
    a0, b0, _ = fits[k]
    p0 = float(ps[k])
    x0 = B * S ** p0
    scale = float(x0.max())

    def resid(v):
        a, bs, p = v
        return t - (a + bs * (B * S ** p) / scale)

    sol = least_squares(resid, [a0, b0 * scale, p0],
                        bounds=([-np.inf, -np.inf, p_lo],
                                [np.inf, np.inf, p_hi]),
                        xtol=1e-15, ftol=1e-15, gtol=1e-15, max_nfev=10000)
    a, bs, p = (float(v) for v in sol.x)
    b = bs / scale
    r = rss(a, b, p, B, S, t)
    if fits[k][2] < r:  # the grid start was already better
        a, b, p, r = a0, b0, p0, fits[k][2]
    return a, b, p, r


def bshape_real(S: int, m_mem: int, m_comp: float, p: float) -> int:
    """max(1, min(m_mem // S, floor(m_comp / S^p))), the compute bound from
    the double-precision quotient."""
    if S <= 0 or m_mem < 0 or not (m_comp >= 0) or not (p >= 0):
        return -1
    q = math.floor(m_comp / math.pow(float(S), p))
    return max(1, min(m_mem // S, q))


def m_comp(p: float, m_mem: int, s_ref: int) -> float:
    """Compute bound implied by an exponent p: the B * S^p of the
    memory-bound bucket of the reference length s_ref (the reading of how
    section 2.A's M_comp follows from the fit), floor(m_mem / s_ref) *
    s_ref^p; -1.0 for invalid arguments."""
    if s_ref <= 0 or m_mem < 0 or not (p >= 0) or not math.isfinite(p):
        return -1.0
    return float(m_mem // s_ref) * math.pow(float(s_ref), p)
