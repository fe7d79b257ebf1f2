"""Parity helpers: run the HIP path and the oracle on the same seeded inputs
and compare them under the tolerances below.

Tolerances (per element; r = oracle value in float64, g = GPU value):

* float32 outputs (y, dx of float32 inputs): |g - r| <= 1e-5 * max(|r|, rms)
  where rms is the root mean square of the whole output tensor -- relative
  1e-5 with a scale floor, since cancellation leaves some entries near 0.
* bfloat16 outputs (y, dx of bfloat16 inputs), contract bound:
  |g - r| <= 2e-2 + (2^-8 + 2^-16) * |r|.  2e-2 absolute, widened by the
  half-ulp of bfloat16 (2^-8 relative) that correct rounding alone costs once
  |r| >= 8, plus float32 slack.  The count of elements over the plain 2e-2
  bound is reported.
* bfloat16 outputs, strict bound (checked too): |g - r| <= 2^-8 * |r| +
  1e-4 * rms, i.e. the stored value is the correctly rounded bfloat16 of a
  float32 result that lies within 1e-4 * rms of the exact one.  Without it
  the 2e-2 bound would be vacuous for dx, whose entries are about 1e-2.
* bfloat16 outputs, also reported: the normwise relative error
  ||g - r||_2 / ||r||_2, held to <= 1e-2 (bfloat16 rounding alone gives
  about 2e-3).
* dscale, dshift (float32 sums over N): |g - r| <= 1e-3 * max(|r|, rms).
* mean: |g - r| <= 1e-5 * max(|r|, rms of the row's x);
  rstd: |g - r| <= 1e-5 * |r|.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Optional, Sequence

import numpy as np
import torch

F32_RTOL = 1e-5
BF16_ATOL = 2e-2
BF16_RTOL = 2.0 ** -8 + 2.0 ** -16
STRICT_RTOL = 2.0 ** -8
STRICT_RMS = 1e-4
DMOD_RTOL = 1e-3
STAT_RTOL = 1e-5
NORMWISE_MAX = 1e-2


def _np(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def _rms(r: np.ndarray) -> float:
    return float(np.sqrt(np.mean(r * r))) if r.size else 0.0


@dataclass
class Report:
    name: str
    max_err: float
    max_ratio: float      # max over elements of err / allowed (<= 1 passes)
    over_plain: int = 0   # bf16: elements over the plain 2e-2 bound
    n: int = 0
    normwise: Optional[float] = None  # bf16: ||g - r|| / ||r||

    def __str__(self):
        s = (f"{self.name}: n={self.n} max_err={self.max_err:.3e} "
             f"worst/allowed={self.max_ratio:.3f}")
        if self.over_plain:
            s += f" over_2e-2={self.over_plain}"
        if self.normwise is not None:
            s += f" normwise={self.normwise:.2e}"
        return s


def _grade(name, g, r, allowed, over_plain=0) -> Report:
    err = np.abs(g - r)
    ratio = np.max(err / allowed) if err.size else 0.0
    rep = Report(name, float(err.max()) if err.size else 0.0, float(ratio),
                 over_plain, int(err.size))
    assert ratio <= 1.0, f"parity failure: {rep}"
    return rep


def check_out(name: str, got, ref, dtype: str) -> Sequence[Report]:
    """y or dx: float32 or bfloat16 rules."""
    g, r = _np(got), _np(ref)
    assert g.shape == r.shape, (name, g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{name}: non-finite GPU values"
    rms = _rms(r)
    if dtype == "f32":
        return [_grade(name, g, r, F32_RTOL * np.maximum(np.abs(r), rms))]
    over = int(np.sum(np.abs(g - r) > BF16_ATOL))
    a = _grade(name + "[contract]", g, r, BF16_ATOL + BF16_RTOL * np.abs(r),
               over)
    ref_norm = float(np.linalg.norm(r))
    if ref_norm > 0:
        a.normwise = float(np.linalg.norm(g - r)) / ref_norm
        assert a.normwise <= NORMWISE_MAX, f"parity failure: {a}"
    b = _grade(name + "[strict]", g, r,
               STRICT_RTOL * np.abs(r) + STRICT_RMS * rms + 1e-30)
    return [a, b]


def check_dmod(name: str, got, ref) -> Report:
    g, r = _np(got), _np(ref)
    assert g.shape == r.shape
    rms = _rms(r)
    return _grade(name, g, r, DMOD_RTOL * np.maximum(np.abs(r), rms) + 1e-30)


def check_stats(got_mean, got_rstd, ref_mean, ref_rstd, x_rows) -> Sequence[Report]:
    gm, rm = _np(got_mean), _np(ref_mean)
    gr, rr = _np(got_rstd), _np(ref_rstd)
    xr = _np(x_rows)
    row_rms = np.sqrt(np.mean(xr * xr, axis=-1))
    a = _grade("mean", gm, rm, STAT_RTOL * np.maximum(np.abs(rm), row_rms)
               + 1e-30)
    b = _grade("rstd", gr, rr, STAT_RTOL * np.abs(rr))
    return [a, b]


# ----------------------------------------------------------------- running

def to_device(inp, device="cuda"):
    return {k: (None if v is None else v.to(device))
            for k, v in (("x", inp.x), ("scale", inp.scale),
                         ("shift", inp.shift), ("dy", inp.dy))}


def gpu_fwd_bwd(dev: Dict[str, torch.Tensor], stream=None):
    """The HIP path as a caller runs it: adaln_fwd then adaln_bwd."""
    import adaln_fwd_amd as A
    y, mean, rstd = A.fwd(dev["x"], dev["scale"], dev["shift"], stream=stream)
    dx, dscale, dshift = A.bwd(dev["dy"], dev["x"], dev["scale"], mean, rstd,
                               stream=stream)
    return dict(y=y, mean=mean, rstd=rstd, dx=dx, dscale=dscale,
                dshift=dshift)


def oracle_rows(inp, rows: np.ndarray):
    """Oracle forward and dx for the token rows `rows` (flat b*N + n)."""
    import oracle
    B, N, D = inp.x.shape
    rows = np.asarray(rows, dtype=np.int64)
    xr = inp.x.reshape(B * N, D)[torch.from_numpy(rows)].unsqueeze(1)
    gr = inp.dy.reshape(B * N, D)[torch.from_numpy(rows)].unsqueeze(1)
    bidx = torch.from_numpy(rows // N)
    s = inp.scale[bidx]
    h = inp.shift[bidx]
    y, mean, rstd = oracle.fwd(xr, s, h)
    dx, _, _ = oracle.bwd(gr, xr, s, want_dmod=False)
    return dict(y=y[:, 0], mean=mean[:, 0], rstd=rstd[:, 0], dx=dx[:, 0],
                x=xr[:, 0])


def compare_rows(inp, out, rows: np.ndarray, dtype: str):
    """Compare GPU outputs (CPU copies) on `rows` with the oracle."""
    B, N, D = inp.x.shape
    ref = oracle_rows(inp, rows)
    t = torch.from_numpy(np.asarray(rows, np.int64))
    reps = []
    reps += check_out("y", out["y"].reshape(B * N, D)[t], ref["y"], dtype)
    reps += check_out("dx", out["dx"].reshape(B * N, D)[t], ref["dx"], dtype)
    reps += check_stats(out["mean"].reshape(-1)[t], out["rstd"].reshape(-1)[t],
                        ref["mean"], ref["rstd"], ref["x"])
    return reps


def compare_full(inp, out, dtype: str, with_rows: bool = True):
    """Full element-by-element comparison (sizes the oracle finishes fast)."""
    import oracle
    reps = []
    if with_rows:
        y, mean, rstd = oracle.fwd(inp.x, inp.scale, inp.shift)
        dx, ds, dh = oracle.bwd(inp.dy, inp.x, inp.scale)
        reps += check_out("y", out["y"], y, dtype)
        reps += check_out("dx", out["dx"], dx, dtype)
        reps += check_stats(out["mean"], out["rstd"], mean, rstd, inp.x)
    else:
        _, ds, dh = oracle.bwd(inp.dy, inp.x, inp.scale, want_dx=False)
    reps.append(check_dmod("dscale", out["dscale"], ds))
    reps.append(check_dmod("dshift", out["dshift"], dh))
    return reps


def _tol(dtype: str):
    """(atol, rtol, rel, rtol_stat) of the row checker for y and dx."""
    if dtype == "f32":
        return (0.0, F32_RTOL, F32_RTOL, STAT_RTOL)
    return (BF16_ATOL, BF16_RTOL, STRICT_RTOL, STAT_RTOL)


def _grade_stat(name: str, st, dtype: str) -> Sequence[Report]:
    """Reports of one output of the row checker under the rules above.

    The bounds with a whole-tensor rms floor are decided from running
    quantities: an element fails ``err <= rel*|r| + f*rms`` (bf16 strict)
    exactly when ``max(err - rel*|r|) > f*rms``, and fails ``err <= rtol *
    max(|r|, rms)`` (float32) exactly when some element with err > rtol*|r|
    has err > rtol*rms.  Their worst/allowed figure is that maximum over the
    floor."""
    assert st.n > 0, f"{name}: nothing compared"
    assert st.nonfinite == 0, f"{name}: {st.nonfinite} non-finite GPU values"
    rms = float(np.sqrt(st.sum_sq_ref / st.n))
    if dtype == "f32":
        ratio = st.max_above / (F32_RTOL * rms) if st.max_above > 0 else 0.0
        rep = Report(name, st.max_err, ratio, 0, st.n)
        assert ratio <= 1.0, f"parity failure: {rep}"
        return [rep]
    a = Report(name + "[contract]", st.max_err, st.max_ratio, st.over_atol,
               st.n)
    assert a.max_ratio <= 1.0, f"parity failure: {a}"
    if st.sum_sq_ref > 0:
        a.normwise = float(np.sqrt(st.sum_sq_err / st.sum_sq_ref))
        assert a.normwise <= NORMWISE_MAX, f"parity failure: {a}"
    floor = STRICT_RMS * rms + 1e-30
    b = Report(name + "[strict]", st.max_err, max(st.max_excess, 0.0) / floor,
               0, st.n)
    assert b.max_ratio <= 1.0, f"parity failure: {b}"
    return [a, b]


def check_all_rows(x, dy, scale, shift, got, dtype: str, N: int = 1,
                   row_mod=None) -> Sequence[Report]:
    """Every token row of y, dx, mean and rstd (host copies in ``got``)
    against the oracle, through the oracle library's row checker; x, dy are
    [T, D] or [B, N, D] host tensors, row r modulated by vector row_mod[r]
    or r // N."""
    import oracle
    st = oracle.check_rows(x, dy, scale, shift, y=got["y"], dx=got["dx"],
                           mean=got["mean"], rstd=got["rstd"], N=N,
                           row_mod=row_mod, tol=_tol(dtype))
    reps = []
    reps += _grade_stat("y", st["y"], dtype)
    reps += _grade_stat("dx", st["dx"], dtype)
    for k in ("mean", "rstd"):
        s = st[k]
        assert s.nonfinite == 0, f"{k}: non-finite GPU values"
        rep = Report(k, s.max_err, s.max_ratio, 0, s.n)
        assert rep.max_ratio <= 1.0, f"parity failure: {rep}"
        reps.append(rep)
    return reps


def compare_all_rows(inp, out, dtype: str) -> Sequence[Report]:
    """Every row of a batched result (host copies) against the oracle."""
    B, N, D = inp.x.shape
    got = {k: out[k].contiguous() for k in ("y", "dx", "mean", "rstd")}
    return check_all_rows(inp.x, inp.dy, inp.scale, inp.shift, got, dtype,
                          N=N)


def sample_rows(total: int, k: int, seed: int = 0) -> np.ndarray:
    """k distinct rows: the first and last 8 plus a seeded random draw."""
    g = np.random.default_rng(seed)
    edge = np.r_[np.arange(min(8, total)), np.arange(max(0, total - 8), total)]
    rnd = g.choice(total, size=min(k, total), replace=False)
    return np.unique(np.r_[edge, rnd])


# ------------------------------------------------------- packed segments

def packed_to_device(inp, device="cuda"):
    return {k: (None if v is None else v.to(device))
            for k, v in (("x", inp.x), ("scale", inp.scale),
                         ("shift", inp.shift), ("dy", inp.dy))}


def gpu_packed(inp, dev: Dict[str, torch.Tensor], stream=None):
    """adaln_fwd_segments then adaln_bwd_segments on a packed layout."""
    import adaln_fwd_amd as A
    off, mod = inp.seg_offsets, inp.seg_mod
    y, mean, rstd = A.fwd_segments(dev["x"], dev["scale"], dev["shift"], off,
                                   mod, stream=stream)
    dx, dscale, dshift = A.bwd_segments(dev["dy"], dev["x"], dev["scale"],
                                        mean, rstd, off, mod, stream=stream)
    return dict(y=y, mean=mean, rstd=rstd, dx=dx, dscale=dscale,
                dshift=dshift)


def row_mods(inp) -> np.ndarray:
    """Modulation vector of every token row of a packed layout."""
    lengths = np.diff(inp.seg_offsets)
    idx = (np.arange(lengths.size) if inp.seg_mod is None
           else np.asarray(inp.seg_mod))
    return np.repeat(idx, lengths).astype(np.int64)


def compare_packed_full(inp, out, dtype: str, with_rows: bool = True):
    import oracle
    off, mod = inp.seg_offsets, inp.seg_mod
    reps = []
    if with_rows:
        y, mean, rstd = oracle.fwd_segments(inp.x, inp.scale, inp.shift, off,
                                            mod)
        dx, ds, dh = oracle.bwd_segments(inp.dy, inp.x, inp.scale, off, mod)
        reps += check_out("y", out["y"], y, dtype)
        reps += check_out("dx", out["dx"], dx, dtype)
        reps += check_stats(out["mean"], out["rstd"], mean, rstd, inp.x)
    else:
        _, ds, dh = oracle.bwd_segments(inp.dy, inp.x, inp.scale, off, mod,
                                        want_dx=False)
    reps.append(check_dmod("dscale", out["dscale"], ds))
    reps.append(check_dmod("dshift", out["dshift"], dh))
    return reps


def compare_packed_rows(inp, got, rows: np.ndarray, dtype: str):
    """GPU outputs on sampled rows of a packed layout (``got`` holds y, dx,
    mean and rstd of just those rows, in order) against the oracle, which
    takes each row as a one-row segment with its modulation vector."""
    import oracle
    rows = np.asarray(rows, dtype=np.int64)
    t = torch.from_numpy(rows)
    xr, gr = inp.x[t], inp.dy[t]
    mods = row_mods(inp)[rows].astype(np.int32)
    off = np.arange(rows.size + 1, dtype=np.int64)
    y, mean, rstd = oracle.fwd_segments(xr, inp.scale, inp.shift, off, mods)
    dx, _, _ = oracle.bwd_segments(gr, xr, inp.scale, off, mods,
                                   want_dmod=False)
    reps = []
    reps += check_out("y", got["y"], y, dtype)
    reps += check_out("dx", got["dx"], dx, dtype)
    reps += check_stats(got["mean"], got["rstd"], mean, rstd, xr)
    return reps
