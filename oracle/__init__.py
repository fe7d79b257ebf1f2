"""Oracle of the fused AdaLN (LayerNorm-Modulate) operator: a plain,
double-precision CPU implementation written from the AdaptiveLoad technical
summary pages (gist.science, arXiv 2605.17923), section "Methodology", parts
A (dual-constraint bucket sizing) and B (fused LayerNorm-Modulate kernels).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may call it; the GPU path never imports it, and it imports
nothing from the GPU path.  The arithmetic lives in ``adaln_oracle.c``; this
module marshals arrays through ctypes.

Every function is pinned by ``tests/test_oracle.py`` to facts that do not come
from the oracle itself (a float64 library LayerNorm with autograd, central
finite differences, closed forms, hand-evaluated bucket sizes).
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np

from . import build as _build

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIB):
        _build.build()
    lib = ctypes.CDLL(_build.LIB)
    i64, f64, vp = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
    lib.oracle_bshape.argtypes = [i64, i64, i64, ctypes.c_int32]
    lib.oracle_bshape.restype = i64
    lib.oracle_fwd.argtypes = [vp, vp, vp, i64, i64, i64, f64, vp, vp, vp]
    lib.oracle_fwd.restype = None
    lib.oracle_bwd.argtypes = [vp, vp, vp, i64, i64, i64, f64, vp, vp, vp]
    lib.oracle_bwd.restype = None
    lib.oracle_fwd_segments.argtypes = [vp, vp, vp, vp, vp, i64, i64, f64,
                                        vp, vp, vp]
    lib.oracle_fwd_segments.restype = None
    lib.oracle_bwd_segments.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64,
                                        f64, vp, vp, vp]
    lib.oracle_bwd_segments.restype = None
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_num_threads.restype = None
    lib.check_rows.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, i64, i64,
                               i64, i64, vp, vp, vp, vp, vp, f64, vp]
    lib.check_rows.restype = ctypes.c_int
    _lib = lib
    return lib


def _f64(a) -> np.ndarray:
    """Float64 C-contiguous numpy copy of a numpy array or torch tensor.

    bfloat16, float32 and float64 values convert exactly."""
    if hasattr(a, "detach"):  # torch tensor
        import torch
        a = a.detach().to("cpu", torch.float64).contiguous().numpy()
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def bshape(S: int, m_mem: int, m_comp: int, p: int) -> int:
    """max(1, min(M_mem // S, M_comp // S**p)); -1 on invalid arguments."""
    return int(_load().oracle_bshape(int(S), int(m_mem), int(m_comp), int(p)))


def fwd(x, scale, shift, eps: float = 1e-6, want_y: bool = True
        ) -> Tuple[Optional[np.ndarray], np.ndarray, np.ndarray]:
    """Forward of AdaLN in float64.

    x: [B, N, D]; scale, shift: [B, D].  Returns (y [B,N,D] or None,
    mean [B,N], rstd [B,N]) as float64 arrays."""
    x, scale, shift = _f64(x), _f64(scale), _f64(shift)
    B, N, D = x.shape
    assert scale.shape == (B, D) and shift.shape == (B, D)
    y = np.empty((B, N, D), np.float64) if want_y else None
    mean = np.empty((B, N), np.float64)
    rstd = np.empty((B, N), np.float64)
    _load().oracle_fwd(_ptr(x), _ptr(scale), _ptr(shift), B, N, D,
                       float(eps), _ptr(y), _ptr(mean), _ptr(rstd))
    return y, mean, rstd


def bwd(dy, x, scale, eps: float = 1e-6, want_dx: bool = True,
        want_dmod: bool = True):
    """Backward of AdaLN in float64.

    Returns (dx [B,N,D] or None, dscale [B,D] or None, dshift [B,D] or None).
    """
    dy, x, scale = _f64(dy), _f64(x), _f64(scale)
    B, N, D = x.shape
    assert dy.shape == (B, N, D) and scale.shape == (B, D)
    dx = np.empty((B, N, D), np.float64) if want_dx else None
    dscale = np.empty((B, D), np.float64) if want_dmod else None
    dshift = np.empty((B, D), np.float64) if want_dmod else None
    _load().oracle_bwd(_ptr(dy), _ptr(x), _ptr(scale), B, N, D, float(eps),
                       _ptr(dx), _ptr(dscale), _ptr(dshift))
    return dx, dscale, dshift


def _segments(seg_offsets, seg_mod, T: int, nmod: int):
    off = np.ascontiguousarray(np.asarray(seg_offsets, dtype=np.int64))
    nseg = off.size - 1
    assert nseg >= 0 and off[0] == 0 and off[-1] == T
    assert np.all(np.diff(off) >= 0)
    mod = None
    if seg_mod is not None:
        mod = np.ascontiguousarray(np.asarray(seg_mod, dtype=np.int32))
        assert mod.shape == (nseg,)
        assert nseg == 0 or (mod.min() >= 0 and mod.max() < nmod)
    else:
        assert nseg <= nmod
    return off, mod, nseg


def fwd_segments(x, scale, shift, seg_offsets, seg_mod=None,
                 eps: float = 1e-6, want_y: bool = True):
    """Forward over a packed [T, D] array of segments; segment s is rows
    seg_offsets[s]..seg_offsets[s+1]-1, modulated by scale/shift[seg_mod[s]]
    (row s if seg_mod is None).  Returns (y [T,D] or None, mean [T],
    rstd [T]) in float64."""
    x, scale, shift = _f64(x), _f64(scale), _f64(shift)
    T, D = x.shape
    nmod = scale.shape[0]
    assert scale.shape == (nmod, D) and shift.shape == (nmod, D)
    off, mod, nseg = _segments(seg_offsets, seg_mod, T, nmod)
    y = np.empty((T, D), np.float64) if want_y else None
    mean = np.empty(T, np.float64)
    rstd = np.empty(T, np.float64)
    _load().oracle_fwd_segments(_ptr(x), _ptr(scale), _ptr(shift), _ptr(off),
                                _ptr(mod), nseg, D, float(eps), _ptr(y),
                                _ptr(mean), _ptr(rstd))
    return y, mean, rstd


def bwd_segments(dy, x, scale, seg_offsets, seg_mod=None, eps: float = 1e-6,
                 want_dx: bool = True, want_dmod: bool = True):
    """Backward of :func:`fwd_segments`.  Returns (dx [T,D] or None,
    dscale [nmod,D] or None, dshift [nmod,D] or None) in float64."""
    dy, x, scale = _f64(dy), _f64(x), _f64(scale)
    T, D = x.shape
    nmod = scale.shape[0]
    assert dy.shape == (T, D) and scale.shape == (nmod, D)
    off, mod, nseg = _segments(seg_offsets, seg_mod, T, nmod)
    dx = np.empty((T, D), np.float64) if want_dx else None
    dscale = np.empty((nmod, D), np.float64) if want_dmod else None
    dshift = np.empty((nmod, D), np.float64) if want_dmod else None
    _load().oracle_bwd_segments(_ptr(dy), _ptr(x), _ptr(scale), _ptr(off),
                                _ptr(mod), nseg, nmod, D, float(eps),
                                _ptr(dx), _ptr(dscale), _ptr(dshift))
    return dx, dscale, dshift


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    _load().oracle_set_num_threads(int(n))


class CheckStat(ctypes.Structure):
    """Running comparison of one output (``check_rows.c``)."""
    _fields_ = [("n", ctypes.c_int64), ("nonfinite", ctypes.c_int64),
                ("over_atol", ctypes.c_int64), ("max_err", ctypes.c_double),
                ("max_ratio", ctypes.c_double),
                ("max_excess", ctypes.c_double),
                ("max_above", ctypes.c_double),
                ("sum_sq_err", ctypes.c_double),
                ("sum_sq_ref", ctypes.c_double)]


def check_rows(x, dy, scale, shift, *, y=None, dx=None, mean=None,
               rstd=None, N: int = 1, row_mod=None, row0: int = 0,
               nrows: Optional[int] = None, tol=(0.0, 0.0, 0.0, 0.0),
               eps: float = 1e-6):
    """Compare device outputs (host copies) with the oracle, row by row.

    x, dy: [T, D] (or [B, N, D]) CPU tensors in float32 or bfloat16;
    scale, shift: [nmod, D] in the same dtype; y, dx: outputs of x's shape
    and dtype; mean, rstd: float32 [T].  Row r uses modulation vector
    row_mod[r] (int64 [T]) or, if row_mod is None, r // N.  tol =
    (atol, rtol, rel, rtol_stat), see ``check_rows.c``.  Returns a dict of
    CheckStat for "y", "dx", "mean" and "rstd" (n == 0 where not given)."""
    import torch

    def raw(t, dtype=None):
        if t is None:
            return None
        assert t.device.type == "cpu" and t.is_contiguous()
        if dtype is not None:
            assert t.dtype == dtype, (t.dtype, dtype)
        return t

    codes = {torch.float32: 0, torch.bfloat16: 1}
    dt = x.dtype
    code = codes[dt]
    D = x.shape[-1]
    T = x.numel() // D
    tensors = [raw(x, dt), raw(dy, dt), raw(scale, dt), raw(shift, dt),
               raw(y, dt), raw(dx, dt), raw(mean, torch.float32),
               raw(rstd, torch.float32)]
    ptrs = [None if t is None else t.data_ptr() for t in tensors]
    mods = None
    if row_mod is not None:
        mods = np.ascontiguousarray(np.asarray(row_mod, dtype=np.int64))
        assert mods.shape == (T,)
    n = T - row0 if nrows is None else nrows
    assert 0 <= row0 and row0 + n <= T
    tolv = (ctypes.c_double * 4)(*[float(v) for v in tol])
    out = (CheckStat * 4)()
    rc = _load().check_rows(code, ptrs[0], ptrs[1], ptrs[2], ptrs[3],
                            _ptr(mods), int(N), int(D), int(row0), int(n),
                            ptrs[4], ptrs[5], ptrs[6], ptrs[7],
                            ctypes.cast(tolv, ctypes.c_void_p), float(eps),
                            ctypes.cast(out, ctypes.c_void_p))
    if rc != 0:
        raise MemoryError("check_rows: out of host memory")
    return dict(zip(("y", "dx", "mean", "rstd"), out))
