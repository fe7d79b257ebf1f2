"""The library's host-side scheduler arithmetic (adaln_costfit,
adaln_bshape_real) against the oracle, without a GPU."""

import ctypes

import numpy as np
import pytest

import adaln_fwd_amd as A
from adaln_fwd_amd import _lib
from oracle import costfit as C


def _lib_fit(B, S, t, p_lo=0.5, p_hi=3.0):
    B, S, t = (np.ascontiguousarray(v, dtype=np.float64) for v in (B, S, t))
    out = (ctypes.c_double * 4)()
    rc = A.load().adaln_costfit(B.ctypes.data, S.ctypes.data, t.ctypes.data,
                                B.size, p_lo, p_hi, ctypes.cast(out,
                                                                ctypes.c_void_p))
    return rc, tuple(out)


def _data(seed, noise):
    g = np.random.default_rng(seed)
    S = g.choice([1560, 4096, 8190, 12288, 16380, 24576, 32760], size=24)
    B = np.maximum(1, (131072 // S) // g.integers(1, 5, size=24))
    a = g.uniform(0.01, 2.0)
    p = g.uniform(1.0, 2.4)
    b = g.uniform(0.5, 2.0) / (131072 * 32760.0 ** (p - 1))
    t = (a + b * B * S.astype(float) ** p) * (1 + noise * g.standard_normal(24))
    return B.astype(float), S.astype(float), t


@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("noise", [0.0, 0.03])
def test_costfit_matches_oracle(seed, noise):
    B, S, t = _data(seed, noise)
    rc, (a, b, p, r) = _lib_fit(B, S, t)
    assert rc == _lib.OK
    oa, ob, op, orr = C.fit(B, S, t)
    assert abs(p - op) < 1e-6
    assert abs(a - oa) < 1e-6 * max(1.0, abs(oa))
    assert abs(b - ob) < 1e-5 * abs(ob)
    scale = float(t @ t)
    assert abs(r - orr) <= 1e-9 * max(orr, 1e-12 * scale)
    # the residual the library reports is the one its parameters give
    assert abs(r - C.rss(a, b, p, B, S, t)) <= 1e-9 * max(r, 1e-12 * scale)


def test_costfit_validation():
    B, S, t = _data(0, 0.0)
    assert _lib_fit(B[:2], S[:2], t[:2])[0] == _lib.ERR_INVALID
    assert _lib_fit(B, S, t, 2.0, 1.0)[0] == _lib.ERR_INVALID
    bad = S.copy()
    bad[3] = 0.0
    assert _lib_fit(B, bad, t)[0] == _lib.ERR_INVALID
    tn = t.copy()
    tn[0] = np.nan
    assert _lib_fit(B, S, tn)[0] == _lib.ERR_INVALID
    out = (ctypes.c_double * 4)()
    assert A.load().adaln_costfit(None, None, None, 5, 0.5, 3.0,
                                  ctypes.cast(out, ctypes.c_void_p)) == \
        _lib.ERR_INVALID


def test_bshape_real_matches_oracle():
    lib = A.load()
    g = np.random.default_rng(5)
    for _ in range(5000):
        S = int(g.integers(1, 70000))
        m_mem = int(g.integers(0, 400000))
        p = float(g.uniform(0.0, 2.5))
        m_comp = float(g.uniform(0, 5e9))
        assert lib.adaln_bshape_real(S, m_mem, m_comp, p) == \
            C.bshape_real(S, m_mem, m_comp, p)
    assert lib.adaln_bshape_real(0, 10, 1.0, 1.0) == _lib.ERR_INVALID
    assert lib.adaln_bshape_real(10, 10, -1.0, 1.0) == _lib.ERR_INVALID
    assert lib.adaln_bshape_real(10, 10, 1.0, float("nan")) == _lib.ERR_INVALID


def test_mcomp_matches_oracle():
    g = np.random.default_rng(4)
    lib = _lib.load()
    for _ in range(500):
        p = float(g.uniform(0.0, 3.0))
        s_ref = int(g.integers(1, 10 ** 6))
        m_mem = int(g.integers(0, 10 ** 8))
        got = lib.adaln_mcomp(p, m_mem, s_ref)
        assert got == pytest.approx(C.m_comp(p, m_mem, s_ref), rel=1e-15,
                                    abs=0.0), (p, m_mem, s_ref)
    assert lib.adaln_mcomp(2.0, 131072, 16380) == 2_146_435_200.0
    for bad in ((2.0, 131072, 0), (-0.5, 131072, 16380),
                (float("inf"), 131072, 16380), (2.0, -1, 16380)):
        assert lib.adaln_mcomp(*bad) == -1.0
        assert C.m_comp(*bad) == -1.0


def test_python_scheduler_helpers(oracle_mod):
    from adaln_fwd_amd import sched
    B, S, t = _data(7, 0.02)
    m = sched.costfit(B, S, t)
    oa, ob, op, orr = C.fit(B, S, t)
    assert abs(m.p - op) < 1e-6 and abs(m.a - oa) < 1e-6 * max(1, abs(oa))
    assert 0.0 < m.r2 <= 1.0
    assert m.predict(4, 8190) == pytest.approx(C.model(m.a, m.b, m.p, 4, 8190))
    # the compute bound of the reference length's memory-bound bucket; with
    # p = 2 and 16380 it reproduces the mixed schedule's bucket sizes
    mc = sched.m_comp_for(2.0, 131072, 16380)
    assert mc == 8 * 16380.0 ** 2
    assert sched.buckets((1560, 8190, 16380, 32760), 131072, mc, 2.0) == \
        {S_: oracle_mod.bshape(S_, 131072, 2_200_000_000, 2)
         for S_ in (1560, 8190, 16380, 32760)}
    # that bucket is exactly at the bound: B_mem(S_ref) * S_ref^p == m_comp
    for p in (1.5, 1.84, 2.0):
        mc = sched.m_comp_for(p, 131072, 16380)
        assert sched.bshape_real(16380, 131072, mc * (1 + 1e-12), p) == 8
    assert sched.pearson([1, 2, 3], [2, 4, 6]) == pytest.approx(1.0)
    assert sched.pearson([1, 2, 3], [3, 2, 1]) == pytest.approx(-1.0)
    assert sched.cv([1.0, 1.0, 1.0]) == 0.0
    assert sched.cv([1.0, 3.0]) == pytest.approx(0.5)
    shapes = sched.sweep_shapes((1560, 32760), 131072)
    assert (84, 1560) in shapes and (4, 32760) in shapes
    assert all(B * S_ <= 131072 for B, S_ in shapes)
    with pytest.raises(_lib.AdalnError):
        sched.costfit([1, 2], [3, 4], [5, 6])
