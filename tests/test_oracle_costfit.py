"""Pins of the cost-model oracle (oracle/costfit.py) to facts that do not come
from it: exact recovery of the parameters that generated noiseless samples,
global optimality against a brute-force scan, invariances of least squares,
and the bucket rule against a brute-force search and the integer rule."""

import numpy as np
import pytest

from oracle import costfit as C

LENGTHS = np.array([1560, 4096, 8190, 12288, 16380, 24576, 32760], float)


def _shapes():
    B, S = [], []
    for s in LENGTHS:
        for b in (1, 2, max(1, int(131072 // s) // 2), int(131072 // s)):
            B.append(b)
            S.append(s)
    return np.array(B, float), np.array(S, float)


@pytest.mark.parametrize("a,b,p", [(0.4, 3e-9, 1.8), (2.0, 5e-5, 1.0),
                                   (0.05, 1e-11, 2.3)])
def test_noiseless_samples_recover_the_parameters(a, b, p):
    B, S = _shapes()
    t = a + b * B * S ** p
    fa, fb, fp, r = C.fit(B, S, t)
    assert abs(fp - p) < 1e-7
    assert abs(fa - a) < 1e-7 * max(1.0, abs(a))
    assert abs(fb - b) < 1e-6 * abs(b)
    assert r < 1e-18 * float(t @ t)


def test_fit_is_the_global_minimum_of_a_brute_force_scan():
    g = np.random.default_rng(1)
    B, S = _shapes()
    t = 0.3 + 2e-9 * B * S ** 1.85 * (1 + 0.05 * g.standard_normal(B.size))
    fa, fb, fp, r = C.fit(B, S, t)
    # brute force: a fine scan over p, each point's best (a, b) from the
    # normal equations solved with numpy.linalg.solve
    best = np.inf
    for p in np.linspace(0.5, 3.0, 25001):
        x = B * S ** p / (B * S ** p).max()
        M = np.array([[B.size, x.sum()], [x.sum(), x @ x]])
        a, bs = np.linalg.solve(M, [t.sum(), x @ t])
        res = t - a - bs * x
        best = min(best, float(res @ res))
    assert r <= best * (1 + 1e-12)
    assert r >= best * (1 - 1e-3)


def test_invariances():
    g = np.random.default_rng(2)
    B, S = _shapes()
    t = 1.0 + 1e-8 * B * S ** 1.6 * (1 + 0.1 * g.standard_normal(B.size))
    a, b, p, r = C.fit(B, S, t)
    # scaling the times scales a and b, not p
    a2, b2, p2, r2 = C.fit(B, S, 3.0 * t)
    assert abs(p2 - p) < 1e-6 and abs(a2 - 3 * a) < 1e-6 * abs(a)
    assert abs(b2 - 3 * b) < 1e-5 * abs(b) and abs(r2 - 9 * r) < 1e-6 * r
    # a constant added to every time moves a only
    a3, b3, p3, _ = C.fit(B, S, t + 0.7)
    assert abs(p3 - p) < 1e-6 and abs(a3 - (a + 0.7)) < 1e-6
    # the order of the samples does not matter
    perm = g.permutation(B.size)
    a4, b4, p4, _ = C.fit(B[perm], S[perm], t[perm])
    assert abs(p4 - p) < 1e-7 and abs(a4 - a) < 1e-7


def test_exponent_outside_the_range_lands_on_the_bound():
    B, S = _shapes()
    t = 0.1 + 1e-13 * B * S ** 2.9
    _, _, p, _ = C.fit(B, S, t, p_lo=0.5, p_hi=2.0)
    assert p == pytest.approx(2.0, abs=1e-9)


def test_bshape_real_brute_force_and_integer_rule(oracle_mod):
    g = np.random.default_rng(3)
    for _ in range(2000):
        S = int(g.integers(1, 70000))
        m_mem = int(g.integers(0, 400000))
        p = float(g.uniform(0.0, 2.5))
        m_comp = float(g.uniform(0, 5e9))
        got = C.bshape_real(S, m_mem, m_comp, p)
        # brute force: the largest B >= 1 with B*S <= m_mem and
        # B*S^p <= m_comp, else 1
        hi = m_mem // S
        b = 0
        lo_b, hi_b = 0, hi
        while lo_b < hi_b:   # bisection on the monotone compute condition
            mid = (lo_b + hi_b + 1) // 2
            if mid * S ** p <= m_comp:
                lo_b = mid
            else:
                hi_b = mid - 1
        b = lo_b
        assert got == max(1, b), (S, m_mem, m_comp, p)
    # integer exponent and bound: the integer rule (pinned by hand values)
    for _ in range(2000):
        S = int(g.integers(1, 70000))
        m_mem = int(g.integers(0, 400000))
        p = int(g.integers(0, 4))
        m_comp = int(g.integers(0, 10 ** 12))
        assert C.bshape_real(S, m_mem, float(m_comp), float(p)) == \
            oracle_mod.bshape(S, m_mem, m_comp, p)
    # the mixed schedule with p = 2 and with a fitted-looking p = 1.9
    assert [C.bshape_real(S, 131072, 2.2e9, 2.0)
            for S in (1560, 8190, 16380, 32760)] == [84, 16, 8, 2]
    # 32760^1.9 = 3.80e8, so the compute bound is 5 and memory (4) binds
    assert C.bshape_real(32760, 131072, 2.2e9, 1.9) == 4


def test_m_comp_on_the_pages_constants(oracle_mod):
    """Section 2.A quotes p = 2, M_mem = 131072 tokens and M_comp = 2.2e9.
    The reading of how M_comp follows from a fit -- the B * S^p of the
    memory-bound bucket of a reference length -- gives, for the reference
    length 16380, 8 * 16380^2 = 2,146,435,200 (by hand: 16380^2 =
    268,304,400), which is the quoted 2.2e9 to two digits, and the same
    bucket batches for the four lengths (tests/golden/bucket_sizes.txt)."""
    mc = C.m_comp(2.0, 131072, 16380)
    assert mc == 2_146_435_200.0
    assert abs(mc - 2.2e9) / 2.2e9 < 0.025
    lengths = (1560, 8190, 16380, 32760)
    assert [C.bshape_real(S, 131072, mc, 2.0) for S in lengths] == \
        [oracle_mod.bshape(S, 131072, 2_200_000_000, 2) for S in lengths] == \
        [84, 16, 8, 2]


def test_m_comp_is_the_reference_buckets_cost():
    """Brute force over the memory-feasible batches of the reference length:
    M_comp is the largest B * s_ref^p among them, so the bucket rule at M_comp
    gives the reference length its memory-bound batch, and a longer length
    never a batch whose B * S^p exceeds M_comp (unless that batch is 1)."""
    g = np.random.default_rng(11)
    for _ in range(300):
        p = float(g.uniform(0.5, 3.0))
        s_ref = int(g.integers(100, 40000))
        m_mem = int(g.integers(s_ref, 400000))
        mc = C.m_comp(p, m_mem, s_ref)
        best = max(B * float(s_ref) ** p for B in range(1, m_mem // s_ref + 1))
        assert mc == pytest.approx(best, rel=1e-12)
        assert C.bshape_real(s_ref, m_mem, mc * (1 + 1e-12), p) == \
            m_mem // s_ref
        S = int(g.integers(s_ref, 4 * s_ref + 1))
        b = C.bshape_real(S, m_mem, mc, p)
        assert b == 1 or b * float(S) ** p <= mc * (1 + 1e-12)
    assert C.m_comp(2.0, 131072, 0) == -1.0
    assert C.m_comp(-1.0, 131072, 16380) == -1.0
    assert C.m_comp(float("nan"), 131072, 16380) == -1.0
