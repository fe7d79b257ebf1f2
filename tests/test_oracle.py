"""Pins of the oracle to facts that do not come from the oracle itself.

* bucket sizing: hand-evaluated sizes of the mixed schedule, and a brute-force
  search for the largest batch that meets both constraints;
* forward: torch's float64 LayerNorm (a library routine, with the per-sample
  modulation as its affine weight 1+scale and bias shift), hand-worked rows
  with closed-form statistics, and invariants;
* backward: torch float64 autograd of the same composition, central finite
  differences of L = sum(dy * y), and closed-form invariants.

A dropped term, a sign error, a wrong index or a transposed operand anywhere
in the oracle changes at least one of these comparisons.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

EPS = 1e-6


def _rng(seed):
    return np.random.default_rng(seed)


def _inputs(B, N, D, seed, x_std=1.0, offset=True, mod_std=0.3):
    g = _rng(seed)
    x = g.standard_normal((B, N, D)) * x_std
    if offset:
        x = x + g.standard_normal(D) * 0.5
    s = g.standard_normal((B, D)) * mod_std
    h = g.standard_normal((B, D)) * mod_std
    dy = g.standard_normal((B, N, D))
    return x, s, h, dy


# ---------------------------------------------------------------- bucket sizing

@pytest.mark.parametrize("S,expect", [(1560, 84), (8190, 16), (16380, 8),
                                      (32760, 2)])
def test_bshape_mixed_schedule_by_hand(oracle_mod, S, expect):
    # 131072 // 1560 = 84 (memory binds; 2.2e9 // 1560**2 = 904)
    # 131072 // 8190 = 16 (memory binds; 2.2e9 // 8190**2 = 32)
    # 131072 // 16380 = 8 and 2.2e9 // 16380**2 = 8 (both bind)
    # 131072 // 32760 = 4, 2.2e9 // 32760**2 = 2 (compute binds)
    assert oracle_mod.bshape(S, 131072, 2_200_000_000, 2) == expect


def _golden_buckets():
    import os
    path = os.path.join(os.path.dirname(__file__), "golden",
                        "bucket_sizes.txt")
    rows = []
    for line in open(path):
        line = line.split("#", 1)[0].split()
        if line:
            rows.append(tuple(int(v) for v in line))
    return rows


def test_bshape_golden_table(oracle_mod):
    """The hand-evaluated table in tests/golden/bucket_sizes.txt."""
    rows = _golden_buckets()
    assert len(rows) == 6
    for S, m_mem, m_comp, p, mem_b, comp_b, b in rows:
        assert m_mem // S == mem_b and m_comp // S ** p == comp_b
        assert oracle_mod.bshape(S, m_mem, m_comp, p) == b


def test_bshape_tokens_per_bucket(oracle_mod):
    toks = {S: S * oracle_mod.bshape(S, 131072, 2_200_000_000, 2)
            for S in (1560, 8190, 16380, 32760)}
    assert toks == {1560: 131040, 8190: 131040, 16380: 131040, 32760: 65520}


def test_bshape_brute_force(oracle_mod):
    """The rule is the largest B >= 1 with B*S <= M_mem and B*S^p <= M_comp,
    and 1 when no B >= 1 meets both; found here by search."""
    g = _rng(7)
    for _ in range(400):
        S = int(g.integers(1, 120))
        m_mem = int(g.integers(0, 3000))
        p = int(g.integers(0, 4))
        m_comp = int(g.integers(0, 4 * 10 ** 5))
        best, B = 1, 1
        while B * S <= m_mem and B * S ** p <= m_comp:
            best = B
            B += 1
        assert oracle_mod.bshape(S, m_mem, m_comp, p) == best, (S, m_mem,
                                                                m_comp, p)


def test_bshape_edges(oracle_mod):
    assert oracle_mod.bshape(200_000, 131072, 2_200_000_000, 2) == 1  # S > M_mem
    assert oracle_mod.bshape(1, 131072, 2_200_000_000, 2) == 131072
    assert oracle_mod.bshape(10 ** 6, 10 ** 18, 10 ** 18, 4) == 1  # S^p overflows
    assert oracle_mod.bshape(0, 1, 1, 2) == -1
    assert oracle_mod.bshape(-5, 1, 1, 2) == -1
    assert oracle_mod.bshape(5, -1, 1, 2) == -1
    assert oracle_mod.bshape(5, 1, 1, -1) == -1


# --------------------------------------------------------------------- forward

def _torch_fwd(x, s, h):
    x = torch.from_numpy(x)
    s = torch.from_numpy(s)
    h = torch.from_numpy(h)
    ys = [F.layer_norm(x[b], (x.shape[-1],), weight=1 + s[b], bias=h[b],
                       eps=EPS) for b in range(x.shape[0])]
    return torch.stack(ys).numpy()


@pytest.mark.parametrize("B,N,D,x_std", [(3, 5, 48, 1.0), (2, 4, 64, 1.0),
                                         (2, 3, 5120, 20.0), (1, 9, 7, 1e-2)])
def test_fwd_matches_library_layer_norm(oracle_mod, B, N, D, x_std):
    x, s, h, _ = _inputs(B, N, D, seed=B * 1000 + D, x_std=x_std)
    y, mean, rstd = oracle_mod.fwd(x, s, h)
    y_ref = _torch_fwd(x, s, h)
    scale = np.abs(y_ref).max()
    assert np.abs(y - y_ref).max() <= 1e-12 * scale
    var_ref, mean_ref = torch.var_mean(torch.from_numpy(x), dim=-1,
                                       unbiased=False)
    np.testing.assert_allclose(mean, mean_ref.numpy(), rtol=0,
                               atol=1e-13 * (1 + np.abs(x).max()))
    np.testing.assert_allclose(rstd, 1 / np.sqrt(var_ref.numpy() + EPS),
                               rtol=1e-12)


def test_fwd_hand_worked_rows(oracle_mod):
    # Row [1, 2, 3, 4]: mean 2.5, biased variance (2.25+0.25+0.25+2.25)/4 = 1.25.
    # Row [a, -a, a, -a] with a = 3: mean 0, variance 9.
    x = np.array([[[1.0, 2.0, 3.0, 4.0], [3.0, -3.0, 3.0, -3.0]]])
    s = np.array([[0.5, -0.25, 0.0, 1.0]])
    h = np.array([[0.1, 0.2, -0.3, 0.0]])
    y, mean, rstd = oracle_mod.fwd(x, s, h)
    r0 = 1.0 / np.sqrt(1.25 + 1e-6)
    r1 = 1.0 / np.sqrt(9.0 + 1e-6)
    assert mean[0, 0] == 2.5 and mean[0, 1] == 0.0
    assert rstd[0, 0] == pytest.approx(r0, rel=1e-15)
    assert rstd[0, 1] == pytest.approx(r1, rel=1e-15)
    xhat0 = np.array([-1.5, -0.5, 0.5, 1.5]) * r0
    xhat1 = np.array([3.0, -3.0, 3.0, -3.0]) * r1
    np.testing.assert_allclose(y[0, 0], xhat0 * np.array([1.5, 0.75, 1.0, 2.0])
                               + h[0], rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(y[0, 1], xhat1 * np.array([1.5, 0.75, 1.0, 2.0])
                               + h[0], rtol=1e-15, atol=1e-15)


def test_fwd_invariants(oracle_mod):
    B, N, D = 2, 6, 96
    x, _, _, _ = _inputs(B, N, D, seed=11)
    zeros = np.zeros((B, D))
    y, mean, rstd = oracle_mod.fwd(x, zeros, zeros)
    # xhat has zero mean and variance sigma^2 / (sigma^2 + eps), not exactly 1
    var = x.var(axis=-1)
    assert np.abs(y.mean(axis=-1)).max() <= 1e-14
    np.testing.assert_allclose(y.var(axis=-1), var / (var + EPS), rtol=1e-13)
    # adding a constant to a row leaves it unchanged
    c = np.arange(B * N, dtype=np.float64).reshape(B, N, 1) * 0.37 - 1.0
    y2, mean2, rstd2 = oracle_mod.fwd(x + c, zeros, zeros)
    np.testing.assert_allclose(y2, y, rtol=0, atol=1e-12)
    np.testing.assert_allclose(mean2, mean + c[..., 0], rtol=0, atol=1e-12)
    # a constant row normalises to zero, with rstd = 1/sqrt(eps)
    xc = np.full((1, 1, 16), 2.5)
    yc, mc, rc = oracle_mod.fwd(xc, np.ones((1, 16)), np.full((1, 16), 0.25))
    assert np.all(yc == 0.25) and mc[0, 0] == 2.5
    assert rc[0, 0] == pytest.approx(1 / np.sqrt(EPS), rel=1e-15)


def test_fwd_modulation_is_per_sample(oracle_mod):
    x, s, h, _ = _inputs(3, 4, 32, seed=5)
    y, _, _ = oracle_mod.fwd(x, s, h)
    for b in range(3):
        yb, _, _ = oracle_mod.fwd(x[b:b + 1], s[b:b + 1], h[b:b + 1])
        np.testing.assert_array_equal(yb[0], y[b])


# -------------------------------------------------------------------- backward

def _torch_bwd(x, s, h, dy):
    xt = torch.from_numpy(x).requires_grad_(True)
    st = torch.from_numpy(s).requires_grad_(True)
    ht = torch.from_numpy(h).requires_grad_(True)
    y = F.layer_norm(xt, (x.shape[-1],), eps=EPS) * (1 + st[:, None, :]) \
        + ht[:, None, :]
    (y * torch.from_numpy(dy)).sum().backward()
    return xt.grad.numpy(), st.grad.numpy(), ht.grad.numpy()


@pytest.mark.parametrize("B,N,D,x_std", [(3, 7, 40, 1.0), (2, 33, 64, 1.0),
                                         (1, 4, 5120, 20.0), (2, 5, 3, 1e-3)])
def test_bwd_matches_library_autograd(oracle_mod, B, N, D, x_std):
    x, s, h, dy = _inputs(B, N, D, seed=N * 31 + D, x_std=x_std)
    dx, ds, dh = oracle_mod.bwd(dy, x, s)
    dx_ref, ds_ref, dh_ref = _torch_bwd(x, s, h, dy)
    for got, ref in ((dx, dx_ref), (ds, ds_ref), (dh, dh_ref)):
        assert np.abs(got - ref).max() <= 1e-11 * np.abs(ref).max()


def test_bwd_finite_differences(oracle_mod):
    """Central differences of L = sum(dy * y) through the oracle's forward."""
    B, N, D = 2, 3, 8
    x, s, h, dy = _inputs(B, N, D, seed=3)
    dx, ds, dh = oracle_mod.bwd(dy, x, s)
    step = 1e-6

    def loss(xx, ss, hh):
        y, _, _ = oracle_mod.fwd(xx, ss, hh)
        return float((y * dy).sum())

    for arr, grad in ((x, dx), (s, ds), (h, dh)):
        fd = np.empty_like(arr)
        for i in np.ndindex(arr.shape):
            orig = arr[i]
            arr[i] = orig + step
            lp = loss(x, s, h)
            arr[i] = orig - step
            lm = loss(x, s, h)
            arr[i] = orig
            fd[i] = (lp - lm) / (2 * step)
        np.testing.assert_allclose(grad, fd, rtol=0, atol=2e-8)


def test_bwd_invariants(oracle_mod):
    B, N, D = 2, 10, 48
    x, s, h, dy = _inputs(B, N, D, seed=9)
    dx, ds, dh = oracle_mod.bwd(dy, x, s)
    _, mean, rstd = oracle_mod.fwd(x, s, h)
    # dx is orthogonal to the constant row: sum_d dx = 0
    assert np.abs(dx.sum(axis=-1)).max() <= 1e-13 * np.abs(dx).max() * D
    # sum_d dx * xhat = rstd * c2 * D * eps / (var + eps)
    xhat = (x - mean[..., None]) * rstd[..., None]
    g = dy * (1 + s[:, None, :])
    c2 = (g * xhat).mean(axis=-1)
    var = x.var(axis=-1)
    closed = rstd * c2 * D * EPS / (var + EPS)
    np.testing.assert_allclose((dx * xhat).sum(axis=-1), closed, rtol=0,
                               atol=1e-14 * np.abs(dx).max() * D)
    # dshift is the plain sum of dy over the tokens of each sample
    np.testing.assert_allclose(dh, dy.sum(axis=1), rtol=1e-14)
    # dy = 1 everywhere: dshift = N exactly
    _, _, dh1 = oracle_mod.bwd(np.ones_like(dy), x, s)
    assert np.all(dh1 == N)


def test_bwd_linear_in_dy(oracle_mod):
    x, s, h, dy = _inputs(2, 6, 24, seed=21)
    dy2 = _rng(22).standard_normal(dy.shape)
    a = 0.75
    r1 = oracle_mod.bwd(dy, x, s)
    r2 = oracle_mod.bwd(dy2, x, s)
    r3 = oracle_mod.bwd(a * dy + dy2, x, s)
    for g1, g2, g3 in zip(r1, r2, r3):
        np.testing.assert_allclose(g3, a * g1 + g2, rtol=0,
                                   atol=1e-13 * np.abs(g3).max())


def test_bwd_token_order_and_split(oracle_mod):
    """dscale/dshift sum over tokens: permuting the tokens of a sample or
    splitting them into two calls and adding gives the same result."""
    B, N, D = 2, 12, 16
    x, s, h, dy = _inputs(B, N, D, seed=33)
    _, ds, dh = oracle_mod.bwd(dy, x, s)
    perm = _rng(34).permutation(N)
    _, ds_p, dh_p = oracle_mod.bwd(dy[:, perm], x[:, perm], s)
    np.testing.assert_allclose(ds_p, ds, rtol=0, atol=1e-13)
    np.testing.assert_allclose(dh_p, dh, rtol=0, atol=1e-13)
    _, ds_a, dh_a = oracle_mod.bwd(dy[:, :5], x[:, :5], s)
    _, ds_b, dh_b = oracle_mod.bwd(dy[:, 5:], x[:, 5:], s)
    np.testing.assert_allclose(ds_a + ds_b, ds, rtol=0, atol=1e-13)
    np.testing.assert_allclose(dh_a + dh_b, dh, rtol=0, atol=1e-13)


def test_oracle_independent_of_thread_count(oracle_mod):
    x, s, h, dy = _inputs(3, 40, 200, seed=41)
    n0 = oracle_mod.num_threads()
    try:
        oracle_mod.set_num_threads(1)
        a = oracle_mod.fwd(x, s, h) + oracle_mod.bwd(dy, x, s)
        oracle_mod.set_num_threads(max(2, n0))
        b = oracle_mod.fwd(x, s, h) + oracle_mod.bwd(dy, x, s)
    finally:
        oracle_mod.set_num_threads(n0)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


def test_empty_inputs(oracle_mod):
    x = np.zeros((2, 0, 8))
    y, mean, rstd = oracle_mod.fwd(x, np.zeros((2, 8)), np.zeros((2, 8)))
    assert y.shape == (2, 0, 8) and mean.shape == (2, 0)
    dx, ds, dh = oracle_mod.bwd(x, x, np.zeros((2, 8)))
    assert dx.shape == (2, 0, 8)
    assert np.all(ds == 0) and np.all(dh == 0)
