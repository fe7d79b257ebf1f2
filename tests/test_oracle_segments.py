"""Pins of the oracle's packed-segment functions to facts that do not come
from those functions: torch float64 autograd of LayerNorm followed by a
modulation gathered per row (the gather's backward is a scatter-add over the
rows that use each vector), the batched oracle (already pinned) on the
uniform layout, and closed forms (dshift of a shared vector is the sum of
dy over all its rows; an unused vector gets zero)."""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

EPS = 1e-6


def _layout(lengths, mods, nmod, D, seed):
    g = np.random.default_rng(seed)
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T = int(off[-1])
    x = g.standard_normal((T, D)) * 1.5 + g.standard_normal(D) * 0.5
    s = g.standard_normal((nmod, D)) * 0.3
    h = g.standard_normal((nmod, D)) * 0.3
    dy = g.standard_normal((T, D))
    return off, (None if mods is None else np.asarray(mods, np.int32)), x, s, h, dy


def _row_mod(off, mods):
    lengths = np.diff(off)
    idx = np.arange(len(lengths)) if mods is None else mods
    return torch.from_numpy(np.repeat(idx, lengths).astype(np.int64))


def _torch_ref(off, mods, x, s, h, dy):
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    st = torch.tensor(s, dtype=torch.float64, requires_grad=True)
    ht = torch.tensor(h, dtype=torch.float64, requires_grad=True)
    rm = _row_mod(off, mods)
    xhat = F.layer_norm(xt, (x.shape[1],), eps=EPS)
    y = xhat * (1 + st[rm]) + ht[rm]
    (y * torch.from_numpy(dy)).sum().backward()
    return (y.detach().numpy(), xt.grad.numpy(), st.grad.numpy(),
            ht.grad.numpy())


CASES = [
    # lengths, modulation index per segment (None: identity), nmod
    ([5, 3, 9], None, 3),
    ([4, 0, 7, 2], [1, 0, 1, 3], 4),          # empty segment, shared and unused vectors
    ([12, 12], [0, 0], 2),                    # text + video tokens of one sample share one vector
    ([1, 1, 1, 1, 1], [4, 3, 2, 1, 0], 5),    # reversed table, one row each
]


@pytest.mark.parametrize("lengths,mods,nmod", CASES)
@pytest.mark.parametrize("D", [8, 33])
def test_segments_match_autograd(oracle_mod, lengths, mods, nmod, D):
    off, mod, x, s, h, dy = _layout(lengths, mods, nmod, D, seed=len(lengths) * D)
    y_ref, dx_ref, ds_ref, dh_ref = _torch_ref(off, mod, x, s, h, dy)
    y, mean, rstd = oracle_mod.fwd_segments(x, s, h, off, mod)
    dx, ds, dh = oracle_mod.bwd_segments(dy, x, s, off, mod)
    np.testing.assert_allclose(y, y_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dx, dx_ref, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(ds, ds_ref, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dh, dh_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(mean, x.mean(axis=1), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(rstd, 1 / np.sqrt(x.var(axis=1) + EPS),
                               rtol=1e-12)


def test_uniform_layout_equals_batched(oracle_mod):
    """B segments of N rows with the identity table are the batched layout:
    the same sums in the same order, so the results are equal bit for bit."""
    B, N, D = 3, 6, 20
    off, _, x, s, h, dy = _layout([N] * B, None, B, D, seed=5)
    y, mean, rstd = oracle_mod.fwd_segments(x, s, h, off)
    dx, ds, dh = oracle_mod.bwd_segments(dy, x, s, off)
    yb, mb, rb = oracle_mod.fwd(x.reshape(B, N, D), s, h)
    dxb, dsb, dhb = oracle_mod.bwd(dy.reshape(B, N, D), x.reshape(B, N, D), s)
    assert np.array_equal(y, yb.reshape(B * N, D))
    assert np.array_equal(mean, mb.reshape(-1)) and np.array_equal(rstd, rb.reshape(-1))
    assert np.array_equal(dx, dxb.reshape(B * N, D))
    assert np.array_equal(ds, dsb) and np.array_equal(dh, dhb)


def test_shared_and_unused_vectors(oracle_mod):
    lengths, mods, nmod, D = [3, 5, 4], [2, 0, 2], 4, 16
    off, mod, x, s, h, dy = _layout(lengths, mods, nmod, D, seed=11)
    _, ds, dh = oracle_mod.bwd_segments(dy, x, s, off, mod)
    # closed form for dshift: the plain sum of dy over the rows using m
    np.testing.assert_allclose(dh[2], dy[0:3].sum(0) + dy[8:12].sum(0),
                               rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(dh[0], dy[3:8].sum(0), rtol=1e-13, atol=1e-13)
    assert not ds[1].any() and not dh[1].any()
    assert not ds[3].any() and not dh[3].any()


def test_empty_table(oracle_mod):
    x = np.zeros((0, 8))
    s = np.zeros((2, 8))
    y, mean, rstd = oracle_mod.fwd_segments(x, s, s, [0])
    assert y.shape == (0, 8) and mean.shape == (0,)
    dx, ds, dh = oracle_mod.bwd_segments(x, x, s, [0])
    assert dx.shape == (0, 8) and not ds.any() and not dh.any()
