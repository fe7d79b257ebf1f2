"""The largest batch the boundary accepts: one sample of 2^31 - 1 token rows
(B*N <= 2^31 - 1) at D = 8 bf16, about 34 GB per activation tensor.

Every entry point that walks rows runs on it: the forward (512 launches of
its row grid), the fused backward and its finish, the unfused dx and D-tile
entry points, and the packed forward and backward with one segment of all
rows.  x tiles 4099 seeded base rows (row n is base row n mod 4099), so the
oracle can rebuild any row on the host; dy is 1 everywhere.  Sampled rows of y,
mean, rstd and dx -- the first and last rows, both sides of every 2^22-row
launch boundary and a seeded draw -- are compared with the oracle, and
dscale and dshift in full: with dy = 1 each is a weighted sum of the base
rows' own gradients (weights: how often each base row occurs), which the
oracle gives as a one-row backward per base row.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import workloads as W
from tests import parity as P

pytestmark = pytest.mark.gpu

ROWS = (1 << 31) - 1
D = 8
BASE = 4099  # base rows, prime so that row n % BASE cycles through them all


def _say(msg):
    print(f"[max rows] {msg}", flush=True)


@pytest.fixture(scope="module")
def A():
    import adaln_fwd_amd
    adaln_fwd_amd.load()
    return adaln_fwd_amd


def _sample_rows():
    g = np.random.default_rng(31)
    launch = 1 << 22
    edges = [np.arange(8), np.arange(ROWS - 8, ROWS)]
    for k in range(1, ROWS // launch + 1):
        edges.append(np.arange(k * launch - 2, min(k * launch + 2, ROWS)))
    edges.append(g.integers(0, ROWS, size=512))
    return np.unique(np.concatenate(edges)).astype(np.int64)


def _rows_of(t, rows_t):
    """Host copy of the listed rows of a [ROWS, D] (or [ROWS]) GPU tensor."""
    return t.index_select(0, rows_t).cpu()


def test_max_rows(A):
    torch.cuda.empty_cache()
    free, _ = torch.cuda.mem_get_info()
    if free < 130e9:
        pytest.skip(f"needs about 130 GB of free device memory, {free / 1e9:.0f} "
                    "GB free")
    wl = W.custom(1, BASE, D, "bf16", x_kind="normal")
    base = synth.make_inputs(wl, seed=7)
    bx = base.x.reshape(BASE, D)
    scale, shift = base.scale, base.shift            # [1, D]
    rows = _sample_rows()
    rows_t = torch.from_numpy(rows).cuda()
    xr = bx[torch.from_numpy(rows % BASE)]           # host rows of x
    # oracle: the sampled rows, each as a one-row sample of the same vectors
    k = rows.size
    sk, hk = scale.expand(k, D), shift.expand(k, D)
    y_ref, m_ref, r_ref = oracle.fwd(xr.unsqueeze(1), sk, hk)
    ones_k = torch.ones(k, 1, D, dtype=torch.bfloat16)
    dx_ref, _, _ = oracle.bwd(ones_k, xr.unsqueeze(1), sk, want_dmod=False)
    # dscale, dshift: sum over base rows of count * (one-row gradient)
    counts = np.full(BASE, ROWS // BASE, dtype=np.float64)
    counts[: ROWS % BASE] += 1
    _, ds1, dh1 = oracle.bwd(torch.ones(BASE, 1, D, dtype=torch.bfloat16),
                             bx.unsqueeze(1), scale.expand(BASE, D))
    ds_ref = (counts[:, None] * ds1).sum(0, keepdims=True)
    dh_ref = (counts[:, None] * dh1).sum(0, keepdims=True)
    assert np.all(dh_ref == ROWS)

    def check(label, y=None, mean=None, rstd=None, dx=None, ds=None, dh=None):
        reps = []
        if y is not None:
            reps += P.check_out("y", _rows_of(y, rows_t), y_ref[:, 0], "bf16")
            reps += P.check_stats(_rows_of(mean, rows_t), _rows_of(rstd, rows_t),
                                  m_ref[:, 0], r_ref[:, 0], xr)
        if dx is not None:
            reps += P.check_out("dx", _rows_of(dx, rows_t), dx_ref[:, 0],
                                "bf16")
        if ds is not None:
            reps.append(P.check_dmod("dscale", ds.cpu(), ds_ref))
            reps.append(P.check_dmod("dshift", dh.cpu(), dh_ref))
        for r in reps:
            _say(f"  {label} {r}")

    _say(f"tiling x: {ROWS} rows x {D} bf16; {rows.size} sampled rows")
    reps_needed = -(-ROWS // BASE)
    x = bx.cuda().repeat(reps_needed, 1)[:ROWS]
    dy = torch.ones(ROWS, D, dtype=torch.bfloat16, device="cuda")
    s, h = scale.cuda(), shift.cuda()

    _say("batched forward, fused backward")
    y, mean, rstd = A.fwd(x.view(1, ROWS, D), s, h)
    torch.cuda.synchronize()
    check("fwd", y=y.view(ROWS, D), mean=mean.view(ROWS), rstd=rstd.view(ROWS))
    del y
    dx, ds, dh = A.bwd(dy.view(1, ROWS, D), x.view(1, ROWS, D), s, mean, rstd)
    torch.cuda.synchronize()
    check("bwd", dx=dx.view(ROWS, D), ds=ds, dh=dh)

    _say("unfused dx and D-tile entry points")
    A.bwd_dx(dy.view(1, ROWS, D), x.view(1, ROWS, D), s, mean, rstd, dx=dx)
    ds, dh = A.bwd_dmod(dy.view(1, ROWS, D), x.view(1, ROWS, D), mean, rstd)
    torch.cuda.synchronize()
    check("unfused", dx=dx.view(ROWS, D), ds=ds, dh=dh)
    del dx, mean, rstd

    _say("packed forward and backward, one segment of every row")
    off = np.array([0, ROWS], dtype=np.int64)
    y, mean, rstd = A.fwd_segments(x, s, h, off)
    torch.cuda.synchronize()
    check("packed fwd", y=y, mean=mean, rstd=rstd)
    del y
    dx, ds, dh = A.bwd_segments(dy, x, s, mean, rstd, off)
    torch.cuda.synchronize()
    check("packed bwd", dx=dx, ds=ds, dh=dh)
    del dx, mean, rstd, x, dy
    torch.cuda.empty_cache()
