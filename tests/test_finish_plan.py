"""The launch that sums the backward's partial rows into dscale and dshift,
on the host: for seeded random shapes, the plan adaln_plan reports for it
(which = 2), replayed through the mapping the header documents (column
blocks of F features, workgroup g -> logical block L(g), its cpb blocks and
then every G-th group of them; wpc wavefronts per block cutting the partial
rows into contiguous slices), serves every (sample, feature) output exactly
once, sums every partial row of it exactly once, and fits a workgroup.  The
choice of F is pinned too.  CPU only."""

import numpy as np
import pytest
import torch

import adaln_fwd_amd as A

BF16, F32 = torch.bfloat16, torch.float32
D_BF16 = [8, 520, 1536, 2560, 3072, 4096, 5120, 8192, 10240, 16384]
D_F32 = [4, 64, 1024, 1280, 2560, 4096, 8192]


def _shapes(seed, n):
    g = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        dt = BF16 if g.random() < 0.6 else F32
        D = int(g.choice(D_BF16 if dt is BF16 else D_F32))
        B = int(np.exp(g.uniform(0, np.log(2000))))
        N = int(np.exp(g.uniform(0, np.log(80000))))
        N = max(1, min(N, 2_000_000 // B))
        out.append((B, N, D, dt))
    return out


def _logical(g, G, F):
    per = G // 8
    if F < 64 and g < 8 * per:
        return (g % 8) * per + g // 8
    return g


def _served(p, B, D):
    """Times each (sample, feature) output is written under the mapping."""
    F, cpb, G = p["F"], p["cpb"], p["workgroups"]
    C = -(-D // F)
    total = B * C
    count = np.zeros(total, dtype=np.int32)
    starts = []
    for g in range(G):
        L = _logical(g, G, F)
        while L * cpb < total:
            starts.append(L * cpb)
            L += G
    starts = np.asarray(starts, dtype=np.int64)
    logical = sorted(_logical(g, G, F) for g in range(G))
    assert logical == list(range(G)), "the block order is not a bijection"
    for j in range(cpb):
        k = starts + j
        np.add.at(count, k[k < total], 1)
    # every block of F features, clipped to D
    per_feature = np.repeat(count.reshape(B, C), F, axis=1)[:, :D]
    return per_feature


@pytest.mark.parametrize("B,N,D,dt", _shapes(11, 200))
def test_every_output_once(B, N, D, dt):
    p = A.plan("finish", B, N, D, dt)
    assert p["F"] in (16, 32, 64)
    wpc = p["wpc"]
    assert wpc in (1, 2, 4, 8, 16)
    assert p["threads"] == wpc * p["cpb"] * 64 <= 1024
    assert 1 <= p["workgroups"] <= 1 << 20
    # the partial rows summed per output: the fused plan's workgroups per
    # sample where the fused backward runs
    try:
        fused = A.plan("bwd", B, N, D, dt)
        assert p["rows"] == fused["bps"]
    except A.AdalnError as e:
        assert e.code == -6
    # every output once
    served = _served(p, B, D)
    assert served.shape == (B, D) and (served == 1).all()
    # the slices of the wpc wavefronts partition the partial rows, and a
    # wavefront's lanes hold at most 8 loads per array per pass over them
    P = p["rows"]
    cuts = [s * P // wpc for s in range(wpc + 1)]
    assert cuts[0] == 0 and cuts[-1] == P and cuts == sorted(cuts)
    if wpc < 16:
        assert max(b - a for a, b in zip(cuts, cuts[1:])) <= 8 * (64 // p["F"])


@pytest.mark.parametrize("B,D,dt,F", [
    (16, 1536, BF16, 64),   # 384 blocks of 64 features: one per CU
    (1, 5120, BF16, 32),    # 80 blocks of 64 are too few; 160 of 32 do
    (1, 1536, BF16, 16),    # 48 blocks of 32 are too few: 96 of 16
    (84, 3072, BF16, 64),
    (2, 3072, BF16, 32),
    (1, 64, F32, 16),
])
def test_block_width(B, D, dt, F):
    assert A.plan("finish", B, 4096, D, dt)["F"] == F


def test_empty_batch():
    p = A.plan("finish", 0, 100, 1536, BF16)
    assert p["workgroups"] == 0
    p = A.plan("finish", 3, 0, 1536, BF16)      # dscale = dshift = 0
    assert p["rows"] == 0 and (_served(p, 3, 1536) == 1).all()
