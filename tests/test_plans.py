"""The launch planner, on the host: for seeded random shapes over every
kernel family, the plans adaln_plan reports, replayed through the work
mapping the header documents (the backward's persistent grids: workgroup
g -> samples g / bps, + groups, ...; walker w -> rows (g % bps) * walkers
+ w, + bps * walkers, ...; the forward: walker w of workgroup g -> row
(4/W)g + w of the batch), visit every token row exactly once, fit the
resident grid, and for the fused backward give each (sample, workgroup)
pair its own partial row inside the workspace.  The shape-dependent choices
are pinned too: the wavefront pairs past 320 vectors (quads past 1280, eight
wavefronts past 2560, up to the widest row), the fewest long
samples in flight (paired backward), and the balanced workgroups per
sample.  CPU only."""

import numpy as np
import pytest
import torch

import adaln_fwd_amd as A

BF16, F32 = torch.bfloat16, torch.float32
D_BF16 = [8, 520, 1536, 2560, 2568, 3072, 4096, 5120, 5128, 7000, 8192,
          10240, 10248, 12288, 16384, 20480, 20488, 32768]
D_F32 = [4, 64, 1024, 1280, 1288, 2560, 4096, 5120, 5124, 8192, 10240,
         10244, 16384]
MAX_GRID = 256 * 8   # 256 CUs, at most 8 workgroups each


def _shapes(seed, n):
    g = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        dt = BF16 if g.random() < 0.6 else F32
        D = int(g.choice(D_BF16 if dt is BF16 else D_F32))
        B = int(np.exp(g.uniform(0, np.log(3000))))
        N = int(np.exp(g.uniform(0, np.log(80000))))
        N = max(1, min(N, 2_000_000 // B))
        out.append((B, N, D, dt))
    return out


def _weighted_positions(g, k, w, bps, walkers, N, m):
    """Walk positions of walker w of workgroup g (number k of its sample's
    bps) in the rounds the header documents for the weighted backward walk:
    m regular steps, then one more for the walkers of even workgroups."""
    S = bps * walkers
    first = g - k                       # the sample's first workgroup
    even_k = [kk for kk in range(bps) if (first + kk) % 2 == 0]
    Wf = len(even_k) * walkers
    L = m * S + Wf
    out = []
    t = 0
    while t * L < N:
        out += [t * L + r * S + k * walkers + w for r in range(m)]
        if g % 2 == 0:
            out.append(t * L + m * S + even_k.index(k) * walkers + w)
        t += 1
    return [q for q in out if q < N]


def _visits(p, B, N, m=0):
    """Times each (sample, row) is visited under the documented mapping."""
    pos = np.zeros((B, N), dtype=np.int32)  # by walk position
    bps, groups, walkers = p["bps"], p["groups"], p["walkers"]
    stride = bps * walkers
    for g in range(p["workgroups"]):
        slot, k = divmod(g, bps)
        if slot >= groups:
            continue
        for w in range(walkers):
            if m:
                pos[slot::groups, _weighted_positions(g, k, w, bps, walkers,
                                                      N, m)] += 1
            else:
                pos[slot::groups, k * walkers + w::stride] += 1
    # position n of sample b is row (n + b * skew) mod N
    count = np.zeros_like(pos)
    n = np.arange(N)
    for b in range(B):
        count[b, (n + b * p["skew"]) % N] = pos[b]
    return count


@pytest.mark.parametrize("B,N,D,dt", _shapes(7, 300))
def test_every_row_once(B, N, D, dt):
    for which in ("fwd", "bwd"):
        # every row width up to the widest has a forward and a fused plan
        p = A.plan(which, B, N, D, dt)
        if which == "fwd":
            # a grid over the rows: walker j of workgroup g -> row wg + j,
            # w = 4 / W walkers (one row each) per workgroup
            w = p["walkers"]
            assert p["bps"] == 0 and p["groups"] == 0
            assert w * p["waves_per_row"] == 4
            assert p["workgroups"] == -(-B * N // w)
            rows = (w * np.arange(p["workgroups"])[:, None]
                    + np.arange(w)[None, :]).ravel()
            rows = rows[rows < B * N]
            assert np.all(np.bincount(rows, minlength=B * N) == 1)
            continue
        assert 1 <= p["bps"] and 1 <= p["groups"]
        assert p["workgroups"] == p["bps"] * min(p["groups"], B)
        assert p["bps"] * p["groups"] <= MAX_GRID
        # four-wavefront workgroups of row walkers (single wavefronts, pairs
        # or quads), or eight wavefronts on one row
        w = p["waves_per_row"]
        assert p["walkers"] * w == (8 if w == 8 else 4)
        m = {3072: 12, 5120: 16}.get(D, 0) if dt is BF16 else 0
        assert np.all(_visits(p, B, N, m) == 1), (which, p)
        if which == "bwd":
            # partial row b * bps + (g % bps) of [B, bps, D], and room for it
            q = A.bwd_fused_plan(B, N, D, dt)
            assert q["partial_rows"] == p["bps"]
            need = 2 * B * p["bps"] * D * 4
            assert A.bwd_workspace_bytes(B, N, D, dt) >= need


def test_rows_past_320_vectors_take_pairs():
    assert A.plan("bwd", 1, 75600, 2560, BF16)["waves_per_row"] == 1
    assert A.plan("bwd", 1, 75600, 2568, BF16)["waves_per_row"] == 2
    assert A.plan("bwd", 1, 75600, 5120, BF16)["waves_per_row"] == 2
    assert A.plan("bwd", 1, 75600, 1280, F32)["waves_per_row"] == 1
    assert A.plan("bwd", 1, 75600, 1288, F32)["waves_per_row"] == 2
    # past 1280 vectors four wavefronts share a row, one row per workgroup,
    # up to 2560 vectors; past that eight (a 512-thread workgroup, one per
    # CU), up to the widest row, 4096 vectors
    for D, dt in ((10240, BF16), (5120, F32)):
        assert A.plan("bwd", 1, 75600, D, dt)["waves_per_row"] == 2
    for D, dt in ((10248, BF16), (20480, BF16), (5124, F32), (10240, F32)):
        p = A.plan("bwd", 1, 30000, D, dt)
        assert p["waves_per_row"] == 4 and p["walkers"] == 1
    for D, dt, V in ((20488, BF16, 6), (24576, BF16, 6), (24584, BF16, 8),
                     (32768, BF16, 8), (10244, F32, 6), (12288, F32, 6),
                     (12292, F32, 8), (16384, F32, 8)):
        p = A.plan("bwd", 3, 30000, D, dt)
        assert (p["waves_per_row"], p["walkers"], p["V"]) == (8, 1, V), (D, p)
        assert p["workgroups"] <= 256   # at most one per CU
        assert A.bwd_fused_plan(3, 30000, D, dt)["waves_per_row"] == 8
    # the forward keeps one wavefront per row up to 1024 vectors, then
    # pairs up to 1536 and quads up to 4096
    assert A.plan("fwd", 1, 75600, 8192, BF16)["waves_per_row"] == 1
    for D, dt, w in ((8200, BF16, 2), (12288, BF16, 2), (4100, F32, 2),
                     (6144, F32, 2), (12296, BF16, 4), (32768, BF16, 4),
                     (6148, F32, 4), (16384, F32, 4)):
        p = A.plan("fwd", 1, 30000, D, dt)
        assert p["waves_per_row"] == w and p["walkers"] == 4 // w, (D, p)


def test_forward_rows_take_a_grid_over_the_rows():
    # every row its own row walker: one wavefront up to 1024 vectors, a pair
    # or a quad of wavefronts beyond (4 / W rows per workgroup)
    for B, N, D, dt, W in ((16, 1560, 1536, BF16, 1), (1, 75600, 5120, BF16, 1),
                           (84, 1560, 3072, BF16, 1), (5, 7, 8192, BF16, 1),
                           (3, 5, 4096, F32, 1), (2, 256, 64, F32, 1),
                           (16, 8190, 12288, BF16, 2), (3, 7, 6144, F32, 2),
                           (1, 8192, 32768, BF16, 4), (5, 3, 16384, F32, 4)):
        p = A.plan("fwd", B, N, D, dt)
        assert p["waves_per_row"] == W and p["bps"] == 0, (B, N, D, p)
        assert p["workgroups"] == -(-B * N * W // 4)


def test_long_samples_fewer_in_flight():
    # short samples keep one group each
    assert A.plan("bwd", 84, 1560, 3072, BF16)["groups"] >= 84
    # the backward with pairs of wavefronts per row (2 walkers per
    # workgroup) follows the same rule: 16 rows per pair
    p = A.plan("bwd", 16, 8190, 3072, BF16)
    assert p["walkers"] == 2 and p["groups"] == 4
    assert 8190 / (p["bps"] * p["walkers"]) >= 16
    p = A.plan("bwd", 8, 16380, 3072, BF16)
    assert p["groups"] == 2 and 16380 / (p["bps"] * p["walkers"]) >= 16
    # the one-wavefront backward keeps one sample per slot
    assert A.plan("bwd", 16, 8190, 1536, BF16)["groups"] >= 16


def test_balanced_workgroups_per_sample():
    # 16 x 1560 rows, D = 1536: 30 workgroups of 4 walkers give every walker
    # 13 rows, as 32 would (12.2, rounded up) -- the fewest that do
    p = A.plan("bwd", 16, 1560, 1536, BF16)
    rows = -(-1560 // (p["bps"] * p["walkers"]))
    assert rows == -(-1560 // (32 * p["walkers"]))
    assert -(-1560 // ((p["bps"] - 1) * p["walkers"])) > rows


def test_skewed_walks_in_the_backward_of_many_samples():
    # one-wavefront backward rows, 16 or more samples: skewed by 97 rows
    assert A.plan("bwd", 16, 1560, 1536, BF16)["skew"] == 97
    assert A.plan("bwd", 15, 1560, 1536, BF16)["skew"] == 0
    # pairs of wavefronts (D = 3072), and the forward: aligned
    assert A.plan("bwd", 84, 1560, 3072, BF16)["skew"] == 0
    assert A.plan("fwd", 16, 1560, 1536, BF16)["skew"] == 0


@pytest.mark.parametrize("B,N,D,dt", _shapes(11, 100))
def test_dtile_grid_covers_every_row_and_feature(B, N, D, dt):
    """The (d_tile, n_tile, b) grid of adaln_bwd_dmod: d_tiles of 64
    vectors cover the row, n_tiles of n_tile rows cover the sample, one
    workgroup per (d_tile, n_tile, b), and its partial sums fit the
    workspace."""
    p = A.plan("dmod", B, N, D, dt)
    nvec = D // (8 if dt is BF16 else 4)
    assert p["d_tiles"] == -(-nvec // 64)
    assert p["n_tile"] % 16 == 0 and p["n_tile"] >= 16
    assert p["n_tile"] * p["n_tiles"] >= N > p["n_tile"] * (p["n_tiles"] - 1)
    assert p["workgroups"] == p["d_tiles"] * p["n_tiles"] * B
    assert A.bwd_workspace_bytes(B, N, D, dt) >= 2 * B * p["n_tiles"] * D * 4


def test_plan_validation():
    with pytest.raises(A.AdalnError):
        A.plan("fwd", 1, 1, 12, BF16)          # D not a multiple of 8
    with pytest.raises(ValueError):
        A.plan("both", 1, 1, 64, BF16)
    with pytest.raises(A.AdalnError) as e:
        A.plan("bwd", 1, 10, 32776, BF16)      # past the widest row
    assert e.value.code == -6


@pytest.mark.parametrize("B,N,D", [(1, 75600, 5120), (84, 1560, 3072),
                                   (16, 8190, 3072), (3, 7, 3072),
                                   (600, 3, 5120), (2, 32760, 3072)])
def test_weighted_walk_visits_every_row(B, N, D):
    """The backward of bf16 rows of D = 3072 and 5120 walks in rounds where
    the walkers of even workgroups take one extra row: every row of every
    sample is still visited exactly once, and those walkers take more rows."""
    p = A.plan("bwd", B, N, D, BF16)
    m = {3072: 12, 5120: 16}[D]
    assert p["waves_per_row"] == 2 and np.all(_visits(p, B, N, m) == 1)
    if N >= 2 * m * p["bps"] * p["walkers"]:
        per = [len(_weighted_positions(g, g, 0, p["bps"], p["walkers"], N, m))
               for g in range(min(p["bps"], 8))]
        assert min(per[0::2]) > max(per[1::2])
