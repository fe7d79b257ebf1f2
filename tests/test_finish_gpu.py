"""The launches that sum the backward's partial rows, checked exactly.

adaln_bwd_finish is called directly on a workspace whose partial rows hold
small integers, so every float32 sum is exact and must equal the integer sum
of the P partial rows of its (sample, feature); the bytes after the partial
rows hold NaN, so a read past them shows.  The cases cover every column-block
width (16, 32, 64 features), 1 to 16 wavefronts per block and several blocks
per workgroup (adaln_plan(2, ...) reports which).

The packed backward has no separate finishing entry point; with dy drawn as
small integers, dshift of every modulation vector is an exact integer sum
over the rows of every segment that uses the vector, so the segment finish's
row mapping is checked exactly through adaln_bwd_segments.
"""

import numpy as np
import pytest
import torch

import synth
from synth import workloads as W

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[finish] {msg}", flush=True)


@pytest.fixture(scope="module")
def A():
    import adaln_fwd_amd
    adaln_fwd_amd.load()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return adaln_fwd_amd


# (B, N, D, dtype): one shape per (F, wpc, cpb > 1) the planner produces,
# plus the large model's (511 partial rows) and a wide f32 row.
CASES = [
    (1, 1, 64, "bf16"), (8, 300, 64, "bf16"), (1, 300, 64, "bf16"),
    (2, 1560, 64, "bf16"), (1, 1560, 64, "bf16"), (8, 1, 520, "bf16"),
    (3, 64, 1536, "f32"), (8, 300, 520, "bf16"), (3, 300, 1536, "bf16"),
    (3, 300, 1536, "f32"), (2, 1, 8192, "bf16"), (4, 1, 8192, "bf16"),
    (32, 64, 520, "bf16"), (16, 64, 3072, "f32"), (2, 64, 8192, "bf16"),
    (4, 64, 8192, "bf16"), (4, 300, 5120, "f32"), (4, 300, 8192, "bf16"),
    (2, 300, 8192, "bf16"), (1, 75600, 5120, "bf16"), (16, 1560, 1536, "bf16"),
    (1, 32760, 1536, "bf16"), (84, 1560, 3072, "bf16"), (5, 999, 2560, "f32"),
]


def test_cases_cover_every_plan_family(A):
    seen = set()
    for B, N, D, dt in CASES:
        p = A.plan("finish", B, N, D, synth.torch_dtype(dt))
        seen.add((p["F"], p["wpc"], p["cpb"] > 1))
    for F in (16, 32, 64):
        for wpc in (1, 2, 4, 8, 16):
            assert (F, wpc, False) in seen, (F, wpc)
    assert any(k[2] for k in seen)


@pytest.mark.parametrize("B,N,D,dt", CASES)
def test_finish_exact_integer_sums(A, B, N, D, dt):
    tdt = synth.torch_dtype(dt)
    p = A.plan("finish", B, N, D, tdt)
    P = p["rows"]
    _say(f"B={B} N={N} D={D} {dt}: F={p['F']} wpc={p['wpc']} cpb={p['cpb']} "
         f"workgroups={p['workgroups']} P={P}")
    need = A.bwd_workspace_bytes(B, N, D, tdt)
    assert need >= 2 * B * P * D * 4
    g = torch.Generator().manual_seed(B * 1000003 + N * 101 + D)
    ints = torch.randint(-64, 65, (2, B, P, D), generator=g, dtype=torch.int64)
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32)
    ws[:ints.numel()] = ints.reshape(-1).float()
    ws = ws.cuda()
    pad = 64
    out = torch.full((2, B * D + 2 * pad), -3.0, dtype=torch.float32,
                     device="cuda")
    dscale = out[0, pad:pad + B * D].view(B, D)
    dshift = out[1, pad:pad + B * D].view(B, D)
    A.bwd_finish(ws.view(torch.uint8), B, N, D, tdt, dscale=dscale,
                 dshift=dshift)
    torch.cuda.synchronize()
    want = ints.sum(dim=2).double()
    assert torch.equal(dscale.cpu().double(), want[0])
    assert torch.equal(dshift.cpu().double(), want[1])
    guard = out.cpu()
    assert torch.all(guard[:, :pad] == -3.0) and torch.all(guard[:, -pad:] == -3.0)


def _layouts():
    """(D, lengths, mods, nmod): several segments per modulation vector,
    empty segments, and vectors no segment uses."""
    g = np.random.default_rng(5)
    out = [
        (64, [300, 0, 17, 1200, 5], [0, 1, 0, 0, 2], 4),
        (1536, [1560] * 6 + [40] * 10, [0, 1, 2, 0, 1, 2] + [3] * 10, 5),
        (3072, [8190, 512, 8190, 512, 1], [1, 0, 1, 0, 1], 2),
        (5120, [700, 1, 2000, 300], [2, 2, 0, 2], 3),
    ]
    for _ in range(4):
        nseg = int(g.integers(2, 129))
        D = int(g.choice([64, 520, 1536, 3072]))
        lengths = g.integers(0, max(2, 60000 // nseg), size=nseg).tolist()
        nmod = int(g.integers(1, nseg + 1))
        mods = g.integers(0, nmod, size=nseg).tolist()
        out.append((D, lengths, mods, nmod))
    return out


@pytest.mark.parametrize("case", range(8))
def test_segment_finish_exact_dshift(A, case):
    D, lengths, mods, nmod = _layouts()[case]
    T = int(sum(lengths))
    _say(f"segments {case}: D={D} nseg={len(lengths)} T={T} nmod={nmod}")
    wl = W.custom(1, max(T, 1), D, "bf16", x_kind="offset", dy_std=1.0)
    inp = synth.make_packed(wl, lengths, mods, nmod=nmod, seed=case)
    g = torch.Generator().manual_seed(case)
    dy = torch.randint(-4, 5, (T, D), generator=g).to(torch.bfloat16)
    dev = {k: getattr(inp, k).cuda() for k in ("x", "scale", "shift")}
    dyd = dy.cuda()
    y, mean, rstd = A.fwd_segments(dev["x"], dev["scale"], dev["shift"],
                                   inp.seg_offsets, inp.seg_mod)
    _, dscale, dshift = A.bwd_segments(dyd, dev["x"], dev["scale"], mean,
                                       rstd, inp.seg_offsets, inp.seg_mod)
    torch.cuda.synchronize()
    want = torch.zeros(nmod, D, dtype=torch.float64)
    off = inp.seg_offsets
    for s, m in enumerate(mods):
        want[m] += dy[off[s]:off[s + 1]].double().sum(dim=0)
    assert torch.equal(dshift.cpu().double(), want)
    assert torch.isfinite(dscale).all()
