"""Packed variable-length entry points (adaln_fwd_segments,
adaln_bwd_segments) against the oracle's segment functions: several
sequences back to back in one [T, D] tensor, each with its own modulation
vector -- mixed-length samples packed without padding, and the text and
video token segments of two-stream (MMDiT) samples.

Every case is compared in full: small layouts element by element in Python,
the full-size packed mixed-length pack and the MMDiT layout row by row through
the oracle library's row checker, with dscale and dshift in full.
"""

import numpy as np
import pytest
import torch

import synth
from synth import workloads as W
from tests import parity as P

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[segments] {msg}", flush=True)


@pytest.fixture(scope="module")
def A():
    import adaln_fwd_amd
    adaln_fwd_amd.load()
    return adaln_fwd_amd


def _wl(D, dtype, x_kind="offset", dy_std=1e-2):
    return W.custom(1, 1, D, dtype, x_kind=x_kind, dy_std=dy_std, index=107)


SMALL = [
    # D, dtype, lengths, seg_mod (None: identity), nmod
    (256, "f32", [300, 0, 1, 77, 1024], [2, 0, 2, 1, 0], 4),   # vector 3 unused
    (1536, "bf16", [1560, 390, 5], None, 3),
    (520, "bf16", [17, 250, 3], [0, 0, 0], 1),                  # ragged row
    (2560, "f32", [100, 200], [1, 0], 2),                       # widest f32 bwd
    (5120, "bf16", [40, 1, 333], None, 3),                      # widest bf16 bwd
    (64, "f32", [2000, 7], None, 2),                            # row of 16 vectors
    (1536, "bf16", [20000] + [1] * 40, [0] * 41, 1),            # one long, many tiny
    (8192, "bf16", [300, 0, 17, 1001], [1, 0, 1, 2], 3),        # two-wavefront rows
    (7000, "bf16", [5, 64, 3], None, 3),                        # ragged two-wavefront
    (4096, "f32", [100, 257], [0, 0], 1),
    (10240, "bf16", [33, 0, 120], [0, 1, 0], 2),   # widest paired bwd
    # four wavefronts per backward row (1281..2560 vectors), and per
    # forward row past 1536
    (10248, "bf16", [7, 130, 0, 1], [0, 1, 1, 0], 2),  # narrowest, ragged
    (20480, "bf16", [40, 3], None, 2),                 # widest quad bwd
    (6144, "f32", [99, 0, 250], [2, 0, 1], 3),
    # eight wavefronts per backward row (2561..4096 vectors)
    (20488, "bf16", [10, 0, 21, 1], [1, 0, 0, 1], 2),  # narrowest, ragged
    (32768, "bf16", [6, 40], None, 2),                 # widest row
    (28000, "bf16", [3, 17, 9], [0, 2, 0], 3),         # scale read at use
    (16384, "f32", [25, 2], [0, 0], 1),                # widest f32 row
    (10244, "f32", [1, 50], None, 2),                  # ragged f32
]


@pytest.mark.parametrize("case", range(len(SMALL)))
def test_small_layouts_full(A, case):
    D, dt, lengths, mods, nmod = SMALL[case]
    _say(f"small case {case}: D={D} {dt} nseg={len(lengths)} "
         f"T={sum(lengths)} nmod={nmod}")
    inp = synth.make_packed(_wl(D, dt), lengths, mods, nmod=nmod, seed=case)
    out = P.gpu_packed(inp, P.packed_to_device(inp))
    torch.cuda.synchronize()
    out = {k: v.cpu() for k, v in out.items()}
    for r in P.compare_packed_full(inp, out, dt):
        _say(f"  {r}")


def test_128_segments_random_table(A):
    """The largest table: 128 segments of 0..300 rows (some empty), random
    modulation indices (some vectors unused), inside guard bytes."""
    g = np.random.default_rng(3)
    lengths = g.integers(0, 300, size=128)
    lengths[[5, 17, 90]] = 0
    mods = g.integers(0, 60, size=128).astype(np.int32)
    D = 3072
    _say(f"128 segments, T={lengths.sum()} D={D}")
    inp = synth.make_packed(_wl(D, "bf16"), lengths, mods, nmod=64, seed=9)
    dev = P.packed_to_device(inp)
    T, nmod = int(lengths.sum()), 64
    pad = 4096

    def guarded(n, dtype):
        buf = torch.full((n + 2 * pad,), -7.0, dtype=dtype, device="cuda")
        return buf, buf[pad:pad + n]

    yb, y = guarded(T * D, torch.bfloat16)
    mb, mean = guarded(T, torch.float32)
    rb, rstd = guarded(T, torch.float32)
    xb, dx = guarded(T * D, torch.bfloat16)
    sb, dscale = guarded(nmod * D, torch.float32)
    hb, dshift = guarded(nmod * D, torch.float32)
    need = A.bwd_segments_workspace_bytes(inp.seg_offsets, D, torch.bfloat16)
    wb, ws = guarded(need // 4, torch.float32)
    A.fwd_segments(dev["x"], dev["scale"], dev["shift"], inp.seg_offsets,
                   inp.seg_mod, y=y.view(T, D), mean=mean, rstd=rstd)
    A.bwd_segments(dev["dy"], dev["x"], dev["scale"], mean, rstd,
                   inp.seg_offsets, inp.seg_mod, dx=dx.view(T, D),
                   dscale=dscale.view(nmod, D), dshift=dshift.view(nmod, D),
                   workspace=ws)
    torch.cuda.synchronize()
    for buf in (yb, mb, rb, xb, sb, hb, wb):
        assert torch.all(buf[:pad] == -7.0) and torch.all(buf[-pad:] == -7.0)
    out = dict(y=y.view(T, D).cpu(), mean=mean.cpu(), rstd=rstd.cpu(),
               dx=dx.view(T, D).cpu(), dscale=dscale.view(nmod, D).cpu(),
               dshift=dshift.view(nmod, D).cpu())
    for r in P.compare_packed_full(inp, out, "bf16"):
        _say(f"  {r}")
    unused = sorted(set(range(nmod)) - set(int(m) for m in mods))
    assert unused and not out["dscale"][unused].any()


def test_uniform_layout_matches_batched_path(A):
    """B equal segments with the identity table are the batched layout: the
    per-row outputs are the same kernels' arithmetic, bit for bit; dscale
    and dshift are sums in another grouping, so within tolerance."""
    B, N, D = 6, 1000, 1536
    _say(f"uniform layout B={B} N={N} D={D}")
    inp = synth.make_packed(_wl(D, "bf16"), [N] * B, seed=4)
    dev = P.packed_to_device(inp)
    seg = P.gpu_packed(inp, dev)
    bat = dict(x=dev["x"].view(B, N, D), scale=dev["scale"],
               shift=dev["shift"], dy=dev["dy"].view(B, N, D))
    ref = P.gpu_fwd_bwd(bat)
    torch.cuda.synchronize()
    assert torch.equal(seg["y"], ref["y"].view(B * N, D))
    assert torch.equal(seg["mean"], ref["mean"].view(-1))
    assert torch.equal(seg["rstd"], ref["rstd"].view(-1))
    assert torch.equal(seg["dx"], ref["dx"].view(B * N, D))
    P.check_dmod("dscale", seg["dscale"].cpu(), ref["dscale"].cpu().double())
    P.check_dmod("dshift", seg["dshift"].cpu(), ref["dshift"].cpu().double())


def test_deterministic(A):
    lengths, mods = [700, 3, 4096, 0, 129], [3, 1, 0, 2, 1]
    inp = synth.make_packed(_wl(3072, "bf16"), lengths, mods, nmod=4, seed=2)
    dev = P.packed_to_device(inp)
    a = P.gpu_packed(inp, dev)
    b = P.gpu_packed(inp, dev)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k], b[k]), k


WIDE_FORWARD = [
    # D, dtype, lengths, seg_mod, nmod: rows past 1024 vectors (pairs and
    # quads of wavefronts)
    (16384, "bf16", [10, 20, 0, 7], [1, 0, 1, 0], 2),
    (32768, "bf16", [3, 5], None, 2),                 # widest row
    (12288, "bf16", [1, 200, 31], [0, 0, 0], 1),
    (16384, "f32", [4, 9], None, 2),                  # widest f32 row
    (8200, "bf16", [64, 1], None, 2),                 # ragged, just past 1024
    (6148, "f32", [33, 100], [1, 1], 2),              # ragged quad, f32
    (14000, "f32", [20, 0, 33], [1, 0, 1], 2),        # f32, late scale loads
]


@pytest.mark.parametrize("case", range(len(WIDE_FORWARD)))
def test_wide_forward_full(A, case):
    """The forward of rows wider than one wavefront holds, packed, against
    the oracle on every element."""
    import oracle
    D, dt, lengths, mods, nmod = WIDE_FORWARD[case]
    _say(f"wide forward case {case}: D={D} {dt} lengths={lengths}")
    inp = synth.make_packed(_wl(D, dt), lengths, mods, nmod=nmod, seed=case)
    dev = P.packed_to_device(inp)
    y, mean, rstd = A.fwd_segments(dev["x"], dev["scale"], dev["shift"],
                                   inp.seg_offsets, inp.seg_mod)
    torch.cuda.synchronize()
    ry, rm, rr = oracle.fwd_segments(inp.x, inp.scale, inp.shift,
                                     inp.seg_offsets, inp.seg_mod)
    for r in P.check_out("y", y.cpu(), ry, dt):
        _say(f"  {r}")
    for r in P.check_stats(mean.cpu(), rstd.cpu(), rm, rr, inp.x):
        _say(f"  {r}")


def test_wide_forward_uniform_matches_batched(A):
    """Equal segments with the identity table through the wide kernel equal
    the batched forward bit for bit (same per-row arithmetic)."""
    B, N, D = 3, 300, 16384
    inp = synth.make_packed(_wl(D, "bf16"), [N] * B, seed=5)
    dev = P.packed_to_device(inp)
    y, mean, rstd = A.fwd_segments(dev["x"], dev["scale"], dev["shift"],
                                   inp.seg_offsets)
    ref = A.fwd(dev["x"].view(B, N, D), dev["scale"], dev["shift"])
    torch.cuda.synchronize()
    assert torch.equal(y, ref[0].view(B * N, D))
    assert torch.equal(mean, ref[1].view(-1))
    assert torch.equal(rstd, ref[2].view(-1))


def test_wide_rows_rejected(A):
    """Rows past the widest row (4096 vectors) are refused before anything
    is enqueued, by the packed forward and backward alike."""
    x = torch.zeros(4, 32776, device="cuda", dtype=torch.bfloat16)
    v = torch.zeros(1, 32776, device="cuda", dtype=torch.bfloat16)
    m = torch.zeros(4, device="cuda")
    off = np.array([0, 4], dtype=np.int64)
    with pytest.raises(A.AdalnError) as e:
        A.fwd_segments(x, v, v, off)
    assert e.value.code == -6
    with pytest.raises(A.AdalnError) as e:
        A.bwd_segments(x, x, v, m, m, off)
    assert e.value.code == -6


def _full_size(A, inp, name):
    """Every row of y, dx, mean and rstd (through the oracle's row checker,
    each row with its segment's modulation vector) and dscale/dshift in
    full."""
    T = int(inp.seg_offsets[-1])
    D = inp.x.shape[1]
    _say(f"{name}: nseg={len(inp.seg_offsets) - 1} T={T} D={D}, every row")
    dev = P.packed_to_device(inp)
    out = P.gpu_packed(inp, dev)
    torch.cuda.synchronize()
    got = {k: v.cpu() for k, v in out.items()}
    del dev, out
    for r in P.check_all_rows(inp.x, inp.dy, inp.scale, inp.shift, got,
                              "bf16", row_mod=P.row_mods(inp)):
        _say(f"  rows {r}")
    for r in P.compare_packed_full(inp, got, "bf16", with_rows=False):
        _say(f"  full {r}")


def test_packed_mixed_full_size(A):
    lengths = synth.pack_lengths(seed=0)
    inp = synth.make_packed(synth.PACKED_MIXED, lengths, seed=0)
    _full_size(A, inp, "packed mixed-length pack")


def test_mmdit_layout_full_size(A):
    wl = synth.MMDIT_PACKED
    lengths, mods = synth.mmdit_layout(wl.B)
    inp = synth.make_packed(wl, lengths, mods, nmod=2 * wl.B, seed=0)
    _full_size(A, inp, "two-stream layout")


def test_forward_launches_past_2_22_rows(A):
    """Packed rows past one launch of the forward's row grid (2^22 rows):
    the middle segment spans the launch boundary; every row and
    dscale/dshift against the oracle."""
    lengths = [4_000_000, 194_305, 1000]
    assert lengths[0] < 1 << 22 < lengths[0] + lengths[1]
    inp = synth.make_packed(_wl(8, "bf16", x_kind="normal"), lengths,
                            [1, 0, 1], nmod=2, seed=5)
    _full_size(A, inp, "pack past one forward launch")


def _random_tables(seed, count):
    g = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        dtype = "bf16" if g.random() < 0.75 else "f32"
        E = 8 if dtype == "bf16" else 4
        nvec = int(g.choice([g.integers(1, 65), g.integers(65, 641),
                             g.integers(641, 1025)], p=[0.3, 0.5, 0.2]))
        nseg = int(g.integers(1, 129))
        lengths = g.integers(0, max(2, 40000 // (nseg * nvec)), size=nseg)
        nmod = int(g.integers(1, nseg + 1))
        mods = g.integers(0, nmod, size=nseg).tolist()
        out.append((nvec * E, dtype, lengths.tolist(), mods, nmod))
    return out


@pytest.mark.parametrize("case", range(8))
def test_random_tables(A, case):
    """Seeded random segment tables (1-128 segments, empty ones, shared and
    unused vectors) at widths of every kernel family, compared in full."""
    D, dt, lengths, mods, nmod = _random_tables(77, 8)[case]
    _say(f"random table {case}: D={D} {dt} nseg={len(lengths)} "
         f"T={sum(lengths)} nmod={nmod}")
    inp = synth.make_packed(_wl(D, dt), lengths, mods, nmod=nmod, seed=case)
    out = P.gpu_packed(inp, P.packed_to_device(inp))
    torch.cuda.synchronize()
    out = {k: v.cpu() for k, v in out.items()}
    P.compare_packed_full(inp, out, dt)
