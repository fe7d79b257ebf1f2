"""The entry points inside a captured graph: they allocate nothing, set no
memory with memset nodes and never synchronise, so torch.cuda.graph can
capture a forward + backward; every replay (with eager work of the program
between replays) must equal the eager results bit for bit."""

import pytest
import torch

import synth
from synth import workloads as W
from tests import parity as P

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[graph] {msg}", flush=True)


def _replays_match(run, outs, eager, other):
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()                        # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run()
    for i in range(3):
        for t in outs:
            t.fill_(float("nan")) if t.is_floating_point() else t.zero_()
        other()                      # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        for t, e in zip(outs, eager):
            assert torch.equal(t, e), f"replay {i}"


def test_batched_fwd_bwd_in_a_graph():
    import adaln_fwd_amd as A
    B, N, D = 4, 1000, 1536
    _say(f"batched B={B} N={N} D={D} bf16")
    dev = P.to_device(synth.make_inputs(W.custom(B, N, D, "bf16",
                                                 x_kind="offset",
                                                 dy_std=1e-2)))
    y = torch.empty_like(dev["x"])
    dx = torch.empty_like(dev["x"])
    mean = torch.empty(B, N, device="cuda")
    rstd = torch.empty(B, N, device="cuda")
    ds = torch.empty(B, D, device="cuda")
    dh = torch.empty(B, D, device="cuda")
    ws = torch.empty(A.bwd_workspace_bytes(B, N, D, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")

    def run():
        A.fwd(dev["x"], dev["scale"], dev["shift"], y=y, mean=mean, rstd=rstd)
        A.bwd(dev["dy"], dev["x"], dev["scale"], mean, rstd, dx=dx,
              dscale=ds, dshift=dh, workspace=ws)

    run()
    torch.cuda.synchronize()
    outs = [y, mean, rstd, dx, ds, dh]
    eager = [t.clone() for t in outs]
    junk = torch.empty_like(dev["x"])

    def other():
        A.fwd(dev["dy"], dev["scale"], dev["shift"], y=junk)

    _replays_match(run, outs, eager, other)


def test_packed_fwd_bwd_in_a_graph():
    import adaln_fwd_amd as A
    lengths, mods = [700, 3, 2048, 0, 129], [3, 1, 0, 2, 1]
    _say(f"packed lengths={lengths}")
    inp = synth.make_packed(W.custom(1, 1, 3072, "bf16", x_kind="offset",
                                     dy_std=1e-2), lengths, mods, nmod=4)
    dev = P.packed_to_device(inp)
    table = A.SegTable(inp.seg_offsets, inp.seg_mod)
    T, D = inp.x.shape
    y = torch.empty_like(dev["x"])
    dx = torch.empty_like(dev["x"])
    mean = torch.empty(T, device="cuda")
    rstd = torch.empty(T, device="cuda")
    ds = torch.empty(4, D, device="cuda")
    dh = torch.empty(4, D, device="cuda")
    ws = torch.empty(A.bwd_segments_workspace_bytes(table, D, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")

    def run():
        A.fwd_segments(dev["x"], dev["scale"], dev["shift"], table, y=y,
                       mean=mean, rstd=rstd)
        A.bwd_segments(dev["dy"], dev["x"], dev["scale"], mean, rstd, table,
                       dx=dx, dscale=ds, dshift=dh, workspace=ws)

    run()
    torch.cuda.synchronize()
    outs = [y, mean, rstd, dx, ds, dh]
    eager = [t.clone() for t in outs]
    junk = torch.empty_like(dev["x"])

    def other():
        A.fwd_segments(dev["dy"], dev["scale"], dev["shift"], table, y=junk)

    _replays_match(run, outs, eager, other)
