"""The mixed-length batch schedule at full size: 64 buckets drawn uniformly
from S in {1560, 8190, 16380, 32760}, each with the dual-constraint batch
B_shape(S) (M_mem = 131072, M_comp = 2.2e9, p = 2), D = 3072, bf16, run
through adaln_fwd and adaln_bwd exactly as the benchmark does.

Per bucket: y, dx, mean and rstd on sampled token rows against the oracle,
and dshift against its closed form (the float64 sum of dy over the tokens of
each sample).  dscale and dshift in full against the oracle for the first
bucket of each sequence length.
"""

import numpy as np
import pytest
import torch

import synth
from tests import parity as P

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[mixed] {msg}", flush=True)


def test_bucket_sizes_match_oracle_and_constraints(oracle_mod):
    import adaln_fwd_amd as A
    for S in synth.MIXED_LENGTHS:
        b = A.bshape(S, synth.MIXED_M_MEM, synth.MIXED_M_COMP, synth.MIXED_P)
        assert b == oracle_mod.bshape(S, synth.MIXED_M_MEM, synth.MIXED_M_COMP,
                                      synth.MIXED_P)
        assert b == 1 or (b * S <= synth.MIXED_M_MEM
                          and b * S ** 2 <= synth.MIXED_M_COMP)


def test_mixed_schedule_full_size(oracle_mod):
    import adaln_fwd_amd as A
    sched = synth.mixed_schedule()
    shapes = {S: A.bshape(S, synth.MIXED_M_MEM, synth.MIXED_M_COMP,
                          synth.MIXED_P) for S in set(sched)}
    D = synth.MIXED_SCHEDULE.D
    max_rows = max(b * S for S, b in shapes.items())
    dev = torch.device("cuda")
    x_buf = torch.empty(max_rows * D, dtype=torch.bfloat16, device=dev)
    dy_buf = torch.empty_like(x_buf)
    y_buf = torch.empty_like(x_buf)
    dx_buf = torch.empty_like(x_buf)
    max_b = max(shapes.values())
    ws = torch.empty(max(A.bwd_workspace_bytes(b, S, D, torch.bfloat16)
                         for S, b in shapes.items()), dtype=torch.uint8,
                     device=dev)
    full_checked = set()
    tokens = 0
    for k, S in enumerate(sched):
        B = shapes[S]
        wl = synth.mixed_bucket(B, S)
        _say(f"bucket {k}: B={B} S={S} D={D}")
        inp = synth.make_inputs(wl, bucket=k)
        n = B * S * D
        x = x_buf[:n].view(B, S, D)
        dy = dy_buf[:n].view(B, S, D)
        y = y_buf[:n].view(B, S, D)
        dx = dx_buf[:n].view(B, S, D)
        x.copy_(inp.x)
        dy.copy_(inp.dy)
        scale = inp.scale.to(dev)
        shift = inp.shift.to(dev)
        _, mean, rstd = A.fwd(x, scale, shift, y=y)
        _, dscale, dshift = A.bwd(dy, x, scale, mean, rstd, dx=dx,
                                  workspace=ws)
        rows = P.sample_rows(B * S, 48, seed=k)
        idx = torch.from_numpy(rows).to(dev)
        out = dict(y=y.view(B * S, D).index_select(0, idx).cpu(),
                   dx=dx.view(B * S, D).index_select(0, idx).cpu(),
                   mean=mean.view(-1).index_select(0, idx).cpu(),
                   rstd=rstd.view(-1).index_select(0, idx).cpu(),
                   dscale=dscale.cpu(), dshift=dshift.cpu())
        torch.cuda.synchronize()
        # the sampled rows, compared in the compact layout
        compact = {key: out[key] for key in ("y", "dx")}
        ref = P.oracle_rows(inp, rows)
        P.check_out("y", compact["y"], ref["y"], "bf16")
        P.check_out("dx", compact["dx"], ref["dx"], "bf16")
        P.check_stats(out["mean"], out["rstd"], ref["mean"], ref["rstd"],
                      ref["x"])
        # dshift: the plain float64 sum of dy over each sample's tokens
        P.check_dmod("dshift", out["dshift"],
                     inp.dy.double().sum(dim=1).numpy())
        if S not in full_checked:
            full_checked.add(S)
            for r in P.compare_full(inp, out, "bf16", with_rows=False):
                _say(f"  full {r}")
        tokens += B * S
    _say(f"{len(sched)} buckets, {tokens} tokens checked")
    assert full_checked == set(synth.MIXED_LENGTHS)
