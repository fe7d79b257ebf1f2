"""The shape benchmark's synthetic step (AdaLN forward, fused attention
forward and backward, AdaLN backward) on the GPU: finite, positive
durations, and AdaLN results inside the step that equal, bit for bit, those
of adaln_fwd / adaln_bwd called on their own with the same inputs, which in
turn match the oracle."""

import math

import pytest
import torch

import synth
from tests import parity as P

pytestmark = pytest.mark.gpu


def test_synthetic_step_times_and_results():
    import adaln_fwd_amd as A
    from adaln_fwd_amd import sched
    print("[sched] synthetic step B=2 S=1560 D=3072", flush=True)
    step = sched.SyntheticStep(D=3072, heads=24)
    ms = step.run(2, 1560, iters=3, warmup=1)
    assert len(ms) == 3 and all(math.isfinite(v) and v > 0 for v in ms)
    got = step.last
    y, mean, rstd = A.fwd(got["x"], got["scale"], got["shift"])
    dx, dscale, dshift = A.bwd(got["dy"], got["x"], got["scale"], mean, rstd)
    torch.cuda.synchronize()
    alone = dict(y=y, mean=mean, rstd=rstd, dx=dx, dscale=dscale,
                 dshift=dshift)
    for k, v in alone.items():
        assert torch.equal(v, got[k]), k
    inp = synth.Inputs(x=got["x"].cpu(), scale=got["scale"].cpu(),
                       shift=got["shift"].cpu(), dy=got["dy"].cpu(),
                       workload=None, seed=0, bucket=0)
    out = {k: v.cpu() for k, v in alone.items()}
    for r in P.compare_full(inp, out, "bf16"):
        print(f"[sched]   {r}", flush=True)
