"""The mixed-length batch schedule at full size: 64 buckets drawn uniformly
from S in {1560, 8190, 16380, 32760}, each with the dual-constraint batch
B_shape(S) (M_mem = 131072, M_comp = 2.2e9, p = 2), D = 3072, bf16, run
through adaln_fwd and adaln_bwd exactly as the benchmark does: one set of
device buffers sized for the largest bucket, reused by every bucket.

One test per bucket: y, dx, mean and rstd on every token row against the
oracle (through the oracle library's row checker); dscale and dshift in full
against the oracle, and dshift also against its closed form (the float64 sum
of dy over the tokens of each sample).
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


@pytest.fixture(scope="module")
def schedule():
    """The schedule's lengths, batch sizes and the shared device buffers."""
    import adaln_fwd_amd as A
    sched = synth.mixed_schedule()
    assert len(sched) == synth.MIXED_BUCKETS
    shapes = {S: A.bshape(S, synth.MIXED_M_MEM, synth.MIXED_M_COMP,
                          synth.MIXED_P) for S in set(sched)}
    D = synth.MIXED_SCHEDULE.D
    max_rows = max(b * S for S, b in shapes.items())
    dev = torch.device("cuda")
    bufs = {k: torch.empty(max_rows * D, dtype=torch.bfloat16, device=dev)
            for k in ("x", "dy", "y", "dx")}
    bufs["ws"] = torch.empty(max(A.bwd_workspace_bytes(b, S, D, torch.bfloat16)
                                 for S, b in shapes.items()),
                             dtype=torch.uint8, device=dev)
    yield sched, shapes, D, bufs
    del bufs
    torch.cuda.empty_cache()


@pytest.mark.parametrize("k", range(synth.MIXED_BUCKETS))
def test_mixed_bucket_full_size(schedule, k):
    import adaln_fwd_amd as A
    sched, shapes, D, bufs = schedule
    S = sched[k]
    B = shapes[S]
    dev = bufs["x"].device
    _say(f"bucket {k}: B={B} S={S} D={D}")
    inp = synth.make_inputs(synth.mixed_bucket(B, S), bucket=k)
    n = B * S * D
    x, dy, y, dx = (bufs[key][:n].view(B, S, D) for key in ("x", "dy", "y",
                                                             "dx"))
    x.copy_(inp.x)
    dy.copy_(inp.dy)
    scale = inp.scale.to(dev)
    shift = inp.shift.to(dev)
    _, mean, rstd = A.fwd(x, scale, shift, y=y)
    _, dscale, dshift = A.bwd(dy, x, scale, mean, rstd, dx=dx,
                              workspace=bufs["ws"])
    torch.cuda.synchronize()
    got = dict(y=y.cpu(), dx=dx.cpu(), mean=mean.cpu(), rstd=rstd.cpu(),
               dscale=dscale.cpu(), dshift=dshift.cpu())
    reps = list(P.compare_all_rows(inp, got, "bf16"))
    reps += P.compare_full(inp, got, "bf16", with_rows=False)
    reps.append(P.check_dmod("dshift[closed form]", got["dshift"],
                             inp.dy.double().sum(dim=1).numpy()))
    _say("; ".join(str(r) for r in reps))
