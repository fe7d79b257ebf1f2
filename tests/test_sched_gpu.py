"""The shape benchmark's synthetic step runs on the GPU (AdaLN forward,
fused attention, AdaLN backward) and yields finite, positive durations."""

import math

import pytest

pytestmark = pytest.mark.gpu


def test_synthetic_step_times():
    from adaln_fwd_amd import sched
    print("[sched] synthetic step B=2 S=1560 D=3072", flush=True)
    step = sched.SyntheticStep(D=3072, heads=24)
    ms = step.run(2, 1560, iters=3, warmup=1)
    assert len(ms) == 3 and all(math.isfinite(v) and v > 0 for v in ms)
