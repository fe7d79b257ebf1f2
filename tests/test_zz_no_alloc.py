"""adaln_bwd_noalloc, the backward entry point that allocates nothing (its
partial rows live in the library's own static device scratch), called through
the C ABI and compared with adaln_bwd (same kernels, caller's workspace) on
two calls in a row, the second smaller than the first, and with the oracle.
(Shapes whose workspace exceeds the scratch are refused before any HIP call;
tests/test_abi.py checks that on the host.)"""

import pytest
import torch

import synth
from synth import workloads as W
from tests import parity as P

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[noalloc] {msg}", flush=True)


@pytest.fixture(scope="module")
def lib():
    import adaln_fwd_amd
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return adaln_fwd_amd.load()


def _p(t):
    return t.data_ptr() if t is not None and t.numel() > 0 else None


def _both(lib, wl, seed):
    """adaln_bwd with a workspace, then adaln_bwd_noalloc, on the same
    inputs; returns the inputs and both outputs (host copies)."""
    import adaln_fwd_amd as A
    B, N, D = wl.shape
    dt = synth.torch_dtype(wl.dtype)
    code = A.BF16 if dt == torch.bfloat16 else A.F32
    inp = synth.make_inputs(wl, seed=seed)
    dev = P.to_device(inp)
    y, mean, rstd = A.fwd(dev["x"], dev["scale"], dev["shift"])
    need = A.bwd_workspace_bytes(B, N, D, dt)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    outs = []
    s = torch.cuda.current_stream().cuda_stream
    for noalloc in (False, True):
        dx = torch.full_like(dev["x"], 7.0)
        ds = torch.full((B, D), 7.0, dtype=torch.float32, device="cuda")
        dh = torch.full((B, D), 7.0, dtype=torch.float32, device="cuda")
        if noalloc:
            rc = lib.adaln_bwd_noalloc(_p(dev["dy"]), _p(dev["x"]),
                                       _p(dev["scale"]), _p(mean), _p(rstd),
                                       _p(dx), _p(ds), _p(dh), B, N, D, code,
                                       s)
        else:
            rc = lib.adaln_bwd(_p(dev["dy"]), _p(dev["x"]), _p(dev["scale"]),
                               _p(mean), _p(rstd), _p(dx), _p(ds), _p(dh),
                               _p(ws), need, B, N, D, code, s)
        assert rc == 0, lib.adaln_last_error()
        torch.cuda.synchronize()
        outs.append(dict(dx=dx.cpu(), dscale=ds.cpu(), dshift=dh.cpu(),
                         y=y.cpu(), mean=mean.cpu(), rstd=rstd.cpu()))
    return inp, outs


def test_two_calls_in_a_row_second_smaller(lib):
    cases = [W.custom(1, 75600, 5120, "bf16", x_kind="outliers",
                      dy_std=1e-2),
             W.custom(16, 1560, 1536, "bf16", x_kind="offset", dy_std=1e-2)]
    for k, wl in enumerate(cases):
        _say(f"call {k}: {wl.shape} {wl.dtype}")
        inp, (ref, got) = _both(lib, wl, seed=k)
        for key in ("dx", "dscale", "dshift"):
            assert torch.equal(ref[key], got[key]), key
        for r in P.compare_full(inp, got, wl.dtype, with_rows=False):
            _say(f"  {r}")
        if k == 1:
            for r in P.compare_full(inp, got, wl.dtype):
                _say(f"  {r}")


@pytest.mark.parametrize("D", [12288, 32768])
def test_wide_rows(lib, D):
    # four wavefronts per row in the fused backward (12288), and eight
    # (32768: 2 samples x 100 workgroups of partial rows, 50 of the 64 MiB
    # of scratch)
    wl = W.custom(2, 300, D, "bf16", x_kind="normal", dy_std=1e-2)
    _say(f"wide rows {wl.shape}")
    inp, (ref, got) = _both(lib, wl, seed=5)
    for key in ("dx", "dscale", "dshift"):
        assert torch.equal(ref[key], got[key]), key
    for r in P.compare_full(inp, got, wl.dtype):
        _say(f"  {r}")


def test_f32_and_empty(lib):
    import adaln_fwd_amd as A
    wl = W.custom(3, 257, 1024, "f32", x_kind="offset", dy_std=1.0)
    _say(f"f32 {wl.shape}")
    inp, (ref, got) = _both(lib, wl, seed=9)
    for key in ("dx", "dscale", "dshift"):
        assert torch.equal(ref[key], got[key]), key
    # no rows: dscale and dshift are zero, nothing else is touched
    ds = torch.full((2, 64), 7.0, device="cuda")
    dh = torch.full((2, 64), 7.0, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    assert lib.adaln_bwd_noalloc(None, None, None, None, None, None, _p(ds),
                                 _p(dh), 2, 0, 64, A.F32, s) == 0
    torch.cuda.synchronize()
    assert torch.equal(ds.cpu(), torch.zeros(2, 64))
    assert torch.equal(dh.cpu(), torch.zeros(2, 64))
