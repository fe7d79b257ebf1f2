"""The oracle library's row checker (oracle/check_rows.c), which the GPU
parity tests use to compare every token row of the large workloads, against
the element-by-element comparison of tests/parity.py on the same data.

The "device" outputs here are the oracle's own float64 results rounded to the
storage type on the CPU (what a correctly rounding device would write), with
mistakes planted in copies of them; no GPU is involved.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import workloads as W
from tests import parity as P


def _rounded_outputs(inp, dtype):
    dt = synth.torch_dtype(dtype)
    y, mean, rstd = oracle.fwd(inp.x, inp.scale, inp.shift)
    dx, _, _ = oracle.bwd(inp.dy, inp.x, inp.scale, want_dmod=False)
    return dict(y=torch.from_numpy(y).to(dt), dx=torch.from_numpy(dx).to(dt),
                mean=torch.from_numpy(mean).float(),
                rstd=torch.from_numpy(rstd).float())


def _numpy_reports(inp, got, dtype):
    y, mean, rstd = oracle.fwd(inp.x, inp.scale, inp.shift)
    dx, _, _ = oracle.bwd(inp.dy, inp.x, inp.scale, want_dmod=False)
    reps = list(P.check_out("y", got["y"], y, dtype))
    reps += P.check_out("dx", got["dx"], dx, dtype)
    reps += P.check_stats(got["mean"], got["rstd"], mean, rstd, inp.x)
    return {r.name: r for r in reps}


CASES = [(3, 50, 264, "bf16", "offset"), (2, 70, 1536, "bf16", "outliers"),
         (2, 40, 64, "f32", "normal"), (1, 33, 520, "f32", "offset")]


@pytest.mark.parametrize("B,N,D,dtype,kind", CASES)
def test_checker_agrees_with_elementwise_comparison(B, N, D, dtype, kind):
    wl = W.custom(B, N, D, dtype, x_kind=kind,
                  dy_std=1e-2 if dtype == "bf16" else 1.0)
    inp = synth.make_inputs(wl, seed=7)
    got = _rounded_outputs(inp, dtype)
    ref = _numpy_reports(inp, got, dtype)
    full = {r.name: r for r in P.compare_all_rows(inp, got, dtype)}
    assert set(full) == set(ref)
    for name, r in ref.items():
        f = full[name]
        assert f.n == r.n, name
        assert f.max_err == pytest.approx(r.max_err, rel=1e-12, abs=1e-300)
        if name.endswith("[strict]") or dtype == "f32" and name in ("y", "dx"):
            # the checker reports the worst excess over the rms floor; both
            # pass, and a worse element raises both (tests below)
            assert f.max_ratio <= 1.0 and r.max_ratio <= 1.0
        else:
            assert f.max_ratio == pytest.approx(r.max_ratio, rel=1e-9), name
        if r.normwise is not None:
            assert f.normwise == pytest.approx(r.normwise, rel=1e-9)
        assert f.over_plain == r.over_plain, name


def _inputs(dtype="bf16"):
    wl = W.custom(2, 40, 512, dtype, x_kind="offset",
                  dy_std=1e-2 if dtype == "bf16" else 1.0)
    inp = synth.make_inputs(wl, seed=3)
    return inp, _rounded_outputs(inp, dtype)


def _both_fail(inp, got, dtype):
    with pytest.raises(AssertionError, match="parity failure|non-finite"):
        _numpy_reports(inp, got, dtype)
    with pytest.raises(AssertionError, match="parity failure|non-finite"):
        P.compare_all_rows(inp, got, dtype)


@pytest.mark.parametrize("what", ["y", "dx"])
def test_planted_contract_error_fails(what):
    inp, got = _inputs()
    got[what][1, 17, 300] += 0.5
    _both_fail(inp, got, "bf16")


def test_planted_strict_only_error_fails():
    # dx entries are ~1e-2: an error of 3e-3 passes the 2e-2 contract bound
    # but is many bf16 ulps off, which the strict bound catches
    inp, got = _inputs()
    v = float(got["dx"][0, 5, 7])
    got["dx"][0, 5, 7] = v + 3e-3
    _both_fail(inp, got, "bf16")


def test_planted_f32_error_fails():
    inp, got = _inputs("f32")
    got["y"][1, 3, 9] *= 1.0001
    _both_fail(inp, got, "f32")


@pytest.mark.parametrize("what", ["mean", "rstd"])
def test_planted_stat_error_fails(what):
    inp, got = _inputs()
    got[what][0, 11] *= 1.001
    _both_fail(inp, got, "bf16")


def test_planted_nan_fails():
    inp, got = _inputs()
    got["y"][0, 0, 0] = float("nan")
    with pytest.raises(AssertionError, match="non-finite"):
        P.compare_all_rows(inp, got, "bf16")


def test_last_row_is_checked():
    inp, got = _inputs()
    got["dx"][-1, -1, -1] += 0.5
    with pytest.raises(AssertionError, match="parity failure"):
        P.compare_all_rows(inp, got, "bf16")


def test_row_modulation_index():
    """Rows modulated through an explicit index table give the same result
    as the batched rule r // N; a wrong index is caught."""
    inp, got = _inputs()
    B, N, D = inp.x.shape
    flat = {k: got[k].reshape(B * N, -1).squeeze(-1) if k in ("mean", "rstd")
            else got[k].reshape(B * N, D) for k in got}
    mods = np.repeat(np.arange(B), N)
    reps = P.check_all_rows(inp.x.reshape(B * N, D), inp.dy.reshape(B * N, D),
                            inp.scale, inp.shift, flat, "bf16", row_mod=mods)
    ref = {r.name: r for r in P.compare_all_rows(inp, got, "bf16")}
    for r in reps:
        assert r.max_err == ref[r.name].max_err
    with pytest.raises(AssertionError, match="parity failure"):
        P.check_all_rows(inp.x.reshape(B * N, D), inp.dy.reshape(B * N, D),
                         inp.scale, inp.shift, flat, "bf16",
                         row_mod=mods[::-1].copy())
