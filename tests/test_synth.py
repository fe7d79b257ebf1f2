"""The seeded input generators: determinism, independence from the thread
count, shapes, dtypes and value distributions."""

import numpy as np
import pytest
import torch

import synth
from synth import workloads as W


def test_same_seed_same_bits():
    a = synth.make_inputs(W.custom(2, 300, 64, "bf16", x_kind="outliers"))
    b = synth.make_inputs(W.custom(2, 300, 64, "bf16", x_kind="outliers"))
    for u, v in ((a.x, b.x), (a.scale, b.scale), (a.shift, b.shift),
                 (a.dy, b.dy)):
        assert torch.equal(u.view(torch.int16), v.view(torch.int16))


def test_seed_and_bucket_change_bits():
    wl = W.custom(1, 64, 128, "f32")
    a = synth.make_inputs(wl, seed=0)
    b = synth.make_inputs(wl, seed=1)
    c = synth.make_inputs(wl, seed=0, bucket=1)
    assert not torch.equal(a.x, b.x) and not torch.equal(a.x, c.x)
    assert not torch.equal(a.dy, a.x)


def test_independent_of_worker_count(monkeypatch):
    monkeypatch.setattr(synth.gen, "BLOCK_ELEMS", 1 << 12)  # many blocks
    wl = W.custom(3, 500, 96, "bf16", x_kind="offset")
    a = synth.make_inputs(wl, workers=1)
    b = synth.make_inputs(wl, workers=7)
    assert torch.equal(a.x.view(torch.int16), b.x.view(torch.int16))
    assert torch.equal(a.dy.view(torch.int16), b.dy.view(torch.int16))


def test_shapes_and_dtypes():
    t = synth.make_inputs(synth.TINY_F32)
    assert t.x.shape == (2, 256, 64) and t.x.dtype == torch.float32
    assert t.scale.shape == (2, 64) and t.shift.shape == (2, 64)
    assert t.dy.shape == (2, 256, 64)
    wl = W.mixed_bucket(84, 1560)
    assert wl.shape == (84, 1560, 3072) and wl.dtype == "bf16"


def test_bf16_rounding_is_nearest_even():
    # the generator rounds through torch; check torch's rule on ties
    vals = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8),
                     1.0 + 2 ** -8 + 2 ** -20], dtype=np.float32)
    got = torch.from_numpy(vals).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(
        got, np.array([1.0, 1.0 + 2 ** -6, -1.0, 1.0 + 2 ** -7], np.float32))


def test_distributions():
    wl = W.custom(4, 2000, 256, "f32", x_kind="normal", mod_std=0.1,
                  dy_std=1e-2)
    t = synth.make_inputs(wl)
    assert abs(t.x.mean().item()) < 0.01
    assert abs(t.x.std().item() - 1) < 0.01
    assert abs(t.dy.std().item() - 1e-2) < 1e-4
    assert abs(t.scale.std().item() - 0.1) < 0.01


def test_offsets_shared_by_rows():
    wl = W.custom(2, 4000, 64, "f32", x_kind="offset")
    t = synth.make_inputs(wl)
    col_means = t.x.mean(dim=(0, 1))
    assert 0.35 < col_means.std().item() < 0.65  # o ~ N(0, 0.5)
    wl2 = W.mixed_bucket(2, 1560)
    a = synth.make_inputs(wl2, bucket=0, with_dy=False)
    b = synth.make_inputs(wl2, bucket=5, with_dy=False)
    # the same offset vector in every bucket of the mixed schedule
    d = (a.x.float().mean(dim=(0, 1)) - b.x.float().mean(dim=(0, 1)))
    assert d.abs().max().item() < 0.2


def test_outlier_fraction():
    wl = W.custom(1, 4000, 512, "f32", x_kind="outliers")
    t = synth.make_inputs(wl)
    frac = (t.x.abs() > 8).float().mean().item()
    # P(|N(0,20)| > 8) = 0.689; P(|N(0,1)| > 8) ~ 1e-15
    assert abs(frac - 1e-3 * 0.689) < 2e-4


def test_mixed_schedule():
    s = synth.mixed_schedule()
    assert len(s) == 64 and set(s) <= set(W.MIXED_LENGTHS)
    assert s == synth.mixed_schedule(0)
    assert s != synth.mixed_schedule(1)
    assert len(set(s)) == 4
