"""GPU parity of the HIP path against the oracle, through the C ABI.

Every output element of every case is compared: small and medium shapes in
Python, the two largest workloads (the large model and the wide rows) row by
row through the oracle library's row checker (y, dx, mean, rstd), with
dscale/dshift in full.  Every case prints its name before touching the GPU.
"""

import ctypes

import numpy as np
import pytest
import torch

import synth
from synth import workloads as W
from tests import parity as P

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[parity] {msg}", flush=True)


@pytest.fixture(scope="module")
def A():
    import adaln_fwd_amd
    adaln_fwd_amd.load()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return adaln_fwd_amd


def _run_full(A, wl, seed=0, bucket=0, label=None):
    _say(f"{label or wl.name} B={wl.B} N={wl.N} D={wl.D} {wl.dtype} seed={seed}")
    inp = synth.make_inputs(wl, seed=seed, bucket=bucket)
    dev = P.to_device(inp)
    out = P.gpu_fwd_bwd(dev)
    torch.cuda.synchronize()
    out = {k: v.cpu() for k, v in out.items()}
    reps = P.compare_full(inp, out, wl.dtype)
    for r in reps:
        _say(f"  {r}")
    return inp, out


def test_tiny_f32(A):
    _run_full(A, synth.TINY_F32)


def test_image_bucket_full(A):
    _run_full(A, synth.IMAGE_BUCKET)


def test_video_bucket_full(A):
    _run_full(A, synth.VIDEO_BUCKET)


@pytest.mark.parametrize("B,N,D,dtype,kind", [
    (1, 1, 1536, "bf16", "offset"),        # a single token
    (3, 1, 64, "f32", "normal"),           # one token per sample
    (2, 1000, 1536, "bf16", "offset"),     # ragged n_tiles
    (5, 77, 3072, "bf16", "offset"),       # several samples, ragged
    (2, 300, 5120, "bf16", "outliers"),
    (1, 40, 8, "bf16", "normal"),          # smallest bf16 row
    (2, 33, 4, "f32", "normal"),           # smallest f32 row
    (2, 130, 520, "bf16", "normal"),       # partial last vector column
    (2, 64, 4104, "bf16", "normal"),       # V rounded up (513 vectors)
    (1, 50, 6144, "bf16", "normal"),
    (1, 30, 8192, "bf16", "normal"),
    (1, 20, 12288, "bf16", "normal"),      # two wavefronts per row
    (1, 9, 32768, "bf16", "normal"),       # fwd quads, bwd eights (max D)
    (2, 17, 8192, "f32", "normal"),        # two wavefronts per row, f32
    (1, 5, 16384, "f32", "normal"),        # largest f32 row
    (3, 257, 1024, "f32", "offset"),
    (2, 333, 2560, "f32", "offset"),       # widest one-wavefront f32 bwd
    (1, 100, 4096, "f32", "normal"),       # f32 stream forward, paired bwd
    (600, 5, 1536, "bf16", "offset"),      # more samples than workgroups
    (1100, 1, 5120, "bf16", "outliers"),   # several samples per workgroup
    (2000, 3, 64, "f32", "normal"),
    (300, 17, 520, "bf16", "normal"),      # many samples, ragged row
    (6, 8192, 3072, "bf16", "offset"),     # long samples: 2 in flight (fwd)
    (8, 6000, 2048, "f32", "normal"),      # long samples: 4 in flight (fwd)
    # backward rows split between two wavefronts (321..1280 vectors; two
    # wavefronts per SIMD up to 640)
    (3, 123, 2568, "bf16", "offset"),      # narrowest, ragged half
    (2, 150, 4000, "bf16", "normal"),      # 4 vectors per lane, ragged
    (4, 100, 1288, "f32", "normal"),       # f32, ragged
    (700, 2, 3072, "bf16", "offset"),      # more samples than workgroups
    (3, 333, 5128, "bf16", "outliers"),    # one wavefront per SIMD, ragged
    (2, 1001, 10240, "bf16", "offset"),    # widest
    (1, 777, 7000, "bf16", "normal"),      # ragged half
    (5, 64, 4096, "f32", "normal"),
    (600, 3, 6144, "bf16", "offset"),      # odd rows per workgroup
    # backward rows split between four wavefronts (1281..2560 vectors), one
    # row per workgroup
    (2, 77, 10248, "bf16", "offset"),      # narrowest, ragged quarter
    (1, 300, 16384, "bf16", "normal"),     # 8 vectors per lane, exact
    (3, 50, 20480, "bf16", "outliers"),    # widest fused backward
    (2, 99, 5124, "f32", "normal"),        # f32, ragged
    (1, 64, 10240, "f32", "offset"),       # widest fused f32 backward
    (5, 333, 6144, "f32", "normal"),       # 6 vectors per lane, exact
    (700, 2, 12288, "bf16", "offset"),     # more samples than workgroups
    # backward rows split between eight wavefronts (2561..4096 vectors), one
    # row per 512-thread workgroup; bf16 rows of 8 vectors per lane read the
    # scale at each use and derive their indices in each row
    (2, 77, 20488, "bf16", "offset"),      # narrowest, ragged eighth
    (1, 200, 24576, "bf16", "normal"),     # 6 vectors per lane, exact
    (3, 50, 28000, "bf16", "outliers"),    # 8 vectors per lane, ragged
    (1, 120, 32768, "bf16", "offset"),     # widest row
    (600, 2, 24584, "bf16", "offset"),     # more samples than workgroups
    (2, 99, 10244, "f32", "normal"),       # f32, ragged
    (5, 300, 12292, "f32", "normal"),      # f32, 8 vectors per lane, ragged
    (3, 150, 14000, "f32", "offset"),      # f32 forward: late scale loads
    (1, 64, 16384, "f32", "offset"),       # widest f32 row
])
def test_shapes(A, B, N, D, dtype, kind):
    wl = W.custom(B, N, D, dtype, x_kind=kind, dy_std=1e-2 if dtype ==
                  "bf16" else 1.0)
    _run_full(A, wl, seed=B + N + D)


@pytest.mark.parametrize("B,N,D,dtype", [
    (3, 1_500_001, 8, "bf16"),   # 4,500,003 rows: two launches
    (1, 4_194_305, 16, "f32"),   # one row past the first launch
])
def test_forward_launches_past_2_22_rows(A, B, N, D, dtype):
    """The forward of one-wavefront rows takes one launch per 2^22 rows:
    every row of batches that need a second launch (the rows on either side
    of the launch boundary among them), with the backward, and dscale and
    dshift in full.  The f32 case has rows of 16 features: among 4.19 M
    rows of 4 N(0, 1) features some have a variance near 1e-3 of their mean
    square (rstd up to ~140), where float32 arithmetic in any order exceeds
    the float32 tolerance against the float64 oracle (a float32 emulation of
    the kernels' order, which the GPU matches bit for bit there, 5.5x)."""
    assert B * N > 1 << 22
    wl = W.custom(B, N, D, dtype, x_kind="normal",
                  dy_std=1e-2 if dtype == "bf16" else 1.0)
    _say(f"{B}x{N}x{D} {dtype}: {B * N} rows, every row")
    _run_all_rows(A, wl)


def _run_all_rows(A, wl):
    inp = synth.make_inputs(wl)
    dev = P.to_device(inp)
    out = P.gpu_fwd_bwd(dev)
    torch.cuda.synchronize()
    out = {k: v.cpu() for k, v in out.items()}
    del dev
    for r in P.compare_all_rows(inp, out, wl.dtype):
        _say(f"  {r}")
    for r in P.compare_full(inp, out, wl.dtype, with_rows=False):
        _say(f"  {r}")


def test_large_model_all_rows(A):
    """D=5120, N=75600 at full size: every row, and dscale/dshift."""
    wl = synth.LARGE_MODEL
    _say(f"{wl.name} {wl.shape}, every row")
    _run_all_rows(A, wl)


def test_wide_rows_all_rows(A):
    """D=8192 (rows split between two wavefronts in the backward) at the
    large model's activation size: every row, and dscale/dshift."""
    wl = synth.WIDE_ROWS
    _say(f"{wl.name} {wl.shape}, every row")
    assert A.bwd_fused_plan(*wl.shape, torch.bfloat16)["waves_per_row"] == 2
    _run_all_rows(A, wl)


def test_quad_rows_all_rows(A):
    """D=16384 bf16 (2048 vectors, four wavefronts per backward row) at
    half the large model's activation size: every row, and dscale/dshift."""
    wl = W.custom(1, 12288, 16384, "bf16", x_kind="outliers", dy_std=1e-2,
                  index=211)
    _say(f"quad rows {wl.shape}, every row")
    assert A.bwd_fused_plan(*wl.shape, torch.bfloat16)["waves_per_row"] == 4
    _run_all_rows(A, wl)


@pytest.mark.parametrize("B,N,D,dtype", [
    (1, 6000, 32768, "bf16"),    # the widest row, 8 vectors per lane
    (3, 2500, 27992, "bf16"),    # ragged, several samples
    (1, 9000, 16384, "f32"),     # the widest f32 row
])
def test_eight_wave_rows_all_rows(A, B, N, D, dtype):
    """Rows of 2561 to 4096 vectors (eight wavefronts per backward row) at
    about a quarter of the large model's activation size: every row, and
    dscale/dshift."""
    wl = W.custom(B, N, D, dtype, x_kind="outliers",
                  dy_std=1e-2 if dtype == "bf16" else 1.0, index=223)
    _say(f"eight-wave rows {wl.shape} {dtype}, every row")
    assert A.bwd_fused_plan(*wl.shape, synth.torch_dtype(dtype))[
        "waves_per_row"] == 8
    _run_all_rows(A, wl)


def test_constant_and_extreme_rows(A):
    B, N, D = 2, 6, 1024
    x = torch.randn(B, N, D, generator=torch.Generator().manual_seed(3))
    x[0, 0] = 2.5                 # constant row: var = 0, rstd = 1/sqrt(eps)
    x[0, 1] = 0.0                 # all-zero row
    x[1, 2] *= 1e4                # huge row
    x[1, 3] *= 1e-4               # tiny row (var below eps)
    x = x.to(torch.bfloat16)
    g = torch.Generator().manual_seed(4)
    inp = synth.Inputs(x=x, scale=(0.1 * torch.randn(B, D, generator=g)).to(
        torch.bfloat16), shift=(0.1 * torch.randn(B, D, generator=g)).to(
        torch.bfloat16), dy=(0.01 * torch.randn(B, N, D, generator=g)).to(
        torch.bfloat16), workload=None, seed=0, bucket=0)
    _say("constant/zero/huge/tiny rows")
    out = P.gpu_fwd_bwd(P.to_device(inp))
    torch.cuda.synchronize()
    out = {k: v.cpu() for k, v in out.items()}
    for r in P.compare_full(inp, out, "bf16"):
        _say(f"  {r}")


def test_deterministic(A):
    wl = W.custom(2, 3000, 1536, "bf16", x_kind="offset", dy_std=1e-2)
    _say("bitwise determinism")
    dev = P.to_device(synth.make_inputs(wl))
    a = P.gpu_fwd_bwd(dev)
    b = P.gpu_fwd_bwd(dev)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k], b[k]), k


def test_side_stream(A):
    wl = W.custom(3, 500, 3072, "bf16", x_kind="offset", dy_std=1e-2)
    _say("non-default stream")
    inp = synth.make_inputs(wl)
    dev = P.to_device(inp)
    ref = P.gpu_fwd_bwd(dev)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        got = P.gpu_fwd_bwd(dev, stream=s)
    s.synchronize()
    for k in ref:
        assert torch.equal(ref[k], got[k]), k


@pytest.mark.parametrize("handle", [False, True])
def test_stream_argument_without_context(A, handle):
    """stream= names a side stream while the current stream stays the
    default one.  The backward's temporary workspace must not go back to
    the default stream's pool while the side stream's kernels still write
    partial sums into it: a buffer of the workspace's size is allocated and
    filled on the default stream right after the call."""
    wl = W.custom(1, 20000, 5120, "bf16", x_kind="outliers", dy_std=1e-2)
    _say(f"stream= without entering it (raw handle: {handle})")
    inp = synth.make_inputs(wl)
    dev = P.to_device(inp)
    y, mean, rstd = A.fwd(dev["x"], dev["scale"], dev["shift"])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    need = A.bwd_workspace_bytes(*wl.shape, torch.bfloat16)
    dx, dscale, dshift = A.bwd(dev["dy"], dev["x"], dev["scale"], mean, rstd,
                               stream=s.cuda_stream if handle else s)
    junk = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    junk.fill_(0x7F)
    torch.cuda.synchronize()
    out = dict(dscale=dscale.cpu(), dshift=dshift.cpu())
    for r in P.compare_full(inp, out, "bf16", with_rows=False):
        _say(f"  {r}")


def test_guard_bytes_untouched(A):
    """Outputs written through views into larger buffers leave the bytes
    before and after them untouched."""
    B, N, D = 3, 123, 1536
    wl = W.custom(B, N, D, "bf16", x_kind="offset", dy_std=1e-2)
    _say("guard bytes around outputs")
    inp = synth.make_inputs(wl)
    dev = P.to_device(inp)
    pad = 4096  # elements, keeps 16-byte alignment

    def guarded(n, dtype):
        buf = torch.full((n + 2 * pad,), -7.0, dtype=dtype, device="cuda")
        return buf, buf[pad:pad + n]

    yb, y = guarded(B * N * D, torch.bfloat16)
    mb, mean = guarded(B * N, torch.float32)
    rb, rstd = guarded(B * N, torch.float32)
    xb, dx = guarded(B * N * D, torch.bfloat16)
    sb, dscale = guarded(B * D, torch.float32)
    hb, dshift = guarded(B * D, torch.float32)
    need = A.bwd_workspace_bytes(B, N, D, torch.bfloat16)
    wb, ws = guarded(need // 4, torch.float32)
    A.fwd(dev["x"], dev["scale"], dev["shift"], y=y.view(B, N, D),
          mean=mean.view(B, N), rstd=rstd.view(B, N))
    A.bwd(dev["dy"], dev["x"], dev["scale"], mean.view(B, N), rstd.view(B, N),
          dx=dx.view(B, N, D), dscale=dscale.view(B, D),
          dshift=dshift.view(B, D), workspace=ws)
    torch.cuda.synchronize()
    for buf in (yb, mb, rb, xb, sb, hb, wb):
        assert torch.all(buf[:pad] == -7.0) and torch.all(buf[-pad:] == -7.0)
    out = dict(y=y.view(B, N, D).cpu(), mean=mean.view(B, N).cpu(),
               rstd=rstd.view(B, N).cpu(), dx=dx.view(B, N, D).cpu(),
               dscale=dscale.view(B, D).cpu(), dshift=dshift.view(B, D).cpu())
    P.compare_full(inp, out, "bf16")


def test_split_entry_points_match_bwd(A):
    """adaln_bwd is exactly adaln_bwd_fused followed by adaln_bwd_finish."""
    wl = W.custom(2, 700, 3072, "bf16", x_kind="offset", dy_std=1e-2)
    _say("bwd == bwd_fused + bwd_finish")
    dev = P.to_device(synth.make_inputs(wl))
    out = P.gpu_fwd_bwd(dev)
    dx, ws = A.bwd_fused(dev["dy"], dev["x"], dev["scale"], out["mean"],
                         out["rstd"])
    ds, dh = A.bwd_finish(ws, 2, 700, 3072, torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(dx, out["dx"])
    assert torch.equal(ds, out["dscale"]) and torch.equal(dh, out["dshift"])


@pytest.mark.parametrize("wl", [synth.TINY_F32, synth.IMAGE_BUCKET,
                                synth.VIDEO_BUCKET,
                                W.custom(3, 77, 5120, "bf16", x_kind="outliers",
                                         dy_std=1e-2),
                                W.custom(2, 50, 520, "bf16"),
                                W.custom(2, 9, 20488, "bf16", dy_std=1e-2),
                                W.custom(1, 9, 32768, "bf16", dy_std=1e-2),
                                W.custom(2, 7, 16384, "f32")],
                         ids=lambda w: w.name + f"_{w.D}")
def test_unfused_entry_points(A, wl):
    """adaln_bwd_dx and adaln_bwd_dmod (the separate dx kernel and the
    D-tile reduction grid) against the oracle."""
    _say(f"unfused bwd_dx + bwd_dmod on {wl.name} {wl.shape}")
    inp = synth.make_inputs(wl)
    dev = P.to_device(inp)
    y, mean, rstd = A.fwd(dev["x"], dev["scale"], dev["shift"])
    dx = A.bwd_dx(dev["dy"], dev["x"], dev["scale"], mean, rstd)
    ds, dh = A.bwd_dmod(dev["dy"], dev["x"], mean, rstd)
    torch.cuda.synchronize()
    out = dict(y=y.cpu(), mean=mean.cpu(), rstd=rstd.cpu(), dx=dx.cpu(),
               dscale=ds.cpu(), dshift=dh.cpu())
    for r in P.compare_full(inp, out, wl.dtype):
        _say(f"  {r}")


def test_empty(A):
    _say("empty inputs")
    d = "cuda"
    x = torch.empty(0, 5, 64, dtype=torch.bfloat16, device=d)
    y, m, r = A.fwd(x, torch.empty(0, 64, dtype=torch.bfloat16, device=d),
                    torch.empty(0, 64, dtype=torch.bfloat16, device=d))
    assert y.shape == (0, 5, 64)
    # N = 0: dscale/dshift are defined (empty sums) and zero
    x = torch.empty(3, 0, 64, dtype=torch.bfloat16, device=d)
    s = torch.zeros(3, 64, dtype=torch.bfloat16, device=d)
    y, m, r = A.fwd(x, s, s)
    ds = torch.full((3, 64), 5.0, device=d)
    dh = torch.full((3, 64), 5.0, device=d)
    A.bwd(x, x, s, m, r, dscale=ds, dshift=dh)
    torch.cuda.synchronize()
    assert torch.all(ds == 0) and torch.all(dh == 0)


def test_abi_errors_on_device_buffers(A):
    _say("error codes with device buffers")
    lib = A.load()
    # every buffer is large enough for the call it is passed to, so even a
    # missed check could not write out of bounds
    B, N, D = 2, 4, 1536
    x = torch.zeros(B * N * D + 64, dtype=torch.bfloat16, device="cuda")
    y = torch.zeros(B * N * D, dtype=torch.bfloat16, device="cuda")
    s = torch.zeros(B, D, dtype=torch.bfloat16, device="cuda")
    st = torch.zeros(B, N, dtype=torch.float32, device="cuda")
    dm = torch.zeros(B, D, dtype=torch.float32, device="cuda")
    p = x.data_ptr()
    # misaligned x
    rc = lib.adaln_fwd(p + 2, s.data_ptr(), s.data_ptr(), y.data_ptr(),
                       st.data_ptr(), st.data_ptr(), B, N, D, 1, None)
    assert rc == -3
    # workspace too small
    need = lib.adaln_bwd_workspace_bytes(B, N, D, 1)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    rc = lib.adaln_bwd(p, p, s.data_ptr(), st.data_ptr(), st.data_ptr(),
                       y.data_ptr(), dm.data_ptr(), dm.data_ptr(),
                       ws.data_ptr(), need - 1, B, N, D, 1, None)
    assert rc == -4
    torch.cuda.synchronize()


def test_threads_and_streams(A):
    """Two host threads, each on its own stream with its own buffers and
    workspace, run forward + backward concurrently; every result equals the
    serial one bit for bit, and an invalid call in one thread leaves the
    other thread's error message untouched."""
    import threading
    from adaln_fwd_amd import _lib
    _say("two threads, two streams")
    wls = [W.custom(4, 900, 3072, "bf16", x_kind="offset", dy_std=1e-2),
           W.custom(1, 5000, 5120, "bf16", x_kind="outliers", dy_std=1e-2)]
    devs = [P.to_device(synth.make_inputs(w, seed=i)) for i, w in
            enumerate(wls)]
    serial = [P.gpu_fwd_bwd(d) for d in devs]
    torch.cuda.synchronize()
    results = [None, None]
    errors = []
    lib = A.load()

    def work(i):
        try:
            s = torch.cuda.Stream()
            outs = []
            with torch.cuda.stream(s):
                for _ in range(5):
                    outs.append(P.gpu_fwd_bwd(devs[i], stream=s))
                    if i == 0:
                        # a failing call: only this thread sees its message
                        rc = lib.adaln_fwd(None, None, None, None, None, None,
                                           1, 1, 64, 9, None)
                        assert rc == _lib.ERR_DTYPE
                        assert b"dtype" in lib.adaln_last_error()
                    else:
                        assert lib.adaln_last_error() == b""
            s.synchronize()
            results[i] = outs
        except BaseException as e:  # reported by the main thread
            errors.append(e)

    ts = [threading.Thread(target=work, args=(i,)) for i in range(2)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert not errors, errors
    for i in range(2):
        for out in results[i]:
            for k in serial[i]:
                assert torch.equal(out[k], serial[i][k]), (i, k)


def _random_shapes(seed, count):
    g = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        dtype = "bf16" if g.random() < 0.7 else "f32"
        E = 8 if dtype == "bf16" else 4
        # widths across every kernel family: one wavefront, a pair in the
        # backward, several wavefronts in the forward
        nvec = int(g.choice([g.integers(1, 65), g.integers(65, 641),
                             g.integers(641, 1281), g.integers(1281, 2049)],
                            p=[0.3, 0.4, 0.2, 0.1]))
        B = int(g.integers(1, 9))
        N = int(g.integers(1, max(2, 60000 // (B * nvec))))
        out.append((B, N, nvec * E, dtype))
    return out


@pytest.mark.parametrize("B,N,D,dtype", _random_shapes(2024, 24))
def test_random_shapes(A, B, N, D, dtype):
    """Seeded random shapes over every kernel family, compared in full."""
    wl = W.custom(B, N, D, dtype, x_kind="offset",
                  dy_std=1e-2 if dtype == "bf16" else 1.0)
    _run_full(A, wl, seed=B * 7 + N * 3 + D)


def test_non_finite_rows_stay_local(A):
    """A row holding NaN or Inf gives non-finite outputs in that row (and in
    its sample's dscale/dshift) only; every other row and sample is
    unchanged, bit for bit."""
    B, N, D = 3, 40, 1536
    wl = W.custom(B, N, D, "bf16", x_kind="offset", dy_std=1e-2)
    _say("non-finite rows")
    inp = synth.make_inputs(wl)
    dev = P.to_device(inp)
    clean = P.gpu_fwd_bwd(dev)
    bad = dict(dev)
    bad["x"] = dev["x"].clone()
    bad["x"][1, 7, 100] = float("nan")
    bad["x"][1, 9, 5] = float("inf")
    out = P.gpu_fwd_bwd(bad)
    torch.cuda.synchronize()
    for n in (7, 9):
        assert not torch.isfinite(out["y"][1, n].float()).all()
    keep = torch.ones(B, N, dtype=torch.bool, device="cuda")
    keep[1, 7] = keep[1, 9] = False
    assert torch.equal(out["y"][keep], clean["y"][keep])
    assert torch.equal(out["dx"][keep], clean["dx"][keep])
    assert torch.equal(out["mean"][keep], clean["mean"][keep])
    for b in (0, 2):
        assert torch.equal(out["dscale"][b], clean["dscale"][b])
        assert torch.equal(out["dshift"][b], clean["dshift"][b])
