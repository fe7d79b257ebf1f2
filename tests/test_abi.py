"""The C ABI without a GPU: the library loads, exports every function the
header declares, validates arguments on the host before any HIP call, and
its host-side bucket rule matches the oracle bit for bit."""

import ctypes
import os
import re
import subprocess

import pytest

import adaln_fwd_amd as A
from adaln_fwd_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "adaln.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(adaln_\w+)\s*\(", src)))


def test_header_declares_the_binding():
    assert _declared() == sorted(_lib.SIGNATURES)


def test_library_exports_every_declared_symbol():
    lib = A.load()
    for name in _declared():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", A.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r" T (adaln_\w+)", out))
    assert exported == set(_declared())


@pytest.fixture(scope="module")
def lib():
    return A.load()


def _no_gpu():
    """The calls below pass fake device addresses that validation must
    reject; they run only where no GPU is visible, so a validation bug can
    never turn one of them into a real launch."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("host-validation tests run only without a GPU")


def test_fwd_validation(lib):
    _no_gpu()
    f = lib.adaln_fwd
    p = 0x1000  # 16-byte aligned, never dereferenced
    assert f(p, p, p, p, p, p, 2, 3, 64, 7, None) == _lib.ERR_DTYPE
    assert f(p, p, p, p, p, p, -1, 3, 64, 1, None) == _lib.ERR_INVALID
    assert f(p, p, p, p, p, p, 2, -3, 64, 1, None) == _lib.ERR_INVALID
    assert f(p, p, p, p, p, p, 2, 3, 0, 1, None) == _lib.ERR_INVALID
    assert f(p, p, p, p, p, p, 2, 3, 60, 1, None) == _lib.ERR_ALIGN   # bf16: %8
    assert f(p, p, p, p, p, p, 2, 3, 62, 0, None) == _lib.ERR_ALIGN   # f32: %4
    assert f(p, p, p, p, p, p, 1, 1, 32776, 1, None) == _lib.ERR_UNSUPPORTED
    assert f(p, p, p, p, p, p, 1, 1, 16388, 0, None) == _lib.ERR_UNSUPPORTED
    assert f(None, p, p, p, p, p, 2, 3, 64, 1, None) == _lib.ERR_INVALID
    assert f(p, p, p, None, p, p, 2, 3, 64, 1, None) == _lib.ERR_INVALID
    assert f(p, p, p, p, p, None, 2, 3, 64, 1, None) == _lib.ERR_INVALID
    assert f(p + 4, p, p, p, p, p, 2, 3, 64, 1, None) == _lib.ERR_ALIGN
    assert f(p, p, p, p, p + 8, p, 2, 3, 64, 1, None) == _lib.ERR_ALIGN
    assert b"aligned" in lib.adaln_last_error()
    assert f(p, p, p, p, p, p, 1 << 21, 1, 64, 1, None) == _lib.ERR_INVALID
    assert f(p, p, p, p, p, p, 1 << 16, 1 << 16, 64, 1, None) == _lib.ERR_INVALID
    assert b"rows" in lib.adaln_last_error()


def test_empty_calls_succeed_without_a_launch(lib):
    _no_gpu()
    # no rows: nothing to do, NULL pointers allowed, no HIP call is made
    assert lib.adaln_fwd(None, None, None, None, None, None, 0, 5, 64, 1,
                         None) == _lib.OK
    assert lib.adaln_fwd(None, None, None, None, None, None, 4, 0, 64, 0,
                         None) == _lib.OK
    assert lib.adaln_bwd_dx(None, None, None, None, None, None, 0, 9, 64, 1,
                            None) == _lib.OK
    assert lib.adaln_last_error() == b""


def test_bwd_validation(lib):
    _no_gpu()
    p = 0x1000
    need = lib.adaln_bwd_workspace_bytes(2, 100, 1536, 1)
    assert need > 0
    f = lib.adaln_bwd
    assert f(p, p, p, p, p, p, p, p, p, need - 1, 2, 100, 1536, 1,
             None) == _lib.ERR_WORKSPACE
    assert f(p, p, p, p, p, p, p, p, None, need, 2, 100, 1536, 1,
             None) == _lib.ERR_WORKSPACE
    assert f(p, p, p, p, p, p, p, p, p + 4, need, 2, 100, 1536, 1,
             None) == _lib.ERR_ALIGN
    assert f(p, p, p, p, p, p, None, p, p, need, 2, 100, 1536, 1,
             None) == _lib.ERR_INVALID
    assert f(p, p, p, p, p, p, p, p, p, need, 2, 100, 1536, 9,
             None) == _lib.ERR_DTYPE
    g = lib.adaln_bwd_dmod
    assert g(p, p, p, p, p, p, None, 0, 2, 100, 1536, 1,
             None) == _lib.ERR_WORKSPACE
    assert g(p, p, p, p, None, p, p, need, 2, 100, 1536, 1,
             None) == _lib.ERR_INVALID
    assert b"workspace" in lib.adaln_last_error() or lib.adaln_last_error()


def test_workspace_bytes(lib):
    ws = lib.adaln_bwd_workspace_bytes
    assert ws(1, 75600, 5120, 1) % 16 == 0
    assert ws(2, 0, 64, 1) == 0          # no rows: no partials
    assert ws(2, 3, 60, 1) == 0          # invalid: 0
    assert ws(2, 3, 64, 5) == 0
    # a pure function of the shape: partial sums for every (b, n_tile, d)
    for B, N, D, dt in [(16, 1560, 1536, 1), (1, 32760, 1536, 1),
                        (1, 75600, 5120, 1), (2, 256, 64, 0)]:
        n = ws(B, N, D, dt)
        assert n == ws(B, N, D, dt)
        assert n % (2 * 4 * B * D) == 0
        n_tiles = n // (2 * 4 * B * D)
        assert 1 <= n_tiles <= N


def _table(offs, mods=None):
    o = (ctypes.c_int64 * len(offs))(*offs)
    m = None if mods is None else (ctypes.c_int32 * len(mods))(*mods)
    return (ctypes.cast(o, ctypes.c_void_p),
            None if m is None else ctypes.cast(m, ctypes.c_void_p), (o, m))


def test_segments_validation(lib):
    _no_gpu()
    p = 0x1000
    f = lib.adaln_fwd_segments
    off, mod, keep = _table([0, 100, 250], [1, 0])
    assert f(p, p, p, p, p, p, off, mod, 2, 2, 1536, 7, None) == _lib.ERR_DTYPE
    assert f(p, p, p, p, p, p, off, mod, 2, 2, 1540, 1, None) == _lib.ERR_ALIGN
    assert f(p + 8, p, p, p, p, p, off, mod, 2, 2, 1536, 1,
             None) == _lib.ERR_ALIGN
    assert f(p, p, p, None, p, p, off, mod, 2, 2, 1536, 1,
             None) == _lib.ERR_INVALID
    # modulation index out of range
    assert f(p, p, p, p, p, p, off, mod, 2, 1, 1536, 1,
             None) == _lib.ERR_INVALID
    assert b"modulation" in lib.adaln_last_error()
    # identity table needs nmod >= nseg
    assert f(p, p, p, p, p, p, off, None, 2, 1, 1536, 1,
             None) == _lib.ERR_INVALID
    # table errors: NULL, first offset, decreasing, too many segments
    assert f(p, p, p, p, p, p, None, None, 2, 2, 1536, 1,
             None) == _lib.ERR_INVALID
    bad, _, k2 = _table([5, 100, 250])
    assert f(p, p, p, p, p, p, bad, None, 2, 2, 1536, 1,
             None) == _lib.ERR_INVALID
    dec, _, k3 = _table([0, 100, 50])
    assert f(p, p, p, p, p, p, dec, None, 2, 2, 1536, 1,
             None) == _lib.ERR_INVALID
    many, _, k4 = _table(list(range(130)))
    assert f(p, p, p, p, p, p, many, None, 129, 129, 1536, 1,
             None) == _lib.ERR_INVALID
    # rows wider than the segment kernels take (the forward takes every
    # width adaln_fwd takes)
    assert f(p, p, p, p, p, p, off, mod, 2, 2, 32776, 1,
             None) == _lib.ERR_UNSUPPORTED
    assert f(p, p, p, p, p, p, off, mod, 2, 2, 16388, 0,
             None) == _lib.ERR_UNSUPPORTED
    g = lib.adaln_bwd_segments
    need = lib.adaln_bwd_segments_workspace_bytes(off, 2, 1536, 1)
    assert need > 0
    assert g(p, p, p, p, p, p, p, p, p, need - 4, off, mod, 2, 2, 1536, 1,
             None) == _lib.ERR_WORKSPACE
    assert g(p, p, p, p, p, p, p, None, p, need, off, mod, 2, 2, 1536, 1,
             None) == _lib.ERR_INVALID
    # past the widest row (4096 vectors)
    assert g(p, p, p, p, p, p, p, p, p, need, off, mod, 2, 2, 32776, 1,
             None) == _lib.ERR_UNSUPPORTED
    # the packed backward takes every width up to it: with eight wavefronts
    # per row from 2561 vectors, so only the workspace is short here
    assert g(p, p, p, p, p, p, p, p, p, need, off, mod, 2, 2, 20488, 1,
             None) == _lib.ERR_WORKSPACE
    # nothing to do: no segments and no modulation vectors
    assert f(None, None, None, None, None, None, None, None, 0, 0, 64, 1,
             None) == _lib.OK
    assert g(None, None, None, None, None, None, None, None, None, 0, None,
             None, 0, 0, 64, 1, None) == _lib.OK
    del keep, k2, k3, k4


def test_segments_workspace_bytes(lib):
    ws = lib.adaln_bwd_segments_workspace_bytes
    for offs, D, dt in [([0, 100, 250], 1536, 1), ([0, 32760, 32760, 33272],
                                                    3072, 1),
                        ([0] + [1560 * (i + 1) for i in range(84)], 3072, 1),
                        ([0, 7], 64, 0)]:
        off, _, keep = _table(offs)
        nseg = len(offs) - 1
        n = ws(off, nseg, D, dt)
        assert n % (2 * 4 * D) == 0
        wgs = n // (2 * 4 * D)
        busy = sum(1 for a, b in zip(offs, offs[1:]) if b > a)
        # at least one workgroup per non-empty segment, at most the
        # workgroups resident at once (256 CUs x at most 4)
        assert busy <= wgs <= 1024
        del keep
    off, _, keep = _table([0, 10])
    assert ws(off, 1, 60, 1) == 0            # invalid: 0
    assert ws(off, 200, 64, 1) == 0
    assert ws(None, 0, 64, 1) == 0           # no segments: no partials


def test_noalloc_refuses_shapes_beyond_its_scratch(lib):
    _no_gpu()
    p = 0x1000
    # 1024 samples of 10240 bf16 features: 80 MiB of partial rows > 64 MiB
    assert lib.adaln_bwd_workspace_bytes(1024, 100, 10240, 1) > 64 << 20
    rc = lib.adaln_bwd_noalloc(p, p, p, p, p, p, p, p, 1024, 100, 10240, 1,
                               None)
    assert rc == _lib.ERR_WORKSPACE
    assert b"scratch" in lib.adaln_last_error()
    # the argument checks of adaln_bwd come first
    assert lib.adaln_bwd_noalloc(p, p, p, p, p, p, p, p, 2, 3, 60, 1,
                                 None) == _lib.ERR_ALIGN
    assert lib.adaln_bwd_noalloc(None, p, p, p, p, p, p, p, 2, 3, 64, 1,
                                 None) == _lib.ERR_INVALID


def test_max_d(lib):
    assert lib.adaln_max_d(1) == 32768
    assert lib.adaln_max_d(0) == 16384
    assert lib.adaln_max_d(3) == 0


def test_strerror(lib):
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert lib.adaln_strerror(code)
    assert lib.adaln_strerror(-99) == b"unknown error code"


def test_bshape_by_hand_and_against_oracle(oracle_mod):
    table = {1560: 84, 8190: 16, 16380: 8, 32760: 2}
    for S, b in table.items():
        assert A.bshape(S, 131072, 2_200_000_000, 2) == b
    import numpy as np
    g = np.random.default_rng(0)
    for _ in range(2000):
        S = int(g.integers(1, 10 ** 6))
        mm = int(g.integers(0, 10 ** 7))
        mc = int(g.integers(0, 10 ** 13))
        p = int(g.integers(0, 5))
        assert A.bshape(S, mm, mc, p) == oracle_mod.bshape(S, mm, mc, p)
    with pytest.raises(A.AdalnError):
        A.bshape(0, 1, 1, 2)
    assert A.load().adaln_bshape(-1, 1, 1, 2) == _lib.ERR_INVALID


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(1, 2, 64, dtype=torch.bfloat16)
    s = torch.zeros(1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        A.fwd(x, s, s)
    with pytest.raises(TypeError):
        A.fwd(x.half(), s.half(), s.half())


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libadaln.so"))
    with pytest.raises(ImportError):
        _lib.load()
