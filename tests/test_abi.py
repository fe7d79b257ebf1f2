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
