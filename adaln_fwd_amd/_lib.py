"""ctypes loader for ``libadaln.so`` (the C ABI in include/adaln.h).

The library is built in-tree by ``adaln_fwd_amd.build``.  There is no
fallback: if the library is missing or fails to load, import of the operators
raises."""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libadaln.so")

F32 = 0
BF16 = 1

OK = 0
ERR_INVALID = -1
ERR_DTYPE = -2
ERR_ALIGN = -3
ERR_WORKSPACE = -4
ERR_HIP = -5
ERR_UNSUPPORTED = -6

# Every function the header declares, with its ctypes signature.
_VP, _I64, _INT, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
SIGNATURES = {
    "adaln_fwd": (_INT, [_VP, _VP, _VP, _VP, _VP, _VP, _I64, _I64, _I64, _INT,
                         _VP]),
    "adaln_bwd_workspace_bytes": (_SZ, [_I64, _I64, _I64, _INT]),
    "adaln_bwd": (_INT, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ,
                         _I64, _I64, _I64, _INT, _VP]),
    "adaln_bwd_noalloc": (_INT, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                 _I64, _I64, _I64, _INT, _VP]),
    "adaln_bwd_fused": (_INT, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _I64,
                               _I64, _I64, _INT, _VP]),
    "adaln_bwd_finish": (_INT, [_VP, _SZ, _VP, _VP, _I64, _I64, _I64, _INT,
                                _VP]),
    "adaln_bwd_fused_plan": (_INT, [_I64, _I64, _I64, _INT,
                                    ctypes.POINTER(ctypes.c_int64)]),
    "adaln_plan": (_INT, [_INT, _I64, _I64, _I64, _INT,
                          ctypes.POINTER(ctypes.c_int64)]),
    "adaln_bwd_dx": (_INT, [_VP, _VP, _VP, _VP, _VP, _VP, _I64, _I64, _I64,
                            _INT, _VP]),
    "adaln_bwd_dmod": (_INT, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _I64,
                              _I64, _I64, _INT, _VP]),
    "adaln_fwd_segments": (_INT, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                  _I64, _I64, _I64, _INT, _VP]),
    "adaln_bwd_segments_workspace_bytes": (_SZ, [_VP, _I64, _I64, _INT]),
    "adaln_bwd_segments": (_INT, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                  _SZ, _VP, _VP, _I64, _I64, _I64, _INT,
                                  _VP]),
    "adaln_bshape": (_I64, [_I64, _I64, _I64, ctypes.c_int32]),
    "adaln_bshape_real": (_I64, [_I64, _I64, ctypes.c_double,
                                 ctypes.c_double]),
    "adaln_mcomp": (ctypes.c_double, [ctypes.c_double, _I64, _I64]),
    "adaln_costfit": (_INT, [_VP, _VP, _VP, _I64, ctypes.c_double,
                             ctypes.c_double, _VP]),
    "adaln_max_d": (_I64, [_INT]),
    "adaln_strerror": (ctypes.c_char_p, [_INT]),
    "adaln_last_error": (ctypes.c_char_p, []),
}

_lib = None


class AdalnError(RuntimeError):
    """A non-zero return code from the library."""

    def __init__(self, code: int, where: str, message: str):
        self.code = code
        super().__init__(f"{where}: {message} (code {code})")


def load() -> ctypes.CDLL:
    """Load the library once; raise if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run adaln_fwd_amd.build.build() "
            "first")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(code: int, where: str) -> None:
    if code != OK:
        lib = load()
        msg = lib.adaln_last_error().decode() or lib.adaln_strerror(
            code).decode()
        raise AdalnError(code, where, msg)
