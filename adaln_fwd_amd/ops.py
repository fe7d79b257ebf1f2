"""Python binding of the fused AdaLN C ABI for torch tensors.

Argument marshalling only: shapes, dtypes, devices and contiguity are checked
here because the C ABI cannot see torch metadata; every step of the operator
runs in the HIP kernels of ``libadaln.so``.  Outputs that are not passed in
are allocated with torch on the input's device; work is enqueued on the
current torch stream of that device unless ``stream`` is given (a
torch.cuda.Stream or a raw hipStream_t), in which case the outputs and any
temporary workspace are allocated on that stream, so torch's allocator does
not hand the workspace to another stream while the kernels still use it.
"""

from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import torch

from . import _lib

_DTYPES = {torch.float32: _lib.F32, torch.bfloat16: _lib.BF16}


def _code(t: torch.Tensor) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}; use float32 or "
                        "bfloat16") from None


def _check(t: torch.Tensor, name: str, shape, dtype, device) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor, got {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected "
                         f"{tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _ptr(t: Optional[torch.Tensor]):
    return t.data_ptr() if t is not None and t.numel() > 0 else None


def _stream(device: torch.device, stream) -> int:
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _on(device: torch.device, stream):
    """Context in which the outputs and the workspace of a call are
    allocated: the stream the call's kernels run on.  torch's caching
    allocator hands a freed block only to later allocations on the stream it
    was allocated on, so a workspace dropped when the call returns cannot be
    reused by another stream while the kernels still write to it.  (When
    `stream` is the device's current stream, only the device is set.)"""
    if stream is not None:
        handle = (stream.cuda_stream if isinstance(stream, torch.cuda.Stream)
                  else int(stream))
        if handle != torch.cuda.current_stream(device).cuda_stream:
            if not isinstance(stream, torch.cuda.Stream):
                stream = torch.cuda.ExternalStream(handle, device=device)
            return torch.cuda.stream(stream)
    return torch.cuda.device(device)


def _shape3(x: torch.Tensor) -> Tuple[int, int, int]:
    if x.dim() != 3:
        raise ValueError(f"x must be [B, N, D], got shape {tuple(x.shape)}")
    return tuple(x.shape)


def fwd(x: torch.Tensor, scale: torch.Tensor, shift: torch.Tensor, *,
        y: Optional[torch.Tensor] = None,
        mean: Optional[torch.Tensor] = None,
        rstd: Optional[torch.Tensor] = None, stream=None):
    """y = LayerNorm(x) * (1 + scale[b]) + shift[b]; returns (y, mean, rstd).

    x: [B, N, D]; scale, shift: [B, D] (same dtype); mean, rstd: [B, N] f32."""
    B, N, D = _shape3(x)
    dev, dt = x.device, x.dtype
    code = _code(x)
    _check(x, "x", (B, N, D), dt, dev)
    _check(scale, "scale", (B, D), dt, dev)
    _check(shift, "shift", (B, D), dt, dev)
    lib = _lib.load()
    with _on(dev, stream):
        if y is None:
            y = torch.empty_like(x)
        if mean is None:
            mean = torch.empty(B, N, dtype=torch.float32, device=dev)
        if rstd is None:
            rstd = torch.empty(B, N, dtype=torch.float32, device=dev)
        _check(y, "y", (B, N, D), dt, dev)
        _check(mean, "mean", (B, N), torch.float32, dev)
        _check(rstd, "rstd", (B, N), torch.float32, dev)
        rc = lib.adaln_fwd(_ptr(x), _ptr(scale), _ptr(shift), _ptr(y),
                           _ptr(mean), _ptr(rstd), B, N, D, code,
                           _stream(dev, stream))
    _lib.check(rc, "adaln_fwd")
    return y, mean, rstd


def bwd_workspace_bytes(B: int, N: int, D: int, dtype: torch.dtype) -> int:
    code = _DTYPES.get(dtype, -1)
    return int(_lib.load().adaln_bwd_workspace_bytes(B, N, D, code))


def _bwd_common(dy, x, scale, mean, rstd):
    B, N, D = _shape3(x)
    dev, dt = x.device, x.dtype
    _code(x)
    _check(dy, "dy", (B, N, D), dt, dev)
    _check(x, "x", (B, N, D), dt, dev)
    if scale is not None:
        _check(scale, "scale", (B, D), dt, dev)
    _check(mean, "mean", (B, N), torch.float32, dev)
    _check(rstd, "rstd", (B, N), torch.float32, dev)
    return B, N, D, dev, dt


def _workspace(workspace, B, N, D, dt, dev):
    need = bwd_workspace_bytes(B, N, D, dt)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on "
                         f"{dev}")
    return workspace, workspace.numel() * workspace.element_size()


def bwd(dy: torch.Tensor, x: torch.Tensor, scale: torch.Tensor,
        mean: torch.Tensor, rstd: torch.Tensor, *,
        dx: Optional[torch.Tensor] = None,
        dscale: Optional[torch.Tensor] = None,
        dshift: Optional[torch.Tensor] = None,
        workspace: Optional[torch.Tensor] = None, stream=None):
    """Backward of :func:`fwd`; returns (dx, dscale, dshift).

    dscale and dshift are float32 [B, D]; the workspace (bytes from
    :func:`bwd_workspace_bytes`) is allocated if not given."""
    B, N, D, dev, dt = _bwd_common(dy, x, scale, mean, rstd)
    lib = _lib.load()
    with _on(dev, stream):
        if dx is None:
            dx = torch.empty_like(x)
        if dscale is None:
            dscale = torch.empty(B, D, dtype=torch.float32, device=dev)
        if dshift is None:
            dshift = torch.empty(B, D, dtype=torch.float32, device=dev)
        _check(dx, "dx", (B, N, D), dt, dev)
        _check(dscale, "dscale", (B, D), torch.float32, dev)
        _check(dshift, "dshift", (B, D), torch.float32, dev)
        workspace, wbytes = _workspace(workspace, B, N, D, dt, dev)
        rc = lib.adaln_bwd(_ptr(dy), _ptr(x), _ptr(scale), _ptr(mean),
                           _ptr(rstd), _ptr(dx), _ptr(dscale), _ptr(dshift),
                           _ptr(workspace), wbytes, B, N, D, _code(x),
                           _stream(dev, stream))
    _lib.check(rc, "adaln_bwd")
    return dx, dscale, dshift


def bwd_noalloc(dy: torch.Tensor, x: torch.Tensor, scale: torch.Tensor,
                mean: torch.Tensor, rstd: torch.Tensor, *,
                dx: Optional[torch.Tensor] = None,
                dscale: Optional[torch.Tensor] = None,
                dshift: Optional[torch.Tensor] = None, stream=None):
    """:func:`bwd` through ``adaln_bwd_noalloc``: the library keeps the
    partial sums in its own static device scratch, so the call needs no
    workspace (outputs not passed in are still allocated here).  Calls that
    overlap on one GPU share that scratch and must be ordered."""
    B, N, D, dev, dt = _bwd_common(dy, x, scale, mean, rstd)
    lib = _lib.load()
    with _on(dev, stream):
        if dx is None:
            dx = torch.empty_like(x)
        if dscale is None:
            dscale = torch.empty(B, D, dtype=torch.float32, device=dev)
        if dshift is None:
            dshift = torch.empty(B, D, dtype=torch.float32, device=dev)
        _check(dx, "dx", (B, N, D), dt, dev)
        _check(dscale, "dscale", (B, D), torch.float32, dev)
        _check(dshift, "dshift", (B, D), torch.float32, dev)
        rc = lib.adaln_bwd_noalloc(_ptr(dy), _ptr(x), _ptr(scale),
                                   _ptr(mean), _ptr(rstd), _ptr(dx),
                                   _ptr(dscale), _ptr(dshift), B, N, D,
                                   _code(x), _stream(dev, stream))
    _lib.check(rc, "adaln_bwd_noalloc")
    return dx, dscale, dshift


def bwd_fused(dy, x, scale, mean, rstd, *, dx=None, workspace=None,
              stream=None):
    """First launch of :func:`bwd`: dx plus dscale/dshift partial sums in
    the workspace.  Returns (dx, workspace); pass the workspace to
    :func:`bwd_finish`."""
    B, N, D, dev, dt = _bwd_common(dy, x, scale, mean, rstd)
    lib = _lib.load()
    with _on(dev, stream):
        if dx is None:
            dx = torch.empty_like(x)
        _check(dx, "dx", (B, N, D), dt, dev)
        workspace, wbytes = _workspace(workspace, B, N, D, dt, dev)
        rc = lib.adaln_bwd_fused(_ptr(dy), _ptr(x), _ptr(scale), _ptr(mean),
                                 _ptr(rstd), _ptr(dx), _ptr(workspace),
                                 wbytes, B, N, D, _code(x),
                                 _stream(dev, stream))
    _lib.check(rc, "adaln_bwd_fused")
    return dx, workspace


def bwd_finish(workspace, B: int, N: int, D: int, dtype: torch.dtype, *,
               dscale=None, dshift=None, stream=None):
    """Second launch of :func:`bwd`: dscale, dshift from the partial sums
    that :func:`bwd_fused` left in ``workspace``."""
    dev = workspace.device
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    code = _DTYPES.get(dtype)
    if code is None:
        raise TypeError(f"unsupported dtype {dtype}")
    lib = _lib.load()
    with _on(dev, stream):
        if dscale is None:
            dscale = torch.empty(B, D, dtype=torch.float32, device=dev)
        if dshift is None:
            dshift = torch.empty(B, D, dtype=torch.float32, device=dev)
        _check(dscale, "dscale", (B, D), torch.float32, dev)
        _check(dshift, "dshift", (B, D), torch.float32, dev)
        rc = lib.adaln_bwd_finish(_ptr(workspace),
                                  workspace.numel() * workspace.element_size(),
                                  _ptr(dscale), _ptr(dshift), B, N, D, code,
                                  _stream(dev, stream))
    _lib.check(rc, "adaln_bwd_finish")
    return dscale, dshift


def bwd_dx(dy, x, scale, mean, rstd, *, dx=None, stream=None):
    """Input gradient only (one launch); returns dx."""
    B, N, D, dev, dt = _bwd_common(dy, x, scale, mean, rstd)
    lib = _lib.load()
    with _on(dev, stream):
        if dx is None:
            dx = torch.empty_like(x)
        _check(dx, "dx", (B, N, D), dt, dev)
        rc = lib.adaln_bwd_dx(_ptr(dy), _ptr(x), _ptr(scale), _ptr(mean),
                              _ptr(rstd), _ptr(dx), B, N, D, _code(x),
                              _stream(dev, stream))
    _lib.check(rc, "adaln_bwd_dx")
    return dx


def bwd_dmod(dy, x, mean, rstd, *, dscale=None, dshift=None, workspace=None,
             stream=None):
    """Modulation gradients only (D-tile reduction); returns (dscale, dshift)."""
    B, N, D, dev, dt = _bwd_common(dy, x, None, mean, rstd)
    lib = _lib.load()
    with _on(dev, stream):
        if dscale is None:
            dscale = torch.empty(B, D, dtype=torch.float32, device=dev)
        if dshift is None:
            dshift = torch.empty(B, D, dtype=torch.float32, device=dev)
        _check(dscale, "dscale", (B, D), torch.float32, dev)
        _check(dshift, "dshift", (B, D), torch.float32, dev)
        workspace, wbytes = _workspace(workspace, B, N, D, dt, dev)
        rc = lib.adaln_bwd_dmod(_ptr(dy), _ptr(x), _ptr(mean), _ptr(rstd),
                                _ptr(dscale), _ptr(dshift), _ptr(workspace),
                                wbytes, B, N, D, _code(x),
                                _stream(dev, stream))
    _lib.check(rc, "adaln_bwd_dmod")
    return dscale, dshift


def bwd_fused_plan(B: int, N: int, D: int, dtype: torch.dtype) -> dict:
    """Launch plan of :func:`bwd_fused` for this shape (host-only)."""
    out = (ctypes.c_int64 * 4)()
    rc = _lib.load().adaln_bwd_fused_plan(B, N, D, _DTYPES.get(dtype, -1),
                                          out)
    _lib.check(rc, "adaln_bwd_fused_plan")
    return dict(V=out[0], waves_per_row=out[1], workgroups=out[2],
                partial_rows=out[3])


def plan(which: str, B: int, N: int, D: int, dtype: torch.dtype) -> dict:
    """How :func:`fwd` (``which="fwd"``) or :func:`bwd_fused` (``"bwd"``)
    splits a [B, N, D] batch into work (host-only): vectors per lane,
    wavefronts per row, workgroups, workgroups per sample, samples in
    flight, row walkers per workgroup, and the skew of each sample's walk
    (position n of sample b is row (n + b * skew) mod N).  ``which="finish"``: the launch that
    sums the backward's partial rows: features per column block, wavefronts
    per block, blocks per workgroup, workgroups, threads per workgroup,
    partial rows summed per output.  ``which="dmod"``: the (d_tile, n_tile,
    b) grid of :func:`bwd_dmod` (d_tiles, rows per n_tile, n_tiles,
    workgroups, threads per workgroup)."""
    codes = {"fwd": 0, "bwd": 1, "finish": 2, "dmod": 3}
    if which not in codes:
        raise ValueError(f"which must be 'fwd', 'bwd', 'finish' or 'dmod', "
                         f"got {which!r}")
    out = (ctypes.c_int64 * 7)()
    rc = _lib.load().adaln_plan(codes[which], B, N, D,
                                _DTYPES.get(dtype, -1), out)
    _lib.check(rc, "adaln_plan")
    if which == "finish":
        return dict(F=out[0], wpc=out[1], cpb=out[2], workgroups=out[3],
                    threads=out[4], rows=out[5])
    if which == "dmod":
        return dict(d_tiles=out[0], n_tile=out[1], n_tiles=out[2],
                    workgroups=out[3], threads=out[4])
    return dict(V=out[0], waves_per_row=out[1], workgroups=out[2],
                bps=out[3], groups=out[4], walkers=out[5], skew=out[6])


class SegTable:
    """Host copy of a segment table in the ABI's layout (int64 offsets,
    int32 modulation indices).  The segment functions accept one in place of
    ``seg_offsets`` (with ``seg_mod`` left None) to skip the conversion in a
    loop that reuses a layout."""

    def __init__(self, seg_offsets, seg_mod=None):
        offs = [int(v) for v in seg_offsets]
        if len(offs) < 1:
            raise ValueError("seg_offsets needs at least one entry (0)")
        self.nseg = len(offs) - 1
        self.rows = offs[-1]
        self.offsets = (ctypes.c_int64 * len(offs))(*offs)
        self.mod = None
        if seg_mod is not None:
            mods = [int(v) for v in seg_mod]
            if len(mods) != self.nseg:
                raise ValueError(f"seg_mod has {len(mods)} entries for "
                                 f"{self.nseg} segments")
            self.mod = (ctypes.c_int32 * max(len(mods), 1))(*mods)

    @property
    def offsets_ptr(self):
        return ctypes.cast(self.offsets, ctypes.c_void_p)

    @property
    def mod_ptr(self):
        return None if self.mod is None else ctypes.cast(self.mod,
                                                         ctypes.c_void_p)


def _table(seg_offsets, seg_mod) -> SegTable:
    if isinstance(seg_offsets, SegTable):
        if seg_mod is not None:
            raise ValueError("pass seg_mod inside the SegTable")
        return seg_offsets
    return SegTable(seg_offsets, seg_mod)


def bwd_segments_workspace_bytes(seg_offsets, D: int,
                                 dtype: torch.dtype) -> int:
    tab = _table(seg_offsets, None)
    return int(_lib.load().adaln_bwd_segments_workspace_bytes(
        tab.offsets_ptr, tab.nseg, D, _DTYPES.get(dtype, -1)))


def fwd_segments(x: torch.Tensor, scale: torch.Tensor, shift: torch.Tensor,
                 seg_offsets, seg_mod=None, *, y=None, mean=None, rstd=None,
                 stream=None):
    """Packed variable-length forward: x [T, D] holds the token rows of
    several segments back to back, segment s being rows
    seg_offsets[s] .. seg_offsets[s+1]-1 and modulated by
    scale/shift[seg_mod[s]] (row s if seg_mod is None); scale, shift:
    [nmod, D].  Returns (y, mean, rstd) with mean, rstd float32 [T]."""
    tab = _table(seg_offsets, seg_mod)
    if x.dim() != 2:
        raise ValueError(f"x must be [T, D], got shape {tuple(x.shape)}")
    T, D = x.shape
    if T != tab.rows:
        raise ValueError(f"x has {T} rows, seg_offsets ends at {tab.rows}")
    nmod = scale.shape[0] if scale.dim() == 2 else -1
    dev, dt = x.device, x.dtype
    code = _code(x)
    _check(x, "x", (T, D), dt, dev)
    _check(scale, "scale", (nmod, D), dt, dev)
    _check(shift, "shift", (nmod, D), dt, dev)
    lib = _lib.load()
    with _on(dev, stream):
        if y is None:
            y = torch.empty_like(x)
        if mean is None:
            mean = torch.empty(T, dtype=torch.float32, device=dev)
        if rstd is None:
            rstd = torch.empty(T, dtype=torch.float32, device=dev)
        _check(y, "y", (T, D), dt, dev)
        _check(mean, "mean", (T,), torch.float32, dev)
        _check(rstd, "rstd", (T,), torch.float32, dev)
        rc = lib.adaln_fwd_segments(_ptr(x), _ptr(scale), _ptr(shift),
                                    _ptr(y), _ptr(mean), _ptr(rstd),
                                    tab.offsets_ptr, tab.mod_ptr, tab.nseg,
                                    nmod, D, code, _stream(dev, stream))
    _lib.check(rc, "adaln_fwd_segments")
    return y, mean, rstd


def bwd_segments(dy, x, scale, mean, rstd, seg_offsets, seg_mod=None, *,
                 dx=None, dscale=None, dshift=None, workspace=None,
                 stream=None):
    """Backward of :func:`fwd_segments`; returns (dx, dscale, dshift) with
    dscale, dshift float32 [nmod, D] summed over every segment that uses
    each modulation vector."""
    tab = _table(seg_offsets, seg_mod)
    if x.dim() != 2:
        raise ValueError(f"x must be [T, D], got shape {tuple(x.shape)}")
    T, D = x.shape
    if T != tab.rows:
        raise ValueError(f"x has {T} rows, seg_offsets ends at {tab.rows}")
    nmod = scale.shape[0] if scale.dim() == 2 else -1
    dev, dt = x.device, x.dtype
    code = _code(x)
    _check(dy, "dy", (T, D), dt, dev)
    _check(x, "x", (T, D), dt, dev)
    _check(scale, "scale", (nmod, D), dt, dev)
    _check(mean, "mean", (T,), torch.float32, dev)
    _check(rstd, "rstd", (T,), torch.float32, dev)
    lib = _lib.load()
    need = int(lib.adaln_bwd_segments_workspace_bytes(tab.offsets_ptr,
                                                      tab.nseg, D, code))
    with _on(dev, stream):
        if dx is None:
            dx = torch.empty_like(x)
        if dscale is None:
            dscale = torch.empty(nmod, D, dtype=torch.float32, device=dev)
        if dshift is None:
            dshift = torch.empty(nmod, D, dtype=torch.float32, device=dev)
        _check(dx, "dx", (T, D), dt, dev)
        _check(dscale, "dscale", (nmod, D), torch.float32, dev)
        _check(dshift, "dshift", (nmod, D), torch.float32, dev)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8,
                                    device=dev)
        if workspace.device != dev or not workspace.is_contiguous():
            raise ValueError(f"workspace must be a contiguous tensor on "
                             f"{dev}")
        wbytes = workspace.numel() * workspace.element_size()
        rc = lib.adaln_bwd_segments(_ptr(dy), _ptr(x), _ptr(scale),
                                    _ptr(mean), _ptr(rstd), _ptr(dx),
                                    _ptr(dscale), _ptr(dshift),
                                    _ptr(workspace), wbytes, tab.offsets_ptr,
                                    tab.mod_ptr, tab.nseg, nmod, D, code,
                                    _stream(dev, stream))
    _lib.check(rc, "adaln_bwd_segments")
    return dx, dscale, dshift


def bshape(S: int, m_mem: int, m_comp: int, p: int) -> int:
    """Dual-constraint bucket batch size (host integer arithmetic in the
    library); raises on invalid arguments."""
    v = int(_lib.load().adaln_bshape(int(S), int(m_mem), int(m_comp), int(p)))
    if v < 1:
        _lib.check(v, "adaln_bshape")
    return v


def max_d(dtype: torch.dtype) -> int:
    return int(_lib.load().adaln_max_d(_DTYPES.get(dtype, -1)))
