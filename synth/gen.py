"""Seeded synthetic inputs for the fused AdaLN operator.

Both sides of every parity check -- the HIP path and the CPU oracle -- take
their inputs from here, and this module holds none of the method's arithmetic:
it only draws random tensors of the workload's shapes and distributions.

Determinism: every tensor is cut into blocks of whole rows, and each block is
drawn by its own PCG64 stream seeded with
``SeedSequence(seed, spawn_key=(workload.index, bucket, tensor_id, block))``.
The bits therefore depend only on (seed, workload, bucket, tensor, shape),
never on how many threads drew them.

Values are drawn in float32 and rounded to the workload's dtype; bfloat16
rounding is round-to-nearest-even (torch's conversion).
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import List, Optional

import numpy as np
import torch

from .workloads import (MIXED_BUCKETS, MIXED_LENGTHS, MIXED_M_MEM,
                        MIXED_SCHEDULE, MMDIT_PACKED, MMDIT_TEXT_TOKENS,
                        PACKED_MIXED, Workload)

TENSOR_X = 0
TENSOR_OFFSET = 1
TENSOR_SCALE = 2
TENSOR_SHIFT = 3
TENSOR_DY = 4
SCHEDULE_KEY = 0xC4
PACK_KEY = 0xC5

# Target number of elements per independently seeded block.
BLOCK_ELEMS = 1 << 22

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def torch_dtype(name: str) -> torch.dtype:
    return _TORCH_DTYPE[name]


def _rng(seed: int, wl: Workload, bucket: int, tensor: int,
         block: int) -> np.random.Generator:
    ss = np.random.SeedSequence(seed, spawn_key=(wl.index, bucket, tensor,
                                                 block))
    return np.random.Generator(np.random.PCG64(ss))


def _workers(workers: Optional[int]) -> int:
    if workers is not None:
        return max(1, workers)
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _draw_rows(out: torch.Tensor, rows: int, D: int, fill, workers):
    """Fill ``out`` (a [rows, D] tensor of any dtype) block by block.

    ``fill(block_index, nrows) -> np.ndarray[float32] of shape [nrows, D]``.
    """
    block_rows = max(1, BLOCK_ELEMS // max(D, 1))
    nblocks = (rows + block_rows - 1) // block_rows
    out2 = out.view(rows, D)

    def one(i):
        r0 = i * block_rows
        r1 = min(rows, r0 + block_rows)
        vals = fill(i, r1 - r0)
        out2[r0:r1].copy_(torch.from_numpy(vals))

    if nblocks <= 1 or _workers(workers) == 1:
        for i in range(nblocks):
            one(i)
    else:
        with ThreadPoolExecutor(_workers(workers)) as ex:
            list(ex.map(one, range(nblocks)))


def _offsets(wl: Workload, seed: int) -> np.ndarray:
    """The per-channel offset vector o[D] of an ``"offset"`` workload.

    Drawn once per workload (all buckets of the mixed schedule share it)."""
    g = _rng(seed, wl, 0, TENSOR_OFFSET, 0)
    return (wl.offset_std * g.standard_normal(wl.D, dtype=np.float32)).astype(
        np.float32)


def _x_block(wl: Workload, seed: int, bucket: int, offsets):
    D = wl.D

    def fill(i, nrows):
        g = _rng(seed, wl, bucket, TENSOR_X, i)
        z = g.standard_normal((nrows, D), dtype=np.float32)
        if wl.x_kind == "offset":
            z += offsets[None, :]
        elif wl.x_kind == "outliers":
            u = g.random((nrows, D), dtype=np.float32)
            mask = u < wl.outlier_p
            cnt = int(mask.sum())
            if cnt:
                z[mask] = wl.outlier_std * g.standard_normal(
                    cnt, dtype=np.float32)
        elif wl.x_kind != "normal":
            raise ValueError(f"unknown x_kind {wl.x_kind!r}")
        return z

    return fill


def _normal_block(wl: Workload, seed: int, bucket: int, tensor: int,
                  std: float):
    D = wl.D

    def fill(i, nrows):
        g = _rng(seed, wl, bucket, tensor, i)
        z = g.standard_normal((nrows, D), dtype=np.float32)
        z *= np.float32(std)
        return z

    return fill


@dataclass
class Inputs:
    """Host (CPU) tensors of one AdaLN call, in the workload's dtype.

    x, dy: [B, N, D]; scale, shift: [B, D]."""
    x: torch.Tensor
    scale: torch.Tensor
    shift: torch.Tensor
    dy: Optional[torch.Tensor]
    workload: Workload
    seed: int
    bucket: int


def make_inputs(wl: Workload, seed: int = 0, bucket: int = 0,
                with_dy: bool = True, workers: Optional[int] = None,
                pin_memory: bool = False) -> Inputs:
    """Draw the inputs of workload ``wl`` (which must have B and N set)."""
    B, N, D = wl.shape
    dt = torch_dtype(wl.dtype)
    rows = B * N
    offsets = _offsets(wl, seed) if wl.x_kind == "offset" else None

    def empty(*shape):
        return torch.empty(*shape, dtype=dt, pin_memory=pin_memory)

    x = empty(B, N, D)
    _draw_rows(x, rows, D, _x_block(wl, seed, bucket, offsets), workers)
    scale = empty(B, D)
    _draw_rows(scale, B, D,
               _normal_block(wl, seed, bucket, TENSOR_SCALE, wl.mod_std), 1)
    shift = empty(B, D)
    _draw_rows(shift, B, D,
               _normal_block(wl, seed, bucket, TENSOR_SHIFT, wl.mod_std), 1)
    dy = None
    if with_dy:
        dy = empty(B, N, D)
        _draw_rows(dy, rows, D,
                   _normal_block(wl, seed, bucket, TENSOR_DY, wl.dy_std),
                   workers)
    return Inputs(x=x, scale=scale, shift=shift, dy=dy, workload=wl,
                  seed=seed, bucket=bucket)


def mixed_schedule(seed: int = 0, count: int = MIXED_BUCKETS) -> List[int]:
    """Sequence lengths S of the mixed-length schedule: ``count`` draws,
    uniform over {1560, 8190, 16380, 32760}."""
    ss = np.random.SeedSequence(seed, spawn_key=(MIXED_SCHEDULE.index,
                                                 SCHEDULE_KEY))
    g = np.random.Generator(np.random.PCG64(ss))
    idx = g.integers(0, len(MIXED_LENGTHS), size=count)
    return [int(MIXED_LENGTHS[i]) for i in idx]


@dataclass
class PackedInputs:
    """Host tensors of one packed call: x, dy [T, D]; scale, shift
    [nmod, D]; segment s is rows seg_offsets[s] .. seg_offsets[s+1]-1 and
    uses modulation vector seg_mod[s] (vector s if seg_mod is None)."""
    x: torch.Tensor
    scale: torch.Tensor
    shift: torch.Tensor
    dy: Optional[torch.Tensor]
    seg_offsets: np.ndarray
    seg_mod: Optional[np.ndarray]
    workload: Workload
    seed: int

    @property
    def lengths(self) -> np.ndarray:
        return np.diff(self.seg_offsets)


def pack_lengths(seed: int = 0, budget: int = MIXED_M_MEM,
                 max_segments: int = 128, max_misses: int = 16) -> List[int]:
    """Sequence lengths of one pack of the packed mixed-length layout:
    lengths drawn uniformly from the mixed schedule's four, a draw that
    would overflow the token budget skipped, until ``max_misses`` draws in a
    row were skipped or the pack holds ``max_segments`` sequences."""
    ss = np.random.SeedSequence(seed, spawn_key=(PACKED_MIXED.index,
                                                 PACK_KEY))
    g = np.random.Generator(np.random.PCG64(ss))
    out: List[int] = []
    total, misses = 0, 0
    while misses < max_misses and len(out) < max_segments:
        S = int(MIXED_LENGTHS[int(g.integers(0, len(MIXED_LENGTHS)))])
        if total + S > budget:
            misses += 1
            continue
        misses = 0
        out.append(S)
        total += S
    return out


def mmdit_layout(B: int, text: int = MMDIT_TEXT_TOKENS,
                 video: int = MMDIT_PACKED.N - MMDIT_TEXT_TOKENS):
    """Segment lengths and modulation indices of B two-stream samples packed
    as [text_0, video_0, text_1, video_1, ...], with the modulation vectors
    laid out [2, B, D]: text of sample b uses vector b, its video B + b."""
    lengths, mods = [], []
    for b in range(B):
        lengths += [text, video]
        mods += [b, B + b]
    return lengths, mods


def make_packed(wl: Workload, lengths, seg_mod=None, nmod: Optional[int] = None,
                seed: int = 0, with_dy: bool = True,
                workers: Optional[int] = None,
                pin_memory: bool = False) -> PackedInputs:
    """Draw the inputs of a packed layout with workload ``wl``'s dtype and
    distributions: x, dy over the T = sum(lengths) rows, scale and shift for
    ``nmod`` vectors (default: one per segment, or max(seg_mod) + 1)."""
    lengths = [int(v) for v in lengths]
    off = np.concatenate([[0], np.cumsum(lengths, dtype=np.int64)]).astype(
        np.int64)
    mods = None if seg_mod is None else np.asarray(seg_mod, dtype=np.int32)
    if nmod is None:
        nmod = len(lengths) if mods is None else (
            int(mods.max()) + 1 if mods.size else 0)
    T, D = int(off[-1]), wl.D
    dt = torch_dtype(wl.dtype)
    offsets = _offsets(wl, seed) if wl.x_kind == "offset" else None

    def empty(*shape):
        return torch.empty(*shape, dtype=dt, pin_memory=pin_memory)

    x = empty(T, D)
    _draw_rows(x, T, D, _x_block(wl, seed, 0, offsets), workers)
    scale = empty(nmod, D)
    _draw_rows(scale, nmod, D,
               _normal_block(wl, seed, 0, TENSOR_SCALE, wl.mod_std), 1)
    shift = empty(nmod, D)
    _draw_rows(shift, nmod, D,
               _normal_block(wl, seed, 0, TENSOR_SHIFT, wl.mod_std), 1)
    dy = None
    if with_dy:
        dy = empty(T, D)
        _draw_rows(dy, T, D,
                   _normal_block(wl, seed, 0, TENSOR_DY, wl.dy_std), workers)
    return PackedInputs(x=x, scale=scale, shift=shift, dy=dy, seg_offsets=off,
                        seg_mod=mods, workload=wl, seed=seed)
