"""Fused AdaLN (LayerNorm-Modulate) forward and backward for AMD Instinct
MI355X (gfx950), as hand-written HIP kernels behind a C ABI
(include/adaln.h).  PyTorch supplies device memory and streams only."""

from ._lib import AdalnError, BF16, F32, LIB_PATH, load
from .ops import (SegTable, bshape, bwd, bwd_dmod, bwd_dx, bwd_finish,
                  bwd_fused, bwd_fused_plan, bwd_noalloc, bwd_segments,
                  bwd_segments_workspace_bytes, bwd_workspace_bytes, fwd,
                  fwd_segments, max_d, plan)

__all__ = ["AdalnError", "BF16", "F32", "LIB_PATH", "SegTable", "load",
           "bshape", "bwd", "bwd_dmod", "bwd_dx", "bwd_finish", "bwd_fused",
           "bwd_fused_plan", "bwd_noalloc", "bwd_segments", "bwd_segments_workspace_bytes",
           "bwd_workspace_bytes", "fwd", "fwd_segments", "max_d", "plan"]
