"""Seeded synthetic workloads and inputs for the fused AdaLN operator.

Shared by the HIP path's callers and the oracle's tests; holds no part of the
method's arithmetic."""

from .workloads import (ALL, BY_NAME, EPS, IMAGE_BUCKET, LARGE_MODEL,
                        MIXED_BUCKETS, MIXED_LENGTHS, MIXED_M_COMP,
                        MIXED_M_MEM, MIXED_P, MIXED_SCHEDULE, MMDIT_PACKED,
                        MMDIT_TEXT_TOKENS, PACKED, PACKED_MIXED, TINY_F32,
                        VIDEO_BUCKET, WIDE_ROWS, Workload, custom,
                        mixed_bucket)
from .gen import (Inputs, PackedInputs, make_inputs, make_packed,
                  mixed_schedule, mmdit_layout, pack_lengths, torch_dtype)

__all__ = [
    "ALL", "BY_NAME", "EPS", "IMAGE_BUCKET", "LARGE_MODEL", "MIXED_BUCKETS",
    "MIXED_LENGTHS", "MIXED_M_COMP", "MIXED_M_MEM", "MIXED_P",
    "MIXED_SCHEDULE", "TINY_F32", "VIDEO_BUCKET", "Workload", "custom",
    "mixed_bucket", "Inputs", "make_inputs", "mixed_schedule", "torch_dtype",
    "MMDIT_PACKED", "MMDIT_TEXT_TOKENS", "PACKED", "PACKED_MIXED",
    "PackedInputs", "make_packed", "mmdit_layout", "pack_lengths",
    "WIDE_ROWS",
]
