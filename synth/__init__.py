"""Seeded synthetic workloads and inputs for the fused AdaLN operator.

Shared by the HIP path's callers and the oracle's tests; holds no part of the
method's arithmetic."""

from .workloads import (ALL, BY_NAME, EPS, IMAGE_BUCKET, LARGE_MODEL,
                        MIXED_BUCKETS, MIXED_LENGTHS, MIXED_M_COMP,
                        MIXED_M_MEM, MIXED_P, MIXED_SCHEDULE, TINY_F32,
                        VIDEO_BUCKET, Workload, custom, mixed_bucket)
from .gen import Inputs, make_inputs, mixed_schedule, torch_dtype

__all__ = [
    "ALL", "BY_NAME", "EPS", "IMAGE_BUCKET", "LARGE_MODEL", "MIXED_BUCKETS",
    "MIXED_LENGTHS", "MIXED_M_COMP", "MIXED_M_MEM", "MIXED_P",
    "MIXED_SCHEDULE", "TINY_F32", "VIDEO_BUCKET", "Workload", "custom",
    "mixed_bucket", "Inputs", "make_inputs", "mixed_schedule", "torch_dtype",
]
