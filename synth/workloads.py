"""Workload definitions for the fused AdaLN operator: shapes, dtypes and the
value distributions of the synthetic inputs.

Each workload stands in for the activations of Wan 2.1 video-diffusion
training, which the AdaptiveLoad technical summary (gist.science) trains on a
10M-sample WebDataset + Koala-36M corpus (section 4, experimental results).
Neither the corpus nor the model weights are available, so every tensor here
is drawn from a seeded distribution with the shapes of that model's token
rows: one latent frame of 30x52 patches, 21 frames of 30x52, and 21 frames of
45x80 latent tokens.

Notation: ``N(m, s)`` takes ``s`` as the standard deviation.

Nothing in this module computes any part of the AdaLN method.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple

# Modulation bounds for the mixed-length schedule (dual-constraint bucket
# sizing of section 2.A of the AdaptiveLoad technical summary): memory bound,
# compute bound and exponent.
MIXED_M_MEM = 131_072
MIXED_M_COMP = 2_200_000_000
MIXED_P = 2
MIXED_LENGTHS = (1560, 8190, 16380, 32760)
MIXED_BUCKETS = 64

EPS = 1e-6


@dataclass(frozen=True)
class Workload:
    """One synthetic AdaLN workload.

    ``x_kind`` selects how token activations are drawn:

    * ``"normal"``   -- x ~ N(0, 1)
    * ``"offset"``   -- x ~ N(0, 1) + o[d], one offset vector o ~ N(0, 0.5)
                        of length D per workload, added to every token row
    * ``"outliers"`` -- x ~ N(0, 1), with each entry independently replaced,
                        with probability 0.001, by a draw from N(0, 20)

    ``scale`` and ``shift`` are per-sample vectors of shape [B, D] drawn from
    N(0, ``mod_std``); ``dy`` is drawn from N(0, ``dy_std``).
    """

    name: str
    index: int                 # stable id, part of every seed
    B: Optional[int]           # None for the mixed schedule (per bucket)
    N: Optional[int]
    D: int
    dtype: str                 # "f32" or "bf16"
    x_kind: str
    mod_std: float = 0.1
    dy_std: float = 1.0
    offset_std: float = 0.5
    outlier_p: float = 1e-3
    outlier_std: float = 20.0
    note: str = ""

    @property
    def rows(self) -> int:
        assert self.B is not None and self.N is not None
        return self.B * self.N

    @property
    def shape(self) -> Tuple[int, int, int]:
        assert self.B is not None and self.N is not None
        return (self.B, self.N, self.D)


TINY_F32 = Workload(
    name="tiny_f32", index=0, B=2, N=256, D=64, dtype="f32", x_kind="normal",
    mod_std=0.1, dy_std=1.0,
    note="tiny fp32 case; the oracle finishes it in well under a second")

IMAGE_BUCKET = Workload(
    name="image_bucket", index=1, B=16, N=1560, D=1536, dtype="bf16",
    x_kind="offset", mod_std=0.1, dy_std=1e-2,
    note="16 images, one latent frame of 30x52 patches each")

VIDEO_BUCKET = Workload(
    name="video_bucket", index=2, B=1, N=32760, D=1536, dtype="bf16",
    x_kind="offset", mod_std=0.1, dy_std=1e-2,
    note="one video, 21x30x52 latent tokens; long-N column reduction")

LARGE_MODEL = Workload(
    name="large_model", index=3, B=1, N=75600, D=5120, dtype="bf16",
    x_kind="outliers", mod_std=0.1, dy_std=1e-2,
    note="one video, 21x45x80 latent tokens, D=5120 hidden width")

MIXED_SCHEDULE = Workload(
    name="mixed_schedule", index=4, B=None, N=None, D=3072, dtype="bf16",
    x_kind="offset", mod_std=0.1, dy_std=1e-2,
    note="64 buckets with S drawn uniformly from {1560, 8190, 16380, 32760}, "
         "batch per bucket from the dual-constraint rule")

# Packed (unpadded) layouts: the token rows of several sequences back to back
# in one [T, D] tensor, each sequence (segment) with its own modulation.
PACKED_MIXED = Workload(
    name="packed_mixed", index=5, B=None, N=None, D=3072, dtype="bf16",
    x_kind="offset", mod_std=0.1, dy_std=1e-2,
    note="mixed-length samples (lengths uniform over the mixed schedule's "
         "four) packed back to back up to the 131072-token memory budget, "
         "one modulation vector per sample")

MMDIT_TEXT_TOKENS = 512
MMDIT_PACKED = Workload(
    name="mmdit_packed", index=6, B=4, N=MMDIT_TEXT_TOKENS + 16380, D=3072,
    dtype="bf16", x_kind="offset", mod_std=0.1, dy_std=1e-2,
    note="4 samples of a two-stream (MMDiT) block, each a 512-token text "
         "segment followed by a 16380-token video segment; text and video "
         "tokens have their own modulation vectors, laid out [2, B, D] "
         "(text of every sample, then video)")

# Rows wider than one wavefront's registers in the backward (8192 features,
# split between two wavefronts), at the large model's activation size.
WIDE_ROWS = Workload(
    name="wide_rows", index=7, B=1, N=49152, D=8192, dtype="bf16",
    x_kind="outliers", mod_std=0.1, dy_std=1e-2,
    note="one sequence of 49152 tokens at D=8192 (805 MB per activation "
         "tensor), the large model's distributions")

ALL = (TINY_F32, IMAGE_BUCKET, VIDEO_BUCKET, LARGE_MODEL, MIXED_SCHEDULE)
PACKED = (PACKED_MIXED, MMDIT_PACKED)
EXTRA = (WIDE_ROWS,)
BY_NAME = {w.name: w for w in ALL + PACKED + EXTRA}


def custom(B: int, N: int, D: int, dtype: str, x_kind: str = "normal",
           index: int = 100, mod_std: float = 0.1, dy_std: float = 1.0,
           name: str = "custom") -> Workload:
    """A workload of arbitrary shape, for edge-case tests."""
    return Workload(name=name, index=index, B=B, N=N, D=D, dtype=dtype,
                    x_kind=x_kind, mod_std=mod_std, dy_std=dy_std)


def mixed_bucket(B: int, S: int) -> Workload:
    """The workload of one bucket of the mixed schedule: [B, S, 3072] bf16."""
    w = MIXED_SCHEDULE
    return Workload(name=f"mixed_S{S}_B{B}", index=w.index, B=B, N=S, D=w.D,
                    dtype=w.dtype, x_kind=w.x_kind, mod_std=w.mod_std,
                    dy_std=w.dy_std)
