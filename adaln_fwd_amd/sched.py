"""Dual-constraint bucket scheduling on one GPU (AdaptiveLoad technical
summary, section 2.A): shape benchmarking of a synthetic training step, the
step-time cost model t = a + b * B * S^p, the compute bound it implies, and
the resulting bucket batch sizes.

The arithmetic (the least-squares fit, the compute bound it implies and the
bucket rule) runs in ``libadaln.so`` (``adaln_costfit``, ``adaln_mcomp``,
``adaln_bshape_real``); this module marshals arrays and times the synthetic
step.

The synthetic step of a [B, S, D] bucket is the AdaLN forward (this
library), self-attention over the normalised tokens, forward and backward
(PyTorch's fused scaled-dot-product attention, flash or memory-efficient
kernels only -- no fallback to the unfused path), and the AdaLN backward
(this library): the operator the pages fuse plus the O(S^2) part whose cost
the compute constraint accounts for, both directions of a training step.
"""

from __future__ import annotations

import ctypes
import math
from dataclasses import asdict, dataclass
from typing import Dict, Iterable, List, Sequence, Tuple

from . import _lib


@dataclass
class CostModel:
    """t = a + b * B * S^p (t in the unit of the samples)."""
    a: float
    b: float
    p: float
    rss: float
    r2: float = float("nan")

    def predict(self, B: float, S: float) -> float:
        return self.a + self.b * B * S ** self.p


def costfit(B: Sequence[float], S: Sequence[float], t: Sequence[float],
            p_lo: float = 0.5, p_hi: float = 3.0) -> CostModel:
    """Least-squares fit of the cost model to measured samples."""
    n = len(t)
    if not (len(B) == len(S) == n):
        raise ValueError("B, S and t must have the same length")
    arr = ctypes.c_double * n
    b_, s_, t_ = arr(*map(float, B)), arr(*map(float, S)), arr(*map(float, t))
    out = (ctypes.c_double * 4)()
    lib = _lib.load()
    rc = lib.adaln_costfit(ctypes.cast(b_, ctypes.c_void_p),
                           ctypes.cast(s_, ctypes.c_void_p),
                           ctypes.cast(t_, ctypes.c_void_p), n, float(p_lo),
                           float(p_hi), ctypes.cast(out, ctypes.c_void_p))
    _lib.check(rc, "adaln_costfit")
    tm = sum(t) / n
    tss = sum((v - tm) ** 2 for v in t)
    r2 = 1.0 - out[3] / tss if tss > 0 else float("nan")
    return CostModel(a=out[0], b=out[1], p=out[2], rss=out[3], r2=r2)


def bshape_real(S: int, m_mem: int, m_comp: float, p: float) -> int:
    """Bucket batch size with a real exponent and compute bound."""
    v = int(_lib.load().adaln_bshape_real(int(S), int(m_mem), float(m_comp),
                                          float(p)))
    if v < 1:
        _lib.check(v, "adaln_bshape_real")
    return v


def m_comp_for(p: float, m_mem: int, s_ref: int) -> float:
    """The compute bound that caps every bucket at the predicted cost of the
    memory-bound bucket of length s_ref (``adaln_mcomp`` in the library)."""
    lib = _lib.load()
    v = float(lib.adaln_mcomp(float(p), int(m_mem), int(s_ref)))
    if v < 0:
        _lib.check(_lib.ERR_INVALID, "adaln_mcomp")
    return v


def buckets(lengths: Iterable[int], m_mem: int, m_comp: float,
            p: float) -> Dict[int, int]:
    return {int(S): bshape_real(S, m_mem, m_comp, p) for S in lengths}


def pearson(x: Sequence[float], y: Sequence[float]) -> float:
    n = len(x)
    mx, my = sum(x) / n, sum(y) / n
    sxy = sum((a - mx) * (b - my) for a, b in zip(x, y))
    sxx = sum((a - mx) ** 2 for a in x)
    syy = sum((b - my) ** 2 for b in y)
    return sxy / math.sqrt(sxx * syy) if sxx > 0 and syy > 0 else float("nan")


def cv(values: Sequence[float], weights: Sequence[float] = None) -> float:
    """Coefficient of variation (weighted standard deviation / mean)."""
    if weights is None:
        weights = [1.0] * len(values)
    w = sum(weights)
    m = sum(v * q for v, q in zip(values, weights)) / w
    var = sum(q * (v - m) ** 2 for v, q in zip(values, weights)) / w
    return math.sqrt(var) / m


class SyntheticStep:
    """Times the synthetic step of one bucket shape on the current GPU."""

    def __init__(self, D: int = 3072, heads: int = 24, device="cuda",
                 attention_backward: bool = True):
        import torch
        if D % heads:
            raise ValueError("D must be a multiple of heads")
        self.D, self.heads, self.device = D, heads, torch.device(device)
        self.attention_backward = attention_backward

    def run(self, B: int, S: int, iters: int = 5, warmup: int = 2
            ) -> List[float]:
        """Durations (ms) of `iters` steps after `warmup` untimed ones."""
        import torch
        import torch.nn.functional as F
        from torch.nn.attention import SDPBackend, sdpa_kernel
        from . import ops
        D, H = self.D, self.heads
        dev = self.device
        g = torch.Generator(device=dev)
        g.manual_seed(B * 100003 + S)
        x = torch.randn(B, S, D, device=dev, dtype=torch.bfloat16,
                        generator=g)
        dy = torch.randn(B, S, D, device=dev, dtype=torch.bfloat16,
                         generator=g) * 0.01
        scale = torch.randn(B, D, device=dev, dtype=torch.bfloat16,
                            generator=g) * 0.1
        shift = torch.randn(B, D, device=dev, dtype=torch.bfloat16,
                            generator=g) * 0.1
        y = torch.empty_like(x)
        dx = torch.empty_like(x)
        mean = torch.empty(B, S, device=dev, dtype=torch.float32)
        rstd = torch.empty_like(mean)
        dscale = torch.empty(B, D, device=dev, dtype=torch.float32)
        dshift = torch.empty_like(dscale)
        ws = torch.empty(max(1, ops.bwd_workspace_bytes(B, S, D,
                                                        torch.bfloat16)),
                         dtype=torch.uint8, device=dev)
        # q = k = v: the normalised tokens as H heads (a view of y); the
        # attention's own gradient input is a fixed random tensor
        qkv = y.view(B, S, H, D // H).transpose(1, 2).detach()
        back = self.attention_backward
        if back:
            qkv.requires_grad_(True)
            d_out = torch.randn(B, H, S, D // H, device=dev,
                                dtype=torch.bfloat16, generator=g)

        def step():
            ops.fwd(x, scale, shift, y=y, mean=mean, rstd=rstd)
            with sdpa_kernel([SDPBackend.FLASH_ATTENTION,
                              SDPBackend.EFFICIENT_ATTENTION]):
                out = F.scaled_dot_product_attention(qkv, qkv, qkv)
                if back:
                    out.backward(d_out)
                    qkv.grad = None
            ops.bwd(dy, x, scale, mean, rstd, dx=dx, dscale=dscale,
                    dshift=dshift, workspace=ws)

        for _ in range(warmup):
            step()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(iters + 1)]
        torch.cuda.synchronize(dev)
        ev[0].record()
        for i in range(iters):
            step()
            ev[i + 1].record()
        torch.cuda.synchronize(dev)
        # the last step's AdaLN inputs and outputs, for callers that check
        # them against the operator called on its own
        self.last = dict(x=x, dy=dy, scale=scale, shift=shift, y=y, dx=dx,
                         mean=mean, rstd=rstd, dscale=dscale, dshift=dshift)
        return [ev[i].elapsed_time(ev[i + 1]) for i in range(iters)]


def sweep_shapes(lengths: Iterable[int], m_mem: int) -> List[Tuple[int, int]]:
    """(B, S) pairs of a shape benchmark: for each length the memory-bound
    batch B_mem = m_mem // S, its half and quarter, and 1 and 2."""
    out = []
    for S in lengths:
        bm = max(1, m_mem // S)
        for B in sorted({1, 2, max(1, bm // 4), max(1, bm // 2), bm}):
            if B <= bm:
                out.append((B, int(S)))
    return out


def report_dict(model: CostModel) -> dict:
    return asdict(model)
