"""Host-side reading of the quantization-noise diagnostic.

"FP4 All the Way" (Describir) observes that fully quantized training stops making progress once
the gradient norm falls below about sqrt(3) times the quantization noise.  The library's
``*_noise`` quantizers return the two sums this needs (sum g^2 and sum (Q(g) - g)^2, fp64 on the
device); this module turns them into the two norms, their ratio and the sqrt(3) flag.  It is an
analysis step on two scalars, outside the quantization path, and calls no library function.
"""
from __future__ import annotations

import math

import torch

SQRT3 = math.sqrt(3.0)


def noise_report(sums: torch.Tensor) -> dict:
    """Norms and ratio from the two sums: quantized training is flagged as inefficient when
    ||g|| < sqrt(3) * ||Q(g) - g||."""
    g2, e2 = (float(v) for v in sums.cpu().tolist())
    g, e = math.sqrt(g2), math.sqrt(e2)
    ratio = g / e if e > 0 else float("inf")
    return {"grad_norm": g, "noise_norm": e, "ratio": ratio, "below_sqrt3": ratio < SQRT3}


__all__ = ["noise_report", "SQRT3"]
