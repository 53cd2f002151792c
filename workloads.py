"""Seeded synthetic inputs for the NVFP4 hot path (shared by the tests, the smoke check and the
benchmark).

This module only draws random numbers and casts them to the input dtype; it holds none of the
quantization arithmetic, so both the HIP path and the CPU oracle can take their inputs from it.

Recipe (every tensor): numpy ``Generator(PCG64(seed))`` in float64 -> float32 -> torch cast to
bf16 (round to nearest even) where the workload is bf16.  Outliers and spikes pick exactly
``floor(frac * n)`` distinct positions with ``rng.choice(n, k, replace=False)`` (drawn after the
base values from the same generator) and multiply them in float64.

The workloads are LLM-shaped linear-layer tensors: activations are heavy-tailed (Student-t with
3 degrees of freedom), weights N(0, 0.02), output gradients N(0, 1e-3) with 0.1% spikes x100.
They stand in for the training runs the pages describe (no datasets or checkpoints are used).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _finish(v: np.ndarray, shape, dtype: torch.dtype) -> torch.Tensor:
    t = torch.from_numpy(v.astype(np.float32).reshape(shape))
    return t if dtype == torch.float32 else t.to(dtype)


def normal(shape, sigma: float, seed: int, spike_frac: float = 0.0, spike_mult: float = 1.0,
           dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """N(0, sigma^2) with floor(spike_frac * n) distinct entries multiplied by spike_mult."""
    rng = _rng(seed)
    n = int(np.prod(shape))
    v = rng.standard_normal(n) * sigma
    k = int(np.floor(spike_frac * n))
    if k > 0:
        idx = rng.choice(n, k, replace=False)
        v[idx] *= spike_mult
    return _finish(v, shape, dtype)


def edge_fp32(kind: str, shape, seed: int, dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """Tensors at the edges of the formats' ranges (the degenerate cases of the method), fp32
    unless dtype says otherwise (bf16 has the same exponent range):
      "tiny"       N(0,1) * 1e-38: fp32 subnormals, amax below the 2^-100 zero threshold
      "near_zero"  N(0,1) * 1e-29: amax just above that threshold (huge tensor scale factors)
      "huge"       N(0,1) * 1e37: amax near the top of the fp32 range
      "wide"       random signs times 2^u, u uniform in [-70, 12): blocks whose E4M3 scale is
                   subnormal or zero next to blocks with large values
      "signed_zeros" mostly +0 and -0, with 1% N(0,1) entries
      "tiny_mix"   N(0,1) * 2^-131 (subnormal) with 2% of the entries times 2^36: an amax
                   around 2^-93, blocks of subnormal values, and subnormal values beside
                   normal ones in a block
      "below_2p120", "above_2p120"  N(0,1) * 2^115 and * 2^119: a Hadamard-transformed amax just
                   below and just above 2^120."""
    rng = _rng(seed)
    n = int(np.prod(shape))
    if kind == "tiny_mix":
        v = rng.standard_normal(n) * 2.0 ** -131
        k = n // 50
        idx = rng.choice(n, k, replace=False)
        v[idx] = v[idx] * 2.0 ** 36
        return _finish(v, shape, dtype)
    if kind in ("below_2p120", "above_2p120"):
        v = rng.standard_normal(n) * 2.0 ** (115 if kind == "below_2p120" else 119)
        return _finish(v, shape, dtype)
    if kind == "tiny":
        v = rng.standard_normal(n) * 1e-38
    elif kind == "near_zero":
        v = rng.standard_normal(n) * 1e-29
    elif kind == "huge":
        v = rng.standard_normal(n) * 1e37
    elif kind == "wide":
        v = np.where(rng.random(n) < 0.5, -1.0, 1.0) * np.exp2(rng.uniform(-70.0, 12.0, n))
    elif kind == "signed_zeros":
        v = np.where(rng.random(n) < 0.5, -0.0, 0.0)
        k = n // 100
        if k > 0:
            v[rng.choice(n, k, replace=False)] = rng.standard_normal(k)
    else:
        raise ValueError(kind)
    return _finish(v, shape, dtype)


def student_t(shape, nu: float, seed: int, dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    rng = _rng(seed)
    n = int(np.prod(shape))
    v = rng.standard_t(nu, n)
    return _finish(v, shape, dtype)


def device_normal_rows(shape, seed: int, device: str = "cuda") -> torch.Tensor:
    """A bf16 tensor too large to draw on the host in reasonable time (billions of elements):
    N(0, 1) drawn by torch's generator on the device, each row times 2^k with k uniform in
    [-12, 12] (exact in bf16), so that block scales span a wide range.  Seeded and deterministic;
    the oracle takes a host copy of the same tensor."""
    g = torch.Generator(device=device).manual_seed(seed)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.bfloat16)
    k = torch.randint(-12, 13, (shape[0], 1), generator=g, device=device)
    x.mul_(torch.exp2(k.to(torch.float32)).to(torch.bfloat16))
    return x


def bits(t: torch.Tensor) -> np.ndarray:
    """numpy view for the oracle: float32 as is, bf16 as its raw uint16 bit patterns."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    raise TypeError(t.dtype)


# ---- the five workloads ---------------------------------------------------------------------------
SR_SEED_DGRAD = 0x5EED0003
SR_SEED_WGRAD = 0x5EED0004
SIGN_SEED_WGRAD = 0x51E40004


def act(shape, seed):          # activations: Student-t(3)
    return student_t(shape, 3.0, seed)


def weight(shape, seed):       # weights: N(0, 0.02)
    return normal(shape, 0.02, seed)


def grad(shape, seed):         # output gradients: N(0, 1e-3), 0.1% spikes x100
    return normal(shape, 1e-3, seed, spike_frac=1e-3, spike_mult=100.0)


def small_fp32(shape, seed):   # 1% outliers x50 on N(0, 1), fp32
    return normal(shape, 1.0, seed, spike_frac=1e-2, spike_mult=50.0, dtype=torch.float32)


@dataclass(frozen=True)
class Linear:
    """One linear layer's training-step shapes: tokens T, in-features K_in, out-features N_out."""
    tokens: int
    k_in: int
    n_out: int


# cfg1: 256x256 fp32 quantize/dequantize + 256^3 GEMM (seeds 101, 102)
CFG1 = dict(shape=(256, 256), seeds=(101, 102))
# cfg2: fprop Y = X W^T, X 8192x4096 Student-t(3) (seed 201), W 4096x4096 N(0,0.02) (seed 202)
CFG2 = dict(x=(8192, 4096), w=(4096, 4096), seeds=(201, 202))
# cfg3: dgrad dX = dY W, dY 8192x4096 N(0,1e-3) + spikes (seed 301), SR seed 0x5EED0003
CFG3 = dict(dy=(8192, 4096), seed=301, sr_seed=SR_SEED_DGRAD)
# cfg4: wgrad dW = dY^T X with the random Hadamard on the token dim, 16384 tokens
CFG4 = dict(x=(16384, 4096), dy=(16384, 4096), seeds=(401, 402), sign_seed=SIGN_SEED_WGRAD,
            sr_seed=SR_SEED_WGRAD)
# cfg5: FFN pair up 5120->20480, down 20480->5120, 16384 tokens (seeds 501..506)
CFG5 = dict(tokens=16384, d_model=5120, d_ff=20480, seeds=(501, 502, 503, 504, 505, 506),
            # per layer: Hadamard sign seed, SR seed of the dgrad operand, SR seed of the wgrad one
            layer_seeds={"up": (0x51E40051, 0x5EED0051, 0x5EED0052),
                         "down": (0x51E40052, 0x5EED0053, 0x5EED0054)})
