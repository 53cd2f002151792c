"""Format / rounding design-space sweep ("FP4 All the Way", Describir: block size, scale format and
rounding method are the FP4 design choices explored; 16-element blocks with E4M3 scales, NVFP4,
come out best, with stochastic rounding on gradients and round-to-nearest in the forward pass).

For every configuration (block 8 / 16 / 32) x (E4M3 under the fp32 tensor scale, or E8M0) x
(RNE, SR) the HIP quantize-dequantize kernel (``nvfp4_qdq``) measures, per tensor, the relative
quantization MSE ||Q(x) - x||^2 / ||x||^2 (summed in the same pass), and, per GEMM, the relative
L2 error of the product of the dequantized operands against the product of the originals.  The
products themselves are an analysis step, not part of the training path: they run as fp32
matrix products (torch, full fp32 precision) on the dequantized values, whose accumulation error
(~1e-6) is far below the quantization errors measured (~1e-2 to 1e-1).  The two configurations
the library trains with, NVFP4 (block 16, E4M3) and MXFP4 (block 32, E8M0), also get the error of
the training path itself (``gemm_library``): the operands through the library's 1D quantizers
(the same codes as the sweep kernel's, with the same seeds) and the product through its NVFP4 or
MXFP4 GEMM.
"""
from __future__ import annotations

import torch

from . import E4M3, E8M0, RNE, SR, gemm, mx_gemm, mx_quantize_1d, qdq, quantize_1d

CONFIGS = [(b, f, r) for b in (8, 16, 32) for f in (E4M3, E8M0) for r in (RNE, SR)]


def config_name(block: int, fmt: int, rounding: int) -> str:
    return f"B{block}-{'E4M3' if fmt == E4M3 else 'E8M0'}-{'RNE' if rounding == RNE else 'SR'}"


def bits_per_element(block: int, fmt: int, numel: int) -> float:
    """Storage: 4-bit codes, one 8-bit scale per block, plus the fp32 tensor scale for E4M3."""
    return 4.0 + 8.0 / block + (32.0 / numel if fmt == E4M3 else 0.0)


def rel_mse(x: torch.Tensor, block: int, fmt: int, rounding: int, seed: int = 0) -> float:
    sums = torch.empty(2, dtype=torch.float64, device=x.device)
    qdq(x, block, fmt, rounding, seed, sums=sums)
    g2, e2 = sums.tolist()
    return e2 / g2 if g2 > 0 else 0.0


def gemm_rel_error(a: torch.Tensor, b: torch.Tensor, block: int, fmt: int, rounding_a: int,
                   rounding_b: int, seed: int = 0, ref: torch.Tensor | None = None) -> float:
    """||Q(A) Q(B)^T - A B^T|| / ||A B^T|| with both operands quantized along K (their rows)."""
    qa, _, _ = qdq(a, block, fmt, rounding_a, seed)
    qb, _, _ = qdq(b, block, fmt, rounding_b, seed + 1)
    if ref is None:
        ref = a.float() @ b.float().t()
    return float(torch.linalg.norm(qa @ qb.t() - ref) / torch.linalg.norm(ref))


def gemm_library_rel_error(a: torch.Tensor, b: torch.Tensor, block: int, fmt: int, rounding_a: int,
                           rounding_b: int, seed: int, ref: torch.Tensor) -> float | None:
    """The same error through the training path: NVFP4 (block 16, E4M3) or MXFP4 (block 32, E8M0)
    operands from the library's 1D quantizers (seeds as in gemm_rel_error) multiplied by its
    GEMM with fp32 output; None for the configurations the library does not train with."""
    if (block, fmt) == (16, E4M3):
        c = gemm(quantize_1d(a, rounding_a, seed), quantize_1d(b, rounding_b, seed + 1))
    elif (block, fmt) == (32, E8M0):
        c = mx_gemm(mx_quantize_1d(a, rounding_a, seed), mx_quantize_1d(b, rounding_b, seed + 1))
    else:
        return None
    return float(torch.linalg.norm(c - ref) / torch.linalg.norm(ref))


def format_sweep(tensors: dict, gemms: list, configs=CONFIGS) -> dict:
    """tensors: name -> 2-D tensor (K contiguous).  gemms: (name, A, B, a_is_gradient) with
    C = A B^T.  Following the recipe (forward operands round to nearest, gradients
    stochastically), a gradient A takes the configuration's rounding and every other operand
    rounds to nearest; the per-tensor MSE uses the configuration's rounding for every tensor.
    Returns {config: {"bits": b, "mse": {tensor: rel MSE}, "gemm": {gemm: rel L2}}}, with
    "gemm_library" ({gemm: rel L2} through the library's quantizers and GEMMs) for NVFP4 and MXFP4."""
    prev = torch.backends.cuda.matmul.allow_tf32
    torch.backends.cuda.matmul.allow_tf32 = False
    try:
        refs = {name: a.float() @ b.float().t() for name, a, b, _ in gemms}
        out = {}
        for block, fmt, rnd in configs:
            numel = max(t.numel() for t in tensors.values())
            res = {"bits": round(bits_per_element(block, fmt, numel), 4), "mse": {}, "gemm": {}}
            for name, t in tensors.items():
                res["mse"][name] = rel_mse(t, block, fmt, rnd, 7)
            for name, a, b, a_grad in gemms:
                ra = rnd if a_grad else RNE
                res["gemm"][name] = gemm_rel_error(a, b, block, fmt, ra, RNE, 11, refs[name])
                lib_err = gemm_library_rel_error(a, b, block, fmt, ra, RNE, 11, refs[name])
                if lib_err is not None:
                    res.setdefault("gemm_library", {})[name] = lib_err
            out[config_name(block, fmt, rnd)] = res
        return out
    finally:
        torch.backends.cuda.matmul.allow_tf32 = prev


__all__ = ["CONFIGS", "config_name", "bits_per_element", "rel_mse", "gemm_rel_error",
           "gemm_library_rel_error", "format_sweep"]
