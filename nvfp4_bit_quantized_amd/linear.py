"""NVFP4 linear layer for training: a ``torch.autograd.Function`` over the C ABI, and a module
with a per-layer flag that keeps a layer in BF16.

The recipe of "Entrenamiento de Modelos de Lenguaje con 4 Bits de Precision" (Metodologia de
Entrenamiento) has four parts; three of them live in the kernels, and the fourth, keeping a few
numerically sensitive layers in higher precision ("I ricercatori di Nvidia ...", Come funziona
NVFP4?: most layers quantized, a small share kept in BF16), is the ``high_precision`` flag here.

One training step of ``y = x W^T`` (x [T x in], W [out x in]; "FP4 All the Way", Describir: the
forward pass rounds to nearest, backward and update passes round stochastically):
  forward   x -> row-wise NVFP4 (RNE) and, when a gradient will be needed, the random-Hadamard
            transposed copy [in x T] (one fused read of x); W -> 16x16-tile NVFP4 and its
            transposed copy [in x out]; y = gemm(x_q, W_q)
  backward  dy -> row-wise NVFP4 (SR, dgrad seed) and Hadamard-transposed copy [out x T] (SR,
            wgrad seed), one fused read; dx = gemm(dy_q, W_q^T) [T x in];
            dW = gemm(dy_q^T', x_q^T') [out x in], K = tokens, both operands through the same
            random signs so that the transform cancels in the product.
Every one of these steps runs in the HIP library; this file only allocates outputs and passes
pointers.  Shapes: T, in and out multiples of 16.

dW comes back in the weight's dtype, as autograd requires: for fp32 (master) weights it is the
wgrad GEMM's fp32 accumulation as is; for bf16 weights the GEMM rounds that fp32 result once to
bf16 (round to nearest even) on output.

The MXFP4 comparison format ("I ricercatori di Nvidia ...", NVFP4 in pratica: MXFP4 needed more
training data to match NVFP4) runs the same three GEMMs with every operand in MXFP4 (32-element
blocks, power-of-two scales applied by the matrix core), the same rounding per pass, and plain
transposes instead of the Hadamard transform, which belongs to the NVFP4 recipe.  Shapes there:
T, in and out multiples of 32.
"""
from __future__ import annotations

import torch

from . import (RNE, SR, gemm, mx_gemm, mx_quantize_1d, mx_quantize_1d_t, mx_quantize_dual,
               quantize_1d, quantize_2d, quantize_dual)

_MASK64 = (1 << 64) - 1


def _mix(a: int, b: int) -> int:
    """A 64-bit seed for call b of stream a (splitmix64 finaliser of a + b * golden ratio)."""
    z = (a + (b + 1) * 0x9E3779B97F4A7C15) & _MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


class NVFP4LinearFn(torch.autograd.Function):
    """y = x W^T with every GEMM operand in NVFP4 and fp32 accumulation."""

    @staticmethod
    def forward(ctx, x: torch.Tensor, w: torch.Tensor, sign_seed: int, seed_dgrad: int,
                seed_wgrad: int):
        need_grad = ctx.needs_input_grad[0] or ctx.needs_input_grad[1]
        if need_grad:
            qx, qxt = quantize_dual(x, sign_seed, RNE)          # fprop + wgrad operands of x
        else:
            qx, qxt = quantize_1d(x, RNE), None
        qw, qwt = quantize_2d(w, transposed=need_grad)          # fprop + dgrad operands of W
        y = gemm(qx, qw, x.dtype)
        ctx.q = (qxt, qwt)
        ctx.seeds = (sign_seed, seed_dgrad, seed_wgrad)
        ctx.dtypes = (x.dtype, w.dtype)
        return y

    @staticmethod
    def backward(ctx, dy: torch.Tensor):
        qxt, qwt = ctx.q
        sign_seed, seed_dgrad, seed_wgrad = ctx.seeds
        x_dt, w_dt = ctx.dtypes
        dy = dy.contiguous()
        qdy, qdyt = quantize_dual(dy, sign_seed, SR, seed_dgrad, seed_wgrad)
        dx = gemm(qdy, qwt, x_dt) if ctx.needs_input_grad[0] else None
        dw = gemm(qdyt, qxt, w_dt) if ctx.needs_input_grad[1] else None
        ctx.q = None
        return dx, dw, None, None, None


class MXFP4LinearFn(torch.autograd.Function):
    """y = x W^T with every GEMM operand in MXFP4 and fp32 accumulation (the comparison format).
    forward   x, W -> MXFP4 row-wise (RNE); y = mx_gemm(x_q, W_q); when a gradient will be
              needed, the same read of x and of W also gives x^T [in x T] and W^T [in x out]
              (mxfp4_quantize_dual)
    backward  dY -> MXFP4 row-wise (SR, dgrad seed) and dY^T [out x T] (SR, wgrad seed), from one
              read when both are needed; dx = mx_gemm(dY_q, W^T_q), dW = mx_gemm(dY^T_q, x^T_q)."""

    @staticmethod
    def forward(ctx, x: torch.Tensor, w: torch.Tensor, seed_dgrad: int, seed_wgrad: int):
        need_grad = ctx.needs_input_grad[0] or ctx.needs_input_grad[1]
        if need_grad:
            qx, qxt = mx_quantize_dual(x, RNE)
            qw, qwt = mx_quantize_dual(w, RNE)
            ctx.q = (qxt, qwt)
        else:
            qx, qw = mx_quantize_1d(x, RNE), mx_quantize_1d(w, RNE)
            ctx.q = None
        y = mx_gemm(qx, qw, x.dtype)
        ctx.seeds = (seed_dgrad, seed_wgrad)
        ctx.dtypes = (x.dtype, w.dtype)
        return y

    @staticmethod
    def backward(ctx, dy: torch.Tensor):
        qxt, qwt = ctx.q
        seed_dgrad, seed_wgrad = ctx.seeds
        x_dt, w_dt = ctx.dtypes
        dy = dy.contiguous()
        dx = dw = None
        if ctx.needs_input_grad[0] and ctx.needs_input_grad[1]:
            qdy, qdyt = mx_quantize_dual(dy, SR, seed_dgrad, seed_wgrad)
            dx, dw = mx_gemm(qdy, qwt, x_dt), mx_gemm(qdyt, qxt, w_dt)
        elif ctx.needs_input_grad[0]:
            dx = mx_gemm(mx_quantize_1d(dy, SR, seed_dgrad), qwt, x_dt)
        elif ctx.needs_input_grad[1]:
            dw = mx_gemm(mx_quantize_1d_t(dy, SR, seed_wgrad), qxt, w_dt)
        ctx.q = None
        return dx, dw, None, None


class NVFP4Linear(torch.nn.Module):
    """Linear layer without bias, W [out x in] in bf16 or fp32.

    high_precision=False: the NVFP4 path above.  high_precision=True: the layer stays in its own
    dtype (torch's linear), the selective-precision part of the recipe.  fmt="mxfp4" runs the
    MXFP4 comparison format instead of NVFP4.  ``sign_seed`` fixes the layer's random Hadamard
    signs; the stochastic-rounding seeds of each backward pass derive from ``seed`` and a
    per-layer call counter, so runs are reproducible."""

    def __init__(self, in_features: int, out_features: int, high_precision: bool = False,
                 dtype: torch.dtype = torch.bfloat16, device="cuda", seed: int = 0,
                 sign_seed: int | None = None, fmt: str = "nvfp4"):
        super().__init__()
        if fmt not in ("nvfp4", "mxfp4"):
            raise ValueError("fmt must be 'nvfp4' or 'mxfp4'")
        self.fmt, self.align = fmt, 16 if fmt == "nvfp4" else 32
        if in_features % self.align or out_features % self.align:
            raise ValueError(f"NVFP4Linear ({fmt}) needs in_features and out_features divisible "
                             f"by {self.align}")
        self.in_features, self.out_features = in_features, out_features
        self.high_precision = high_precision
        self.weight = torch.nn.Parameter(torch.empty((out_features, in_features), dtype=dtype,
                                                     device=device))
        self.seed = seed & _MASK64
        self.sign_seed = _mix(self.seed, _MASK64 >> 1) if sign_seed is None else sign_seed
        self.calls = 0

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        lead = x.shape[:-1]
        x2 = x.reshape(-1, self.in_features)
        if self.high_precision:
            y = torch.nn.functional.linear(x2, self.weight)
        else:
            if x2.shape[0] % self.align:
                raise ValueError(f"NVFP4Linear ({self.fmt}) needs the token count divisible by "
                                 f"{self.align}")
            x2 = x2.contiguous()
            s_d, s_w = _mix(self.seed, 2 * self.calls), _mix(self.seed, 2 * self.calls + 1)
            self.calls += 1
            if self.fmt == "mxfp4":
                y = MXFP4LinearFn.apply(x2, self.weight, s_d, s_w)
            else:
                y = NVFP4LinearFn.apply(x2, self.weight, self.sign_seed, s_d, s_w)
        return y.reshape(*lead, self.out_features)

    def extra_repr(self) -> str:
        mode = "bf16" if self.high_precision else self.fmt
        return f"in={self.in_features}, out={self.out_features}, {mode}"


__all__ = ["NVFP4LinearFn", "MXFP4LinearFn", "NVFP4Linear"]
