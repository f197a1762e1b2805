"""PyTorch autograd wiring for the library's entry points.

`rms_norm(x, w, ...)` and `fused_add_rms_norm(x, residual, w, ...)` behave
like differentiable torch ops: their forward calls `rmsnorm_fwd` /
`fused_add_rmsnorm_fwd`, their backward `rmsnorm_backward` (the VJP of the
MLX pull request "RMSNormVJP backward writes a full {n_rows, D} gw_temp
intermediate", with the weight gradient summed over rows inside the library
and returned in the weight's dtype).  Every arithmetic step runs in the HIP
kernels; this module only saves tensors for the backward and routes
gradients.  `RMSNorm` is a module holding the weight; `silu_gate_op` is the
differentiable gated activation (backward: `silu_gate_vjp`).
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import binding as B


def _c(t: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    return None if t is None else t.contiguous()


class _RMSNormFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, w, eps, weight_bias):
        x, w = x.contiguous(), w.contiguous()
        y = B.rmsnorm_fwd(x, w, eps, weight_bias)
        ctx.save_for_backward(x, w)
        ctx.eps, ctx.wb = eps, weight_bias
        return y

    @staticmethod
    def backward(ctx, dy):
        x, w = ctx.saved_tensors
        _, dx, dw = B.rmsnorm_backward(x, w, dy.contiguous(), ctx.eps, ctx.wb, dw_dtype=w.dtype)
        return dx, dw, None, None


class _FusedAddRMSNormFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, residual, w, eps, weight_bias):
        x, residual, w = x.contiguous(), residual.contiguous(), w.contiguous()
        normed, new_residual = B.fused_add_rmsnorm_fwd(x, residual, w, eps, weight_bias)
        # the backward recomputes the row statistic from the saved sum
        ctx.save_for_backward(new_residual, w)
        ctx.eps, ctx.wb = eps, weight_bias
        return normed, new_residual

    @staticmethod
    def backward(ctx, d_normed, d_new_residual):
        h, w = ctx.saved_tensors
        if d_normed is None:
            d_normed = torch.zeros_like(h)
        _, dh, dw = B.rmsnorm_backward(h, w, d_normed.contiguous(), ctx.eps, ctx.wb,
                                       d_new_residual=_c(d_new_residual), dw_dtype=w.dtype)
        # h = x + residual: the same gradient reaches both
        return dh, dh, dw, None, None


class _SiluGateFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x):
        x = x.contiguous()
        ctx.save_for_backward(x)
        return B.silu_gate(x)

    @staticmethod
    def backward(ctx, dy):
        (x,) = ctx.saved_tensors
        return B.silu_gate_vjp(x, dy.contiguous())


def silu_gate_op(x: torch.Tensor) -> torch.Tensor:
    """Differentiable silu(x[..., :d]) * x[..., d:2d]."""
    return _SiluGateFn.apply(x)


def rms_norm(x: torch.Tensor, w: torch.Tensor, eps: float = 1e-5,
             weight_bias: float = 0.0) -> torch.Tensor:
    """Differentiable y = x * rsqrt(mean(x^2, -1) + eps) * (weight_bias + w)."""
    return _RMSNormFn.apply(x, w, eps, weight_bias)


def fused_add_rms_norm(x: torch.Tensor, residual: torch.Tensor, w: torch.Tensor,
                       eps: float = 1e-6, weight_bias: float = 0.0
                       ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Differentiable (normed, new_residual) of the fused residual add."""
    return _FusedAddRMSNormFn.apply(x, residual, w, eps, weight_bias)


class RMSNorm(torch.nn.Module):
    """RMSNorm over the last axis with a learnable weight (initialised to
    1 - weight_bias, so that weight_bias + w starts at 1)."""

    def __init__(self, dim: int, eps: float = 1e-6, weight_bias: float = 0.0,
                 device=None, dtype=None):
        super().__init__()
        self.eps, self.weight_bias = float(eps), float(weight_bias)
        self.weight = torch.nn.Parameter(
            torch.full((dim,), 1.0 - self.weight_bias, device=device, dtype=dtype))

    def forward(self, x: torch.Tensor, residual: Optional[torch.Tensor] = None):
        if residual is None:
            return rms_norm(x, self.weight, self.eps, self.weight_bias)
        return fused_add_rms_norm(x, residual, self.weight, self.eps, self.weight_bias)
