"""Autograd wrapper of the training RMSNorm over the C ABI.

The forward saves only (x or h_new, w, rstd) -- no other [T, H] tensor -- and the backward
is one dn_train_backward call (norm docs, "Training RMSNorm (Cake)": cake_rmsnorm and
CakeRMSNormFunction; norm guide §6.4).  With a residual the forward returns (y, h_new),
h_new = BF16(x + residual); the gradient reaching h_new directly is passed to the kernel as
g_residual, and the resulting dx is the gradient of both x and residual (norm guide §6.2).
dw is accumulated in FP32 by the kernel and written in w's dtype (for a BF16 weight, the FP32
value rounded once more, in the kernel).
"""
from __future__ import annotations

import torch

from . import dnorm as dn


class RMSNormTrainFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, w, eps, w_bias, residual):
        if residual is None:
            y, rstd = dn.dn_train_forward(x, w, eps, w_bias=w_bias)
            ctx.save_for_backward(x, w, rstd)
            ctx.residual = False
            ctx.w_bias = w_bias
            return y
        y, rstd, h_new = dn.dn_train_forward(x, w, eps, w_bias=w_bias, residual=residual)
        ctx.save_for_backward(h_new, w, rstd)
        ctx.residual = True
        ctx.w_bias = w_bias
        return y, h_new

    @staticmethod
    def backward(ctx, *grads):
        x, w, rstd = ctx.saved_tensors
        gy = grads[0]
        gh = grads[1] if ctx.residual and len(grads) > 1 else None
        if gy is None:
            gy = torch.zeros_like(x)
        # Gradients are read in place when their rows are addressable (row-strided views
        # included); broadcast or transposed ones are copied once by the binding.
        dx, dw = dn.dn_train_backward(gy, x, w, rstd, w_bias=ctx.w_bias, g_residual=gh,
                                      dw_dtype=w.dtype)
        if ctx.residual:
            return dx, dw, None, None, dx
        return dx, dw, None, None, None


def rmsnorm_train(x, w, eps: float = 1e-6, *, w_bias: float = 0.0, residual=None):
    """Autograd-enabled RMSNorm: y (or (y, h_new) with a residual).

    x, residual: BF16 [..., H]; w: BF16 or FP32 [H] (FP32 with w_bias = 1 for a
    zero-centred weight whose effective value is 1 + w).
    """
    return RMSNormTrainFunction.apply(x, w, eps, w_bias, residual)
