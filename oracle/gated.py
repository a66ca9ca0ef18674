"""Plain FP64 reference of the gated-residual RMSNorms (slow, obviously correct).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  It shares no code with the GPU library.

norm docs, Fixed-Width Fused Norms: gated_residual_rmsnorm(branch, residual, ...) blends a
normalised branch into the residual stream; gated_residual_next_rmsnorm(branch, ...) also
applies the next RMSNorm in the same launch (the pages' kernels take hidden 8192 only).
The pages give no formula.  Reading implemented (the plainest that the names support):
    n = RMSNorm(branch, w)                       (as oracle.rmsnorm, unrounded)
    h = residual + gate * n                      (gate BF16: one row per token, or one row
                                                  shared by every token)
    residual <- BF16(h)
    next:  y = RMSNorm(BF16(h), w_next)          (the norm sees the stored BF16 stream)
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .formats import bf16_round
from .rmsnorm import rmsnorm


@dataclass
class GatedResidual:
    h_exact: np.ndarray
    h: np.ndarray            # BF16, the new residual stream
    h_mag: np.ndarray        # |residual| + |gate * n|
    y_exact: np.ndarray | None
    y_mag: np.ndarray | None
    rstd_branch: np.ndarray
    rstd_next: np.ndarray | None


def gated_residual_rmsnorm(branch, residual, gate, w, eps: float = 1e-6, bias: float = 0.0,
                           next_w=None, next_bias: float = 0.0) -> GatedResidual:
    branch = np.asarray(branch, dtype=np.float64)
    residual = np.asarray(residual, dtype=np.float64)
    g = np.broadcast_to(np.asarray(gate, dtype=np.float64), branch.shape)
    nb = rmsnorm(branch, w, bias, eps)
    gn = g * nb.y_exact
    h_exact = residual + gn
    h = bf16_round(h_exact)
    y_exact = y_mag = rn = None
    h_mag = np.abs(residual) + np.abs(gn)
    if next_w is not None:
        nx = rmsnorm(h, next_w, next_bias, eps)
        y_exact, rn = nx.y_exact, nx.rstd
        # An FP32 evaluation of h may round to the other BF16 neighbour where h sits within
        # 2^-20 of its term magnitude from a rounding midpoint; the next norm then sees a
        # stream one ulp away there, which moves that element's y by one more ulp.  Such
        # elements get a magnitude that admits two ulps; the others one.
        band = 2.0 ** -20 * h_mag
        near = bf16_round(h_exact - band) != bf16_round(h_exact + band)
        y_mag = np.abs(y_exact) * np.where(near, 2.0 ** 15, 1.0)
    return GatedResidual(h_exact, h, h_mag, y_exact, y_mag, nb.rstd, rn)


__all__ = ["gated_residual_rmsnorm", "GatedResidual"]
