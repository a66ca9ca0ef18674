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
    if next_w is not None:
        nx = rmsnorm(h, next_w, next_bias, eps)
        y_exact, rn = nx.y_exact, nx.rstd
        # the GPU's BF16 stream may differ from h by one ulp at rounding ties, which moves
        # y by up to one ulp of its own
        y_mag = np.abs(y_exact)
    return GatedResidual(h_exact, h, np.abs(residual) + np.abs(gn), y_exact, y_mag, nb.rstd, rn)


__all__ = ["gated_residual_rmsnorm", "GatedResidual"]
