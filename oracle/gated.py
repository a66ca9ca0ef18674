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
Tolerances (h_mag, y_mag feed the cancellation-aware BF16 gate: one ulp, or within 2^-21 of
the magnitude): h_mag = |residual| + |gate * n|; y_mag = |y|, widened where h's band crosses
a BF16 rounding midpoint (below).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .formats import bf16_round
from .rmsnorm import effective_weight, rmsnorm


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
        # An FP32 evaluation of h lands within 2^-20 of its term magnitude h_mag of the exact
        # value (the h gate admits that much).  Where that band reaches past a BF16 rounding
        # midpoint, the stored h may be another BF16 number than the oracle's -- one ulp
        # away next to a midpoint, several where the sum cancels far below its terms -- and
        # the next norm sees that stream.  Such elements admit the band carried through the
        # next norm (h_mag * r * |w_eff|, the deviation of h times the factor the norm
        # applies) plus two ulps of y; the others one ulp.
        band = 2.0 ** -20 * h_mag
        near = bf16_round(h_exact - band) != bf16_round(h_exact + band)
        carried = 2.0 * h_mag * nx.r64[:, None] * np.abs(effective_weight(next_w, next_bias))
        y_mag = np.where(near, np.abs(y_exact) * 2.0 ** 15 + carried, np.abs(y_exact))
    return GatedResidual(h_exact, h, h_mag, y_exact, y_mag, nb.rstd, rn)


__all__ = ["gated_residual_rmsnorm", "GatedResidual"]
