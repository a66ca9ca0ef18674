"""Plain FP64 reference of the LayerNorm family (slow, obviously correct).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  It shares no code with the GPU library.

Page abbreviations as in ``oracle.rmsnorm``.  Definitions followed:
  * layernorm / layernorm_quant -- norm docs, API table; norm guide §4: BF16 input, FP32
    gamma and beta of shape (hidden,), output in the input's dtype;
    quant: out = (((x - E[x]) / sqrt(Var[x] + eps)) * gamma + beta) / scale, to FP8.
  * the DiT trio -- norm docs, API table; norm guide §5.3:
      gate_residual + gamma/beta:  residual_out = residual + x * (gate + gate_bias);
                                   norm_out = LayerNorm(residual_out, gamma, beta)
      gate_residual + scale/shift: norm_out = LayerNorm(residual_out)
                                              * (1 + scale + scale_bias) + (shift + shift_bias)
      residual + scale/shift:      residual_out = residual + x (or x alone without a
                                   residual), then the scale/shift form.
    gate, scale and shift are per-row BF16 tensors (rows of the temb.chunk(6) views).
Readings where the pages are silent: the variance is the population variance over the
row; the scale/shift forms normalise without gamma/beta; the biases are FP32 scalars; the
gated sum is one FP32 rounding of x * FP32(gate + gate_bias) + residual (an FMA), stored as
BF16, and the norm is taken over that BF16 residual_out.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .formats import bf16_round, f32_round, f32_round_exact_sum
from .rmsnorm import Quant, quantize_static


def _2d(a) -> np.ndarray:
    a = np.asarray(a, dtype=np.float64)
    return a.reshape(1, -1) if a.ndim == 1 else a


@dataclass
class LayerNorm:
    n_exact: np.ndarray     # (h - mean) / sqrt(var + eps)
    y_exact: np.ndarray     # n * gamma + beta
    y: np.ndarray           # BF16(y_exact)
    mag: np.ndarray         # |h - mean| magnitude scale of the evaluation: (|h| + |mean|) * rstd * |gamma| + |beta|
    mean: np.ndarray
    rstd: np.ndarray        # 1 / sqrt(var + eps), FP64


def layernorm(h, gamma=None, beta=None, eps: float = 1e-6) -> LayerNorm:
    """y = (h - E[h]) / sqrt(Var[h] + eps) * gamma + beta over each row (norm guide §4).

    E and Var are the mean and the population variance of the row, in FP64 (two passes);
    eps is an FP32 number; gamma and beta default to 1 and 0.
    """
    h = _2d(h)
    hidden = h.shape[1]
    g = np.ones(hidden) if gamma is None else np.asarray(gamma, dtype=np.float64)
    b = np.zeros(hidden) if beta is None else np.asarray(beta, dtype=np.float64)
    eps32 = float(np.float32(eps))
    mean = np.sum(h, axis=1) / hidden
    d = h - mean[:, None]
    var = np.sum(d * d, axis=1) / hidden
    rstd = 1.0 / np.sqrt(var + eps32)
    n = d * rstd[:, None]
    y = n * g[None, :] + b[None, :]
    mag = (np.abs(h) + np.abs(mean)[:, None]) * rstd[:, None] * np.abs(g)[None, :] + np.abs(b)
    return LayerNorm(n, y, bf16_round(y), mag, mean, rstd)


def layernorm_quant(h, gamma, beta, scale: float, eps: float = 1e-6):
    """out = e4m3fn(LayerNorm(h, gamma, beta) / scale) (norm guide §4)."""
    ln = layernorm(h, gamma, beta, eps)
    return ln, quantize_static(ln.y_exact, scale, ln.mag)


def dit_gate_residual(residual, x, gate, gate_bias: float = 0.0) -> np.ndarray:
    """residual_out = BF16(residual + x * FP32(gate + gate_bias)), one FP32 rounding of the
    sum (norm guide §5.3).  x * g of a BF16 and an FP32 number is exact in FP64."""
    g = f32_round(_2d(gate) + float(np.float32(gate_bias)))
    return bf16_round(f32_round_exact_sum(_2d(x) * g, _2d(residual)))


@dataclass
class DitNorm:
    residual_out: np.ndarray
    o_exact: np.ndarray
    o: np.ndarray
    mag: np.ndarray


def _modulate(ln: LayerNorm, scale, shift, scale_bias: float, shift_bias: float):
    sb = float(np.float32(scale_bias))
    shb = float(np.float32(shift_bias))
    m = 1.0 + _2d(scale) + sb
    s = _2d(shift) + shb
    o = ln.n_exact * m + s
    mag = (ln.mag * np.abs(m) + np.abs(s)) + np.abs(ln.n_exact) * (1.0 + np.abs(_2d(scale)) + abs(sb))
    return o, mag


def dit_gate_residual_layernorm_gamma_beta(residual, x, gate, gamma, beta, gate_bias=0.0,
                                           eps: float = 1e-6) -> DitNorm:
    """fused_dit_gate_residual_layernorm_gamma_beta (norm docs, API table; norm guide §5.3)."""
    h = dit_gate_residual(residual, x, gate, gate_bias)
    ln = layernorm(h, gamma, beta, eps)
    return DitNorm(h, ln.y_exact, ln.y, ln.mag)


def dit_gate_residual_layernorm_scale_shift(residual, x, gate, scale, shift, gate_bias=0.0,
                                            scale_bias=0.0, shift_bias=0.0,
                                            eps: float = 1e-6) -> DitNorm:
    """fused_dit_gate_residual_layernorm_scale_shift (norm docs, API table; norm guide §5.3)."""
    h = dit_gate_residual(residual, x, gate, gate_bias)
    ln = layernorm(h, None, None, eps)
    o, mag = _modulate(ln, scale, shift, scale_bias, shift_bias)
    return DitNorm(h, o, bf16_round(o), mag)


def dit_residual_layernorm_scale_shift(x, scale, shift, residual=None, scale_bias=0.0,
                                       shift_bias=0.0, eps: float = 1e-6) -> DitNorm:
    """fused_dit_residual_layernorm_scale_shift: residual_out = BF16(residual + x) (x alone
    without a residual), then LayerNorm and the scale/shift modulation (norm guide §5.3)."""
    h = _2d(x) if residual is None else bf16_round(_2d(x) + _2d(residual))
    ln = layernorm(h, None, None, eps)
    o, mag = _modulate(ln, scale, shift, scale_bias, shift_bias)
    return DitNorm(h, o, bf16_round(o), mag)


__all__ = ["layernorm", "layernorm_quant", "dit_gate_residual",
           "dit_gate_residual_layernorm_gamma_beta", "dit_gate_residual_layernorm_scale_shift",
           "dit_residual_layernorm_scale_shift", "LayerNorm", "DitNorm", "Quant"]
