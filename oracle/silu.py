"""Plain FP64 reference of the fused RMSNorm + SiLU (slow, obviously correct).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  It shares no code with the GPU library.

norm guide §5.1 and the norm docs API table (fused_rmsnorm_silu): y = SiLU(RMSNorm(input,
weight, eps)) with SiLU(x) = x / (1 + exp(-x)); BF16 input; the output dtype is the out
tensor's: BF16 or float8_e4m3fn [tokens, hidden] (NVFP4 is out of scope).
Readings where the pages are silent: the RMSNorm is the one of oracle.rmsnorm (FP32 weight
effective value w + bias, the unrounded normalised value feeds the SiLU); the FP8 output
is e4m3fn(SiLU(y) / scale) with a static FP32 scale (1 when none is given), like the
other static FP8 outputs.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .formats import bf16_round
from .rmsnorm import Quant, quantize_static, rmsnorm


def silu(y) -> np.ndarray:
    """x / (1 + exp(-x)) in FP64 (exp overflow for very negative x gives the limit 0)."""
    y = np.asarray(y, dtype=np.float64)
    with np.errstate(over="ignore"):
        return y / (1.0 + np.exp(-y))


@dataclass
class RMSNormSilu:
    s_exact: np.ndarray      # SiLU of the unrounded normalised value
    s: np.ndarray            # BF16(s_exact)
    mag: np.ndarray          # |s| * (2 + |y|): SiLU amplifies y's relative error by up to 1 + |y|
    y_exact: np.ndarray
    rstd: np.ndarray


def fused_rmsnorm_silu(x, w, eps: float = 1e-6, bias: float = 0.0) -> RMSNormSilu:
    """SiLU(RMSNorm(x, w, eps)) (norm guide §5.1)."""
    n = rmsnorm(x, w, bias, eps)
    s = silu(n.y_exact)
    mag = np.abs(s) * (2.0 + np.abs(n.y_exact))
    return RMSNormSilu(s, bf16_round(s), mag, n.y_exact, n.rstd)


def fused_rmsnorm_silu_fp8(x, w, scale: float, eps: float = 1e-6, bias: float = 0.0):
    """e4m3fn(SiLU(RMSNorm(x)) / scale)."""
    r = fused_rmsnorm_silu(x, w, eps, bias)
    return r, quantize_static(r.s_exact, scale, r.mag)


__all__ = ["silu", "fused_rmsnorm_silu", "fused_rmsnorm_silu_fp8", "RMSNormSilu", "Quant"]


def sigmoid(g) -> np.ndarray:
    """1 / (1 + exp(-g)) in FP64."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-g))


@dataclass
class SigmoidGate:
    o_exact: np.ndarray      # RMSNorm(x) * w * sigmoid(gate)
    o: np.ndarray            # BF16, written over x
    mag: np.ndarray          # |o| * (2 + |gate|): the gate's exponential carries |g| ulps
    rstd: np.ndarray


def rmsnorm_sigmoid_gate(x, gate, w=None, eps: float = 1e-6, bias: float = 0.0) -> SigmoidGate:
    """Per-head RMSNorm and sigmoid gate (norm docs, Fixed-Width Fused Norms:
    rmsnorm_sigmoid_gate).  Reading: rows are heads ([tokens*heads, head_dim]); the head
    is normalised as rmsnorm (weight [head_dim], ones when absent) and multiplied element by
    element by sigmoid(gate) of the same shape; the result replaces x."""
    x = np.asarray(x, dtype=np.float64)
    hd = x.shape[-1]
    ww = np.ones(hd) if w is None else np.asarray(w, dtype=np.float64)
    n = rmsnorm(x.reshape(-1, hd), ww, bias, eps)
    g = np.asarray(gate, dtype=np.float64).reshape(-1, hd)
    o = n.y_exact * sigmoid(g)
    return SigmoidGate(o, bf16_round(o), np.abs(o) * (2.0 + np.abs(g)), n.rstd)


__all__ += ["sigmoid", "rmsnorm_sigmoid_gate", "SigmoidGate"]
