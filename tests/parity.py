"""Comparison gates of the GPU parity tests (GPU result vs the FP64 oracle).

The tolerances are those the RMSNorm family is built to (made exact):
  h_new, gate_out     bit-exact
  rstd                |gpu - r| <= 2e-7 * r against the unrounded FP64 r
  BF16 y              within one BF16 ulp of the exactly rounded value, and equal to it
                      wherever the exact value is not within 2^-20 (relative) of a BF16
                      rounding midpoint (an FP32 evaluation cannot cross a midpoint otherwise)
  FP8 codes           equal, or one code step apart where the oracle flags a rounding tie
  block scales        bit-exact outside blocks whose amax sits at a BF16 tie
  dx                  |gpu - ref| <= 1e-2 + 1e-2*|ref| after dividing both by the RMS of ref
  dw                  |gpu - ref| <= 1e-5 * |ref| per element
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import formats as F
from tests.conftest import bits16, bits8, values


def sample_rows(n: int, k: int = 64, seed: int = 0) -> np.ndarray:
    """Sorted distinct row indices: the first two, the last two and k random ones."""
    rng = np.random.default_rng(seed)
    pick = {0, min(1, n - 1), max(n - 2, 0), n - 1}
    pick.update(rng.integers(0, n, size=min(k, n)).tolist())
    return np.array(sorted(pick), dtype=np.int64)


def rows_of(t: torch.Tensor, rows: np.ndarray) -> torch.Tensor:
    """Host copy of the given rows of a [rows, ...] tensor."""
    idx = torch.as_tensor(rows, device=t.device)
    return t.index_select(0, idx).cpu()


def assert_bf16(gpu: torch.Tensor, ref_exact: np.ndarray, what: str, mag=None):
    """BF16 output gate.  `mag`, when given, is the sum of the magnitudes of the terms of a
    value that may cancel (Ada's n*(1+scale)+shift); FP32 evaluation is then held to an
    absolute error of 2^-21*mag plus the output's own rounding."""
    g = bits16(gpu).reshape(ref_exact.shape)
    r = F.f64_to_bf16_bits(ref_exact)
    steps = F.bf16_ulp_steps(g, r)
    if mag is None:
        bad = steps > 1
        assert not bad.any(), f"{what}: {bad.sum()} elements more than 1 BF16 ulp away " \
                              f"(first at {np.argwhere(bad)[0]})"
        strict = ~F.bf16_near_tie(ref_exact)
        off = (steps != 0) & strict
        assert not off.any(), f"{what}: {off.sum()} elements differ away from a rounding tie " \
                              f"(first at {np.argwhere(off)[0]})"
    else:
        gv = F.bf16_bits_to_f64(g)
        ulp = np.abs(gv) * 2.0 ** -7 + 2.0 ** -133
        ok = (steps <= 1) | (np.abs(gv - ref_exact) <= 2.0 ** -21 * mag + ulp)
        assert ok.all(), f"{what}: {(~ok).sum()} elements outside the cancellation-aware gate"


def assert_bits_equal(gpu: torch.Tensor, ref_values: np.ndarray, what: str):
    g = bits16(gpu).reshape(ref_values.shape)
    r = F.f64_to_bf16_bits(ref_values)
    bad = g != r
    assert not bad.any(), f"{what}: {bad.sum()} elements not bit-exact " \
                          f"(first at {np.argwhere(bad)[0]})"


def assert_rstd(gpu: torch.Tensor, r64: np.ndarray, what: str = "rstd"):
    g = gpu.detach().cpu().double().numpy().reshape(r64.shape)
    rel = np.abs(g - r64) / np.abs(r64)
    assert rel.max() <= 2e-7, f"{what}: max relative error {rel.max():.3e}"


def assert_fp8(gpu: torch.Tensor, q_codes: np.ndarray, tie: np.ndarray, what: str,
               allow=None):
    """FP8 gate: equal codes, or one step apart where `tie` (or `allow`) marks the element."""
    g = bits8(gpu).reshape(q_codes.shape)
    eq = F.codes_equal_e4m3(g, q_codes)
    near = F.e4m3_code_steps(g, q_codes) <= 1
    ok_alt = tie if allow is None else (tie | allow)
    bad = ~eq & ~(ok_alt & near)
    assert not bad.any(), f"{what}: {bad.sum()} FP8 codes off (first at {np.argwhere(bad)[0]}: " \
                          f"gpu {g[tuple(np.argwhere(bad)[0])]:#04x} " \
                          f"ref {q_codes[tuple(np.argwhere(bad)[0])]:#04x})"


def assert_dx(gpu: torch.Tensor, ref_exact: np.ndarray, what: str = "dx"):
    g = values(gpu).reshape(ref_exact.shape)
    scale = np.sqrt(np.mean(ref_exact ** 2))
    scale = scale if scale > 0 else 1.0
    a, b = g / scale, ref_exact / scale
    bad = np.abs(a - b) > 1e-2 + 1e-2 * np.abs(b)
    assert not bad.any(), f"{what}: {bad.sum()} elements outside the normalised 1e-2 gate"


def assert_dw(gpu: torch.Tensor, ref_exact: np.ndarray, what: str = "dw"):
    g = gpu.detach().cpu().double().numpy()
    err = np.abs(g - ref_exact)
    bad = err > 1e-5 * np.abs(ref_exact) + 1e-30
    assert not bad.any(), f"{what}: {bad.sum()} columns beyond 1e-5 relative " \
                          f"(max rel {np.max(err / np.maximum(np.abs(ref_exact), 1e-30)):.3e})"
