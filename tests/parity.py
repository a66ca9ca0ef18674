"""Comparison gates of the GPU parity tests (GPU result vs the FP64 oracle).

The tolerances are those the RMSNorm family is built to (made exact):
  h_new, gate_out     bit-exact
  rstd                |gpu - r| <= 2e-7 * r against the unrounded FP64 r
  BF16 y              within one BF16 ulp of the exactly rounded value, and equal to it
                      wherever the exact value is not within 2^-20 (relative) of a BF16
                      rounding midpoint (an FP32 evaluation cannot cross a midpoint otherwise)
  FP8 codes           equal, or one code step apart where the oracle flags a rounding tie
  block scales        bit-exact, or the oracle's other candidate in a block whose amax has
                      two possible values (an element next to a BF16 midpoint); the codes
                      then follow the scale the GPU took (block_quant_ok)
  dx                  |gpu - ref| <= 1e-2 + 1e-2*|ref| after dividing both by the RMS of ref,
                      and per element within one BF16 rounding of an FP32 evaluation
                      (assert_dx)
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
    # one step along the code line, never onto or off a NaN code (0x7E and 0x7F are
    # neighbours as codes)
    near = (F.e4m3_code_steps(g, q_codes) <= 1) & ((g & 0x7F) != 0x7F) & \
        ((np.asarray(q_codes) & 0x7F) != 0x7F)
    ok_alt = tie if allow is None else (tie | allow)
    bad = ~eq & ~(ok_alt & near)
    assert not bad.any(), f"{what}: {bad.sum()} FP8 codes off (first at {np.argwhere(bad)[0]}: " \
                          f"gpu {g[tuple(np.argwhere(bad)[0])]:#04x} " \
                          f"ref {q_codes[tuple(np.argwhere(bad)[0])]:#04x})"


def assert_dx(gpu: torch.Tensor, ref, what: str = "dx"):
    """dx gates.  `ref` is the oracle's TrainBackward (or a bare exact dx array, the first
    gate only).

    1. The pages' unit-scaled tolerance: both divided by the RMS of the exact dx,
       |gpu - ref| <= 1e-2 + 1e-2*|ref|.
    2. Per element, cancellation-aware: one BF16 rounding of an FP32 evaluation,
       |gpu - ref| <= 2^-8*|ref| + 2^-20*M1 + 2^-17*M2 + 2^-133, with M1 = |r*g*w_eff| +
       |g_residual| the direct terms and M2 = |x|*r^3*mean_j|g*w_eff*x| the bound of the
       coupled term.  An FP32 evaluation of the row dot product over at most 32 terms per
       lane is within ~2^-19*sum|g*w*x|, the rest of the chain within a few 2^-24 of M1;
       the bound doubles both, leaving room for an rstd that differs from the oracle's by an
       FP32 ulp (the autograd route saves the kernel's own).  A wrong coefficient of the
       coupled term fails it wherever that term is not negligible."""
    exact = ref.dx_exact if hasattr(ref, "dx_exact") else np.asarray(ref)
    g = values(gpu).reshape(exact.shape)
    scale = np.sqrt(np.mean(exact ** 2))
    scale = scale if scale > 0 else 1.0
    a, b = g / scale, exact / scale
    bad = np.abs(a - b) > 1e-2 + 1e-2 * np.abs(b)
    assert not bad.any(), f"{what}: {bad.sum()} elements outside the normalised 1e-2 gate"
    if hasattr(ref, "dx_mag_direct"):
        lim = 2.0 ** -8 * np.abs(exact) + 2.0 ** -20 * ref.dx_mag_direct + \
            2.0 ** -17 * ref.dx_mag_coupled + 2.0 ** -133
        bad = np.abs(g - exact) > lim
        assert not bad.any(), f"{what}: {bad.sum()} elements outside the per-element gate " \
                              f"(first at {np.argwhere(bad)[0]})"


def assert_dw(gpu: torch.Tensor, ref_exact: np.ndarray, what: str = "dw"):
    g = gpu.detach().cpu().double().numpy()
    err = np.abs(g - ref_exact)
    bad = err > 1e-5 * np.abs(ref_exact) + 1e-30
    assert not bad.any(), f"{what}: {bad.sum()} columns beyond 1e-5 relative " \
                          f"(max rel {np.max(err / np.maximum(np.abs(ref_exact), 1e-30)):.3e})"


def block_quant_ok(gpu_scale: np.ndarray, gpu_codes: np.ndarray, ref):
    """Gate of the 1x128 block quantiser (ref: oracle.rmsnorm.BlockQuant), as masks.

    gpu_scale: float64 [rows, hidden/128] logical scales; gpu_codes: uint8 [rows, hidden].
    A block's scale must be the oracle's, or, in a block whose amax has two possible values
    (ref.block_flag), its other candidate (ref.scale_alt).  Each code is then checked
    against the oracle's codes under the scale the GPU took: the code of the normalised
    value, or of its other BF16 neighbour where that value lies next to a BF16 midpoint,
    or one code step from either where it lies next to an e4m3 midpoint.  Returns
    (scale_ok [rows, nb], codes_ok [rows, hidden])."""
    rows, hidden = ref.q.shape
    nominal = gpu_scale == ref.scale
    alt = ref.block_flag & (gpu_scale == ref.scale_alt) & ~nominal
    scale_ok = nominal | alt
    use_alt = np.repeat(alt, 128, axis=1)
    pick = lambda a, b: np.where(use_alt, b, a)
    q, tie = pick(ref.q, ref.q_alt), pick(ref.fp8_tie, ref.fp8_tie_alt)
    q_nb, nb_tie = pick(ref.q_nb, ref.q_nb_alt), pick(ref.nb_tie, ref.nb_tie_alt)
    g = np.asarray(gpu_codes, dtype=np.uint8).reshape(rows, hidden)

    def matches(want, near_tie):
        # one step along the code line, never onto or off a NaN code
        step = (F.e4m3_code_steps(g, want) <= 1) & ((g & 0x7F) != 0x7F) & \
            ((want & 0x7F) != 0x7F)
        return F.codes_equal_e4m3(g, want) | (near_tie & step)

    codes_ok = matches(q, tie) | (ref.bf_tie & matches(q_nb, nb_tie))
    return scale_ok, codes_ok


def assert_block_quant(gpu_codes: torch.Tensor, gpu_scale_t, ref, what: str):
    """block_quant_ok as an assertion; gpu_scale_t: logical [rows, hidden/128] scales."""
    s = gpu_scale_t.detach().cpu().double().numpy() if isinstance(gpu_scale_t, torch.Tensor) \
        else np.asarray(gpu_scale_t, dtype=np.float64)
    scale_ok, codes_ok = block_quant_ok(s, bits8(gpu_codes).reshape(ref.q.shape), ref)
    assert scale_ok.all(), f"{what}: {(~scale_ok).sum()} block scales differ " \
                           f"(first {np.argwhere(~scale_ok)[0]}: " \
                           f"{s[tuple(np.argwhere(~scale_ok)[0])]!r} vs " \
                           f"{ref.scale[tuple(np.argwhere(~scale_ok)[0])]!r})"
    assert codes_ok.all(), f"{what}: {(~codes_ok).sum()} FP8 codes off " \
                           f"(first at {np.argwhere(~codes_ok)[0]})"


def assert_bf16_nonfinite(gpu, ref_exact, what, mag=None):
    """NaN and infinities exactly where the oracle's IEEE evaluation has them; every finite
    element through assert_bf16."""
    g = values(gpu).reshape(ref_exact.shape)
    r = ref_exact
    assert (np.isnan(g) == np.isnan(r)).all(), f"{what}: NaN positions differ"
    inf = np.isinf(r)
    assert (g[inf] == r[inf]).all() and (np.isinf(g) == inf).all(), f"{what}: infinities differ"
    fin = np.isfinite(r)
    assert_bf16(gpu.reshape(-1)[torch.as_tensor(np.flatnonzero(fin), device=gpu.device)],
                r[fin], what, mag=None if mag is None else mag[fin])


def assert_fp8_nonfinite(q, ref, what):
    """NaN codes exactly where the oracle's value is NaN; every other code equal (or a
    neighbour at a flagged tie), infinities saturating to +-448."""
    g = bits8(q).reshape(ref.q.shape)
    nan_ref = np.isnan(ref.v)
    assert (((g & 0x7F) == 0x7F) == nan_ref).all(), f"{what}: e4m3 NaN codes"
    ok = F.codes_equal_e4m3(g, ref.q) | ref.tie
    assert ok[~nan_ref].all(), f"{what}: e4m3 codes"
