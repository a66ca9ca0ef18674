"""Pins of the oracle's gated-residual RMSNorms: torch's float64 rms_norm composed by hand,
the gate = 0 and gate = 1 reductions, and broadcast gate == repeated gate rows."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import gated as G
from oracle import rmsnorm as O

RNG = np.random.default_rng(41)


def bf(shape, std=1.0, mean=0.0):
    return F.bf16_round(RNG.normal(mean, std, shape))


def torch_rms(x, w):
    return torch.nn.functional.rms_norm(torch.from_numpy(x), (x.shape[-1],),
                                        weight=torch.from_numpy(w),
                                        eps=float(np.float32(1e-6))).numpy()


def test_matches_torch_composition():
    b, r, g = bf((20, 512)), bf((20, 512)), bf((20, 512), 0.5)
    w, w2 = bf(512, 0.1, 1.0), bf(512, 0.1, 1.0)
    out = G.gated_residual_rmsnorm(b, r, g, w, 1e-6, next_w=w2)
    h = r + g * torch_rms(b, w)
    np.testing.assert_allclose(out.h_exact, h, rtol=1e-13, atol=1e-13)
    assert (out.h == F.bf16_round(out.h_exact)).all()
    np.testing.assert_allclose(out.y_exact, torch_rms(out.h, w2), rtol=1e-12, atol=1e-13)


def test_gate_zero_and_one():
    b, r = bf((9, 256)), bf((9, 256))
    w, w2 = bf(256, 0.1, 1.0), bf(256, 0.1, 1.0)
    z = G.gated_residual_rmsnorm(b, r, np.zeros((9, 256)), w, 1e-6, next_w=w2)
    assert (z.h == r).all()
    assert (z.y_exact == O.rmsnorm(r, w2, 0.0, 1e-6).y_exact).all()
    one = G.gated_residual_rmsnorm(b, r, np.ones(256), w, 1e-6)
    np.testing.assert_allclose(one.h_exact, r + O.rmsnorm(b, w, 0.0, 1e-6).y_exact, rtol=0,
                               atol=0)


def test_broadcast_gate_equals_repeated_rows():
    b, r = bf((7, 128)), bf((7, 128))
    w = bf(128, 0.1, 1.0)
    g1 = bf((1, 128))
    a = G.gated_residual_rmsnorm(b, r, g1, w, 1e-6)
    c = G.gated_residual_rmsnorm(b, r, np.repeat(g1, 7, axis=0), w, 1e-6)
    assert (a.h_exact == c.h_exact).all()


def test_next_norm_band_marks_only_elements_at_rounding_ties():
    b, r, g = bf((50, 1024)), bf((50, 1024)), bf((50, 1024), 0.5)
    w = bf(1024, 0.1, 1.0)
    out = G.gated_residual_rmsnorm(b, r, g, w, 1e-6, next_w=w)
    wide = out.y_mag > np.abs(out.y_exact)
    # flagged elements are rare and each sits next to a BF16 rounding midpoint of h
    assert wide.mean() < 1e-2
    hb = F.bf16_round(out.h_exact)
    mid_dist = np.abs(hb - out.h_exact)
    _, e = np.frexp(np.abs(out.h_exact))
    ulp = np.ldexp(1.0, e - 8)                 # BF16 spacing in |h|'s binade
    assert (np.abs(mid_dist - ulp / 2)[wide] <= 2.0 ** -19 * out.h_mag[wide] + 1e-30).all()


def _bf16_tensor(v):
    return torch.from_numpy(F.f64_to_bf16_bits(v).view(np.int16)).view(torch.bfloat16)


def _fp32_gated_next(b, r, g, w, w2, eps):
    """An FP32 evaluation of the gated residual + next norm, in the order a kernel takes:
    rstd of the branch rounded to FP32, n = FP32(FP32(b * rstd) * w), h = BF16(FMA(g, n, r))
    (the FMA's product is exact in FP64, its sum rounded to FP64 and then to FP32), the next
    rstd from the BF16 h, y = BF16(FP32(FP32(h * rstd2) * w2))."""
    f32 = np.float32
    e = float(f32(eps))
    rs = (1.0 / np.sqrt(np.mean(b * b, axis=1) + e)).astype(f32)
    n = ((b.astype(f32) * rs[:, None]).astype(f32) * w.astype(f32)).astype(f32)
    h = F.bf16_round((g * n.astype(np.float64) + r).astype(f32).astype(np.float64))
    r2 = (1.0 / np.sqrt(np.mean(h * h, axis=1) + e)).astype(f32)
    y = ((h.astype(f32) * r2[:, None]).astype(f32) * w2.astype(f32)).astype(f32)
    return h, F.bf16_round(y.astype(np.float64))


def test_next_norm_gate_admits_an_fp32_evaluation_where_h_cancels():
    """Residuals set to -BF16(gate * n) make h = residual + gate * n cancel far below its
    terms on many elements.  There an FP32 evaluation of h is off by many of h's ulps (within
    h's own gate), and the next norm carries that into y.  The oracle's y band must admit
    such an evaluation, which the band of a one-ulp neighbour alone does not; it must still
    reject y moved by eight times the carried band."""
    from tests.parity import assert_bf16
    b, r, g = bf((64, 1024)), bf((64, 1024)), bf((64, 1024), 0.5)
    w, w2 = bf(1024, 0.1, 1.0), bf(1024, 0.1, 1.0)
    n = O.rmsnorm(b, w, 0.0, 1e-6).y_exact
    r[:, :512] = F.bf16_round(-g[:, :512] * n[:, :512])
    out = G.gated_residual_rmsnorm(b, r, g, w, 1e-6, next_w=w2)
    cancel = np.abs(out.h_exact) < 2.0 ** -14 * out.h_mag
    assert cancel.sum() >= 100
    h, y = _fp32_gated_next(b, r, g, w, w2, 1e-6)
    assert (h != out.h)[cancel].sum() >= 50           # h itself moved there
    assert_bf16(_bf16_tensor(h), out.h_exact, "FP32 h", mag=out.h_mag)
    assert_bf16(_bf16_tensor(y), out.y_exact, "FP32 next-norm y", mag=out.y_mag)
    band = 2.0 ** -20 * out.h_mag
    near = F.bf16_round(out.h_exact - band) != F.bf16_round(out.h_exact + band)
    one_ulp_only = np.abs(out.y_exact) * np.where(near, 2.0 ** 15, 1.0)
    with pytest.raises(AssertionError):
        assert_bf16(_bf16_tensor(y), out.y_exact, "one-ulp band", mag=one_ulp_only)
    r2 = O.rmsnorm(out.h, w2, 0.0, 1e-6).r64
    carried = 2.0 ** -20 * out.h_mag * r2[:, None] * np.abs(w2)
    moved = np.where(cancel, y + 8.0 * carried, y)
    with pytest.raises(AssertionError):
        assert_bf16(_bf16_tensor(moved), out.y_exact, "moved y", mag=out.y_mag)
