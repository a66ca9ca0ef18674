"""Pins of the oracle's gated-residual RMSNorms: torch's float64 rms_norm composed by hand,
the gate = 0 and gate = 1 reductions, and broadcast gate == repeated gate rows."""
from __future__ import annotations

import numpy as np
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
