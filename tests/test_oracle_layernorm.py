"""Pins of the oracle's LayerNorm family against things other than the oracle itself: torch
CPU float64 layer_norm (library routine), closed forms, exact scale invariance, exact
rational arithmetic, and reductions to already pinned operations."""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import layernorm as L
from oracle import rmsnorm as O

RNG = np.random.default_rng(11)


def bf16_values(shape, std=1.0, mean=0.0):
    return F.bf16_round(RNG.normal(mean, std, shape))


def torch_layer_norm64(h, gamma, beta, eps):
    eps32 = float(np.float32(eps))
    t = torch.from_numpy(np.ascontiguousarray(h))
    g = None if gamma is None else torch.from_numpy(np.asarray(gamma, dtype=np.float64))
    b = None if beta is None else torch.from_numpy(np.asarray(beta, dtype=np.float64))
    return torch.nn.functional.layer_norm(t, (h.shape[-1],), weight=g, bias=b, eps=eps32).numpy()


@pytest.mark.parametrize("hidden", [8, 128, 3072, 4096])
def test_layernorm_matches_torch(hidden):
    h = bf16_values((25, hidden), std=2.0, mean=0.5)
    g = RNG.normal(1.0, 0.2, hidden).astype(np.float32).astype(np.float64)
    b = RNG.normal(0.0, 0.2, hidden).astype(np.float32).astype(np.float64)
    ln = L.layernorm(h, g, b, 1e-6)
    np.testing.assert_allclose(ln.y_exact, torch_layer_norm64(h, g, b, 1e-6), rtol=1e-12,
                               atol=1e-12)
    np.testing.assert_allclose(ln.n_exact, torch_layer_norm64(h, None, None, 1e-6), rtol=1e-12,
                               atol=1e-12)
    assert (ln.y == F.bf16_round(ln.y_exact)).all()


def test_layernorm_worked_example():
    # Row [1, 2, 3, 4], eps = 0: mean 2.5, population variance 1.25.
    ln = L.layernorm(np.array([[1.0, 2.0, 3.0, 4.0]]), None, None, 0.0)
    want = np.array([-1.5, -0.5, 0.5, 1.5]) / np.sqrt(1.25)
    np.testing.assert_allclose(ln.n_exact[0], want, rtol=1e-15)
    assert ln.mean[0] == 2.5


def test_constant_row_gives_beta():
    b = RNG.normal(0, 1, 64)
    ln = L.layernorm(np.full((2, 64), 3.0), RNG.normal(1, 0.1, 64), b, 1e-6)
    assert (ln.y_exact == b).all()


@pytest.mark.parametrize("k", [-9, 5])
def test_power_of_two_scale_invariance(k):
    h = bf16_values((8, 512), std=3.0, mean=1.0)
    a = L.layernorm(h, None, None, 0.0)
    b = L.layernorm(h * 2.0 ** k, None, None, 0.0)
    assert (a.n_exact == b.n_exact).all()
    assert (b.rstd == a.rstd * 2.0 ** -k).all()


def test_layernorm_quant_known_codes_and_torch_cast():
    # Constant rows: y = beta exactly; scale 1 -> e4m3(beta).
    beta = np.array([1.0625, 432.0, -500.0, 0.5, 3 * 2.0 ** -10, 1.0, 448.0, 2.0 ** -9])
    ln, q = L.layernorm_quant(np.full((2, 8), -7.0), np.ones(8), beta, 1.0, 1e-6)
    assert list(q.q[0]) == [0x38, 0x7E, 0xFE, 0x30, 0x02, 0x38, 0x7E, 0x01]
    h = bf16_values((16, 1024))
    ln, q = L.layernorm_quant(h, np.ones(1024), np.zeros(1024), 0.04, 1e-6)
    v = (ln.y_exact / float(np.float32(0.04))).astype(np.float32)
    ok = np.abs(v) < 448
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    agree = F.codes_equal_e4m3(q.q, ref)
    assert (agree | q.tie | ~ok).all()


def test_gated_residual_is_one_rounding_of_the_exact_sum():
    r = bf16_values(400, std=3.0)
    x = bf16_values(400)
    g = bf16_values(400)
    got = L.dit_gate_residual(r, x, g, 0.375)[0]
    for i in range(400):
        gp = Fraction(float(np.float32(float(g[i]) + 0.375)))    # FP32(gate + gate_bias)
        exact = Fraction(float(r[i])) + Fraction(float(x[i])) * gp
        f = np.float32(float(exact))
        cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
        best = min(cands, key=lambda c: (abs(Fraction(float(c)) - exact),
                                         int(np.array(c, np.float32).view(np.uint32)) & 1))
        assert got[i] == F.bf16_round(np.array([float(best)]))[0]


def test_gated_residual_with_unit_gate_is_the_fused_add():
    r, x = bf16_values((10, 256)), bf16_values((10, 256))
    a = L.dit_gate_residual(r, x, np.zeros((10, 256)), 1.0)
    assert (a == O.residual_add(x, r)).all()


def test_dit_scale_shift_matches_torch():
    rows, hidden = 12, 768
    r, x, g = bf16_values((rows, hidden)), bf16_values((rows, hidden)), bf16_values((rows, hidden))
    sc, sh = bf16_values((rows, hidden), std=0.3), bf16_values((rows, hidden), std=0.3)
    d = L.dit_gate_residual_layernorm_scale_shift(r, x, g, sc, sh, 0.5, 0.25, -0.125, 1e-6)
    n = torch_layer_norm64(d.residual_out, None, None, 1e-6)
    ref = n * (1.0 + sc + 0.25) + (sh - 0.125)
    np.testing.assert_allclose(d.o_exact, ref, rtol=1e-12, atol=1e-12)
    d2 = L.dit_residual_layernorm_scale_shift(x, sc, sh, r, 0.25, -0.125, 1e-6)
    n2 = torch_layer_norm64(O.residual_add(x, r), None, None, 1e-6)
    np.testing.assert_allclose(d2.o_exact, n2 * (1.0 + sc + 0.25) + (sh - 0.125), rtol=1e-12,
                               atol=1e-12)
    d3 = L.dit_residual_layernorm_scale_shift(x, sc, sh, None)
    np.testing.assert_allclose(d3.o_exact, torch_layer_norm64(x, None, None, 1e-6) * (1 + sc) + sh,
                               rtol=1e-12, atol=1e-12)


def test_dit_gamma_beta_matches_torch_and_reduces_to_layernorm():
    rows, hidden = 9, 512
    r, x, g = bf16_values((rows, hidden)), bf16_values((rows, hidden)), bf16_values((rows, hidden))
    gam = RNG.normal(1, 0.1, hidden).astype(np.float32).astype(np.float64)
    bet = RNG.normal(0, 0.1, hidden).astype(np.float32).astype(np.float64)
    d = L.dit_gate_residual_layernorm_gamma_beta(r, x, g, gam, bet, 0.0, 1e-6)
    np.testing.assert_allclose(d.o_exact, torch_layer_norm64(d.residual_out, gam, bet, 1e-6),
                               rtol=1e-12, atol=1e-12)
    zero = np.zeros((rows, hidden))
    s = L.dit_gate_residual_layernorm_scale_shift(r, x, g, zero, zero, 0.0, 0.0, 0.0, 1e-6)
    plain = L.layernorm(s.residual_out, None, None, 1e-6)
    assert (s.o_exact == plain.y_exact).all()



def _fp32_layernorm_quant(h, gamma, beta, scale, eps, compensated=True):
    """An FP32 evaluation of layernorm_quant in the kernel's order: FP64 statistics; mu =
    FP32(mean) and rstd rounded once to FP32; n = FMA(FP32(h - mu), rstd, lo) with lo =
    FP32(-(mean - mu) * rstd) (uncompensated: lo = 0); gamma and beta multiplied by FP32(1/scale);
    y = FMA(n, gamma', beta') (its product exact in FP64, the sum rounded to FP64 and then to
    FP32); then the e4m3 conversion."""
    f32 = np.float32
    hidden = h.shape[1]
    mean = h.sum(axis=1) / hidden
    var = np.maximum((h * h).sum(axis=1) / hidden - mean * mean, 0.0)
    rs = (1.0 / np.sqrt(var + float(f32(eps)))).astype(f32)
    mu = mean.astype(f32)
    lo = (-(mean - mu.astype(np.float64)) * rs).astype(f32) if compensated else np.zeros_like(mu)
    d = (h.astype(f32) - mu[:, None]).astype(f32)
    n = (d.astype(np.float64) * rs[:, None].astype(np.float64) + lo[:, None]).astype(f32)
    inv = f32(1.0) / f32(scale)
    g = (gamma.astype(f32) * inv).astype(f32)
    b = (beta.astype(f32) * inv).astype(f32)
    y = (n.astype(np.float64) * g.astype(np.float64) + b.astype(np.float64)).astype(f32)
    return F.f64_to_e4m3_code(y.astype(np.float64))


def test_quant_gate_sees_the_mean_rounding_where_the_output_cancels():
    """Rows of width 1000 sitting 1000 of their spreads away from zero, and a beta that
    cancels row 0's n*gamma on 256 columns, quantised at a scale of 1e-3: those outputs lie
    next to zero, in e4m3's subnormals.  The kernel's evaluation, which carries the mean as
    an FP32 pair, passes the one-step gate; the same evaluation with the mean rounded once to
    FP32 (whose error there is 2^-25 of the mean) moves them by several subnormal steps and
    fails it."""
    from tests.parity import assert_fp8
    h = bf16_values((16, 1000), 1.0, 1000.0)     # a width whose mean FP32 cannot hold exactly
    gamma = 1.0 + RNG.normal(0, 0.1, 1000)
    ln0 = L.layernorm(h, gamma, np.zeros(1000), 1e-6)
    beta = RNG.normal(0, 0.1, 1000)
    beta[:256] = -ln0.y_exact[0, :256]
    gamma = gamma.astype(np.float32).astype(np.float64)
    beta = beta.astype(np.float32).astype(np.float64)
    _, q = L.layernorm_quant(h, gamma, beta, 1e-3, 1e-6)
    as_t = lambda c: torch.from_numpy(np.ascontiguousarray(c, dtype=np.uint8))
    codes = _fp32_layernorm_quant(h, gamma, beta, 1e-3, 1e-6)
    assert_fp8(as_t(codes), q.q, q.tie, "FP32 evaluation, mean as an FP32 pair")
    plain = _fp32_layernorm_quant(h, gamma, beta, 1e-3, 1e-6, compensated=False)
    assert (F.e4m3_code_steps(plain, q.q)[0, :256] >= 2).sum() >= 10
    with pytest.raises(AssertionError):
        assert_fp8(as_t(plain), q.q, q.tie, "FP32 evaluation, mean rounded once")
