"""Pins of the oracle's fused RMSNorm + SiLU: torch's float64 silu and rms_norm (library
routines), the closed forms silu(0) = 0 and silu(y) - silu(-y) = y, the limits, and
torch's FP8 cast."""
from __future__ import annotations

import numpy as np
import torch

from oracle import formats as F
from oracle import silu as S

RNG = np.random.default_rng(31)


def test_silu_matches_torch_and_closed_forms():
    y = np.concatenate([RNG.normal(0, 4, 5000), [0.0, -0.0, 1e-300, -50.0, 80.0]])
    np.testing.assert_allclose(S.silu(y), torch.nn.functional.silu(torch.from_numpy(y)).numpy(),
                               rtol=1e-14, atol=1e-300)
    assert S.silu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(S.silu(y) - S.silu(-y), y, rtol=1e-13, atol=1e-13)
    assert S.silu(np.array([-800.0]))[0] == 0.0           # exp overflow: the limit
    assert S.silu(np.array([800.0]))[0] == 800.0


def test_fused_rmsnorm_silu_matches_torch():
    x = F.bf16_round(RNG.normal(0, 1, (33, 640)))
    w = F.bf16_round(RNG.normal(1, 0.1, 640))
    r = S.fused_rmsnorm_silu(x, w, 1e-6)
    n = torch.nn.functional.rms_norm(torch.from_numpy(x), (640,), weight=torch.from_numpy(w),
                                     eps=float(np.float32(1e-6)))
    np.testing.assert_allclose(r.s_exact, torch.nn.functional.silu(n).numpy(), rtol=1e-12,
                               atol=1e-14)
    assert (r.s == F.bf16_round(r.s_exact)).all()


def test_fp8_matches_torch_cast():
    x = F.bf16_round(RNG.normal(0, 1, (16, 256)))
    w = F.bf16_round(RNG.normal(1, 0.1, 256))
    r, q = S.fused_rmsnorm_silu_fp8(x, w, 0.02)
    v = (r.s_exact / float(np.float32(0.02))).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ok = np.abs(v) < 448
    assert (F.codes_equal_e4m3(q.q, ref) | q.tie | ~ok).all()


def test_sigmoid_gate_matches_torch_and_identities():
    x = F.bf16_round(RNG.normal(0, 1, (40, 64)))
    g = F.bf16_round(RNG.normal(0, 3, (40, 64)))
    w = F.bf16_round(RNG.normal(1, 0.1, 64))
    r = S.rmsnorm_sigmoid_gate(x, g, w, 1e-6)
    n = torch.nn.functional.rms_norm(torch.from_numpy(x), (64,), weight=torch.from_numpy(w),
                                     eps=float(np.float32(1e-6)))
    ref = (n * torch.sigmoid(torch.from_numpy(g))).numpy()
    np.testing.assert_allclose(r.o_exact, ref, rtol=1e-12, atol=1e-14)
    # gate 0 halves the norm exactly; gates g and -g add up to the norm
    half = S.rmsnorm_sigmoid_gate(x, np.zeros_like(g), w, 1e-6)
    np.testing.assert_array_equal(half.o_exact, n.numpy() * 0.5)
    neg = S.rmsnorm_sigmoid_gate(x, -g, w, 1e-6)
    np.testing.assert_allclose(r.o_exact + neg.o_exact, n.numpy(), rtol=1e-13, atol=1e-13)
    # no weight = ones
    none = S.rmsnorm_sigmoid_gate(x, g, None, 1e-6)
    ones = S.rmsnorm_sigmoid_gate(x, g, np.ones(64), 1e-6)
    assert (none.o_exact == ones.o_exact).all()
