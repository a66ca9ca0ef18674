"""Seeded random shapes for the row engines: hidden sizes (any multiple of 8 up to 32768),
row counts, padded row strides and weight dtypes drawn at random, each checked against the
FP64 oracle with the standard gates.  DN_RANDOM_SHAPES (default 24) sets the number of seeds
for the fused add; LayerNorm and the training pair take the first half of them."""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import workloads as W
from oracle import layernorm as L
from oracle import rmsnorm as O
from tests.conftest import values
from tests.parity import (assert_bf16, assert_bits_equal, assert_dw, assert_dx, assert_fp8,
                          assert_rstd)

pytestmark = pytest.mark.gpu

CASES = list(range(int(os.environ.get("DN_RANDOM_SHAPES", "24"))))


@pytest.fixture(scope="module")
def dn():
    from dit_normalization_amd import dnorm
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return dnorm


def draw(case):
    rng = np.random.default_rng(1000 + case)
    hidden = int(8 * rng.integers(1, 4097))
    rows = int(rng.integers(1, max(2, min(300, (1 << 22) // hidden))))
    pad = int(8 * rng.integers(0, 5))
    f32w = bool(rng.integers(0, 2))
    return rows, hidden, pad, f32w


def padded(t, pad):
    """A view of t with `pad` extra elements at the end of every row (row stride H + pad)."""
    if pad == 0:
        return t
    big = torch.zeros((t.shape[0], t.shape[1] + pad), dtype=t.dtype, device=t.device)
    big[:, :t.shape[1]] = t
    return big[:, :t.shape[1]]


@pytest.mark.parametrize("case", CASES)
def test_random_fused_add_and_quant(dn, case):
    rows, hidden, pad, f32w = draw(case)
    x = W.normal((rows, hidden), 2000 + case, 0)
    r = W.normal((rows, hidden), 2000 + case, 1)
    w = W.normal((hidden,), 2000 + case, 2, mean=0.0 if f32w else 1.0, std=0.1,
                 dtype=torch.float32 if f32w else torch.bfloat16)
    bias = 1.0 if f32w else 0.0
    xd, rd = padded(x.cuda(), pad), padded(r.cuda(), pad)
    rstd = torch.empty(rows, dtype=torch.float32, device="cuda")
    dn.dn_fused_add_rmsnorm(xd, rd, w.cuda(), 1e-6, w_bias=bias, rstd=rstd)
    fa = O.fused_add_rmsnorm(values(x), values(r), values(w), bias, 1e-6)
    what = f"case {case}: [{rows},{hidden}] pad {pad} f32w {f32w}"
    assert_bits_equal(rd, fa.h_new, f"h_new {what}")
    assert_bf16(xd, fa.norm.y_exact, f"y {what}")
    assert_rstd(rstd, fa.norm.r64, f"rstd {what}")
    xq = padded(x.cuda(), pad)
    rq = padded(r.cuda(), pad)
    q = dn.dn_fused_add_rmsnorm_quant(xq, rq, w.cuda(), 0.04, 1e-6, w_bias=bias)
    _, ref = O.fused_add_rmsnorm_quant(values(x), values(r), values(w), 0.04, bias, 1e-6)
    assert_fp8(q, ref.q, ref.tie, f"fp8 {what}")


@pytest.mark.parametrize("case", CASES[:len(CASES) // 2])
def test_random_layernorm(dn, case):
    rows, hidden, pad, _ = draw(case)
    x = W.normal((rows, hidden), 3000 + case, 0, mean=0.3)
    g = W.normal((hidden,), 3000 + case, 1, mean=1.0, std=0.1, dtype=torch.float32)
    b = W.normal((hidden,), 3000 + case, 2, std=0.1, dtype=torch.float32)
    y = torch.empty((rows, hidden + pad), dtype=torch.bfloat16, device="cuda")[:, :hidden]
    dn.dn_layernorm(padded(x.cuda(), pad), g.cuda(), b.cuda(), 1e-6, out=y)
    ln = L.layernorm(values(x), values(g), values(b), 1e-6)
    assert_bf16(y, ln.y_exact, f"layernorm case {case} [{rows},{hidden}] pad {pad}", mag=ln.mag)


@pytest.mark.parametrize("case", CASES[:len(CASES) // 2])
def test_random_train(dn, case):
    rows, hidden, pad, f32w = draw(case)
    h = W.normal((rows, hidden), 4000 + case, 0)
    g = W.normal((rows, hidden), 4000 + case, 1)
    w = W.normal((hidden,), 4000 + case, 2, std=0.02, dtype=torch.float32)
    fwd = O.train_forward(values(h), values(w), 1.0, 1e-6)
    # the backward runs on the oracle's rstd and the BF16 input (never on GPU outputs)
    rstd = torch.from_numpy(fwd.rstd.astype(np.float32)).cuda()
    dx, dw = dn.dn_train_backward(padded(g.cuda(), pad), padded(h.cuda(), pad), w.cuda(), rstd,
                                  w_bias=1.0)
    ref = O.train_backward(values(g), values(h), values(w), fwd.rstd, 1.0)
    assert_dx(dx, ref, f"dx case {case} [{rows},{hidden}]")
    assert_dw(dw, ref.dw_exact, f"dw case {case} [{rows},{hidden}]")
