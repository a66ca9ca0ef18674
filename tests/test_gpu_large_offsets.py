"""Tensors larger than 4 GiB: rows whose byte offset passes 2^32 against the oracle.

Each large input is a 64-row block tiled on the GPU (524,352 rows x 4096 BF16 = 4 GiB + 512
KiB per tensor), so the oracle runs on the 64 distinct rows only.  The last 64 rows start at
byte offset 2^32 exactly: a 32-bit offset anywhere in the address arithmetic (row base,
per-row scalars, the block-scale column index, the backward's chunk strides) would send
them to the wrong place.  They must match the oracle and, bit for bit, the first 64 rows
(a row's result does not depend on where it sits)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from oracle import formats as F
from oracle import rmsnorm as O
from tests.conftest import bits8, values
from tests.parity import (assert_bf16, assert_bits_equal, assert_block_quant, assert_dw,
                          assert_dx, assert_rstd)

pytestmark = pytest.mark.gpu

BASE = 64
REPS = 8193                     # 524,352 rows
ROWS = BASE * REPS
HIDDEN = 4096                   # 8 KiB per BF16 row: row 524,288 starts at 2^32 bytes
assert (ROWS - BASE) * HIDDEN * 2 == 1 << 32


@pytest.fixture(scope="module")
def dn():
    from dit_normalization_amd import dnorm
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return dnorm


@pytest.fixture(autouse=True)
def _free():
    yield
    torch.cuda.empty_cache()


def tiled(base: torch.Tensor) -> torch.Tensor:
    return base.to("cuda").repeat(REPS, 1)


def first_and_last(t: torch.Tensor):
    """Host copies of the first and the last BASE rows."""
    return t[:BASE].cpu(), t[ROWS - BASE:].cpu()


def bits_of(t: torch.Tensor) -> torch.Tensor:
    return t.contiguous().view(torch.int16)


def bf16_tensor(v: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(F.f64_to_bf16_bits(v).view(np.int16)).view(torch.bfloat16)


def test_fused_add_rmsnorm_beyond_4gib(dn):
    xb = W.normal((BASE, HIDDEN), 90, 0)
    rb = W.normal((BASE, HIDDEN), 90, 1)
    w = W.normal((HIDDEN,), 90, 2, mean=1.0, std=0.1)
    x, r = tiled(xb), tiled(rb)
    rstd = torch.empty(ROWS, dtype=torch.float32, device="cuda")
    dn.dn_fused_add_rmsnorm(x, r, w.to("cuda"), 1e-6, rstd=rstd)
    ref = O.fused_add_rmsnorm(values(xb), values(rb), values(w), 0.0, 1e-6)
    hh, ht = first_and_last(r)
    yh, yt = first_and_last(x)
    assert torch.equal(bits_of(hh), bits_of(ht)), "h_new past 2^32 bytes differs"
    assert torch.equal(bits_of(yh), bits_of(yt)), "y past 2^32 bytes differs"
    assert_bits_equal(ht, ref.h_new, "h_new past 2^32 bytes")
    assert_bf16(yt, ref.norm.y_exact, "y past 2^32 bytes")
    assert_rstd(rstd[ROWS - BASE:], ref.norm.r64, "rstd past 2^32 bytes")


def test_block_quant_beyond_4gib(dn):
    """Block FP8: h_new rows past 2^32 bytes, FP8 rows past 2^31, and the column-major
    scales of the last rows (column index times a leading dimension of 524,352)."""
    xb = W.normal((BASE, HIDDEN), 91, 0)
    rb = W.normal((BASE, HIDDEN), 91, 1)
    w = W.normal((HIDDEN,), 91, 2, mean=1.0, std=0.1)
    x, r = tiled(xb), tiled(rb)
    q, bs = dn.dn_fused_add_rmsnorm_fp8_block_quant(x, r, w.to("cuda"), 1e-6)
    ref = O.fused_add_rmsnorm_fp8_block_quant(values(xb), values(rb), values(w), 0.0, 1e-6)
    qh, qt = first_and_last(q)
    assert (bits8(qh) == bits8(qt)).all(), "FP8 codes of the last rows differ"
    scales = bs.t()
    sh, st = scales[:BASE].cpu(), scales[ROWS - BASE:ROWS].cpu()
    assert torch.equal(sh, st), "block scales of the last rows differ"
    assert_block_quant(qt, st, ref, "block FP8 past 2^32 bytes")
    assert_bits_equal(r[ROWS - BASE:].cpu(), ref.h_new, "h_new past 2^32 bytes")


def test_training_forward_and_backward_beyond_4gib(dn):
    hb = W.normal((BASE, HIDDEN), 92, 0)
    ub = W.normal((BASE, HIDDEN), 92, 1)
    gb = W.normal((BASE, HIDDEN), 92, 2)
    w = W.normal((HIDDEN,), 92, 3, std=0.02).float()
    wd = w.to("cuda")
    fref = O.train_forward(values(hb), values(w), 1.0, 1e-6, residual=values(ub))

    h, u = tiled(hb), tiled(ub)
    y, rstd, hn = dn.dn_train_forward(h, wd, 1e-6, w_bias=1.0, residual=u)
    del h, u
    yh, yt = first_and_last(y)
    del y
    assert torch.equal(bits_of(yh), bits_of(yt)), "y past 2^32 bytes differs"
    assert_bf16(yt, fref.y_exact, "y past 2^32 bytes")
    assert_bits_equal(hn[ROWS - BASE:].cpu(), fref.h_new, "h_new past 2^32 bytes")
    assert_rstd(rstd[ROWS - BASE:], fref.r64, "rstd past 2^32 bytes")

    # The backward on the oracle's own forward results, tiled the same way.
    hb_new = bf16_tensor(fref.h_new)
    rs_b = torch.from_numpy(fref.rstd.astype(np.float32))
    del hn, rstd
    g, x = tiled(gb), tiled(hb_new)
    rs = rs_b.to("cuda").repeat(REPS)
    dx, dw = dn.dn_train_backward(g, x, wd, rs, w_bias=1.0)
    bref = O.train_backward(values(gb), fref.h_new, values(w), rs_b.double().numpy(), 1.0)
    dh, dt = first_and_last(dx)
    assert torch.equal(bits_of(dh), bits_of(dt)), "dx past 2^32 bytes differs"
    assert_dx(dt, bref, "dx past 2^32 bytes")
    assert_dw(dw, REPS * bref.dw_exact, f"dw over {ROWS} rows")


@pytest.mark.parametrize("hidden", [64, 4096])
def test_rmsnorm_and_fused_add_at_the_largest_row_stride(dn, hidden):
    """Row strides of 2^24 elements, the most the boundary accepts: 32 rows of a narrow tier
    share one buffer descriptor spanning 1 GiB, and a 40-row matrix spans 1.25 GiB."""
    stride, rows = 1 << 24, 40
    xb = W.normal((rows, hidden), 93, hidden)
    rb = W.normal((rows, hidden), 94, hidden)
    w = W.normal((hidden,), 95, hidden, mean=1.0, std=0.1)
    wd = w.to("cuda")

    def strided(t):
        big = torch.zeros((rows, stride), dtype=torch.bfloat16, device="cuda")
        big[:, :hidden] = t.to("cuda")
        return big[:, :hidden]

    x, y = strided(xb), strided(torch.zeros_like(xb))
    dn.dn_rmsnorm(x, wd, 1e-6, out=y)
    ref = O.rmsnorm(values(xb), values(w), 0.0, 1e-6)
    assert_bf16(y.cpu(), ref.y_exact, f"rmsnorm at stride 2^24, H={hidden}")
    del x, y
    x, r = strided(xb), strided(rb)
    dn.dn_fused_add_rmsnorm(x, r, wd, 1e-6)
    fref = O.fused_add_rmsnorm(values(xb), values(rb), values(w), 0.0, 1e-6)
    assert_bits_equal(r.cpu(), fref.h_new, f"h_new at stride 2^24, H={hidden}")
    assert_bf16(x.cpu(), fref.norm.y_exact, f"fused add y at stride 2^24, H={hidden}")
