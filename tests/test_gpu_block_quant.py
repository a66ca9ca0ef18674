"""GPU parity of fused_add_rmsnorm_fp8_block_quant (1x128 FP8 blocks, MN-major scales)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from oracle import formats as F
from oracle import rmsnorm as O
from tests.conftest import bits16, bits8, values
from tests.parity import (assert_bf16, assert_bits_equal, assert_block_quant, rows_of,
                          sample_rows)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dn():
    from dit_normalization_amd import dnorm
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return dnorm


def dev(t):
    return t.to("cuda")


def check_block(gpu_q, gpu_scale_t, gpu_normed, ref: O.BlockQuant, what: str):
    """gpu_scale_t: logical [rows, hidden/128] scales."""
    assert_block_quant(gpu_q, gpu_scale_t, ref, what)
    if gpu_normed is not None:
        assert_bf16(gpu_normed, ref.normed_exact, what + " normed_out")


@pytest.mark.parametrize("rows,hidden", [(301, 7168), (64, 128), (33, 256), (130, 4096),
                                         (97, 5120), (45, 6656), (5, 8192), (17, 16384)])
def test_block_quant_against_oracle(dn, rows, hidden):
    wl = W.block_quant(rows=rows, hidden=hidden)
    x, r, w = wl.tensors["x"], wl.tensors["residual"], wl.tensors["w"]
    rd = dev(r)
    normed = torch.empty((rows, hidden), dtype=torch.bfloat16, device="cuda")
    q, bs = dn.dn_fused_add_rmsnorm_fp8_block_quant(dev(x), rd, dev(w), 1e-6, normed_out=normed)
    ld = (rows + 3) // 4 * 4
    assert bs.shape == (hidden // 128, ld)
    ref = O.fused_add_rmsnorm_fp8_block_quant(values(x), values(r), values(w), 0.0, 1e-6)
    assert_bits_equal(rd, ref.h_new, "h_new")
    check_block(q, bs.t()[:rows], normed, ref, f"block quant [{rows},{hidden}]")
    pads = bs[:, rows:].cpu()
    assert (pads == 0).all(), "scale padding must be zero"


def test_block_quant_16384x7168(dn):
    wl = W.block_quant()
    x, r, w = wl.tensors["x"], wl.tensors["residual"], wl.tensors["w"]
    rd = dev(r)
    q, bs = dn.dn_fused_add_rmsnorm_fp8_block_quant(dev(x), rd, dev(w), 1e-6)
    s = sample_rows(16384, k=96)
    ref = O.fused_add_rmsnorm_fp8_block_quant(values(x[s]), values(r[s]), values(w), 0.0, 1e-6)
    assert_bits_equal(rows_of(rd, s), ref.h_new, "h_new")
    scales = bs.t().cpu()[torch.as_tensor(s)]
    check_block(rows_of(q, s), scales, None, ref, "block quant [16384,7168]")


def test_zero_blocks_get_zero_scale(dn):
    x = torch.zeros((8, 512), dtype=torch.bfloat16)
    r = torch.zeros((8, 512), dtype=torch.bfloat16)
    r[2, :128] = 1.0
    w = torch.ones(512, dtype=torch.bfloat16)
    q, bs = dn.dn_fused_add_rmsnorm_fp8_block_quant(dev(x), dev(r), dev(w), 1e-6)
    sc = bs.t().cpu()
    assert (sc[0] == 0).all() and (sc[2, 1:] == 0).all() and sc[2, 0] > 0
    qb = bits8(q)
    assert (qb[0] & 0x7F == 0).all()
    assert (qb[2, :128] == 0x7E).all()       # a repeated value maps to 448


def test_tiny_blocks_next_to_a_huge_element(dn):
    """Rows with one huge element and tiny others: the blocks without it have normalised
    values near 1e-37 and scales far below FP32's normal range; their codes must still be
    those of n / s (no overflow of 1/s)."""
    rows, hidden = 6, 1024
    x = torch.zeros((rows, hidden), dtype=torch.bfloat16)
    r = W.normal((rows, hidden), 77, 0, std=1e-8)
    r[:, 3] = 1e30
    r[1, 700] = -2e30
    w = W.normal((hidden,), 77, 1, mean=1.0, std=0.1)
    rd = dev(r)
    q, bs = dn.dn_fused_add_rmsnorm_fp8_block_quant(dev(x), rd, dev(w), 1e-6)
    ref = O.fused_add_rmsnorm_fp8_block_quant(values(x), values(r), values(w), 0.0, 1e-6)
    assert (ref.scale[:, 1:] < 1e-36).any(), "the case must reach sub-normal-range scales"
    check_block(q, bs.t()[:rows], None, ref, "tiny blocks")
