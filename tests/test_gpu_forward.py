"""GPU parity of the forward family (rmsnorm, Gemma, FP32 weights, fused add, static FP8,
3-D per-head rows) against the FP64 oracle on seeded inputs, through the C ABI."""
from __future__ import annotations

import json
import os

import numpy as np
import pytest
import torch

import workloads as W
from oracle import formats as F
from oracle import rmsnorm as O
from tests.conftest import bits16, bits8, values
from tests.parity import (assert_bf16, assert_bits_equal, assert_fp8, assert_rstd, rows_of,
                          sample_rows)

pytestmark = pytest.mark.gpu

GRID = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_test_grid.json")))


@pytest.fixture(scope="module")
def dn():
    from dit_normalization_amd import dnorm
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return dnorm


def dev(t):
    return t.to("cuda")


def check_rmsnorm(dn, x, w, bias=0.0, eps=1e-6, what="rmsnorm"):
    y, rstd = dn.dn_rmsnorm(dev(x), dev(w), eps, w_bias=bias, return_rstd=True)
    ref = O.rmsnorm(values(x).reshape(-1, x.shape[-1]), values(w), bias, eps)
    assert_bf16(y.reshape(-1, x.shape[-1]), ref.y_exact, what)
    assert_rstd(rstd.reshape(-1), ref.r64, what + " rstd")


def test_rmsnorm_32x4096(dn):
    wl = W.rmsnorm_fwd()
    check_rmsnorm(dn, wl.tensors["x"], wl.tensors["w"], 0.0, wl.params["eps"], "rmsnorm [32,4096]")


@pytest.mark.parametrize("hidden", [8, 16, 24, 64, 72, 128, 136, 256, 264, 512, 520, 1000, 1024,
                                    1536, 2048, 2056, 3072, 4096, 4104, 5120, 5128, 6144, 6152,
                                    7168, 7176, 8192, 8200, 10240, 12288, 12296, 16384, 24576,
                                    32768])
def test_rmsnorm_every_row_tier(dn, hidden):
    x = W.normal((67, hidden), 11, hidden)
    w = W.normal((hidden,), 12, hidden, mean=1.0, std=0.2)
    check_rmsnorm(dn, x, w, what=f"rmsnorm H={hidden}")


@pytest.mark.parametrize("hidden", [128, 1024, 4096, 5120, 7168, 8192])
@pytest.mark.parametrize("tpr", [8, 16, 32, 64, 128, 256, 320, 448, 512, 1024])
def test_rmsnorm_forced_row_mapping(dn, hidden, tpr):
    x = W.normal((45, hidden), 13, hidden)
    w = W.normal((hidden,), 14, hidden, mean=1.0, std=0.2)
    dn.dn_force_threads_per_row(tpr)
    try:
        check_rmsnorm(dn, x, w, what=f"rmsnorm H={hidden} tpr={tpr}")
    finally:
        dn.dn_force_threads_per_row(0)


@pytest.mark.parametrize("hidden", GRID["hidden"])
@pytest.mark.parametrize("pad", GRID["row_stride_padding"])
def test_rmsnorm_page_grid_rows_and_strides(dn, hidden, pad):
    extra = {"0": 0, "64": 64, "2H": 2 * hidden}[pad]
    for rows in [r for r in GRID["rows"] if r < 1000]:
        big = W.normal((rows, hidden + extra), 15, rows)
        x = big[:, :hidden]                    # a row-strided view, read in place
        w = W.normal((hidden,), 16, hidden)
        xd = dev(big)[:, :hidden]
        y, rstd = dn.dn_rmsnorm(xd, dev(w), 1e-6, return_rstd=True)
        ref = O.rmsnorm(values(x), values(w), 0.0, 1e-6)
        assert_bf16(y, ref.y_exact, f"rows={rows} H={hidden} pad={pad}")
        assert_rstd(rstd, ref.r64)


def test_misaligned_views_are_copied_once(dn):
    """A view whose base is not 16-byte aligned (one element into a buffer) is read through
    one aligned copy; an output view like that receives the result through a copy back."""
    x = W.normal((19, 512), 19, 0)
    w = W.normal((512,), 19, 1)
    buf = torch.empty(19 * 512 + 1, dtype=torch.bfloat16, device="cuda")
    xv = buf[1:].view(19, 512)
    xv.copy_(dev(x))
    assert xv.data_ptr() % 16 != 0 and xv.is_contiguous()
    obuf = torch.zeros(19 * 512 + 3, dtype=torch.bfloat16, device="cuda")
    ov = obuf[3:].view(19, 512)
    y = dn.dn_rmsnorm(xv, dev(w), 1e-6, out=ov)
    ref = O.rmsnorm(values(x), values(w), 0.0, 1e-6)
    assert y.data_ptr() == ov.data_ptr()
    assert_bf16(ov, ref.y_exact, "misaligned in and out")
    assert torch.equal(obuf[:3], torch.zeros(3, dtype=torch.bfloat16, device="cuda"))


@pytest.mark.parametrize("rows", [16172, 16231])
def test_rmsnorm_page_grid_large_rows(dn, rows):
    x = W.normal((rows, 2048), 17, rows)
    w = W.normal((2048,), 18, rows)
    y, rstd = dn.dn_rmsnorm(dev(x), dev(w), 1e-6, return_rstd=True)
    s = sample_rows(rows)
    ref = O.rmsnorm(values(x[s]), values(w), 0.0, 1e-6)
    assert_bf16(rows_of(y, s), ref.y_exact, f"rows={rows}")
    assert_rstd(rows_of(rstd, s), ref.r64)


def test_gemma_and_fp32_weights(dn):
    x = W.normal((99, 3072), 19, 0)
    w = W.normal((3072,), 19, 1, std=0.1)
    check_rmsnorm(dn, x, w, 1.0, what="gemma bf16 weight")
    w32 = W.normal((3072,), 19, 2, std=0.02, dtype=torch.float32)
    check_rmsnorm(dn, x, w32, 1.0, what="fp32 zero-centred weight")
    check_rmsnorm(dn, x, w32, 0.0, what="fp32 weight, no bias")


@pytest.mark.parametrize("scale", GRID["input_scales"])
def test_input_scales_and_zero_rows(dn, scale):
    x = (W.normal((40, 2048), 20, 0).float() * scale).to(torch.bfloat16)
    x[3] = 0
    x[17] = 0
    w = W.normal((2048,), 20, 1)
    check_rmsnorm(dn, x, w, what=f"scale {scale}")


def test_3d_per_head_rows(dn):
    x = W.normal((64, 32, 128), 21, 0)
    w = W.normal((128,), 21, 1, mean=1.0, std=0.1)
    check_rmsnorm(dn, x, w, what="[64,32,128] per head")


def test_fp8_conversion_of_every_bf16_value(dn):
    # Constant rows of a power of two with eps = 0 make (x * r) exactly +-1, so the value
    # handed to the FP8 rounding is exactly w (times 1/scale, a power of two): every finite
    # BF16 number goes through the kernel's conversion, ties included, and the codes must
    # equal the format's round-to-nearest-even with saturation.
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = F.bf16_bits_to_f64(bits)
    finite = bits[np.isfinite(vals)]
    hidden = 4096
    n = (finite.size + hidden - 1) // hidden * hidden
    padded = np.concatenate([finite, np.zeros(n - finite.size, np.uint16)])
    for scale in [1.0, 2.0 ** -6, 2.0 ** 5]:
        for k in range(n // hidden):
            wb = padded[k * hidden:(k + 1) * hidden]
            w = torch.from_numpy(wb.view(np.int16).copy()).view(torch.bfloat16)
            x = torch.full((3, hidden), -4.0 if k % 2 else 0.5, dtype=torch.bfloat16)
            q = dn.dn_rmsnorm_quant(dev(x), dev(w), scale, 0.0)
            sign = -1.0 if k % 2 else 1.0
            want = F.f64_to_e4m3_code(sign * F.bf16_bits_to_f64(wb) / scale)
            got = bits8(q)
            for r in range(3):
                bad = ~F.codes_equal_e4m3(got[r], want)
                assert not bad.any(), f"scale {scale} chunk {k}: {bad.sum()} codes differ, " \
                                      f"first w={F.bf16_bits_to_f64(wb[bad])[0]!r}"


def test_fp8_conversion_of_every_fp32_rounding_class(dn):
    """FP32 weights make the value handed to the FP8 rounding any FP32 number (rows of a
    power of two, eps = 0: x * r = +-1 exactly).  The e4m3fn code of an FP32 value depends
    only on its binade, its leading mantissa bits and whether the bits below them are zero
    (the sticky information), so every binade from the FP32 subnormals up to [512, 1024)
    is fed its 32 five-bit mantissa heads, each with the bits below zero, one, all ones and
    random: every rounding class of the conversion, ties and saturation included."""
    rng = np.random.default_rng(31)
    vals = []
    for e in range(-150, 10):                  # e = -150: the FP32 subnormal binades
        for head in range(32):
            for low in (0, 1, (1 << 18) - 1, int(rng.integers(2, (1 << 18) - 1))):
                mant = (head << 18) | low
                if e == -150:
                    v = np.float32(np.ldexp(float(mant), -149))        # subnormal pattern
                else:
                    v = np.float32(np.ldexp(1.0 + mant / 2.0 ** 23, e))
                vals.append(v)
    w32 = np.array(vals, dtype=np.float32)
    hidden = 32768
    assert w32.size <= hidden
    w_pad = np.zeros(hidden, np.float32)
    w_pad[:w32.size] = w32
    w = torch.from_numpy(w_pad)
    for scale in [1.0, 2.0 ** -6, 2.0 ** 5]:
        x = torch.tensor([[0.5] * hidden, [-4.0] * hidden], dtype=torch.bfloat16)
        q = bits8(dn.dn_rmsnorm_quant(dev(x), dev(w), scale, 0.0))
        for r, sign in ((0, 1.0), (1, -1.0)):
            want = F.f64_to_e4m3_code(sign * w_pad.astype(np.float64) / scale)
            bad = ~F.codes_equal_e4m3(q[r], want)
            assert not bad.any(), f"scale {scale} sign {sign}: {bad.sum()} codes differ, " \
                                  f"first w={float(w_pad[bad][0])!r}"


def test_rmsnorm_quant(dn):
    x = W.normal((130, 4096), 22, 0)
    w = W.normal((4096,), 22, 1, mean=1.0, std=0.1)
    q = dn.dn_rmsnorm_quant(dev(x), dev(w), 0.04)
    n, ref = O.rmsnorm_quant(values(x), values(w), 0.04)
    assert_fp8(q, ref.q, ref.tie, "rmsnorm_quant")


def test_fused_add_rmsnorm_in_place(dn):
    wl = W.fused_add_quant(rows=300)
    x, r, w = wl.tensors["x"], wl.tensors["residual"], wl.tensors["w"]
    xd, rd = dev(x), dev(r)
    rstd = torch.empty(300, dtype=torch.float32, device="cuda")
    dn.dn_fused_add_rmsnorm(xd, rd, dev(w), 1e-6, rstd=rstd)
    ref = O.fused_add_rmsnorm(values(x), values(r), values(w), 0.0, 1e-6)
    assert_bits_equal(rd, ref.h_new, "h_new")
    assert_bf16(xd, ref.norm.y_exact, "y (in input)")
    assert_rstd(rstd, ref.norm.r64)


@pytest.mark.parametrize("gemma", [False, True])
def test_fused_add_rmsnorm_8192x4096_in_place(dn, gemma):
    """The plain in-place fused add at its benchmark shape, every row against the oracle:
    there each block walks several grid-stride steps and rows that span two waves meet in
    alternating reduction slots, which launches of a few hundred rows never reach.  With
    gemma the BF16 weight takes the +1 offset (w_bias = 1)."""
    wl = W.fused_add_quant()
    x, r = wl.tensors["x"], wl.tensors["residual"]
    w = W.normal((4096,), 2, 7, std=0.1) if gemma else wl.tensors["w"]
    bias = 1.0 if gemma else 0.0
    xd, rd = dev(x), dev(r)
    rstd = torch.empty(8192, dtype=torch.float32, device="cuda")
    dn.dn_fused_add_rmsnorm(xd, rd, dev(w), 1e-6, w_bias=bias, rstd=rstd)
    torch.cuda.synchronize()
    ref = O.fused_add_rmsnorm(values(x), values(r), values(w), bias, 1e-6)
    what = "gemma " if gemma else ""
    assert_bits_equal(rd, ref.h_new, f"{what}h_new [8192,4096]")
    assert_bf16(xd, ref.norm.y_exact, f"{what}y (in input) [8192,4096]")
    assert_rstd(rstd, ref.norm.r64, f"{what}rstd [8192,4096]")


def test_fused_add_equals_add_then_norm(dn):
    x = W.normal((77, 2048), 23, 0)
    r = W.normal((77, 2048), 23, 1)
    w = W.normal((2048,), 23, 2)
    xd, rd = dev(x), dev(r)
    dn.dn_fused_add_rmsnorm(xd, rd, dev(w), 1e-6)
    y2 = dn.dn_rmsnorm(rd.clone(), dev(w), 1e-6)
    assert torch.equal(bits_t(xd), bits_t(y2)), "fused result differs from add-then-rmsnorm"


def bits_t(t):
    return t.view(torch.int16)


def test_fused_add_quant_8192x4096(dn):
    wl = W.fused_add_quant()
    x, r, w = wl.tensors["x"], wl.tensors["residual"], wl.tensors["w"]
    rd = dev(r)
    q = dn.dn_fused_add_rmsnorm_quant(dev(x), rd, dev(w), wl.params["scale"], 1e-6)
    h_all = O.residual_add(values(x), values(r))
    assert_bits_equal(rd, h_all, "h_new [8192,4096]")
    s = sample_rows(8192)
    fa, ref = O.fused_add_rmsnorm_quant(values(x[s]), values(r[s]), values(w), 0.04, 0.0, 1e-6)
    assert_fp8(rows_of(q, s), ref.q, ref.tie, "fp8 out [8192,4096]")


def test_fused_add_quant_gemma_8192x4096(dn):
    wl = W.fused_add_quant()
    x, r = wl.tensors["x"], wl.tensors["residual"]
    w = W.normal((4096,), 2, 7, std=0.1)
    q = dn.dn_fused_add_rmsnorm_quant(dev(x), dev(r), dev(w), 0.04, 1e-6, w_bias=1.0)
    s = sample_rows(8192, seed=1)
    fa, ref = O.fused_add_rmsnorm_quant(values(x[s]), values(r[s]), values(w), 0.04, 1.0, 1e-6)
    assert_fp8(rows_of(q, s), ref.q, ref.tie, "gemma fp8 out")


def test_fused_add_quant_3d_per_head(dn):
    wl = W.fused_add_quant(heads=32, hidden=128)
    x, r, w = wl.tensors["x"], wl.tensors["residual"], wl.tensors["w"]
    rd = dev(r)
    q = dn.dn_fused_add_rmsnorm_quant(dev(x), rd, dev(w), 0.04, 1e-6)
    x2, r2 = x.reshape(-1, 128), r.reshape(-1, 128)
    s = sample_rows(x2.shape[0], k=512)
    assert_bits_equal(rows_of(rd.reshape(-1, 128), s), O.residual_add(values(x2[s]),
                                                                      values(r2[s])), "h_new 3d")
    fa, ref = O.fused_add_rmsnorm_quant(values(x2[s]), values(r2[s]), values(w), 0.04, 0.0, 1e-6)
    assert_fp8(rows_of(q.reshape(-1, 128), s), ref.q, ref.tie, "fp8 out 3d")


def test_rows_do_not_depend_on_token_count(dn):
    # The same rows give the same bits whatever the number of rows in the call.
    x = W.normal((8192, 4096), 24, 0)
    r = W.normal((8192, 4096), 24, 1)
    w = W.normal((4096,), 24, 2)
    outs = {}
    for t in [1, 7, 64, 1000, 8192]:
        rd = dev(r[:t].clone())
        outs[t] = (bits8(dn.dn_fused_add_rmsnorm_quant(dev(x[:t]), rd, dev(w), 0.04, 1e-6)),
                   bits16(rd))
    for t in [1, 7, 64, 1000]:
        assert (outs[t][0] == outs[8192][0][:t]).all(), f"fp8 rows differ at T={t}"
        assert (outs[t][1] == outs[8192][1][:t]).all(), f"h_new rows differ at T={t}"


def test_zero_rows_is_a_no_op(dn):
    x = torch.empty((0, 4096), dtype=torch.bfloat16, device="cuda")
    w = torch.ones(4096, dtype=torch.bfloat16, device="cuda")
    y = dn.dn_rmsnorm(x, w)
    assert y.shape == (0, 4096)
