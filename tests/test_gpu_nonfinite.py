"""Non-finite inputs propagate as IEEE arithmetic says, on the GPU as in the FP64 oracle: a
row holding an infinity has rstd 0 and NaN where 0 * inf is taken, a row holding a NaN is
NaN throughout, and the other rows of the call are untouched by them.  The pages define no
special case, so the oracle's plain FP64 evaluation is the reference: NaN positions must
agree, infinities must agree, and every finite value passes the usual gates."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from oracle import formats as F
from oracle import layernorm as L
from oracle import rmsnorm as O
from oracle import silu as S
from tests.conftest import bits8, values
from tests.parity import assert_bf16_nonfinite, assert_fp8_nonfinite, block_quant_ok

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dn():
    from dit_normalization_amd import dnorm
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return dnorm


def dev(t):
    return t.to("cuda")


def with_specials(rows, hidden, seed):
    """BF16 rows; row 1 holds +inf, row 2 -inf, row 3 a NaN, row 4 +inf and -inf."""
    x = W.normal((rows, hidden), seed, 0).float()
    x[1, 3] = float("inf")
    x[2, hidden - 1] = float("-inf")
    x[3, hidden // 2] = float("nan")
    x[4, 0], x[4, 1] = float("inf"), float("-inf")
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("hidden", [128, 4096])
def test_rmsnorm_and_rstd_with_infinities_and_nans(dn, hidden):
    x = with_specials(9, hidden, 401)
    w = W.normal((hidden,), 401, 1, mean=1.0, std=0.1)
    with np.errstate(invalid="ignore", over="ignore"):
        ref = O.rmsnorm(values(x), values(w), 0.0, 1e-6)
    y, rstd = dn.dn_rmsnorm(dev(x), dev(w), 1e-6, return_rstd=True)
    assert_bf16_nonfinite(y, ref.y_exact, f"y H={hidden}")
    r = rstd.cpu().double().numpy()
    assert (np.isnan(r) == np.isnan(ref.r64)).all()
    ok = np.isfinite(ref.r64)
    assert (r[~ok & ~np.isnan(ref.r64)] == ref.r64[~ok & ~np.isnan(ref.r64)]).all()
    assert np.all(np.abs(r[ok] - ref.r64[ok]) <= 2e-7 * np.abs(ref.r64[ok]))


def test_fused_add_with_opposite_infinities(dn):
    x = with_specials(9, 1024, 402)
    r = W.normal((9, 1024), 402, 1).float()
    r[5, 7] = float("inf")
    r = r.to(torch.bfloat16)
    x2 = x.float()
    x2[5, 7] = float("-inf")                  # inf + (-inf) = NaN in h_new
    x = x2.to(torch.bfloat16)
    w = W.normal((1024,), 402, 2, mean=1.0, std=0.1)
    xd, rd = dev(x), dev(r)
    dn.dn_fused_add_rmsnorm(xd, rd, dev(w), 1e-6)
    with np.errstate(invalid="ignore", over="ignore"):
        ref = O.fused_add_rmsnorm(values(x), values(r), values(w), 0.0, 1e-6)
    h = values(rd)
    assert (np.isnan(h) == np.isnan(ref.h_new)).all()
    fin = ~np.isnan(ref.h_new)
    assert (h[fin] == ref.h_new[fin]).all(), "h_new"
    assert_bf16_nonfinite(xd, ref.norm.y_exact, "y")


def test_static_fp8_with_infinities_and_nans(dn):
    x = with_specials(9, 512, 403)
    w = W.normal((512,), 403, 1, mean=1.0, std=0.1)
    q = dn.dn_rmsnorm_quant(dev(x), dev(w), 0.04, 1e-6)
    with np.errstate(invalid="ignore", over="ignore"):
        _, ref = O.rmsnorm_quant(values(x), values(w), 0.04, 0.0, 1e-6)
    g = bits8(q).reshape(ref.q.shape)
    nan_ref = np.isnan(ref.v)
    assert (((g & 0x7F) == 0x7F) == nan_ref).all(), "e4m3 NaN codes"
    ok = F.codes_equal_e4m3(g, ref.q) | ref.tie
    assert ok[~nan_ref].all(), "e4m3 codes"


def test_layernorm_with_infinities_and_nans(dn):
    x = with_specials(9, 1024, 404)
    g = W.normal((1024,), 404, 1, std=0.1, dtype=torch.float32) + 1.0
    b = W.normal((1024,), 404, 2, std=0.1, dtype=torch.float32)
    y = dn.dn_layernorm(dev(x), dev(g), dev(b), 1e-6)
    with np.errstate(invalid="ignore", over="ignore"):
        ref = L.layernorm(values(x), g.double().numpy(), b.double().numpy(), 1e-6)
    assert_bf16_nonfinite(y, ref.y_exact, "layernorm y")


def test_silu_with_infinities_and_nans(dn):
    """SiLU of the IEEE norm: NaN stays NaN (the epilogue's maximum and its in-range vote
    skip it), rows holding an infinity are SiLU(0) = 0 apart from their NaN elements."""
    x = with_specials(9, 512, 405)
    w = W.normal((512,), 405, 1, mean=1.0, std=0.1)
    with np.errstate(invalid="ignore", over="ignore"):
        ref = S.fused_rmsnorm_silu(values(x), values(w), 1e-6)
        _, ref8 = S.fused_rmsnorm_silu_fp8(values(x), values(w), 0.02, 1e-6)
    y = dn.dn_fused_rmsnorm_silu(dev(x), dev(w), 1e-6)
    assert_bf16_nonfinite(y, ref.s_exact, "silu y", mag=ref.mag)
    q = dn.dn_fused_rmsnorm_silu(dev(x), dev(w), 1e-6, output_fp8=True, scale=0.02)
    assert_fp8_nonfinite(q, ref8, "silu e4m3")


@pytest.mark.parametrize("interleave", [True, False])
def test_qk_rope_fp8_with_infinities_and_nans(dn, interleave):
    """A Q head holding +inf (rstd 0: NaN where 0 * inf is taken, the rest of the head 0),
    a K head holding a NaN, V holding +-inf (saturating to +-448) and a NaN (the NaN code)."""
    from oracle import qk_rope as Q
    wl = W.qk_rope(2, 2, 3, 1, 4, 4, 4, 128, (44, 42, 42))
    t, p = wl.tensors, wl.params
    qkv = t["qkv"].float()
    qkv[1, 5] = float("inf")
    qkv[2, 4 * 128 + 9] = float("nan")
    qkv[3, 8 * 128 + 1] = float("inf")
    qkv[3, 8 * 128 + 2] = float("-inf")
    qkv[4, 9 * 128 + 3] = float("nan")
    qkv = qkv.to(torch.bfloat16)
    qo, ko, vo = dn.dn_fused_qk_rmsnorm_rope(
        dev(qkv), dev(t["q_weight"]), dev(t["k_weight"]), p["nq"], p["nk"], p["nv"],
        p["head_dim"], p["ppf"], p["pph"], p["ppw"], p["channels"], p["eps"], base=p["base"],
        interleave=interleave, output_fp8=True, output_quant_scale=p["output_scale"],
        v_quant_scale=p["v_scale"])
    with np.errstate(invalid="ignore", over="ignore"):
        r = Q.qk_rmsnorm_rope(values(qkv), values(t["q_weight"]), values(t["k_weight"]),
                              p["nq"], p["nk"], p["nv"], p["head_dim"], p["channels"], p["ppf"],
                              p["pph"], p["ppw"], p["eps"], p["base"], interleave, 1.0, 0.0, 0.0,
                              1.0, True)
        q8, k8, v8 = Q.qk_rmsnorm_rope_fp8(r, p["output_scale"], p["v_scale"])
    assert np.isnan(q8.v).any() and np.isnan(k8.v).any() and np.isnan(v8.v).any()
    assert (v8.q == 0x7E).any() and (v8.q == 0xFE).any()
    assert_fp8_nonfinite(qo, q8, "Q e4m3")
    assert_fp8_nonfinite(ko, k8, "K e4m3")
    assert_fp8_nonfinite(vo, v8, "V e4m3")


def test_block_quant_with_infinities_and_nans(dn):
    """1x128 FP8 blocks under the IEEE maxNum reading: a NaN element neither sets nor hides
    its block's scale and is coded NaN.  Rows 1-4 carry infinities and a NaN; a NaN weight
    column puts one NaN among numbers in every row's first block."""
    x = with_specials(9, 256, 406)
    r = W.normal((9, 256), 406, 1)
    w = W.normal((256,), 406, 2, mean=1.0, std=0.1).float()
    w[9] = float("nan")
    w = w.to(torch.bfloat16)
    rd = dev(r)
    normed = torch.empty((9, 256), dtype=torch.bfloat16, device="cuda")
    q, bs = dn.dn_fused_add_rmsnorm_fp8_block_quant(dev(x), rd, dev(w), 1e-6, normed_out=normed)
    with np.errstate(invalid="ignore", over="ignore"):
        ref = O.fused_add_rmsnorm_fp8_block_quant(values(x), values(r), values(w), 0.0, 1e-6)
    h = values(rd)
    assert (np.isnan(h) == np.isnan(ref.h_new)).all()
    assert (h[~np.isnan(h)] == ref.h_new[~np.isnan(ref.h_new)]).all(), "h_new"
    s = bs.t()[:9].cpu().double().numpy()
    g = bits8(q).reshape(ref.q.shape)
    scale_ok, codes_ok = block_quant_ok(s, g, ref)
    assert scale_ok.all(), f"block scales: {s[~scale_ok]} vs {ref.scale[~scale_ok]}"
    nan_ref = np.isnan(ref.normed)
    assert nan_ref[:, 9].all() and (ref.scale > 0).any()
    assert (((g & 0x7F) == 0x7F) == nan_ref).all(), "e4m3 NaN codes"
    assert codes_ok[~nan_ref].all(), "e4m3 codes"
    assert_bf16_nonfinite(normed, ref.normed_exact, "normed_out")
