"""The degenerate row of the norms: every element zero (or, for LayerNorm, every element
equal) with eps = 0.  The mean square (the variance) is then exactly 0, the reciprocal
1/sqrt(0) is +inf, and the normalised value 0 * inf is NaN.  The pages name no special case
for it, so the oracle's plain FP64 evaluation is the reference: rstd +inf, NaN outputs (NaN
codes in e4m3fn) on those rows, block scales of 0 (a block of NaN has no finite amax), NaN in
every dw column, and the other rows of the call untouched.  The rows sit in several tiers and
next to ordinary rows in the same launch."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from oracle import gated as G
from oracle import layernorm as L
from oracle import rmsnorm as O
from oracle import silu as S
from tests.conftest import bits8, bits16, values
from tests.parity import (assert_bf16_nonfinite, assert_bits_equal, assert_dw, assert_dx,
                          assert_fp8_nonfinite, assert_rstd, block_quant_ok)

pytestmark = pytest.mark.gpu

ZERO_ROWS = (1, 4, 6)


@pytest.fixture(scope="module")
def dn():
    from dit_normalization_amd import dnorm
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return dnorm


def dev(t):
    return t.to("cuda")


def with_zero_rows(rows, hidden, seed, slot=0):
    x = W.normal((rows, hidden), seed, slot).float()
    for r in ZERO_ROWS:
        x[r] = 0.0
    return x.to(torch.bfloat16)


def live_rows(rows):
    return np.array([r for r in range(rows) if r not in ZERO_ROWS])


def assert_rstd_with_inf(gpu, r64, what="rstd"):
    r = gpu.detach().cpu().double().numpy()
    dead = np.isinf(r64)
    assert dead[list(ZERO_ROWS)].all() and (r[dead] == np.inf).all(), f"{what}: +inf rows"
    assert_rstd(gpu[torch.as_tensor(np.flatnonzero(~dead), device=gpu.device)], r64[~dead], what)


@pytest.mark.parametrize("hidden", [8, 128, 1032, 4096, 7168, 32768])
def test_rmsnorm_zero_rows_eps0(dn, hidden):
    x = with_zero_rows(9, hidden, 501)
    w = W.normal((hidden,), 501, 1, mean=1.0, std=0.1)
    with np.errstate(divide="ignore", invalid="ignore"):
        ref = O.rmsnorm(values(x), values(w), 0.0, 0.0)
    assert np.isnan(ref.y_exact[list(ZERO_ROWS)]).all()
    y, rstd = dn.dn_rmsnorm(dev(x), dev(w), 0.0, return_rstd=True)
    assert_bf16_nonfinite(y, ref.y_exact, f"y H={hidden}")
    assert_rstd_with_inf(rstd, ref.r64, f"rstd H={hidden}")


def test_static_fp8_zero_rows_eps0(dn):
    x = with_zero_rows(9, 2048, 502)
    w = W.normal((2048,), 502, 1, mean=1.0, std=0.1)
    with np.errstate(divide="ignore", invalid="ignore"):
        _, ref = O.rmsnorm_quant(values(x), values(w), 0.05, 0.0, 0.0)
    q = dn.dn_rmsnorm_quant(dev(x), dev(w), 0.05, 0.0)
    assert_fp8_nonfinite(q, ref, "rmsnorm_quant")


@pytest.mark.parametrize("fp8", [False, True])
def test_fused_add_cancelling_to_zero_eps0(dn, fp8):
    """x = -residual on three rows: h_new is +0 there (x + (-x) rounds to +0), bit for bit,
    and the norm of that zero row is NaN."""
    r = W.normal((9, 4096), 503, 1)
    x = W.normal((9, 4096), 503, 0)
    for i in ZERO_ROWS:
        x[i] = -r[i]
    w = W.normal((4096,), 503, 2, mean=1.0, std=0.1)
    xd, rd = dev(x), dev(r)
    with np.errstate(divide="ignore", invalid="ignore"):
        if fp8:
            _, ref = O.fused_add_rmsnorm_quant(values(x), values(r), values(w), 0.05, 0.0, 0.0)
            h_new = ref_h = O.residual_add(values(x), values(r))
            q = dn.dn_fused_add_rmsnorm_quant(xd, rd, dev(w), 0.05, 0.0)
        else:
            ref = O.fused_add_rmsnorm(values(x), values(r), values(w), 0.0, 0.0)
            h_new = ref_h = ref.h_new
            rstd = torch.empty(9, dtype=torch.float32, device="cuda")
            dn.dn_fused_add_rmsnorm(xd, rd, dev(w), 0.0, rstd=rstd)
    assert (h_new[list(ZERO_ROWS)] == 0).all()
    assert_bits_equal(rd, ref_h, "h_new")
    assert (bits16(rd)[list(ZERO_ROWS)] == 0).all(), "h_new of a cancelled row is +0"
    if fp8:
        assert_fp8_nonfinite(q, ref, "fused add + static FP8")
    else:
        assert_bf16_nonfinite(xd, ref.norm.y_exact, "fused add y")
        assert_rstd_with_inf(rstd, ref.norm.r64)


@pytest.mark.parametrize("hidden", [256, 7168])
def test_block_fp8_zero_rows_eps0(dn, hidden):
    """A row of NaN has no finite amax: its block scales are 0 and every code is NaN."""
    x = with_zero_rows(9, hidden, 504)
    r = torch.zeros((9, hidden), dtype=torch.bfloat16)
    w = W.normal((hidden,), 504, 2, mean=1.0, std=0.1)
    rd = dev(r)
    normed = torch.empty((9, hidden), dtype=torch.bfloat16, device="cuda")
    q, bs = dn.dn_fused_add_rmsnorm_fp8_block_quant(dev(x), rd, dev(w), 0.0, normed_out=normed)
    with np.errstate(divide="ignore", invalid="ignore"):
        ref = O.fused_add_rmsnorm_fp8_block_quant(values(x), values(r), values(w), 0.0, 0.0)
    assert (ref.scale[list(ZERO_ROWS)] == 0).all()
    assert_bits_equal(rd, ref.h_new, "h_new")
    s = bs.t()[:9].cpu().double().numpy()
    g = bits8(q).reshape(ref.q.shape)
    scale_ok, codes_ok = block_quant_ok(s, g, ref)
    assert scale_ok.all(), f"block scales: {s[~scale_ok]} vs {ref.scale[~scale_ok]}"
    nan_ref = np.isnan(ref.normed)
    assert (((g & 0x7F) == 0x7F) == nan_ref).all(), "e4m3 NaN codes"
    assert codes_ok[~nan_ref].all(), "e4m3 codes"
    assert_bf16_nonfinite(normed, ref.normed_exact, "normed_out")


def test_training_forward_and_backward_zero_rows_eps0(dn):
    """Forward: rstd +inf and y NaN on the zero rows.  Backward on those results: dx NaN on
    those rows (x * rstd = 0 * inf), finite and within the gates on the others; every dw
    column sums one NaN per zero row, so dw is NaN throughout."""
    rows, hidden = 9, 2048
    h = with_zero_rows(rows, hidden, 505)
    u = torch.zeros((rows, hidden), dtype=torch.bfloat16)
    g = W.normal((rows, hidden), 505, 2)
    w = W.normal((hidden,), 505, 3, std=0.02).float()
    with np.errstate(divide="ignore", invalid="ignore"):
        fref = O.train_forward(values(h), values(w), 1.0, 0.0, residual=values(u))
    y, rstd, hn = dn.dn_train_forward(dev(h), dev(w), 0.0, w_bias=1.0, residual=dev(u))
    assert_bits_equal(hn, fref.h_new, "h_new")
    assert_bf16_nonfinite(y, fref.y_exact, "train y")
    assert_rstd_with_inf(rstd, fref.r64, "train rstd")

    rs = torch.from_numpy(fref.rstd.astype(np.float32))
    dx, dw = dn.dn_train_backward(dev(g), dev(h), dev(w), dev(rs), w_bias=1.0)
    with np.errstate(divide="ignore", invalid="ignore"):
        full = O.train_backward(values(g), values(h), values(w), rs.double().numpy(), 1.0)
    live = live_rows(rows)
    ref_live = O.train_backward(values(g)[live], values(h)[live], values(w),
                                rs.double().numpy()[live], 1.0)
    d = values(dx)
    assert (np.isnan(d) == np.isnan(full.dx_exact)).all(), "dx NaN positions"
    assert np.isnan(full.dx_exact[list(ZERO_ROWS)]).all()
    assert_dx(dx[torch.as_tensor(live, device="cuda")], ref_live, "dx of the other rows")
    assert np.isnan(full.dw_exact).all() and torch.isnan(dw).all(), "dw is NaN in every column"


def test_backward_of_zero_rows_with_finite_rstd(dn):
    """The same zero rows through a forward with eps > 0: rstd = 1/sqrt(eps) is finite, x * rstd
    is 0, dx = rstd * g * w on those rows, and they add nothing to dw."""
    rows, hidden = 9, 2048
    h = with_zero_rows(rows, hidden, 506)
    g = W.normal((rows, hidden), 506, 2)
    w = W.normal((hidden,), 506, 3, std=0.02).float()
    fref = O.train_forward(values(h), values(w), 1.0, 1e-6)
    assert np.isfinite(fref.r64).all()
    rs = torch.from_numpy(fref.rstd.astype(np.float32))
    dx, dw = dn.dn_train_backward(dev(g), dev(h), dev(w), dev(rs), w_bias=1.0)
    ref = O.train_backward(values(g), values(h), values(w), rs.double().numpy(), 1.0)
    assert_dx(dx, ref, "dx")
    live = live_rows(rows)
    ref_live = O.train_backward(values(g)[live], values(h)[live], values(w),
                                rs.double().numpy()[live], 1.0)
    assert np.allclose(ref.dw_exact, ref_live.dw_exact, rtol=1e-13, atol=0)
    assert_dw(dw, ref_live.dw_exact, "dw without the zero rows")


@pytest.mark.parametrize("hidden", [64, 3072, 8192])
def test_layernorm_constant_rows_eps0(dn, hidden):
    """A constant BF16 row has mean c and variance 0 exactly, so with eps = 0 the centred
    value 0 times 1/sqrt(0) is NaN; rows of zeros as well as rows of 0.75 and -3."""
    x = W.normal((9, hidden), 507, 0).float()
    x[1] = 0.0
    x[4] = 0.75
    x[6] = -3.0
    x = x.to(torch.bfloat16)
    gamma = W.normal((hidden,), 507, 1, std=0.1, dtype=torch.float32) + 1.0
    beta = W.normal((hidden,), 507, 2, std=0.1, dtype=torch.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        ref = L.layernorm(values(x), gamma.double().numpy(), beta.double().numpy(), 0.0)
    assert np.isnan(ref.y_exact[list(ZERO_ROWS)]).all()
    y = dn.dn_layernorm(dev(x), dev(gamma), dev(beta), 0.0)
    assert_bf16_nonfinite(y, ref.y_exact, f"layernorm H={hidden}")


def test_silu_zero_rows_eps0(dn):
    x = with_zero_rows(9, 1536, 508)
    w = W.normal((1536,), 508, 1, mean=1.0, std=0.1)
    with np.errstate(divide="ignore", invalid="ignore"):
        ref = S.fused_rmsnorm_silu(values(x), values(w), 0.0)
        _, ref8 = S.fused_rmsnorm_silu_fp8(values(x), values(w), 0.02, 0.0)
    y = dn.dn_fused_rmsnorm_silu(dev(x), dev(w), 0.0)
    assert_bf16_nonfinite(y, ref.s_exact, "silu y", mag=ref.mag)
    q = dn.dn_fused_rmsnorm_silu(dev(x), dev(w), 0.0, output_fp8=True, scale=0.02)
    assert_fp8_nonfinite(q, ref8, "silu e4m3")


@pytest.mark.parametrize("next_norm", [False, True])
def test_gated_residual_zero_branch_rows_eps0(dn, next_norm):
    """A zero branch row normalises to NaN, so residual + gate * NaN is NaN on that row (and
    the next norm of a NaN row is NaN); the other rows are ordinary."""
    wl = W.gated_residual(9, 4096, per_token_gate=True)
    t = wl.tensors
    branch = t["branch"].clone()
    for i in ZERO_ROWS:
        branch[i] = 0
    r = dev(t["residual"])
    with np.errstate(divide="ignore", invalid="ignore"):
        ref = G.gated_residual_rmsnorm(values(branch), values(t["residual"]), values(t["gate"]),
                                       values(t["w"]), 0.0,
                                       next_w=values(t["w_next"]) if next_norm else None)
    if next_norm:
        _, y = dn.dn_gated_residual_next_rmsnorm(dev(branch), r, dev(t["gate"]), dev(t["w"]),
                                                 dev(t["w_next"]), 0.0)
    else:
        dn.dn_gated_residual_rmsnorm(dev(branch), r, dev(t["gate"]), dev(t["w"]), 0.0)
    assert np.isnan(ref.h_exact[list(ZERO_ROWS)]).all()
    assert_bf16_nonfinite(r, ref.h_exact, "h", mag=ref.h_mag)
    if next_norm:
        assert_bf16_nonfinite(y, ref.y_exact, "next y", mag=ref.y_mag)


@pytest.mark.parametrize("interleave", [True, False])
def test_qk_rope_zero_tokens_eps0(dn, interleave):
    """The Q/K norm runs across all heads of a token: a token whose Q channels are all zero
    (and another whose K channels are) normalises to NaN there, and the rotation keeps it NaN.
    The V copy and the other tokens are unaffected."""
    from oracle import qk_rope as Q
    wl = W.qk_rope(2, 2, 3, 1, 4, 4, 4, 128, (44, 42, 42))
    t, p = wl.tensors, wl.params
    qkv = t["qkv"].clone()
    qw = p["nq"] * p["head_dim"]
    kw = p["nk"] * p["head_dim"]
    qkv[1, :qw] = 0
    qkv[5, qw:qw + kw] = 0
    qkv[6, :qw + kw] = 0
    qo, ko, vo = dn.dn_fused_qk_rmsnorm_rope(
        dev(qkv), dev(t["q_weight"]), dev(t["k_weight"]), p["nq"], p["nk"], p["nv"],
        p["head_dim"], p["ppf"], p["pph"], p["ppw"], p["channels"], 0.0, base=p["base"],
        interleave=interleave)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = Q.qk_rmsnorm_rope(values(qkv), values(t["q_weight"]), values(t["k_weight"]),
                              p["nq"], p["nk"], p["nv"], p["head_dim"], p["channels"], p["ppf"],
                              p["pph"], p["ppw"], 0.0, p["base"], interleave, 1.0, 0.0, 0.0,
                              1.0, True)
    assert np.isnan(r.q_exact[[1, 6]]).all() and np.isnan(r.k_exact[[5, 6]]).all()
    assert_bits_equal(vo, r.v, "V copy")
    assert_bf16_nonfinite(qo, r.q_exact, "Q", mag=r.q_mag)
    assert_bf16_nonfinite(ko, r.k_exact, "K", mag=r.k_mag)
