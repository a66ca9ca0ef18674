"""Properties of the NEXT-row kernels that hold at any size: a row's bits do not depend on
how many rows share the call (the row mapping depends on the width only), outputs written
through padded row strides equal the packed ones, and in-place / out-of-place agree."""
from __future__ import annotations

import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dn():
    from dit_normalization_amd import dnorm
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return dnorm


def bits(t):
    return t.detach().contiguous().view(torch.int16) if t.dtype == torch.bfloat16 else \
        t.detach().contiguous().view(torch.uint8)


@pytest.mark.parametrize("hidden", [64, 1024, 3072, 8192])
def test_row_results_do_not_depend_on_row_count(dn, hidden):
    wl = W.dit(rows=300, hidden=hidden)
    t, p = wl.tensors, wl.params
    x, r = t["x"].cuda(), t["residual"].cuda()
    temb = t["temb"].cuda()
    ch = {n: temb[:, k * hidden:(k + 1) * hidden] for k, n in enumerate(W.DIT_CHUNKS)}
    g, b = t["gamma"].cuda(), t["beta"].cuda()
    full_ln = dn.dn_layernorm(x, g, b)
    _, full_dit = dn.dn_fused_dit_gate_residual_layernorm_scale_shift(
        x, r, ch["gate"], ch["scale"], ch["shift"], gate_bias=0.25, scale_bias=0.125)
    full_silu = dn.dn_fused_rmsnorm_silu(x, g.to(torch.bfloat16))
    for lo, hi in ((0, 1), (7, 8), (5, 37), (299, 300)):
        assert torch.equal(bits(dn.dn_layernorm(x[lo:hi], g, b)), bits(full_ln[lo:hi]))
        _, d = dn.dn_fused_dit_gate_residual_layernorm_scale_shift(
            x[lo:hi], r[lo:hi], ch["gate"][lo:hi], ch["scale"][lo:hi], ch["shift"][lo:hi],
            gate_bias=0.25, scale_bias=0.125)
        assert torch.equal(bits(d), bits(full_dit[lo:hi]))
        assert torch.equal(bits(dn.dn_fused_rmsnorm_silu(x[lo:hi], g.to(torch.bfloat16))),
                           bits(full_silu[lo:hi]))


def test_padded_output_strides_equal_packed_outputs(dn):
    wl = W.dit(rows=129, hidden=3072)
    t, p = wl.tensors, wl.params
    x, r = t["x"].cuda(), t["residual"].cuda()
    temb = t["temb"].cuda()
    gate, scale, shift = (temb[:, k * 3072:(k + 1) * 3072] for k in range(2, -1, -1))
    ro, no = dn.dn_fused_dit_gate_residual_layernorm_scale_shift(x, r, gate, scale, shift)
    big_r = torch.zeros((129, 3072 + 128), dtype=torch.bfloat16, device="cuda")
    big_n = torch.zeros((129, 3072 + 64), dtype=torch.bfloat16, device="cuda")
    dn.dn_fused_dit_gate_residual_layernorm_scale_shift(
        x, r, gate, scale, shift, residual_out=big_r[:, :3072], norm_out=big_n[:, :3072])
    assert torch.equal(bits(big_r[:, :3072]), bits(ro))
    assert torch.equal(bits(big_n[:, :3072]), bits(no))
    assert not big_r[:, 3072:].any() and not big_n[:, 3072:].any()   # padding untouched


def test_in_place_and_out_of_place_agree(dn):
    wl = W.dit(rows=64, hidden=3072)
    t = wl.tensors
    x, r = t["x"].cuda(), t["residual"].cuda()
    temb = t["temb"].cuda()
    gate = temb[:, 2 * 3072:3 * 3072]
    g, b = t["gamma"].cuda(), t["beta"].cuda()
    ro, no = dn.dn_fused_dit_gate_residual_layernorm_gamma_beta(x, r, gate, g, b, gate_bias=0.5)
    r2, x2 = r.clone(), x.clone()
    dn.dn_fused_dit_gate_residual_layernorm_gamma_beta(x2, r2, gate, g, b, gate_bias=0.5,
                                                       residual_out=r2, norm_out=x2)
    assert torch.equal(bits(r2), bits(ro)) and torch.equal(bits(x2), bits(no))


def test_gated_residual_row_count_invariance(dn):
    wl = W.gated_residual(200, 8192)
    t = wl.tensors
    b, g, w, w2 = (t[k].cuda() for k in ("branch", "gate", "w", "w_next"))
    r = t["residual"].cuda()
    r_full = r.clone()
    _, y_full = dn.dn_gated_residual_next_rmsnorm(b, r_full, g, w, w2)
    for lo, hi in ((0, 1), (99, 100), (150, 200)):
        rr = r[lo:hi].clone()
        _, y = dn.dn_gated_residual_next_rmsnorm(b[lo:hi], rr, g[lo:hi], w, w2)
        assert torch.equal(bits(rr), bits(r_full[lo:hi])) and torch.equal(bits(y), bits(y_full[lo:hi]))
