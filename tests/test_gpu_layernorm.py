"""GPU parity of the LayerNorm family: layernorm, layernorm_quant and the three DiT
gate/residual + LayerNorm modes, against the FP64 oracle.

Gates: residual_out bit-exact; BF16 outputs within one BF16 ulp, held to the
cancellation-aware bound (the oracle's magnitude of the terms) since n = (h - mean)*rstd
subtracts the mean; FP8 codes equal or one step apart at flagged ties."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from oracle import formats as F
from oracle import layernorm as L
from tests.conftest import values
from tests.parity import assert_bf16, assert_bits_equal, assert_fp8, rows_of, sample_rows

pytestmark = pytest.mark.gpu

SHAPES = [(2520, 3072), (37, 64), (9, 264), (65, 1024), (5, 4096), (11, 4616), (7, 7168),
          (3, 8192), (2, 16384), (2, 24576), (1, 32768), (1, 8), (300, 128)]


@pytest.fixture(scope="module")
def dn():
    from dit_normalization_amd import dnorm
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return dnorm


def dev(t):
    return t.to("cuda")


def dit_device(wl):
    """The DiT workload on the device, with gate/scale/shift as strided views of one
    device-resident modulation tensor (row stride 6*hidden, as the model lays them out)."""
    t = wl.tensors
    H = wl.params["hidden"]
    temb = dev(t["temb"])
    d = {k: dev(t[k]) for k in ("x", "residual", "gamma", "beta")}
    for k, name in enumerate(W.DIT_CHUNKS):
        d[name] = temb[:, k * H:(k + 1) * H]
    assert d["gate"].stride(0) == 6 * H
    return d


@pytest.mark.parametrize("rows,hidden", SHAPES)
def test_layernorm(dn, rows, hidden):
    wl = W.layernorm(rows=rows, hidden=hidden)
    t = wl.tensors
    y = dn.dn_layernorm(dev(t["x"]), dev(t["gamma"]), dev(t["beta"]), 1e-6)
    ln = L.layernorm(values(t["x"]), values(t["gamma"]), values(t["beta"]), 1e-6)
    assert_bf16(y, ln.y_exact, f"layernorm [{rows},{hidden}]", mag=ln.mag)


@pytest.mark.parametrize("rows,hidden", [(2520, 3072), (37, 64), (65, 1024), (3, 8192),
                                         (2, 24576)])
def test_layernorm_quant(dn, rows, hidden):
    wl = W.layernorm(rows=rows, hidden=hidden)
    t = wl.tensors
    q = dn.dn_layernorm_quant(dev(t["x"]), dev(t["gamma"]), dev(t["beta"]), 0.04, 1e-6)
    ln, ref = L.layernorm_quant(values(t["x"]), values(t["gamma"]), values(t["beta"]), 0.04,
                                1e-6)
    assert_fp8(q, ref.q, ref.tie, f"layernorm_quant [{rows},{hidden}]")


def test_layernorm_large_mean(dn):
    """Rows whose mean is 100 standard deviations away from zero: the one-pass FP64
    statistics must still centre them."""
    wl = W.layernorm(rows=64, hidden=3072, mean=100.0)
    t = wl.tensors
    y = dn.dn_layernorm(dev(t["x"]), dev(t["gamma"]), dev(t["beta"]), 1e-6)
    ln = L.layernorm(values(t["x"]), values(t["gamma"]), values(t["beta"]), 1e-6)
    assert_bf16(y, ln.y_exact, "layernorm mean 100", mag=ln.mag)


def test_layernorm_constant_rows_give_beta(dn):
    x = torch.full((7, 3072), -2.5, dtype=torch.bfloat16)
    beta = W.normal((3072,), 60, 0, dtype=torch.float32)
    gamma = W.normal((3072,), 60, 1, mean=1.0, dtype=torch.float32)
    y = dn.dn_layernorm(dev(x), dev(gamma), dev(beta), 1e-6)
    assert_bits_equal(y, np.broadcast_to(F.bf16_round(values(beta)), (7, 3072)), "constant rows")


def test_layernorm_empty_and_3d(dn):
    g = dev(torch.ones(1024, dtype=torch.float32))
    b = dev(torch.zeros(1024, dtype=torch.float32))
    y = dn.dn_layernorm(dev(torch.empty((0, 1024), dtype=torch.bfloat16)), g, b)
    assert y.shape == (0, 1024)
    x = W.normal((3, 11, 1024), 61, 0, mean=-1.0)
    y = dn.dn_layernorm(dev(x), g, b, 1e-6)
    ln = L.layernorm(values(x).reshape(-1, 1024), None, None, 1e-6)
    assert_bf16(y.reshape(-1, 1024), ln.y_exact, "layernorm 3-D", mag=ln.mag)


@pytest.mark.parametrize("rows,hidden", [(2520, 3072), (37, 64), (65, 1024), (3, 8192),
                                         (2, 24576)])
def test_dit_gate_residual_gamma_beta(dn, rows, hidden):
    wl = W.dit(rows=rows, hidden=hidden)
    t, p = wl.tensors, wl.params
    d = dit_device(wl)
    ro, no = dn.dn_fused_dit_gate_residual_layernorm_gamma_beta(
        d["x"], d["residual"], d["gate"], d["gamma"], d["beta"], 1e-6, gate_bias=p["gate_bias"])
    ref = L.dit_gate_residual_layernorm_gamma_beta(
        values(t["residual"]), values(t["x"]), values(t["gate"]), values(t["gamma"]),
        values(t["beta"]), p["gate_bias"], 1e-6)
    assert_bits_equal(ro, ref.residual_out, "residual_out (bit-exact)")
    assert_bf16(no, ref.o_exact, f"DiT gamma/beta norm_out [{rows},{hidden}]", mag=ref.mag)


@pytest.mark.parametrize("rows,hidden", [(2520, 3072), (37, 64), (65, 1024), (3, 8192),
                                         (2, 24576)])
def test_dit_gate_residual_scale_shift(dn, rows, hidden):
    wl = W.dit(rows=rows, hidden=hidden)
    t, p = wl.tensors, wl.params
    d = dit_device(wl)
    ro, no = dn.dn_fused_dit_gate_residual_layernorm_scale_shift(
        d["x"], d["residual"], d["gate"], d["scale"], d["shift"], 1e-6,
        gate_bias=p["gate_bias"], scale_bias=p["scale_bias"], shift_bias=p["shift_bias"])
    ref = L.dit_gate_residual_layernorm_scale_shift(
        values(t["residual"]), values(t["x"]), values(t["gate"]), values(t["scale"]),
        values(t["shift"]), p["gate_bias"], p["scale_bias"], p["shift_bias"], 1e-6)
    assert_bits_equal(ro, ref.residual_out, "residual_out (bit-exact)")
    assert_bf16(no, ref.o_exact, f"DiT scale/shift norm_out [{rows},{hidden}]", mag=ref.mag)


@pytest.mark.parametrize("with_residual", [True, False])
@pytest.mark.parametrize("rows,hidden", [(2520, 3072), (37, 64), (3, 8192)])
def test_dit_residual_scale_shift(dn, rows, hidden, with_residual):
    wl = W.dit(rows=rows, hidden=hidden)
    t, p = wl.tensors, wl.params
    d = dit_device(wl)
    ro, no = dn.dn_fused_dit_residual_layernorm_scale_shift(
        d["x"], d["scale"], d["shift"], d["residual"] if with_residual else None, 1e-6,
        scale_bias=p["scale_bias"], shift_bias=p["shift_bias"])
    ref = L.dit_residual_layernorm_scale_shift(
        values(t["x"]), values(t["scale"]), values(t["shift"]),
        values(t["residual"]) if with_residual else None, p["scale_bias"], p["shift_bias"], 1e-6)
    if with_residual:
        assert_bits_equal(ro, ref.residual_out, "residual_out (bit-exact)")
    else:
        assert ro is None
    assert_bf16(no, ref.o_exact, f"DiT residual scale/shift [{rows},{hidden}]", mag=ref.mag)


def test_dit_in_place_residual_and_zero_gate(dn):
    """residual_out may be residual itself; with gate = 0 and gate_bias = 1 the gated sum is
    the plain residual add, and zero scale/shift biases leave the plain LayerNorm."""
    wl = W.dit(rows=128, hidden=3072)
    t = wl.tensors
    d = dit_device(wl)
    zero = torch.zeros((128, 3072), dtype=torch.bfloat16, device="cuda")
    r = d["residual"].clone()
    ro, no = dn.dn_fused_dit_gate_residual_layernorm_scale_shift(
        d["x"], r, zero, zero, zero, 1e-6, gate_bias=1.0, residual_out=r)
    assert ro.data_ptr() == r.data_ptr()
    h = F.bf16_round(values(t["x"]) + values(t["residual"]))
    assert_bits_equal(r, h, "in-place residual_out")
    ln = L.layernorm(h, None, None, 1e-6)
    assert_bf16(no, ln.y_exact, "zero modulation", mag=ln.mag)


def test_dit_full_size_sampled(dn):
    """[16384, 3072] in the launch shape of the measured workload: sampled rows against the
    oracle, every row's residual_out against the oracle's gated sum on a row sample."""
    rows, H = 16384, 3072
    wl = W.dit(rows=rows, hidden=H)
    t, p = wl.tensors, wl.params
    d = dit_device(wl)
    ro, no = dn.dn_fused_dit_gate_residual_layernorm_scale_shift(
        d["x"], d["residual"], d["gate"], d["scale"], d["shift"], 1e-6,
        gate_bias=p["gate_bias"], scale_bias=p["scale_bias"], shift_bias=p["shift_bias"])
    idx = sample_rows(rows, 96, seed=5)
    sel = lambda k: values(t[k])[idx]
    ref = L.dit_gate_residual_layernorm_scale_shift(
        sel("residual"), sel("x"), sel("gate"), sel("scale"), sel("shift"), p["gate_bias"],
        p["scale_bias"], p["shift_bias"], 1e-6)
    assert_bits_equal(rows_of(ro, idx), ref.residual_out, "residual_out sampled")
    assert_bf16(rows_of(no, idx), ref.o_exact, "norm_out sampled", mag=ref.mag)


def test_layernorm_full_size_sampled(dn):
    rows, H = 8192, 4096
    wl = W.layernorm(rows=rows, hidden=H)
    t = wl.tensors
    y = dn.dn_layernorm(dev(t["x"]), dev(t["gamma"]), dev(t["beta"]), 1e-6)
    idx = sample_rows(rows, 96, seed=6)
    ln = L.layernorm(values(t["x"])[idx], values(t["gamma"]), values(t["beta"]), 1e-6)
    assert_bf16(rows_of(y, idx), ln.y_exact, "layernorm sampled", mag=ln.mag)


@pytest.mark.parametrize("tpr", [8, 16, 32, 64, 128, 256])
def test_layernorm_forced_row_mappings(dn, tpr):
    """Every row mapping that can cover the row gives the same gate-passing result."""
    wl = W.dit(rows=67, hidden=1024)
    t, p = wl.tensors, wl.params
    d = dit_device(wl)
    dn.dn_force_threads_per_row(tpr)
    try:
        ro, no = dn.dn_fused_dit_gate_residual_layernorm_gamma_beta(
            d["x"], d["residual"], d["gate"], d["gamma"], d["beta"], 1e-6,
            gate_bias=p["gate_bias"])
        torch.cuda.synchronize()
    finally:
        dn.dn_force_threads_per_row(0)
    ref = L.dit_gate_residual_layernorm_gamma_beta(
        values(t["residual"]), values(t["x"]), values(t["gate"]), values(t["gamma"]),
        values(t["beta"]), p["gate_bias"], 1e-6)
    assert_bits_equal(ro, ref.residual_out, f"residual_out tpr {tpr}")
    assert_bf16(no, ref.o_exact, f"norm_out tpr {tpr}", mag=ref.mag)
