"""Seeded random shapes for the other row engines: block FP8, the Ada calls, the gated residual
(+ next), RMSNorm + SiLU, the per-head sigmoid gate, the three DiT modes and the QK RMSNorm +
3-D RoPE, and seeded random value ranges (row scales, eps, outliers, LayerNorm offsets, FP8
scales) for the plain and quantised norms.  Each seed draws the shape (and the call's
options), builds the inputs from the workload generators and checks the kernel against the
FP64 oracle with the standard gates.  DN_RANDOM_SHAPES_NEXT (default 8) sets the number of
seeds per test, DN_RANDOM_FIRST_SEED (default 0) the first."""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import workloads as W
from oracle import formats as F
from oracle import gated as G
from oracle import layernorm as L
from oracle import qk_rope as Q
from oracle import rmsnorm as O
from oracle import silu as S
from tests.conftest import values
from tests.parity import (assert_bf16, assert_bits_equal, assert_block_quant, assert_dw,
                          assert_dx, assert_fp8, assert_rstd)

pytestmark = pytest.mark.gpu

_FIRST = int(os.environ.get("DN_RANDOM_FIRST_SEED", "0"))
CASES = list(range(_FIRST, _FIRST + int(os.environ.get("DN_RANDOM_SHAPES_NEXT", "8"))))
MAX_ELEMS = 1 << 20           # per tensor, so the oracle stays quick


@pytest.fixture(scope="module")
def dn():
    from dit_normalization_amd import dnorm
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return dnorm


def dev(t):
    return t.to("cuda")


def rng_of(test: int, case: int):
    return np.random.default_rng(7000 + 1000 * test + case)


def rows_for(rng, hidden: int, cap: int = 300) -> int:
    return int(rng.integers(1, max(2, min(cap, MAX_ELEMS // hidden)) + 1))


def padded(t, pad):
    """A device view of t with `pad` extra elements at the end of every row."""
    if pad == 0:
        return dev(t)
    big = torch.zeros((t.shape[0], t.shape[1] + pad), dtype=t.dtype, device="cuda")
    big[:, :t.shape[1]] = dev(t)
    return big[:, :t.shape[1]]


@pytest.mark.parametrize("case", CASES)
def test_random_block_quant(dn, case):
    rng = rng_of(0, case)
    hidden = 128 * int(rng.integers(1, 129))
    rows = rows_for(rng, hidden)
    pad = 8 * int(rng.integers(0, 3))
    with_normed = bool(rng.integers(0, 2))
    wl = W.block_quant(rows=rows, hidden=hidden, seed=100 + case)
    x, r, w = wl.tensors["x"], wl.tensors["residual"], wl.tensors["w"]
    xd, rd = padded(x, pad), padded(r, pad)
    normed = torch.empty((rows, hidden), dtype=torch.bfloat16, device="cuda") \
        if with_normed else None
    q, bs = dn.dn_fused_add_rmsnorm_fp8_block_quant(xd, rd, dev(w), 1e-6, normed_out=normed)
    ref = O.fused_add_rmsnorm_fp8_block_quant(values(x), values(r), values(w), 0.0, 1e-6)
    what = f"block quant case {case}: [{rows},{hidden}] pad {pad}"
    assert_bits_equal(rd, ref.h_new, f"h_new {what}")
    assert_block_quant(q, bs.t()[:rows], ref, what)
    assert (bs[:, rows:].cpu() == 0).all(), f"scale padding {what}"
    if with_normed:
        assert_bf16(normed, ref.normed_exact, f"normed_out {what}")


@pytest.mark.parametrize("case", CASES)
def test_random_ada(dn, case):
    rng = rng_of(1, case)
    dim = 8 * int(rng.integers(1, 1025))
    rows = rows_for(rng, dim, cap=200)
    broadcast = bool(rng.integers(0, 2))
    wl = W.ada(rows=rows, dim=dim, seed=200 + case, broadcast=broadcast)
    t = wl.tensors
    what = f"Ada case {case}: [{rows},{dim}] broadcast {broadcast}"
    w = W.normal((dim,), 200 + case, 9, mean=1.0, std=0.1)
    out, gout = dn.dn_ada_rms_norm(dev(t["x"]), dev(w), dev(t["style"]), 1e-6)
    a, _ = O.ada_rms_norm(values(t["x"]), values(w), values(t["style"]), 1e-6)
    assert_bf16(out, a.o_exact, f"BF16 {what}", mag=a.o_mag)
    assert_bits_equal(gout, a.gate_out, f"gate_out {what}")
    rd = dev(t["residual"])
    _, q, gout8 = dn.dn_gate_residual_ada_norm_fp8(rd, dev(t["x"]), dev(t["gate"]), dev(t["w"]),
                                                    dev(t["style"]), 0.04, 1e-6)
    g, ref = O.gate_residual_ada_norm_fp8(values(t["residual"]), values(t["x"]),
                                          values(t["gate"]), values(t["w"]), values(t["style"]),
                                          0.04, 1e-6)
    assert_bits_equal(rd, g.h, f"residual {what}")
    assert_bits_equal(gout8, g.gate_out, f"gated gate_out {what}")
    assert_fp8(q, ref.q, ref.tie, f"FP8 {what}")


@pytest.mark.parametrize("case", CASES)
def test_random_gated_residual(dn, case):
    rng = rng_of(2, case)
    hidden = 8 * int(rng.integers(1, 4097))
    rows = rows_for(rng, hidden, cap=200)
    per_token = bool(rng.integers(0, 2))
    next_norm = bool(rng.integers(0, 2))
    wl = W.gated_residual(rows, hidden, seed=300 + case, per_token_gate=per_token)
    t = wl.tensors
    r = dev(t["residual"])
    gate = dev(t["gate"]) if per_token else dev(t["gate"][0])
    if next_norm:
        _, y = dn.dn_gated_residual_next_rmsnorm(dev(t["branch"]), r, gate, dev(t["w"]),
                                                 dev(t["w_next"]), 1e-6)
    else:
        dn.dn_gated_residual_rmsnorm(dev(t["branch"]), r, gate, dev(t["w"]), 1e-6)
    ref = G.gated_residual_rmsnorm(values(t["branch"]), values(t["residual"]), values(t["gate"]),
                                   values(t["w"]), 1e-6,
                                   next_w=values(t["w_next"]) if next_norm else None)
    what = f"gated residual case {case}: [{rows},{hidden}] per-token {per_token} next {next_norm}"
    assert_bf16(r, ref.h_exact, f"h {what}", mag=ref.h_mag)
    if next_norm:
        assert_bf16(y, ref.y_exact, f"next {what}", mag=ref.y_mag)


@pytest.mark.parametrize("case", CASES)
def test_random_silu(dn, case):
    rng = rng_of(3, case)
    hidden = 8 * int(rng.integers(1, 513))
    tokens = rows_for(rng, hidden, cap=2000)
    wl = W.rmsnorm_silu(tokens, hidden, seed=400 + case)
    t = wl.tensors
    what = f"silu case {case}: [{tokens},{hidden}]"
    out = dn.dn_fused_rmsnorm_silu(dev(t["x"]), dev(t["w"]), 1e-6)
    r = S.fused_rmsnorm_silu(values(t["x"]), values(t["w"]), 1e-6)
    assert_bf16(out, r.s_exact, f"BF16 {what}", mag=r.mag)
    q = dn.dn_fused_rmsnorm_silu(dev(t["x"]), dev(t["w"]), 1e-6, output_fp8=True,
                                 scale=wl.params["scale"])
    _, ref = S.fused_rmsnorm_silu_fp8(values(t["x"]), values(t["w"]), wl.params["scale"], 1e-6)
    assert_fp8(q, ref.q, ref.tie, f"e4m3 {what}")


@pytest.mark.parametrize("case", CASES)
def test_random_sigmoid_gate(dn, case):
    rng = rng_of(4, case)
    head_dim = 8 * int(rng.integers(1, 129))
    heads = int(rng.integers(1, 17))
    tokens = rows_for(rng, heads * head_dim, cap=200)
    with_weight = bool(rng.integers(0, 2))
    wl = W.sigmoid_gate(tokens, heads, head_dim, seed=500 + case)
    t = wl.tensors
    x = dev(t["x"]).reshape(tokens, heads, head_dim)
    dn.dn_rmsnorm_sigmoid_gate(x, dev(t["gate"]).reshape(tokens, heads, head_dim), 1e-6,
                               weight=dev(t["w"]) if with_weight else None)
    r = S.rmsnorm_sigmoid_gate(values(t["x"]).reshape(-1, head_dim),
                               values(t["gate"]).reshape(-1, head_dim),
                               values(t["w"]) if with_weight else None, 1e-6)
    assert_bf16(x.reshape(-1, head_dim), r.o_exact,
                f"sigmoid gate case {case}: [{tokens},{heads},{head_dim}] weight {with_weight}",
                mag=r.mag)


@pytest.mark.parametrize("case", CASES)
def test_random_dit_modes(dn, case):
    rng = rng_of(5, case)
    hidden = 8 * int(rng.integers(1, 1025))
    rows = rows_for(rng, 6 * hidden, cap=200)
    wl = W.dit(rows=rows, hidden=hidden, seed=600 + case)
    t, p = wl.tensors, wl.params
    temb = dev(t["temb"])
    ch = {name: temb[:, k * hidden:(k + 1) * hidden] for k, name in enumerate(W.DIT_CHUNKS)}
    x, res = dev(t["x"]), dev(t["residual"])
    what = f"DiT case {case}: [{rows},{hidden}]"

    ro, no = dn.dn_fused_dit_gate_residual_layernorm_gamma_beta(
        x, res, ch["gate"], dev(t["gamma"]), dev(t["beta"]), 1e-6, gate_bias=p["gate_bias"])
    ref = L.dit_gate_residual_layernorm_gamma_beta(
        values(t["residual"]), values(t["x"]), values(t["gate"]), values(t["gamma"]),
        values(t["beta"]), p["gate_bias"], 1e-6)
    assert_bits_equal(ro, ref.residual_out, f"gamma/beta residual_out {what}")
    assert_bf16(no, ref.o_exact, f"gamma/beta {what}", mag=ref.mag)

    ro, no = dn.dn_fused_dit_gate_residual_layernorm_scale_shift(
        x, res, ch["gate"], ch["scale"], ch["shift"], 1e-6, gate_bias=p["gate_bias"],
        scale_bias=p["scale_bias"], shift_bias=p["shift_bias"])
    ref = L.dit_gate_residual_layernorm_scale_shift(
        values(t["residual"]), values(t["x"]), values(t["gate"]), values(t["scale"]),
        values(t["shift"]), p["gate_bias"], p["scale_bias"], p["shift_bias"], 1e-6)
    assert_bits_equal(ro, ref.residual_out, f"scale/shift residual_out {what}")
    assert_bf16(no, ref.o_exact, f"scale/shift {what}", mag=ref.mag)

    ro, no = dn.dn_fused_dit_residual_layernorm_scale_shift(
        x, ch["scale"], ch["shift"], res, 1e-6, scale_bias=p["scale_bias"],
        shift_bias=p["shift_bias"])
    ref = L.dit_residual_layernorm_scale_shift(
        values(t["x"]), values(t["scale"]), values(t["shift"]), values(t["residual"]),
        p["scale_bias"], p["shift_bias"], 1e-6)
    assert_bits_equal(ro, ref.residual_out, f"residual residual_out {what}")
    assert_bf16(no, ref.o_exact, f"residual scale/shift {what}", mag=ref.mag)


def draw_rope(rng):
    head_dim = int(rng.choice([64, 128, 256]))
    half = head_dim // 2
    a = int(rng.integers(0, half + 1))
    b = int(rng.integers(0, half - a + 1))
    channels = (2 * a, 2 * b, head_dim - 2 * a - 2 * b)
    heads = [int(rng.integers(1, 33)) for _ in range(3)]
    ppf, pph, ppw = (int(rng.integers(1, 6)) for _ in range(3))
    seq = ppf * pph * ppw
    width = sum(heads) * head_dim
    batch = int(rng.integers(1, max(2, min(4, MAX_ELEMS // (seq * width)) + 1)))
    return ppf, pph, ppw, batch, heads, head_dim, channels


@pytest.mark.parametrize("case", CASES)
def test_random_qk_rope(dn, case):
    rng = rng_of(6, case)
    ppf, pph, ppw, batch, (nq, nk, nv), hd, chn = draw_rope(rng)
    interleave = bool(rng.integers(0, 2))
    yarn = bool(rng.integers(0, 2))
    factor, low, high, af = (4.0, 2.0, 10.0, 1.2) if yarn else (1.0, 0.0, 0.0, 1.0)
    wl = W.qk_rope(ppf, pph, ppw, batch, nq, nk, nv, hd, chn, seed=700 + case)
    t, p = wl.tensors, wl.params
    what = (f"qk rope case {case}: grid {ppf}x{pph}x{ppw} batch {batch} heads {nq}/{nk}/{nv} "
            f"hd {hd} channels {chn} interleave {interleave} yarn {yarn}")

    def call(fp8):
        return dn.dn_fused_qk_rmsnorm_rope(
            dev(t["qkv"]), dev(t["q_weight"]), dev(t["k_weight"]), nq, nk, nv, hd, ppf, pph, ppw,
            chn, p["eps"], base=p["base"], interleave=interleave, yarn_factor=factor,
            yarn_low=low, yarn_high=high, attention_factor=af, output_fp8=fp8,
            output_quant_scale=p["output_scale"], v_quant_scale=p["v_scale"])

    r = Q.qk_rmsnorm_rope(values(t["qkv"]), values(t["q_weight"]), values(t["k_weight"]), nq, nk,
                          nv, hd, chn, ppf, pph, ppw, p["eps"], p["base"], interleave, factor,
                          low, high, af, True)
    qo, ko, vo = call(False)
    assert_bits_equal(vo, r.v, f"V copy {what}")
    assert_bf16(qo, r.q_exact, f"Q {what}", mag=r.q_mag)
    assert_bf16(ko, r.k_exact, f"K {what}", mag=r.k_mag)
    q8, k8, v8 = Q.qk_rmsnorm_rope_fp8(r, p["output_scale"], p["v_scale"])
    qo, ko, vo = call(True)
    assert_fp8(qo, q8.q, q8.tie, f"Q e4m3 {what}")
    assert_fp8(ko, k8.q, k8.tie, f"K e4m3 {what}")
    assert_fp8(vo, v8.q, v8.tie, f"V e4m3 {what}")


NUMERIC_OPS = ("rmsnorm", "rmsnorm_quant", "fused_add_quant", "block_quant", "layernorm",
               "layernorm_quant", "silu", "silu_fp8")


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("op", NUMERIC_OPS)
def test_random_numerics(dn, op, case):
    """Random value ranges on the plain and quantised norms: rows scaled by 10^U(-25, 25),
    1 % outliers at 50x on half the seeds, eps in {0, 1e-6, 1e-3, 1}, LayerNorm rows offset
    by up to 100 of their scale, FP8 scales 10^U(-3, 1) (saturating and not).  These drive
    the kernels' FP64 re-sum path for squares that leave FP32, the fast and NaN-safe FP8
    paths and the tiny-block-scale path."""
    rng = rng_of(10 + NUMERIC_OPS.index(op), case)
    hidden = 128 * int(rng.integers(1, 65)) if op == "block_quant" else 8 * int(rng.integers(1, 2049))
    rows = rows_for(rng, hidden, cap=100)
    scale_x = float(10.0 ** rng.uniform(-25, 25))
    eps = float(rng.choice([0.0, 1e-6, 1e-3, 1.0]))
    fp8_scale = float(np.float32(10.0 ** rng.uniform(-3, 1)))
    outliers = bool(rng.integers(0, 2))
    seed = 900 + 10 * NUMERIC_OPS.index(op) + case

    def act(tid, offset=0.0):
        t = W.normal((rows, hidden), seed, tid)
        if outliers:
            t = W.with_outliers(t, seed, 50 + tid)
        return ((t.double() + offset) * scale_x).to(torch.bfloat16)

    w = W.normal((hidden,), seed, 9, mean=1.0, std=0.1)
    what = (f"{op} case {case}: [{rows},{hidden}] scale {scale_x:.2e} eps {eps} "
            f"fp8 scale {fp8_scale:.3e} outliers {outliers}")
    if op == "rmsnorm":
        x = act(0)
        y, rstd = dn.dn_rmsnorm(dev(x), dev(w), eps, return_rstd=True)
        ref = O.rmsnorm(values(x), values(w), 0.0, eps)
        assert_bf16(y, ref.y_exact, what)
        assert_rstd(rstd, ref.r64, f"rstd {what}")
    elif op == "rmsnorm_quant":
        x = act(0)
        q = dn.dn_rmsnorm_quant(dev(x), dev(w), fp8_scale, eps)
        _, ref = O.rmsnorm_quant(values(x), values(w), fp8_scale, 0.0, eps)
        assert_fp8(q, ref.q, ref.tie, what)
    elif op == "fused_add_quant":
        x, r = act(0), act(1)
        rd = dev(r)
        q = dn.dn_fused_add_rmsnorm_quant(dev(x), rd, dev(w), fp8_scale, eps)
        fa, ref = O.fused_add_rmsnorm_quant(values(x), values(r), values(w), fp8_scale, 0.0, eps)
        assert_bits_equal(rd, fa.h_new, f"h_new {what}")
        assert_fp8(q, ref.q, ref.tie, what)
    elif op == "block_quant":
        x, r = act(0), act(1)
        rd = dev(r)
        q, bs = dn.dn_fused_add_rmsnorm_fp8_block_quant(dev(x), rd, dev(w), eps)
        ref = O.fused_add_rmsnorm_fp8_block_quant(values(x), values(r), values(w), 0.0, eps)
        assert_bits_equal(rd, ref.h_new, f"h_new {what}")
        assert_block_quant(q, bs.t()[:rows], ref, what)
    elif op in ("layernorm", "layernorm_quant"):
        x = act(0, offset=float(rng.uniform(-100, 100)))
        ga = W.normal((hidden,), seed, 7, std=0.1, dtype=torch.float32) + 1.0
        be = W.normal((hidden,), seed, 8, std=0.1, dtype=torch.float32)
        if op == "layernorm":
            y = dn.dn_layernorm(dev(x), dev(ga), dev(be), eps)
            ln = L.layernorm(values(x), ga.double().numpy(), be.double().numpy(), eps)
            assert_bf16(y, ln.y_exact, what, mag=ln.mag)
        else:
            q = dn.dn_layernorm_quant(dev(x), dev(ga), dev(be), fp8_scale, eps)
            _, ref = L.layernorm_quant(values(x), ga.double().numpy(), be.double().numpy(),
                                       fp8_scale, eps)
            assert_fp8(q, ref.q, ref.tie, what)
    else:
        x = act(0)
        if op == "silu":
            y = dn.dn_fused_rmsnorm_silu(dev(x), dev(w), eps)
            r = S.fused_rmsnorm_silu(values(x), values(w), eps)
            assert_bf16(y, r.s_exact, what, mag=r.mag)
        else:
            q = dn.dn_fused_rmsnorm_silu(dev(x), dev(w), eps, output_fp8=True, scale=fp8_scale)
            _, ref = S.fused_rmsnorm_silu_fp8(values(x), values(w), fp8_scale, eps)
            assert_fp8(q, ref.q, ref.tie, what)


@pytest.mark.parametrize("case", CASES)
def test_random_numerics_train(dn, case):
    """The training pair over random value ranges: the residual stream scaled by
    10^U(-20, 20), the gradient by 10^U(-20, 20) (kept where dx is a normal BF16 number and
    g * x a normal FP32 one), eps in {0, 1e-6, 1e-3, 1}, FP32 or BF16 weights (bias 1 or
    0), with or without the residual route and a residual gradient."""
    rng = rng_of(30, case)
    hidden = 8 * int(rng.integers(1, 2049))
    rows = rows_for(rng, hidden, cap=150)
    sx, sg = (float(10.0 ** rng.uniform(-20, 20)) for _ in range(2))
    eps = float(rng.choice([0.0, 1e-6, 1e-3, 1.0]))
    # dx ~ g * r stays inside BF16's normal range (the unit-scaled dx gate has no absolute
    # floor, and BF16 subnormals are coarser than it), and the products g * x, which the
    # backward forms in FP32, inside FP32's (the operating range the header states)
    s = max(sx, eps ** 0.5)
    sg = min(max(sg, 1e-30 * s, 1e-30 / sx), 1e30 * s, 1e30 / sx)
    f32w, residual, gres = (bool(rng.integers(0, 2)) for _ in range(3))
    seed = 1900 + case
    sc = lambda t, s: (t.double() * s).to(torch.bfloat16)
    x = sc(W.normal((rows, hidden), seed, 0), sx)
    u = sc(W.normal((rows, hidden), seed, 1), sx) if residual else None
    g = sc(W.normal((rows, hidden), seed, 2), sg)
    gr = sc(W.normal((rows, hidden), seed, 3), sg) if gres else None
    w = W.normal((hidden,), seed, 4, std=0.02, dtype=torch.float32) if f32w else \
        W.normal((hidden,), seed, 4, mean=1.0, std=0.1)
    bias = 1.0 if f32w else 0.0
    what = (f"train case {case}: [{rows},{hidden}] x {sx:.1e} g {sg:.1e} eps {eps} f32w {f32w} "
            f"residual {residual} g_residual {gres}")
    out = dn.dn_train_forward(dev(x), dev(w), eps, w_bias=bias,
                              residual=None if u is None else dev(u))
    fwd = O.train_forward(values(x), values(w), bias, eps,
                          residual=None if u is None else values(u))
    if residual:
        assert_bits_equal(out[2], fwd.h_new, f"h_new {what}")
    assert_bf16(out[0], fwd.y_exact, f"y {what}")
    assert_rstd(out[1], fwd.r64, f"rstd {what}")
    # the backward runs on the oracle's forward results (never on GPU outputs)
    xb = torch.from_numpy(F.f64_to_bf16_bits(fwd.h_new).view(np.int16)).view(torch.bfloat16) \
        if residual else x
    rstd = torch.from_numpy(fwd.rstd.astype(np.float32))
    dx, dw = dn.dn_train_backward(dev(g), dev(xb), dev(w), dev(rstd), w_bias=bias,
                                  g_residual=None if gr is None else dev(gr))
    ref = O.train_backward(values(g), values(xb), values(w), rstd.double().numpy(), bias,
                           None if gr is None else values(gr))
    assert_dx(dx, ref, f"dx {what}")
    assert_dw(dw, ref.dw_exact, f"dw {what}")



def scaled(t, s):
    return (t.double() * s).to(torch.bfloat16)


@pytest.mark.parametrize("case", CASES)
def test_random_numerics_ada(dn, case):
    """The Ada calls over random value ranges: x and the residual scaled by 10^U(-20, 20),
    the style rows (scale, shift, gate) by 10^U(-3, 3), eps in {0, 1e-6, 1e-3, 1}, static
    FP8 scales 10^U(-3, 1)."""
    rng = rng_of(31, case)
    dim = 8 * int(rng.integers(1, 1025))
    rows = rows_for(rng, dim, cap=100)
    broadcast = bool(rng.integers(0, 2))
    sx, ss = float(10.0 ** rng.uniform(-20, 20)), float(10.0 ** rng.uniform(-3, 3))
    eps = float(rng.choice([0.0, 1e-6, 1e-3, 1.0]))
    fp8_scale = float(np.float32(10.0 ** rng.uniform(-3, 1)))
    wl = W.ada(rows=rows, dim=dim, seed=2000 + case, broadcast=broadcast)
    t = wl.tensors
    x, res = scaled(t["x"], sx), scaled(t["residual"], sx)
    style = scaled(t["style"], ss)
    w = W.normal((dim,), 2000 + case, 9, mean=1.0, std=0.1)
    what = (f"Ada numerics case {case}: [{rows},{dim}] broadcast {broadcast} x {sx:.1e} "
            f"style {ss:.1e} eps {eps} fp8 scale {fp8_scale:.2e}")
    out, gout = dn.dn_ada_rms_norm(dev(x), dev(w), dev(style), eps)
    a, _ = O.ada_rms_norm(values(x), values(w), values(style), eps)
    assert_bf16(out, a.o_exact, f"BF16 {what}", mag=a.o_mag)
    assert_bits_equal(gout, a.gate_out, f"gate_out {what}")
    rd = dev(res)
    _, q, _ = dn.dn_gate_residual_ada_norm_fp8(rd, dev(x), dev(t["gate"]), dev(t["w"]),
                                               dev(style), fp8_scale, eps)
    g, ref = O.gate_residual_ada_norm_fp8(values(res), values(x), values(t["gate"]),
                                          values(t["w"]), values(style), fp8_scale, eps)
    assert_bits_equal(rd, g.h, f"residual {what}")
    assert_fp8(q, ref.q, ref.tie, f"FP8 {what}")


@pytest.mark.parametrize("case", CASES)
def test_random_numerics_gates(dn, case):
    """The gated residual (+ next) and the sigmoid gate over random value ranges: streams
    scaled by 10^U(-20, 20), gates by 10^U(-3, 3) (past the |gate| > 80 path of the
    sigmoid), eps in {0, 1e-6, 1e-3, 1}."""
    rng = rng_of(32, case)
    hidden = 8 * int(rng.integers(1, 1025))
    rows = rows_for(rng, hidden, cap=100)
    sb, sr, sgt = (float(10.0 ** rng.uniform(lo, hi)) for lo, hi in ((-20, 20), (-20, 20), (-3, 3)))
    eps = float(rng.choice([0.0, 1e-6, 1e-3, 1.0]))
    per_token = bool(rng.integers(0, 2))
    wl = W.gated_residual(rows, hidden, seed=2100 + case, per_token_gate=per_token)
    t = wl.tensors
    br, res, gate = scaled(t["branch"], sb), scaled(t["residual"], sr), scaled(t["gate"], sgt)
    what = (f"gates numerics case {case}: [{rows},{hidden}] branch {sb:.1e} residual {sr:.1e} "
            f"gate {sgt:.1e} eps {eps} per-token {per_token}")
    r = dev(res)
    _, y = dn.dn_gated_residual_next_rmsnorm(dev(br), r, dev(gate) if per_token else dev(gate[0]),
                                             dev(t["w"]), dev(t["w_next"]), eps)
    ref = G.gated_residual_rmsnorm(values(br), values(res), values(gate), values(t["w"]), eps,
                                   next_w=values(t["w_next"]))
    assert_bf16(r, ref.h_exact, f"h {what}", mag=ref.h_mag)
    assert_bf16(y, ref.y_exact, f"next {what}", mag=ref.y_mag)
    heads = int(rng.integers(1, 9))
    hd = 8 * int(rng.integers(1, 65))
    tokens = rows_for(rng, heads * hd, cap=100)
    sw = W.sigmoid_gate(tokens, heads, hd, seed=2200 + case)
    xs, gs = scaled(sw.tensors["x"], sb), scaled(sw.tensors["gate"], sgt)
    xd = dev(xs).reshape(tokens, heads, hd)
    dn.dn_rmsnorm_sigmoid_gate(xd, dev(gs).reshape(tokens, heads, hd), eps,
                               weight=dev(sw.tensors["w"]))
    s = S.rmsnorm_sigmoid_gate(values(xs).reshape(-1, hd), values(gs).reshape(-1, hd),
                               values(sw.tensors["w"]), eps)
    assert_bf16(xd.reshape(-1, hd), s.o_exact, f"sigmoid gate [{tokens},{heads},{hd}] {what}",
                mag=s.mag)


@pytest.mark.parametrize("case", CASES)
def test_random_numerics_rope(dn, case):
    """QK RMSNorm + 3-D RoPE over random parameters: qkv scaled by 10^U(-20, 20), base
    10^U(2, 6), eps in {0, 1e-6, 1e-3, 1}, YaRN factor U(1, 16) with random ramp bounds and
    attention factor (plain RoPE on half the seeds), both pairings, with and without the
    norm, BF16 and FP8 outputs at random scales."""
    rng = rng_of(33, case)
    ppf, pph, ppw, batch, (nq, nk, nv), hd, chn = draw_rope(rng)
    interleave, norm = bool(rng.integers(0, 2)), bool(rng.integers(0, 4) > 0)
    sq = float(10.0 ** rng.uniform(-20, 20))
    base = float(10.0 ** rng.uniform(2, 6))
    eps = float(rng.choice([0.0, 1e-6, 1e-3, 1.0]))
    if rng.integers(0, 2):
        factor = float(rng.uniform(1.0, 16.0))
        low = float(rng.uniform(0.0, hd / 4))
        high = float(low + rng.choice([0.0, rng.uniform(0.0, hd / 4)]))
        af = float(rng.uniform(0.5, 2.0))
    else:
        factor, low, high, af = 1.0, 0.0, 0.0, 1.0
    oscale, vscale = (float(np.float32(10.0 ** rng.uniform(-3, 0))) for _ in range(2))
    if not norm:
        sq = float(10.0 ** rng.uniform(-3, 2))      # no norm: values pass through, keep them finite
    wl = W.qk_rope(ppf, pph, ppw, batch, nq, nk, nv, hd, chn, seed=2300 + case)
    t = wl.tensors
    qkv = scaled(t["qkv"], sq)
    what = (f"rope numerics case {case}: grid {ppf}x{pph}x{ppw}x{batch} heads {nq}/{nk}/{nv} "
            f"hd {hd} ch {chn} il {interleave} norm {norm} x {sq:.1e} base {base:.1e} eps {eps} "
            f"yarn ({factor:.2f}, {low:.1f}, {high:.1f}, {af:.2f}) scales {oscale:.2e}/{vscale:.2e}")

    def call(fp8):
        return dn.dn_fused_qk_rmsnorm_rope(
            dev(qkv), dev(t["q_weight"]), dev(t["k_weight"]), nq, nk, nv, hd, ppf, pph, ppw, chn,
            eps, base=base, interleave=interleave, yarn_factor=factor, yarn_low=low,
            yarn_high=high, attention_factor=af, is_qk_norm=norm, output_fp8=fp8,
            output_quant_scale=oscale, v_quant_scale=vscale)

    r = Q.qk_rmsnorm_rope(values(qkv), values(t["q_weight"]), values(t["k_weight"]), nq, nk, nv,
                          hd, chn, ppf, pph, ppw, eps, base, interleave, factor, low, high, af,
                          norm)
    qo, ko, vo = call(False)
    assert_bits_equal(vo, r.v, f"V copy {what}")
    assert_bf16(qo, r.q_exact, f"Q {what}", mag=r.q_mag)
    assert_bf16(ko, r.k_exact, f"K {what}", mag=r.k_mag)
    q8, k8, v8 = Q.qk_rmsnorm_rope_fp8(r, oscale, vscale)
    qo, ko, vo = call(True)
    assert_fp8(qo, q8.q, q8.tie, f"Q e4m3 {what}")
    assert_fp8(ko, k8.q, k8.tie, f"K e4m3 {what}")
    assert_fp8(vo, v8.q, v8.tie, f"V e4m3 {what}")


FORCED_TPR = (8, 16, 32, 64, 128, 256, 320, 448, 512, 1024)
FORCED_OPS = ("rmsnorm", "rmsnorm_quant", "fused_add", "fused_add_quant", "block_quant",
              "layernorm", "layernorm_quant", "silu_fp8", "ada", "train_forward")


@pytest.mark.parametrize("case", CASES)
def test_random_forced_row_mappings(dn, case):
    """Every forward row mapping (the test hook that forces threads per row; a mapping whose
    lanes cannot cover the row falls back to the automatic one) on a random row-engine call,
    hidden and row count, against the oracle."""
    rng = rng_of(40, case)
    tpr = int(rng.choice(FORCED_TPR))
    op = FORCED_OPS[int(rng.integers(0, len(FORCED_OPS)))]
    hidden = 128 * int(rng.integers(1, 65)) if op == "block_quant" else 8 * int(rng.integers(1, 1025))
    rows = rows_for(rng, hidden, cap=120)
    seed = 3000 + case
    x, r = W.normal((rows, hidden), seed, 0), W.normal((rows, hidden), seed, 1)
    w = W.normal((hidden,), seed, 2, mean=1.0, std=0.1)
    what = f"forced tpr {tpr} {op} case {case}: [{rows},{hidden}]"
    dn.dn_force_threads_per_row(tpr)
    try:
        if op == "rmsnorm":
            y, rstd = dn.dn_rmsnorm(dev(x), dev(w), 1e-6, return_rstd=True)
            ref = O.rmsnorm(values(x), values(w), 0.0, 1e-6)
            assert_bf16(y, ref.y_exact, what)
            assert_rstd(rstd, ref.r64, what)
        elif op == "rmsnorm_quant":
            q = dn.dn_rmsnorm_quant(dev(x), dev(w), 0.04, 1e-6)
            _, ref = O.rmsnorm_quant(values(x), values(w), 0.04, 0.0, 1e-6)
            assert_fp8(q, ref.q, ref.tie, what)
        elif op in ("fused_add", "fused_add_quant"):
            xd, rd = dev(x), dev(r)
            if op == "fused_add":
                dn.dn_fused_add_rmsnorm(xd, rd, dev(w), 1e-6)
                ref = O.fused_add_rmsnorm(values(x), values(r), values(w), 0.0, 1e-6)
                assert_bf16(xd, ref.norm.y_exact, what)
                assert_bits_equal(rd, ref.h_new, what)
            else:
                q = dn.dn_fused_add_rmsnorm_quant(xd, rd, dev(w), 0.04, 1e-6)
                fa, ref = O.fused_add_rmsnorm_quant(values(x), values(r), values(w), 0.04, 0.0, 1e-6)
                assert_bits_equal(rd, fa.h_new, what)
                assert_fp8(q, ref.q, ref.tie, what)
        elif op == "block_quant":
            rd = dev(r)
            q, bs = dn.dn_fused_add_rmsnorm_fp8_block_quant(dev(x), rd, dev(w), 1e-6)
            ref = O.fused_add_rmsnorm_fp8_block_quant(values(x), values(r), values(w), 0.0, 1e-6)
            assert_bits_equal(rd, ref.h_new, what)
            assert_block_quant(q, bs.t()[:rows], ref, what)
        elif op in ("layernorm", "layernorm_quant"):
            ga = W.normal((hidden,), seed, 7, std=0.1, dtype=torch.float32) + 1.0
            be = W.normal((hidden,), seed, 8, std=0.1, dtype=torch.float32)
            if op == "layernorm":
                y = dn.dn_layernorm(dev(x), dev(ga), dev(be), 1e-6)
                ln = L.layernorm(values(x), ga.double().numpy(), be.double().numpy(), 1e-6)
                assert_bf16(y, ln.y_exact, what, mag=ln.mag)
            else:
                q = dn.dn_layernorm_quant(dev(x), dev(ga), dev(be), 0.04, 1e-6)
                _, ref = L.layernorm_quant(values(x), ga.double().numpy(), be.double().numpy(),
                                           0.04, 1e-6)
                assert_fp8(q, ref.q, ref.tie, what)
        elif op == "silu_fp8":
            q = dn.dn_fused_rmsnorm_silu(dev(x), dev(w), 1e-6, output_fp8=True, scale=0.02)
            _, ref = S.fused_rmsnorm_silu_fp8(values(x), values(w), 0.02, 1e-6)
            assert_fp8(q, ref.q, ref.tie, what)
        elif op == "ada":
            style = W.normal((rows, 3 * hidden), seed, 3)
            out, gout = dn.dn_ada_rms_norm(dev(x), dev(w), dev(style), 1e-6)
            a, _ = O.ada_rms_norm(values(x), values(w), values(style), 1e-6)
            assert_bf16(out, a.o_exact, what, mag=a.o_mag)
            assert_bits_equal(gout, a.gate_out, what)
        else:
            wf = W.normal((hidden,), seed, 4, std=0.02, dtype=torch.float32)
            y, rstd, hn = dn.dn_train_forward(dev(x), dev(wf), 1e-6, w_bias=1.0, residual=dev(r))
            ref = O.train_forward(values(x), values(wf), 1.0, 1e-6, residual=values(r))
            assert_bits_equal(hn, ref.h_new, what)
            assert_bf16(y, ref.y_exact, what)
            assert_rstd(rstd, ref.r64, what)
    finally:
        dn.dn_force_threads_per_row(0)


LAYOUT_OPS = ("layernorm", "silu", "ada", "ada_gated_fp8", "gated_next", "sigmoid_gate",
              "train", "qk_rope")


def padded_out(shape, pad, dtype=torch.bfloat16):
    """(view, buffer): an output view with `pad` elements after every row of a buffer filled
    with a sentinel, so writes past a row show up."""
    rows, h = shape
    big = torch.full((rows, h + pad), 7.0, dtype=torch.float32, device="cuda").to(dtype)
    return big[:, :h], big


def assert_pads_untouched(buf, h, what):
    if buf.shape[1] > h:
        tail = buf[:, h:].float()
        assert bool((tail == 7.0).all()), f"{what}: a write landed in the row padding"


@pytest.mark.parametrize("case", CASES)
def test_random_layouts(dn, case):
    """Padded row strides on the inputs and the outputs of the other row engines (and 3-D
    activations where the call takes them): the results match the oracle and nothing is
    written into the padding between rows."""
    rng = rng_of(41, case)
    op = LAYOUT_OPS[int(rng.integers(0, len(LAYOUT_OPS)))]
    pad_in, pad_out = (8 * int(rng.integers(0, 5)) for _ in range(2))
    seed = 3200 + case
    what = f"layout {op} case {case}: pads {pad_in}/{pad_out}"
    if op == "qk_rope":
        ppf, pph, ppw, batch, (nq, nk, nv), hd, chn = draw_rope(rng)
        wl = W.qk_rope(ppf, pph, ppw, batch, nq, nk, nv, hd, chn, seed=seed)
        t, p = wl.tensors, wl.params
        qkv = padded(t["qkv"], pad_in)
        outs = [padded_out((qkv.shape[0], n * hd), pad_out) for n in (nq, nk, nv)]
        qo, ko, vo = dn.dn_fused_qk_rmsnorm_rope(
            qkv, dev(t["q_weight"]), dev(t["k_weight"]), nq, nk, nv, hd, ppf, pph, ppw, chn,
            p["eps"], base=p["base"], q_out=outs[0][0], k_out=outs[1][0], v_out=outs[2][0])
        r = Q.qk_rmsnorm_rope(values(t["qkv"]), values(t["q_weight"]), values(t["k_weight"]),
                              nq, nk, nv, hd, chn, ppf, pph, ppw, p["eps"], p["base"], True,
                              1.0, 0.0, 0.0, 1.0, True)
        assert_bf16(outs[0][0], r.q_exact, f"Q {what}", mag=r.q_mag)
        assert_bf16(outs[1][0], r.k_exact, f"K {what}", mag=r.k_mag)
        assert_bits_equal(outs[2][0], r.v, f"V {what}")
        for (v, buf), n in zip(outs, (nq, nk, nv)):
            assert_pads_untouched(buf, n * hd, what)
        return
    hidden = 8 * int(rng.integers(1, 769))
    rows = rows_for(rng, hidden, cap=96)
    x = W.normal((rows, hidden), seed, 0)
    w = W.normal((hidden,), seed, 2, mean=1.0, std=0.1)
    xd = padded(x, pad_in)
    if op == "layernorm":
        ga = W.normal((hidden,), seed, 7, std=0.1, dtype=torch.float32) + 1.0
        be = W.normal((hidden,), seed, 8, std=0.1, dtype=torch.float32)
        y, buf = padded_out((rows, hidden), pad_out)
        dn.dn_layernorm(xd, dev(ga), dev(be), 1e-6, out=y)
        ln = L.layernorm(values(x), ga.double().numpy(), be.double().numpy(), 1e-6)
        assert_bf16(y, ln.y_exact, what, mag=ln.mag)
        assert_pads_untouched(buf, hidden, what)
    elif op == "silu":
        y, buf = padded_out((rows, hidden), pad_out)
        dn.dn_fused_rmsnorm_silu(xd, dev(w), 1e-6, out=y)
        s = S.fused_rmsnorm_silu(values(x), values(w), 1e-6)
        assert_bf16(y, s.s_exact, what, mag=s.mag)
        assert_pads_untouched(buf, hidden, what)
    elif op in ("ada", "ada_gated_fp8"):
        style = W.normal((rows, 3 * hidden), seed, 3)
        sd = padded(style, pad_in)
        if op == "ada":
            y, buf = padded_out((rows, hidden), pad_out)
            go, gbuf = padded_out((rows, hidden), pad_out)
            dn.dn_ada_rms_norm(xd, dev(w), sd, 1e-6, out=y, gate_out=go)
            a, _ = O.ada_rms_norm(values(x), values(w), values(style), 1e-6)
            assert_bf16(y, a.o_exact, what, mag=a.o_mag)
            assert_bits_equal(go, a.gate_out, what)
            assert_pads_untouched(buf, hidden, what)
            assert_pads_untouched(gbuf, hidden, what)
        else:
            res = W.normal((rows, hidden), seed, 1)
            gate = W.normal((rows, hidden), seed, 4)
            rd = padded(res, pad_in)
            _, q, go = dn.dn_gate_residual_ada_norm_fp8(rd, xd, padded(gate, pad_in), dev(w), sd,
                                                        0.04, 1e-6)
            g, ref = O.gate_residual_ada_norm_fp8(values(res), values(x), values(gate),
                                                  values(w), values(style), 0.04, 1e-6)
            assert_bits_equal(rd, g.h, f"residual {what}")
            assert_bits_equal(go, g.gate_out, what)
            assert_fp8(q, ref.q, ref.tie, what)
    elif op == "gated_next":
        wl = W.gated_residual(rows, hidden, seed=seed, per_token_gate=True)
        t = wl.tensors
        r = padded(t["residual"], pad_in)
        y, buf = padded_out((rows, hidden), pad_out)
        dn.dn_gated_residual_next_rmsnorm(padded(t["branch"], pad_in), r, padded(t["gate"], pad_in),
                                          dev(t["w"]), dev(t["w_next"]), 1e-6, out=y)
        ref = G.gated_residual_rmsnorm(values(t["branch"]), values(t["residual"]),
                                       values(t["gate"]), values(t["w"]), 1e-6,
                                       next_w=values(t["w_next"]))
        assert_bf16(r, ref.h_exact, f"h {what}", mag=ref.h_mag)
        assert_bf16(y, ref.y_exact, f"next {what}", mag=ref.y_mag)
        assert_pads_untouched(buf, hidden, what)
    elif op == "sigmoid_gate":
        heads = int(rng.integers(1, 5))
        hd = 8 * int(rng.integers(1, 33))
        xs = W.normal((rows, heads * hd), seed, 5)
        gs = W.normal((rows, heads * hd), seed, 6, std=2.0)
        ws = W.normal((hd,), seed, 9, mean=1.0, std=0.1)
        xp = padded(xs.reshape(-1, hd), pad_in)          # head rows hd + pad apart
        dn.dn_rmsnorm_sigmoid_gate(xp, padded(gs.reshape(-1, hd), pad_in), 1e-6, weight=dev(ws))
        s = S.rmsnorm_sigmoid_gate(values(xs).reshape(-1, hd), values(gs).reshape(-1, hd),
                                   values(ws), 1e-6)
        assert_bf16(xp, s.o_exact, what, mag=s.mag)
    else:
        res = W.normal((rows, hidden), seed, 1)
        gr = W.normal((rows, hidden), seed, 3)
        wf = W.normal((hidden,), seed, 4, std=0.02, dtype=torch.float32)
        y, ybuf = padded_out((rows, hidden), pad_out)
        hn, hbuf = padded_out((rows, hidden), pad_out)
        rs = torch.empty(rows, dtype=torch.float32, device="cuda")
        dn.dn_train_forward(xd, dev(wf), 1e-6, w_bias=1.0, residual=padded(res, pad_in), out=y,
                            rstd=rs, residual_out=hn)
        fwd = O.train_forward(values(x), values(wf), 1.0, 1e-6, residual=values(res))
        assert_bits_equal(hn, fwd.h_new, f"h_new {what}")
        assert_bf16(y, fwd.y_exact, f"y {what}")
        assert_pads_untouched(ybuf, hidden, what)
        assert_pads_untouched(hbuf, hidden, what)
        g = W.normal((rows, hidden), seed, 6)
        hb = torch.from_numpy(F.f64_to_bf16_bits(fwd.h_new).view(np.int16)).view(torch.bfloat16)
        rsd = torch.from_numpy(fwd.rstd.astype(np.float32))
        dx, dxbuf = padded_out((rows, hidden), pad_out)
        dn.dn_train_backward(padded(g, pad_in), padded(hb, pad_in), dev(wf), dev(rsd), w_bias=1.0,
                             g_residual=padded(gr, pad_in), dx=dx)
        ref = O.train_backward(values(g), fwd.h_new, values(wf), rsd.double().numpy(), 1.0,
                               values(gr))
        assert_dx(dx, ref, f"dx {what}")
        assert_pads_untouched(dxbuf, hidden, what)
