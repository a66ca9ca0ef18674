"""GPU parity at the edges of the BF16 range: rows whose squares overflow FP32 (|x| ~ 1e20
.. 1e30) or underflow it (|x| ~ 1e-30, with eps = 0 so that nothing hides the loss), mixed
with ordinary rows inside one wave.  These rows take the kernels' FP64 sum of squares; the
results are held to the same gates as everywhere else, against the FP64 oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from oracle import gated as G
from oracle import qk_rope as Q
from oracle import rmsnorm as O
from oracle import silu as S
from tests.conftest import values
from tests.parity import assert_bf16, assert_bits_equal, assert_rstd

pytestmark = pytest.mark.gpu

SCALES = (1e-30, 1e-12, 1.0, 1e20, 1e30)


@pytest.fixture(scope="module")
def dn():
    from dit_normalization_amd import dnorm
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return dnorm


def dev(t):
    return t.to("cuda")


def scaled(shape, seed, tid, scales=SCALES):
    """BF16 N(0,1) rows times a per-row scale that cycles through `scales`."""
    base = W.normal(shape, seed, tid).float()
    s = torch.tensor([scales[i % len(scales)] for i in range(shape[0])], dtype=torch.float32)
    return (base * s.view(-1, *([1] * (len(shape) - 1)))).to(torch.bfloat16)


@pytest.mark.parametrize("eps", [1e-6, 0.0])
@pytest.mark.parametrize("hidden", [64, 1024, 3072, 4096, 8192])
def test_rmsnorm_rows_of_every_magnitude(dn, hidden, eps):
    x = scaled((40, hidden), 301, hidden)
    w = W.normal((hidden,), 302, hidden, mean=1.0, std=0.2)
    y, rstd = dn.dn_rmsnorm(dev(x), dev(w), eps, return_rstd=True)
    ref = O.rmsnorm(values(x), values(w), 0.0, eps)
    assert np.isfinite(ref.r64).all()
    assert_bf16(y, ref.y_exact, f"rmsnorm H={hidden} eps={eps}")
    assert_rstd(rstd, ref.r64, f"rstd H={hidden} eps={eps}")


@pytest.mark.parametrize("hidden", [128, 4096])
def test_fused_add_and_training_forward_with_huge_rows(dn, hidden):
    x = scaled((30, hidden), 303, 0)
    r = scaled((30, hidden), 303, 1)
    w = W.normal((hidden,), 303, 2, mean=1.0, std=0.1)
    xd, rd = dev(x), dev(r)
    rstd = torch.empty(30, dtype=torch.float32, device="cuda")
    dn.dn_fused_add_rmsnorm(xd, rd, dev(w), 0.0, rstd=rstd)
    ref = O.fused_add_rmsnorm(values(x), values(r), values(w), 0.0, 0.0)
    assert_bits_equal(rd, ref.h_new, "h_new")
    assert_bf16(xd, ref.norm.y_exact, "y")
    assert_rstd(rstd, ref.norm.r64)
    w32 = W.normal((hidden,), 303, 3, std=0.02, dtype=torch.float32)
    y, rs, h = dn.dn_train_forward(dev(x), dev(w32), 0.0, w_bias=1.0, residual=dev(r))
    tf = O.train_forward(values(x), values(w32), 1.0, 0.0, residual=values(r))
    assert_bits_equal(h, tf.h_new, "training h_new")
    assert_bf16(y, tf.y_exact, "training y")
    assert_rstd(rs, tf.r64, "training rstd")


@pytest.mark.parametrize("next_norm", [False, True])
def test_gated_residual_with_huge_and_tiny_streams(dn, next_norm):
    rows, hidden = 25, 8192
    b = scaled((rows, hidden), 304, 0)
    r = scaled((rows, hidden), 304, 1, scales=(1e30, 1.0, 1e-30, 1e20, 1e-12))
    g = W.normal((rows, hidden), 304, 2, std=0.5)
    w, w2 = W.normal((hidden,), 304, 3, mean=1.0, std=0.1), W.normal((hidden,), 304, 4)
    rd = dev(r)
    if next_norm:
        _, y = dn.dn_gated_residual_next_rmsnorm(dev(b), rd, dev(g), dev(w), dev(w2), 0.0)
    else:
        dn.dn_gated_residual_rmsnorm(dev(b), rd, dev(g), dev(w), 0.0)
    ref = G.gated_residual_rmsnorm(values(b), values(r), values(g), values(w), 0.0,
                                   next_w=values(w2) if next_norm else None)
    assert_bf16(rd, ref.h_exact, "h", mag=ref.h_mag)
    if next_norm:
        assert_bf16(y, ref.y_exact, "next norm", mag=ref.y_mag)


@pytest.mark.parametrize("interleave", [True, False])
def test_qk_rope_with_huge_and_tiny_tokens(dn, interleave):
    wl = W.qk_rope(2, 3, 2, 2, 4, 2, 2, 128, (44, 42, 42))
    t, p = wl.tensors, wl.params
    qkv = scaled(tuple(t["qkv"].shape), 305, 0)
    q, k, v = dn.dn_fused_qk_rmsnorm_rope(
        dev(qkv), dev(t["q_weight"]), dev(t["k_weight"]), p["nq"], p["nk"], p["nv"],
        p["head_dim"], p["ppf"], p["pph"], p["ppw"], p["channels"], 0.0, base=p["base"],
        interleave=interleave)
    r = Q.qk_rmsnorm_rope(values(qkv), values(t["q_weight"]), values(t["k_weight"]), p["nq"],
                          p["nk"], p["nv"], p["head_dim"], p["channels"], p["ppf"], p["pph"],
                          p["ppw"], 0.0, p["base"], interleave)
    assert_bits_equal(v, r.v, "V copy")
    assert_bf16(q, r.q_exact, "Q", mag=r.q_mag)
    assert_bf16(k, r.k_exact, "K", mag=r.k_mag)


@pytest.mark.parametrize("hidden", [128, 512])
def test_rmsnorm_silu_with_huge_and_tiny_rows(dn, hidden):
    x = scaled((45, hidden), 306, 0)
    w = W.normal((hidden,), 306, 1, mean=1.0, std=0.1)
    out = dn.dn_fused_rmsnorm_silu(dev(x), dev(w), 0.0)
    r = S.fused_rmsnorm_silu(values(x), values(w), 0.0)
    assert_bf16(out, r.s_exact, f"silu H={hidden}", mag=r.mag)
