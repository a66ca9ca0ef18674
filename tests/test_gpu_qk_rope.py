"""GPU parity of the fused QK RMSNorm + 3-D RoPE + V copy against the FP64 oracle.

Gates: V bit-exact (BF16) or FP8 codes equal except at flagged ties; Q and K within one
BF16 ulp, held to the cancellation-aware bound with the rotation's term magnitude
(|a| + |b|) * attention_factor of each pair."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from oracle import qk_rope as Q
from tests.conftest import values
from tests.parity import assert_bf16, assert_bits_equal, assert_fp8, rows_of, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dn():
    from dit_normalization_amd import dnorm
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return dnorm


def dev(t):
    return t.to("cuda")


def run(dn, wl, interleave=True, factor=1.0, low=0.0, high=0.0, af=1.0, norm=True, fp8=False,
        weights=None, qkv=None):
    t, p = wl.tensors, wl.params
    wq, wk = weights if weights is not None else (t["q_weight"], t["k_weight"])
    x = dev(t["qkv"]) if qkv is None else qkv
    return dn.dn_fused_qk_rmsnorm_rope(
        x, dev(wq), dev(wk), p["nq"], p["nk"], p["nv"], p["head_dim"], p["ppf"], p["pph"],
        p["ppw"], p["channels"], p["eps"], base=p["base"], interleave=interleave,
        yarn_factor=factor, yarn_low=low, yarn_high=high, attention_factor=af,
        is_qk_norm=norm, output_fp8=fp8, output_quant_scale=p["output_scale"],
        v_quant_scale=p["v_scale"])


def oracle(wl, interleave=True, factor=1.0, low=0.0, high=0.0, af=1.0, norm=True, rows=None,
           weights=None):
    t, p = wl.tensors, wl.params
    wq, wk = weights if weights is not None else (t["q_weight"], t["k_weight"])
    x = values(t["qkv"])
    r = Q.qk_rmsnorm_rope(x, values(wq), values(wk), p["nq"], p["nk"], p["nv"], p["head_dim"],
                          p["channels"], p["ppf"], p["pph"], p["ppw"], p["eps"], p["base"],
                          interleave, factor, low, high, af, norm)
    return r


def check_bf16(outs, r, what, rows=None):
    qo, ko, vo = outs
    sel = (lambda a: a) if rows is None else (lambda a: a[rows])
    got = (lambda t: t) if rows is None else (lambda t: rows_of(t, rows))
    assert_bits_equal(got(vo), sel(r.v), f"{what}: V copy")
    assert_bf16(got(qo), sel(r.q_exact), f"{what}: Q", mag=sel(r.q_mag))
    assert_bf16(got(ko), sel(r.k_exact), f"{what}: K", mag=sel(r.k_mag))


SHAPES = [  # (ppf, pph, ppw, batch, nq, nk, nv, head_dim, channels)
    (3, 4, 5, 2, 24, 24, 24, 128, (44, 42, 42)),
    (2, 3, 2, 3, 2, 1, 3, 64, (24, 20, 20)),
    (2, 2, 3, 2, 4, 4, 4, 256, (86, 84, 86)),
    (4, 3, 2, 1, 1, 1, 1, 64, (64, 0, 0)),
    (2, 2, 2, 2, 32, 32, 32, 256, (88, 84, 84)),
    (5, 1, 1, 4, 8, 2, 2, 128, (0, 0, 128)),
]


@pytest.mark.parametrize("interleave", [True, False])
@pytest.mark.parametrize("shape", SHAPES)
def test_qk_rope_bf16(dn, shape, interleave):
    ppf, pph, ppw, b, nq, nk, nv, hd, ch = shape
    wl = W.qk_rope(ppf, pph, ppw, b, nq, nk, nv, hd, ch)
    outs = run(dn, wl, interleave)
    check_bf16(outs, oracle(wl, interleave), f"{shape} interleave={interleave}")


@pytest.mark.parametrize("interleave", [True, False])
def test_qk_rope_yarn_and_attention_factor(dn, interleave):
    wl = W.qk_rope(4, 5, 6, 1, 6, 6, 6, 128, (44, 42, 42))
    outs = run(dn, wl, interleave, factor=4.0, low=3.0, high=12.0, af=1.3)
    check_bf16(outs, oracle(wl, interleave, 4.0, 3.0, 12.0, 1.3), "yarn")
    outs = run(dn, wl, interleave, factor=2.0, low=5.0, high=5.0, af=0.9)
    check_bf16(outs, oracle(wl, interleave, 2.0, 5.0, 5.0, 0.9), "yarn step")


@pytest.mark.parametrize("interleave", [True, False])
def test_qk_rope_without_norm(dn, interleave):
    wl = W.qk_rope(3, 4, 5, 1, 4, 2, 2, 128, (44, 42, 42))
    outs = run(dn, wl, interleave, norm=False)
    check_bf16(outs, oracle(wl, interleave, norm=False), "no norm")


@pytest.mark.parametrize("interleave", [True, False])
def test_qk_rope_fp8(dn, interleave):
    wl = W.qk_rope(3, 4, 5, 2, 24, 24, 24, 128, (44, 42, 42))
    qo, ko, vo = run(dn, wl, interleave, fp8=True)
    r = oracle(wl, interleave)
    q8, k8, v8 = Q.qk_rmsnorm_rope_fp8(r, wl.params["output_scale"], wl.params["v_scale"])
    assert_fp8(qo, q8.q, q8.tie, "Q e4m3")
    assert_fp8(ko, k8.q, k8.tie, "K e4m3")
    assert_fp8(vo, v8.q, v8.tie, "V e4m3")


@pytest.mark.parametrize("interleave", [True, False])
def test_qk_rope_fp8_saturation(dn, interleave):
    """e4m3 outputs beyond +-448 saturate.  Tokens 0..9 carry a spike in head 0 of Q and
    of K (normalised to ~11, past 448 after the rotation at scale 0.02) and in V (50 at
    V scale 0.02); the other tokens stay in range, so both sides of the kernel's in-range
    vote run."""
    wl = W.qk_rope(3, 4, 5, 2, 24, 24, 24, 128, (44, 42, 42))
    wl.params["output_scale"] = 0.02
    qkv = wl.tensors["qkv"]
    qkv[:10, 5] = 60.0
    qkv[:10, 24 * 128 + 3] = 60.0
    qkv[:10, 48 * 128 + 7] = 50.0
    qo, ko, vo = run(dn, wl, interleave, fp8=True)
    r = oracle(wl, interleave)
    q8, k8, v8 = Q.qk_rmsnorm_rope_fp8(r, wl.params["output_scale"], wl.params["v_scale"])
    for ref in (q8, k8, v8):
        sat = ((ref.q.astype(np.int64) & 0x7F) == 0x7E).any(axis=1)
        assert sat[:10].all() and not sat[10:].any()
    assert_fp8(qo, q8.q, q8.tie, "Q e4m3 saturation")
    assert_fp8(ko, k8.q, k8.tie, "K e4m3 saturation")
    assert_fp8(vo, v8.q, v8.tie, "V e4m3 saturation")


def test_qk_rope_fp32_weights_and_3d_input(dn):
    wl = W.qk_rope(2, 3, 4, 2, 4, 4, 4, 128, (44, 42, 42))
    t, p = wl.tensors, wl.params
    wq = t["q_weight"].float()
    wk = t["k_weight"].float()
    x3 = dev(t["qkv"]).reshape(2, 24, -1)
    qo, ko, vo = run(dn, wl, weights=(wq, wk), qkv=x3)
    assert qo.shape == (2, 24, 4 * 128)
    r = oracle(wl, weights=(wq, wk))
    check_bf16((qo.reshape(48, -1), ko.reshape(48, -1), vo.reshape(48, -1)), r, "3-D, FP32 w")


def test_qk_rope_strided_rows_and_empty(dn):
    wl = W.qk_rope(2, 3, 4, 1, 2, 2, 2, 64, (24, 20, 20))
    t = wl.tensors
    width = 6 * 64
    big = torch.zeros((24, width + 64), dtype=torch.bfloat16, device="cuda")
    big[:, :width] = dev(t["qkv"])
    outs = run(dn, wl, qkv=big[:, :width])
    check_bf16(outs, oracle(wl), "strided qkv")
    e = torch.empty((0, width), dtype=torch.bfloat16, device="cuda")
    qo, ko, vo = run(dn, wl, qkv=e)
    assert qo.shape == (0, 128) and vo.shape == (0, 128)


@pytest.mark.parametrize("interleave", [True, False])
def test_qk_rope_full_size_sampled(dn, interleave):
    """The measured workload (12288 tokens x 72 heads of 128): sampled rows."""
    wl = W.qk_rope()
    outs = run(dn, wl, interleave)
    rows = sample_rows(wl.params["tokens"], 48, seed=9)
    t, p = wl.tensors, wl.params
    x = values(t["qkv"][torch.as_tensor(rows)])
    r = Q.qk_rmsnorm_rope(x, values(t["q_weight"]), values(t["k_weight"]), p["nq"], p["nk"],
                          p["nv"], p["head_dim"], p["channels"], p["ppf"], p["pph"], p["ppw"],
                          p["eps"], p["base"], interleave, token_ids=rows)
    qo, ko, vo = outs
    check_bf16((rows_of(qo, rows), rows_of(ko, rows), rows_of(vo, rows)), r, "full size")
