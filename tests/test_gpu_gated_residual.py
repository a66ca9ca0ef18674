"""GPU parity of the gated-residual RMSNorm (and the next RMSNorm in the same launch)
against the FP64 oracle.  The new stream h and the next norm's output are held to one BF16
ulp (h with the cancellation-aware bound of |residual| + |gate * n|; the next norm may move
one ulp where the two sides' BF16 streams differ at a rounding tie)."""
from __future__ import annotations

import pytest
import torch

import workloads as W
from oracle import gated as G
from tests.conftest import values
from tests.parity import assert_bf16, rows_of, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dn():
    from dit_normalization_amd import dnorm
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return dnorm


def dev(t):
    return t.to("cuda")


@pytest.mark.parametrize("next_norm", [False, True])
@pytest.mark.parametrize("per_token", [True, False])
@pytest.mark.parametrize("rows,hidden", [(37, 8192), (5, 4096), (65, 64), (9, 264), (3, 1024),
                                         (6, 5120), (5, 7168), (2, 16384), (2, 24576)])
def test_gated_residual(dn, rows, hidden, per_token, next_norm):
    wl = W.gated_residual(rows, hidden, per_token_gate=per_token)
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
    assert_bf16(r, ref.h_exact, f"h [{rows},{hidden}]", mag=ref.h_mag)
    if next_norm:
        assert_bf16(y, ref.y_exact, f"next [{rows},{hidden}]", mag=ref.y_mag)


def test_gated_residual_fp32_weights_and_biases(dn):
    wl = W.gated_residual(33, 2048)
    t = wl.tensors
    w = W.normal((2048,), 90, 0, std=0.1, dtype=torch.float32)
    w2 = W.normal((2048,), 90, 1, std=0.1, dtype=torch.float32)
    r = dev(t["residual"])
    _, y = dn.dn_gated_residual_next_rmsnorm(dev(t["branch"]), r, dev(t["gate"]), dev(w),
                                             dev(w2), 1e-6, w_bias=1.0, w_next_bias=1.0)
    ref = G.gated_residual_rmsnorm(values(t["branch"]), values(t["residual"]), values(t["gate"]),
                                   values(w), 1e-6, bias=1.0, next_w=values(w2), next_bias=1.0)
    assert_bf16(r, ref.h_exact, "h, FP32 w + 1", mag=ref.h_mag)
    assert_bf16(y, ref.y_exact, "next, FP32 w + 1", mag=ref.y_mag)


def test_gated_residual_full_size_sampled(dn):
    wl = W.gated_residual()
    t, p = wl.tensors, wl.params
    r = dev(t["residual"])
    _, y = dn.dn_gated_residual_next_rmsnorm(dev(t["branch"]), r, dev(t["gate"]), dev(t["w"]),
                                             dev(t["w_next"]), 1e-6)
    rows = sample_rows(p["rows"], 64, seed=11)
    sel = lambda k: values(t[k][torch.as_tensor(rows)])
    ref = G.gated_residual_rmsnorm(sel("branch"), sel("residual"), sel("gate"), values(t["w"]),
                                   1e-6, next_w=values(t["w_next"]))
    assert_bf16(rows_of(r, rows), ref.h_exact, "h sampled", mag=ref.h_mag)
    assert_bf16(rows_of(y, rows), ref.y_exact, "next sampled", mag=ref.y_mag)
