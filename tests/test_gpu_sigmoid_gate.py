"""GPU parity of the per-head RMSNorm + sigmoid gate (in place) against the FP64 oracle:
BF16 within one ulp, held to the cancellation-aware bound |o| * (2 + |gate|) * 2^-21."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from oracle import silu as S
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


@pytest.mark.parametrize("weight", ["none", "bf16", "fp32+1"])
@pytest.mark.parametrize("heads,head_dim", [(4, 64), (3, 128), (2, 256), (5, 8), (1, 1024)])
def test_sigmoid_gate(dn, heads, head_dim, weight):
    wl = W.sigmoid_gate(37, heads, head_dim)
    t = wl.tensors
    w, bias = None, 0.0
    if weight == "bf16":
        w = t["w"]
    elif weight == "fp32+1":
        w, bias = W.normal((head_dim,), 80, 0, std=0.1, dtype=torch.float32), 1.0
    x = dev(t["x"]).reshape(37, heads, head_dim)
    out = dn.dn_rmsnorm_sigmoid_gate(x, dev(t["gate"]).reshape(37, heads, head_dim), 1e-6,
                                     weight=None if w is None else dev(w), w_bias=bias)
    assert out.data_ptr() == x.data_ptr()
    r = S.rmsnorm_sigmoid_gate(values(t["x"]).reshape(-1, head_dim),
                               values(t["gate"]).reshape(-1, head_dim),
                               None if w is None else values(w), 1e-6, bias)
    assert_bf16(x.reshape(-1, head_dim), r.o_exact, f"[{heads}x{head_dim}] {weight}", mag=r.mag)


def test_sigmoid_gate_wide_gates(dn):
    x = W.normal((64, 256), 81, 0)
    g = W.normal((64, 256), 81, 1, std=60.0)
    xd = dev(x).reshape(64, 4, 64)
    dn.dn_rmsnorm_sigmoid_gate(xd, dev(g).reshape(64, 4, 64), 1e-6)
    r = S.rmsnorm_sigmoid_gate(values(x).reshape(-1, 64), values(g).reshape(-1, 64), None, 1e-6)
    assert np.abs(values(g)).max() > 100
    assert_bf16(xd.reshape(-1, 64), r.o_exact, "wide gates", mag=r.mag)


def test_sigmoid_gate_full_size_sampled(dn):
    wl = W.sigmoid_gate()
    t, p = wl.tensors, wl.params
    T, Hh, hd = p["tokens"], p["heads"], p["head_dim"]
    x = dev(t["x"]).reshape(T, Hh, hd)
    dn.dn_rmsnorm_sigmoid_gate(x, dev(t["gate"]).reshape(T, Hh, hd), 1e-6, weight=dev(t["w"]))
    rows = sample_rows(T * Hh, 256, seed=3)
    xr = values(t["x"]).reshape(-1, hd)[rows]
    gr = values(t["gate"]).reshape(-1, hd)[rows]
    r = S.rmsnorm_sigmoid_gate(xr, gr, values(t["w"]), 1e-6)
    assert_bf16(rows_of(x.reshape(-1, hd), rows), r.o_exact, "full size sampled", mag=r.mag)
