"""GPU parity of the AdaRMSNorm calls (style scale/shift/gate, gated residual, static FP8),
per-row and broadcast style."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from oracle import formats as F
from oracle import rmsnorm as O
from tests.conftest import bits16, values
from tests.parity import assert_bf16, assert_bits_equal, assert_fp8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dn():
    from dit_normalization_amd import dnorm
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return dnorm


def dev(t):
    return t.to("cuda")


@pytest.mark.parametrize("broadcast", [False, True])
def test_gate_residual_ada_fp8_2520x3072(dn, broadcast):
    wl = W.ada(broadcast=broadcast)
    t = wl.tensors
    rd = dev(t["residual"])
    res, q, gout = dn.dn_gate_residual_ada_norm_fp8(rd, dev(t["x"]), dev(t["gate"]), dev(t["w"]),
                                                     dev(t["style"]), wl.params["scale"], 1e-6)
    a, ref = O.gate_residual_ada_norm_fp8(values(t["residual"]), values(t["x"]), values(t["gate"]),
                                          values(t["w"]), values(t["style"]), 0.04, 1e-6)
    assert_bits_equal(rd, a.h, "residual (bit-exact)")
    assert_bits_equal(gout, a.gate_out, "gate_out (bit-exact)")
    assert_fp8(q, ref.q, ref.tie, "Ada FP8 out")


@pytest.mark.parametrize("broadcast", [False, True])
@pytest.mark.parametrize("rows,dim", [(2520, 3072), (37, 64), (9, 264), (65, 1024), (5, 4096),
                                      (9, 4608), (7, 7168), (3, 8192)])
def test_ada_rms_norm_bf16(dn, rows, dim, broadcast):
    wl = W.ada(rows=rows, dim=dim, broadcast=broadcast)
    t = wl.tensors
    w = W.normal((dim,), 5, 9, mean=1.0, std=0.1)
    out, gout = dn.dn_ada_rms_norm(dev(t["x"]), dev(w), dev(t["style"]), 1e-6)
    a, ref = O.ada_rms_norm(values(t["x"]), values(w), values(t["style"]), 1e-6)
    assert_bf16(out, a.o_exact, f"Ada BF16 [{rows},{dim}]", mag=a.o_mag)
    assert_bits_equal(gout, a.gate_out, "gate_out")


@pytest.mark.parametrize("rows,dim", [(37, 64), (9, 264), (65, 1024), (5, 4096)])
def test_gate_residual_small_shapes(dn, rows, dim):
    wl = W.ada(rows=rows, dim=dim)
    t = wl.tensors
    rd = dev(t["residual"])
    _, q, gout = dn.dn_gate_residual_ada_norm_fp8(rd, dev(t["x"]), dev(t["gate"]), dev(t["w"]),
                                                   dev(t["style"]), 0.04, 1e-6)
    a, ref = O.gate_residual_ada_norm_fp8(values(t["residual"]), values(t["x"]), values(t["gate"]),
                                          values(t["w"]), values(t["style"]), 0.04, 1e-6)
    assert_bits_equal(rd, a.h, "residual")
    assert_fp8(q, ref.q, ref.tie, f"Ada FP8 [{rows},{dim}]")


def test_broadcast_equals_repeated_style(dn):
    wl = W.ada(rows=100, dim=3072, broadcast=True)
    t = wl.tensors
    rep = t["style"].repeat(100, 1)
    r1, r2 = dev(t["residual"]), dev(t["residual"])
    _, q1, g1 = dn.dn_gate_residual_ada_norm_fp8(r1, dev(t["x"]), dev(t["gate"]), dev(t["w"]),
                                                 dev(t["style"]), 0.04)
    _, q2, g2 = dn.dn_gate_residual_ada_norm_fp8(r2, dev(t["x"]), dev(t["gate"]), dev(t["w"]),
                                                 dev(rep), 0.04)
    assert torch.equal(q1.view(torch.uint8), q2.view(torch.uint8))
    assert torch.equal(g1.view(torch.int16), g2.view(torch.int16))
