"""GPU parity of the training forward and backward (dx, deterministic dw)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from oracle import formats as F
from oracle import rmsnorm as O
from tests.conftest import bits16, values
from tests.parity import (assert_bf16, assert_bits_equal, assert_dw, assert_dx, assert_rstd,
                          rows_of, sample_rows)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dn():
    from dit_normalization_amd import dnorm
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return dnorm


def dev(t):
    return t.to("cuda")


def bf16_tensor(v: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(F.f64_to_bf16_bits(v).view(np.int16)).view(torch.bfloat16)


def backward_inputs(t, chunk: int = 2048):
    """The backward's inputs as the oracle's forward makes them: h_new = BF16(h + residual)
    and the FP32 rstd (computed in row chunks for large inputs).  Both the kernel and the
    oracle backward take these, so the backward is checked on its own."""
    hs, rs = [], []
    w = values(t["w"])
    for s in range(0, t["h"].shape[0], chunk):
        f = O.train_forward(values(t["h"][s:s + chunk]), w, 1.0, 1e-6,
                            residual=values(t["residual"][s:s + chunk]))
        hs.append(bf16_tensor(f.h_new))
        rs.append(torch.from_numpy(f.rstd.astype(np.float32)))
    return torch.cat(hs), torch.cat(rs)


def dw_oracle(g, x, rstd, w, chunk: int = 1024):
    """dw over all rows: the oracle's FP64 column sums, accumulated over row chunks."""
    total = np.zeros(x.shape[1])
    r = rstd.double().numpy()
    for s in range(0, x.shape[0], chunk):
        total += O.train_backward(values(g[s:s + chunk]), values(x[s:s + chunk]), values(w),
                                  r[s:s + chunk], 1.0).dw_exact
    return total


@pytest.mark.parametrize("rows,hidden", [(257, 8192), (1, 512), (2, 2048), (7, 6144), (63, 64),
                                         (129, 1024), (65, 128), (31, 16384), (9, 5120),
                                         (11, 7168)])
def test_train_forward_residual_fp32_weight(dn, rows, hidden):
    wl = W.train(rows=rows, hidden=hidden)
    t = wl.tensors
    y, rstd, h = dn.dn_train_forward(dev(t["h"]), dev(t["w"]), 1e-6, w_bias=1.0,
                                     residual=dev(t["residual"]))
    ref = O.train_forward(values(t["h"]), values(t["w"]), 1.0, 1e-6, residual=values(t["residual"]))
    assert_bits_equal(h, ref.h_new, "h_new")
    assert_bf16(y, ref.y_exact, "y")
    assert_rstd(rstd, ref.r64)


def test_train_forward_plain_bf16_weight(dn):
    x = W.normal((200, 4096), 30, 0)
    w = W.normal((4096,), 30, 1, mean=1.0, std=0.1)
    y, rstd = dn.dn_train_forward(dev(x), dev(w), 1e-6)
    ref = O.train_forward(values(x), values(w), 0.0, 1e-6)
    assert_bf16(y, ref.y_exact, "y")
    assert_rstd(rstd, ref.r64)


@pytest.mark.parametrize("rows,hidden", [(257, 8192), (1, 512), (2, 2048), (7, 6144), (63, 64),
                                         (129, 1024), (65, 128), (300, 8), (31, 16384),
                                         (9, 32768), (1000, 256), (513, 4096),
                                         (37, 1032), (300, 3072), (45, 5128)])
def test_train_backward_against_oracle(dn, rows, hidden):
    wl = W.train(rows=rows, hidden=hidden)
    t = wl.tensors
    h, rstd = backward_inputs(t)
    dx, dw = dn.dn_train_backward(dev(t["g"]), dev(h), dev(t["w"]), dev(rstd), w_bias=1.0)
    ref = O.train_backward(values(t["g"]), values(h), values(t["w"]), rstd.double().numpy(), 1.0)
    assert_dx(dx, ref, f"dx [{rows},{hidden}]")
    assert_dw(dw, ref.dw_exact, f"dw [{rows},{hidden}]")


@pytest.mark.parametrize("rows,hidden", [(100, 2048), (77, 4096), (259, 8192)])
def test_train_backward_g_residual(dn, rows, hidden):
    """The residual gradient on each row-group layout (four 64-lane, four 128-lane and two
    256-lane groups per block), with chunks whose rows do not divide among the groups."""
    wl = W.train(rows=rows, hidden=hidden)
    t = wl.tensors
    h, rstd = backward_inputs(t)
    gres = W.normal((rows, hidden), 31, 0)
    dx, dw = dn.dn_train_backward(dev(t["g"]), dev(h), dev(t["w"]), dev(rstd), w_bias=1.0,
                                  g_residual=dev(gres))
    ref = O.train_backward(values(t["g"]), values(h), values(t["w"]), rstd.double().numpy(), 1.0,
                           values(gres))
    assert_dx(dx, ref, "dx with g_residual")
    assert_dw(dw, ref.dw_exact, "dw with g_residual")


def test_dw_is_bitwise_reproducible_and_workspace_reusable(dn):
    wl = W.train(rows=3000, hidden=4096)
    t = wl.tensors
    h, rstd = (dev(a) for a in backward_inputs(t))
    g, w = dev(t["g"]), dev(t["w"])
    ws = dn.train_backward_workspace(4096, "cuda")
    first_dx, first_dw = dn.dn_train_backward(g, h, w, rstd, w_bias=1.0, workspace=ws)
    first_dx, first_dw = first_dx.clone(), first_dw.clone()
    for i in range(10):
        # A call with another token count in between reuses the same workspace.
        dn.dn_train_backward(g[:777], h[:777], w, rstd[:777], w_bias=1.0, workspace=ws)
        dx, dw = dn.dn_train_backward(g, h, w, rstd, w_bias=1.0, workspace=ws)
        assert torch.equal(dw.view(torch.int32), first_dw.view(torch.int32)), f"dw bits moved (run {i})"
        assert torch.equal(dx.view(torch.int16), first_dx.view(torch.int16)), f"dx bits moved (run {i})"


def test_split_stages_equal_the_combined_call(dn):
    wl = W.train(rows=600, hidden=8192)
    t = wl.tensors
    h, rstd = (dev(a) for a in backward_inputs(t))
    g, w = dev(t["g"]), dev(t["w"])
    dx1, dw1 = dn.dn_train_backward(g, h, w, rstd, w_bias=1.0)
    ws = dn.train_backward_workspace(8192, "cuda")
    dx2 = dn.dn_train_backward_partials(g, h, w, rstd, ws, w_bias=1.0)
    dw2 = dn.dn_train_backward_reduce(ws, 600, 8192)
    assert torch.equal(dx1.view(torch.int16), dx2.view(torch.int16))
    assert torch.equal(dw1.view(torch.int32), dw2.view(torch.int32))


def test_dx_rows_do_not_depend_on_token_count(dn):
    wl = W.train(rows=2048, hidden=8192)
    t = wl.tensors
    h, rstd = (dev(a) for a in backward_inputs(t))
    g, w = dev(t["g"]), dev(t["w"])
    full, _ = dn.dn_train_backward(g, h, w, rstd, w_bias=1.0)
    for n in [1, 5, 300]:
        part, _ = dn.dn_train_backward(g[:n], h[:n], w, rstd[:n], w_bias=1.0)
        assert torch.equal(part.view(torch.int16), full[:n].view(torch.int16)), f"T={n}"


def test_train_16384x8192(dn):
    wl = W.train()
    t = wl.tensors
    y, rstd, hnew = dn.dn_train_forward(dev(t["h"]), dev(t["w"]), 1e-6, w_bias=1.0,
                                        residual=dev(t["residual"]))
    s = sample_rows(16384)
    ref = O.train_forward(values(t["h"][s]), values(t["w"]), 1.0, 1e-6,
                          residual=values(t["residual"][s]))
    assert_bits_equal(rows_of(hnew, s), ref.h_new, "h_new")
    assert_bf16(rows_of(y, s), ref.y_exact, "y")
    assert_rstd(rows_of(rstd, s), ref.r64)
    del y, rstd, hnew
    h, rs = backward_inputs(t)
    hd, rsd, gd, wd = dev(h), dev(rs), dev(t["g"]), dev(t["w"])
    dx, dw = dn.dn_train_backward(gd, hd, wd, rsd, w_bias=1.0)
    refb = O.train_backward(values(t["g"][s]), values(h[s]), values(t["w"]),
                            rs.double().numpy()[s], 1.0)
    assert_dx(rows_of(dx, s), refb, "dx [16384,8192]")
    assert_dw(dw, dw_oracle(t["g"], h, rs, t["w"]), "dw [16384,8192]")
    dw_again = dn.dn_train_backward(gd, hd, wd, rsd, w_bias=1.0)[1]
    assert torch.equal(dw.view(torch.int32), dw_again.view(torch.int32))


@pytest.mark.parametrize("rows,hidden", [(2048, 8192), (1, 520), (255, 64), (257, 8192),
                                         (3000, 4096), (40, 24576)])
def test_backward_equals_its_two_launches_and_bf16_dw(dn, rows, hidden):
    """dn_train_backward gives the bits of its two launches called apart (partials, then the
    reduction), FP32 and BF16 dw (the BF16 dw is the FP32 dw rounded once more, checked with
    the oracle's codec); dw against the oracle."""
    wl = W.train(rows=rows, hidden=hidden)
    t = wl.tensors
    h, rstd = backward_inputs(t)
    g, hd, w, rs = dev(t["g"]), dev(h), dev(t["w"]), dev(rstd)
    dx1, dw1 = dn.dn_train_backward(g, hd, w, rs, w_bias=1.0)
    ws2 = dn.train_backward_workspace(hidden, "cuda")
    dx2 = dn.dn_train_backward_partials(g, hd, w, rs, ws2, w_bias=1.0)
    dw2 = dn.dn_train_backward_reduce(ws2, rows, hidden)
    assert torch.equal(dx1.view(torch.int16), dx2.view(torch.int16))
    assert torch.equal(dw1.view(torch.int32), dw2.view(torch.int32))
    ref = O.train_backward(values(t["g"]), values(h), values(t["w"]), rstd.double().numpy(), 1.0)
    assert_dw(dw1, ref.dw_exact, f"dw [{rows},{hidden}]")
    _, dwb = dn.dn_train_backward(g, hd, w, rs, w_bias=1.0, dw_dtype=torch.bfloat16)
    assert dwb.dtype == torch.bfloat16
    assert (bits16(dwb) == F.f64_to_bf16_bits(dw1.cpu().double().numpy())).all()
    dwb2 = dn.dn_train_backward_reduce(ws2, rows, hidden, dw_dtype=torch.bfloat16)
    assert torch.equal(dwb.view(torch.int16), dwb2.view(torch.int16))
