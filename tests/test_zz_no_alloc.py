"""The allocation-free backward entry point (dn_train_backward_noalloc), called through the
C ABI: its dx and dw equal those of dn_train_backward with a workspace, bit for bit, on two
calls in a row (the second with fewer rows and a narrower hidden, so the scratch holds
the first call's chunk rows when the second starts), FP32 and BF16 dw; hidden beyond the
scratch is refused before any launch."""
from __future__ import annotations

import ctypes

import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dn():
    from dit_normalization_amd import dnorm
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return dnorm


def _inputs(rows, hidden, seed):
    wl = W.train(rows=rows, hidden=hidden, seed=seed)
    g, h, w = (wl.tensors[k].cuda() for k in ("g", "h", "w"))
    rstd = (1.0 / torch.sqrt(h.float().pow(2).mean(1) + 1e-6)).contiguous()
    return g, h, w, rstd


def _noalloc(dn, g, x, w, rstd, dw_code):
    rows, hidden = x.shape
    dx = torch.empty_like(x)
    dw = torch.empty(hidden, dtype=torch.float32 if dw_code == 1 else torch.bfloat16,
                     device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    rc = dn.lib.dn_train_backward_noalloc(
        ctypes.c_void_p(dx.data_ptr()), hidden, ctypes.c_void_p(dw.data_ptr()), dw_code,
        ctypes.c_void_p(g.data_ptr()), hidden, ctypes.c_void_p(x.data_ptr()), hidden,
        ctypes.c_void_p(w.data_ptr()), 1, 1.0, ctypes.c_void_p(rstd.data_ptr()), None, 0,
        rows, hidden, ctypes.c_void_p(st))
    assert rc == 0, dn.lib.dn_last_error()
    return dx, dw


@pytest.mark.parametrize("dw_code", [1, 0])
def test_noalloc_matches_the_workspace_entry_point(dn, dw_code):
    dt = torch.float32 if dw_code == 1 else torch.bfloat16
    for rows, hidden, seed in ((4096, 8192, 61), (333, 2048, 62)):
        g, h, w, rstd = _inputs(rows, hidden, seed)
        dx, dw = _noalloc(dn, g, h, w, rstd, dw_code)
        ref_dx, ref_dw = dn.dn_train_backward(g, h, w, rstd, w_bias=1.0, dw_dtype=dt)
        torch.cuda.synchronize()
        assert torch.equal(dx.view(torch.int16), ref_dx.view(torch.int16)), (rows, hidden)
        assert torch.equal(dw.view(torch.int16 if dw_code == 0 else torch.int32),
                           ref_dw.view(torch.int16 if dw_code == 0 else torch.int32)), \
            (rows, hidden)


def test_noalloc_refuses_hidden_beyond_its_scratch(dn):
    rc = dn.lib.dn_train_backward_noalloc(None, 16384, None, 1, None, 16384, None, 16384,
                                          None, 1, 1.0, None, None, 0, 4, 16384, None)
    assert rc == -6 and b"scratch" in dn.lib.dn_last_error()


@pytest.mark.parametrize("case", range(8))
def test_noalloc_random_calls_in_a_row(dn, case):
    """Seeded random pairs of calls (rows, hidden up to the scratch's 8192, with or without a
    residual gradient, FP32 or BF16 dw, FP32 or BF16 weights), each through the binding's
    allocation-free entry point, bit for bit against the workspace entry point; the second
    call of a pair runs on the scratch the first left behind."""
    import numpy as np
    rng = np.random.default_rng(8000 + case)
    for k in range(2):
        hidden = 8 * int(rng.integers(1, 1025))
        rows = int(rng.integers(1, max(2, min(3000, (1 << 22) // hidden)) + 1))
        gres, bf16_dw, f32w = (bool(rng.integers(0, 2)) for _ in range(3))
        wl = W.train(rows=rows, hidden=hidden, seed=8100 + 2 * case + k)
        g, h = wl.tensors["g"].cuda(), wl.tensors["h"].cuda()
        w = wl.tensors["w"].cuda() if f32w else \
            W.normal((hidden,), 8100 + case, 5, mean=1.0, std=0.1).cuda()
        bias = 1.0 if f32w else 0.0
        rstd = (1.0 / torch.sqrt(h.float().pow(2).mean(1) + 1e-6)).contiguous()
        gr = W.normal((rows, hidden), 8100 + case, 6).cuda() if gres else None
        dt = torch.bfloat16 if bf16_dw else torch.float32
        dx, dw = dn.dn_train_backward_noalloc(g, h, w, rstd, w_bias=bias, g_residual=gr,
                                              dw_dtype=dt)
        ref_dx, ref_dw = dn.dn_train_backward(g, h, w, rstd, w_bias=bias, g_residual=gr,
                                              dw_dtype=dt)
        torch.cuda.synchronize()
        what = (case, k, rows, hidden, gres, bf16_dw, f32w)
        assert torch.equal(dx.view(torch.int16), ref_dx.view(torch.int16)), what
        iv = torch.int16 if bf16_dw else torch.int32
        assert torch.equal(dw.view(iv), ref_dw.view(iv)), what
