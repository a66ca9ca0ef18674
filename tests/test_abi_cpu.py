"""The C-ABI library on the host, without a GPU: it loads, exports every entry point that
include/dnorm.h declares, and rejects bad arguments before touching any device state.
Only argument checks and rows == 0 calls are made here (they return before any HIP call);
nothing is computed."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, E_NULL, E_SHAPE, E_ALIGN, E_DTYPE, E_WS, E_UNSUP = 0, -1, -2, -3, -4, -5, -6

A = 0x100000        # a 256-byte aligned stand-in address (never dereferenced here)
B = 0x200000
C = 0x300000
D = 0x400000
E = 0x500000


@pytest.fixture(scope="module")
def dn():
    from dit_normalization_amd import dnorm
    return dnorm


@pytest.fixture(scope="module")
def lib(dn):
    return dn.lib


def declared_entry_points():
    text = open(os.path.join(ROOT, "include", "dnorm.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const char\*|int|size_t|dn_status)\s+(dn_\w+)\(", text,
                                 re.M)))


def test_header_declares_the_expected_calls():
    names = declared_entry_points()
    for n in ["dn_rmsnorm", "dn_rmsnorm_quant", "dn_fused_add_rmsnorm", "dn_fused_add_rmsnorm_quant",
              "dn_fused_add_rmsnorm_fp8_block_quant", "dn_ada_rms_norm",
              "dn_gate_residual_ada_norm_fp8", "dn_train_forward", "dn_train_backward",
              "dn_train_backward_workspace_bytes", "dn_train_backward_partials",
              "dn_train_backward_reduce", "dn_layernorm", "dn_layernorm_quant",
              "dn_fused_dit_gate_residual_layernorm_gamma_beta",
              "dn_fused_dit_gate_residual_layernorm_scale_shift",
              "dn_fused_dit_residual_layernorm_scale_shift", "dn_fused_qk_rmsnorm_rope",
              "dn_fused_rmsnorm_silu", "dn_rmsnorm_sigmoid_gate", "dn_gated_residual_rmsnorm",
              "dn_gated_residual_next_rmsnorm", "dn_last_error"]:
        assert n in names


def test_every_declared_symbol_is_exported_and_bound(dn):
    raw = ctypes.CDLL(dn.LIB_PATH)
    for name in declared_entry_points():
        assert hasattr(raw, name), name
        assert name in dn.SIGNATURES, name


def test_binding_names_match_the_c_entry_points(dn):
    for name in declared_entry_points():
        if name in ("dn_last_error", "dn_version"):
            continue
        assert callable(getattr(dn, name)), name


def test_info_calls(lib):
    assert lib.dn_max_hidden() == 32768
    assert b"gfx950" in lib.dn_version()


def test_workspace_bytes(lib):
    assert lib.dn_train_backward_workspace_bytes(8192) == 256 * 8192 * 8
    assert lib.dn_train_backward_workspace_bytes(0) == 0
    assert lib.dn_train_backward_workspace_bytes(10 ** 6) == 0


def rms(lib, y=A, ys=4096, rstd=0, x=B, xs=4096, w=C, wd=0, rows=4, h=4096):
    return lib.dn_rmsnorm(y, ys, rstd, x, xs, w, wd, 0.0, rows, h, 1e-6, None)


def test_rmsnorm_argument_checks(lib):
    assert rms(lib, rows=0) == OK                          # empty: no launch
    assert rms(lib, rows=-1) == E_SHAPE
    assert b"rows" in lib.dn_last_error()
    assert rms(lib, h=0) == E_SHAPE
    assert rms(lib, h=40000, xs=40000, ys=40000) == E_SHAPE
    assert rms(lib, h=12, xs=16, ys=16) == E_UNSUP
    assert rms(lib, x=0) == E_NULL
    assert b"x" in lib.dn_last_error()
    assert rms(lib, y=0) == E_NULL
    assert rms(lib, w=0) == E_NULL
    assert rms(lib, x=B + 8) == E_ALIGN
    assert rms(lib, xs=4000) == E_SHAPE                    # stride < hidden
    assert rms(lib, xs=4100) == E_ALIGN                    # stride not a multiple of 8
    assert rms(lib, xs=(1 << 24) + 8) == E_SHAPE           # stride beyond 2^24 elements
    assert rms(lib, wd=7) == E_DTYPE
    assert rms(lib, w=C + 4) == E_ALIGN
    assert rms(lib, rstd=D + 2) == E_ALIGN
    assert rms(lib, rows=0, rstd=D) == OK
    assert rms(lib, rows=0, x=0, y=0, w=0) == OK           # empty tensors carry NULL


def test_quant_and_fused_add_checks(lib):
    q = lib.dn_rmsnorm_quant
    assert q(A, 4096, B, 4096, C, 0, 0.0, D, 0, 4096, 1e-6, None) == OK
    assert q(A, 4096, B, 4096, C, 0, 0.0, 0, 4, 4096, 1e-6, None) == E_NULL       # scale
    assert q(A + 4, 4096, B, 4096, C, 0, 0.0, D, 4, 4096, 1e-6, None) == E_ALIGN  # fp8 out
    fa = lib.dn_fused_add_rmsnorm
    assert fa(A, 4096, B, 4096, C, 0, 1.0, 0, 0, 4096, 1e-6, None) == OK
    assert fa(A, 4096, 0, 4096, C, 0, 1.0, 0, 4, 4096, 1e-6, None) == E_NULL
    faq = lib.dn_fused_add_rmsnorm_quant
    assert faq(A, 4096, B, 4096, C, 4096, D, 0, 0.0, E, 0, 4096, 1e-6, None) == OK
    assert faq(A, 4096, B, 4096, C, 4096, D, 2, 0.0, E, 4, 4096, 1e-6, None) == E_DTYPE


def test_block_quant_checks(lib):
    bq = lib.dn_fused_add_rmsnorm_fp8_block_quant
    args = dict(out=A, os=7168, bs=B, ld=16384, no=0, ns=0, x=C, xs=7168, r=D, rs=7168, w=E,
                wd=0, rows=16384, h=7168)

    def call(**kw):
        a = dict(args, **kw)
        return bq(a["out"], a["os"], a["bs"], a["ld"], a["no"], a["ns"], a["x"], a["xs"], a["r"],
                  a["rs"], a["w"], a["wd"], 0.0, a["rows"], a["h"], 1e-6, None)

    assert call(rows=0) == OK
    assert call(h=7160, os=7160, xs=7160, rs=7160) == E_UNSUP   # not a multiple of 128
    assert call(ld=100) == E_SHAPE                              # scale_ld < rows
    assert call(bs=0) == E_NULL
    assert call(no=A + 16, ns=7000, rows=5, ld=8) == E_SHAPE    # normed_out stride < hidden
    assert call(out=0, bs=0, x=0, r=0, rows=0) == OK            # empty: NULL pointers allowed


def test_ada_checks(lib):
    ada = lib.dn_ada_rms_norm
    assert ada(A, 3072, 0, 0, B, 3072, C, D, 9216, 1, 0, 3072, 1e-6, None) == OK
    assert ada(A, 3072, 0, 0, B, 3072, C, D, 9216, 3, 10, 3072, 1e-6, None) == E_SHAPE
    assert b"style_rows" in lib.dn_last_error()
    assert ada(A, 3072, 0, 0, B, 3072, C, D, 9000, 1, 10, 3072, 1e-6, None) == E_SHAPE
    g = lib.dn_gate_residual_ada_norm_fp8
    assert g(A, 3072, B, 3072, 0, 0, C, 3072, D, 3072, E, A, 9216, 1, B, 0, 3072, 1e-6,
             None) == OK
    assert g(A, 3072, B, 3072, 0, 0, C, 3072, D, 3072, E, A, 9216, 1, 0, 5, 3072, 1e-6,
             None) == E_NULL                                    # scale
    assert g(A, 3072, B, 3072, 0, 0, C, 3072, 0, 3072, E, A, 9216, 1, B, 5, 3072, 1e-6,
             None) == E_NULL                                    # gate


def test_train_checks(lib):
    f = lib.dn_train_forward
    assert f(A, 8192, B, C, 8192, D, 8192, E, 8192, A, 1, 1.0, 0, 8192, 1e-6, None) == OK
    assert f(A, 8192, 0, C, 8192, D, 8192, E, 8192, A, 1, 1.0, 5, 8192, 1e-6, None) == E_NULL
    assert f(A, 8192, B, 0, 8192, D, 8192, E, 8192, A, 1, 1.0, 5, 8192, 1e-6, None) == E_NULL
    ws = 256 * 8192 * 8
    b = lib.dn_train_backward
    F32, BF = 1, 0
    assert b(A, 8192, B, F32, C, 8192, D, 8192, E, 1, 1.0, A, 0, 0, B, ws, 0, 8192, None) == OK
    assert b(A, 8192, B, F32, C, 8192, D, 8192, E, 1, 1.0, A, 0, 0, B, ws - 8, 5, 8192,
             None) == E_WS
    assert b(A, 8192, B, F32, C, 8192, D, 8192, E, 1, 1.0, A, 0, 0, B + 64, ws, 5, 8192,
             None) == E_WS
    assert b(A, 8192, 0, F32, C, 8192, D, 8192, E, 1, 1.0, A, 0, 0, B, ws, 5, 8192,
             None) == E_NULL
    assert b(A, 8192, B, 7, C, 8192, D, 8192, E, 1, 1.0, A, 0, 0, B, ws, 5, 8192,
             None) == E_DTYPE
    assert b(A, 8192, B + 2, F32, C, 8192, D, 8192, E, 1, 1.0, A, 0, 0, B, ws, 5, 8192,
             None) == E_ALIGN                                   # FP32 dw: 4-byte aligned
    assert b(A, 8192, B + 1, BF, C, 8192, D, 8192, E, 1, 1.0, A, 0, 0, B, ws, 5, 8192,
             None) == E_ALIGN                                   # BF16 dw: 2-byte aligned
    r = lib.dn_train_backward_reduce
    assert r(A, F32, B, ws, 0, 8192, None) == OK
    assert r(A, F32, B, ws // 2, 5, 8192, None) == E_WS
    assert r(A, 3, B, ws, 5, 8192, None) == E_DTYPE


def test_binding_rejects_a_nondeterministic_backward(dn):
    """The pages' backward takes deterministic=True only; the binding refuses False before
    it looks at any tensor, with a ValueError naming the rule."""
    with pytest.raises(ValueError, match="deterministic"):
        dn.dn_train_backward(None, None, None, None, deterministic=False)
    assert issubclass(dn.DnormError, ValueError)


def test_layernorm_checks(lib):
    ln = lib.dn_layernorm
    assert ln(A, 3072, B, 3072, C, D, 0, 3072, 1e-6, None) == OK
    assert ln(A, 3072, B, 3072, 0, D, 4, 3072, 1e-6, None) == E_NULL          # gamma
    assert b"gamma" in lib.dn_last_error()
    assert ln(A, 3072, B, 3072, C, 0, 4, 3072, 1e-6, None) == E_NULL          # beta
    assert ln(A, 3072, B, 3072, C + 4, D, 4, 3072, 1e-6, None) == E_ALIGN     # gamma alignment
    assert ln(A, 3072, B, 3064, C, D, 4, 3072, 1e-6, None) == E_SHAPE         # stride < hidden
    lq = lib.dn_layernorm_quant
    assert lq(A, 3072, B, 3072, C, D, E, 0, 3072, 1e-6, None) == OK
    assert lq(A, 3072, B, 3072, C, D, 0, 4, 3072, 1e-6, None) == E_NULL       # scale


def test_dit_checks(lib):
    gb = lib.dn_fused_dit_gate_residual_layernorm_gamma_beta
    # gate as a chunk of a [rows, 6*hidden] modulation tensor: row stride 18432
    assert gb(0, 0, A, 3072, B, 3072, C, 3072, D, 18432, 0.0, E, A, 0, 3072, 1e-6, None) == OK
    assert gb(0, 0, A, 3072, B, 3072, C, 3072, 0, 18432, 0.0, E, A, 4, 3072, 1e-6, None) == E_NULL
    assert gb(0, 0, 0, 3072, B, 3072, C, 3072, D, 18432, 0.0, E, A, 4, 3072, 1e-6, None) == E_NULL
    assert gb(0, 0, A, 3072, B, 3072, C, 3072, D, 18436, 0.0, E, A, 4, 3072, 1e-6,
              None) == E_ALIGN                                   # gate stride not 8-aligned
    ss = lib.dn_fused_dit_gate_residual_layernorm_scale_shift
    assert ss(A, 3072, B, 3072, C, 3072, D, 3072, E, 18432, 0.0, A, 18432, 0.0, B, 18432, 0.0,
              0, 3072, 1e-6, None) == OK
    assert ss(A, 3072, B, 3072, C, 3072, D, 3072, E, 18432, 0.0, 0, 18432, 0.0, B, 18432, 0.0,
              4, 3072, 1e-6, None) == E_NULL                     # scale
    rs = lib.dn_fused_dit_residual_layernorm_scale_shift
    assert rs(0, 0, A, 3072, B, 3072, 0, 0, C, 18432, 0.0, D, 18432, 0.0, 0, 3072, 1e-6,
              None) == OK
    assert rs(E, 3072, A, 3072, B, 3072, 0, 0, C, 18432, 0.0, D, 18432, 0.0, 4, 3072, 1e-6,
              None) == E_UNSUP                                   # residual_out without residual
    assert rs(0, 0, A, 3072, B, 3072, 0, 0, C, 18432, 0.0, 0, 18432, 0.0, 4, 3072, 1e-6,
              None) == E_NULL                                    # shift


def rope(lib, tokens=12, nq=24, nk=24, nv=24, hd=128, ppf=1, pph=3, ppw=4, ch=(44, 42, 42),
         fp8=0, qs=A, vs=B, qkv=C, qkv_s=None, wq=D, wk=E, norm=1, factor=1.0, af=1.0):
    w = (nq + nk + nv) * hd
    return lib.dn_fused_qk_rmsnorm_rope(
        A, nq * hd, B, nk * hd, C, nv * hd, fp8, qs, vs, qkv, w if qkv_s is None else qkv_s,
        wq, wk, 0, norm, tokens, nq, nk, nv, hd, ppf, pph, ppw, ch[0], ch[1], ch[2], 10000.0, 1,
        factor, 0.0, 0.0, af, 1e-6, None)


def test_qk_rope_checks(lib):
    assert rope(lib, tokens=0) == OK
    assert rope(lib, tokens=0, qkv=0, wq=0, wk=0) == OK          # empty: NULL pointers
    assert rope(lib, tokens=0, hd=96, ch=(32, 32, 32)) == E_UNSUP   # head_dim not 64/128/256
    assert rope(lib, tokens=0, nq=33) == E_SHAPE                  # more than 32 heads
    assert rope(lib, tokens=0, ch=(44, 41, 43)) == E_SHAPE        # odd channel counts
    assert rope(lib, tokens=0, ch=(44, 42, 40)) == E_SHAPE        # do not sum to head_dim
    assert rope(lib, tokens=13) == E_SHAPE                        # not a multiple of 12
    assert b"multiple" in lib.dn_last_error()
    assert rope(lib, tokens=0, af=1.5) == E_SHAPE                 # af != 1 needs yarn
    assert rope(lib, tokens=0, factor=4.0, af=1.5) == OK
    assert rope(lib, wq=0) == E_NULL
    assert rope(lib, fp8=1, qs=0) == E_NULL                        # FP8 needs its scales
    assert rope(lib, qkv_s=9208) == E_SHAPE                       # stride < width
    assert rope(lib, ch=(128, 0, 0), tokens=0) == OK              # empty groups allowed


def test_silu_checks(lib):
    f = lib.dn_fused_rmsnorm_silu
    assert f(A, 512, 0, 0, B, 512, C, 0, 0.0, 0, 512, 1e-6, None) == OK
    assert f(A, 512, 2, 0, B, 512, C, 0, 0.0, 4, 512, 1e-6, None) == E_DTYPE      # fp8 flag
    assert f(A, 512, 1, 0, B, 512, C, 0, 0.0, 4, 512, 1e-6, None) == E_NULL       # FP8 scale
    assert f(A, 512, 0, 0, B, 512, 0, 0, 0.0, 4, 512, 1e-6, None) == E_NULL       # weight
    assert f(A, 512, 0, 0, B, 512, C, 0, 0.0, 4, 164, 1e-6, None) == E_UNSUP      # 164 % 8
    assert f(A + 4, 160, 1, D, B, 160, C, 0, 0.0, 4, 160, 1e-6, None) == E_ALIGN  # fp8 base


def test_sigmoid_gate_checks(lib):
    f = lib.dn_rmsnorm_sigmoid_gate
    assert f(A, 64, B, 64, 0, 0, 0.0, 0, 64, 1e-6, None) == OK
    assert f(A, 64, 0, 64, 0, 0, 0.0, 4, 64, 1e-6, None) == E_NULL          # gate
    assert f(A, 64, B, 64, C, 5, 0.0, 4, 64, 1e-6, None) == E_DTYPE         # weight dtype
    assert f(A, 64, B, 60, 0, 0, 0.0, 4, 64, 1e-6, None) == E_SHAPE         # gate stride
    assert f(A, 64, B, 64, C + 2, 0, 0.0, 4, 64, 1e-6, None) == E_ALIGN     # weight base


def test_gated_residual_checks(lib):
    f = lib.dn_gated_residual_rmsnorm
    assert f(A, 8192, B, 8192, C, 8192, 1, D, 0, 0.0, 0, 8192, 1e-6, None) == OK
    assert f(A, 8192, B, 8192, C, 8192, 3, D, 0, 0.0, 5, 8192, 1e-6, None) == E_SHAPE  # rows
    assert b"gate_rows" in lib.dn_last_error()
    assert f(A, 8192, 0, 8192, C, 8192, 1, D, 0, 0.0, 5, 8192, 1e-6, None) == E_NULL   # branch
    n = lib.dn_gated_residual_next_rmsnorm
    assert n(E, 8192, A, 8192, B, 8192, C, 8192, 5, D, 0, 0.0, 0, 0, 0.0, 5, 8192, 1e-6,
             None) == E_NULL                                                  # w_next
    assert n(0, 8192, A, 8192, B, 8192, C, 8192, 5, D, 0, 0.0, E, 0, 0.0, 5, 8192, 1e-6,
             None) == E_NULL                                                  # out
    assert n(0, 0, 0, 0, 0, 0, 0, 0, 1, 0, 0, 0.0, 0, 0, 0.0, 0, 8192, 1e-6, None) == OK


def test_force_threads_per_row(lib):
    assert lib.dn_force_threads_per_row(3) == E_SHAPE
    assert lib.dn_force_threads_per_row(384) == E_SHAPE
    assert lib.dn_force_threads_per_row(128) == OK
    assert lib.dn_force_threads_per_row(448) == OK
    assert lib.dn_force_threads_per_row(0) == OK
