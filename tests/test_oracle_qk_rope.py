"""Pins of the oracle's fused QK RMSNorm + 3-D RoPE against things other than the oracle:
numpy's unravel_index, torch's complex arithmetic (torch.polar), the rotate-half form of
NeoX RoPE built from torch.cat, torch's rms_norm, YaRN ramp end points in closed form, and
the invariants that define a rotary embedding (norm preservation, relative positions)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import qk_rope as Q

RNG = np.random.default_rng(21)


def bf16_values(shape, std=1.0):
    return F.bf16_round(RNG.normal(0.0, std, shape))


def test_positions_match_unravel_index():
    f, h, w = Q.token_positions(2 * 3 * 4 * 5, 3, 4, 5)
    t = np.arange(120) % 60
    ef, eh, ew = np.unravel_index(t, (3, 4, 5))
    assert (f == ef).all() and (h == eh).all() and (w == ew).all()


@pytest.mark.parametrize("count", [2, 16, 44, 128])
def test_inv_freq_matches_the_usual_table(count):
    ref = 1.0 / (10000.0 ** (torch.arange(0, count, 2, dtype=torch.float64) / count))
    np.testing.assert_allclose(Q.inv_freq(count), ref.numpy(), rtol=1e-15)


def test_yarn_ramp_end_points():
    base = Q.inv_freq(32)
    y = Q.inv_freq(32, factor=4.0, low=2.0, high=6.0)
    assert (y[:3] == base[:3]).all()                   # i <= low: extrapolation (unchanged)
    np.testing.assert_allclose(y[6:], base[6:] / 4.0, rtol=1e-15)   # i >= high: / factor
    np.testing.assert_allclose(y[4], base[4] * (0.5 / 4.0 + 0.5), rtol=1e-15)   # half way
    z = Q.inv_freq(32, factor=4.0, low=5.0, high=5.0)  # equal bounds: a step at 5
    assert (z[:6] == base[:6]).all() and np.allclose(z[6:], base[6:] / 4.0)


def _torch_polar_rope(x, theta, af):
    """Interleaved RoPE as complex multiplication with torch.polar."""
    t = torch.from_numpy(np.ascontiguousarray(x))
    xc = torch.view_as_complex(t.reshape(*t.shape[:-1], -1, 2).contiguous())
    th = torch.from_numpy(theta)[:, None, :]
    rot = torch.polar(torch.full_like(th, af), th)
    return torch.view_as_real(xc * rot).reshape(t.shape).numpy()


def _torch_rotate_half_rope(x, theta, af):
    """NeoX RoPE in the rotate-half form: x*cos + rotate_half(x)*sin, halves concatenated."""
    t = torch.from_numpy(np.ascontiguousarray(x))
    th = torch.from_numpy(theta)[:, None, :]
    cos = torch.cat([th.cos(), th.cos()], dim=-1) * af
    sin = torch.cat([th.sin(), th.sin()], dim=-1) * af
    h = t.shape[-1] // 2
    rh = torch.cat([-t[..., h:], t[..., :h]], dim=-1)
    return (t * cos + rh * sin).numpy()


@pytest.mark.parametrize("af", [1.0, 1.25])
def test_rotation_interleaved_is_complex_multiplication(af):
    x = RNG.normal(size=(12, 3, 64))
    th = RNG.uniform(-50, 50, size=(12, 32))
    out, _ = Q.rotate(x, th, True, af)
    np.testing.assert_allclose(out, _torch_polar_rope(x, th, af), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("af", [1.0, 0.75])
def test_rotation_neox_is_rotate_half(af):
    x = RNG.normal(size=(12, 3, 64))
    th = RNG.uniform(-50, 50, size=(12, 32))
    out, _ = Q.rotate(x, th, False, af)
    np.testing.assert_allclose(out, _torch_rotate_half_rope(x, th, af), rtol=1e-12,
                               atol=1e-12)


def test_interleaved_and_neox_agree_up_to_a_channel_permutation():
    hd = 32
    perm = np.empty(hd, dtype=np.int64)           # interleaved channel of each NeoX channel
    perm[:hd // 2] = np.arange(0, hd, 2)
    perm[hd // 2:] = np.arange(1, hd, 2)
    x = RNG.normal(size=(5, 2, hd))
    th = RNG.uniform(-9, 9, size=(5, hd // 2))
    a, _ = Q.rotate(x, th, True)
    b, _ = Q.rotate(x[..., perm], th, False)
    np.testing.assert_allclose(b, a[..., perm], rtol=1e-14, atol=1e-14)


def test_rotation_preserves_pair_norms_and_position_zero_is_identity():
    x = RNG.normal(size=(4, 2, 16))
    th = RNG.uniform(-9, 9, size=(4, 8))
    out, _ = Q.rotate(x, th, True, 1.5)
    n_in = np.hypot(x[..., 0::2], x[..., 1::2])
    n_out = np.hypot(out[..., 0::2], out[..., 1::2])
    np.testing.assert_allclose(n_out, 1.5 * n_in, rtol=1e-13)
    same, _ = Q.rotate(x, np.zeros((4, 8)), False)
    assert (same == x).all()


@pytest.mark.parametrize("interleave", [True, False])
def test_scores_depend_only_on_relative_positions(interleave):
    """<rope(q, p), rope(k, p')> is a function of p - p' in every group: shifting the frame,
    height and width of both tokens by the same amounts leaves the score unchanged."""
    hd, ch = 48, (16, 16, 16)
    ppf, pph, ppw = 6, 5, 4
    T = ppf * pph * ppw
    qv, kv = RNG.normal(size=hd), RNG.normal(size=hd)
    x = np.zeros((T, 1, hd))
    th = Q.rope_angles(T, hd, ch, ppf, pph, ppw)
    tok = lambda f, h, w: (f * pph + h) * ppw + w

    def score(tq, tk):
        xq = x.copy(); xq[tq, 0] = qv
        xk = x.copy(); xk[tk, 0] = kv
        rq, _ = Q.rotate(xq, th, interleave)
        rk, _ = Q.rotate(xk, th, interleave)
        return float(rq[tq, 0] @ rk[tk, 0])

    s0 = score(tok(1, 1, 0), tok(3, 0, 2))
    s1 = score(tok(3, 4, 1), tok(5, 3, 3))       # both shifted by (2, 3, 1)
    assert abs(s0 - s1) < 1e-12 * max(1.0, abs(s0))
    s2 = score(tok(1, 1, 0), tok(3, 0, 3))       # a different offset gives another score
    assert abs(s0 - s2) > 1e-6


def test_cross_head_rmsnorm_matches_torch():
    x = bf16_values((9, 3 * 64), std=2.0)
    w = bf16_values(3 * 64)
    n, r = Q.cross_head_rmsnorm(x, w, 1e-6)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (192,),
                                       weight=torch.from_numpy(w),
                                       eps=float(np.float32(1e-6))).numpy()
    np.testing.assert_allclose(n, ref, rtol=1e-12, atol=1e-12)


def test_full_call_assembles_the_pieces():
    nq, nk, nv, hd = 2, 1, 3, 32
    ch = (12, 10, 10)
    ppf, pph, ppw = 2, 3, 2
    T = 2 * ppf * pph * ppw
    qkv = bf16_values((T, (nq + nk + nv) * hd))
    wq, wk = bf16_values(nq * hd), bf16_values(nk * hd)
    r = Q.qk_rmsnorm_rope(qkv, wq, wk, nq, nk, nv, hd, ch, ppf, pph, ppw, interleave=False,
                          factor=2.0, low=1.0, high=4.0, attention_factor=1.1)
    # V is untouched; Q and K are the torch rotate-half RoPE of torch's rms_norm
    assert (r.v == qkv[:, (nq + nk) * hd:]).all()
    th = Q.rope_angles(T, hd, ch, ppf, pph, ppw, factor=2.0, low=1.0, high=4.0)
    for part, w, n, off, got in ((0, wq, nq, 0, r.q_exact), (1, wk, nk, nq * hd, r.k_exact)):
        x = torch.from_numpy(qkv[:, off:off + n * hd])
        nrm = torch.nn.functional.rms_norm(x, (n * hd,), weight=torch.from_numpy(w),
                                           eps=float(np.float32(1e-6))).numpy()
        ref = _torch_rotate_half_rope(nrm.reshape(T, n, hd), th, 1.1).reshape(T, -1)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    assert (r.q == F.bf16_round(r.q_exact)).all()
    # without the norm the raw values rotate
    raw = Q.qk_rmsnorm_rope(qkv, wq, wk, nq, nk, nv, hd, ch, ppf, pph, ppw, is_qk_norm=False)
    ref = _torch_polar_rope(qkv[:, :nq * hd].reshape(T, nq, hd),
                            Q.rope_angles(T, hd, ch, ppf, pph, ppw), 1.0).reshape(T, -1)
    np.testing.assert_allclose(raw.q_exact, ref, rtol=1e-12, atol=1e-12)


def test_fp8_outputs_match_torch_cast():
    nq, nk, nv, hd = 2, 2, 2, 64
    T = 8
    qkv = bf16_values((T, (nq + nk + nv) * hd))
    r = Q.qk_rmsnorm_rope(qkv, np.ones(nq * hd), np.ones(nk * hd), nq, nk, nv, hd,
                          (32, 16, 16), 2, 2, 2)
    q8, k8, v8 = Q.qk_rmsnorm_rope_fp8(r, 0.05, 0.02)
    for qq, vals, s in ((q8, r.q_exact, 0.05), (v8, r.v, 0.02)):
        x = (vals / float(np.float32(s))).astype(np.float32)
        ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        ok = np.abs(x) < 448
        assert (F.codes_equal_e4m3(qq.q, ref) | qq.tie | ~ok).all()


@pytest.mark.parametrize("axis", [0, 1, 2])
def test_each_channel_group_follows_its_own_axis(axis):
    """Patches along one axis only: that axis's group turns by position * base^(-2i/count),
    the other groups do not turn at all."""
    hd, ch = 40, (16, 12, 12)
    dims = [1, 1, 1]
    dims[axis] = 7
    th = Q.rope_angles(7, hd, ch, *dims)
    start = [0, 8, 14, 20][axis]
    stop = [0, 8, 14, 20][axis + 1]
    i = np.arange(stop - start)
    expect = np.arange(7)[:, None] * 10000.0 ** (-2.0 * i / ch[axis])[None, :]
    np.testing.assert_allclose(th[:, start:stop], expect, rtol=1e-15)
    others = np.ones(20, dtype=bool)
    others[start:stop] = False
    assert (th[:, others] == 0).all()


def test_token_ids_select_rows_of_the_full_call():
    nq, nk, nv, hd = 1, 1, 1, 64
    qkv = bf16_values((24, 3 * hd))
    w = np.ones(hd)
    full = Q.qk_rmsnorm_rope(qkv, w, w, nq, nk, nv, hd, (24, 20, 20), 2, 3, 4)
    ids = np.array([0, 5, 17, 23])
    part = Q.qk_rmsnorm_rope(qkv[ids], w, w, nq, nk, nv, hd, (24, 20, 20), 2, 3, 4,
                             token_ids=ids)
    assert (part.q_exact == full.q_exact[ids]).all() and (part.k == full.k[ids]).all()
