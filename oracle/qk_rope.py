"""Plain FP64 reference of the fused QK RMSNorm + 3-D RoPE + V copy (slow, obviously correct).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  It shares no code with the GPU library.

Follows norm guide §5.2 (fused_qk_rmsnorm_rope) and the norm docs API table.  What the
pages fix: qkv is BF16 [tokens, (nq + nk + nv) * head_dim]; a RMSNorm of Q and of K taken
across their heads; a rotary embedding split into frame / height / width channel groups
(even counts summing to head_dim, each with its own frequency table of count/2 entries);
ppf, pph, ppw patches per frame / height / width with tokens a multiple of ppf*pph*ppw;
base 10000 by default; interleaved or NeoX pairing; YaRN factor / low / high /
attention_factor; is_qk_norm = False skips the norm; V is copied to its own contiguous
output; optional e4m3 outputs with an output scale for Q/K and one for V.

Readings where the pages are silent (each listed with the design notes):
  * cross-head norm: one rstd per token over all nq*head_dim channels of Q (and one over K),
    weights q_weight [nq*head_dim] and k_weight [nk*head_dim];
  * token t of its sequence sits at frame t // (pph*ppw), height (t // ppw) % pph,
    width t % ppw (row-major patches); a token's index in its sequence is t mod ppf*pph*ppw;
  * a group of `count` channels rotates with inv_freq_i = base^(-2i/count), i < count/2;
  * pair j of a head (j < head_dim/2) is channels (2j, 2j+1) when interleaved and
    (j, j + head_dim/2) in NeoX style; pairs j < cf/2 use the frame position and table
    index j, then cf/2 <= j < (cf+ch)/2 the height position (index j - cf/2), the rest the
    width position;
  * YaRN (factor != 1), per group: ramp_i = clip((i - low) / (high - low), 0, 1) and
    inv_freq_i = inv_freq_i / factor * ramp_i + inv_freq_i * (1 - ramp_i) (high == low
    takes high + 0.001); cos and sin are multiplied by attention_factor;
  * (a, b) -> (a cos - b sin, a sin + b cos) on the normalised FP32 value (no BF16
    rounding before the rotation); outputs round once (BF16) or are divided by their scale
    and encoded as e4m3fn (saturating);
  * V is a bit copy (BF16) or e4m3fn(v / v_scale).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .formats import bf16_round
from .rmsnorm import Quant, quantize_static


def token_positions(tokens, ppf: int, pph: int, ppw: int):
    """(frame, height, width) patch coordinates of every token (row-major patches).
    `tokens` is a token count (tokens 0 .. tokens-1) or an array of token indices."""
    seq = ppf * pph * ppw
    ids = np.arange(tokens) if np.ndim(tokens) == 0 else np.asarray(tokens)
    t = ids.astype(np.int64) % seq
    return t // (pph * ppw), (t // ppw) % pph, t % ppw


def inv_freq(count: int, base: float = 10000.0, factor: float = 1.0, low: float = 0.0,
             high: float = 0.0) -> np.ndarray:
    """Rotary frequencies of one channel group of `count` channels (count/2 of them), with
    the YaRN blend when factor != 1."""
    i = np.arange(count // 2, dtype=np.float64)
    f = np.power(float(base), -2.0 * i / count)
    if factor != 1.0:
        hi = high if high != low else high + 0.001
        ramp = np.clip((i - low) / (hi - low), 0.0, 1.0)
        f = f / factor * ramp + f * (1.0 - ramp)
    return f


def pair_tables(head_dim: int, channels, base=10000.0, factor=1.0, low=0.0, high=0.0):
    """For each pair j < head_dim/2: which position group it uses (0 frame, 1 height,
    2 width) and its inverse frequency."""
    cf, ch, cw = channels
    assert cf + ch + cw == head_dim and cf % 2 == ch % 2 == cw % 2 == 0
    group = np.concatenate([np.full(cf // 2, 0), np.full(ch // 2, 1), np.full(cw // 2, 2)])
    freq = np.concatenate([inv_freq(cf, base, factor, low, high),
                           inv_freq(ch, base, factor, low, high),
                           inv_freq(cw, base, factor, low, high)])
    return group.astype(np.int64), freq


def rope_angles(tokens, head_dim: int, channels, ppf: int, pph: int, ppw: int,
                base=10000.0, factor=1.0, low=0.0, high=0.0) -> np.ndarray:
    """theta[t, j] = position of token t in pair j's group * inv_freq[j], FP64 (`tokens` as
    in token_positions)."""
    pos = np.stack(token_positions(tokens, ppf, pph, ppw), axis=1).astype(np.float64)
    group, freq = pair_tables(head_dim, channels, base, factor, low, high)
    return pos[:, group] * freq[None, :]


def rotate(x, theta, interleave: bool, attention_factor: float = 1.0):
    """Rotate every pair of x [tokens, heads, head_dim] by theta [tokens, head_dim/2].
    Returns (rotated, magnitude) where magnitude = (|a| + |b|) * |attention_factor| per
    output element (the size of the terms the rotation adds)."""
    x = np.asarray(x, dtype=np.float64)
    hd = x.shape[-1]
    c = np.cos(theta)[:, None, :] * attention_factor
    s = np.sin(theta)[:, None, :] * attention_factor
    if interleave:
        a, b = x[..., 0::2], x[..., 1::2]
    else:
        a, b = x[..., :hd // 2], x[..., hd // 2:]
    ra = a * c - b * s
    rb = a * s + b * c
    m = (np.abs(a) + np.abs(b)) * abs(attention_factor)
    out = np.empty_like(x)
    mag = np.empty_like(x)
    if interleave:
        out[..., 0::2], out[..., 1::2] = ra, rb
        mag[..., 0::2], mag[..., 1::2] = m, m
    else:
        out[..., :hd // 2], out[..., hd // 2:] = ra, rb
        mag[..., :hd // 2], mag[..., hd // 2:] = m, m
    return out, mag


def cross_head_rmsnorm(x, w, eps: float):
    """n = x * rstd * w over all channels of the token's heads (x [tokens, width]); FP64."""
    x = np.asarray(x, dtype=np.float64)
    eps32 = float(np.float32(eps))
    r = 1.0 / np.sqrt(np.mean(x * x, axis=1) + eps32)
    return x * r[:, None] * np.asarray(w, dtype=np.float64)[None, :], r


@dataclass
class QKRope:
    q_exact: np.ndarray      # [tokens, nq*hd] rotated FP64 values
    k_exact: np.ndarray
    q_mag: np.ndarray
    k_mag: np.ndarray
    q: np.ndarray            # BF16 outputs
    k: np.ndarray
    v: np.ndarray            # BF16 copy
    rstd_q: np.ndarray | None
    rstd_k: np.ndarray | None


def qk_rmsnorm_rope(qkv, q_weight, k_weight, nq: int, nk: int, nv: int, head_dim: int,
                    channels, ppf: int, pph: int, ppw: int, eps: float = 1e-6,
                    base: float = 10000.0, interleave: bool = True, factor: float = 1.0,
                    low: float = 0.0, high: float = 0.0, attention_factor: float = 1.0,
                    is_qk_norm: bool = True, token_ids=None) -> QKRope:
    """Q and K: cross-head RMSNorm (unless is_qk_norm is False), then the 3-D rotary
    embedding; V: copied (norm guide §5.2).  `token_ids` gives the token index of each row
    of qkv when the rows are a sample of a longer call (default: rows 0, 1, ...)."""
    qkv = np.asarray(qkv, dtype=np.float64)
    tokens = qkv.shape[0]
    hd = head_dim
    assert qkv.shape[1] == (nq + nk + nv) * hd
    if token_ids is None:
        assert tokens % (ppf * pph * ppw) == 0
        token_ids = tokens
    q = qkv[:, :nq * hd]
    k = qkv[:, nq * hd:(nq + nk) * hd]
    v = qkv[:, (nq + nk) * hd:]
    rq = rk = None
    if is_qk_norm:
        q, rq = cross_head_rmsnorm(q, q_weight, eps)
        k, rk = cross_head_rmsnorm(k, k_weight, eps)
    theta = rope_angles(token_ids, hd, channels, ppf, pph, ppw, base, factor, low, high)
    qo, qm = rotate(q.reshape(tokens, nq, hd), theta, interleave, attention_factor)
    ko, km = rotate(k.reshape(tokens, nk, hd), theta, interleave, attention_factor)
    qo, qm = qo.reshape(tokens, -1), qm.reshape(tokens, -1)
    ko, km = ko.reshape(tokens, -1), km.reshape(tokens, -1)
    return QKRope(qo, ko, qm, km, bf16_round(qo), bf16_round(ko), v.copy(), rq, rk)


def qk_rmsnorm_rope_fp8(ref: QKRope, output_scale: float, v_scale: float):
    """e4m3fn outputs: Q and K divided by output_scale, V by v_scale (norm guide §5.2:
    output_fp8 with output_quant_scale and v_quant_scale)."""
    return (quantize_static(ref.q_exact, output_scale, ref.q_mag),
            quantize_static(ref.k_exact, output_scale, ref.k_mag),
            quantize_static(ref.v, v_scale))


__all__ = ["token_positions", "inv_freq", "pair_tables", "rope_angles", "rotate",
           "cross_head_rmsnorm", "qk_rmsnorm_rope", "qk_rmsnorm_rope_fp8", "QKRope", "Quant"]
