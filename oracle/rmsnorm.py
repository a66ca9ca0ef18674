"""Plain FP64 reference of the row-wise RMSNorm family (slow, obviously correct).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  It shares no code with the GPU library.

Every function takes float64 arrays holding the input VALUES (BF16 or FP32 numbers, already
decoded) and returns float64 values, FP8 codes or flags.  Each step is evaluated in FP64 and
rounded only where the definition stores a value (BF16 outputs, the FP32 rstd, FP8 codes,
FP32 scales and dw).  Arrays are [rows, hidden]; a per-head 3-D tensor [T, heads, hd] is
passed as [T*heads, hd], the rows being normalised independently.

Page abbreviations used below:
  "norm docs"    -- flashinfer.norm API reference (the API table and the "Training RMSNorm
                    (Cake)" section);
  "norm guide"   -- FlashInfer 归一化算子库全解 (the walk-through article), by its section;
  "cake fwd docs"-- flashinfer.cake_rmsnorm_det_train.cake_rmsnorm_det_train_forward;
  "flashrt README" -- flashrt-adaptive-norms README.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .formats import (
    bf16_near_tie,
    bf16_round,
    e4m3_code_to_f64,
    e4m3_near_tie,
    f32_round,
    f32_round_exact_sum,
    f64_to_e4m3_code,
    E4M3_MAX,
)

BLOCK = 128  # 1x128 block quantisation (norm docs, fused_add_rmsnorm_fp8_block_quant)


def _2d(a) -> np.ndarray:
    a = np.asarray(a, dtype=np.float64)
    return a.reshape(1, -1) if a.ndim == 1 else a


# ----------------------------------------------------------------------------- statistics

def rms_reciprocal(h, eps: float) -> np.ndarray:
    """r_t = 1 / sqrt(mean_j h_tj^2 + eps), exact up to FP64 rounding.

    The mean of squares over the row and eps inside the square root: norm guide §2.1 (RMS)
    and §6.1 (r_t = (mean_j x_tj^2 + eps)^-1/2); cake fwd docs, Returns
    (1 / sqrt(mean(h_new^2) + eps)).  eps is an FP32 number inside the kernel (cake fwd
    docs, Parameters: eps), so it is rounded to FP32 first.
    """
    h = _2d(h)
    eps32 = float(np.float32(eps))
    mean_sq = np.sum(h * h, axis=1) / h.shape[1]
    return 1.0 / np.sqrt(mean_sq + eps32)


def effective_weight(w, bias: float) -> np.ndarray:
    """w_eff = FP32(w + bias).

    bias 0 is rmsnorm; bias 1 is the Gemma form out = x/RMS * (w + 1) (norm guide §2.2,
    where one kernel serves both through a weight_bias constant).  For an FP32 weight of a
    zero-centred model, the effective weight 1 + w is formed in FP32 (cake fwd docs,
    Parameters: w).  Both cases are the FP32 sum of the weight and the bias.
    """
    return f32_round(np.asarray(w, dtype=np.float64) + bias)


@dataclass
class Norm:
    y_exact: np.ndarray   # h * r * w_eff before the output rounding
    y: np.ndarray         # BF16(y_exact)
    rstd: np.ndarray      # FP32 per-row reciprocal RMS
    r64: np.ndarray       # the same in FP64 (unrounded)


def rmsnorm(x, w, bias: float = 0.0, eps: float = 1e-6) -> Norm:
    """y = BF16(x * r * w_eff) with r = 1/sqrt(mean(x^2)+eps); rstd = FP32(r).

    norm docs, API table: rmsnorm and gemma_rmsnorm; norm guide §2.1-2.2 (definition,
    2-D [batch, hidden] or 3-D [batch, heads, hidden] normalised per (batch, head) row);
    norm guide §6.1 (y = BF16((x*r)*w), FP32 statistics, one FP32 rstd per row).
    """
    x = _2d(x)
    r64 = rms_reciprocal(x, eps)
    w_eff = effective_weight(w, bias)
    y_exact = x * r64[:, None] * w_eff[None, :]
    return Norm(y_exact, bf16_round(y_exact), f32_round(r64), r64)


def residual_add(x, residual) -> np.ndarray:
    """h_new = BF16(x + residual), written back to the residual buffer.

    norm guide §3.1 (residual[i] += input[i]) and §6.1; cake fwd docs, Parameters: x
    (h_new = BF16(h + residual)).  The FP64 sum of two BF16 numbers whose exponents differ
    by less than 46 is exact; otherwise the smaller one is far below half an ulp of the
    larger, so rounding the FP64 sum gives the correctly rounded BF16 sum either way.
    """
    return bf16_round(_2d(x) + _2d(residual))


@dataclass
class FusedAdd:
    h_new: np.ndarray
    norm: Norm


def fused_add_rmsnorm(x, residual, w, bias: float = 0.0, eps: float = 1e-6) -> FusedAdd:
    """residual <- h_new = BF16(x + residual); input <- rmsnorm(h_new).

    norm docs, API table: fused_add_rmsnorm / gemma_fused_add_rmsnorm; norm guide §3.1.
    The norm is taken over the BF16 h_new (cake fwd docs, Parameters: x, "the normalized
    value is h_new"), the reading used for every residual route.
    """
    h = residual_add(x, residual)
    return FusedAdd(h, rmsnorm(h, w, bias, eps))


# ----------------------------------------------------------------------------- FP8 static

@dataclass
class Quant:
    v: np.ndarray        # exact value handed to the FP8 rounding
    q: np.ndarray        # e4m3fn codes (uint8)
    tie: np.ndarray      # True where either adjacent code is acceptable


def quantize_static(y_exact, scale: float, mag=None) -> Quant:
    """q = e4m3fn(y / scale), saturating.

    The static FP32 scale is a shape-(1,) tensor (norm guide §3.2; flashrt README, Tensor
    Conventions).  The value is divided by the scale, as in the one quantised formula the
    pages print in full, layernorm_quant's (...)/scale (norm guide §4).  The quantiser
    sees the unrounded normalised value (norm guide §3.2: ((residual/RMS)*weight).to(fp8)).
    """
    s = float(np.float32(scale))
    v = np.asarray(y_exact, dtype=np.float64) / s
    m = None if mag is None else np.asarray(mag, dtype=np.float64) / abs(s)
    return Quant(v, f64_to_e4m3_code(v), e4m3_near_tie(v, m))


def rmsnorm_quant(x, w, scale: float, bias: float = 0.0, eps: float = 1e-6):
    """out = e4m3fn(rmsnorm(x) / scale) (norm docs, API table: rmsnorm_quant)."""
    n = rmsnorm(x, w, bias, eps)
    return n, quantize_static(n.y_exact, scale)


def fused_add_rmsnorm_quant(x, residual, w, scale: float, bias: float = 0.0,
                            eps: float = 1e-6):
    """residual <- h_new; out = e4m3fn(rmsnorm(h_new) / scale); input untouched.

    norm docs, API table: fused_add_rmsnorm_quant(out, input, residual, weight, scale);
    norm guide §3.2.  The FP8 result goes to ``out`` (the signature's destination).
    """
    fa = fused_add_rmsnorm(x, residual, w, bias, eps)
    return fa, quantize_static(fa.norm.y_exact, scale)


# ----------------------------------------------------------------------------- FP8 1x128 blocks

@dataclass
class BlockQuant:
    h_new: np.ndarray
    normed: np.ndarray          # BF16 normalised values, the quantiser's input
    normed_exact: np.ndarray
    rstd: np.ndarray
    scale: np.ndarray           # FP32 [rows, hidden/128], logical layout
    q: np.ndarray               # e4m3fn codes [rows, hidden]
    fp8_tie: np.ndarray         # normed / scale lies next to an e4m3 rounding midpoint
    bf_tie: np.ndarray          # the normalised value lies next to a BF16 midpoint
    q_nb: np.ndarray            # codes of the other BF16 neighbour (bf_tie elements)
    nb_tie: np.ndarray          # fp8_tie of the other neighbour
    block_flag: np.ndarray      # [rows, hidden/128]: the block's amax has two possible values
    scale_alt: np.ndarray       # the other possible FP32 scale of a flagged block (else scale)
    q_alt: np.ndarray           # q, fp8_tie, q_nb and nb_tie under scale_alt
    fp8_tie_alt: np.ndarray
    q_nb_alt: np.ndarray
    nb_tie_alt: np.ndarray


def block_scale_of(amax) -> np.ndarray:
    """s = FP32(amax / 448): the per-block dynamic scale (norm guide §3.3, step 3)."""
    return f32_round(np.asarray(amax, dtype=np.float64) / E4M3_MAX)


def _block_codes(blocks, s, nan):
    """e4m3fn codes of blocks / s (a zero-scale block coded 0 except its NaN elements), and
    where blocks / s lies next to an e4m3 rounding midpoint."""
    safe = np.where(s > 0, s, 1.0)
    v = blocks / safe[:, :, None]
    q = np.where((s > 0)[:, :, None] | nan, f64_to_e4m3_code(v), np.uint8(0)).astype(np.uint8)
    return q, e4m3_near_tie(v) & (s > 0)[:, :, None]


def fused_add_rmsnorm_fp8_block_quant(x, residual, w, bias: float = 0.0,
                                      eps: float = 1e-6) -> BlockQuant:
    """One pass: residual <- h_new; normed = BF16(rmsnorm(h_new)); per 1x128 block
    amax = max|normed|, s = FP32(amax/448), out = e4m3fn(normed / s).

    norm docs, API table: fused_add_rmsnorm_fp8_block_quant; norm guide §3.3 (the three
    steps, normed is BF16 and is what gets quantised; one dynamic FP32 scale per 1x128
    block; hidden a multiple of 128).  A block whose amax is 0 gets scale 0 and zero codes
    (the pages are silent; a zero block has nothing to scale).

    Non-finite inputs (the pages define none; the plain IEEE reading): amax is the largest
    magnitude that is a number, IEEE maxNum, so a NaN element neither sets nor hides its
    block's scale (0 when the block holds no number), and a NaN element is coded NaN in
    every block, a zero-scale block included.

    Results that are not unique: an FP32 evaluation of the normalised value may round an
    element that lies next to a BF16 midpoint (bf16_near_tie) to either neighbour, so each
    such element takes one of two adjacent BF16 magnitudes lo < hi, and every other element
    its nominal magnitude.  The block's amax is then one of at most two values: with m the
    largest of the fixed magnitudes and of every tied element's lo, any tied element whose
    hi exceeds m has lo <= m < hi, and as lo and hi are adjacent BF16 magnitudes and m is a
    BF16 magnitude, lo = m and hi is m's successor.  So the amax is m, or m's successor when
    some tied element has lo = m; block_flag marks the blocks where both are possible, and
    the *_alt fields give the codes under the value the nominal rounding did not take.
    Under either scale, a tied element is coded from either neighbour (q or q_nb), and a
    value next to an e4m3 midpoint may take either adjacent code (fp8_tie, nb_tie).
    """
    fa = fused_add_rmsnorm(x, residual, w, bias, eps)
    n = fa.norm.y
    rows, hidden = n.shape
    nb = hidden // BLOCK
    blocks = n.reshape(rows, nb, BLOCK)
    nan = np.isnan(blocks)
    mags = np.where(nan, 0.0, np.abs(blocks))            # magnitudes are >= 0: NaN drops out
    amax = np.max(mags, axis=2)
    s = block_scale_of(amax)

    y_ex = fa.norm.y_exact.reshape(rows, nb, BLOCK)
    bf_tie = bf16_near_tie(y_ex)
    other = bf16_round(np.where(bf_tie, 2.0 * y_ex - blocks, blocks))  # mirror: the other
    lo = np.where(bf_tie, np.minimum(mags, np.abs(other)), mags)       # neighbour
    hi = np.where(bf_tie, np.maximum(mags, np.abs(other)), mags)
    m_lo = np.max(lo, axis=2)                            # every tied element rounded down
    m_hi = np.max(hi, axis=2)                            # ... or up
    block_flag = m_hi != m_lo
    scale_alt = np.where(block_flag, block_scale_of(np.where(amax == m_lo, m_hi, m_lo)), s)

    shape = (rows, hidden)
    q, fp8_tie = _block_codes(blocks, s, nan)
    q_nb, nb_tie = _block_codes(other, s, nan)
    q_alt, fp8_tie_alt = _block_codes(blocks, scale_alt, nan)
    q_nb_alt, nb_tie_alt = _block_codes(other, scale_alt, nan)
    r = lambda a: a.reshape(shape)
    return BlockQuant(fa.h_new, n, fa.norm.y_exact, fa.norm.rstd, s, r(q), r(fp8_tie),
                      r(bf_tie), r(q_nb), r(nb_tie), block_flag, scale_alt, r(q_alt),
                      r(fp8_tie_alt), r(q_nb_alt), r(nb_tie_alt))


def dequantize_blocks(q, scale) -> np.ndarray:
    """normed ~= e4m3fn value * scale, per 1x128 block (used by the pins)."""
    rows, hidden = q.shape
    vals = e4m3_code_to_f64(q).reshape(rows, hidden // BLOCK, BLOCK)
    return (vals * np.asarray(scale)[:, :, None]).reshape(rows, hidden)


# ----------------------------------------------------------------------------- AdaRMSNorm

def _style_rows(style, rows: int, dim: int):
    style = _2d(style)
    if style.shape[1] != 3 * dim or style.shape[0] not in (1, rows):
        raise ValueError("style must be (rows, 3*dim) or (1, 3*dim)")
    if style.shape[0] == 1:
        style = np.repeat(style, rows, axis=0)
    return style[:, :dim], style[:, dim:2 * dim], style[:, 2 * dim:]


@dataclass
class Ada:
    h: np.ndarray          # the normalised stream (x, or the updated residual)
    o_exact: np.ndarray    # norm * (1 + style_scale) + style_shift
    o_mag: np.ndarray      # |norm * (1 + style_scale)| + |style_shift| (cancellation scale)
    gate_out: np.ndarray   # third chunk of the style row(s)
    rstd: np.ndarray


def _ada(h, w, style, eps) -> Ada:
    """o = RMSNorm(h, w) * (1 + style_scale) + style_shift (flashrt README, opening diagram;
    Tensor Conventions: style chunks are [scale | shift | gate], one row per token or one
    row broadcast to all).  gate_out is the style's third chunk, one row per token."""
    h = _2d(h)
    rows, dim = h.shape
    sc, sh, gt = _style_rows(style, rows, dim)
    n = rmsnorm(h, w, 0.0, eps)
    a = n.y_exact * (1.0 + sc)
    return Ada(h, a + sh, np.abs(a) + np.abs(sh), gt.copy(), n.rstd)


def ada_rms_norm(x, w, style, eps: float = 1e-6):
    """out = BF16(AdaRMSNorm(x)), gate_out (flashrt README, Exported APIs:
    ada_rms_norm_style_bf16)."""
    a = _ada(x, w, style, eps)
    return a, bf16_round(a.o_exact)


def gated_residual(residual, x, gate) -> np.ndarray:
    """residual + x * gate with one FP32 rounding (a fused multiply-add), then BF16.

    flashrt README, opening diagram (residual += x * gate).  x*gate of two BF16 numbers is
    exact in FP64; the FP32 rounding of the exact sum is the single rounding of an FP32 FMA,
    and the BF16 residual buffer stores that FP32 result rounded once more.
    """
    p = _2d(x) * _2d(gate)
    return bf16_round(f32_round_exact_sum(p, _2d(residual)))


def gate_residual_ada_norm_fp8(residual, x, gate, w, style, scale: float, eps: float = 1e-6):
    """residual <- BF16(residual + x*gate); out = e4m3fn(AdaRMSNorm(residual) / scale).

    flashrt README, Exported APIs: gate_residual_ada_norm_fp8_static_bf16, returning
    (residual, out_fp8, gate_out); static FP32 scale (Tensor Conventions).
    """
    h = gated_residual(residual, x, gate)
    a = _ada(h, w, style, eps)
    return a, quantize_static(a.o_exact, scale, a.o_mag)


# ----------------------------------------------------------------------------- training

@dataclass
class TrainForward:
    y: np.ndarray
    y_exact: np.ndarray
    rstd: np.ndarray
    r64: np.ndarray
    h_new: np.ndarray | None


def train_forward(x, w, bias: float = 0.0, eps: float = 1e-6, residual=None) -> TrainForward:
    """(y, rstd) or, with a residual, (y, rstd, h_new) with h_new = BF16(h + residual).

    norm docs, "Training RMSNorm (Cake)": cake_rmsnorm_train_forward; cake fwd docs,
    Parameters and Returns; norm guide §6.1.  w may be BF16 (bias 0) or FP32 (the
    zero-centred form, bias 1).
    """
    h = _2d(x) if residual is None else residual_add(x, residual)
    n = rmsnorm(h, w, bias, eps)
    return TrainForward(n.y, n.y_exact, n.rstd, n.r64, None if residual is None else h)


@dataclass
class TrainBackward:
    dx_exact: np.ndarray
    dx: np.ndarray
    dw_exact: np.ndarray
    dw: np.ndarray
    dx_mag_direct: np.ndarray   # |r*g*w_eff| + |g_residual|: magnitude of dx's direct terms
    dx_mag_coupled: np.ndarray  # |x|*r^3*mean_j|g*w_eff*x|: bound of the coupled term


def train_backward(g, x, w, rstd, bias: float = 0.0, g_residual=None) -> TrainBackward:
    """dx = BF16(r*g*w_eff - x*r^3*mean_j(g*w_eff*x) [+ g_residual]),
    dw = FP32(sum_t g*x*r).

    norm guide §6.1 (the two formulas; FP32 accumulation), §6.2 (x is the tensor the
    forward normalised -- h_new on the residual route -- and rstd the FP32 tensor the
    forward returned; g_residual is the gradient reaching h_new directly and dx serves both
    residual inputs).  dw is the gradient with respect to w_eff, which equals the one with
    respect to w when w_eff = 1 + w.  Here r is the saved FP32 rstd taken as an exact
    number, and every sum is carried in FP64.
    """
    g = _2d(g)
    x = _2d(x)
    r = np.asarray(rstd, dtype=np.float64).reshape(-1)
    w_eff = effective_weight(w, bias)
    hidden = x.shape[1]
    gw = g * w_eff[None, :]
    c = np.sum(gw * x, axis=1) / hidden
    dx_exact = r[:, None] * gw - x * (r ** 3 * c)[:, None]
    direct = np.abs(r[:, None] * gw)
    if g_residual is not None:
        dx_exact = dx_exact + _2d(g_residual)
        direct = direct + np.abs(_2d(g_residual))
    coupled = np.abs(x) * (r ** 3 * np.sum(np.abs(gw * x), axis=1) / hidden)[:, None]
    dw_exact = np.sum(g * x * r[:, None], axis=0)
    return TrainBackward(dx_exact, bf16_round(dx_exact), dw_exact, f32_round(dw_exact), direct,
                         coupled)
