"""Number formats of the RMSNorm family, written from their definitions (FP64 host code).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module. The GPU library never does.

Formats (the pages name the tensor dtypes; the bit layouts are the formats' own definitions):

* BF16 -- the upper half of an IEEE-754 binary32: 1 sign bit, 8 exponent bits (bias 127),
  7 fraction bits. Every activation tensor on the pages is BF16 (flashinfer.norm docs,
  API table; cake_rmsnorm_det_train_forward docs, Parameters).
* FP32 -- IEEE-754 binary32; statistics, rstd and dw are FP32 (FlashInfer norm guide §6.1).
* FP8 e4m3fn -- 1 sign bit, 4 exponent bits (bias 7), 3 fraction bits. Exponent field 0
  holds subnormals m/8 * 2^-6; the code S.1111.111 is NaN; there is no infinity; the
  largest finite magnitude is 1.75 * 2^8 = 448. The pages fix this dtype for every FP8
  output (FlashInfer norm guide §3.2, §3.3; flashrt-adaptive-norms README, Tensor
  Conventions).

Rounding is round-to-nearest, ties to even, throughout. Conversions to FP8 saturate to
+-448 first: the pages do not say what happens above the largest code, and clamping is
the reading taken (see the design notes, reading "FP8 overflow").
"""
from __future__ import annotations

import numpy as np

BF16_FRACTION_BITS = 7
BF16_MIN_EXP = -126          # smallest normal exponent; subnormals share its quantum
E4M3_FRACTION_BITS = 3
E4M3_MIN_EXP = -6
E4M3_MAX = 448.0


def _round_to_binary_grid(v: np.ndarray, fraction_bits: int, min_exp: int) -> np.ndarray:
    """Round float64 values to the nearest point of a binary floating-point grid, ties to even.

    The grid has ``fraction_bits`` stored fraction bits and normal exponents down to
    ``min_exp``; below that the spacing stays 2^(min_exp - fraction_bits) (subnormals).
    No upper limit is applied here.  Signs (including -0) are kept; NaN stays NaN.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    finite = np.isfinite(a) & (a > 0)
    safe = np.where(finite, a, 1.0)
    _, e2 = np.frexp(safe)               # safe = m * 2**e2 with 0.5 <= m < 1
    lead = np.maximum(e2 - 1, min_exp)   # exponent of the leading bit, clamped to the subnormal range
    quantum = np.ldexp(1.0, lead - fraction_bits)
    # safe / quantum is exact (division by a power of two); np.round is half-to-even.
    r = np.round(safe / quantum) * quantum
    out = np.where(finite, r, a)
    return np.copysign(out, v)


# ----------------------------------------------------------------------------- FP32

def f32_round(v) -> np.ndarray:
    """Nearest binary32 value (ties to even) of float64 values, returned as float64."""
    with np.errstate(over="ignore"):         # beyond the binary32 range: +-inf
        return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)


def two_sum(a: np.ndarray, b: np.ndarray):
    """Knuth's TwoSum: s = fl(a+b) and the exact error e with a + b = s + e (float64)."""
    s = a + b
    bb = s - a
    e = (a - (s - bb)) + (b - bb)
    return s, e


def f32_round_exact_sum(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """binary32 rounding (ties to even) of the EXACT sum a + b of two float64 values.

    This is the single rounding an FP32 fused multiply-add performs when a is an exact
    product.  The float64 sum s may itself be rounded; TwoSum recovers the exact residual
    e, and e only matters when s lies exactly half-way between two binary32 values.
    """
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    s, e = two_sum(a, b)
    c = f32_round(s)
    s32 = s.astype(np.float32)
    up = np.nextafter(s32, np.float32(np.inf)).astype(np.float64)
    dn = np.nextafter(s32, np.float32(-np.inf)).astype(np.float64)
    # Neighbours of s on the binary32 grid that bracket it.
    lo = np.where(c <= s, c, dn)
    hi = np.where(c >= s, c, up)
    tie = (s - lo == hi - s) & (lo != hi) & (e != 0)
    return np.where(tie, np.where(e > 0, hi, lo), c)


# ----------------------------------------------------------------------------- BF16

def bf16_bits_to_f64(bits) -> np.ndarray:
    """Decode BF16 bit patterns (uint16) to float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):      # NaN patterns stay NaN
        return b.view(np.float32).astype(np.float64)


def bf16_round(v) -> np.ndarray:
    """Round float64 values to BF16 values (ties to even); overflow goes to +-inf."""
    r = _round_to_binary_grid(v, BF16_FRACTION_BITS, BF16_MIN_EXP)
    return np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, r), r)


def f64_to_bf16_bits(v) -> np.ndarray:
    """BF16 bit patterns (uint16) of float64 values rounded to nearest even; NaN -> 0x7FC0."""
    r = bf16_round(v)
    bits = (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return np.where(np.isnan(r), np.uint16(0x7FC0), bits).astype(np.uint16)


def bf16_near_tie(v, rel: float = 2.0 ** -20) -> np.ndarray:
    """True where float64 v lies within rel*|v| of a midpoint between adjacent BF16 values.

    A kernel that evaluates v in FP32 (a few roundings of 2^-24 each) may round such a value
    to the other neighbour; everywhere else its BF16 result is unique.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    ok = np.isfinite(a) & (a > 0)
    safe = np.where(ok, a, 1.0)
    _, e2 = np.frexp(safe)
    quantum = np.ldexp(1.0, np.maximum(e2 - 1, BF16_MIN_EXP) - BF16_FRACTION_BITS)
    t = safe / quantum
    dist = np.abs((t - np.floor(t)) - 0.5) * quantum
    return ok & (dist <= rel * safe)


# ----------------------------------------------------------------------------- FP8 e4m3fn

def e4m3_code_to_f64(codes) -> np.ndarray:
    """Decode FP8 e4m3fn codes (uint8) to float64 values, from the format definition."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    exp_field = (c >> 3) & 0xF
    frac = c & 0x7
    normal = np.ldexp(1.0 + frac / 8.0, exp_field - 7)
    subnormal = np.ldexp(frac / 8.0, E4M3_MIN_EXP)
    mag = np.where(exp_field == 0, subnormal, normal)
    mag = np.where((exp_field == 0xF) & (frac == 0x7), np.nan, mag)
    return sign * mag


def e4m3_round_sat(v) -> np.ndarray:
    """Round float64 values to e4m3fn values: nearest, ties to even, saturating at +-448."""
    r = _round_to_binary_grid(v, E4M3_FRACTION_BITS, E4M3_MIN_EXP)
    return np.where(np.isnan(r), np.nan, np.clip(r, -E4M3_MAX, E4M3_MAX))


def f64_to_e4m3_code(v) -> np.ndarray:
    """e4m3fn codes (uint8) of float64 values (nearest-even, saturating); NaN -> 0x7F."""
    r = e4m3_round_sat(v)
    nan = np.isnan(r)
    a = np.where(nan, 0.0, np.abs(r))
    sign = np.where(np.signbit(r) & ~nan, 0x80, 0).astype(np.int64)
    sub = a < 2.0 ** E4M3_MIN_EXP
    safe = np.where(a > 0, a, 1.0)
    _, e2 = np.frexp(safe)
    lead = e2 - 1
    frac_norm = np.round((safe / np.ldexp(1.0, lead) - 1.0) * 8.0).astype(np.int64)
    code_norm = ((lead + 7) << 3) | frac_norm
    code_sub = np.round(a / 2.0 ** (E4M3_MIN_EXP - E4M3_FRACTION_BITS)).astype(np.int64)
    code = np.where(sub, code_sub, code_norm) | sign
    return np.where(nan, 0x7F, code).astype(np.uint8)


def e4m3_near_tie(v, mag=None, rel: float = 2.0 ** -16) -> np.ndarray:
    """True where float64 v lies within rel*mag of a rounding midpoint of e4m3fn.

    ``mag`` is the magnitude that sets the evaluation error of the producer (|v| when
    omitted; the sum of the magnitudes of the terms when v is a difference that may
    cancel).  Values at or above the saturation point have no tie.  Where this is True
    either adjacent code is an acceptable result; elsewhere the code is unique.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    m = a if mag is None else np.asarray(mag, dtype=np.float64)
    ok = np.isfinite(a) & (a > 0) & (a < E4M3_MAX + 2.0 ** 4)
    safe = np.where(ok, a, 1.0)
    _, e2 = np.frexp(safe)
    quantum = np.ldexp(1.0, np.maximum(e2 - 1, E4M3_MIN_EXP) - E4M3_FRACTION_BITS)
    t = safe / quantum
    dist = np.abs((t - np.floor(t)) - 0.5) * quantum
    # Midpoints between 448 and the next binade do not exist (saturation); 432 does.
    dist = np.where(safe > E4M3_MAX, np.inf, dist)
    return ok & (dist <= rel * m)


def codes_equal_e4m3(a, b) -> np.ndarray:
    """Code equality that treats +0 (0x00) and -0 (0x80) as the same value."""
    a = np.asarray(a, dtype=np.uint8)
    b = np.asarray(b, dtype=np.uint8)
    zero = lambda c: (c & 0x7F) == 0
    return (a == b) | (zero(a) & zero(b))


def e4m3_code_steps(a, b) -> np.ndarray:
    """Distance, in codes along the number line, between two e4m3fn codes (NaN excluded)."""
    def ordinal(c):
        c = np.asarray(c, dtype=np.uint8).astype(np.int64)
        mag = c & 0x7F
        return np.where(c & 0x80, -mag, mag)
    return np.abs(ordinal(a) - ordinal(b))


def bf16_ulp_steps(a_bits, b_bits) -> np.ndarray:
    """Distance in BF16 units-in-the-last-place between two bit patterns (+0 == -0)."""
    def ordinal(c):
        c = np.asarray(c, dtype=np.uint16).astype(np.int64)
        mag = c & 0x7FFF
        return np.where(c & 0x8000, -mag, mag)
    return np.abs(ordinal(a_bits) - ordinal(b_bits))
