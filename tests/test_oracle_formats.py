"""Pins of the oracle's number formats against things other than the oracle itself:
brute-force nearest-value searches over every code, torch's CPU casts (library routines),
exact rational arithmetic, and values derived by hand from the format definitions."""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F

RNG = np.random.default_rng(20240611)


# ----------------------------------------------------------------------------- BF16

def all_bf16_bits():
    return np.arange(65536, dtype=np.uint32).astype(np.uint16)


def test_bf16_decode_matches_torch_for_every_pattern():
    bits = all_bf16_bits()
    ours = F.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def test_bf16_encode_roundtrips_every_finite_pattern():
    bits = all_bf16_bits()
    v = F.bf16_bits_to_f64(bits)
    fin = np.isfinite(v)
    assert (F.f64_to_bf16_bits(v[fin]) == bits[fin]).all()


def test_bf16_round_matches_torch_cast_on_fp32_inputs():
    raw = RNG.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    f = raw.view(np.float32)
    f = f[np.isfinite(f)]
    ours = F.f64_to_bf16_bits(f.astype(np.float64))
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (ours == ref).all()


def _nearest_even_search(v, grid_vals, grid_codes):
    """Brute force: nearest grid value, ties to the even code (code & 1 == 0)."""
    d = np.abs(grid_vals[None, :] - v[:, None])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    even = (grid_codes[None, :] & 1) == 0
    pick = np.where((cand & even).any(axis=1), np.argmax(cand & even, axis=1), np.argmax(cand, axis=1))
    return grid_vals[pick], grid_codes[pick]


def test_bf16_round_matches_brute_force_search_on_float64_inputs():
    bits = all_bf16_bits()
    vals = F.bf16_bits_to_f64(bits)
    keep = np.isfinite(vals) & (bits < 0x8000) & (vals <= 2.0 ** 10) & (vals >= 2.0 ** -10)
    gv, gc = vals[keep], bits[keep].astype(np.int64)
    order = np.argsort(gv)
    gv, gc = gv[order], gc[order]
    # Random values, exact midpoints, and midpoints nudged by one float64 ulp.
    x = np.exp(RNG.uniform(np.log(2.0 ** -9), np.log(2.0 ** 9), 4000))
    mids = (gv[:-1] + gv[1:]) / 2
    pick = RNG.choice(mids.size, 2000, replace=False)
    x = np.concatenate([x, mids[pick], np.nextafter(mids[pick], 0), np.nextafter(mids[pick], np.inf)])
    want, _ = _nearest_even_search(x, gv, gc)
    assert (F.bf16_round(x) == want).all()
    assert (F.bf16_round(-x) == -want).all()


def test_bf16_round_overflow_and_subnormals():
    big = (2 - 2 ** -7) * 2.0 ** 127            # largest finite BF16
    assert F.bf16_round(np.array([big]))[0] == big
    assert np.isinf(F.bf16_round(np.array([big + 2.0 ** 119]))[0])      # half an ulp above: tie to even -> inf
    assert F.bf16_round(np.array([big + 2.0 ** 118]))[0] == big
    tiny = 2.0 ** -133                           # smallest BF16 subnormal
    assert F.bf16_round(np.array([tiny * 0.5]))[0] == 0.0               # tie to even (0)
    assert F.bf16_round(np.array([tiny * 1.5]))[0] == 2 * tiny           # tie to even (2)


def test_bf16_tie_flag_marks_midpoints_only():
    one_up = 1 + 2 ** -7
    mid = (1 + one_up) / 2
    assert F.bf16_near_tie(np.array([mid]))[0]
    assert F.bf16_near_tie(np.array([mid * (1 + 2 ** -23)]))[0]
    assert not F.bf16_near_tie(np.array([1.0, one_up, 1 + 2 ** -9]))[0]


# ----------------------------------------------------------------------------- FP8 e4m3fn

def all_e4m3():
    codes = np.arange(256, dtype=np.uint8)
    return codes, F.e4m3_code_to_f64(codes)


def test_e4m3_decode_matches_torch_for_every_code():
    codes, ours = all_e4m3()
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def test_e4m3_codes_derived_by_hand_from_the_format():
    # (value, code): 1.0 = exp 7 frac 0; 448 = exp 15 frac 6 (frac 7 is NaN); smallest
    # subnormal 2^-9 = code 1; smallest normal 2^-6 = exp 1; -2 = sign | exp 8.
    table = [(1.0, 0x38), (448.0, 0x7E), (2.0 ** -9, 0x01), (2.0 ** -6, 0x08), (-2.0, 0xC0),
             (0.5, 0x30), (1.125, 0x39), (240.0, 0x77), (-448.0, 0xFE), (7 * 2.0 ** -9, 0x07)]
    for v, c in table:
        assert F.f64_to_e4m3_code(np.array([v]))[0] == c, (v, c)
        assert F.e4m3_code_to_f64(np.array([c], dtype=np.uint8))[0] == v
    # Rounding, ties to even, saturation (all derived from the grid spacing):
    #  1.0625 is half-way between 1.0 (0x38, even) and 1.125 (0x39) -> 1.0
    #  1.1875 is half-way between 1.125 (0x39) and 1.25 (0x3A, even) -> 1.25
    #  432 is half-way between 416 (0x7D) and 448 (0x7E, even) -> 448
    #  500 and 1e6 saturate to 448; 2^-10 is half of the smallest subnormal -> +0
    #  3*2^-10 is half-way between 2^-9 (0x01) and 2^-8 (0x02, even) -> 0x02
    cases = [(1.0625, 0x38), (1.1875, 0x3A), (432.0, 0x7E), (500.0, 0x7E), (1e6, 0x7E),
             (-500.0, 0xFE), (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02), (417.0, 0x7D)]
    for v, c in cases:
        assert F.f64_to_e4m3_code(np.array([v]))[0] == c, (v, hex(c))
    assert F.f64_to_e4m3_code(np.array([np.nan]))[0] == 0x7F


def test_e4m3_round_matches_brute_force_search():
    codes, vals = all_e4m3()
    fin = np.isfinite(vals) & ~((codes == 0x80))
    gv, gc = vals[fin], codes[fin].astype(np.int64)
    order = np.argsort(gv)
    gv, gc = gv[order], gc[order]
    mids = (gv[:-1] + gv[1:]) / 2
    x = np.concatenate([
        RNG.uniform(-448, 448, 20000),
        np.exp(RNG.uniform(np.log(2.0 ** -12), np.log(448.0), 20000)) * RNG.choice([-1, 1], 20000),
        mids, np.nextafter(mids, -np.inf), np.nextafter(mids, np.inf),
    ])
    want_v, want_c = _nearest_even_search(x, gv, gc)
    got = F.e4m3_round_sat(x)
    assert (got == want_v).all()
    got_c = F.f64_to_e4m3_code(x)
    assert F.codes_equal_e4m3(got_c, want_c.astype(np.uint8)).all()
    # Beyond the largest code: saturate.
    big = np.array([448.0 + 1e-9, 460.0, 464.0, 1e30, -1e30])
    assert (F.e4m3_round_sat(big) == np.sign(big) * 448.0).all()


def test_e4m3_round_matches_torch_cast_in_range():
    x = np.concatenate([RNG.normal(0, 50, 200000), RNG.normal(0, 0.01, 50000)])
    x = np.clip(x, -448, 448).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = F.f64_to_e4m3_code(x.astype(np.float64))
    assert F.codes_equal_e4m3(ours, ref).all()


def test_e4m3_tie_flag():
    assert F.e4m3_near_tie(np.array([1.0625, 432.0, 3 * 2.0 ** -10])).all()
    assert not F.e4m3_near_tie(np.array([1.0, 1.09, 448.0, 450.0, 1000.0])).any()
    # A relative band of 2^-16 around the midpoint.
    assert F.e4m3_near_tie(np.array([1.0625 * (1 + 2.0 ** -18)]))[0]
    assert not F.e4m3_near_tie(np.array([1.0625 * (1 + 2.0 ** -12)]))[0]


# ----------------------------------------------------------------------------- FP32 of an exact sum

def _f32_of_fraction(q: Fraction) -> float:
    """binary32 nearest (ties even) to an exact rational, by bracketing on the float32 grid."""
    x = np.float32(float(q))                      # within one float32 ulp of q
    cands = [np.nextafter(x, np.float32(-np.inf)), x, np.nextafter(x, np.float32(np.inf))]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - q),
                                     int(np.array(c, np.float32).view(np.uint32)) & 1))
    return float(best)


def test_f32_round_exact_sum_matches_rational_arithmetic():
    # Products of BF16 numbers plus BF16 numbers, plus constructed double-rounding traps.
    a = F.bf16_round(RNG.normal(0, 4, 3000)) * F.bf16_round(RNG.normal(0, 4, 3000))
    b = F.bf16_round(RNG.normal(0, 4, 3000))
    # Traps: a = 1 + 2^-24 (an exact FP32 midpoint) plus a tiny b of either sign.
    a = np.concatenate([a, [1 + 2.0 ** -24] * 4, [2.0 ** 30 + 2.0 ** 6] * 2])
    b = np.concatenate([b, [2.0 ** -80, -2.0 ** -80, 2.0 ** -60, -2.0 ** -60], [2.0 ** -40, -2.0 ** -40]])
    got = F.f32_round_exact_sum(a, b)
    want = np.array([_f32_of_fraction(Fraction(float(p)) + Fraction(float(q))) for p, q in zip(a, b)])
    assert (got == want).all()
