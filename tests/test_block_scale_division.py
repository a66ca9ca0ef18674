"""The block-scale division of the 1x128 FP8 path, s = FP32(amax / 448), is evaluated in the
kernel as q0 = amax * RN(1/448), r = FMA(-q0, 448, amax), s = FMA(r, RN(1/448), q0) instead
of an IEEE divide.  amax is always the magnitude of a BF16 value, so the identity can be
checked for every input it can see: here, with exact rational arithmetic modelling one
rounding per FP32 operation (FMA: one rounding of the exact a*b + c), against the correctly
rounded quotient."""
from __future__ import annotations

import struct
from fractions import Fraction

import numpy as np


def rn32(x: Fraction) -> Fraction:
    """Round a rational to the nearest FP32 value (ties to even), subnormals included."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)
    ulp = Fraction(2) ** (e - 23)
    q = a / ulp
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * ulp


def test_rn32_agrees_with_numpy_float32():
    rng = np.random.default_rng(5)
    for v in np.concatenate([rng.normal(size=200) * 10.0 ** rng.integers(-40, 38, 200),
                             [1e-45, 3e-39, 1.0 / 3.0, 448.0]]):
        assert rn32(Fraction(float(v))) == Fraction(float(np.float32(v)))


def test_three_op_division_by_448_is_exact_for_every_bf16():
    inv = rn32(Fraction(1, 448))
    assert inv == Fraction(float(np.float32(1.0) / np.float32(448.0)))
    bad = []
    for bits in range(1, 0x7F80):          # every positive finite BF16 pattern
        a = Fraction(struct.unpack(">f", struct.pack(">I", bits << 16))[0])
        q0 = rn32(a * inv)
        r = rn32(a - q0 * 448)
        q = rn32(q0 + r * inv)
        if q != rn32(a / 448):
            bad.append(bits)
    assert not bad, f"{len(bad)} BF16 inputs round differently, first {bad[0]:#06x}"
