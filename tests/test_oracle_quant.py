"""Pins of oracle/quant.py: round-trip bound, special cases, exact arithmetic."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import formats, quant


def _bf16_vectors(n, D, scale=1.0, seed=0):
    x = np.random.default_rng(seed).standard_normal((n, D)) * scale
    return formats.to_bf16(x)


def test_roundtrip_within_half_step():                 # Q1
    for scale in (1e-30, 1e-3, 1.0, 20.0, 1e30):
        x = _bf16_vectors(2000, 128, scale, 1)
        q, s = quant.quantise(x)
        err = np.abs(x - quant.dequantise(q, s))
        bound = 0.5 * s.astype(np.float64)[:, None] * (1 + 2.0 ** -16)
        assert np.all(err <= bound)


def test_special_cases():                              # Q2
    x = _bf16_vectors(500, 64, 3.0, 2)
    q, s = quant.quantise(x)
    idx = np.argmax(np.abs(x), axis=1)
    assert np.all(np.abs(q[np.arange(500), idx]) == 127)
    qn, sn = quant.quantise(-x)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    for k in (-20, -3, 5, 17):
        qk, sk = quant.quantise(x * 2.0 ** k)
        assert np.array_equal(qk, q)
        assert np.array_equal(sk.astype(np.float64), s.astype(np.float64) * 2.0 ** k)
    qz, sz = quant.quantise(np.zeros((3, 128)))
    assert np.all(qz == 0) and np.all(sz == 0)
    assert q.dtype == np.int8 and s.dtype == np.float32


def test_ties_round_to_even():                         # Q2: the tie rule of round-half-even
    # absmax 127 makes the scale exactly 1, so each code is the rounded value
    # itself; .5 ties between an even and an odd code go to the even one
    vals = [127.0, 0.5, 1.5, 2.5, 3.5, 62.5, 63.5, -0.5, -2.5, -62.5, 2.25, -2.75]
    want = [127, 0, 2, 2, 4, 62, 64, 0, -2, -62, 2, -3]
    x = np.zeros((1, 64))
    x[0, :len(vals)] = vals
    q, s = quant.quantise(x)
    assert float(s[0]) == 1.0
    assert list(q[0, :len(vals)]) == want


def test_every_code_is_exact_in_bf16():                # Q4
    codes = np.arange(-127, 128, dtype=np.float64)
    assert np.array_equal(formats.to_bf16(codes), codes)


def _rn32(fr):
    """Correctly rounded float32 value (as Fraction) of a positive Fraction."""
    if fr == 0:
        return Fraction(0)
    e = fr.numerator.bit_length() - fr.denominator.bit_length()
    while Fraction(2) ** e > fr:
        e -= 1
    while Fraction(2) ** (e + 1) <= fr:
        e += 1
    q = max(e - 23, -149)                  # quantum 2**q
    scaled = fr / Fraction(2) ** q
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return Fraction(n) * Fraction(2) ** q


def _rne_int(fr):
    n = fr.numerator // fr.denominator
    rem = fr - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 != 0):
        n += 1
    return n


# 0x3F96 and 0x3FB4 hold x = m/2, whose float32 quotient rounds onto the tie 63.5:
# they separate "round the quotient to float32, then to an integer" from rounding
# the exact quotient. At 0x3A8F the float32 scale lies above m/127, so x = m/2
# divided by it gives 63 while x divided by the unrounded m/127 gives the tie
# 63.5 and 64: it separates codes against the stored (float32) scale from codes
# against the exact one.
@pytest.mark.parametrize("m_bits", [0x3F80, 0x4080, 0x40A0, 0x42A0, 0x3A83, 0x0081, 0x3F96, 0x3FB4, 0x3A8F])
def test_exhaustive_against_exact_rational(m_bits):    # Q5
    # all non-negative bf16 x <= m (and their negatives by symmetry of the code)
    m = float(formats.from_bf16_bits(np.array([m_bits], np.uint16))[0])
    pos = np.arange(0, m_bits + 1, dtype=np.uint16)
    xs = formats.from_bf16_bits(pos)
    vec = np.concatenate([xs, [m]])                       # absmax is m
    q, s = quant.quantise(vec[None, :])
    s_exact = _rn32(Fraction(m) / 127)
    assert Fraction(float(s[0])) == s_exact
    alt_disagree = 0
    for xi, qi in zip(xs, q[0, :-1]):
        r = _rn32(Fraction(float(xi)) / s_exact)
        assert _rne_int(r) == int(qi), (m, xi)
        # the other reading, RNE of the exact x*127/m, differs only next to ties
        alt = _rne_int(Fraction(float(xi)) * 127 / Fraction(m))
        if alt != int(qi):
            alt_disagree += 1
            frac = Fraction(float(xi)) * 127 / Fraction(m)
            assert abs(frac - (Fraction(int(qi) + alt, 2))) < Fraction(1, 2 ** 12)
    assert alt_disagree <= len(xs) // 100


def test_dequantised_values_are_exact_products():
    # the attention reference sees code * scale exactly (no bf16 rounding): with
    # the float32 scale of 0.1, code 3 dequantises to 3 * 0.100000001490116...
    s = np.array([np.float32(0.1)], np.float32)
    q = np.array([[3, -127, 1]], np.int8)
    x = quant.dequantise(q, s)
    s64 = float(np.float32(0.1))          # 0.100000001490116119384765625
    assert x[0, 0] == 0.300000004470348358154296875 == 3 * s64
    assert x[0, 1] == -12.7000001892447471618652343750 and x[0, 2] == s64
