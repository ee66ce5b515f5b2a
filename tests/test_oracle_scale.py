"""Pins for the oracle's per-head scale rule (CPU only).

The rule (a reading; the pages only say the cache holds FP8 with per-head scales): with the
head's absmax A floored at 2^-100, scale = A / 448 and inverse = 448 / A, each the correctly
rounded float32 result of the exact quotient.  The inverse is its own division, not 1 / scale.
Every expected value here is computed from exact rationals and rounded to float32 by
`nearest_f32` below, which shares nothing with the oracle's float32 arithmetic."""

from fractions import Fraction
import math

import numpy as np

from oracle import per_head_scale, e4m3_encode
from oracle.kvcache import quantize_per_head


def nearest_f32(x: Fraction) -> np.float32:
    """The float32 nearest to the positive rational x (ties to the even significand), for x in
    float32's finite range; subnormal results included."""
    assert x > 0
    e = x.numerator.bit_length() - x.denominator.bit_length()   # 2^e <= x < 2^(e+2)
    if Fraction(2) ** e > x:
        e -= 1
    if Fraction(2) ** (e + 1) <= x:
        e += 1
    # 2^e <= x < 2^(e+1); significand step 2^(e-23), or 2^-149 below the normal range
    step_exp = max(e, -126) - 23
    q = x / Fraction(2) ** step_exp
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    v = math.ldexp(float(n), step_exp)     # exact: n <= 2^24
    f = np.float32(v)
    assert float(f) == v
    return f


def expected(a: float):
    floor = Fraction(2) ** -100
    A = max(Fraction(float(np.float32(a))), floor)
    return nearest_f32(A / 448), nearest_f32(448 / A)


def _check(a):
    s, inv = per_head_scale(np.array([a], dtype=np.float32))
    es, ei = expected(a)
    assert s.dtype == np.float32 and inv.dtype == np.float32
    assert s[0] == es and inv[0] == ei, (a, s[0], es, inv[0], ei)


def test_rounding_helper_against_known_floats():
    # values a float32 holds exactly come back unchanged; halfway points go to the even neighbour
    for v in [1.0, 3.0, 448.0, 2.0 ** -149, 2.0 ** -126, 1.5 * 2.0 ** -140, 3.4028234663852886e38]:
        assert nearest_f32(Fraction(v)) == np.float32(v)
    one_up = Fraction(1) + Fraction(1, 2 ** 23)
    assert nearest_f32(Fraction(1) + Fraction(1, 2 ** 24)) == np.float32(1.0)           # tie -> even
    assert nearest_f32(one_up + Fraction(1, 2 ** 24)) == np.float32(1.0 + 2.0 ** -22)   # tie -> even (up)
    assert nearest_f32(Fraction(1, 3)) == np.float32(1.0 / 3.0)


def test_three():
    s, inv = per_head_scale(np.array([3.0], dtype=np.float32))
    assert s[0] == nearest_f32(Fraction(3, 448))
    assert inv[0] == nearest_f32(Fraction(448, 3))


def test_zero_and_subnormal_absmax_take_the_floor():
    floor_s, floor_i = nearest_f32(Fraction(2) ** -100 / 448), nearest_f32(448 * Fraction(2) ** 100)
    for a in [0.0, -0.0, 2.0 ** -149, 1e-40, 2.0 ** -101]:
        s, inv = per_head_scale(np.array([a], dtype=np.float32))
        assert s[0] == floor_s and inv[0] == floor_i and np.isfinite(inv[0]), a
    # an all-zero head encodes to zero codes
    codes, sc = quantize_per_head(np.zeros((4, 2, 64), dtype=np.float32))
    assert not codes.any() and np.all(sc == floor_s)


def test_exact_quotients_over_many_absmax_values():
    rng = np.random.default_rng(7)
    bits = np.concatenate([
        rng.integers(0x00000001, 0x7F7FFFFF, size=3000, dtype=np.uint32),   # every binade
        rng.integers(0x3F000000, 0x45000000, size=2000, dtype=np.uint32),   # the usual range
        np.array([0x3F800000, 0x43E00000, 0x7F7FFFFF, 0x0D800000, 0x0D7FFFFF], dtype=np.uint32),
    ])
    a = bits.view(np.float32)
    s, inv = per_head_scale(a)
    for j in range(a.size):
        es, ei = expected(a[j])
        assert s[j] == es and inv[j] == ei, (a[j], s[j], es, inv[j], ei)


def _search(pred, start=0x3F800000, count=200000):
    for a in np.arange(start, start + count, dtype=np.uint32).view(np.float32):
        if pred(float(a)):
            return float(a)
    raise AssertionError("no witness found")


def test_inverse_is_its_own_division_not_one_over_scale():
    """A witness where round(448 / A) differs from round(1 / round(A / 448)): the oracle must
    give the former."""
    def differs(a):
        A = Fraction(a)
        s = nearest_f32(A / 448)
        return nearest_f32(448 / A) != nearest_f32(1 / Fraction(float(s)))
    a = _search(differs)
    _check(a)
    s, inv = per_head_scale(np.array([a], dtype=np.float32))
    assert inv[0] != nearest_f32(1 / Fraction(float(s[0])))


def test_scale_is_a_division_not_a_product_with_a_rounded_reciprocal():
    """A witness where round(A / 448) differs from round(A * round(1 / 448))."""
    r = Fraction(float(nearest_f32(Fraction(1, 448))))

    def differs(a):
        A = Fraction(a)
        return nearest_f32(A / 448) != nearest_f32(A * r)
    a = _search(differs)
    _check(a)


def test_absmax_value_encodes_to_the_largest_code():
    # x = A encodes (after x * inverse) to 448 or the code just below: the inverse rounds
    # either way, but never past saturation
    rng = np.random.default_rng(11)
    a = rng.uniform(1e-3, 1e3, size=500).astype(np.float32)
    _, inv = per_head_scale(a)
    codes = e4m3_encode((a * inv).astype(np.float32))
    assert np.all(codes == 0x7E)
