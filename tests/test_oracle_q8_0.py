"""Pins of the oracle's q8_0 key quantiser: exact rational brute force, bounds, ties."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import q8_0_decode, q8_0_encode


def _rn16(r: Fraction) -> Fraction:
    """Round a non-negative rational to the nearest fp16 value, ties to even."""
    assert r >= 0
    if r == 0:
        return Fraction(0)
    e = r.numerator.bit_length() - r.denominator.bit_length()
    if Fraction(2) ** e > r:
        e -= 1
    # now 2^e <= r < 2^(e+1)
    ulp = Fraction(2) ** (max(e, -14) - 10)
    m = r / ulp
    lo = m.numerator // m.denominator
    rem = m - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return lo * ulp


def _rne_int(r: Fraction) -> int:
    lo = r.numerator // r.denominator
    rem = r - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 != 0):
        lo += 1
    return lo


def _brute_block(x16):
    xs = [Fraction(float(v)) for v in x16]
    amax = max(abs(v) for v in xs)
    s = _rn16(amax / 127)
    if s == 0:
        return [0] * len(xs), s
    return [max(-127, min(127, _rne_int(v / s))) for v in xs], s


@pytest.mark.parametrize("seed,scale", [(0, 1.0), (1, 30.0), (2, 1e-3), (3, 1e-5), (4, 6e4 / 4)])
def test_exact_rational_brute_force(seed, scale):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((24, 64)) * scale).astype(np.float16)
    codes, scales = q8_0_encode(x)
    for r in range(x.shape[0]):
        for b in range(2):
            blk = x[r, 32 * b:32 * b + 32]
            want_q, want_s = _brute_block(blk)
            assert Fraction(float(scales[r, b])) == want_s
            assert list(codes[r, 32 * b:32 * b + 32]) == want_q


def test_error_bound_and_full_range():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((512, 128)) * rng.lognormal(0, 2, size=(512, 1))).astype(np.float16)
    codes, scales = q8_0_encode(x)
    s = scales.astype(np.float64)
    xhat = q8_0_decode(codes, scales)
    err = np.abs(x.astype(np.float64) - xhat).reshape(512, 4, 32)
    normal = s >= 2.0 ** -14
    assert np.all(err[normal] <= s[normal][:, None] / 2)
    # every nonzero block with a normal scale reaches |code| = 127
    c = np.abs(codes.astype(np.int32)).reshape(512, 4, 32).max(axis=-1)
    assert np.all(c[normal & (s > 0)] == 127)


def test_constructed_ties_round_to_even():
    # amax = 127/128 gives the scale 2^-7 exactly; (2k+1)/256 then divides to k + 1/2.
    vals = [127 / 128] + [(2 * k + 1) / 256 for k in range(8)] + [-(2 * k + 1) / 256 for k in range(8)]
    vals += [0.0] * (32 - len(vals))
    x = np.array(vals, dtype=np.float16)
    codes, scales = q8_0_encode(x)
    assert float(scales[0]) == 2.0 ** -7
    assert int(codes[0]) == 127
    assert list(codes[1:9]) == [0, 2, 2, 4, 4, 6, 6, 8]
    assert list(codes[9:17]) == [0, -2, -2, -4, -4, -6, -6, -8]


def test_zero_block_and_negative_zero():
    x = np.zeros((2, 32), dtype=np.float16)
    x[1] = -0.0
    codes, scales = q8_0_encode(x)
    assert np.all(codes == 0) and np.all(scales.astype(np.float32) == 0)


def test_subnormal_scale_clamps():
    # amax tiny: the scale is an fp16 subnormal and the quotient can exceed 127.5
    x = np.zeros(32, dtype=np.float16)
    ulp = 2.0 ** -24                     # smallest fp16 subnormal
    x[0] = np.float16(178 * ulp)         # amax / 127 = 1.40 ulp -> scale 1 ulp
    x[1] = np.float16(-178 * ulp)
    x[2] = np.float16(100 * ulp)
    codes, scales = q8_0_encode(x)
    want, s = _brute_block(x)
    assert Fraction(float(scales[0])) == s
    assert list(codes) == want
    assert float(scales[0]) == ulp
    assert list(codes[:3]) == [127, -127, 100]


def test_never_minus_128_and_types():
    x = (np.random.default_rng(5).standard_normal((100, 32)) * 100).astype(np.float16)
    codes, scales = q8_0_encode(x)
    assert codes.dtype == np.int8 and scales.dtype == np.float16
    assert codes.min() >= -127
    with pytest.raises(TypeError):
        q8_0_encode(x.astype(np.float32))
