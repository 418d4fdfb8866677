"""Pins of the FP8 E4M3 codec (oracle.fp8) against the format's own arithmetic.

Fixed points of the definition (bias 7, three mantissa bits, no infinities, NaN = S.1111.111):
1.0 is 0x38, the largest finite value 448 is 0x7E, the smallest subnormal 2^-9 is 0x01, the
smallest normal 2^-6 is 0x08; each binade holds 8 evenly spaced values; the finite codes
0x00..0x7E increase monotonically.  Encoding is pinned by round trips, by exact midpoints
(ties go to the even code), by saturation, and by a brute-force nearest check.
"""
import math

import numpy as np
import pytest

from oracle import fp8 as F


def test_decode_fixed_points():
    assert F.decode_code(0x38) == 1.0
    assert F.decode_code(0xB8) == -1.0
    assert F.decode_code(0x7E) == 448.0
    assert F.decode_code(0xFE) == -448.0
    assert F.decode_code(0x01) == 2.0 ** -9
    assert F.decode_code(0x07) == 7 * 2.0 ** -9
    assert F.decode_code(0x08) == 2.0 ** -6
    assert F.decode_code(0x00) == 0.0 and math.copysign(1.0, F.decode_code(0x80)) == -1.0
    assert math.isnan(F.decode_code(0x7F)) and math.isnan(F.decode_code(0xFF))
    assert F.decode_code(0x40) == 2.0 and F.decode_code(0x3C) == 1.5 and F.decode_code(0x30) == 0.5


def test_binades_and_monotonicity():
    vals = F.decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(vals) > 0)
    for e in range(1, 16):
        lo = 2.0 ** (e - 7)
        codes = [(e << 3) | m for m in range(8) if not (e == 15 and m == 7)]
        got = [F.decode_code(c) for c in codes]
        assert got == [lo * (1 + m / 8) for m in range(len(codes))]
    # subnormals continue the smallest binade's spacing down to zero
    assert [F.decode_code(m) for m in range(8)] == [m * 2.0 ** -9 for m in range(8)]
    assert np.isfinite(F.decode(np.arange(256, dtype=np.uint8))).sum() == 254


def test_encode_round_trips_every_finite_code():
    for c in list(range(0x7F)) + list(range(0x80, 0xFF)):
        assert F.encode_scalar(F.decode_code(c)) == c


def test_encode_midpoints_go_to_the_even_code():
    for c in range(0x7E):
        a, b = F.decode_code(c), F.decode_code(c + 1)
        mid = (a + b) / 2
        want = c if c % 2 == 0 else c + 1
        assert F.encode_scalar(mid) == want, hex(c)
        assert F.encode_scalar(-mid) == 0x80 | want
        # just off the midpoint goes to the nearer code
        assert F.encode_scalar(mid - (b - a) / 64) == c
        assert F.encode_scalar(mid + (b - a) / 64) == c + 1


def test_encode_saturates_and_keeps_nan():
    for x in (448.0, 449.0, 463.9, 464.0, 480.0, 1e6, 3.4e38):
        assert F.encode_scalar(x) == 0x7E and F.encode_scalar(-x) == 0xFE
    assert F.encode_scalar(float("nan")) == 0x7F
    assert F.encode_scalar(2.0 ** -10) == 0x00          # tie between 0 and 2^-9: even (zero)
    assert F.encode_scalar(3 * 2.0 ** -10) == 0x02      # tie between 1 and 2 (x 2^-9): even
    assert F.encode_scalar(-0.0) == 0x80


def test_encode_is_the_nearest_code():
    rng = np.random.default_rng(0)
    xs = np.concatenate([rng.standard_normal(500) * 4, rng.standard_normal(200) * 0.01,
                         rng.uniform(-460, 460, 200)])
    vals = F.decode(np.arange(0x7F, dtype=np.uint8))
    for x in xs:
        c = F.encode_scalar(float(x))
        got = abs(F.decode_code(c))
        a = min(abs(x), 448.0)        # beyond 448 saturation applies (pinned separately)
        assert abs(a - got) == np.min(np.abs(vals - a))


def test_scale_divides_before_rounding():
    x = np.array([3.0, -7.5, 0.1], dtype=np.float32)
    assert np.array_equal(F.encode(x, 2.0), F.encode(x / 2.0))


def test_fast_encoder_matches_the_brute_force():
    rng = np.random.default_rng(1)
    mids = [(F.decode_code(c) + F.decode_code(c + 1)) / 2 for c in range(0x7E)]
    xs = np.concatenate([rng.standard_normal(3000).astype(np.float32) * 3,
                         np.array(mids + [-m for m in mids] + [0.0, -0.0, 448, 500, -1e9, np.nan, 2.0 ** -11])])
    assert np.array_equal(F.encode_fast(xs), F.encode(xs))
