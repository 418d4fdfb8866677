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


# ---------------------------------------------------------------- per-tensor scales
def test_quantize_rounds_the_quotient_to_fp32_first():
    # Find x where the fp32 quotient x/s lands exactly on a midpoint between two codes while the
    # exact quotient lies off it: the fp32 reading takes the even code, the exact one the nearer.
    from fractions import Fraction
    found = 0
    for s in (np.float32(0.1), np.float32(0.0123), np.float32(7.3)):
        for c in range(8, 0x7D):
            mid = (F.decode_code(c) + F.decode_code(c + 1)) / 2
            x0 = np.float32(mid * float(s))
            xs = [x0]
            for direction in (np.float32(np.inf), np.float32(-np.inf)):
                x = x0
                for _ in range(4):
                    x = np.nextafter(x, direction, dtype=np.float32)
                    xs.append(x)
            for x in xs:
                q32 = np.float32(x) / s
                exact = Fraction(float(x)) / Fraction(float(s))
                if float(q32) != mid or exact == Fraction(mid):
                    continue
                even = c if c % 2 == 0 else c + 1
                nearer = c + 1 if exact > Fraction(mid) else c
                assert F.quantize(np.array([x], np.float32), float(s))[0] == even
                assert F.encode_scalar(float(exact)) == nearer
                found += even != nearer
    assert found > 10


def test_quantize_round_trips_codes_under_power_of_two_scales():
    finite = np.array(list(range(0x7F)) + list(range(0x80, 0xFF)), dtype=np.uint8)
    for s in (2.0 ** -7, 1.0, 4.0):
        x = (F.decode(finite) * s).astype(np.float32)      # exact in fp32
        assert np.array_equal(F.quantize(x, s), finite)
        assert np.array_equal(F.dequantize(finite, s), F.decode(finite) * s)


def test_quantize_saturates_relative_to_the_scale():
    s = 0.01
    x = np.array([4.47, 4.49, 5.0, -100.0, np.inf, -np.inf, np.nan], dtype=np.float32)
    got = F.quantize(x, s)
    assert got.tolist() == [F.encode_scalar(float(np.float32(4.47) / np.float32(s))), 0x7E, 0x7E, 0xFE, 0x7E,
                            0xFE, 0x7F]
    assert abs(F.dequantize(got[:1], s)[0] - 4.47) <= 4.47 / 16      # within half a step of 3 mantissa bits


# ---------------------------------------------------------------- scatter and attention on codes
def test_fp8_scatter_places_the_codes_of_the_new_rows():
    from oracle import scatter as SC
    rng = np.random.default_rng(7)
    N, Hk, D, B = 6, 2, 32, 8
    kp, vp = SC.empty_pools(N, Hk, D, B, np.uint8, 0x7F)
    assert kp.shape == (N, Hk, D // 16, B, 16) and vp.shape == (N, Hk, D, B)
    k = (rng.standard_normal((5, Hk, D)) * 2).astype(np.float32)
    v = (rng.standard_normal((5, Hk, D)) * 2).astype(np.float32)
    slots = np.array([3, 17, -1, 40, 1000])
    SC.reshape_and_cache_fp8(k, v, slots, kp, vp, 0.01, 0.02)
    for t, s in enumerate(slots.tolist()):
        if not 0 <= s < N * B:
            continue
        blk, off = divmod(s, B)
        K, V = SC.gather_logical(kp, vp, [blk], off + 1)
        assert np.array_equal(K[off], F.quantize(k[t], 0.01))
        assert np.array_equal(V[off], F.quantize(v[t], 0.02))
    written = {(s // B, s % B) for s in (3, 17, 40)}
    for blk in range(N):
        for off in range(B):
            if (blk, off) not in written:
                assert np.all(kp[blk, :, :, off, :] == 0x7F) and np.all(vp[blk, :, :, off] == 0x7F)


def _one_block_pools(kc, vc):
    # codes [L, 1, 16] -> pools of one block holding them
    from oracle import scatter as SC
    L = kc.shape[0]
    kp, vp = SC.empty_pools(1, 1, 16, 16, np.uint8, 0x7F)
    SC.reshape_and_cache(kc, vc, np.arange(L), kp, vp)
    return kp, vp


def test_fp8_attention_with_equal_keys_is_the_mean_of_the_scaled_values():
    from oracle import attention as O
    rng = np.random.default_rng(3)
    L = 11
    kc = np.tile(rng.integers(0, 0x7E, size=(1, 1, 16), dtype=np.uint8), (L, 1, 1))
    vc = rng.integers(0, 0x7E, size=(L, 1, 16), dtype=np.uint8)
    kp, vp = _one_block_pools(kc, vc)
    q = (rng.standard_normal((1, 1, 16))).astype(np.float32)
    out = O.paged_attention_decode_fp8(q, "f32", kp, vp, 0.5, 0.125, np.zeros((1, 1), np.int64),
                                       np.array([L]), 0.25)
    want = 0.125 * np.array([np.mean([F.decode_code(c) for c in vc[:, 0, d]]) for d in range(16)])
    assert np.allclose(out[0, 0], want, rtol=1e-12, atol=0)


def test_fp8_attention_on_two_tokens_is_a_sigmoid_blend():
    # two keys: weight of the first = 1 / (1 + exp(-(x1 - x2))), x_j = scale * k_scale * <q, value(k_j)>
    from oracle import attention as O
    rng = np.random.default_rng(4)
    kc = rng.integers(0x20, 0x48, size=(2, 1, 16), dtype=np.uint8)
    vc = rng.integers(0x20, 0x48, size=(2, 1, 16), dtype=np.uint8)
    kp, vp = _one_block_pools(kc, vc)
    q = rng.standard_normal((1, 1, 16)).astype(np.float32)
    ks, vs, sc = 0.75, 3.0, 0.3
    out = O.paged_attention_decode_fp8(q, "f32", kp, vp, ks, vs, np.zeros((1, 1), np.int64), np.array([2]), sc)
    k1 = np.array([F.decode_code(c) for c in kc[0, 0]])
    k2 = np.array([F.decode_code(c) for c in kc[1, 0]])
    d = sc * ks * float(q[0, 0].astype(np.float64) @ (k1 - k2))
    w1 = 1.0 / (1.0 + math.exp(-d))
    v1 = vs * np.array([F.decode_code(c) for c in vc[0, 0]])
    v2 = vs * np.array([F.decode_code(c) for c in vc[1, 0]])
    assert np.allclose(out[0, 0], w1 * v1 + (1 - w1) * v2, rtol=1e-12, atol=1e-15)
