"""FP8 E4M3 storage for a quantised KV cache: encode and decode, written from the format's definition.

Test infrastructure only (see the package docstring).

The pages name quantising the cached keys and values as the memory lever that follows paging: an
8-bit KV cache halves the bytes each sequence's attention reads ("Contiguous vs Paged KV Cache on
RDNA4", section "The order of the memory levers"; "KV-Cache Optimization & PagedAttention for
Long-Context Agents", introduction), but they fix no format.  The reading taken here is the OCP
8-bit floating point format E4M3, which MI355X converts natively:

* one sign bit, four exponent bits with bias 7, three mantissa bits;
* exponent field e > 0: value = (-1)^s * 2^(e - 7) * (1 + m/8);
* e = 0: value = (-1)^s * 2^-6 * (m/8) (subnormals and the two zeros);
* no infinities; the code S.1111.111 is NaN, so the largest finite magnitude is 2^8 * 1.75 = 448.

Encoding a real x takes the nearest representable value, ties to the code with an even
mantissa (round to nearest even), and saturates any magnitude above 448 to +-448; NaN encodes to
NaN.  The decoder is the definition above; the encoder is a brute-force nearest search over all
254 finite codes, which is slow and obviously right.

A cache stores an element x with a per-tensor scale s as the code of x / s and reads it back as
s * value(code) (``quantize`` / ``dequantize``).  The quotient is rounded to fp32 before the
code is chosen: that rounding can move a value onto a midpoint between two codes, so it is part
of what decides the code, and it is the rounding a device that quantises in fp32 performs.
"""
from __future__ import annotations

import math

import numpy as np

MAX_FINITE = 448.0
NAN_CODES = (0x7F, 0xFF)


def decode_code(c: int) -> float:
    """Value of one E4M3 code (a Python float, exact)."""
    c = int(c) & 0xFF
    s = -1.0 if c & 0x80 else 1.0
    e = (c >> 3) & 0xF
    m = c & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return s * math.ldexp(m / 8.0, -6)
    return s * math.ldexp(1.0 + m / 8.0, e - 7)


_TABLE = np.array([decode_code(c) for c in range(256)], dtype=np.float64)
# finite non-negative codes in increasing value order, with their values
_POS_CODES = np.array([c for c in range(0x7F)], dtype=np.int64)   # 0x00 .. 0x7E
_POS_VALUES = _TABLE[_POS_CODES]


def decode(codes: np.ndarray) -> np.ndarray:
    """Values of an array of E4M3 codes (uint8), as float64."""
    return _TABLE[np.asarray(codes, dtype=np.uint8).astype(np.int64)]


def encode_scalar(x: float) -> int:
    """Nearest E4M3 code, ties to even mantissa, saturating above 448, NaN to NaN."""
    if math.isnan(x):
        return 0x7F
    sign = 0x80 if math.copysign(1.0, x) < 0 else 0
    a = abs(x)
    if a >= MAX_FINITE:
        return sign | 0x7E
    d = np.abs(_POS_VALUES - a)
    best = d.min()
    cands = _POS_CODES[d == best]
    if len(cands) == 1:
        code = int(cands[0])
    else:                                   # a tie between two neighbours: the even mantissa wins
        even = [int(c) for c in cands if (int(c) & 1) == 0]
        assert len(even) == 1
        code = even[0]
    return sign | code


def encode(x: np.ndarray, scale: float = 1.0) -> np.ndarray:
    """Codes of x / scale, elementwise (uint8); x is float32 (or float64 holding float32 values)."""
    flat = np.asarray(x, dtype=np.float64).reshape(-1) / float(scale)
    out = np.fromiter((encode_scalar(float(v)) for v in flat), dtype=np.uint8, count=flat.size)
    return out.reshape(np.shape(x))


def encode_fast(x: np.ndarray, scale: float = 1.0) -> np.ndarray:
    """The same codes as ``encode`` for large arrays: nearest neighbour by bisection over the sorted
    finite values, ties resolved to the even code, saturation and NaN as in ``encode_scalar``.
    Pinned against ``encode`` in the tests."""
    v = np.asarray(x, dtype=np.float64) / float(scale)
    a = np.abs(v)
    i = np.clip(np.searchsorted(_POS_VALUES, a), 1, len(_POS_VALUES) - 1)
    lo, hi = _POS_VALUES[i - 1], _POS_VALUES[i]
    dlo, dhi = a - lo, hi - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((_POS_CODES[i] & 1) == 0))
    code = np.where(pick_hi, _POS_CODES[i], _POS_CODES[i - 1]).astype(np.int64)
    code = np.where(a >= MAX_FINITE, 0x7E, code)
    code = np.where(a <= 0, 0, code)
    code = code | np.where(np.signbit(v), 0x80, 0)
    code = np.where(np.isnan(v), 0x7F, code)
    return code.astype(np.uint8)


def quantize(x: np.ndarray, scale: float) -> np.ndarray:
    """Codes of x / scale for a cache with per-tensor scale ``scale``: the quotient of the fp32
    values is rounded to fp32 (IEEE division), then encoded (nearest, ties even, saturating)."""
    xf = np.asarray(x, dtype=np.float32)
    qf = (xf / np.float32(scale)).astype(np.float32)
    return encode_fast(qf.astype(np.float64))


def dequantize(codes: np.ndarray, scale: float) -> np.ndarray:
    """The values a cache with per-tensor scale ``scale`` holds: scale * value(code), in fp64."""
    return float(scale) * decode(codes)
