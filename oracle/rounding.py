"""Roundings used by the codec, written from the number-format definitions.

Test infrastructure only (see the package docstring).

* fp32: IEEE-754 binary32, round to nearest, ties to even; subnormals kept.
* bf16: the upper 16 bits of binary32 (8 significant bits, same exponent
  range), round to nearest, ties to even.  The pages fix BFloat16 as the
  compute type ("qlora" entry, section "a ideia").
* e4m3 ("fn" variant): 1 sign, 4 exponent bits with bias 7, 3 mantissa bits;
  exponent field 0 holds subnormals (m * 2^-9); no infinities; the patterns
  0x7F / 0xFF are NaN; largest finite value 448.  The pages only say "FP8"
  ("qlora" entry, section "como funciona"); e4m3 is the reading taken.
  Encoding is round to nearest, ties to the even mantissa (subnormals
  included), and saturating: any magnitude at or above 448 encodes as 448.
  NaN is never produced.  Negative values that round to zero encode as 0x80.

Pins (tests/test_oracle_rounding.py): bf16 and e4m3 against exact Fraction
brute force over the whole representable set; bf16 against torch's CPU cast;
e4m3 against torch's CPU float8_e4m3fn cast of clamped values; every e4m3
byte decodes and re-encodes to itself.
"""

import math
from fractions import Fraction

import numpy as np

E4M3_MAX = 448.0


def rn32_from_fraction(q: Fraction) -> np.float32:
    """Round an exact rational to the nearest binary32 value, ties to even."""
    if q == 0:
        return np.float32(0.0)
    neg = q < 0
    q = -q if neg else q
    n, d = q.numerator, q.denominator
    # e = floor(log2 q)
    e = n.bit_length() - d.bit_length()
    if (n << max(0, -e)) < (d << max(0, e)):
        e -= 1
    qe = max(e - 23, -149)  # exponent of the last kept bit (subnormals floor at 2^-149)
    if qe >= 0:
        num, den = n, d << qe
    else:
        num, den = n << (-qe), d
    m, r = divmod(num, den)
    if 2 * r > den or (2 * r == den and (m & 1)):
        m += 1
    val = math.ldexp(m, qe)  # exact: m <= 2^24
    f = np.float32(val)
    assert float(f) == val, "binary32 overflow"
    return np.float32(-f) if neg else f


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) exactly to fp32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_rne_bits(x: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bf16 (nearest, ties to even); returns uint16 bits.

    Dropping the low 16 bits of a binary32 pattern truncates the significand
    to 8 bits; adding 0x7FFF plus the kept least-significant bit before the
    shift rounds to nearest with ties to even, and a carry out of the
    significand moves correctly into the exponent.
    """
    x = np.asarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("bf16_rne_bits: non-finite input")
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    return ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)


def _e4m3_value(byte: int) -> float:
    s = -1.0 if byte & 0x80 else 1.0
    e = (byte >> 3) & 0xF
    m = byte & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (8 + m) * 2.0 ** (e - 10)


_E4M3_TABLE = np.array([_e4m3_value(b) for b in range(256)], dtype=np.float64)


def e4m3_decode(q: np.ndarray) -> np.ndarray:
    """Decode e4m3 bytes to their exact values (returned as fp32; all are exact)."""
    return _E4M3_TABLE[np.asarray(q, dtype=np.uint8)].astype(np.float32)


def _e4m3_positive_values():
    return sorted({abs(v) for v in _E4M3_TABLE if not math.isnan(v)})


def e4m3_encode_exact(q: Fraction) -> int:
    """Brute-force e4m3 encoding of an exact rational (the reference definition).

    Nearest representable value; on a tie the one whose mantissa is even;
    magnitudes at or above 448 saturate to 448.
    """
    neg = q < 0
    a = -q if neg else q
    best = None
    for v in _e4m3_positive_values():
        dist = abs(a - Fraction(v))
        byte = _encode_positive_value(v)
        key = (dist, byte & 1)  # smaller distance first, then even mantissa
        if best is None or key < best[0]:
            best = (key, byte)
    byte = best[1]
    if a >= E4M3_MAX:
        byte = _encode_positive_value(E4M3_MAX)
    return byte | (0x80 if neg else 0)


def _encode_positive_value(v: float) -> int:
    """Byte of an exactly representable non-negative e4m3 value."""
    if v == 0.0:
        return 0
    if v < 2.0 ** -6:
        m = v / 2.0 ** -9
        assert m == int(m)
        return int(m)
    e = math.floor(math.log2(v))
    while 2.0 ** e > v:
        e -= 1
    while 2.0 ** (e + 1) <= v:
        e += 1
    m = v / 2.0 ** (e - 3) - 8
    assert m == int(m) and 0 <= m < 8
    return ((e + 7) << 3) | int(m)


def e4m3_encode_f64(v: np.ndarray) -> np.ndarray:
    """Vectorised e4m3 encoding of fp64 values (nearest, ties even, saturating).

    Used on fp64 quotients of two fp32 numbers.  Such a quotient, rounded once
    to fp64, rounds to the same e4m3 value as the exact real quotient: every
    e4m3 rounding boundary has at most 5 significant bits, so a non-zero gap
    between a quotient of two 24-bit significands and a boundary is at least
    about 2^-30 relative, far above the 2^-53 error of the fp64 division.
    tests/test_oracle_rounding.py checks this function against
    ``e4m3_encode_exact`` on random and boundary-hugging inputs.
    """
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("e4m3_encode_f64: non-finite input")
    neg = np.signbit(v)
    a = np.abs(v)
    _, k = np.frexp(a)  # a = f * 2^k with f in [0.5, 1)
    e = k.astype(np.int64) - 1  # floor(log2 a) for a > 0
    qexp = np.where(a >= 2.0 ** -6, e - 3, -9)  # exponent of the mantissa's last bit
    m = np.rint(np.ldexp(a, -qexp))  # exact scaling; rint rounds half to even
    val = np.ldexp(m, qexp)
    val = np.where(a >= E4M3_MAX, E4M3_MAX, val)
    # bytes of the rounded magnitudes
    normal = val >= 2.0 ** -6
    _, k2 = np.frexp(np.where(normal, val, 1.0))
    e2 = k2.astype(np.int64) - 1
    mant_n = np.ldexp(val, -(e2 - 3)) - 8
    byte_n = ((e2 + 7) << 3) + mant_n.astype(np.int64)
    byte_s = np.ldexp(val, 9).astype(np.int64)
    byte = np.where(normal, byte_n, byte_s)
    byte = byte | np.where(neg, 0x80, 0)
    return byte.astype(np.uint8)
