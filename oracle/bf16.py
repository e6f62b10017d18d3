"""bf16 <-> fp64 for the oracle (test infrastructure only).

bf16 is the top half of an IEEE-754 binary32: 1 sign bit, 8 exponent bits
(bias 127), 7 stored fraction bits.  Decoding is exact in fp64.  Encoding an
fp64 value rounds to the nearest representable bf16, ties to the value whose
last fraction bit is 0; magnitudes at or beyond the midpoint between the
largest finite bf16 (2^127 * (2 - 2^-7)) and 2^128 become infinity; NaN maps to
the quiet NaN 0x7FC0.  This is written from that definition (decompose the
value into sign, binade and scaled significand), not by truncating a float32.
"""
import math

import numpy as np

_MIN_EXP = -126          # exponent of the smallest normal bf16
_FRAC = 7                # stored fraction bits


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16 array) -> exact fp64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32)
    sign = np.where(b >> 15, -1.0, 1.0)
    e = ((b >> 7) & 0xFF).astype(np.int64)
    f = (b & 0x7F).astype(np.float64)
    normal = sign * np.ldexp(1.0 + f / 128.0, (e - 127).astype(np.int64))
    sub = sign * np.ldexp(f, _MIN_EXP - _FRAC)  # f * 2^-133
    out = np.where(e == 0, sub, normal)
    out = np.where((e == 0xFF) & (f == 0), sign * np.inf, out)
    out = np.where((e == 0xFF) & (f != 0), np.nan, out)
    return out


def _encode_one(x: float) -> int:
    if math.isnan(x):
        return 0x7FC0
    s = 0x8000 if math.copysign(1.0, x) < 0 else 0
    a = abs(x)
    if a == 0.0:
        return s
    if math.isinf(a):
        return s | 0x7F80
    m, e = math.frexp(a)          # a = m * 2^e, 0.5 <= m < 1
    exp = e - 1                   # a = (2m) * 2^exp, 1 <= 2m < 2
    if exp < _MIN_EXP:            # subnormal range: quantum 2^-133
        q = a / math.ldexp(1.0, _MIN_EXP - _FRAC)
        n = _round_half_even(q)
        return s | n              # n == 128 lands on the smallest normal (0x0080)
    q = (2.0 * m) * 128.0         # significand in units of the last place: [128, 256)
    n = _round_half_even(q)
    if n == 256:                  # rounded up into the next binade
        n, exp = 128, exp + 1
    if exp > 127:
        return s | 0x7F80
    return s | ((exp + 127) << 7) | (n - 128)


def _round_half_even(q: float) -> int:
    fl = math.floor(q)
    r = q - fl                    # exact: q has few significant bits above the point
    if r > 0.5 or (r == 0.5 and (fl % 2) == 1):
        return int(fl) + 1
    return int(fl)


def f64_to_bf16_rne(x) -> np.ndarray:
    """fp64 values -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    a = np.asarray(x, dtype=np.float64)
    flat = a.reshape(-1)
    out = np.empty(flat.shape[0], dtype=np.uint16)
    # Vectorised path for finite values in the normal range; the per-element
    # definition above handles everything else (and is what the tests pin).
    fin = np.isfinite(flat) & (flat != 0)
    safe = np.where(fin, flat, 1.0)
    m, e = np.frexp(np.abs(safe))
    exp = e.astype(np.int64) - 1
    fin &= (exp >= _MIN_EXP) & (exp <= 127)
    q = 2.0 * m * 128.0
    fl = np.floor(q)
    r = q - fl
    up = (r > 0.5) | ((r == 0.5) & (np.mod(fl, 2) == 1))
    n = fl.astype(np.int64) + up
    carry = n == 256
    n = np.where(carry, 128, n)
    exp2 = exp + carry
    sgn = np.where(np.signbit(flat), 0x8000, 0)
    bits = sgn | ((exp2 + 127) << 7) | (n - 128)
    bits = np.where(exp2 > 127, sgn | 0x7F80, bits)
    out[fin] = bits[fin].astype(np.uint16)
    for i in np.nonzero(~fin)[0]:
        out[i] = _encode_one(float(flat[i]))
    return out.reshape(a.shape)
