"""Exact-arithmetic helpers for pinning the oracle (tests only).

Written independently of the oracle: rational arithmetic with
``fractions.Fraction`` and explicit enumeration of representable values.
"""
import bisect
import math
import struct
from fractions import Fraction

import numpy as np


def f32_bits(x):
    return struct.unpack("<I", struct.pack("<f", float(x)))[0]


def bits_f32(b):
    return struct.unpack("<f", struct.pack("<I", int(b) & 0xFFFFFFFF))[0]


def bf16_value(bits):
    """Float value of a bf16 bit pattern (the top 16 bits of a binary32)."""
    return bits_f32((int(bits) & 0xFFFF) << 16)


_POS_BF16 = None  # sorted (Fraction value, bits) of every positive finite bf16


def _pos_bf16():
    global _POS_BF16
    if _POS_BF16 is None:
        vals = []
        for b in range(0x0000, 0x7F80):  # +0 .. largest finite
            vals.append((Fraction(bf16_value(b)), b))
        vals.sort()
        _POS_BF16 = ([v for v, _ in vals], [b for _, b in vals])
    return _POS_BF16


def round_to_bf16(value):
    """Exact round-to-nearest-even of a real (Fraction/int/float) to bf16 bits.

    NaN and infinities must be handled by the caller.
    """
    v = Fraction(value)
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    vals, bits = _pos_bf16()
    top = vals[-1]
    ulp_top = top - vals[-2]
    if a >= top + ulp_top / 2:
        # exactly halfway rounds to even; the largest finite has an odd pattern
        return sign | 0x7F80
    i = bisect.bisect_left(vals, a)
    if i < len(vals) and vals[i] == a:
        return sign | bits[i]
    lo_v, lo_b = vals[i - 1], bits[i - 1]
    if i == len(vals):
        return sign | lo_b
    hi_v, hi_b = vals[i], bits[i]
    d_lo, d_hi = a - lo_v, hi_v - a
    if d_lo < d_hi:
        return sign | lo_b
    if d_hi < d_lo:
        return sign | hi_b
    return sign | (lo_b if lo_b % 2 == 0 else hi_b)


def round_to_f32(value):
    """Exact round-to-nearest-even of a finite real to float32 (returns np.float32)."""
    v = Fraction(value)
    approx = np.float32(float(v))
    cands = {float(approx),
             float(np.nextafter(approx, np.float32(np.inf))),
             float(np.nextafter(approx, np.float32(-np.inf)))}
    best = None
    for c in sorted(cands):
        if math.isinf(c):
            continue
        d = abs(Fraction(c) - v)
        key = (d, f32_bits(c) & 1)  # ties: prefer the even pattern
        if best is None or key < best[0]:
            best = (key, c)
    return np.float32(best[1])


def bf16_ordered(bits):
    """Map bf16 patterns to integers in numeric order (sign-magnitude -> two's complement)."""
    b = np.asarray(bits, dtype=np.int64) & 0xFFFF
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def bf16_ulp_diff(a_bits, b_bits):
    """|difference| in bf16 units in the last place; +0 and -0 are the same point."""
    return np.abs(bf16_ordered(a_bits) - bf16_ordered(b_bits))
