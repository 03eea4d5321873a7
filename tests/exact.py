"""Exact rational reference arithmetic for pinning the oracle (tests only).

Everything here is written from the format definitions with Python's
``fractions.Fraction``: fp32 rounding of a rational (nearest, ties to even,
subnormals kept), the E4M3FN value set, and nearest-magnitude encoding by
brute force.  It shares nothing with the C oracle.
"""
from __future__ import annotations

import bisect
import struct
from fractions import Fraction

F32_MIN_EXP = -126      # smallest normal exponent
F32_MANT = 23           # explicit mantissa bits
F32_MAX = Fraction(2) ** 128 - Fraction(2) ** (128 - 24)


def f32_bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


def bits_f32(b: int) -> float:
    return struct.unpack("<f", struct.pack("<I", b & 0xFFFFFFFF))[0]


def round_f32(q: Fraction, negative_zero: bool = False) -> float:
    """Nearest fp32 to the rational q, ties to even; overflow gives inf."""
    if q == 0:
        return -0.0 if negative_zero else 0.0
    neg = q < 0
    a = -q if neg else q
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    # now 2^e <= a < 2^(e+1)
    e = max(e, F32_MIN_EXP)
    quantum = Fraction(2) ** (e - F32_MANT)
    m = a / quantum
    n = m.numerator // m.denominator
    r = m - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    v = n * quantum
    if v > F32_MAX:
        out = float("inf")
    else:
        out = float(v)  # exact: v is an fp32 value
    return -out if neg else out


def e4m3_magnitudes():
    """[(code, Fraction value)] for the 127 finite non-negative E4M3FN codes."""
    out = []
    for e in range(16):
        for m in range(8):
            if e == 15 and m == 7:
                continue  # NaN
            v = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
            out.append(((e << 3) | m, v))
    return out


_MAGS = e4m3_magnitudes()
_MAG_VALUES = [v for _, v in _MAGS]  # increasing with the code


def e4m3_value(code: int) -> Fraction:
    mag = dict(_MAGS)[code & 0x7F]
    return -mag if code & 0x80 else mag


def e4m3_nearest(y: float) -> int:
    """Brute force: nearest finite magnitude, ties to even code, >= 448 -> 0x7E,
    sign bit copied from y."""
    sign = 0x80 if (f32_bits(y) >> 31) else 0
    a = abs(Fraction(y))
    if a >= 448:
        return sign | 0x7E
    hi = bisect.bisect_right(_MAG_VALUES, a)  # first magnitude > a
    best = None
    for code in (hi - 1, hi):  # the two neighbours of a
        d = abs(a - _MAG_VALUES[code])
        if best is None or d < best[0] or (d == best[0] and code % 2 == 0):
            best = (d, code)
    return sign | best[1]


def quantize_tile_exact(xs):
    """Quantize one tile (iterable of fp32-representable Python floats) by the
    library's rule, evaluated with exact rationals and explicit fp32 rounding.
    Returns (codes list, scale float)."""
    xs = list(xs)
    amax = max(abs(Fraction(x)) for x in xs) if xs else Fraction(0)
    s = round_f32(amax / 448)
    codes = []
    for x in xs:
        neg = f32_bits(x) >> 31
        if s == 0:
            codes.append(0x80 if neg else 0x00)
        else:
            y = round_f32(Fraction(x) / Fraction(s), negative_zero=bool(neg))
            codes.append(e4m3_nearest(y))
    return codes, s


def pow2_scale_exact(amax: Fraction) -> Fraction:
    """Power-of-two scale from its closed form: with amax = r * 2^E,
    1 <= r < 2, the smallest e with 448 * 2^e = 1.75 * 2^(e+8) >= r * 2^E is
    E - 8 when r <= 1.75 and E - 7 otherwise; not below 2^-127; 0 for 0."""
    if amax == 0:
        return Fraction(0)
    E = amax.numerator.bit_length() - amax.denominator.bit_length()
    if Fraction(2) ** E > amax:
        E -= 1
    r = amax / Fraction(2) ** E
    e = E - 8 if r <= Fraction(7, 4) else E - 7
    return Fraction(2) ** max(e, -127)


def quantize_tile_exact_pow2(xs):
    """The power-of-two variant of quantize_tile_exact: (codes, scale)."""
    xs = list(xs)
    amax = max(abs(Fraction(x)) for x in xs) if xs else Fraction(0)
    s = pow2_scale_exact(amax)
    codes = []
    for x in xs:
        neg = f32_bits(x) >> 31
        if s == 0:
            codes.append(0x80 if neg else 0x00)
        else:
            y = round_f32(Fraction(x) / s, negative_zero=bool(neg))
            codes.append(e4m3_nearest(y))
    return codes, float(s)
