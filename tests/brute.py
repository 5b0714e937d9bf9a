"""Brute-force reference arithmetic for pinning the oracle, in pure Python.

Every binary32 operation is done exactly on ``fractions.Fraction`` values and
then rounded to the nearest binary32 (ties to even) by ``round_f32`` below,
which is written from the IEEE 754 definition with integer arithmetic only.
Nothing here relies on the host's floating-point unit, on numpy's float32 or
on the C compiler that built the oracle, so it can catch a contracted
multiply-add, a reordered product or a reciprocal in place of a division.
Integer dot products use Python's unbounded ``int``.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction

F32_MANT = 24            # significand bits including the implicit one
F32_EMIN = -126          # smallest normal exponent
F32_SUB_SCALE = 149      # 2^-149 is the smallest subnormal


def _round_half_even_int(q: Fraction) -> int:
    """Nearest integer to a non-negative rational, ties to even."""
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2):
        return n + 1
    if rem < Fraction(1, 2):
        return n
    return n if n % 2 == 0 else n + 1


def _floor_log2(q: Fraction) -> int:
    """floor(log2(q)) for q > 0, exactly."""
    e = q.numerator.bit_length() - q.denominator.bit_length()
    # now 2^(e-1) < q < 2^(e+1); fix up
    if Fraction(2) ** e > q:
        e -= 1
    return e


def round_f32(q) -> float:
    """Round a rational to the nearest binary32 value (ties to even).
    Returns it as a Python float (binary64 holds every binary32 exactly)."""
    q = Fraction(q)
    if q == 0:
        return 0.0
    sign = -1 if q < 0 else 1
    a = -q if q < 0 else q
    e = _floor_log2(a)
    if e < F32_EMIN:
        # subnormal range: a multiple of 2^-149
        n = _round_half_even_int(a * (Fraction(2) ** F32_SUB_SCALE))
        return sign * float(Fraction(n, 2 ** F32_SUB_SCALE))
    scale = Fraction(2) ** (F32_MANT - 1 - e)
    n = _round_half_even_int(a * scale)          # in [2^23, 2^24]
    val = Fraction(n) / scale
    if val >= Fraction(2) ** 128:
        return sign * float("inf")
    return sign * float(val)


def f32(v) -> Fraction:
    """Exact rational value of a binary32 number given as float/np.float32."""
    return Fraction(float(v))


def f32_bits(v: float) -> int:
    return struct.unpack("<I", struct.pack("<f", v))[0]


def smoothed(x, s) -> float:
    """fl(x/s) for binary32 x and a finite s > 0, exactly rounded; a NaN x
    gives NaN, an infinite x the same infinity, and a quotient beyond the
    binary32 range rounds to an infinity (IEEE overflow)."""
    xf = float(x)
    if math.isnan(xf) or math.isinf(xf):
        return xf
    return round_f32(f32(x) / f32(s))


def quantize_row(x_row, s_row):
    """Per-token quantisation of one row, each binary32 step done exactly and
    rounded: x' = fl(x/s); amax = max|x'|; sx = fl(amax/127);
    q = clamp(rne(fl(x'/sx)), -127, 127), q = 0 when sx = 0.  A row with a
    non-finite x' has no scale: sx = NaN and every q = 0."""
    xs = [smoothed(x, s) for x, s in zip(x_row, s_row)]
    if any(not math.isfinite(v) for v in xs):
        return [0] * len(xs), float("nan")
    amax = max(abs(v) for v in xs)
    sx = round_f32(Fraction(amax) / 127)
    q = []
    for v in xs:
        if sx == 0:
            q.append(0)
            continue
        t = Fraction(round_f32(Fraction(v) / Fraction(sx)))
        r = _round_half_even_int(abs(t)) * (1 if t >= 0 else -1)
        q.append(max(-127, min(127, r)))
    return q, sx


def dot(a, b) -> int:
    return sum(int(x) * int(y) for x, y in zip(a, b))


def epilogue(acc: int, sx, sw, r=None) -> float:
    """fl(fl(fl(float(acc)) * sx) * sw) (+ r, rounded once more)."""
    t0 = round_f32(Fraction(int(acc)))
    t1 = round_f32(Fraction(t0) * f32(sx))
    t2 = round_f32(Fraction(t1) * f32(sw))
    if r is None:
        return t2
    return round_f32(Fraction(t2) + f32(r))


def softmax_decimal(row, digits=40):
    """Softmax of one row of binary32 logits, computed in decimal arithmetic
    with ``digits`` significant digits (``Decimal.exp`` rounds correctly at
    that precision), then rounded to binary64.  A reference far more accurate
    than any binary64 implementation, for bounding one in units in the last
    place."""
    from decimal import Decimal, localcontext
    with localcontext() as ctx:
        ctx.prec = digits
        z = [Decimal(float(v)) for v in row]        # binary32 -> exact decimal
        mx = max(z)
        e = [(v - mx).exp() for v in z]
        s = sum(e, Decimal(0))
        return [float(v / s) for v in e]


def quantize_row_amax(x_row, s_row, amax):
    """Quantisation of one row with a given per-token maximum (the global one
    of a row-parallel layer), each binary32 step exact then rounded:
    sx = fl(amax/127); q = clamp(rne(fl(fl(x/s)/sx)), -127, 127), 0 when sx = 0.
    A maximum that is NaN, negative or infinite gives sx = NaN and every q = 0;
    otherwise an element whose quotient is NaN gives 0 and an infinite one
    clamps to +-127."""
    a = float(amax)
    if not (math.isfinite(a) and a >= 0):
        return [0] * len(x_row), float("nan")
    sx = round_f32(f32(amax) / 127)
    q = []
    for x, s in zip(x_row, s_row):
        if sx == 0:
            q.append(0)
            continue
        v = smoothed(x, s)
        if math.isnan(v):
            q.append(0)
            continue
        if math.isinf(v):
            q.append(127 if v > 0 else -127)
            continue
        tf = round_f32(Fraction(v) / Fraction(sx))
        if math.isinf(tf):
            q.append(127 if tf > 0 else -127)
            continue
        t = Fraction(tf)
        r = _round_half_even_int(abs(t)) * (1 if t >= 0 else -1)
        q.append(max(-127, min(127, r)))
    return q, sx
