"""Exact rational arithmetic with explicit IEEE-754 rounding, for pinning the oracle.

Every value is a Python Fraction; a binary32 operation is the exact rational
result rounded by ``round_binary32`` (nearest, ties to even, with gradual
underflow and overflow to infinity).  This is an independent route to the
numbers the oracle computes with hardware float operations.
"""
import math
from fractions import Fraction

HALF = Fraction(1, 2)


def rne_int(fr):
    """Round a Fraction to the nearest integer, ties to even."""
    fl = math.floor(fr)
    rem = fr - fl
    if rem > HALF or (rem == HALF and fl % 2 == 1):
        fl += 1
    return fl


def _exp2_floor(a):
    """Largest e with 2^e <= a, for a > 0."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_binary(fr, mant_bits, emin, emax):
    """Round to a binary format with ``mant_bits`` significand bits (incl. the
    hidden one), minimum normal exponent ``emin`` and maximum exponent ``emax``.
    Returns a Fraction, or +-inf as float."""
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = max(_exp2_floor(a), emin)
    quantum = Fraction(2) ** (e - (mant_bits - 1))
    n = rne_int(a / quantum)
    v = n * quantum
    if v >= Fraction(2) ** (emax + 1):
        return sign * math.inf
    return sign * v


def round_binary32(fr):
    return round_binary(Fraction(fr), 24, -126, 127)


def round_bf16(fr):
    return round_binary(Fraction(fr), 8, -126, 127)


def f32(fr):
    """binary32 rounding of an exact value, returned as a Python float."""
    v = round_binary32(fr)
    return float(v)


def quant_row_exact(xs, scales=None):
    """The dynamic-int8 formula evaluated exactly, each binary32 operation
    rounded once: returns (q list, scale float)."""
    H = len(xs)
    s = scales if scales is not None else [1.0] * H
    xf = [round_binary32(Fraction(x) * Fraction(float(si))) for x, si in zip(xs, s)]
    amax = max(abs(v) for v in xf)
    if amax == 0:
        return [0] * H, 0.0
    dyn = round_binary32(Fraction(127) / amax)
    if dyn == math.inf:
        q = [0 if v == 0 else (127 if v > 0 else -127) for v in xf]
        return q, 0.0
    q = []
    for v in xf:
        p = round_binary32(v * dyn)
        if p == math.inf or p == -math.inf:
            r = 127 if p > 0 else -127
        else:
            r = rne_int(Fraction(p))
        q.append(max(-127, min(127, r)))
    scale = round_binary32(Fraction(1) / dyn)
    return q, float(scale)
