"""Exact rational arithmetic helpers for pinning the oracle (no numpy math).

Everything here works on ``fractions.Fraction`` and Python integers, so the
results do not depend on numpy's float32 division or on the oracle's
encoder.  Used only by the oracle pin tests.
"""

import math
import struct
from fractions import Fraction

F32_MANT = 24          # significand bits including the hidden one
F32_EMIN = -126        # smallest normal exponent
F32_EMAX = 127


def f32_bits(x):
    return struct.unpack("<I", struct.pack("<f", x))[0]


def f32_from_bits(u):
    return struct.unpack("<f", struct.pack("<I", u & 0xFFFFFFFF))[0]


def round_half_even(q):
    """Nearest integer to the Fraction ``q``, ties to even."""
    fl = math.floor(q)
    rem = q - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def round_to_f32(q):
    """Round a non-negative or negative Fraction to the nearest float32 (ties even).

    Handles subnormals; raises on overflow (not needed by the tests).
    Returns a Python float holding the float32 value exactly.
    """
    if q == 0:
        return 0.0
    sign = -1 if q < 0 else 1
    a = abs(q)
    # exponent e with 2**e <= a < 2**(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, F32_EMIN)                      # subnormal range: fixed quantum
    quantum = Fraction(2) ** (e - (F32_MANT - 1))
    m = round_half_even(a / quantum)
    val = m * quantum
    if val >= Fraction(2) ** (F32_EMAX + 1):
        raise OverflowError("float32 overflow")
    return sign * float(val)


# e4m3 values from the format definition, as Fractions (codes 0x00..0x7E)
def e4m3_value(code):
    e = (code >> 3) & 0xF
    m = code & 7
    if e == 0:
        v = Fraction(m, 8) * Fraction(1, 64)
    else:
        v = (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return -v if code & 0x80 else v


E4M3_NONNEG = [e4m3_value(c) for c in range(0x7F)]


def nearest_e4m3(y):
    """Nearest e4m3 code to the rational ``y`` (|y| <= 448), ties to even code.

    ``y`` may be a Fraction or a float; -0.0 keeps its sign.
    """
    neg = (y < 0) or (isinstance(y, float) and math.copysign(1.0, y) < 0)
    a = abs(Fraction(y))
    if a > 448:
        raise ValueError("out of range")
    best, best_d = None, None
    for c, v in enumerate(E4M3_NONNEG):
        d = abs(a - v)
        if best is None or d < best_d or (d == best_d and c % 2 == 0):
            best, best_d = c, d
    return best | (0x80 if neg else 0)


EPS_F32 = Fraction(struct.unpack("<f", struct.pack("<f", 1e-12))[0])


def exact_quant_block(xs):
    """Quantize one block of float32-representable floats with exact rationals.

    amax -> max(amax, EPS) -> s = RN32(amax / 448) -> y = RN32(x / s) ->
    clamp to 448 -> nearest e4m3 (ties even).  Returns (codes, s as float).
    """
    amax = max(abs(Fraction(x)) for x in xs)
    amax = max(amax, EPS_F32)
    s = round_to_f32(amax / 448)
    codes = []
    for x in xs:
        y = round_to_f32(Fraction(x) / Fraction(s))
        if x == 0 or y == 0:
            y = -0.0 if math.copysign(1.0, x) < 0 else 0.0
        y = max(min(y, 448.0), -448.0)
        codes.append(nearest_e4m3(y))
    return codes, s
