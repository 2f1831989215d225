"""OCP FP8 E4M3 ("FN" variant): decode table and RNE-with-saturation encoder.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages say "float8" (prototype page, description) and never name the
encoding.  The recipe they describe is the e4m3 one with a maximum of 448
(the training recipe's definition: scale = amax / 448), which is the OCP
8-bit floating point specification's E4M3 format:

* 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
* exponent field 0 is subnormal: value = (m / 8) * 2**-6;
* otherwise value = (1 + m / 8) * 2**(e - 7);
* exponent 15 with mantissa 7 (codes 0x7F, 0xFF) is NaN; there are no
  infinities, so the largest finite magnitude is 1.75 * 2**8 = 448 (0x7E).

Encoding: round to nearest, ties to the even code (for non-negative values
code order equals value order, so "even code" is "even mantissa"), sign kept
for values that round to zero, and magnitudes at or beyond 448 saturate to
448 -- never NaN.
"""

import math

import numpy as np

EXP_BIAS = 7
MAX_FINITE = 448.0
NAN_CODES = (0x7F, 0xFF)


def decode_code(code):
    """Value of one e4m3 code, straight from the bit fields (float64)."""
    code = int(code)
    negative = bool(code & 0x80)
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        mag = (m / 8.0) * 2.0 ** (1 - EXP_BIAS)
    else:
        mag = (1.0 + m / 8.0) * 2.0 ** (e - EXP_BIAS)
    return -mag if negative else mag


# Value of every code, float64 (every e4m3 value is exact in float64).
DECODE = np.array([decode_code(c) for c in range(256)], dtype=np.float64)

# The 127 finite non-negative values, in code order 0x00 .. 0x7E; ascending.
_NONNEG = DECODE[:0x7F].copy()


def encode_scalar(y):
    """Encode one finite real ``y`` (a Python or numpy float) to an e4m3 code.

    Plain linear search over the 127 finite non-negative values: take the
    nearest to |y|; on an exact tie take the even code; saturate at 448; put
    the sign of ``y`` (also of -0.0 and of negatives that round to zero) in
    bit 7.
    """
    y = float(y)
    if math.isnan(y) or math.isinf(y):
        raise ValueError("e4m3 encoder: input must be finite")
    sign = 0x80 if math.copysign(1.0, y) < 0 else 0x00
    a = abs(y)
    if a >= MAX_FINITE:
        return sign | 0x7E
    best = 0
    best_err = abs(a - _NONNEG[0])
    for c in range(1, 0x7F):
        err = abs(a - _NONNEG[c])
        if err < best_err or (err == best_err and c % 2 == 0):
            best, best_err = c, err
    return sign | best


def encode(y):
    """Vectorized form of :func:`encode_scalar` for a float32 array.

    For each |y| find the two neighbouring table values by binary search and
    pick the nearer; equal distances go to the even code.  Differences are
    taken in float64.  For |y| >= 2**-10 (the smallest midpoint between two
    e4m3 values) both |y| and the table values are multiples of 2**-33 below
    2**9, so the differences are exact and ties are seen exactly.  Below
    2**-10 the neighbours are 0 and 2**-9 and the exact distance to 2**-9
    exceeds 2**-10 > |y|, which monotone rounding preserves, so the choice of
    0 is still right.
    """
    y = np.asarray(y)
    if y.dtype != np.float32:
        raise TypeError("e4m3.encode expects float32")
    if not np.all(np.isfinite(y)):
        raise ValueError("e4m3 encoder: input must be finite")
    neg = np.signbit(y)
    a = np.minimum(np.abs(y).astype(np.float64), MAX_FINITE)
    hi = np.searchsorted(_NONNEG, a, side="left")  # first table value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_hi = _NONNEG[hi] - a
    d_lo = a - _NONNEG[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    # exact hits of a table value: searchsorted(left) lands on it, d_hi == 0
    code = np.where(d_hi == 0, hi, code).astype(np.uint8)
    return code | np.where(neg, 0x80, 0x00).astype(np.uint8)


def decode(codes):
    """Vectorized decode of a uint8 array to float64 (NaN codes give NaN)."""
    return DECODE[np.asarray(codes, dtype=np.uint8)]
