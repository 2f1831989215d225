"""Gated FFN activation, CPU oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The FFN whose layers the pages test ("add FSDP and TP tests for
Float8BlockwiseLinear", summary: a ToyModel FFN with w1, w2 and out_proj,
w1 and w2 split by output columns under TP) combines the outputs of w1 and
w2 before out_proj; the reading taken is the gated form

    h = silu(a) * b,   silu(a) = a / (1 + exp(-a)),   a = w1 x,  b = w2 x.

Fusing the quantization of h into the kernel that produces it is the first
fusion next to the blockwise path.  The value quantized is h rounded ONCE to
bf16 (nearest, ties to even) from its exact value; here h is evaluated in
float64 (relative error ~1e-16, far below half a bf16 step) and then rounded.

The backward (the derivative of the same function, for the FFN's backward
pass) quantizes [da | db] for the dgrad and wgrad GEMMs of w1 and w2:

    da = dh * b * silu'(a),  silu'(a) = s (1 + a (1 - s)),  s = 1 / (1 + exp(-a))
    db = dh * silu(a)

each rounded once to bf16 from its float64 evaluation (1 - s is evaluated as
1 / (1 + exp(a)) so that no cancellation precedes the one near silu'(a) = 0,
where a (1 - s) = -1; there the float64 error stays ~1e-14 relative for bf16
inputs, still far below half a bf16 step).
"""

import numpy as np

from .quant import bf16_bits_to_f32

_BF16_MANT = 7          # explicit mantissa bits of bf16
_BF16_EMIN = -126       # smallest normal exponent (same as float32)
_BF16_MAX = float(np.float32(np.uint32(0x7F7F0000).view(np.float32)))


def round_to_bf16(v):
    """Float64 values -> bf16 bit patterns (uint16), round to nearest even,
    one rounding from the float64 value.  Overflow goes to +-inf."""
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("round_to_bf16 expects finite values")
    mag = np.abs(v)
    _, ex = np.frexp(mag)                      # mag = m * 2**ex, m in [0.5, 1)
    # value of one unit in the last place: 2**(ex-1-7) for normals, 2**-133
    # (the smallest subnormal) below the normal range
    ulp_exp = np.maximum(ex - 1 - _BF16_MANT, _BF16_EMIN - _BF16_MANT)
    q = np.rint(np.ldexp(mag, -ulp_exp))       # exact scaling; rint = ties to even
    r = np.ldexp(q, ulp_exp)
    r = np.where(r > _BF16_MAX, np.inf, r)
    r = np.copysign(r, v)                      # keeps the sign of zero
    bits = r.astype(np.float32).view(np.uint32) >> 16
    return bits.astype(np.uint16)


def swiglu_f64(a_bits, b_bits):
    """h = silu(a) * b for bf16 inputs (uint16 bit patterns) in float64, before
    its one rounding to bf16."""
    a = bf16_bits_to_f32(np.asarray(a_bits, dtype=np.uint16)).astype(np.float64)
    b = bf16_bits_to_f32(np.asarray(b_bits, dtype=np.uint16)).astype(np.float64)
    with np.errstate(over="ignore"):
        silu = a / (1.0 + np.exp(-a))          # exp overflow -> inf -> silu = -0
    return silu * b


def swiglu(a_bits, b_bits):
    """h = silu(a) * b for bf16 inputs (uint16 bit patterns), as bf16 bits."""
    return round_to_bf16(swiglu_f64(a_bits, b_bits))


def swiglu_backward_f64(a_bits, b_bits, dh_bits):
    """(da, db) of h = silu(a) * b for bf16 a, b and upstream gradient dh
    (uint16 bit patterns) in float64, before their one rounding to bf16."""
    a = bf16_bits_to_f32(np.asarray(a_bits, dtype=np.uint16)).astype(np.float64)
    b = bf16_bits_to_f32(np.asarray(b_bits, dtype=np.uint16)).astype(np.float64)
    dh = bf16_bits_to_f32(np.asarray(dh_bits, dtype=np.uint16)).astype(np.float64)
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-a))           # sigmoid(a)
        sn = 1.0 / (1.0 + np.exp(a))           # sigmoid(-a) = 1 - s
    silu = a * s
    da = dh * b * s * (1.0 + a * sn)
    db = dh * silu
    return da, db


def swiglu_backward(a_bits, b_bits, dh_bits):
    """(da, db) of h = silu(a) * b for bf16 a, b and upstream gradient dh
    (uint16 bit patterns), each rounded once to bf16 bits."""
    da, db = swiglu_backward_f64(a_bits, b_bits, dh_bits)
    return round_to_bf16(da), round_to_bf16(db)
