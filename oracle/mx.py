"""MX (microscaling) FP8 quantizer and GEMM, CPU oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name an MXFP8 recipe ("[mxfp8 moe training] use new 3d colwise
quantization kernel", summary and microbenchmark table: the MXFP8 scaled
grouped GEMMs and a kernel quantizing 3-D expert weights along columns) but
do not define the format.  The reading taken is the OCP Microscaling (MX)
v1.0 definition of MXFP8 with E4M3 elements:

1. blocks of 32 consecutive values along the contraction dimension (for the
   column form: 32 consecutive rows of one column);
2. one shared scale X = 2^e per block, stored as E8M0 (the byte e + 127),
   e = floor(log2(amax)) - 8, where 8 is the exponent of the largest normal
   E4M3 value (448 = 1.75 * 2^8); e is clamped to [-127, 127] and a block
   whose amax is zero takes e = -127 (the smallest scale);
3. every element q = e4m3(clamp(x / X, -448, 448)), round to nearest even,
   sign kept.  x / X is exact (X is a power of two, x a bf16).

With e = floor(log2(amax)) - 8, amax / X lies in [256, 512): values above 448
saturate (the scale is not rounded up), as the definition states.

Operand orientation as in ``quant.py``: ``q`` is [rows, K] with K the
contraction dimension; the logical scale array is [rows, K/32] of E8M0
bytes.
"""

import numpy as np

from . import e4m3
from .quant import _check_finite, bf16_bits_to_f32

MX_BLOCK = 32
E4M3_EMAX = 8           # exponent of 448 = 1.75 * 2^8
E8M0_BIAS = 127
E_MIN, E_MAX = -127, 127


def scale_exponent(amax):
    """e = floor(log2(amax)) - 8, clamped to [-127, 127]; amax == 0 -> -127.
    amax: float array of non-negative values (exact floor via frexp)."""
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(amax)                     # amax = m * 2**ex, m in [0.5, 1)
    e = ex.astype(np.int64) - 1 - E4M3_EMAX
    e = np.where(amax == 0, E_MIN, e)
    return np.clip(e, E_MIN, E_MAX)


def _encode_scaled(x, e):
    """Codes of x (float32 array) under scales 2**e (broadcastable ints)."""
    y = np.ldexp(x.astype(np.float64), -e)     # exact: x / 2**e
    y = np.clip(y, -448.0, 448.0)              # saturate (sign of zero kept by clip)
    return e4m3.encode(y.astype(np.float32))   # exact: y has <= 8 significant bits, or encodes to 0


def quant_mx_rowwise(x_bits):
    """MX blocks of 32 along each row: x [R, C] bf16 bits -> (q [R, C] uint8,
    s [R, C/32] E8M0 uint8)."""
    x = bf16_bits_to_f32(x_bits)
    _check_finite(x)
    R, C = x.shape
    if C % MX_BLOCK:
        raise ValueError("quant_mx_rowwise: C must be a multiple of 32")
    blocks = x.reshape(R, C // MX_BLOCK, MX_BLOCK)
    e = scale_exponent(np.abs(blocks).max(axis=2))            # [R, C/32]
    q = _encode_scaled(blocks, e[:, :, None]).reshape(R, C)
    return q, (e + E8M0_BIAS).astype(np.uint8)


def quant_mx_colwise(x_bits):
    """MX blocks of 32 consecutive rows of each column, in the orientation of
    the wgrad operand: x [R, C] -> (q^T [C, R], s [C, R/32])."""
    xt = np.ascontiguousarray(np.asarray(x_bits, dtype=np.uint16).T)
    return quant_mx_rowwise(xt)


def quant_mx_rowwise_scalar(x_bits):
    """The same definition block by block and element by element (small
    inputs): amax, exponent by repeated halving/doubling, each element
    divided and encoded with the scalar encoder."""
    x = bf16_bits_to_f32(x_bits)
    _check_finite(x)
    R, C = x.shape
    if C % MX_BLOCK:
        raise ValueError("quant_mx_rowwise_scalar: C must be a multiple of 32")
    q = np.zeros((R, C), dtype=np.uint8)
    s = np.zeros((R, C // MX_BLOCK), dtype=np.uint8)
    for r in range(R):
        for b in range(C // MX_BLOCK):
            vals = [float(v) for v in x[r, b * MX_BLOCK:(b + 1) * MX_BLOCK]]
            amax = max(abs(v) for v in vals)
            if amax == 0.0:
                e = E_MIN
            else:
                k = 0                                # 2**k <= amax < 2**(k+1)
                while 2.0 ** k > amax:
                    k -= 1
                while 2.0 ** (k + 1) <= amax:
                    k += 1
                e = min(max(k - E4M3_EMAX, E_MIN), E_MAX)
            s[r, b] = e + E8M0_BIAS
            for i, v in enumerate(vals):
                y = v / 2.0 ** e
                y = max(-448.0, min(448.0, y)) if y != 0.0 else y
                q[r, b * MX_BLOCK + i] = e4m3.encode_scalar(y)
    return q, s


def dequant_mx(q, s):
    """Codes [rows, K] and E8M0 scales [rows, K/32] -> float64 [rows, K]."""
    q = np.asarray(q, dtype=np.uint8)
    rows, K = q.shape
    if K % MX_BLOCK:
        raise ValueError("dequant_mx: K must be a multiple of 32")
    s = np.asarray(s, dtype=np.uint8)
    if s.shape != (rows, K // MX_BLOCK):
        raise ValueError(f"dequant_mx: scale shape {s.shape}, expected {(rows, K // MX_BLOCK)}")
    if (s == 255).any():
        raise ValueError("dequant_mx: E8M0 NaN scale")
    vals = e4m3.decode(q)
    if np.isnan(vals).any():
        raise ValueError("dequant_mx: NaN code in operand")
    scale = np.ldexp(1.0, s.astype(np.int64) - E8M0_BIAS)
    return vals * np.repeat(scale, MX_BLOCK, axis=1)


def mx_scaled_mm(qa, sa, qb, sb):
    """D = A . B^T in float64 from MX codes and scales: A [M, K], B [N, K]."""
    return dequant_mx(qa, sa) @ dequant_mx(qb, sb).T
