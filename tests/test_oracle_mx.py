"""Pins of the MX (microscaling) FP8 oracle (CPU).

The pages name the MXFP8 recipe without defining it; the oracle follows the
OCP Microscaling v1.0 definition (32-element blocks, E8M0 power-of-two
scale 2^(floor(log2 amax) - 8), E4M3 elements saturated at 448).  Pinned
against: exact rational arithmetic (the exponent found by comparing with
powers of two as Fractions, each element's nearest E4M3 value searched in
the format's own value table), closed forms (round trip of E4M3 values times
2^j, saturation of the top binade, zero and tiny blocks), equivariances, the
scalar form, and exact integer arithmetic for the GEMM."""

import math
from fractions import Fraction

import numpy as np
import pytest

from exact import nearest_e4m3
from oracle import e4m3, mx
from oracle.quant import bf16_bits_to_f32


def _bf16_bits(v):
    """float values -> bf16 bits (round to nearest even via float32)."""
    f = np.asarray(v, dtype=np.float32).view(np.uint32)
    r = ((f + 0x7FFF + ((f >> 16) & 1)) >> 16).astype(np.uint16)
    return r


def _rand_bits(shape, seed, spread=8):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal(shape) * np.exp2(rng.integers(-spread, spread, shape))
    return _bf16_bits(v)


def _exact_block(xs):
    """One MX block with Fractions: (codes, E8M0 byte)."""
    amax = max(abs(Fraction(float(x))) for x in xs)
    if amax == 0:
        e = -127
    else:
        k = 0
        while Fraction(2) ** k > amax:
            k -= 1
        while Fraction(2) ** (k + 1) <= amax:
            k += 1
        e = min(max(k - 8, -127), 127)
    X = Fraction(2) ** e
    codes = []
    for x in xs:
        y = Fraction(float(x)) / X
        y = max(min(y, Fraction(448)), Fraction(-448))
        if y == 0:
            y = -0.0 if math.copysign(1.0, float(x)) < 0 else 0.0
        codes.append(nearest_e4m3(y))
    return codes, e + 127


def test_rowwise_matches_exact_rationals():
    x = _rand_bits((6, 128), seed=1, spread=20)
    x[0, :32] = 0                                      # zero block
    x[1, 32:64] = _bf16_bits(np.full(32, 3e-39))       # bf16 subnormals
    x[2, 64:96] = _bf16_bits(np.linspace(-500, 500, 32))   # saturating top binade
    x[3, 96:128] = 0x8000                              # negative zeros
    q, s = mx.quant_mx_rowwise(x)
    xf = bf16_bits_to_f32(x)
    for r in range(x.shape[0]):
        for b in range(x.shape[1] // 32):
            codes, byte = _exact_block(xf[r, 32 * b:32 * (b + 1)])
            assert list(q[r, 32 * b:32 * (b + 1)]) == codes, (r, b)
            assert s[r, b] == byte, (r, b)


def test_scalar_and_vectorized_forms_agree():
    x = _rand_bits((5, 96), seed=2, spread=30)
    q1, s1 = mx.quant_mx_rowwise(x)
    q2, s2 = mx.quant_mx_rowwise_scalar(x)
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)


@pytest.mark.parametrize("j", [-20, -3, 0, 5, 17])
def test_round_trip_of_e4m3_values_times_power_of_two(j):
    rng = np.random.default_rng(j + 50)
    codes = rng.integers(0, 0x7F, 32).astype(np.uint8) | (rng.integers(0, 2, 32) * 0x80).astype(np.uint8)
    codes[0] = 0x7E                                    # amax = 448 * 2^j
    vals = e4m3.decode(codes) * 2.0 ** j
    x = _bf16_bits(vals)[None, :]
    assert np.array_equal(bf16_bits_to_f32(x)[0].astype(np.float64), vals)   # exact in bf16
    q, s = mx.quant_mx_rowwise(x)
    assert s[0, 0] == 127 + j                          # floor(log2(448 * 2^j)) - 8 = j
    assert np.array_equal(q[0], codes)


def test_top_binade_saturates_and_zero_block_takes_smallest_scale():
    x = _bf16_bits([500.0, 460.0, 448.0, -300.0] + [1.0] * 28)[None, :]
    q, s = mx.quant_mx_rowwise(x)
    assert s[0, 0] == 127                              # 2^(8 - 8) = 1
    assert list(q[0, :4]) == [0x7E, 0x7E, 0x7E, 0xF9]  # 500, 460 -> 448; -300 -> -288 (0xF9)
    qz, sz = mx.quant_mx_rowwise(np.zeros((1, 32), dtype=np.uint16))
    assert sz[0, 0] == 0 and not qz.any()


def test_scaling_by_powers_of_two_shifts_the_exponent_only():
    x = _rand_bits((4, 64), seed=3, spread=4)
    q0, s0 = mx.quant_mx_rowwise(x)
    for k in (-7, 3, 11):
        xk = _bf16_bits(bf16_bits_to_f32(x).astype(np.float64) * 2.0 ** k)
        qk, sk = mx.quant_mx_rowwise(xk)
        assert np.array_equal(qk, q0)
        assert np.array_equal(sk.astype(int), s0.astype(int) + k)
    qn, sn = mx.quant_mx_rowwise(x ^ 0x8000)
    assert np.array_equal(qn, q0 ^ 0x80) and np.array_equal(sn, s0)


def test_colwise_is_rowwise_of_the_transpose():
    x = _rand_bits((64, 96), seed=4)
    qt, st = mx.quant_mx_colwise(x)
    q, s = mx.quant_mx_rowwise(np.ascontiguousarray(x.T))
    assert np.array_equal(qt, q) and np.array_equal(st, s)


def test_gemm_matches_exact_integer_arithmetic():
    rng = np.random.default_rng(5)
    M, N, K = 8, 6, 128
    qa = rng.integers(0, 0x7F, (M, K)).astype(np.uint8) | (rng.integers(0, 2, (M, K)) * 0x80).astype(np.uint8)
    qb = rng.integers(0, 0x7F, (N, K)).astype(np.uint8) | (rng.integers(0, 2, (N, K)) * 0x80).astype(np.uint8)
    sa = rng.integers(120, 135, (M, K // 32)).astype(np.uint8)
    sb = rng.integers(120, 135, (N, K // 32)).astype(np.uint8)
    d = mx.mx_scaled_mm(qa, sa, qb, sb)
    # exact: every e4m3 value is an integer times 2^-9, every scale a power of two
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                va = Fraction(e4m3.decode(np.uint8(qa[m, k])).item()) * Fraction(2) ** (int(sa[m, k // 32]) - 127)
                vb = Fraction(e4m3.decode(np.uint8(qb[n, k])).item()) * Fraction(2) ** (int(sb[n, k // 32]) - 127)
                acc += va * vb
            assert Fraction(d[m, n]) == acc, (m, n)
