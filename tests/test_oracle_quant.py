"""Pins of the oracle's blockwise quantizers.

Each pin is independent of the oracle's own arithmetic: exact rational
quantization (tests/exact.py), closed forms (round trip of representable
values, the EPS-floored scale), invariants the definition implies
(saturation at the block maximum, scaling by 2**j, negation, permutation,
the 128x128 scale being the maximum of the 1x128 scales inside it), and the
scalar-loop form against the vectorized form.
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import quant
import exact


def bf16_bits(x):
    """float array -> bf16 bit patterns (torch's round-to-nearest-even cast)."""
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def rand_bf16(rng, shape, sigma=1.0):
    return bf16_bits(rng.standard_normal(shape).astype(np.float32) * sigma)


def f32(bits):
    return quant.bf16_bits_to_f32(bits)


def test_eps_is_the_pages_constant():
    path = os.path.join(os.path.dirname(__file__), "golden", "pages_constants.txt")
    vals = {}
    for line in open(path):
        line = line.split("#")[0].strip()
        if line:
            k, v = line.split()
            vals[k] = v
    assert quant.EPS == np.float32(float(vals["EPS"]))
    assert quant.BLOCK == int(vals["BLOCK"])


def test_exact_rational_blocks(rng):
    """Oracle == exact rational quantization on mixed-magnitude blocks."""
    blocks = []
    for sigma in (1.0, 0.02, 1e-2, 3e4, 1e-8):
        blocks.append(rand_bf16(rng, 128, sigma))
    with_outliers = rand_bf16(rng, 128)
    with_outliers[::17] = bf16_bits(f32(with_outliers[::17]) * 50)
    blocks.append(with_outliers)
    x_bits = np.stack(blocks)
    q, s = quant.quant_1x128_rowwise(x_bits)
    for r in range(x_bits.shape[0]):
        codes, sc = exact.exact_quant_block([float(v) for v in f32(x_bits[r])])
        assert float(s[r, 0]) == sc
        assert list(q[r]) == codes, r


def _find_reciprocal_disagreements(rng, want=6):
    """Blocks where x * fl32(1/s) and fl32(x / s) give different e4m3 codes."""
    found = []
    for _ in range(400):
        x_bits = rand_bf16(rng, (64, 128))
        x = f32(x_bits)
        amax = np.maximum(np.abs(x).max(axis=1), quant.EPS)
        s = (amax / np.float32(448)).astype(np.float32)
        via_div = np.clip(x / s[:, None], -448, 448).astype(np.float32)
        via_rcp = np.clip(x * (np.float32(1) / s)[:, None], -448, 448).astype(np.float32)
        from oracle import e4m3
        diff = e4m3.encode(via_div) != e4m3.encode(via_rcp)
        for r in np.nonzero(diff.any(axis=1))[0]:
            found.append(x_bits[r])
            if len(found) >= want:
                return np.stack(found)
    return np.stack(found) if found else None


def test_division_not_reciprocal_multiply(rng):
    """Pins step 4: the element is divided by the scale (correctly rounded)."""
    blocks = _find_reciprocal_disagreements(rng)
    assert blocks is not None and len(blocks) > 0
    q, s = quant.quant_1x128_rowwise(blocks)
    for r in range(blocks.shape[0]):
        codes, sc = exact.exact_quant_block([float(v) for v in f32(blocks[r])])
        assert list(q[r]) == codes and float(s[r, 0]) == sc


def test_round_trip_of_representable_values(rng):
    """Codes of e4m3 values times 2**j, with 448 * 2**j present, come back."""
    from oracle import e4m3
    finite = [c for c in range(256) if c not in (0x7F, 0xFF)]
    for j in (-20, -3, 0, 5, 30):
        codes = rng.choice(finite, size=128).astype(np.uint8)
        codes[rng.integers(128)] = 0x7E if rng.random() < 0.5 else 0xFE
        vals = e4m3.DECODE[codes] * 2.0 ** j
        x_bits = bf16_bits(vals[None, :])
        assert np.array_equal(f32(x_bits)[0], vals.astype(np.float32))  # exact in bf16
        q, s = quant.quant_1x128_rowwise(x_bits)
        assert float(s[0, 0]) == 2.0 ** j
        assert np.array_equal(q[0], codes)


def test_zero_block_scale_is_floored_eps():
    x_bits = np.zeros((1, 128), dtype=np.uint16)
    x_bits[0, 5] = 0x8000  # a negative zero
    q, s = quant.quant_1x128_rowwise(x_bits)
    expect = exact.round_to_f32(exact.EPS_F32 / 448)
    assert float(s[0, 0]) == expect
    assert abs(expect - 2.2321429e-15) < 1e-21
    assert q[0, 5] == 0x80 and np.all(np.delete(q[0], 5) == 0)


def test_tiny_block_gives_signed_zeros():
    vals = np.array([1e-20, -1e-20, 3e-13, -9e-13] * 32, dtype=np.float32)
    x_bits = bf16_bits(vals[None, :])
    q, s = quant.quant_1x128_rowwise(x_bits)
    assert float(s[0, 0]) == exact.round_to_f32(exact.EPS_F32 / 448)
    neg = np.signbit(f32(x_bits)[0])
    # |x| / s <= 0.9 * 448 in this block, so nonzero codes are allowed; the
    # sign must follow x everywhere and the tiny ones must be +-0.
    assert np.array_equal((q[0] & 0x80) != 0, neg)
    assert np.all((q[0][np.abs(f32(x_bits)[0]) < 1e-19] & 0x7F) == 0)


def test_saturation_at_block_max_and_no_nan(rng):
    x_bits = rand_bf16(rng, (64, 512), 3.0)
    x = f32(x_bits)
    q, s = quant.quant_1x128_rowwise(x_bits)
    assert not np.any((q & 0x7F) == 0x7F)
    xb = np.abs(x).reshape(64, 4, 128)
    qb = q.reshape(64, 4, 128)
    at_max = xb == xb.max(axis=2, keepdims=True)
    assert np.all((qb[at_max] & 0x7F) == 0x7E)


def test_power_of_two_scaling_equivariance(rng):
    x_bits = rand_bf16(rng, (32, 256))
    q0, s0 = quant.quant_1x128_rowwise(x_bits)
    for j in (-7, 1, 12):
        xj = bf16_bits(f32(x_bits) * np.float32(2.0 ** j))
        qj, sj = quant.quant_1x128_rowwise(xj)
        assert np.array_equal(qj, q0)
        assert np.array_equal(sj, (s0 * np.float32(2.0 ** j)).astype(np.float32))


def test_negation_flips_only_sign_bit(rng):
    x_bits = rand_bf16(rng, (32, 256))
    q0, s0 = quant.quant_1x128_rowwise(x_bits)
    q1, s1 = quant.quant_1x128_rowwise(x_bits ^ np.uint16(0x8000))
    assert np.array_equal(s0, s1)
    assert np.array_equal(q1, q0 ^ np.uint8(0x80))


def test_permutation_within_block(rng):
    x_bits = rand_bf16(rng, (8, 128))
    q0, s0 = quant.quant_1x128_rowwise(x_bits)
    perm = rng.permutation(128)
    q1, s1 = quant.quant_1x128_rowwise(x_bits[:, perm])
    assert np.array_equal(s0, s1) and np.array_equal(q1, q0[:, perm])


def test_scalar_and_vectorized_forms_agree(rng):
    x_bits = rand_bf16(rng, (128, 256))
    x_bits[3, :128] = 0
    x_bits[7, 128:] = bf16_bits(f32(x_bits[7, 128:]) * np.float32(1e-14))
    x_bits[9, 5] = bf16_bits(np.float32(3.3e38))   # near bf16 max
    qs, ss = quant.quant_1x128_rowwise_scalar(x_bits)
    qv, sv = quant.quant_1x128_rowwise(x_bits)
    assert np.array_equal(qs, qv) and np.array_equal(ss, sv)
    qs, ss = quant.quant_1x128_colwise_scalar(x_bits)
    qv, sv = quant.quant_1x128_colwise(x_bits)
    assert np.array_equal(qs, qv) and np.array_equal(ss, sv)
    qs, ss = quant.quant_128x128_scalar(x_bits)
    qv, sv = quant.quant_128x128(x_bits)
    assert np.array_equal(qs, qv) and np.array_equal(ss, sv)


def test_colwise_is_rowwise_of_transpose(rng):
    x_bits = rand_bf16(rng, (256, 384))
    qc, sc = quant.quant_1x128_colwise_scalar(x_bits)
    qr, sr = quant.quant_1x128_rowwise(np.ascontiguousarray(x_bits.T))
    assert np.array_equal(qc, qr) and np.array_equal(sc, sr)


def test_128x128_scale_is_max_of_row_scales(rng):
    x_bits = rand_bf16(rng, (256, 384))
    x_bits[:128, :128] = bf16_bits(f32(x_bits[:128, :128]) * np.float32(1e-3))
    q128, s128 = quant.quant_128x128(x_bits)
    q1, s1 = quant.quant_1x128_rowwise(x_bits)
    assert np.array_equal(s128, s1.reshape(2, 128, 3).max(axis=1))


def test_128x128_tile_exact_rational(rng):
    x_bits = rand_bf16(rng, (128, 128), 0.02)
    q, s = quant.quant_128x128(x_bits)
    codes, sc = exact.exact_quant_block([float(v) for v in f32(x_bits).reshape(-1)])
    assert float(s[0, 0]) == sc and list(q.reshape(-1)) == codes


def test_3d_colwise_is_transposed_128x128(rng):
    w_bits = rand_bf16(rng, (3, 256, 384), 0.02)
    q3, s3 = quant.quant_3d_colwise(w_bits)
    for g in range(3):
        qg, sg = quant.quant_128x128_scalar(w_bits[g])
        assert np.array_equal(q3[g], qg.T) and np.array_equal(s3[g], sg.T)


def test_rejects_partial_blocks_and_nonfinite():
    with pytest.raises(ValueError):
        quant.quant_1x128_rowwise(np.zeros((4, 100), dtype=np.uint16))
    with pytest.raises(ValueError):
        quant.quant_128x128(np.zeros((100, 128), dtype=np.uint16))
    bad = np.zeros((1, 128), dtype=np.uint16)
    bad[0, 0] = 0x7F80  # +inf
    with pytest.raises(ValueError):
        quant.quant_1x128_rowwise(bad)


def test_bf16_subnormals_and_extremes(rng):
    vals = np.zeros(128, dtype=np.float32)
    vals[:10] = np.float32(2.0 ** -130) * np.arange(1, 11)  # bf16 subnormals (< EPS)
    vals[10] = np.float32(-3.3e38)
    x_bits = bf16_bits(vals[None, :])
    q, s = quant.quant_1x128_rowwise(x_bits)
    codes, sc = exact.exact_quant_block([float(v) for v in f32(x_bits)[0]])
    assert list(q[0]) == codes and float(s[0, 0]) == sc
