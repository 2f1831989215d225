"""Pins of the oracle's scaled and grouped GEMMs.

Pins: exact integer arithmetic (e4m3 values are integers times 2**-9, so with
power-of-two scales every product and sum is an integer times a power of
two), exact rational sums with general float32 scales, the identity operand,
a single non-zero K block, 128x128 scales expanded to 1x128, and the grouped
forms against masked dense products.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import e4m3, gemm

FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)


def rand_codes(rng, shape):
    return rng.choice(FINITE, size=shape).astype(np.uint8)


def int_value(code):
    """e4m3 value times 2**9 as an exact Python int."""
    v = Fraction(float(e4m3.DECODE[code])) * 512
    assert v.denominator == 1
    return int(v)


def test_brute_force_128_cubed_power_of_two_scales(rng):
    M = N = K = 128
    qa, qb = rand_codes(rng, (M, K)), rand_codes(rng, (N, K))
    ja = rng.integers(-6, 7, size=(M, 1))
    jb = rng.integers(-6, 7, size=(1, 1))
    sa = np.exp2(ja).astype(np.float32)
    sb = np.exp2(jb).astype(np.float32)
    d = gemm.scaled_mm(qa, sa, qb, sb, 128)
    ia = np.vectorize(int_value)(qa).astype(object)
    ib = np.vectorize(int_value)(qb).astype(object)
    for m in range(0, M, 7):
        for n in range(0, N, 5):
            acc = sum(int(ia[m, k]) * int(ib[n, k]) for k in range(K))
            exact = Fraction(acc, 2 ** 18) * Fraction(2) ** int(ja[m, 0]) * Fraction(2) ** int(jb[0, 0])
            assert Fraction(d[m, n]) == exact, (m, n)


def test_general_scales_vs_rationals(rng):
    M, N, K = 8, 8, 384
    qa, qb = rand_codes(rng, (M, K)), rand_codes(rng, (N, K))
    sa = (rng.random((M, 3)) * 1e-2 + 1e-4).astype(np.float32)
    sb = (rng.random((N, 3)) * 3 + 0.1).astype(np.float32)
    d = gemm.scaled_mm(qa, sa, qb, sb, 1)
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            mag = Fraction(0)
            for k in range(K):
                t = (Fraction(float(e4m3.DECODE[qa[m, k]])) * Fraction(float(sa[m, k // 128]))
                     * Fraction(float(e4m3.DECODE[qb[n, k]])) * Fraction(float(sb[n, k // 128])))
                tot += t
                mag += abs(t)
            assert abs(Fraction(d[m, n]) - tot) <= mag * Fraction(1, 10 ** 12)


def test_128x128_b_scales_vs_rationals_several_row_and_k_blocks(rng):
    """128x128 B scales with N = 384 (three row blocks) and K = 384 (three K
    blocks), a distinct scale per (row block, K block): every sampled output
    against a Fraction sum whose B scale is looked up element by element as
    sb[n // 128][k // 128] (no expansion of the scale array).  A scale taken
    from the wrong row block or K block, or a transposed scale array, moves
    the result far outside the 1e-12 bound."""
    M, N, K = 6, 384, 384
    qa, qb = rand_codes(rng, (M, K)), rand_codes(rng, (N, K))
    sa = (rng.random((M, 3)) * 1e-2 + 1e-4).astype(np.float32)
    # distinct, well separated scales: 2^(3i + j) times a random mantissa
    sb = np.array([[(1.0 + rng.random()) * 2.0 ** (3 * i + j - 4) for j in range(3)] for i in range(3)],
                  dtype=np.float32)
    assert len(set(sb.ravel().tolist())) == 9
    d = gemm.scaled_mm(qa, sa, qb, sb, 128)
    for m in range(M):
        for n in list(range(0, N, 37)) + [127, 128, 255, 256, 383]:
            tot = Fraction(0)
            mag = Fraction(0)
            for k in range(K):
                t = (Fraction(float(e4m3.DECODE[qa[m, k]])) * Fraction(float(sa[m, k // 128]))
                     * Fraction(float(e4m3.DECODE[qb[n, k]])) * Fraction(float(sb[n // 128, k // 128])))
                tot += t
                mag += abs(t)
            assert abs(Fraction(d[m, n]) - tot) <= mag * Fraction(1, 10 ** 12), (m, n)


def test_identity_b_returns_dequantized_a(rng):
    M, K = 64, 256
    qa = rand_codes(rng, (M, K))
    sa = (rng.random((M, 2)) + 0.5).astype(np.float32)
    qb = np.zeros((K, K), dtype=np.uint8)
    qb[np.arange(K), np.arange(K)] = 0x38  # 1.0
    sb = np.ones((2, 2), dtype=np.float32)
    d = gemm.scaled_mm(qa, sa, qb, sb, 128)
    expect = np.array([[float(e4m3.DECODE[qa[m, k]]) * float(sa[m, k // 128]) for k in range(K)]
                       for m in range(M)])
    assert np.array_equal(d, expect)


def test_single_k_block_isolates_scale_pair(rng):
    M, N, K = 16, 128, 512
    qa, qb = rand_codes(rng, (M, K)), rand_codes(rng, (N, K))
    keep = 2
    qa[:, :keep * 128] = 0
    qa[:, (keep + 1) * 128:] = 0
    sa = (rng.random((M, 4)) + 0.5).astype(np.float32)
    sb = (rng.random((1, 4)) + 0.5).astype(np.float32)
    d = gemm.scaled_mm(qa, sa, qb, sb, 128)
    blk = slice(keep * 128, (keep + 1) * 128)
    plain = e4m3.DECODE[qa[:, blk]] @ e4m3.DECODE[qb[:, blk]].T
    scale = sa[:, keep:keep + 1].astype(np.float64) * float(sb[0, keep])
    expect = plain * scale
    mag = (np.abs(e4m3.DECODE[qa[:, blk]]) @ np.abs(e4m3.DECODE[qb[:, blk]]).T) * scale
    assert np.all(np.abs(d - expect) <= 1e-13 * mag)


def test_128x128_scales_equal_expanded_1x128(rng):
    M, N, K = 32, 256, 256
    qa, qb = rand_codes(rng, (M, K)), rand_codes(rng, (N, K))
    sa = (rng.random((M, 2)) + 0.1).astype(np.float32)
    sb128 = (rng.random((2, 2)) + 0.1).astype(np.float32)
    sb1 = np.repeat(sb128, 128, axis=0)
    assert np.array_equal(gemm.scaled_mm(qa, sa, qb, sb128, 128), gemm.scaled_mm(qa, sa, qb, sb1, 1))


def test_group_m_vs_masked_dense(rng):
    ends = [128, 128, 384]  # sizes 128, 0, 256
    M, N, K = 384, 128, 256
    qa = rand_codes(rng, (M, K))
    sa = (rng.random((M, 2)) + 0.1).astype(np.float32)
    qb = rand_codes(rng, (3, N, K))
    sb = (rng.random((3, 1, 2)) + 0.1).astype(np.float32)
    d = gemm.grouped_mm_group_m(ends, qa, sa, qb, sb, 128)
    owner = np.repeat([0, 2], [128, 256])
    for g in (0, 2):
        dense = gemm.scaled_mm(qa, sa, qb[g], sb[g], 128)
        assert np.array_equal(d[owner == g], dense[owner == g])


def test_group_k_vs_masked_dense_and_empty_group(rng):
    ends = [256, 256, 384]  # sizes 256, 0, 128
    N, K, T = 128, 256, 384
    qa, qb = rand_codes(rng, (N, T)), rand_codes(rng, (K, T))
    sa = (rng.random((N, 3)) + 0.1).astype(np.float32)
    sb = (rng.random((K, 3)) + 0.1).astype(np.float32)
    d = gemm.grouped_mm_group_k(ends, qa, sa, qb, sb)
    assert d.shape == (3, N, K)
    assert np.all(d[1] == 0)
    starts = [0, 256, 256]
    for g in (0, 2):
        mask = np.zeros(T, dtype=bool)
        mask[starts[g]:ends[g]] = True
        qa_m = np.where(mask[None, :], qa, 0).astype(np.uint8)
        qb_m = np.where(mask[None, :], qb, 0).astype(np.uint8)
        dense = gemm.scaled_mm(qa_m, sa, qb_m, sb, 1)
        mag = np.abs(gemm.dequant(qa_m, sa, 1)) @ np.abs(gemm.dequant(qb_m, sb, 1)).T
        assert np.all(np.abs(d[g] - dense) <= 1e-13 * mag)


def test_tolerance_accepts_bf16_rounding_and_rejects_planted_error(rng):
    M, N, K = 64, 128, 512
    qa, qb = rand_codes(rng, (M, K)), rand_codes(rng, (N, K))
    sa = (rng.random((M, 4)) + 0.1).astype(np.float32)
    sb = (rng.random((1, 4)) + 0.1).astype(np.float32)
    a, b = gemm.dequant(qa, sa, 1), gemm.dequant(qb, sb, 128)
    ref = a @ b.T
    import torch
    d_bf16 = torch.from_numpy(ref).to(torch.bfloat16).double().numpy()
    ok, worst = gemm.check_close(d_bf16, ref, a, b)
    assert ok and worst < 1.0
    bad = ref.copy()
    bad[3, 5] += 2.1e-3 * np.linalg.norm(a[3]) * np.linalg.norm(b[5])
    ok, worst = gemm.check_close(bad, ref, a, b)
    assert not ok and worst > 1.0


def test_rejects_nan_codes_and_bad_groups(rng):
    qa = np.full((1, 128), 0x7F, dtype=np.uint8)
    with pytest.raises(ValueError):
        gemm.dequant(qa, np.ones((1, 1), dtype=np.float32), 1)
    with pytest.raises(ValueError):
        gemm.group_bounds([256, 128])
    with pytest.raises(ValueError):
        gemm.group_bounds([100])
