"""Pins of the gated-activation oracle (CPU).

round_to_bf16 against exact rational rounding; swiglu against closed forms,
against scipy's logistic function (an independent silu), and against torch's
CPU silu in float32 (within one bf16 step)."""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import swiglu
from oracle.quant import bf16_bits_to_f32


def exact_bf16(v):
    """Nearest bf16 to the float64 v (ties to even), by Fractions."""
    x = Fraction(float(v))
    if x == 0:
        return np.uint16(0x8000 if np.signbit(v) else 0)
    sign = 0x8000 if x < 0 else 0
    x = abs(x)
    # exact binade: 2**E <= x < 2**(E+1)
    E = x.numerator.bit_length() - x.denominator.bit_length()
    while Fraction(2) ** E > x:
        E -= 1
    while Fraction(2) ** (E + 1) <= x:
        E += 1
    step = Fraction(2) ** max(E - 7, -133)     # bf16 spacing in that binade (or subnormal)
    k = x / step
    lo = k.numerator // k.denominator
    best = None
    for m in (lo, lo + 1):
        key = (abs(m * step - x), m % 2)        # nearest, then even multiple of the step
        if best is None or key < best[0]:
            best = (key, m * step)
    val = best[1]
    b = np.float32(float(val)).view(np.uint32) >> 16
    return np.uint16(int(b) | sign)


def test_round_to_bf16_matches_exact_rounding():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.integers(-40, 38, 3000),
                        rng.standard_normal(500) * 1e-39,       # bf16 subnormal range
                        [0.0, -0.0, 1.0, -2.5, 3.0e38]])
    got = swiglu.round_to_bf16(v)
    want = np.array([exact_bf16(x) for x in v], dtype=np.uint16)
    assert np.array_equal(got, want)


def test_round_to_bf16_ties_go_to_even():
    # 1 + k/128 are bf16 values; the midpoints between neighbours are ties
    k = np.arange(0, 127)
    lo = 1.0 + k / 128.0
    mid = lo + 1.0 / 256.0
    got = bf16_bits_to_f32(swiglu.round_to_bf16(mid)).astype(np.float64)
    want = np.where(k % 2 == 0, lo, lo + 1.0 / 128.0)
    assert np.array_equal(got, want)
    # representable values are unchanged
    b = np.arange(0, 0x7F80, 37, dtype=np.uint16)
    assert np.array_equal(swiglu.round_to_bf16(bf16_bits_to_f32(b).astype(np.float64)), b)


def _bits(x):
    return torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_swiglu_closed_forms():
    a = _bits([0.0, 0.0, 200.0, 100.0, -200.0, -100.0, 1.0])
    b = _bits([3.0, -3.0, 1.5, -0.75, 2.0, 5.0, 0.0])
    h = bf16_bits_to_f32(swiglu.swiglu(a, b))
    assert h[0] == 0 and not np.signbit(h[0])
    assert h[1] == 0 and np.signbit(h[1])          # +0 * -3 = -0
    assert h[2] == 300.0 and h[3] == -75.0          # silu(a) = a for large a (exp(-a) < 2^-140)
    assert h[4] == 0 and np.signbit(h[4])          # silu(-200) underflows to -0
    assert h[5] == 0 and np.signbit(h[5])          # -100 e^-100 ~ -3.7e-42: below half the smallest bf16
    assert h[6] == 0


def test_swiglu_against_scipy_logistic():
    from scipy.special import expit
    rng = np.random.default_rng(1)
    a = _bits(rng.standard_normal(200000) * 3)
    b = _bits(rng.standard_normal(200000))
    af = bf16_bits_to_f32(a).astype(np.float64)
    bf = bf16_bits_to_f32(b).astype(np.float64)
    want = swiglu.round_to_bf16(af * expit(af) * bf)
    assert np.array_equal(swiglu.swiglu(a, b), want)


def test_swiglu_within_one_bf16_step_of_torch_float32():
    rng = np.random.default_rng(2)
    a = _bits(rng.standard_normal(100000) * 4)
    b = _bits(rng.standard_normal(100000))
    at = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).float()
    bt = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).float()
    ref = (torch.nn.functional.silu(at) * bt).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = swiglu.swiglu(a, b)
    # compare as ordered integers (same sign here except at zero)
    d = np.abs(got.astype(np.int32) - ref.astype(np.int32))
    diff = d[(got & 0x7FFF) != 0]
    assert diff.max() <= 1
    assert (d != 0).mean() < 1e-3


def test_round_to_bf16_rejects_non_finite():
    with pytest.raises(ValueError):
        swiglu.round_to_bf16([np.inf])


# ---- backward: pinned to central differences of the forward function in
# 60-digit decimal arithmetic (no closed-form derivative involved).  Products
# of bf16 values often land exactly on a bf16 tie; when the gate is almost
# fully open (|a| large) or a is tiny, the exact gradient is that product
# times 1 +- something below float64 resolution, so float64 sees the tie ----

from decimal import Decimal, getcontext


def _dec_gate(a, b):
    """silu(a) * b in Decimal (a, b Decimal)."""
    return a * b / (1 + (-a).exp())


def _dec_bf16(x):
    """The two bf16 neighbours of a Decimal (bits, toward and away from
    zero) and whether x is within 2^-48 (relative) of their midpoint: there
    an evaluation in float64 (the precision the oracle takes for these
    transcendental functions) cannot tell the side, and either neighbour is
    the float64 reading's answer.  Otherwise the nearest one comes first."""
    if x == 0:
        return (0, 0), False
    sign = 0x8000 if x < 0 else 0
    x = abs(x)
    E = int(x.log10() / Decimal(2).log10())    # approximate binade, fixed below
    while Decimal(2) ** E > x:
        E -= 1
    while Decimal(2) ** (E + 1) <= x:
        E += 1
    step = Decimal(2) ** max(E - 7, -133)
    k = x / step
    lo = int(k)                                # floor for positive k
    frac = k - lo

    def bits(m):
        v = float(m * step)                    # exactly representable in bf16 (and float)
        if v > swiglu._BF16_MAX:
            return sign | 0x7F80
        return sign | (int(np.float32(v).view(np.uint32)) >> 16)

    near_tie = abs(frac - Decimal("0.5")) * step < x * Decimal(2) ** -48
    m = lo + 1 if frac > Decimal("0.5") or (frac == Decimal("0.5") and lo % 2 == 1) else lo
    return (bits(m), bits(lo + lo + 1 - m)), near_tie


def _matches(got, x):
    (near, other), near_tie = _dec_bf16(x)
    got = int(got)
    if (near & 0x7FFF) == 0 and (got & 0x7FFF) == 0:
        return True                            # zero of either sign
    return got == near or (near_tie and got == other)


def _bf16_dec(bits):
    return Decimal(float(bf16_bits_to_f32(np.array([bits], dtype=np.uint16))[0]))


def test_swiglu_backward_matches_high_precision_central_differences():
    getcontext().prec = 60
    rng = np.random.default_rng(5)
    n = 600
    a = rng.standard_normal(n) * 3.0
    a[:40] = -1.2784645 + rng.standard_normal(40) * 0.01   # around the zero of silu'(a)
    a[40:50] = [0.0, 30.0, -30.0, 80.0, -80.0, 1e-30, -1e-30, 2.5, -2.5, 1.0]
    b = rng.standard_normal(n) * 2.0
    dh = rng.standard_normal(n) * 0.01
    a_bits = swiglu.round_to_bf16(a)
    b_bits = swiglu.round_to_bf16(b)
    dh_bits = swiglu.round_to_bf16(dh)
    da, db = swiglu.swiglu_backward(a_bits, b_bits, dh_bits)
    eps = Decimal("1e-25")
    for i in range(n):
        A, B, G = _bf16_dec(a_bits[i]), _bf16_dec(b_bits[i]), _bf16_dec(dh_bits[i])
        dA = G * (_dec_gate(A + eps, B) - _dec_gate(A - eps, B)) / (2 * eps)
        dB = G * (_dec_gate(A, B + eps) - _dec_gate(A, B - eps)) / (2 * eps)
        assert _matches(da[i], dA), (i, float(A), float(B), float(G), hex(da[i]))
        assert _matches(db[i], dB), (i, float(A), float(B), float(G), hex(db[i]))


def test_swiglu_backward_closed_forms():
    # a = 0: silu'(0) = 1/2, silu(0) = 0
    z = np.zeros(4, dtype=np.uint16)
    b = swiglu.round_to_bf16([1.0, -2.0, 0.5, 3.0])
    dh = swiglu.round_to_bf16([0.25, 0.5, -1.0, 2.0])
    da, db = swiglu.swiglu_backward(z, b, dh)
    want = bf16_bits_to_f32(dh).astype(np.float64) * bf16_bits_to_f32(b).astype(np.float64) * 0.5
    assert np.array_equal(bf16_bits_to_f32(da).astype(np.float64), want)
    assert np.all((db & 0x7FFF) == 0)
    # a large: the gate is open (s = 1 up to 1e-35): da = dh * b, db = dh * a
    a = swiglu.round_to_bf16([90.0, 90.0, 90.0, 90.0])
    da, db = swiglu.swiglu_backward(a, b, dh)
    assert np.array_equal(da, swiglu.round_to_bf16(bf16_bits_to_f32(dh).astype(np.float64) *
                                                   bf16_bits_to_f32(b).astype(np.float64)))
    assert np.array_equal(db, swiglu.round_to_bf16(90.0 * bf16_bits_to_f32(dh).astype(np.float64)))
    # a very negative: the gate is shut, both gradients vanish
    a = swiglu.round_to_bf16([-200.0] * 4)
    da, db = swiglu.swiglu_backward(a, b, dh)
    assert np.all((da & 0x7FFF) == 0) and np.all((db & 0x7FFF) == 0)
