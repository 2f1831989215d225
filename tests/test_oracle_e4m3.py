"""Pins of the oracle's e4m3 format code against the format definition.

The pins are: the OCP table values (tests/golden/e4m3_ocp_table.txt), exact
rational nearest-value search (tests/exact.py), closed forms of the decision
boundaries, and torch's own float8_e4m3fn CPU cast (an independent library
routine; it does not saturate, so inputs are kept within +-448).
"""

import math
import os

import numpy as np
import pytest
import torch

from oracle import e4m3
import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_ocp_table.txt")


def _golden_rows():
    rows = []
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if line:
            code, val = line.split()
            rows.append((int(code, 16), val))
    return rows


def test_decode_matches_ocp_table():
    rows = _golden_rows()
    assert len(rows) >= 10
    for code, val in rows:
        got = e4m3.DECODE[code]
        if val == "nan":
            assert math.isnan(got), hex(code)
        elif val == "-0":
            assert got == 0.0 and math.copysign(1.0, got) < 0
        else:
            assert got == float(val), (hex(code), got, val)


def test_decode_all_codes_vs_torch_cast():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = e4m3.DECODE
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(ref[~nan], ours[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(ours[~nan]))


def test_decode_vs_exact_definition():
    for c in range(0x7F):
        assert e4m3.DECODE[c] == float(exact.e4m3_value(c))
        assert e4m3.DECODE[c | 0x80] == -float(exact.e4m3_value(c))


def test_nonneg_codes_are_increasing_and_max_448():
    v = e4m3.DECODE[:0x7F]
    assert np.all(np.diff(v) > 0)
    assert v[-1] == 448.0 and v[1] == 2.0 ** -9 and v[8] == 2.0 ** -6
    assert math.isnan(e4m3.DECODE[0x7F]) and math.isnan(e4m3.DECODE[0xFF])


def _boundary_points():
    """Every table value, every midpoint, and their float32 neighbours."""
    v = [float(exact.e4m3_value(c)) for c in range(0x7F)]
    pts = set()
    for i, x in enumerate(v):
        pts.add(np.float32(x))
        if i + 1 < len(v):
            mid = np.float32((v[i] + v[i + 1]) / 2)     # exact in float32
            assert float(mid) == (v[i] + v[i + 1]) / 2
            for k in range(-3, 4):
                u = exact.f32_bits(float(mid)) + k
                pts.add(np.float32(exact.f32_from_bits(u)))
    pts = sorted(p for p in pts if 0 <= p <= 448)
    return np.array(pts, dtype=np.float32)


def test_encode_decision_boundaries_exact():
    pts = _boundary_points()
    got = e4m3.encode(pts)
    for p, g in zip(pts, got):
        assert g == exact.nearest_e4m3(float(p)), (float(p), hex(g))
    got_neg = e4m3.encode(-pts)
    assert np.array_equal(got_neg, got | 0x80)


def test_encode_boundaries_vs_torch_cast():
    pts = _boundary_points()
    ref = torch.from_numpy(pts).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3.encode(pts), ref)


def test_encode_ties_go_to_even():
    # 1.0625 is halfway between 1.0 (0x38) and 1.125 (0x39): even code 0x38.
    # 1.1875 is halfway between 1.125 (0x39) and 1.25 (0x3A): even code 0x3A.
    # 2**-10 is halfway between 0 and 2**-9: code 0x00.  432 between 416 and 448.
    y = np.array([1.0625, 1.1875, 2.0 ** -10, 1.5 * 2.0 ** -10, 432.0], dtype=np.float32)
    assert list(e4m3.encode(y)) == [0x38, 0x3A, 0x00, 0x01, 0x7E]
    assert [e4m3.encode_scalar(float(t)) for t in y] == [0x38, 0x3A, 0x00, 0x01, 0x7E]


def test_encode_saturates_and_keeps_sign_of_zero():
    y = np.array([448.0, 449.0, 464.0, 465.0, 1e30, -1e30, -0.0, -1e-30, 0.0], dtype=np.float32)
    assert list(e4m3.encode(y)) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x80, 0x80, 0x00]
    assert [e4m3.encode_scalar(float(t)) for t in y] == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x80, 0x80, 0x00]


def test_encode_rejects_nonfinite():
    with pytest.raises(ValueError):
        e4m3.encode(np.array([np.nan], dtype=np.float32))
    with pytest.raises(ValueError):
        e4m3.encode_scalar(float("inf"))


def test_encode_random_vs_torch_and_scalar(rng):
    # log-uniform magnitudes over the whole e4m3 range plus float32 subnormals
    n = 400_000
    mag = np.exp2(rng.uniform(-40, np.log2(448.0), n)).astype(np.float32)
    mag = np.minimum(mag, np.float32(448.0))
    y = np.where(rng.random(n) < 0.5, -mag, mag).astype(np.float32)
    ours = e4m3.encode(y)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    sample = y[:2000]
    assert [e4m3.encode_scalar(float(t)) for t in sample] == list(ours[:2000])


def test_encode_is_monotone(rng):
    y = np.sort(rng.uniform(0, 448, 100_000).astype(np.float32))
    v = e4m3.DECODE[e4m3.encode(y)]
    assert np.all(np.diff(v) >= 0)
