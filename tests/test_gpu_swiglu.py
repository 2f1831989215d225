"""GPU parity of the fused gated activation + 1x128 quantizer, forward and
backward.

h = silu(a) * b (and, backward, da = dh b silu'(a), db = dh silu(a)) is the
float64 value of its formula rounded once to bf16; the kernels evaluate in
fp32 and switch to float64 near rounding ties, so h, da and db must equal the
oracle's bit for bit, and the codes and scales must equal the oracle's 1x128
quantization of the oracle's own h (or [da | db]), rows and transposed
columns."""

import numpy as np
import pytest
import torch

import blockwise_scaled_fp8_bs_amd as bs
from blockwise_scaled_fp8_bs_amd import inputs
from gpu_support import bits16, check_canaries, check_scale_canaries, guarded, need_gpu, scale_buffer, u8
from oracle import quant, swiglu

pytestmark = pytest.mark.gpu


def _from_bits(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def _inputs(R, C, seed):
    a = inputs.bf16_normal((R, C), 3.0, seed)
    b = inputs.bf16_normal((R, C), 1.0, seed + 1)
    ab = bits16(a).copy()
    if R >= 8 and C >= 128:   # gate inputs at the edges of the fp32 path
        ab[0, :64] = bits16(torch.full((64,), 150.0, dtype=torch.bfloat16))
        ab[1, :64] = bits16(torch.full((64,), -150.0, dtype=torch.bfloat16))
        ab[2, :128] = 0
        ab[3, 3] = 0x8000
        ab[4, :128] = bits16(torch.linspace(-75.0, -60.0, 128).to(torch.bfloat16))   # exp(-a) near fp32 overflow
        ab[5, :128] = bits16(torch.linspace(15.0, 40.0, 128).to(torch.bfloat16))     # silu(a) = a (1 - tiny)
        ab[6, :64] = bits16(torch.full((64,), 1e-30, dtype=torch.bfloat16))
        ab[6, 64:128] = bits16(torch.full((64,), -3e-39, dtype=torch.bfloat16))      # bf16 subnormal
        ab[7, :128] = bits16(torch.linspace(-1.34, -1.22, 128).to(torch.bfloat16))   # around silu'(a) = 0
    a = _from_bits(ab)
    return a, b


def _assert_same_bits(got, want, what):
    bad = np.flatnonzero(got.ravel() != want.ravel())
    assert bad.size == 0, f"{what}: {bad.size} of {got.size} differ, first at {bad[:5]}: " \
                          f"{got.ravel()[bad[:5]]} vs {want.ravel()[bad[:5]]}"


@pytest.mark.parametrize("R,C", [(256, 512), (384, 640), (128, 128)])
def test_swiglu_quant_rows_and_cols(R, C):
    need_gpu()
    a, b = _inputs(R, C, seed=R + C)
    h_full, h = guarded(R, C, torch.bfloat16)
    qr_full, qr = guarded(R, C, torch.uint8)
    sr_full, sr = scale_buffer(C // 128, R)
    qc_full, qc = guarded(C, R, torch.uint8)
    sc_full, sc = scale_buffer(R // 128, C)
    print(f"swiglu_quant R={R} C={C}", flush=True)
    bs.bs_swiglu_quant_1x128(a.cuda(), b.cuda(), h, qr, sr, qc, sc)
    torch.cuda.synchronize()
    h_ref = swiglu.swiglu(bits16(a), bits16(b))
    _assert_same_bits(bits16(h), h_ref, "h")
    q_ref, s_ref = quant.quant_1x128_rowwise(h_ref)
    assert np.array_equal(u8(qr), q_ref)
    assert np.array_equal(sr.cpu().numpy().T[:R], s_ref)
    qc_ref, sc_ref = quant.quant_1x128_colwise(h_ref)
    assert np.array_equal(u8(qc), qc_ref)
    assert np.array_equal(sc.cpu().numpy().T[:C], sc_ref)
    for full, r, c in [(h_full, R, C), (qr_full, R, C), (qc_full, C, R)]:
        check_canaries(full, r, c)
    check_scale_canaries(sr_full, C // 128, R)
    check_scale_canaries(sc_full, R // 128, C)

    # the same codes without writing h, and each output alone
    qr2 = torch.empty_like(qr)
    sr2 = torch.empty_like(sr)
    bs.bs_swiglu_quant_1x128(a.cuda(), b.cuda(), None, qr2, sr2)
    qc2 = torch.empty_like(qc)
    sc2 = torch.empty_like(sc)
    bs.bs_swiglu_quant_1x128(a.cuda(), b.cuda(), None, None, None, qc2, sc2)
    torch.cuda.synchronize()
    assert torch.equal(qr2, qr) and torch.equal(sr2[:, :R], sr[:, :R])
    assert torch.equal(qc2, qc) and torch.equal(sc2[:, :C], sc[:, :C])


@pytest.mark.parametrize("R", [1, 77, 300])
def test_swiglu_quant_ragged_rows(R):
    need_gpu()
    C = 256
    a, b = _inputs(R, C, seed=R)
    h = torch.empty((R, C), dtype=torch.bfloat16, device="cuda")
    qr_full, qr = guarded(R, C, torch.uint8)
    sr = bs.empty_scales(C // 128, R, "cuda")
    print(f"swiglu_quant ragged R={R}", flush=True)
    bs.bs_swiglu_quant_1x128(a.cuda(), b.cuda(), h, qr, sr)
    torch.cuda.synchronize()
    h_ref = swiglu.swiglu(bits16(a), bits16(b))
    _assert_same_bits(bits16(h), h_ref, "h")
    q_ref, s_ref = quant.quant_1x128_rowwise(h_ref)
    assert np.array_equal(u8(qr), q_ref)
    assert np.array_equal(sr.cpu().numpy().T[:R], s_ref)
    check_canaries(qr_full, R, C)


def test_swiglu_quant_rejects_mismatched_b():
    need_gpu()
    a = torch.zeros((128, 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="b must be"):
        bs.bs_swiglu_quant_1x128(a, a[:, :128], None, torch.empty((128, 256), dtype=torch.uint8, device="cuda"),
                                 bs.empty_scales(2, 128, "cuda"))


# ---- backward ----

def _grad_inputs(R, C, seed):
    a, b = _inputs(R, C, seed)
    dh = inputs.bf16_normal((R, C), 0.01, seed + 2)
    if R >= 10 and C >= 128:   # extreme magnitudes: intermediate products leave the normal range
        db = bits16(b).copy()
        dd = bits16(dh).copy()
        db[8, :64] = bits16(torch.full((64,), 3e30, dtype=torch.bfloat16))
        dd[8, 64:128] = bits16(torch.full((64,), 2e-30, dtype=torch.bfloat16))
        dd[9, :128] = bits16(torch.full((128,), 1e-37, dtype=torch.bfloat16))
        b, dh = _from_bits(db), _from_bits(dd)
    return a, b, dh


def _dab_ref(a, b, dh):
    da, db = swiglu.swiglu_backward(bits16(a), bits16(b), bits16(dh))
    return np.concatenate([da, db], axis=1)


@pytest.mark.parametrize("R,C", [(256, 512), (384, 640), (128, 128)])
def test_swiglu_bwd_quant_rows_and_cols(R, C):
    need_gpu()
    a, b, dh = _grad_inputs(R, C, seed=3 * R + C)
    dab_full, dab = guarded(R, 2 * C, torch.bfloat16)
    qr_full, qr = guarded(R, 2 * C, torch.uint8)
    sr_full, sr = scale_buffer(2 * C // 128, R)
    qc_full, qc = guarded(2 * C, R, torch.uint8)
    sc_full, sc = scale_buffer(R // 128, 2 * C)
    print(f"swiglu_bwd_quant R={R} C={C}", flush=True)
    bs.bs_swiglu_bwd_quant_1x128(a.cuda(), b.cuda(), dh.cuda(), dab, qr, sr, qc, sc)
    torch.cuda.synchronize()
    want = _dab_ref(a, b, dh)
    _assert_same_bits(bits16(dab), want, "[da | db]")
    q_ref, s_ref = quant.quant_1x128_rowwise(want)
    assert np.array_equal(u8(qr), q_ref)
    assert np.array_equal(sr.cpu().numpy().T[:R], s_ref)
    qc_ref, sc_ref = quant.quant_1x128_colwise(want)
    assert np.array_equal(u8(qc), qc_ref)
    assert np.array_equal(sc.cpu().numpy().T[:2 * C], sc_ref)
    for full, r, c in [(dab_full, R, 2 * C), (qr_full, R, 2 * C), (qc_full, 2 * C, R)]:
        check_canaries(full, r, c)
    check_scale_canaries(sr_full, 2 * C // 128, R)
    check_scale_canaries(sc_full, R // 128, 2 * C)

    # the same codes without writing [da | db], and each output alone
    qr2, sr2 = torch.empty_like(qr), torch.empty_like(sr)
    bs.bs_swiglu_bwd_quant_1x128(a.cuda(), b.cuda(), dh.cuda(), None, qr2, sr2)
    qc2, sc2 = torch.empty_like(qc), torch.empty_like(sc)
    bs.bs_swiglu_bwd_quant_1x128(a.cuda(), b.cuda(), dh.cuda(), None, None, None, qc2, sc2)
    torch.cuda.synchronize()
    assert torch.equal(qr2, qr) and torch.equal(sr2[:, :R], sr[:, :R])
    assert torch.equal(qc2, qc) and torch.equal(sc2[:, :2 * C], sc[:, :2 * C])


@pytest.mark.parametrize("R", [1, 77, 300])
def test_swiglu_bwd_quant_ragged_rows(R):
    need_gpu()
    C = 256
    a, b, dh = _grad_inputs(R, C, seed=R + 1)
    dab = torch.empty((R, 2 * C), dtype=torch.bfloat16, device="cuda")
    qr_full, qr = guarded(R, 2 * C, torch.uint8)
    sr = bs.empty_scales(2 * C // 128, R, "cuda")
    print(f"swiglu_bwd_quant ragged R={R}", flush=True)
    bs.bs_swiglu_bwd_quant_1x128(a.cuda(), b.cuda(), dh.cuda(), dab, qr, sr)
    torch.cuda.synchronize()
    want = _dab_ref(a, b, dh)
    _assert_same_bits(bits16(dab), want, "[da | db]")
    q_ref, s_ref = quant.quant_1x128_rowwise(want)
    assert np.array_equal(u8(qr), q_ref)
    assert np.array_equal(sr.cpu().numpy().T[:R], s_ref)
    check_canaries(qr_full, R, 2 * C)


def test_swiglu_bwd_quant_views_of_a_stacked_activation():
    # the FFN passes a and b as the two column halves of one [R, 2C] tensor
    need_gpu()
    R, C = 256, 512
    a, b, dh = _grad_inputs(R, C, seed=9)
    ab = torch.cat([a, b], 1).cuda()
    qr = torch.empty((R, 2 * C), dtype=torch.uint8, device="cuda")
    sr = bs.empty_scales(2 * C // 128, R, "cuda")
    print("swiglu_bwd_quant strided views", flush=True)
    bs.bs_swiglu_bwd_quant_1x128(ab[:, :C], ab[:, C:], dh.cuda(), None, qr, sr)
    torch.cuda.synchronize()
    q_ref, s_ref = quant.quant_1x128_rowwise(_dab_ref(a, b, dh))
    assert np.array_equal(u8(qr), q_ref)
    assert np.array_equal(sr.cpu().numpy().T[:R], s_ref)


# ---- operands large enough for one workgroup per tile ----

def _sampled_tiles(R, C, seed, n=24):
    rng = np.random.default_rng(seed)
    tr, tc = R // 128, C // 128
    return [(0, 0), (tr - 1, tc - 1)] + [tuple(int(v) for v in t) for t in rng.integers(0, [tr, tc], size=(n, 2))]


def test_swiglu_quant_large_sampled():
    """8192 x 12288 (6144 tiles, at least 2 persistent grids of this kernel:
    one workgroup per tile): h and the codes and scales of sampled 128x128
    tiles bit-exact against the oracle run on those tiles (blocks are
    independent, so a tile's expected bytes depend on that tile alone)."""
    need_gpu()
    R, C = 8192, 12288
    a, b = _inputs(R, C, seed=71)
    h = torch.empty((R, C), dtype=torch.bfloat16, device="cuda")
    qr = torch.empty((R, C), dtype=torch.uint8, device="cuda")
    sr = bs.empty_scales(C // 128, R, "cuda")
    qc = torch.empty((C, R), dtype=torch.uint8, device="cuda")
    sc = bs.empty_scales(R // 128, C, "cuda")
    print(f"swiglu_quant {R}x{C} (one workgroup per tile)", flush=True)
    bs.bs_swiglu_quant_1x128(a.cuda(), b.cuda(), h, qr, sr, qc, sc)
    torch.cuda.synchronize()
    ab, bb = bits16(a), bits16(b)
    hg, qrg, qcg = bits16(h), u8(qr), u8(qc)
    srg, scg = sr.cpu().numpy(), sc.cpu().numpy()
    for (i, j) in _sampled_tiles(R, C, 71):
        rs, cs = slice(128 * i, 128 * (i + 1)), slice(128 * j, 128 * (j + 1))
        h_ref = swiglu.swiglu(np.ascontiguousarray(ab[rs, cs]), np.ascontiguousarray(bb[rs, cs]))
        _assert_same_bits(hg[rs, cs], h_ref, f"h of tile {(i, j)}")
        q_ref, s_ref = quant.quant_1x128_rowwise(h_ref)
        assert np.array_equal(qrg[rs, cs], q_ref), f"row codes of tile {(i, j)}"
        assert np.array_equal(srg[j, rs], s_ref[:, 0]), f"row scales of tile {(i, j)}"
        q_ref, s_ref = quant.quant_1x128_colwise(h_ref)
        assert np.array_equal(qcg[cs, rs], q_ref), f"column codes of tile {(i, j)}"
        assert np.array_equal(scg[i, cs], s_ref[:, 0]), f"column scales of tile {(i, j)}"


def test_swiglu_bwd_quant_large_sampled():
    """The backward at 8192 x 12288 (one workgroup per tile): [da | db] and its
    codes and scales on sampled tiles bit-exact against the oracle; tile
    (i, j) of the input feeds tiles (i, j) (da) and (i, j + C/128) (db) of the
    [R, 2C] output."""
    need_gpu()
    R, C = 8192, 12288
    a, b, dh = _grad_inputs(R, C, seed=73)
    dab = torch.empty((R, 2 * C), dtype=torch.bfloat16, device="cuda")
    qr = torch.empty((R, 2 * C), dtype=torch.uint8, device="cuda")
    sr = bs.empty_scales(2 * C // 128, R, "cuda")
    qc = torch.empty((2 * C, R), dtype=torch.uint8, device="cuda")
    sc = bs.empty_scales(R // 128, 2 * C, "cuda")
    print(f"swiglu_bwd_quant {R}x{C} (one workgroup per tile)", flush=True)
    bs.bs_swiglu_bwd_quant_1x128(a.cuda(), b.cuda(), dh.cuda(), dab, qr, sr, qc, sc)
    torch.cuda.synchronize()
    ab, bb, db_ = bits16(a), bits16(b), bits16(dh)
    dg, qrg, qcg = bits16(dab), u8(qr), u8(qc)
    srg, scg = sr.cpu().numpy(), sc.cpu().numpy()
    for (i, j) in _sampled_tiles(R, C, 73):
        rs, cs = slice(128 * i, 128 * (i + 1)), slice(128 * j, 128 * (j + 1))
        da, db = swiglu.swiglu_backward(*(np.ascontiguousarray(t[rs, cs]) for t in (ab, bb, db_)))
        for part, ref in ((0, da), (1, db)):
            oc = slice(128 * (j + part * C // 128), 128 * (j + part * C // 128 + 1))
            jj = j + part * C // 128
            _assert_same_bits(dg[rs, oc], ref, f"{'db' if part else 'da'} of tile {(i, j)}")
            q_ref, s_ref = quant.quant_1x128_rowwise(ref)
            assert np.array_equal(qrg[rs, oc], q_ref), f"row codes of tile {(i, jj)}"
            assert np.array_equal(srg[jj, rs], s_ref[:, 0]), f"row scales of tile {(i, jj)}"
            q_ref, s_ref = quant.quant_1x128_colwise(ref)
            assert np.array_equal(qcg[oc, rs], q_ref), f"column codes of tile {(i, jj)}"
            assert np.array_equal(scg[i, oc], s_ref[:, 0]), f"column scales of tile {(i, jj)}"


@pytest.mark.parametrize("b_kind", ["ones", "threes", "normal"])
def test_swiglu_quant_every_bf16_gate_value(b_kind):
    """Every finite bf16 value of a (non-finite patterns replaced by 0) against
    b = 1, b = 3 and seeded normal b: h bit-exact against the oracle's float64
    formula rounded once, and the row codes against its quantization of h.
    Covers the whole range of the fp32 path (its reciprocal, the tie window,
    the a <= -69 and subnormal hand-offs to float64) value by value."""
    need_gpu()
    R, C = 512, 128
    ab = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ab[(ab & 0x7F80) == 0x7F80] = 0                     # inf / NaN patterns
    ab = ab.reshape(R, C)
    if b_kind == "normal":
        b = inputs.bf16_normal((R, C), 1.0, 77)
    else:
        b = torch.full((R, C), 1.0 if b_kind == "ones" else 3.0, dtype=torch.bfloat16)
    a = _from_bits(ab)
    h = torch.empty((R, C), dtype=torch.bfloat16, device="cuda")
    qr = torch.empty((R, C), dtype=torch.uint8, device="cuda")
    sr = bs.empty_scales(C // 128, R, "cuda")
    print(f"swiglu_quant every bf16 a, b={b_kind}", flush=True)
    bs.bs_swiglu_quant_1x128(a.cuda(), b.cuda(), h, qr, sr)
    torch.cuda.synchronize()
    h_ref = swiglu.swiglu(ab, bits16(b))
    got = bits16(h)
    # Where the float64 value is within 2^-48 (relative) of a bf16 tie, float64
    # cannot tell the side (the last bit of exp decides it), and either
    # neighbour is the reading's answer, as in the oracle's own pin; there
    # only, the other neighbour (same sign, one step away) is accepted.
    diff = got != h_ref
    if diff.any():
        v = np.abs(swiglu.swiglu_f64(ab, bits16(b))[diff])
        _, e = np.frexp(v)                                  # v = m 2^e, m in [0.5, 1)
        step = np.ldexp(1.0, np.maximum(e - 1 - 7, -133))   # bf16 spacing in v's binade
        k = v / step
        near_tie = np.abs(k - np.floor(k) - 0.5) * step < v * 2.0 ** -48
        one_step = ((got[diff] ^ h_ref[diff]) & 0x8000 == 0) & \
                   (np.abs(got[diff].astype(np.int32) - h_ref[diff].astype(np.int32)) == 1)
        bad = ~(near_tie & one_step)
        assert not bad.any(), f"h: {bad.sum()} elements differ outside the float64 tie region, first at " \
                              f"{np.argwhere(diff)[np.flatnonzero(bad)[:3]]}"
    # Overflow (|a| near the bf16 maximum times |b| > 1): h is +-inf exactly
    # where the oracle's is, as the header states; the codes and scale of a
    # block holding an infinite h are unspecified there (outside the
    # quantizer's finite domain), so those rows' codes are not compared.
    inf_ref = (h_ref & 0x7FFF) == 0x7F80
    assert not (((h_ref & 0x7F80) == 0x7F80) & ~inf_ref).any(), "the oracle's h is never NaN"
    assert np.array_equal(got[inf_ref], h_ref[inf_ref]), "overflowing h must be written as +-inf"
    assert not ((got & 0x7F80) == 0x7F80)[~inf_ref].any(), "h is finite wherever the oracle's is"
    if b_kind == "threes":
        # b = 3: silu(a) * 3 overflows for the largest bf16 a
        assert inf_ref.any()
    # the codes of every other row equal the oracle's quantization of its h
    # (rows with a float64-tie element of h, whose h may be the other
    # neighbour, excepted: the oracle quantizes its own h only)
    ok = ~inf_ref.any(axis=1) & ~diff.any(axis=1)
    assert (~ok).sum() == (inf_ref.any(axis=1) | diff.any(axis=1)).sum() <= 8
    q_ref, s_ref = quant.quant_1x128_rowwise(np.ascontiguousarray(h_ref[ok]))
    assert np.array_equal(u8(qr)[ok], q_ref)
    assert np.array_equal(sr.cpu().numpy().T[:R][ok], s_ref)


def _tie_tolerant(got, want, v):
    """Positions where got != want are allowed only where the float64 value v
    is within 2^-48 (relative) of a bf16 tie and got is the other neighbour."""
    diff = got != want
    if not diff.any():
        return diff
    x = np.abs(v[diff])
    _, e = np.frexp(x)
    step = np.ldexp(1.0, np.maximum(e - 8, -133))
    k = x / step
    near_tie = np.abs(k - np.floor(k) - 0.5) * step < x * 2.0 ** -48
    one_step = ((got[diff] ^ want[diff]) & 0x8000 == 0) & \
               (np.abs(got[diff].astype(np.int32) - want[diff].astype(np.int32)) == 1)
    bad = ~(near_tie & one_step)
    assert not bad.any(), f"{bad.sum()} elements differ outside the float64 tie region, first at " \
                          f"{np.argwhere(diff)[np.flatnonzero(bad)[:3]]}"
    return diff


@pytest.mark.parametrize("kind", ["unit", "normal"])
def test_swiglu_bwd_every_bf16_gate_value(kind):
    """The backward on every finite bf16 value of a (non-finite patterns
    replaced by 0): b = 3, dh = 1 and seeded normal b, dh.  [da | db]
    bit-exact against the oracle (the other neighbour accepted only within
    2^-48 of a tie, R20), so every branch of the fp32 path and its windows
    is exercised value by value."""
    need_gpu()
    R, C = 512, 128
    ab = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ab[(ab & 0x7F80) == 0x7F80] = 0
    ab = ab.reshape(R, C)
    if kind == "unit":
        b = torch.full((R, C), 3.0, dtype=torch.bfloat16)
        dh = torch.full((R, C), 1.0, dtype=torch.bfloat16)
    else:
        b = inputs.bf16_normal((R, C), 1.0, 78)
        dh = inputs.bf16_normal((R, C), 0.01, 79)
    a = _from_bits(ab)
    dab = torch.empty((R, 2 * C), dtype=torch.bfloat16, device="cuda")
    qr = torch.empty((R, 2 * C), dtype=torch.uint8, device="cuda")
    sr = bs.empty_scales(2 * C // 128, R, "cuda")
    print(f"swiglu_bwd every bf16 a, {kind}", flush=True)
    bs.bs_swiglu_bwd_quant_1x128(a.cuda(), b.cuda(), dh.cuda(), dab, qr, sr)
    torch.cuda.synchronize()
    da, db = swiglu.swiglu_backward(ab, bits16(b), bits16(dh))
    g = bits16(dab)
    va, vb = swiglu.swiglu_backward_f64(ab, bits16(b), bits16(dh))
    diff_a = _tie_tolerant(g[:, :C], da, va)
    diff_b = _tie_tolerant(g[:, C:], db, vb)
    # an overflowing da or db is +-inf exactly where the oracle's is (header);
    # the codes of blocks holding one are unspecified and not compared
    for got_, ref_, nm in ((g[:, :C], da, "da"), (g[:, C:], db, "db")):
        inf_ref = (ref_ & 0x7FFF) == 0x7F80
        assert np.array_equal(got_[inf_ref], ref_[inf_ref]), f"overflowing {nm} must be written as +-inf"
        assert not ((got_ & 0x7F80) == 0x7F80)[~inf_ref].any(), f"{nm} is finite wherever the oracle's is"
    inf_rows = ((da & 0x7FFF) == 0x7F80).any(axis=1) | ((db & 0x7FFF) == 0x7F80).any(axis=1)
    ok = ~inf_rows & ~diff_a.any(axis=1) & ~diff_b.any(axis=1)
    assert (~ok).sum() <= 8
    q_ref, s_ref = quant.quant_1x128_rowwise(np.ascontiguousarray(np.concatenate([da, db], axis=1)[ok]))
    assert np.array_equal(u8(qr)[ok], q_ref)
    assert np.array_equal(sr.cpu().numpy().T[:R][ok], s_ref)


def test_fused_kernels_repeat_byte_for_byte():
    """Three runs of each fused kernel (and the plain 1x128 pass) on the same
    8192x4096 inputs write the same bytes: the LDS exchanges of the column
    quantization and the float64 redo loop leave nothing to timing."""
    need_gpu()
    M, N = 8192, 4096
    a = inputs.bf16_normal((M, N), 1.0, 71, device="cuda")
    b = inputs.bf16_normal((M, N), 1.0, 72, device="cuda")
    dh = inputs.bf16_normal((M, N), 0.01, 73, device="cuda")

    def outs(rows, cols):
        return (torch.full((rows, cols), 0x5A, dtype=torch.uint8, device="cuda"),
                bs.empty_scales(cols // 128, rows, "cuda").fill_(-7.0),
                torch.full((cols, rows), 0x5A, dtype=torch.uint8, device="cuda"),
                bs.empty_scales(rows // 128, cols, "cuda").fill_(-7.0))

    runs = {"forward": [], "backward": [], "plain": []}
    for _ in range(3):
        q, s, qt, st = outs(M, N)
        print("fused forward run", flush=True)
        bs.bs_swiglu_quant_1x128(a, b, None, q, s, qt, st)
        runs["forward"].append((q, s, qt, st))
        q, s, qt, st = outs(M, 2 * N)
        print("fused backward run", flush=True)
        bs.bs_swiglu_bwd_quant_1x128(a, b, dh, None, q, s, qt, st)
        runs["backward"].append((q, s, qt, st))
        q, s, qt, st = outs(M, N)
        bs.bs_quant_1x128(a, q, s, qt, st)
        runs["plain"].append((q, s, qt, st))
    torch.cuda.synchronize()
    for what, rs in runs.items():
        for r in rs[1:]:
            for name, x, y in zip(("row codes", "row scales", "column codes", "column scales"), rs[0], r):
                assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), f"{what}: {name} differ between runs"
