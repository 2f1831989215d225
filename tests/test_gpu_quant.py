"""GPU parity of the quantizers against the CPU oracle: bit-exact codes and
scales, scale padding and guard bands untouched.  Calls go through the C ABI
(via the thin binding)."""

import numpy as np
import pytest
import torch

import blockwise_scaled_fp8_bs_amd as bs
from blockwise_scaled_fp8_bs_amd import inputs
from oracle import quant
from gpu_support import (bits16, check_canaries, check_scale_canaries, f32bits, guarded, need_gpu,
                         scale_buffer, special_input, u8)

pytestmark = pytest.mark.gpu


def assert_scales(s_gpu_view, s_logical):
    """s_gpu_view is K-major [nkb, ld]; s_logical is [count, nkb]."""
    count, nkb = s_logical.shape
    got = f32bits(s_gpu_view[:, :count])
    want = np.ascontiguousarray(s_logical.T).view(np.uint32)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} scale mismatches, first at (kb, row) {bad[0]}: got {got[tuple(bad[0])]:#x} want {want[tuple(bad[0])]:#x}"


def assert_codes(q_gpu, q_ref):
    got = u8(q_gpu)
    bad = np.argwhere(got != q_ref)
    assert bad.size == 0, f"{len(bad)} code mismatches, first at {bad[0]}: got {got[tuple(bad[0])]:#x} want {q_ref[tuple(bad[0])]:#x}"


@pytest.mark.parametrize("R,C", [(256, 512), (384, 640), (128, 128), (512, 256)])
@pytest.mark.parametrize("mode", ["row+col", "row", "col"])
def test_quant_1x128(R, C, mode):
    need_gpu()
    x = special_input(R, C, seed=R * 7 + C)
    xfull = torch.zeros((R, C + 64), dtype=torch.bfloat16)
    xfull[:, :C] = x
    xg = xfull.cuda()[:, :C]  # padded ld_x
    row, col = "row" in mode, "col" in mode
    qr_full, qr = guarded(R, C, torch.uint8) if row else (None, None)
    sr_full, sr = scale_buffer(C // 128, R) if row else (None, None)
    qc_full, qc = guarded(C, R, torch.uint8) if col else (None, None)
    sc_full, sc = scale_buffer(R // 128, C) if col else (None, None)
    print(f"quant_1x128 R={R} C={C} mode={mode}", flush=True)
    bs.bs_quant_1x128(xg, qr, sr, qc, sc)
    torch.cuda.synchronize()
    xb = bits16(x)
    if row:
        q_ref, s_ref = quant.quant_1x128_rowwise(xb)
        assert_codes(qr, q_ref)
        assert_scales(sr, s_ref)
        check_canaries(qr_full, R, C)
        check_scale_canaries(sr_full, C // 128, R)
    if col:
        q_ref, s_ref = quant.quant_1x128_colwise(xb)
        assert_codes(qc, q_ref)
        assert_scales(sc, s_ref)
        check_canaries(qc_full, C, R)
        check_scale_canaries(sc_full, R // 128, C)


@pytest.mark.parametrize("R", [1, 77, 300])
def test_quant_1x128_ragged_rows(R):
    need_gpu()
    C = 384
    x = special_input(R, C, seed=R)
    qr_full, qr = guarded(R, C, torch.uint8)
    sr_full, sr = scale_buffer(C // 128, R)
    bs.bs_quant_1x128(x.cuda(), qr, sr)
    torch.cuda.synchronize()
    q_ref, s_ref = quant.quant_1x128_rowwise(bits16(x))
    assert_codes(qr, q_ref)
    assert_scales(sr, s_ref)
    check_canaries(qr_full, R, C)
    check_scale_canaries(sr_full, C // 128, R)


@pytest.mark.parametrize("R,C,pad", [(256, 512, 0), (384, 640, 4), (128, 896, 0)])
def test_quant_128x128(R, C, pad):
    need_gpu()
    x = special_input(R, C, seed=R + C, sigma=0.02)
    q_full, q = guarded(R, C, torch.uint8)
    s_full, s = scale_buffer(C // 128, R // 128, pad=pad)
    print(f"quant_128x128 R={R} C={C} ld_s={s.stride(0)}", flush=True)
    bs.bs_quant_128x128(x.cuda(), q, s)
    torch.cuda.synchronize()
    q_ref, s_ref = quant.quant_128x128(bits16(x))
    assert_codes(q, q_ref)
    assert_scales(s, s_ref)  # logical [R/128, C/128] -> K-major [C/128][ld >= R/128]
    check_canaries(q_full, R, C)
    check_scale_canaries(s_full, C // 128, R // 128)


@pytest.mark.parametrize("G,R,C", [(1, 256, 512), (3, 256, 384), (2, 384, 128)])
def test_quant_3d_colwise(G, R, C):
    need_gpu()
    x = torch.stack([special_input(R, C, seed=g * 11 + R, sigma=0.02) for g in range(G)])
    ld_s = (C // 128 + 3) // 4 * 4 + 4
    q_full = torch.full((G + 1, C, R + 16), 0xA5, dtype=torch.uint8, device="cuda")
    q = q_full[:G, :, :R]
    s_full = torch.empty((G + 1, R // 128, ld_s), dtype=torch.float32, device="cuda")
    s_full.view(torch.int32).fill_(0x7FBADBAD)
    s = s_full[:G]
    print(f"quant_3d_colwise G={G} R={R} C={C}", flush=True)
    bs.bs_quant_3d_colwise(x.cuda(), q, s)
    torch.cuda.synchronize()
    q_ref, s_ref = quant.quant_3d_colwise(bits16(x))
    qg = u8(q_full)
    assert np.array_equal(qg[:G, :, :R], q_ref)
    assert np.all(qg[:G, :, R:] == 0xA5) and np.all(qg[G:] == 0xA5)
    sg = s_full.cpu().view(torch.int32).numpy().view(np.uint32)
    for g in range(G):
        # s_ref[g] is [C/128, R/128] (rows of the transposed operand x blocks of
        # its contraction); the layout is K-major: s[g][rb][cb]
        assert np.array_equal(sg[g, :, :C // 128], np.ascontiguousarray(s_ref[g].T).view(np.uint32))
    assert np.all(sg[:G, :, C // 128:] == 0x7FBADBAD) and np.all(sg[G:] == 0x7FBADBAD)


@pytest.mark.parametrize("G,R,C,xpad", [(1, 384, 640, 0), (3, 256, 384, 128), (2, 128, 896, 0)])
def test_quant_128x128_both(G, R, C, xpad):
    """The fused pass writes exactly what bs_quant_128x128 on the stacked
    weights and bs_quant_3d_colwise write (oracle codes and scales)."""
    need_gpu()
    x = torch.stack([special_input(R, C, seed=g * 13 + C, sigma=0.02) for g in range(G)])
    xs = torch.zeros((G, R + xpad // 128 * 128, C + 16), dtype=torch.bfloat16)
    xs[:, :R, :C] = x
    xg = xs.cuda()[:, :R, :C]                      # strided experts and rows
    ld_s = (G * R // 128 + 3) // 4 * 4 + 4
    q_full = torch.full((G * R + 1, C + 16), 0xA5, dtype=torch.uint8, device="cuda")
    q = q_full[:G * R, :C]
    s_full = torch.empty((C // 128 + 1, ld_s), dtype=torch.float32, device="cuda")
    s_full.view(torch.int32).fill_(0x7FBADBAD)
    s = s_full[:C // 128]
    ld_st = (C // 128 + 3) // 4 * 4 + 4
    qt_full = torch.full((G + 1, C, R + 16), 0xA5, dtype=torch.uint8, device="cuda")
    qt = qt_full[:G, :, :R]
    st_full = torch.empty((G + 1, R // 128, ld_st), dtype=torch.float32, device="cuda")
    st_full.view(torch.int32).fill_(0x7FBADBAD)
    st = st_full[:G]
    print(f"quant_128x128_both G={G} R={R} C={C}", flush=True)
    bs.bs_quant_128x128_both(xg, q, s, qt, st)
    torch.cuda.synchronize()
    xb = bits16(x)
    q_ref, s_ref = quant.quant_128x128(xb.reshape(G * R, C))
    qt_ref, st_ref = quant.quant_3d_colwise(xb)
    qa = u8(q_full)
    assert np.array_equal(qa[:G * R, :C], q_ref)
    assert np.all(qa[:G * R, C:] == 0xA5) and np.all(qa[G * R:] == 0xA5)
    sa = s_full.cpu().view(torch.int32).numpy().view(np.uint32)
    assert np.array_equal(sa[:C // 128, :G * R // 128], np.ascontiguousarray(s_ref.T).view(np.uint32))
    assert np.all(sa[:C // 128, G * R // 128:] == 0x7FBADBAD) and np.all(sa[C // 128:] == 0x7FBADBAD)
    qta = u8(qt_full)
    assert np.array_equal(qta[:G, :, :R], qt_ref)
    assert np.all(qta[:G, :, R:] == 0xA5) and np.all(qta[G:] == 0xA5)
    sta = st_full.cpu().view(torch.int32).numpy().view(np.uint32)
    for g in range(G):
        assert np.array_equal(sta[g, :, :C // 128], np.ascontiguousarray(st_ref[g].T).view(np.uint32))
    assert np.all(sta[:G, :, C // 128:] == 0x7FBADBAD) and np.all(sta[G:] == 0x7FBADBAD)


def test_quant_division_not_reciprocal():
    """Blocks where x * fl32(1/s) and fl32(x / s) give different codes."""
    need_gpu()
    from oracle import e4m3
    rng = np.random.default_rng(7)
    found = []
    while len(found) < 128:
        xb = bits16(torch.from_numpy(rng.standard_normal((256, 128)).astype(np.float32)).to(torch.bfloat16))
        x = quant.bf16_bits_to_f32(xb)
        s = (np.maximum(np.abs(x).max(axis=1), quant.EPS) / np.float32(448)).astype(np.float32)
        d = e4m3.encode(np.clip(x / s[:, None], -448, 448).astype(np.float32))
        r = e4m3.encode(np.clip(x * (np.float32(1) / s)[:, None], -448, 448).astype(np.float32))
        found.extend(xb[(d != r).any(axis=1)])
    xb = np.stack(found[:128])
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).cuda()
    qr = torch.empty((128, 128), dtype=torch.uint8, device="cuda")
    sr = bs.empty_scales(1, 128, "cuda")
    bs.bs_quant_1x128(x, qr, sr)
    torch.cuda.synchronize()
    q_ref, s_ref = quant.quant_1x128_rowwise(xb)
    assert_codes(qr, q_ref)
    assert_scales(sr, s_ref)


def test_binding_rejects_wrong_layout():
    need_gpu()
    x = torch.zeros((256, 256), dtype=torch.bfloat16, device="cuda").t()  # column-major view
    q = torch.empty((256, 256), dtype=torch.uint8, device="cuda")
    s = bs.empty_scales(2, 256, "cuda")
    with pytest.raises(ValueError, match="unit stride"):
        bs.bs_quant_1x128(x, q, s)
    with pytest.raises(bs.BsError, match="multiple of 4"):
        bs.bs_quant_1x128(x.t(), q, torch.empty((2, 258), device="cuda")[:, :257])


def test_empty_inputs():
    need_gpu()
    x = torch.empty((1, 256), dtype=torch.bfloat16, device="cuda")[:0]
    q = torch.empty((1, 256), dtype=torch.uint8, device="cuda")[:0]
    bs.bs_quant_1x128(x, q, bs.empty_scales(2, 0, "cuda", pad=4))
    torch.cuda.synchronize()


def test_quant_large_one_workgroup_per_tile():
    """Operands of at least 2 persistent grids' worth of tiles (here 8192 tiles
    against 256 CUs x 3 workgroups) are launched with one workgroup per tile:
    the 1x128 row + column pass and the 128x128 pass in both layouts must
    match the oracle bit for bit there too.  Blocks are independent, so the
    oracle run on a 128x128 tile gives that tile's exact expected bytes; 40
    seeded tiles are checked, including the first and the last, with planted
    zero, tiny and saturating tiles among them."""
    need_gpu()
    R, C = 8192, 16384
    x = inputs.bf16_normal((R, C), 1.0, seed=41)
    rng = np.random.default_rng(41)
    tr, tc = R // 128, C // 128
    picks = [(0, 0), (tr - 1, tc - 1)] + [tuple(t) for t in rng.integers(0, [tr, tc], size=(38, 2))]
    (zr, zc), (yr, yc), (br, bc) = picks[2], picks[3], picks[4]
    x[zr * 128:(zr + 1) * 128, zc * 128:(zc + 1) * 128] = 0.0
    x[yr * 128:(yr + 1) * 128, yc * 128:(yc + 1) * 128] *= 1e-20
    x[br * 128:(br + 1) * 128, bc * 128:(bc + 1) * 128] *= 1e30
    xg = x.cuda()
    qr = torch.empty((R, C), dtype=torch.uint8, device="cuda")
    sr = bs.empty_scales(C // 128, R, "cuda")
    qc = torch.empty((C, R), dtype=torch.uint8, device="cuda")
    sc = bs.empty_scales(R // 128, C, "cuda")
    print(f"quant_1x128 rows+cols, one workgroup per tile, {R}x{C}", flush=True)
    bs.bs_quant_1x128(xg, qr, sr, qc, sc)
    qw = torch.empty((R, C), dtype=torch.uint8, device="cuda")
    sw = bs.empty_scales(C // 128, R // 128, "cuda")
    qwt = torch.empty((1, C, R), dtype=torch.uint8, device="cuda")
    swt = bs.empty_scales(R // 128, C // 128, "cuda")[None]
    print(f"quant_128x128 both layouts, one workgroup per tile, {R}x{C}", flush=True)
    bs.bs_quant_128x128_both(xg.view(1, R, C), qw, sw, qwt, swt)
    torch.cuda.synchronize()
    xb = bits16(x)
    got = {n: t.cpu().numpy() for n, t in
           dict(qr=qr, qc=qc, qw=qw, qwt=qwt[0]).items()}
    gs = {n: t.cpu().numpy().view(np.uint32) for n, t in dict(sr=sr, sc=sc, sw=sw, swt=swt[0]).items()}
    for (i, j) in picks:
        rs, cs = slice(i * 128, (i + 1) * 128), slice(j * 128, (j + 1) * 128)
        t = np.ascontiguousarray(xb[rs, cs])
        q, s = quant.quant_1x128_rowwise(t)
        assert np.array_equal(got["qr"][rs, cs], q), f"row codes of tile {(i, j)}"
        assert np.array_equal(gs["sr"][j, rs], s[:, 0].view(np.uint32)), f"row scales of tile {(i, j)}"
        q, s = quant.quant_1x128_colwise(t)
        assert np.array_equal(got["qc"][cs, rs], q), f"column codes of tile {(i, j)}"
        assert np.array_equal(gs["sc"][i, cs], s[:, 0].view(np.uint32)), f"column scales of tile {(i, j)}"
        q, s = quant.quant_128x128(t)
        assert np.array_equal(got["qw"][rs, cs], q), f"128x128 codes of tile {(i, j)}"
        assert gs["sw"][j, i] == s.view(np.uint32)[0, 0], f"128x128 scale of tile {(i, j)}"
        assert np.array_equal(got["qwt"][cs, rs], q.T), f"transposed 128x128 codes of tile {(i, j)}"
        assert gs["swt"][i, j] == s.view(np.uint32)[0, 0], f"transposed 128x128 scale of tile {(i, j)}"


def test_quant_largest_leading_dimensions():
    """x and the row codes stored with leading dimensions just under the 2^22
    limit the boundary accepts: codes and scales still bit-exact."""
    need_gpu()
    R, C = 128, 512
    ld = (1 << 22) - 64
    x = special_input(R, C, seed=93)
    xbuf = torch.zeros((R, ld), dtype=torch.bfloat16, device="cuda")
    xg = xbuf[:, ld - C:]
    xg.copy_(x.cuda())
    qbuf = torch.zeros((R, ld), dtype=torch.uint8, device="cuda")
    qr = qbuf[:, ld - C:]
    sr = bs.empty_scales(C // 128, R, "cuda")
    qc = torch.empty((C, R), dtype=torch.uint8, device="cuda")
    sc = bs.empty_scales(R // 128, C, "cuda")
    print(f"quant_1x128 ld_x=ld_qr={ld}", flush=True)
    bs.bs_quant_1x128(xg, qr, sr, qc, sc)
    q128 = torch.empty((R, C), dtype=torch.uint8, device="cuda")
    s128 = bs.empty_scales(C // 128, R // 128, "cuda")
    bs.bs_quant_128x128(xg, q128, s128)
    torch.cuda.synchronize()
    xb = bits16(x)
    q_ref, s_ref = quant.quant_1x128_rowwise(xb)
    assert_codes(qr, q_ref)
    assert_scales(sr, s_ref)
    q_ref, s_ref = quant.quant_1x128_colwise(xb)
    assert_codes(qc, q_ref)
    assert_scales(sc, s_ref)
    q_ref, s_ref = quant.quant_128x128(xb)
    assert_codes(q128, q_ref)
    assert_scales(s128, s_ref)
    del xbuf, qbuf
    torch.cuda.empty_cache()
