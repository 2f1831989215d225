"""GPU parity of the MXFP8 quantizer and GEMM (32-element blocks, E8M0
scales) against the CPU oracle.

The quantizer's codes and scale bytes must equal the oracle's bit for bit,
rows and transposed columns.  GEMM operands are made on the CPU (the
oracle's quantizer, or codes and scale bytes drawn directly) and the GPU
product is compared with the oracle's float64 product within
2e-3 * ||a_m|| * ||b_n||; the exact-arithmetic case must match bit for bit.
Calls go through the C ABI (thin binding)."""

import numpy as np
import pytest
import torch

import blockwise_scaled_fp8_bs_amd as bs
from blockwise_scaled_fp8_bs_amd import inputs
from gpu_support import CANARY_U8, bf16_from_bits, bits16, check_canaries, guarded, need_gpu, special_input, u8
from oracle import e4m3, gemm, mx

pytestmark = pytest.mark.gpu


def _mx_input(R, C, seed):
    """special_input plus blocks at the MX scale's edges."""
    b = bits16(special_input(R, C, seed)).copy()
    if R >= 12 and C >= 128:
        b[7, 32:64] = bits16(torch.full((32,), 1.0, dtype=torch.bfloat16))
        b[7, 40] = bits16(torch.tensor([480.0], dtype=torch.bfloat16))[0]     # amax / X in [448, 512): saturates
        b[8, 64:96] = bits16(torch.full((32,), -256.0, dtype=torch.bfloat16))  # amax a power of two
        b[9, 0:32] = 0x0001                                                      # smallest bf16 subnormal
        b[9, 32:64] = bits16(torch.full((32,), 2.0 ** -118, dtype=torch.bfloat16))  # scale exponent -126
        b[10, 96:128] = bits16(torch.full((32,), 2.0 ** -120, dtype=torch.bfloat16))  # clamped at -127
        b[11, 0:32] = 0x7F7F                                                     # bf16 max everywhere
    return bf16_from_bits(b)


def _scale_buf(nch, count, pad=16):
    """K-major E8M0 tensor [nch + 1, roundup16(count) + pad] full of the canary; returns (full, view)."""
    ld = (count + 15) // 16 * 16 + pad
    full = torch.full((nch + 1, ld), CANARY_U8, dtype=torch.uint8, device="cuda")
    return full, full[:nch]


def _check_scale_canaries(full, nch, count):
    v = u8(full)
    mask = np.ones(v.shape, dtype=bool)
    mask[:nch, :count] = False
    assert np.all(v[mask] == CANARY_U8), "scale padding or guard row was written"


def _same(got, want, what):
    bad = np.flatnonzero(got.ravel() != want.ravel())
    assert bad.size == 0, f"{what}: {bad.size} of {got.size} differ, first at {bad[:5]}: " \
                          f"{got.ravel()[bad[:5]]} vs {want.ravel()[bad[:5]]}"


@pytest.mark.parametrize("R,C", [(256, 512), (384, 640), (128, 128)])
def test_mx_quant_rows_and_cols(R, C):
    need_gpu()
    x = _mx_input(R, C, seed=R + 2 * C)
    qr_full, qr = guarded(R, C, torch.uint8)
    sr_full, sr = _scale_buf(C // 32, R)
    qc_full, qc = guarded(C, R, torch.uint8)
    sc_full, sc = _scale_buf(R // 32, C)
    print(f"mx_quant R={R} C={C}", flush=True)
    bs.bs_mx_quant_1x32(x.cuda(), qr, sr, qc, sc)
    torch.cuda.synchronize()
    q_ref, s_ref = mx.quant_mx_rowwise(bits16(x))
    _same(u8(qr), q_ref, "row codes")
    _same(u8(sr).T[:R], s_ref, "row scales")
    qc_ref, sc_ref = mx.quant_mx_colwise(bits16(x))
    _same(u8(qc), qc_ref, "column codes")
    _same(u8(sc).T[:C], sc_ref, "column scales")
    check_canaries(qr_full, R, C)
    check_canaries(qc_full, C, R)
    _check_scale_canaries(sr_full, C // 32, R)
    _check_scale_canaries(sc_full, R // 32, C)

    # each output alone gives the same bytes
    qr2, sr2 = torch.empty_like(qr), torch.zeros_like(sr)
    bs.bs_mx_quant_1x32(x.cuda(), qr2, sr2)
    qc2, sc2 = torch.empty_like(qc), torch.zeros_like(sc)
    bs.bs_mx_quant_1x32(x.cuda(), None, None, qc2, sc2)
    torch.cuda.synchronize()
    assert torch.equal(qr2, qr) and torch.equal(sr2[:, :R], sr[:, :R])
    assert torch.equal(qc2, qc) and torch.equal(sc2[:, :C], sc[:, :C])


@pytest.mark.parametrize("R", [1, 77, 300])
def test_mx_quant_ragged_rows(R):
    need_gpu()
    C = 256
    x = _mx_input(R, C, seed=R + 5)
    qr_full, qr = guarded(R, C, torch.uint8)
    sr_full, sr = _scale_buf(C // 32, R)
    print(f"mx_quant ragged R={R}", flush=True)
    bs.bs_mx_quant_1x32(x.cuda(), qr, sr)
    torch.cuda.synchronize()
    q_ref, s_ref = mx.quant_mx_rowwise(bits16(x))
    _same(u8(qr), q_ref, "row codes")
    _same(u8(sr).T[:R], s_ref, "row scales")
    check_canaries(qr_full, R, C)
    _check_scale_canaries(sr_full, C // 32, R)


def test_mx_quant_every_scale_exponent():
    # one row per power of two from 2^-133 (subnormal) to 2^127, each row
    # block a ramp below it: every E8M0 byte the format can produce
    need_gpu()
    exps = np.arange(-133, 128)
    R, C = 384, 128
    rng = np.random.default_rng(7)
    vals = np.zeros((R, C), dtype=np.float64)
    for r, e in enumerate(exps):
        vals[r] = np.ldexp(rng.uniform(-1.99, 1.99, C), int(e))
    x = torch.from_numpy(vals.astype(np.float32)).to(torch.bfloat16)
    q = torch.empty((R, C), dtype=torch.uint8, device="cuda")
    s = bs.empty_mx_scales(C // 32, R, "cuda")
    qc = torch.empty((C, R), dtype=torch.uint8, device="cuda")
    sc = bs.empty_mx_scales(R // 32, C, "cuda")
    print("mx_quant every exponent", flush=True)
    bs.bs_mx_quant_1x32(x.cuda(), q, s, qc, sc)
    torch.cuda.synchronize()
    q_ref, s_ref = mx.quant_mx_rowwise(bits16(x))
    _same(u8(q), q_ref, "row codes")
    _same(u8(s).T[:R], s_ref, "row scales")
    qc_ref, sc_ref = mx.quant_mx_colwise(bits16(x))
    _same(u8(qc), qc_ref, "column codes")
    _same(u8(sc).T[:C], sc_ref, "column scales")


@pytest.mark.parametrize("R,C", [(8192, 4096), (8192, 16384)])
def test_mx_quant_full_size_sampled(R, C):
    # the bench's activation shape (a persistent grid) and one of 8192 tiles
    # (one workgroup per tile); rows and 32-row slabs checked one by one
    need_gpu()
    x = inputs.bf16_normal((R, C), 1.0, 11, device="cuda")
    q = torch.empty((R, C), dtype=torch.uint8, device="cuda")
    s = bs.empty_mx_scales(C // 32, R, "cuda")
    qc = torch.empty((C, R), dtype=torch.uint8, device="cuda")
    sc = bs.empty_mx_scales(R // 32, C, "cuda")
    print(f"mx_quant {R} x {C}", flush=True)
    bs.bs_mx_quant_1x32(x, q, s, qc, sc)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    rows = np.sort(rng.choice(R, 24, replace=False))
    xr = bits16(x[torch.from_numpy(rows).cuda()])
    q_ref, s_ref = mx.quant_mx_rowwise(xr)
    _same(u8(q[torch.from_numpy(rows).cuda()]), q_ref, "row codes")
    _same(u8(s).T[rows], s_ref, "row scales")
    for slab in rng.choice(R // 32, 4, replace=False):
        r0 = int(slab) * 32
        qc_ref, sc_ref = mx.quant_mx_colwise(bits16(x[r0:r0 + 32]))
        _same(u8(qc[:, r0:r0 + 32]), qc_ref, "column codes")
        _same(u8(sc[slab]), sc_ref[:, 0], "column scales")


# ---- GEMM ----

def _to_gpu_mx_scales(s_logical, pad=16):
    """Logical [rows, K/32] E8M0 bytes -> K-major GPU tensor [K/32, roundup16(rows) + pad];
    the padding holds a NaN scale (255) that must never be used."""
    rows, nch = s_logical.shape
    ld = (rows + 15) // 16 * 16 + pad
    buf = np.full((nch, ld), 255, dtype=np.uint8)
    buf[:, :rows] = s_logical.T
    return torch.from_numpy(buf).cuda()


def _operand(rows, K, sigma, seed):
    return mx.quant_mx_rowwise(bits16(inputs.bf16_normal((rows, K), sigma, seed)))


def _normal_codes(rows, K, rng, sigma=64.0):
    """E4M3 codes of N(0, sigma) values (saturated at 448), drawn directly.
    (Uniformly random bytes are heavy-tailed: a dot product can then come
    within a factor of two of ||a|| ||b||, where a bf16 output's own rounding
    exceeds the bound.)"""
    return e4m3.encode(np.clip(rng.standard_normal((rows, K)) * sigma, -448, 448).astype(np.float32))


def _check(d_gpu, qa, sa, qb, sb, exact=False):
    a = mx.dequant_mx(qa, sa)
    b = mx.dequant_mx(qb, sb)
    ref = a @ b.T
    d = d_gpu.float().cpu().numpy().astype(np.float64)
    if exact:
        bad = np.argwhere(d != ref)
        assert bad.size == 0, f"{len(bad)} inexact elements, first {bad[0]}: {d[tuple(bad[0])]} vs {ref[tuple(bad[0])]}"
    else:
        ok, worst = gemm.check_close(d, ref, a, b)
        assert ok, f"worst |err| / bound = {worst}"


@pytest.mark.parametrize("M,N,K", [(256, 256, 512), (384, 640, 768), (300, 384, 640), (512, 128, 1024),
                                   (64, 256, 128), (301, 256, 256)])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_mx_scaled_mm(M, N, K, out_dtype):
    need_gpu()
    qa, sa = _operand(M, K, 1.0, seed=M + K)
    qb, sb = _operand(N, K, 0.02, seed=N + 3 * K)
    full, out = guarded(M, N, out_dtype)
    print(f"mx_scaled_mm M={M} N={N} K={K} {out_dtype}", flush=True)
    bs.bs_mx_scaled_mm(torch.from_numpy(qa).cuda(), _to_gpu_mx_scales(sa), torch.from_numpy(qb).cuda(),
                       _to_gpu_mx_scales(sb), out=out)
    torch.cuda.synchronize()
    _check(out, qa, sa, qb, sb)
    check_canaries(full, M, N)


def test_mx_scaled_mm_exact_small_integers():
    # small integer codes under scales 2^-2 .. 2^2 that differ per row and per
    # 32-block: every partial sum is a multiple of 2^-4 below 2^19, exact in
    # fp32, so the product must match bit for bit -- a scale applied to the
    # wrong row, column or K block shows up as an exact mismatch
    need_gpu()
    M, N, K = 384, 512, 768
    rng = np.random.default_rng(5)
    ints = np.arange(-8, 9, dtype=np.float32)
    qa = e4m3.encode(rng.choice(ints, (M, K)).astype(np.float32))
    qb = e4m3.encode(rng.choice(ints, (N, K)).astype(np.float32))
    sa = rng.integers(125, 130, (M, K // 32)).astype(np.uint8)
    sb = rng.integers(125, 130, (N, K // 32)).astype(np.uint8)
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    print("mx_scaled_mm exact", flush=True)
    bs.bs_mx_scaled_mm(torch.from_numpy(qa).cuda(), _to_gpu_mx_scales(sa), torch.from_numpy(qb).cuda(),
                       _to_gpu_mx_scales(sb), out=out)
    torch.cuda.synchronize()
    _check(out, qa, sa, qb, sb, exact=True)


def test_mx_scaled_mm_wide_scale_range():
    # each row of A has its own scale byte from 40 to 210 (2^-87 .. 2^83),
    # each row of B one from 117 to 137, jittered by +-2 per 32-block: every
    # output's magnitude follows its row's and column's bytes, and every
    # product stays a normal float32
    need_gpu()
    M, N, K = 384, 256, 512
    rng = np.random.default_rng(9)
    qa = rng.integers(0, 256, (M, K)).astype(np.uint8)
    qb = rng.integers(0, 256, (N, K)).astype(np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0x38   # no NaN codes
    qb[(qb & 0x7F) == 0x7F] = 0x38
    jit = lambda rows: rng.integers(-2, 3, (rows, K // 32))
    sa = (np.linspace(42, 208, M).round().astype(np.int64)[:, None] + jit(M)).astype(np.uint8)
    sb = (rng.integers(119, 136, N)[:, None] + jit(N)).astype(np.uint8)
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    print("mx_scaled_mm wide scale range", flush=True)
    bs.bs_mx_scaled_mm(torch.from_numpy(qa).cuda(), _to_gpu_mx_scales(sa), torch.from_numpy(qb).cuda(),
                       _to_gpu_mx_scales(sb), out=out)
    torch.cuda.synchronize()
    _check(out, qa, sa, qb, sb)


def test_mx_scaled_mm_empty_k_writes_zeros():
    need_gpu()
    M, N = 128, 256
    a = torch.empty((M, 16), dtype=torch.uint8, device="cuda")[:, :0]   # lda 16, K 0
    b = torch.empty((N, 16), dtype=torch.uint8, device="cuda")[:, :0]
    s = torch.empty((1, 256), dtype=torch.uint8, device="cuda")[:0]     # non-NULL, zero rows
    out = torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")
    print("mx_scaled_mm K=0", flush=True)
    bs.bs_mx_scaled_mm(a, s, b, s, out=out)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0


def test_mx_scaled_mm_full_size_sampled():
    # the dense bench shape, in the bench's launch configuration; codes and
    # scale bytes drawn directly, sampled rows checked against the oracle
    need_gpu()
    M, N, K = 8192, 4096, 4096
    rng = np.random.default_rng(21)
    qa = _normal_codes(M, K, rng)
    qb = _normal_codes(N, K, rng)
    sa = rng.integers(125, 131, (M, K // 32)).astype(np.uint8)   # bf16 output: scales within 2^5
    sb = rng.integers(125, 131, (N, K // 32)).astype(np.uint8)
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    print("mx_scaled_mm 8192 x 4096 x 4096", flush=True)
    bs.bs_mx_scaled_mm(torch.from_numpy(qa).cuda(), _to_gpu_mx_scales(sa), torch.from_numpy(qb).cuda(),
                       _to_gpu_mx_scales(sb), out=out)
    torch.cuda.synchronize()
    rows = np.sort(rng.choice(M, 16, replace=False))
    a = mx.dequant_mx(qa[rows], sa[rows])
    b = mx.dequant_mx(qb, sb)
    ref = a @ b.T
    d = out[torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
    ok, worst = gemm.check_close(d, ref, a, b)
    assert ok, f"worst |err| / bound = {worst}"


def test_mx_persistent_many_tiles():
    # 18 x 16 = 288 tiles over at most 256 workgroups, ragged last tile row:
    # workgroups walk several tiles, prefetching across tile boundaries.
    # float32 output: with per-block scales spread over 2^15 a row is
    # dominated by a few blocks, a product can come close to ||a|| ||b||, and
    # a bf16 output's own rounding (up to 2^-8 |d|) would exceed the bound
    need_gpu()
    M, N, K = 4452, 4096, 256
    rng = np.random.default_rng(31)
    qa = _normal_codes(M, K, rng)
    qb = _normal_codes(N, K, rng)
    sa = rng.integers(120, 135, (M, K // 32)).astype(np.uint8)
    sb = rng.integers(120, 135, (N, K // 32)).astype(np.uint8)
    full, out = guarded(M, N, torch.float32)
    print("mx_scaled_mm persistent 4452 x 4096 x 256", flush=True)
    bs.bs_mx_scaled_mm(torch.from_numpy(qa).cuda(), _to_gpu_mx_scales(sa), torch.from_numpy(qb).cuda(),
                       _to_gpu_mx_scales(sb), out=out)
    torch.cuda.synchronize()
    _check(out, qa, sa, qb, sb)
    check_canaries(full, M, N)


# ---- grouped (MoE) ----

def _expert_scales(sb_list, interleaved):
    """Per-expert logical scales [N, K/32] -> a [G, K/32, >= N] uint8 GPU view:
    stacked tensors, or one [K/32, G*N] matrix viewed per expert."""
    G = len(sb_list)
    N, nch = sb_list[0].shape
    if interleaved:
        whole = _to_gpu_mx_scales(np.concatenate(sb_list, axis=0))
        return torch.as_strided(whole, (G, nch, N), (N, whole.stride(0), 1))
    return torch.stack([_to_gpu_mx_scales(s) for s in sb_list])


@pytest.mark.parametrize("sizes,interleaved", [((128, 0, 256), False), ((200, 56, 300), True),
                                               ((0, 0, 512), False), ((37, 0, 219, 100), True),
                                               ((1000, 3000, 17, 500), False)])
def test_mx_group_m(sizes, interleaved):
    # group starts at any row (37, 256, 356, 1017, ...): the A scale bytes of
    # a tile are copied from the 16-byte boundary below its first row; M = 4517
    # ends the scale rows inside a dword
    need_gpu()
    G, N, K = len(sizes), 384, 640
    ends = np.cumsum(sizes).astype(np.int32)
    M = int(ends[-1])
    qa, sa = _operand(M, K, 1.0, seed=M + G)
    ops = [_operand(N, K, 0.02, seed=G + 100 + g) for g in range(G)]
    qb = torch.from_numpy(np.stack([q for q, _ in ops])).cuda()
    sb = _expert_scales([s for _, s in ops], interleaved)
    full, out = guarded(M, N, torch.bfloat16)
    print(f"mx group_m sizes={sizes} interleaved={interleaved}", flush=True)
    bs.bs_mx_grouped_scaled_mm(bs.BS_GROUP_M, torch.from_numpy(ends).cuda(), torch.from_numpy(qa).cuda(),
                               _to_gpu_mx_scales(sa), qb, sb, out=out)
    torch.cuda.synchronize()
    d = out.float().cpu().numpy().astype(np.float64)
    start = 0
    for g, e in enumerate(ends):
        if e > start:
            a = mx.dequant_mx(qa[start:e], sa[start:e])
            b = mx.dequant_mx(*ops[g])
            ok, worst = gemm.check_close(d[start:e], a @ b.T, a, b)
            assert ok, f"group {g}: worst {worst}"
        start = e
    check_canaries(full, M, N)


@pytest.mark.parametrize("sizes", [(256, 0, 128), (128, 128, 128, 128), (0, 384)])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_mx_group_k(sizes, out_dtype):
    need_gpu()
    G, M, N = len(sizes), 256, 384
    ends = np.cumsum(sizes).astype(np.int32)
    T = int(ends[-1])
    qa, sa = _operand(M, T, 0.01, seed=T + 1)   # grad_out^T [M, T]
    qb, sb = _operand(N, T, 1.0, seed=T + 2)    # x^T [N, T]
    out_full = torch.full((G + 1, M, N), 5.0, dtype=out_dtype, device="cuda")
    out = out_full[:G]
    print(f"mx group_k sizes={sizes} {out_dtype}", flush=True)
    bs.bs_mx_grouped_scaled_mm(bs.BS_GROUP_K, torch.from_numpy(ends).cuda(), torch.from_numpy(qa).cuda(),
                               _to_gpu_mx_scales(sa), torch.from_numpy(qb).cuda(), _to_gpu_mx_scales(sb), out=out)
    torch.cuda.synchronize()
    d = out.float().cpu().numpy().astype(np.float64)
    start = 0
    for g, e in enumerate(ends):
        if e == start:
            assert np.all(d[g] == 0), f"empty group {g} must be zeros"
        else:
            a = mx.dequant_mx(qa[:, start:e], sa[:, start // 32:e // 32])
            b = mx.dequant_mx(qb[:, start:e], sb[:, start // 32:e // 32])
            ok, worst = gemm.check_close(d[g], a @ b.T, a, b)
            assert ok, f"group {g}: worst {worst}"
        start = e
    assert torch.all(out_full[G] == 5.0)


def test_mx_group_m_equals_dense_per_group():
    # bit-for-bit: a group's rows of the grouped product equal the dense MX
    # product of those rows with the group's expert (same kernel arithmetic)
    need_gpu()
    sizes = (300, 212, 500)
    G, N, K = 3, 256, 512
    ends = np.cumsum(sizes).astype(np.int32)
    M = int(ends[-1])
    qa, sa = _operand(M, K, 1.0, seed=5)
    ops = [_operand(N, K, 0.05, seed=50 + g) for g in range(G)]
    qb = torch.from_numpy(np.stack([q for q, _ in ops])).cuda()
    sb = _expert_scales([s for _, s in ops], False)
    print("mx group_m vs dense", flush=True)
    d = bs.bs_mx_grouped_scaled_mm(bs.BS_GROUP_M, torch.from_numpy(ends).cuda(), torch.from_numpy(qa).cuda(),
                                   _to_gpu_mx_scales(sa), qb, sb, out_dtype=torch.float32)
    start = 0
    for g, e in enumerate(ends):
        dg = bs.bs_mx_scaled_mm(torch.from_numpy(np.ascontiguousarray(qa[start:e])).cuda(),
                                _to_gpu_mx_scales(sa[start:e]), qb[g], _to_gpu_mx_scales(ops[g][1]),
                                out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(d[start:e], dg), f"group {g}"
        start = e


@pytest.mark.parametrize("G", [64, 70])
def test_mx_group_m_many_groups(G):
    # the largest group count ordered in XCD slices (64) and beyond (70)
    need_gpu()
    rng = np.random.default_rng(G + 7)
    sizes = rng.choice([0, 1, 37, 128, 300], G)
    ends = np.cumsum(sizes).astype(np.int32)
    M, N, K = int(ends[-1]), 256, 256
    qa, sa = _operand(M, K, 1.0, seed=G)
    ops = [_operand(N, K, 0.02, seed=1000 + g) for g in range(G)]
    qb = torch.from_numpy(np.stack([q for q, _ in ops])).cuda()
    sb = _expert_scales([s for _, s in ops], True)
    full, out = guarded(M, N, torch.bfloat16)
    print(f"mx group_m G={G} M={M}", flush=True)
    bs.bs_mx_grouped_scaled_mm(bs.BS_GROUP_M, torch.from_numpy(ends).cuda(), torch.from_numpy(qa).cuda(),
                               _to_gpu_mx_scales(sa), qb, sb, out=out)
    torch.cuda.synchronize()
    d = out.float().cpu().numpy().astype(np.float64)
    start = 0
    for g, e in enumerate(ends):
        if e > start:
            a = mx.dequant_mx(qa[start:e], sa[start:e])
            b = mx.dequant_mx(*ops[g])
            ok, worst = gemm.check_close(d[start:e], a @ b.T, a, b)
            assert ok, f"group {g}: worst {worst}"
        start = e
    check_canaries(full, M, N)
