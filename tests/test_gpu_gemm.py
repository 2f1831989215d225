"""GPU parity of the scaled GEMMs (dense and grouped) against the CPU oracle.

Operand codes and scales are made on the CPU by the oracle's quantizer (or
drawn directly), copied to the GPU in the library's layout, and the GPU
result is compared element by element with the oracle's float64 product
within 2e-3 * ||a_m|| * ||b_n||; exact-arithmetic cases must match bit for
bit.  Calls go through the C ABI (thin binding)."""

import numpy as np
import pytest
import torch

import blockwise_scaled_fp8_bs_amd as bs
from blockwise_scaled_fp8_bs_amd import inputs
from oracle import e4m3, gemm, quant
from gpu_support import bits16, check_canaries, guarded, need_gpu

pytestmark = pytest.mark.gpu


def to_gpu_scales(s_logical, pad=4):
    """Logical [rows, nkb] scales -> K-major GPU tensor [nkb, roundup4(rows) + pad]."""
    rows, nkb = s_logical.shape
    ld = (rows + 3) // 4 * 4 + pad
    buf = np.full((nkb, ld), np.nan, dtype=np.float32)
    buf[:, :rows] = s_logical.T
    return torch.from_numpy(buf).cuda()


def operand_1x128(rows, K, sigma, seed):
    x = inputs.bf16_normal((rows, K), sigma, seed)
    return quant.quant_1x128_rowwise(bits16(x))


def operand_128x128(rows, K, sigma, seed):
    x = inputs.bf16_normal((rows, K), sigma, seed)
    return quant.quant_128x128(bits16(x))


def check_result(d_gpu, qa, sa, qb, sb, b_row_block, exact=False):
    a = gemm.dequant(qa, sa, 1)
    b = gemm.dequant(qb, sb, b_row_block)
    ref = a @ b.T
    d = d_gpu.float().cpu().numpy().astype(np.float64)
    if exact:
        bad = np.argwhere(d != ref)
        assert bad.size == 0, f"{len(bad)} inexact elements, first {bad[0]}: {d[tuple(bad[0])]} vs {ref[tuple(bad[0])]}"
    else:
        ok, worst = gemm.check_close(d, ref, a, b)
        assert ok, f"worst |err| / bound = {worst}"
    return ref


@pytest.mark.parametrize("M,N,K", [(256, 256, 512), (384, 640, 768), (300, 384, 512), (512, 128, 1024),
                                   (64, 256, 128)])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_scaled_mm_128x128(M, N, K, out_dtype):
    need_gpu()
    qa, sa = operand_1x128(M, K, 1.0, seed=M + K)
    qb, sb = operand_128x128(N, K, 0.02, seed=N + 3 * K)
    full, out = guarded(M, N, out_dtype)
    print(f"scaled_mm 128x128 M={M} N={N} K={K} {out_dtype}", flush=True)
    bs.bs_scaled_mm(torch.from_numpy(qa).cuda(), to_gpu_scales(sa), torch.from_numpy(qb).cuda(),
                    to_gpu_scales(sb), bs.BS_SCALE_128X128, out=out)
    torch.cuda.synchronize()
    check_result(out, qa, sa, qb, sb, 128)
    check_canaries(full, M, N)


@pytest.mark.parametrize("M,N,K", [(256, 384, 640), (384, 256, 1024), (128, 128, 128), (200, 512, 256)])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_scaled_mm_1x128(M, N, K, out_dtype):
    need_gpu()
    qa, sa = operand_1x128(M, K, 0.01, seed=M + 5 * K)
    qb, sb = operand_1x128(N, K, 1.0, seed=N + 7 * K)
    full, out = guarded(M, N, out_dtype)
    print(f"scaled_mm 1x128 M={M} N={N} K={K} {out_dtype}", flush=True)
    bs.bs_scaled_mm(torch.from_numpy(qa).cuda(), to_gpu_scales(sa), torch.from_numpy(qb).cuda(),
                    to_gpu_scales(sb), bs.BS_SCALE_1X128, out=out)
    torch.cuda.synchronize()
    check_result(out, qa, sa, qb, sb, 1)
    check_canaries(full, M, N)


SMALL_INT_CODES = np.array([0xC4, 0xC0, 0xB8, 0x00, 0x38, 0x40, 0x44], dtype=np.uint8)  # -3..3


@pytest.mark.parametrize("kind", [bs.BS_SCALE_128X128, bs.BS_SCALE_1X128])
def test_scaled_mm_exact_small_integers(kind):
    """Integer codes |v| <= 3 and scales 2^[-2, 2]: every partial sum is exact in
    fp32, so the fp32 result must equal the float64 oracle bit for bit."""
    need_gpu()
    rng = np.random.default_rng(3)
    M, N, K = 384, 256, 4096
    qa = rng.choice(SMALL_INT_CODES, size=(M, K))
    qb = rng.choice(SMALL_INT_CODES, size=(N, K))
    sa = np.exp2(rng.integers(-2, 3, size=(M, K // 128))).astype(np.float32)
    rb = 128 if kind == bs.BS_SCALE_128X128 else 1
    sb = np.exp2(rng.integers(-2, 3, size=(N // rb, K // 128))).astype(np.float32)
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    bs.bs_scaled_mm(torch.from_numpy(qa).cuda(), to_gpu_scales(sa), torch.from_numpy(qb).cuda(),
                    to_gpu_scales(sb), kind, out=out)
    torch.cuda.synchronize()
    check_result(out, qa, sa, qb, sb, rb, exact=True)


def test_scaled_mm_identity_b():
    need_gpu()
    M, K = 256, 512
    qa, sa = operand_1x128(M, K, 1.0, seed=11)
    qb = np.zeros((K, K), dtype=np.uint8)
    qb[np.arange(K), np.arange(K)] = 0x38
    sb = np.ones((K // 128, K // 128), dtype=np.float32)
    out = torch.empty((M, K), dtype=torch.float32, device="cuda")
    bs.bs_scaled_mm(torch.from_numpy(qa).cuda(), to_gpu_scales(sa), torch.from_numpy(qb).cuda(),
                    to_gpu_scales(sb), bs.BS_SCALE_128X128, out=out)
    torch.cuda.synchronize()
    a = gemm.dequant(qa, sa, 1)
    assert np.array_equal(out.cpu().numpy().astype(np.float64), a.astype(np.float32).astype(np.float64))


def test_scaled_mm_empty_k_writes_zeros():
    need_gpu()
    M, N = 256, 256
    a = torch.empty((M, 16), dtype=torch.uint8, device="cuda")[:, :0]
    b = torch.empty((N, 16), dtype=torch.uint8, device="cuda")[:, :0]
    sa = torch.empty((1, 256), dtype=torch.float32, device="cuda")[:0]  # non-NULL, zero rows
    sb = torch.empty((1, 4), dtype=torch.float32, device="cuda")[:0]
    out = torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")
    bs.bs_scaled_mm(a, sa, b, sb, bs.BS_SCALE_128X128, out=out)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0


def test_b_kinds_agree_on_expanded_scales():
    need_gpu()
    M, N, K = 256, 256, 384
    qa, sa = operand_1x128(M, K, 1.0, seed=21)
    qb, sb128 = operand_128x128(N, K, 0.02, seed=22)
    sb1 = np.repeat(sb128, 128, axis=0)
    ga, gsa, gb = torch.from_numpy(qa).cuda(), to_gpu_scales(sa), torch.from_numpy(qb).cuda()
    d1 = bs.bs_scaled_mm(ga, gsa, gb, to_gpu_scales(sb128), bs.BS_SCALE_128X128, out_dtype=torch.float32)
    d2 = bs.bs_scaled_mm(ga, gsa, gb, to_gpu_scales(sb1), bs.BS_SCALE_1X128, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(d1, d2)


# ----------------------------------------------------------------------------
# grouped
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("sizes", [(128, 0, 256), (256, 384, 128, 0), (0, 0, 512), (200, 56, 300)])
def test_group_m(sizes):
    _group_m_case(sizes, 640)


# one and three K blocks: the next block's copies are shared out over MFMAs
# that a one-block tile never reaches, and a three-block tile only in its
# first two blocks
@pytest.mark.parametrize("K", [128, 384])
def test_group_m_short_k(K):
    _group_m_case((256, 128, 384), K)


def _group_m_case(sizes, K):
    need_gpu()
    G, N = len(sizes), 384
    ends = np.cumsum(sizes).astype(np.int32)
    M = int(ends[-1])
    qa, sa = operand_1x128(M, K, 1.0, seed=M + G)
    w = inputs.bf16_normal((G * N, K), 0.02, seed=G + 100)
    qw, sw = quant.quant_128x128(bits16(w))  # W as one [G*N, K] matrix
    # scales K-major [K/128][ld >= G*N/128]; expert g's view starts at column g*N/128
    sw_gpu = to_gpu_scales(sw)
    sb_view = torch.as_strided(sw_gpu, (G, K // 128, N // 128), (N // 128, sw_gpu.stride(0), 1))
    qb = torch.from_numpy(qw).cuda().view(G, N, K)
    full, out = guarded(M, N, torch.bfloat16)
    print(f"group_m sizes={sizes} K={K}", flush=True)
    bs.bs_grouped_scaled_mm(bs.BS_GROUP_M, torch.from_numpy(ends).cuda(), torch.from_numpy(qa).cuda(),
                            to_gpu_scales(sa), qb, sb_view, bs.BS_SCALE_128X128, out=out)
    torch.cuda.synchronize()
    d = out.float().cpu().numpy().astype(np.float64)
    aligned = all(sz % 128 == 0 for sz in sizes)
    ref = gemm.grouped_mm_group_m(list(ends), qa, sa, qw.reshape(G, N, K),
                                  sw.reshape(G, N // 128, K // 128), 128) if aligned else None
    start = 0
    for g, e in enumerate(ends):
        if e > start:
            a = gemm.dequant(qa[start:e], sa[start:e], 1)
            b = gemm.dequant(qw[g * N:(g + 1) * N], sw[g * N // 128:(g + 1) * N // 128], 128)
            want = a @ b.T if ref is None else ref[start:e]
            ok, worst = gemm.check_close(d[start:e], want, a, b)
            assert ok, f"group {g}: worst {worst}"
        start = e
    check_canaries(full, M, N)


@pytest.mark.parametrize("sizes", [(256, 0, 128), (128, 128, 128, 128), (0, 384)])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_group_k(sizes, out_dtype):
    need_gpu()
    G, M, N = len(sizes), 256, 384
    ends = np.cumsum(sizes).astype(np.int32)
    T = int(ends[-1])
    qa, sa = operand_1x128(M, T, 0.01, seed=T + 1)   # grad_out^T [M, T]
    qb, sb = operand_1x128(N, T, 1.0, seed=T + 2)    # A^T [N, T]
    out_full = torch.full((G + 1, M, N), 5.0, dtype=out_dtype, device="cuda")
    out = out_full[:G]
    print(f"group_k sizes={sizes} {out_dtype}", flush=True)
    bs.bs_grouped_scaled_mm(bs.BS_GROUP_K, torch.from_numpy(ends).cuda(), torch.from_numpy(qa).cuda(),
                            to_gpu_scales(sa), torch.from_numpy(qb).cuda(), to_gpu_scales(sb),
                            bs.BS_SCALE_1X128, out=out)
    torch.cuda.synchronize()
    ref = gemm.grouped_mm_group_k(list(ends), qa, sa, qb, sb)
    d = out.float().cpu().numpy().astype(np.float64)
    start = 0
    for g, e in enumerate(ends):
        if e == start:
            assert np.all(d[g] == 0), f"empty group {g} must be zeros"
        else:
            a = gemm.dequant(qa[:, start:e], sa[:, start // 128:e // 128], 1)
            b = gemm.dequant(qb[:, start:e], sb[:, start // 128:e // 128], 1)
            ok, worst = gemm.check_close(d[g], ref[g], a, b)
            assert ok, f"group {g}: worst {worst}"
        start = e
    assert torch.all(out_full[G] == 5.0)


# ----------------------------------------------------------------------------
# more tiles than workgroups: every workgroup walks several tiles, loading the
# next tile's first K block during the current tile's last one
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("kind", [bs.BS_SCALE_128X128, bs.BS_SCALE_1X128])
def test_persistent_dense_many_tiles(kind):
    need_gpu()
    M, N, K = 4452, 4096, 256          # 18 x 16 = 288 tiles, ragged last tile row
    qa, sa = operand_1x128(M, K, 1.0, seed=11)
    if kind == bs.BS_SCALE_128X128:
        qb, sb = operand_128x128(N, K, 0.02, seed=12)
    else:
        qb, sb = operand_1x128(N, K, 0.02, seed=12)
    full, out = guarded(M, N, torch.bfloat16)
    print(f"persistent dense {M}x{N}x{K} kind={kind}", flush=True)
    bs.bs_scaled_mm(torch.from_numpy(qa).cuda(), to_gpu_scales(sa), torch.from_numpy(qb).cuda(),
                    to_gpu_scales(sb), kind, out=out)
    torch.cuda.synchronize()
    check_result(out, qa, sa, qb, sb, 128 if kind == bs.BS_SCALE_128X128 else 1)
    check_canaries(full, M, N)


def test_persistent_group_m_many_tiles():
    need_gpu()
    sizes = (700, 0, 1300, 128, 0, 900, 601, 371)   # ragged and empty groups
    G, N, K = len(sizes), 4096, 256                  # (tile rows = 21) x 16 = 336 tiles
    ends = np.cumsum(sizes).astype(np.int32)
    M = int(ends[-1])
    qa, sa = operand_1x128(M, K, 1.0, seed=21)
    w = inputs.bf16_normal((G * N, K), 0.02, seed=22)
    qw, sw = quant.quant_128x128(bits16(w))
    sw_gpu = to_gpu_scales(sw)
    sb_view = torch.as_strided(sw_gpu, (G, K // 128, N // 128), (N // 128, sw_gpu.stride(0), 1))
    full, out = guarded(M, N, torch.bfloat16)
    print(f"persistent group_m sizes={sizes}", flush=True)
    bs.bs_grouped_scaled_mm(bs.BS_GROUP_M, torch.from_numpy(ends).cuda(), torch.from_numpy(qa).cuda(),
                            to_gpu_scales(sa), torch.from_numpy(qw).cuda().view(G, N, K), sb_view,
                            bs.BS_SCALE_128X128, out=out)
    torch.cuda.synchronize()
    d = out.float().cpu().numpy().astype(np.float64)
    start = 0
    for g, e in enumerate(ends):
        if e > start:
            a = gemm.dequant(qa[start:e], sa[start:e], 1)
            b = gemm.dequant(qw[g * N:(g + 1) * N], sw[g * N // 128:(g + 1) * N // 128], 128)
            ok, worst = gemm.check_close(d[start:e], a @ b.T, a, b)
            assert ok, f"group {g}: worst {worst}"
        start = e
    check_canaries(full, M, N)


@pytest.mark.parametrize("kind", [bs.BS_SCALE_128X128, bs.BS_SCALE_1X128])
def test_persistent_dense_exact_many_k_blocks(kind):
    """More tiles than workgroups, 8 K blocks per tile, ragged last tile row,
    small-integer codes and power-of-two scales (every partial sum exact in
    fp32): a K block read from the wrong LDS stage, a copy issued for the
    wrong block or tile, or a scale of the wrong block shows as a bit
    mismatch against the float64 oracle."""
    need_gpu()
    rng = np.random.default_rng(5)
    M, N, K = 4452, 4096, 1024          # 18 x 16 = 288 tiles
    qa = rng.choice(SMALL_INT_CODES, size=(M, K))
    qb = rng.choice(SMALL_INT_CODES, size=(N, K))
    sa = np.exp2(rng.integers(-2, 3, size=(M, K // 128))).astype(np.float32)
    rb = 128 if kind == bs.BS_SCALE_128X128 else 1
    sb = np.exp2(rng.integers(-2, 3, size=(N // rb, K // 128))).astype(np.float32)
    full, out = guarded(M, N, torch.float32)
    print(f"persistent exact dense {M}x{N}x{K} kind={kind}", flush=True)
    bs.bs_scaled_mm(torch.from_numpy(qa).cuda(), to_gpu_scales(sa), torch.from_numpy(qb).cuda(),
                    to_gpu_scales(sb), kind, out=out)
    torch.cuda.synchronize()
    check_result(out, qa, sa, qb, sb, rb, exact=True)
    check_canaries(full, M, N)


def test_persistent_group_m_exact_many_k_blocks():
    """GROUP_M with ragged and empty groups, more tiles than workgroups and 8 K
    blocks per tile, on exact small-integer arithmetic: every group's rows
    must equal the float64 oracle bit for bit."""
    need_gpu()
    rng = np.random.default_rng(6)
    sizes = (700, 0, 1300, 128, 0, 900, 601, 371)
    G, N, K = len(sizes), 4096, 1024                 # 21 tile rows x 16 = 336 tiles
    ends = np.cumsum(sizes).astype(np.int32)
    M = int(ends[-1])
    qa = rng.choice(SMALL_INT_CODES, size=(M, K))
    sa = np.exp2(rng.integers(-2, 3, size=(M, K // 128))).astype(np.float32)
    qw = rng.choice(SMALL_INT_CODES, size=(G * N, K))
    sw = np.exp2(rng.integers(-2, 3, size=(G * N // 128, K // 128))).astype(np.float32)
    sw_gpu = to_gpu_scales(sw)
    sb_view = torch.as_strided(sw_gpu, (G, K // 128, N // 128), (N // 128, sw_gpu.stride(0), 1))
    full, out = guarded(M, N, torch.float32)
    print(f"persistent exact group_m sizes={sizes} K={K}", flush=True)
    bs.bs_grouped_scaled_mm(bs.BS_GROUP_M, torch.from_numpy(ends).cuda(), torch.from_numpy(qa).cuda(),
                            to_gpu_scales(sa), torch.from_numpy(qw).cuda().view(G, N, K), sb_view,
                            bs.BS_SCALE_128X128, out=out)
    torch.cuda.synchronize()
    d = out.cpu().numpy().astype(np.float64)
    start = 0
    for g, e in enumerate(ends):
        if e > start:
            a = gemm.dequant(qa[start:e], sa[start:e], 1)
            b = gemm.dequant(qw[g * N:(g + 1) * N], sw[g * N // 128:(g + 1) * N // 128], 128)
            bad = np.argwhere(d[start:e] != a @ b.T)
            assert bad.size == 0, f"group {g}: {len(bad)} inexact elements, first {bad[0]}"
        start = e
    check_canaries(full, M, N)


def test_persistent_group_k_many_tiles():
    need_gpu()
    # 20 groups of 16 tiles each (320 tiles); empty groups sit between
    # non-empty ones, so workgroups pass through tiles with no K blocks
    sizes = (256, 0, 128, 0, 0, 384, 128, 0, 256, 128, 0, 128, 0, 0, 256, 128, 0, 128, 0, 256)
    G, M, N = len(sizes), 1024, 1024
    ends = np.cumsum(sizes).astype(np.int32)
    T = int(ends[-1])
    qa, sa = operand_1x128(M, T, 0.01, seed=31)
    qb, sb = operand_1x128(N, T, 1.0, seed=32)
    out_full = torch.full((G + 1, M, N), 5.0, dtype=torch.float32, device="cuda")
    out = out_full[:G]
    print(f"persistent group_k G={G}", flush=True)
    bs.bs_grouped_scaled_mm(bs.BS_GROUP_K, torch.from_numpy(ends).cuda(), torch.from_numpy(qa).cuda(),
                            to_gpu_scales(sa), torch.from_numpy(qb).cuda(), to_gpu_scales(sb),
                            bs.BS_SCALE_1X128, out=out)
    torch.cuda.synchronize()
    d = out.cpu().numpy().astype(np.float64)
    start = 0
    for g, e in enumerate(ends):
        if e == start:
            assert np.all(d[g] == 0), f"empty group {g} must be zeros"
        else:
            a = gemm.dequant(qa[:, start:e], sa[:, start // 128:e // 128], 1)
            b = gemm.dequant(qb[:, start:e], sb[:, start // 128:e // 128], 1)
            ok, worst = gemm.check_close(d[g], a @ b.T, a, b)
            assert ok, f"group {g}: worst {worst}"
        start = e
    assert torch.all(out_full[G] == 5.0)


def test_persistent_group_k_exact_many_k_blocks():
    """GROUP_K with an empty group, more tiles than workgroups and 5 to 15 K
    blocks per group, on exact small-integer arithmetic (codes |v| <= 3,
    scales 2^[-2, 2]: every partial sum, at most 2^19, is exact in fp32):
    the wgrad's copies, issued in two halves after the issuing group's first
    MFMAs, must put every K block of every group in the right stage; each
    group's output equals the float64 oracle bit for bit."""
    need_gpu()
    rng = np.random.default_rng(8)
    sizes = (1024, 0, 1920, 640, 1408)
    G, M, N = len(sizes), 2304, 2048                   # 9 x 8 tiles per group, 288 in all
    ends = np.cumsum(sizes).astype(np.int32)
    T = int(ends[-1])
    qa = rng.choice(SMALL_INT_CODES, size=(M, T))
    qb = rng.choice(SMALL_INT_CODES, size=(N, T))
    sa = np.exp2(rng.integers(-2, 3, size=(M, T // 128))).astype(np.float32)
    sb = np.exp2(rng.integers(-2, 3, size=(N, T // 128))).astype(np.float32)
    out_full = torch.full((G + 1, M, N), 5.0, dtype=torch.float32, device="cuda")
    out = out_full[:G]
    print(f"persistent exact group_k sizes={sizes} M={M} N={N}", flush=True)
    bs.bs_grouped_scaled_mm(bs.BS_GROUP_K, torch.from_numpy(ends).cuda(), torch.from_numpy(qa).cuda(),
                            to_gpu_scales(sa), torch.from_numpy(qb).cuda(), to_gpu_scales(sb),
                            bs.BS_SCALE_1X128, out=out)
    torch.cuda.synchronize()
    d = out.cpu().numpy().astype(np.float64)
    start = 0
    for g, e in enumerate(ends):
        if e == start:
            assert np.all(d[g] == 0), f"empty group {g} must be zeros"
        else:
            a = gemm.dequant(qa[:, start:e], sa[:, start // 128:e // 128], 1)
            b = gemm.dequant(qb[:, start:e], sb[:, start // 128:e // 128], 1)
            bad = np.argwhere(d[g] != a @ b.T)
            assert bad.size == 0, f"group {g}: {len(bad)} inexact elements, first {bad[0]}"
        start = e
    assert torch.all(out_full[G] == 5.0)


def test_group_k_more_groups_than_ranked():
    """GROUP_K with more groups than the kernel ranks by size (256): the
    tiles then follow the natural group order."""
    need_gpu()
    rng = np.random.default_rng(41)
    G, M, N = 300, 256, 256
    sizes = np.where(rng.random(G) < 0.1, 128, 0)
    sizes[[0, 7, 299]] = [256, 128, 384]
    ends = np.cumsum(sizes).astype(np.int32)
    T = int(ends[-1])
    qa, sa = operand_1x128(M, T, 0.01, seed=42)
    qb, sb = operand_1x128(N, T, 1.0, seed=43)
    out = torch.full((G, M, N), 5.0, dtype=torch.bfloat16, device="cuda")
    print(f"group_k G={G} T={T}", flush=True)
    bs.bs_grouped_scaled_mm(bs.BS_GROUP_K, torch.from_numpy(ends).cuda(), torch.from_numpy(qa).cuda(),
                            to_gpu_scales(sa), torch.from_numpy(qb).cuda(), to_gpu_scales(sb),
                            bs.BS_SCALE_1X128, out=out)
    torch.cuda.synchronize()
    d = out.float().cpu().numpy().astype(np.float64)
    start = 0
    for g, e in enumerate(ends):
        if e == start:
            assert np.all(d[g] == 0), f"empty group {g} must be zeros"
        else:
            a = gemm.dequant(qa[:, start:e], sa[:, start // 128:e // 128], 1)
            b = gemm.dequant(qb[:, start:e], sb[:, start // 128:e // 128], 1)
            ok, worst = gemm.check_close(d[g], a @ b.T, a, b)
            assert ok, f"group {g}: worst {worst}"
        start = e


@pytest.mark.parametrize("G", [64, 70])
def test_group_m_many_groups(G):
    """GROUP_M at the largest group count ordered in XCD slices (64) and
    beyond it (70, the plain group order): ragged and empty groups."""
    need_gpu()
    rng = np.random.default_rng(G)
    sizes = rng.choice([0, 1, 37, 128, 300], G)
    ends = np.cumsum(sizes).astype(np.int32)
    M, N, K = int(ends[-1]), 256, 256
    qa, sa = operand_1x128(M, K, 1.0, seed=G + 1)
    w = inputs.bf16_normal((G * N, K), 0.02, seed=G + 2)
    qw, sw = quant.quant_128x128(bits16(w))
    sw_gpu = to_gpu_scales(sw)
    sb_view = torch.as_strided(sw_gpu, (G, K // 128, N // 128), (N // 128, sw_gpu.stride(0), 1))
    qb = torch.from_numpy(qw).cuda().view(G, N, K)
    full, out = guarded(M, N, torch.bfloat16)
    print(f"group_m G={G} M={M}", flush=True)
    bs.bs_grouped_scaled_mm(bs.BS_GROUP_M, torch.from_numpy(ends).cuda(), torch.from_numpy(qa).cuda(),
                            to_gpu_scales(sa), qb, sb_view, bs.BS_SCALE_128X128, out=out)
    torch.cuda.synchronize()
    d = out.float().cpu().numpy().astype(np.float64)
    start = 0
    for g, e in enumerate(ends):
        if e > start:
            a = gemm.dequant(qa[start:e], sa[start:e], 1)
            b = gemm.dequant(qw[g * N:(g + 1) * N], sw[g * N // 128:(g + 1) * N // 128], 128)
            ok, worst = gemm.check_close(d[start:e], a @ b.T, a, b)
            assert ok, f"group {g}: worst {worst}"
        start = e
    check_canaries(full, M, N)


def test_scaled_mm_largest_leading_dimensions():
    """Operands stored with leading dimensions just under the 2^22 limit the
    boundary accepts (1 GiB per operand view): the 32-bit lane and tile
    offsets of the copies must not wrap."""
    need_gpu()
    M, N, K = 256, 256, 512
    ld = (1 << 22) - 128
    qa, sa = operand_1x128(M, K, 1.0, seed=91)
    qb, sb = operand_128x128(N, K, 0.02, seed=92)
    abuf = torch.zeros((M, ld), dtype=torch.uint8, device="cuda")
    bbuf = torch.zeros((N, ld), dtype=torch.uint8, device="cuda")
    a = abuf[:, ld - K:]                 # the operand ends at the last byte of each row
    b = bbuf[:, ld - K:]
    a.copy_(torch.from_numpy(qa).cuda())
    b.copy_(torch.from_numpy(qb).cuda())
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    print(f"scaled_mm lda=ldb={ld}", flush=True)
    bs.bs_scaled_mm(a, to_gpu_scales(sa), b, to_gpu_scales(sb), bs.BS_SCALE_128X128, out=out)
    torch.cuda.synchronize()
    check_result(out, qa, sa, qb, sb, 128)
    del abuf, bbuf
    torch.cuda.empty_cache()
