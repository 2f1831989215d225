"""The forward operands quantized in one launch (bs_quant_fwd_operands):
the activation's 1x128 row and column codes and the weights' 128x128 codes in
both layouts, bit-exact against the CPU oracle with guard bands and scale
padding untouched, and byte-equal to the two separate calls at a dense
linear layer's size."""

import numpy as np
import pytest
import torch

import blockwise_scaled_fp8_bs_amd as bs
from blockwise_scaled_fp8_bs_amd import inputs
from oracle import quant
from gpu_support import bits16, check_canaries, check_scale_canaries, guarded, need_gpu, scale_buffer, special_input, u8
from test_gpu_quant import assert_codes, assert_scales

pytestmark = pytest.mark.gpu


def _weight_buffers(G, N, K):
    """Guarded weight outputs: q [G*N, K], s [K/128, G*N/128 (+pad)], qt [G, K, N], st [G, N/128, K/128 (+pad)]."""
    ld_s = (G * N // 128 + 3) // 4 * 4 + 4
    q_full = torch.full((G * N + 1, K + 16), 0xA5, dtype=torch.uint8, device="cuda")
    s_full = torch.empty((K // 128 + 1, ld_s), dtype=torch.float32, device="cuda")
    s_full.view(torch.int32).fill_(0x7FBADBAD)
    ld_st = (K // 128 + 3) // 4 * 4 + 4
    qt_full = torch.full((G + 1, K, N + 16), 0xA5, dtype=torch.uint8, device="cuda")
    st_full = torch.empty((G + 1, N // 128, ld_st), dtype=torch.float32, device="cuda")
    st_full.view(torch.int32).fill_(0x7FBADBAD)
    return (q_full, s_full, qt_full, st_full), (q_full[:G * N, :K], s_full[:K // 128], qt_full[:G, :, :N],
                                                st_full[:G])


@pytest.mark.parametrize("R,C,G,N,K", [(256, 512, 1, 384, 512), (384, 640, 3, 256, 384), (128, 128, 2, 128, 896),
                                       (0, 256, 2, 256, 256), (256, 384, 0, 128, 384)])
def test_fwd_operands_vs_oracle(R, C, G, N, K):
    need_gpu()
    x = special_input(R, C, seed=R * 5 + C) if R else torch.zeros((0, C), dtype=torch.bfloat16)
    w = (torch.stack([special_input(N, K, seed=g * 11 + K, sigma=0.02) for g in range(G)]) if G
         else torch.zeros((0, N, K), dtype=torch.bfloat16))
    xg = x.cuda()
    wg = w.cuda()
    qr_full, qr = guarded(R, C, torch.uint8)
    sr_full, sr = scale_buffer(C // 128, R)
    qc_full, qc = guarded(C, R, torch.uint8)
    sc_full, sc = scale_buffer(R // 128, C)
    (q_full, s_full, qt_full, st_full), (qw, sw, qwt, swt) = _weight_buffers(G, N, K)
    print(f"quant_fwd_operands x={R}x{C} w={G}x{N}x{K}", flush=True)
    bs.bs_quant_fwd_operands(xg, qr, sr, qc, sc, wg, qw, sw, qwt, swt)
    torch.cuda.synchronize()
    if R:
        xb = bits16(x)
        q_ref, s_ref = quant.quant_1x128_rowwise(xb)
        assert_codes(qr, q_ref)
        assert_scales(sr, s_ref)
        q_ref, s_ref = quant.quant_1x128_colwise(xb)
        assert_codes(qc, q_ref)
        assert_scales(sc, s_ref)
    check_canaries(qr_full, R, C)
    check_scale_canaries(sr_full, C // 128, R)
    check_canaries(qc_full, C, R)
    check_scale_canaries(sc_full, R // 128, C)
    qa, sa = u8(q_full), s_full.cpu().view(torch.int32).numpy().view(np.uint32)
    qta, sta = u8(qt_full), st_full.cpu().view(torch.int32).numpy().view(np.uint32)
    if G:
        wb = bits16(w)
        q_ref, s_ref = quant.quant_128x128(wb.reshape(G * N, K))
        qt_ref, st_ref = quant.quant_3d_colwise(wb)
        assert np.array_equal(qa[:G * N, :K], q_ref)
        assert np.array_equal(sa[:K // 128, :G * N // 128], np.ascontiguousarray(s_ref.T).view(np.uint32))
        assert np.array_equal(qta[:G, :, :N], qt_ref)
        for g in range(G):
            assert np.array_equal(sta[g, :, :K // 128], np.ascontiguousarray(st_ref[g].T).view(np.uint32))
    assert np.all(qa[:G * N, K:] == 0xA5) and np.all(qa[G * N:] == 0xA5)
    assert np.all(sa[:K // 128, G * N // 128:] == 0x7FBADBAD) and np.all(sa[K // 128:] == 0x7FBADBAD)
    assert np.all(qta[:G, :, N:] == 0xA5) and np.all(qta[G:] == 0xA5)
    assert np.all(sta[:G, :, K // 128:] == 0x7FBADBAD) and np.all(sta[G:] == 0x7FBADBAD)


@pytest.mark.parametrize("M,K,N", [(8192, 4096, 4096), (16384, 7168, 2048)])
def test_fwd_operands_equal_the_separate_calls(M, K, N):
    """At dense linear-layer sizes (thousands of tiles in the launch) every
    byte equals what bs_quant_1x128 and bs_quant_128x128_both write."""
    need_gpu()
    x = inputs.bf16_normal((M, K), 1.0, seed=M + K, device="cuda")
    w = inputs.bf16_normal((N, K), 0.02, seed=N + K, device="cuda")
    outs = []
    for paired in (False, True):
        qr = torch.empty((M, K), dtype=torch.uint8, device="cuda")
        sr = bs.empty_scales(K // 128, M, "cuda")
        qc = torch.empty((K, M), dtype=torch.uint8, device="cuda")
        sc = bs.empty_scales(M // 128, K, "cuda")
        qw = torch.empty((N, K), dtype=torch.uint8, device="cuda")
        sw = bs.empty_scales(K // 128, N // 128, "cuda")
        qwt = torch.empty((1, K, N), dtype=torch.uint8, device="cuda")
        swt = bs.empty_scales(N // 128, K // 128, "cuda")[None]
        for t in (sr, sc, sw, swt):
            t.zero_()
        print(f"quant_fwd_operands paired={paired} M={M} K={K} N={N}", flush=True)
        if paired:
            bs.bs_quant_fwd_operands(x, qr, sr, qc, sc, w, qw, sw, qwt, swt)
        else:
            bs.bs_quant_1x128(x, qr, sr, qc, sc)
            bs.bs_quant_128x128_both(w, qw, sw, qwt, swt)
        torch.cuda.synchronize()
        outs.append([t.view(torch.uint8).cpu() for t in (qr, sr, qc, sc, qw, sw, qwt, swt)])
    for name, a, b in zip(("q_row", "s_row", "q_col", "s_col", "qw", "sw", "qwt", "swt"), *outs):
        assert torch.equal(a, b), f"{name} differs between the paired launch and the separate calls"


def test_fwd_operands_strided_views():
    """x as a column slice of a wider tensor (ld_x > C) and the weights as
    experts of a padded stack (stride between experts > N * ld_w, ld_w > K):
    same bytes as the oracle on the logical values."""
    need_gpu()
    R, C, G, N, K = 384, 256, 2, 256, 384
    xs = torch.zeros((R, C + 64), dtype=torch.bfloat16)
    xs[:, 32:32 + C] = special_input(R, C, seed=5)
    ws = torch.zeros((G, N + 128, K + 32), dtype=torch.bfloat16)
    for g in range(G):
        ws[g, :N, 16:16 + K] = special_input(N, K, seed=9 + g, sigma=0.02)
    xg = xs.cuda()[:, 32:32 + C]
    wg = ws.cuda()[:, :N, 16:16 + K]
    assert xg.stride(0) == C + 64 and wg.stride(1) == K + 32 and wg.stride(0) == (N + 128) * (K + 32)
    qr_full, qr = guarded(R, C, torch.uint8)
    sr_full, sr = scale_buffer(C // 128, R)
    qc_full, qc = guarded(C, R, torch.uint8)
    sc_full, sc = scale_buffer(R // 128, C)
    (q_full, s_full, qt_full, st_full), (qw, sw, qwt, swt) = _weight_buffers(G, N, K)
    print("quant_fwd_operands strided views", flush=True)
    bs.bs_quant_fwd_operands(xg, qr, sr, qc, sc, wg, qw, sw, qwt, swt)
    torch.cuda.synchronize()
    xb = bits16(xs[:, 32:32 + C].contiguous())
    q_ref, s_ref = quant.quant_1x128_rowwise(xb)
    assert_codes(qr, q_ref)
    assert_scales(sr, s_ref)
    q_ref, s_ref = quant.quant_1x128_colwise(xb)
    assert_codes(qc, q_ref)
    assert_scales(sc, s_ref)
    check_canaries(qr_full, R, C)
    check_canaries(qc_full, C, R)
    check_scale_canaries(sr_full, C // 128, R)
    check_scale_canaries(sc_full, R // 128, C)
    wb = bits16(ws[:, :N, 16:16 + K].contiguous())
    q_ref, s_ref = quant.quant_128x128(wb.reshape(G * N, K))
    qt_ref, st_ref = quant.quant_3d_colwise(wb)
    assert np.array_equal(u8(q_full)[:G * N, :K], q_ref)
    sa = s_full.cpu().view(torch.int32).numpy().view(np.uint32)
    assert np.array_equal(sa[:K // 128, :G * N // 128], np.ascontiguousarray(s_ref.T).view(np.uint32))
    assert np.array_equal(u8(qt_full)[:G, :, :N], qt_ref)
    sta = st_full.cpu().view(torch.int32).numpy().view(np.uint32)
    for g in range(G):
        assert np.array_equal(sta[g, :, :K // 128], np.ascontiguousarray(st_ref[g].T).view(np.uint32))
