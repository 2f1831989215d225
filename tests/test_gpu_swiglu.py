"""GPU parity of the fused gated activation + 1x128 quantizer.

h = silu(a) * b is computed in fp32 and rounded once to bf16 on the GPU; the
oracle evaluates it in float64 and rounds once.  h must match the oracle
except for rare one-step differences (exact values within fp32 rounding of a
bf16 tie), and the codes and scales must be exactly the oracle's 1x128
quantization of the GPU's own h, rows and transposed columns."""

import numpy as np
import pytest
import torch

import blockwise_scaled_fp8_bs_amd as bs
from blockwise_scaled_fp8_bs_amd import inputs
from gpu_support import bits16, check_canaries, check_scale_canaries, guarded, need_gpu, scale_buffer, u8
from oracle import quant, swiglu

pytestmark = pytest.mark.gpu


def _inputs(R, C, seed):
    a = inputs.bf16_normal((R, C), 3.0, seed)
    b = inputs.bf16_normal((R, C), 1.0, seed + 1)
    ab = bits16(a).copy()
    if R >= 4 and C >= 128:   # very large / very negative / zero gate inputs
        ab[0, :64] = bits16(torch.full((64,), 150.0, dtype=torch.bfloat16))
        ab[1, :64] = bits16(torch.full((64,), -150.0, dtype=torch.bfloat16))
        ab[2, :128] = 0
        ab[3, 3] = 0x8000
    a = torch.from_numpy(ab.view(np.int16)).view(torch.bfloat16)
    return a, b


def _assert_h_close(h_gpu_bits, a, b):
    want = swiglu.swiglu(bits16(a), bits16(b))
    d = np.abs(h_gpu_bits.astype(np.int32) - want.astype(np.int32))
    nonzero = ((h_gpu_bits & 0x7FFF) != 0) | ((want & 0x7FFF) != 0)
    assert d[nonzero].max(initial=0) <= 1, "h differs from the oracle by more than one bf16 step"
    assert np.array_equal(h_gpu_bits[~nonzero] & 0x7FFF, want[~nonzero] & 0x7FFF)
    assert (d != 0).mean() < 2e-3, f"too many one-step differences: {(d != 0).mean()}"


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
    hb = bits16(h)
    _assert_h_close(hb, a, b)
    q_ref, s_ref = quant.quant_1x128_rowwise(hb)
    assert np.array_equal(u8(qr), q_ref)
    assert np.array_equal(sr.cpu().numpy().T[:R], s_ref)
    qc_ref, sc_ref = quant.quant_1x128_colwise(hb)
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
    hb = bits16(h)
    _assert_h_close(hb, a, b)
    q_ref, s_ref = quant.quant_1x128_rowwise(hb)
    assert np.array_equal(u8(qr), q_ref)
    assert np.array_equal(sr.cpu().numpy().T[:R], s_ref)
    check_canaries(qr_full, R, C)


def test_swiglu_quant_rejects_mismatched_b():
    need_gpu()
    a = torch.zeros((128, 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="b must be"):
        bs.bs_swiglu_quant_1x128(a, a[:, :128], None, torch.empty((128, 256), dtype=torch.uint8, device="cuda"),
                                 bs.empty_scales(2, 128, "cuda"))
