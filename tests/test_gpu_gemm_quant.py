"""GPU parity of bs_scaled_mm_quant: the scaled GEMM whose epilogue also
writes the 1x128 quantization (rows and transposed columns) of its bf16
output.

* Exact arithmetic (small-integer codes, power-of-two scales, K <= 1024):
  every partial sum is exact in fp32, so the oracle's float64 product
  rounded once to bf16 (oracle.swiglu.round_to_bf16) IS the GPU's bf16 D;
  the oracle's 1x128 quantization of that D must then equal the GPU's codes
  and scales bit for bit, rows and transposed columns, and D too.
* Random operands: D within the recipe's tolerance of the oracle and equal
  bit for bit to bs_scaled_mm's bf16 output (same accumulation), and the
  codes equal to what bs_quant_1x128 writes from that D (the fused and the
  separate pass agree).
Outputs sit in canary-guarded buffers; scale padding must stay untouched.
"""

import numpy as np
import pytest
import torch

import blockwise_scaled_fp8_bs_amd as bs
from gpu_support import (CANARY_F32_BITS, check_canaries, check_scale_canaries, guarded, need_gpu, scale_buffer,
                         u8)
from oracle import gemm, quant, swiglu
from test_gpu_gemm import SMALL_INT_CODES, check_result, operand_128x128, operand_1x128, to_gpu_scales

pytestmark = pytest.mark.gpu


def _run(qa, sa, qb, sb, kind, rows=True, cols=True, with_d=True):
    M, K = qa.shape
    N = qb.shape[0]
    d_full, d = guarded(M, N, torch.bfloat16) if with_d else (None, None)
    outs = {}
    if rows:
        outs["qr_full"], outs["qr"] = guarded(M, N, torch.uint8)
        outs["sr_full"], outs["sr"] = scale_buffer(N // 128, M)
    if cols:
        outs["qc_full"], outs["qc"] = guarded(N, M, torch.uint8)
        outs["sc_full"], outs["sc"] = scale_buffer(M // 128, N)
    bs.bs_scaled_mm_quant(torch.from_numpy(qa).cuda(), to_gpu_scales(sa), torch.from_numpy(qb).cuda(),
                          to_gpu_scales(sb), kind, out=d, q_row=outs.get("qr"), s_row=outs.get("sr"),
                          q_col=outs.get("qc"), s_col=outs.get("sc"))
    torch.cuda.synchronize()
    if with_d:
        check_canaries(d_full, M, N)
    if rows:
        check_canaries(outs["qr_full"], M, N)
        check_scale_canaries(outs["sr_full"], N // 128, M)
    if cols:
        check_canaries(outs["qc_full"], N, M)
        check_scale_canaries(outs["sc_full"], M // 128, N)
    return d, outs


def _f32bits(t):
    return t.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("M,N,K", [(512, 640, 512), (384, 256, 1024), (4352, 4096, 256)])
@pytest.mark.parametrize("kind", [bs.BS_SCALE_128X128, bs.BS_SCALE_1X128])
def test_gemm_quant_exact_vs_oracle(M, N, K, kind):
    """The bf16 D and its 1x128 codes and scales, rows and transposed columns,
    bit for bit against the oracle (exact-arithmetic operands)."""
    need_gpu()
    rng = np.random.default_rng(M + N + K + kind)
    rb = 128 if kind == bs.BS_SCALE_128X128 else 1
    qa = rng.choice(SMALL_INT_CODES, size=(M, K))
    qb = rng.choice(SMALL_INT_CODES, size=(N, K))
    sa = np.exp2(rng.integers(-2, 3, size=(M, K // 128))).astype(np.float32)
    sb = np.exp2(rng.integers(-2, 3, size=(N // rb, K // 128))).astype(np.float32)
    # rows of zeros and a tiny row: a zero block takes the EPS-floored scale
    qa[5] = 0x00
    print(f"gemm_quant exact M={M} N={N} K={K} kind={kind}", flush=True)
    d, o = _run(qa, sa, qb, sb, kind)
    ref = gemm.scaled_mm(qa, sa, qb, sb, rb)                       # exact in float64
    d_ref = swiglu.round_to_bf16(ref)                              # rounded once to bf16
    assert np.array_equal(d.cpu().view(torch.int16).numpy().view(np.uint16), d_ref), "bf16 D"
    q_r, s_r = quant.quant_1x128_rowwise(d_ref)
    assert np.array_equal(u8(o["qr"]), q_r), "row codes"
    assert np.array_equal(_f32bits(o["sr"])[:, :M], np.ascontiguousarray(s_r.T).view(np.uint32)), "row scales"
    q_c, s_c = quant.quant_1x128_colwise(d_ref)
    assert np.array_equal(u8(o["qc"]), q_c), "column codes"
    assert np.array_equal(_f32bits(o["sc"])[:, :N], np.ascontiguousarray(s_c.T).view(np.uint32)), "column scales"


@pytest.mark.parametrize("M,N,K,cols", [(512, 640, 1024, True), (300, 384, 512, False), (4352, 4096, 512, True)])
@pytest.mark.parametrize("kind", [bs.BS_SCALE_128X128, bs.BS_SCALE_1X128])
def test_gemm_quant_random_matches_separate_pass(M, N, K, cols, kind):
    need_gpu()
    qa, sa = operand_1x128(M, K, 1.0, seed=M + K)
    if kind == bs.BS_SCALE_128X128:
        qb, sb = operand_128x128(N, K, 0.02, seed=N + 3 * K)
        rb = 128
    else:
        qb, sb = operand_1x128(N, K, 0.02, seed=N + 3 * K)
        rb = 1
    print(f"gemm_quant random M={M} N={N} K={K} kind={kind} cols={cols}", flush=True)
    d, o = _run(qa, sa, qb, sb, kind, cols=cols)
    check_result(d, qa, sa, qb, sb, rb)
    plain = bs.bs_scaled_mm(torch.from_numpy(qa).cuda(), to_gpu_scales(sa), torch.from_numpy(qb).cuda(),
                            to_gpu_scales(sb), kind)
    assert torch.equal(plain.view(torch.int16), d.cuda().view(torch.int16)), "D differs from bs_scaled_mm"
    qr = torch.empty((M, N), dtype=torch.uint8, device="cuda")
    sr = bs.empty_scales(N // 128, M, "cuda")
    qc = torch.empty((N, M), dtype=torch.uint8, device="cuda") if cols else None
    sc = bs.empty_scales(M // 128, N, "cuda") if cols else None
    bs.bs_quant_1x128(plain, qr, sr, qc, sc)
    torch.cuda.synchronize()
    assert torch.equal(qr, o["qr"].cuda()) and torch.equal(sr[:, :M], o["sr"][:, :M].cuda())
    if cols:
        assert torch.equal(qc, o["qc"].cuda()) and torch.equal(sc[:, :N], o["sc"][:, :N].cuda())


def test_gemm_quant_without_d_and_single_outputs():
    need_gpu()
    M, N, K = 512, 512, 512
    qa, sa = operand_1x128(M, K, 1.0, seed=5)
    qb, sb = operand_128x128(N, K, 0.02, seed=6)
    _, both = _run(qa, sa, qb, sb, bs.BS_SCALE_128X128)
    _, rows_only = _run(qa, sa, qb, sb, bs.BS_SCALE_128X128, cols=False, with_d=False)
    _, cols_only = _run(qa, sa, qb, sb, bs.BS_SCALE_128X128, rows=False, with_d=False)
    assert torch.equal(both["qr"], rows_only["qr"]) and torch.equal(both["sr"][:, :M], rows_only["sr"][:, :M])
    assert torch.equal(both["qc"], cols_only["qc"]) and torch.equal(both["sc"][:, :N], cols_only["sc"][:, :N])
