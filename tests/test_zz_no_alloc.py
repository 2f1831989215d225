"""The allocation-free stream-K GEMM, bs_scaled_mm_noalloc, called through
the C ABI: its output must equal bs_scaled_mm_ws's (the same kernels with a
caller workspace) bit for bit, and lie within the recipe's tolerance of the
oracle, on two calls in a row -- the second with a smaller problem, so that
it runs on the scratch contents the first left behind -- and on a problem
that is not split."""

import ctypes

import numpy as np
import pytest
import torch

import blockwise_scaled_fp8_bs_amd as bs
from blockwise_scaled_fp8_bs_amd import _lib
from gpu_support import need_gpu
from test_gpu_gemm import check_result, operand_128x128, operand_1x128, to_gpu_scales

pytestmark = pytest.mark.gpu


def _noalloc(a, sa, b, sb, kind, out):
    M, K = a.shape
    N = b.shape[0]
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    dt = bs.BS_OUT_F32 if out.dtype == torch.float32 else bs.BS_OUT_BF16
    st = _lib.load().bs_scaled_mm_noalloc(M, N, K, p(a), a.stride(0), p(sa), sa.stride(0), bs.BS_SCALE_1X128,
                                          p(b), b.stride(0), p(sb), sb.stride(0), kind, p(out), out.stride(0), dt,
                                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, _lib.load().bs_last_error().decode()


def _operands(M, N, K, kind, seed):
    qa, sa = operand_1x128(M, K, 1.0 if kind == bs.BS_SCALE_128X128 else 0.01, seed=seed)
    if kind == bs.BS_SCALE_128X128:
        qb, sb = operand_128x128(N, K, 0.02, seed=seed + 1)
    else:
        qb, sb = operand_1x128(N, K, 1.0, seed=seed + 1)
    return qa, sa, qb, sb


@pytest.mark.parametrize("first,second", [
    # (M, N, K, kind): 272 tiles (one full round + 16 split), then 4 tiles split 8 ways
    ((4352, 4096, 1024, bs.BS_SCALE_1X128), (512, 512, 4096, bs.BS_SCALE_128X128)),
    ((512, 512, 4096, bs.BS_SCALE_1X128), (300, 640, 2048, bs.BS_SCALE_1X128)),
])
def test_noalloc_matches_workspace_form_twice(first, second):
    need_gpu()
    for (M, N, K, kind), seed in ((first, 7), (second, 11)):
        assert bs.bs_scaled_mm_workspace_bytes(M, N, K, kind) > 0, "shape chosen to be split"
        qa, sa, qb, sb = _operands(M, N, K, kind, seed)
        ga, gb, gsa, gsb = (torch.from_numpy(qa).cuda(), torch.from_numpy(qb).cuda(), to_gpu_scales(sa),
                            to_gpu_scales(sb))
        ws = torch.zeros(bs.bs_scaled_mm_workspace_bytes(M, N, K, kind), dtype=torch.uint8, device="cuda")
        ref = bs.bs_scaled_mm_ws(ga, gsa, gb, gsb, kind, ws)
        out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        print(f"noalloc M={M} N={N} K={K} kind={kind}", flush=True)
        _noalloc(ga, gsa, gb, gsb, kind, out)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), "noalloc differs from bs_scaled_mm_ws"
        check_result(out, qa, sa, qb, sb, 128 if kind == bs.BS_SCALE_128X128 else 1)


def test_noalloc_unsplit_problem_is_the_plain_gemm():
    need_gpu()
    M, N, K, kind = 256, 256, 512, bs.BS_SCALE_128X128
    assert bs.bs_scaled_mm_workspace_bytes(M, N, K, kind) == 0
    qa, sa, qb, sb = _operands(M, N, K, kind, 3)
    ga, gb, gsa, gsb = torch.from_numpy(qa).cuda(), torch.from_numpy(qb).cuda(), to_gpu_scales(sa), to_gpu_scales(sb)
    ref = bs.bs_scaled_mm(ga, gsa, gb, gsb, kind, out_dtype=torch.float32)
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    _noalloc(ga, gsa, gb, gsb, kind, out)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), ref.view(torch.int32))
    check_result(out, qa, sa, qb, sb, 128)
