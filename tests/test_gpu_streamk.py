"""GPU parity of bs_scaled_mm_ws, the stream-K form of the dense scaled GEMM.

Shapes are chosen so that the output tiles (256 x 256) do not fill whole
rounds of the GPU's resident workgroups, so the last round's tiles are split
along K and summed through the workspace.  Checks: exact small-integer
arithmetic bit for bit against the oracle (a missing, doubled or misplaced
partial tile shows as an exact mismatch), random operands within the recipe's
tolerance, reproducible results, and the plain kernel when the workspace is
too small.
"""

import numpy as np
import pytest
import torch

import blockwise_scaled_fp8_bs_amd as bs
from gpu_support import check_canaries, guarded, need_gpu
from test_gpu_gemm import SMALL_INT_CODES, check_result, operand_128x128, operand_1x128, to_gpu_scales

pytestmark = pytest.mark.gpu

# (M, N, K): 4 tiles over 32 K blocks (8 pieces per tile); 272 tiles = one
# whole round + 16 split tiles; a ragged M with 6 tiles
SHAPES = [(512, 512, 4096), (4352, 4096, 1024), (300, 640, 2048)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("kind", [bs.BS_SCALE_128X128, bs.BS_SCALE_1X128])
def test_streamk_exact_small_integers(M, N, K, kind):
    need_gpu()
    need = bs.bs_scaled_mm_workspace_bytes(M, N, K, kind, torch.float32)
    assert need > 0, "shape chosen to be split"
    rng = np.random.default_rng(M + N + K + kind)
    rb = 128 if kind == bs.BS_SCALE_128X128 else 1
    qa = rng.choice(SMALL_INT_CODES, size=(M, K))
    qb = rng.choice(SMALL_INT_CODES, size=(N, K))
    sa = np.exp2(rng.integers(-2, 3, size=(M, K // 128))).astype(np.float32)
    sb = np.exp2(rng.integers(-2, 3, size=(N // rb, K // 128))).astype(np.float32)
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")  # no initial contents needed
    full, out = guarded(M, N, torch.float32)
    print(f"stream-K exact M={M} N={N} K={K} kind={kind} workspace={need}", flush=True)
    bs.bs_scaled_mm_ws(torch.from_numpy(qa).cuda(), to_gpu_scales(sa), torch.from_numpy(qb).cuda(),
                       to_gpu_scales(sb), kind, ws, out=out)
    torch.cuda.synchronize()
    check_result(out, qa, sa, qb, sb, rb, exact=True)
    check_canaries(full, M, N)


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("kind", [bs.BS_SCALE_128X128, bs.BS_SCALE_1X128])
def test_streamk_tolerance_and_reproducible(M, N, K, kind):
    need_gpu()
    qa, sa = operand_1x128(M, K, 1.0 if kind == bs.BS_SCALE_128X128 else 0.01, seed=M + 3 * K)
    if kind == bs.BS_SCALE_128X128:
        qb, sb = operand_128x128(N, K, 0.02, seed=N + 5 * K)
        rb = 128
    else:
        qb, sb = operand_1x128(N, K, 1.0, seed=N + 5 * K)
        rb = 1
    ga, gb = torch.from_numpy(qa).cuda(), torch.from_numpy(qb).cuda()
    gsa, gsb = to_gpu_scales(sa), to_gpu_scales(sb)
    ws = bs.streamk_workspace(bs.bs_scaled_mm_workspace_bytes(M, N, K, kind))
    print(f"stream-K tolerance M={M} N={N} K={K} kind={kind}", flush=True)
    d1 = bs.bs_scaled_mm_ws(ga, gsa, gb, gsb, kind, ws)
    d2 = bs.bs_scaled_mm_ws(ga, gsa, gb, gsb, kind, ws)
    torch.cuda.synchronize()
    check_result(d1, qa, sa, qb, sb, rb)
    assert torch.equal(d1.view(torch.int16), d2.view(torch.int16)), "stream-K results must be reproducible"


def test_streamk_small_workspace_runs_the_plain_kernel():
    need_gpu()
    M, N, K = 512, 512, 4096
    qa, sa = operand_1x128(M, K, 1.0, seed=1)
    qb, sb = operand_128x128(N, K, 0.02, seed=2)
    ga, gb, gsa, gsb = torch.from_numpy(qa).cuda(), torch.from_numpy(qb).cuda(), to_gpu_scales(sa), to_gpu_scales(sb)
    plain = bs.bs_scaled_mm(ga, gsa, gb, gsb, bs.BS_SCALE_128X128)
    need = bs.bs_scaled_mm_workspace_bytes(M, N, K, bs.BS_SCALE_128X128)
    ws = torch.zeros(need - 256, dtype=torch.uint8, device="cuda")
    ws.fill_(7)  # not zero: must not be touched by the plain kernel
    got = bs.bs_scaled_mm_ws(ga, gsa, gb, gsb, bs.BS_SCALE_128X128, ws)
    torch.cuda.synchronize()
    assert torch.equal(plain.view(torch.int16), got.view(torch.int16))
    assert bool((ws == 7).all().item())


def test_streamk_full_rounds_need_no_workspace():
    need_gpu()
    # 256 x 256 tiles: 16 x 16 = 256 of them, one per CU of a 256-CU GPU
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if cus != 256:
        pytest.skip("tile count chosen for 256 CUs")
    assert bs.bs_scaled_mm_workspace_bytes(4096, 4096, 8192, bs.BS_SCALE_1X128) == 0
    # 640 tiles: two full rounds and 128 tiles split
    assert bs.bs_scaled_mm_workspace_bytes(8192, 5120, 16384, bs.BS_SCALE_1X128) > 0
    # 224 tiles: a last round at least 3/4 full is not split
    assert bs.bs_scaled_mm_workspace_bytes(2048, 7168, 16384, bs.BS_SCALE_1X128) == 0
