"""GPU parity of the MXFP8 training layers (dense linear and MoE grouped
GEMM), forward and backward.

* Each layer is exactly its kernel calls (bit for bit against calling the
  quantizer and the GEMMs by hand), and the grouped layer equals the dense
  layer applied expert by expert, bit for bit.
* Outputs and gradients match the oracle's recipe -- the oracle quantizes x,
  W and dy itself (rows and transposed columns) and multiplies in float64 --
  within 2e-3 * ||a_m|| * ||b_n|| per element.
"""

import numpy as np
import pytest
import torch

import blockwise_scaled_fp8_bs_amd as bs
from blockwise_scaled_fp8_bs_amd import inputs
from gpu_support import bits16, need_gpu
from oracle import gemm, mx

pytestmark = pytest.mark.gpu


def _oracle_mm(qa_sa, qb_sb):
    a = mx.dequant_mx(*qa_sa)
    b = mx.dequant_mx(*qb_sb)
    return a @ b.T, a, b


def _close(got, ref, a, b, what):
    ok, worst = gemm.check_close(got.detach().float().cpu().numpy().astype(np.float64), ref, a, b)
    assert ok, f"{what}: worst |err| / bound = {worst}"


def test_mx_linear_is_exactly_its_kernel_calls():
    need_gpu()
    M, K, N = 384, 512, 256
    print("mx linear composition", flush=True)
    x = inputs.bf16_normal((M, K), 1.0, 1).cuda().requires_grad_()
    w = inputs.bf16_normal((N, K), 0.02, 2).cuda().requires_grad_()
    dy = inputs.bf16_normal((M, N), 0.01, 3).cuda()
    y = bs.float8_mx_linear(x, w)
    y.backward(dy)
    torch.cuda.synchronize()

    def q(t):
        R, C = t.shape
        out = (torch.empty((R, C), dtype=torch.uint8, device="cuda"), bs.empty_mx_scales(C // 32, R, "cuda"),
               torch.empty((C, R), dtype=torch.uint8, device="cuda"), bs.empty_mx_scales(R // 32, C, "cuda"))
        bs.bs_mx_quant_1x32(t, *out)
        return out

    qx, sx, qxt, sxt = q(x.detach())
    qw, sw, qwt, swt = q(w.detach())
    qg, sg, qgt, sgt = q(dy)
    y_ref = bs.bs_mx_scaled_mm(qx, sx, qw, sw)
    dx_ref = bs.bs_mx_scaled_mm(qg, sg, qwt, swt)
    dw_ref = bs.bs_mx_scaled_mm(qgt, sgt, qxt, sxt)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)
    assert torch.equal(x.grad, dx_ref)
    assert torch.equal(w.grad, dw_ref)


def test_mx_linear_matches_oracle_recipe():
    need_gpu()
    M, K, N = 256, 640, 384
    print("mx linear vs oracle", flush=True)
    x = inputs.bf16_normal((M, K), 1.0, 11)
    w = inputs.bf16_normal((N, K), 0.02, 12)
    dy = inputs.bf16_normal((M, N), 0.01, 13)
    xg = x.cuda().requires_grad_()
    wg = w.cuda().requires_grad_()
    y = bs.float8_mx_linear(xg, wg)
    y.backward(dy.cuda())
    torch.cuda.synchronize()
    xb, wb, gb = bits16(x), bits16(w), bits16(dy)
    ref, a, b = _oracle_mm(mx.quant_mx_rowwise(xb), mx.quant_mx_rowwise(wb))
    _close(y, ref, a, b, "y")
    ref, a, b = _oracle_mm(mx.quant_mx_rowwise(gb), mx.quant_mx_colwise(wb))
    _close(xg.grad, ref, a, b, "dx")
    ref, a, b = _oracle_mm(mx.quant_mx_colwise(gb), mx.quant_mx_colwise(xb))
    _close(wg.grad, ref, a, b, "dW")


def _moe(sizes, K, N, seed):
    G = len(sizes)
    ends = np.cumsum(sizes).astype(np.int32)
    M = int(ends[-1])
    x = inputs.bf16_normal((M, K), 1.0, seed)
    w = inputs.bf16_normal((G, N, K), 0.02, seed + 1)
    dy = inputs.bf16_normal((M, N), 0.01, seed + 2)
    return ends, x, w, dy


@pytest.mark.parametrize("sizes", [(256, 0, 384), (128, 128, 128, 128)])
def test_mx_grouped_mm_matches_oracle_recipe(sizes):
    need_gpu()
    K, N = 512, 384
    ends, x, w, dy = _moe(sizes, K, N, seed=len(sizes))
    print(f"mx grouped mm sizes={sizes}", flush=True)
    xg = x.cuda().requires_grad_()
    wg = w.cuda().requires_grad_()
    y = bs.mx_grouped_mm(xg, wg, torch.from_numpy(ends).cuda())
    y.backward(dy.cuda())
    torch.cuda.synchronize()
    start = 0
    for g, e in enumerate(ends):
        wb = bits16(w[g])
        if e > start:
            xb, gb = bits16(x[start:e]), bits16(dy[start:e])
            ref, a, b = _oracle_mm(mx.quant_mx_rowwise(xb), mx.quant_mx_rowwise(wb))
            _close(y[start:e], ref, a, b, f"y group {g}")
            ref, a, b = _oracle_mm(mx.quant_mx_rowwise(gb), mx.quant_mx_colwise(wb))
            _close(xg.grad[start:e], ref, a, b, f"dx group {g}")
            ref, a, b = _oracle_mm(mx.quant_mx_colwise(gb), mx.quant_mx_colwise(xb))
            _close(wg.grad[g], ref, a, b, f"dW group {g}")
        else:
            assert torch.count_nonzero(wg.grad[g]).item() == 0, f"empty group {g}: dW must be zero"
        start = e


def test_mx_grouped_mm_equals_dense_per_expert():
    need_gpu()
    sizes, K, N = (384, 128, 256), 256, 512
    ends, x, w, dy = _moe(sizes, K, N, seed=40)
    print("mx grouped mm vs dense layer per expert", flush=True)
    xg = x.cuda().requires_grad_()
    wg = w.cuda().requires_grad_()
    y = bs.mx_grouped_mm(xg, wg, torch.from_numpy(ends).cuda())
    y.backward(dy.cuda())
    start = 0
    for g, e in enumerate(ends):
        xe = x[start:e].cuda().requires_grad_()
        we = w[g].cuda().requires_grad_()
        ye = bs.float8_mx_linear(xe, we)
        ye.backward(dy[start:e].cuda())
        torch.cuda.synchronize()
        assert torch.equal(y[start:e], ye), f"y group {g}"
        assert torch.equal(xg.grad[start:e], xe.grad), f"dx group {g}"
        assert torch.equal(wg.grad[g], we.grad), f"dW group {g}"
        start = e


def test_mx_grouped_mm_full_size_sampled():
    # the bench's MoE shape and launch configuration (128000 tokens, 8 experts
    # of [8192, 5120], equal groups); sampled outputs recomputed by the oracle
    # from the bf16 inputs: rows of y and dx in two groups (the expert's W
    # quantized whole, rows and columns), and single elements of dW (a column
    # of dy and of x quantized along the group's tokens)
    need_gpu()
    M, N, K, G = 128000, 8192, 5120, 8
    x = inputs.bf16_normal((M, K), 1.0, 61, device="cuda").requires_grad_()
    w = inputs.bf16_normal((G, N, K), 0.02, 62, device="cuda").requires_grad_()
    dy = inputs.bf16_normal((M, N), 0.01, 63, device="cuda")
    ends = torch.tensor([(g + 1) * M // G for g in range(G)], dtype=torch.int32, device="cuda")
    print("mx grouped mm 128000 x 8192 x 5120, 8 experts", flush=True)
    y = bs.mx_grouped_mm(x, w, ends)
    y.backward(dy)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    per = M // G
    for g in (0, 5):
        rows = np.sort(rng.choice(per, 6, replace=False)) + g * per
        idx = torch.from_numpy(rows).cuda()
        wb = bits16(w[g])
        xb, gb = bits16(x.detach()[idx]), bits16(dy[idx])
        ref, a, b = _oracle_mm(mx.quant_mx_rowwise(xb), mx.quant_mx_rowwise(wb))
        _close(y[idx], ref, a, b, f"y group {g}")
        ref, a, b = _oracle_mm(mx.quant_mx_rowwise(gb), mx.quant_mx_colwise(wb))
        _close(x.grad[idx], ref, a, b, f"dx group {g}")
        lo, hi = g * per, (g + 1) * per
        for _ in range(4):
            n, k = int(rng.integers(N)), int(rng.integers(K))
            qa = mx.quant_mx_rowwise(bits16(dy[lo:hi, n][None]))
            qb = mx.quant_mx_rowwise(bits16(x.detach()[lo:hi, k][None]))
            ref, a, b = _oracle_mm(qa, qb)
            _close(w.grad[g, n, k].reshape(1, 1), ref, a, b, f"dW[{g}, {n}, {k}]")
