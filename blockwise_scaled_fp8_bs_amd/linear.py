"""Blockwise-FP8 linear layer for training: autograd over the five library calls.

("[not for land] float8 blockwise scaling training prototype using
deep_gemm", description, and "add FSDP and TP tests for Float8BlockwiseLinear",
summary: a drop-in replacement for a bias-free linear layer whose three GEMMs
run in FP8 with blockwise scales.)

For y = x W^T with x [M, K] and W [N, K] (bf16):

  forward   q(x) 1x128 along K (rows), and along M (transposed, kept for wgrad)
            q(W) 128x128, and the same blocks written transposed (q(W^T) [K, N],
            kept for dgrad), in one pass -- both operands in one launch
            y        = scaled_mm(q(x), q(W))                     [M, N]
  backward  q(dy) 1x128 along N (rows) and along M (transposed)
            dx       = scaled_mm(q(dy), q(W^T))                  [M, K]
            dW       = scaled_mm(q(dy^T), q(x^T)), both 1x128    [N, K]

Every step runs in the HIP kernels; this module allocates outputs with torch
and wires the calls into autograd.  The forward keeps only FP8 codes and
scales for the backward: the transposed codes of x (about half the bytes of
the bf16 input) and those of W^T.  M, K and N must be multiples of 128 (the colwise blocks run
along M); inputs must be contiguous bf16 GPU tensors -- nothing is copied
behind the caller's back.
"""

import torch

from . import binding as _b


def _check_dims(M, K, N):
    for name, v in (("tokens M", M), ("in_features K", K), ("out_features N", N)):
        if v % 128 != 0:
            raise ValueError(f"{name} = {v} must be a multiple of 128 for blockwise FP8 (1x128 / 128x128 blocks)")


def _quant_rows_cols(x):
    """1x128 codes of x [R, C] along rows and (transposed) along columns."""
    R, C = x.shape
    q = torch.empty((R, C), dtype=torch.uint8, device=x.device)
    s = _b.empty_scales(C // 128, R, x.device)
    qt = torch.empty((C, R), dtype=torch.uint8, device=x.device)
    st = _b.empty_scales(R // 128, C, x.device)
    _b.bs_quant_1x128(x, q, s, qt, st)
    return q, s, qt, st


class _Float8BlockwiseLinearFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x2, w):
        M, K = x2.shape
        N = w.shape[0]
        dev = x2.device
        # x along rows (this GEMM) and columns (kept for the wgrad GEMM), and
        # W in both layouts (rows for this GEMM, W^T contiguous along N kept
        # for the dgrad GEMM), all in one launch
        qx = torch.empty((M, K), dtype=torch.uint8, device=dev)
        sx = _b.empty_scales(K // 128, M, dev)
        qxt = torch.empty((K, M), dtype=torch.uint8, device=dev)
        sxt = _b.empty_scales(M // 128, K, dev)
        qw = torch.empty((N, K), dtype=torch.uint8, device=dev)
        sw = _b.empty_scales(K // 128, N // 128, dev)
        qwt = torch.empty((1, K, N), dtype=torch.uint8, device=dev)
        swt = torch.empty((1, N // 128, _b._round4(K // 128)), dtype=torch.float32, device=dev)
        _b.bs_quant_fwd_operands(x2, qx, sx, qxt, sxt, w, qw, sw, qwt, swt)
        y = _b.bs_scaled_mm(qx, sx, qw, sw, _b.BS_SCALE_128X128, out_dtype=torch.bfloat16)
        ctx.save_for_backward(qxt, sxt, qwt, swt)
        ctx.w_dtype = w.dtype
        return y

    @staticmethod
    def backward(ctx, dy):
        qxt, sxt, qwt, swt = ctx.saved_tensors
        # autograd may hand a non-contiguous gradient; the kernels need rows
        dy = dy.to(torch.bfloat16).contiguous()
        qg, sg, qgt, sgt = _quant_rows_cols(dy)
        dx = dw = None
        if ctx.needs_input_grad[0]:
            dx = _b.bs_scaled_mm(qg, sg, qwt[0], swt[0], _b.BS_SCALE_128X128, out_dtype=torch.bfloat16)
        if ctx.needs_input_grad[1]:
            dw = _b.bs_scaled_mm_ws(qgt, sgt, qxt, sxt, _b.BS_SCALE_1X128, out_dtype=ctx.w_dtype)
        return dx, dw


def float8_blockwise_linear(x, weight):
    """y = x . weight^T with blockwise-FP8 GEMMs in forward and backward.

    x [..., K] bf16 contiguous on the GPU; weight [N, K] bf16 contiguous.
    """
    if x.dtype != torch.bfloat16 or weight.dtype != torch.bfloat16:
        raise ValueError(f"x and weight must be bfloat16, got {x.dtype} and {weight.dtype}")
    if weight.dim() != 2 or not weight.is_contiguous():
        raise ValueError(f"weight must be a contiguous [N, K] matrix, got shape {tuple(weight.shape)}")
    N, K = weight.shape
    if x.shape[-1] != K:
        raise ValueError(f"x has {x.shape[-1]} features, weight expects {K}")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous (row-major); pass a contiguous tensor instead of relying on a copy")
    lead = x.shape[:-1]
    M = x.numel() // K if K else 0
    _check_dims(M, K, N)
    if not (x.is_cuda and weight.is_cuda):
        raise ValueError("x and weight must be GPU tensors")
    y = _Float8BlockwiseLinearFn.apply(x.view(M, K), weight)
    return y.view(*lead, N)


class Float8BlockwiseLinear(torch.nn.Module):
    """Bias-free linear layer whose forward and backward GEMMs run in
    blockwise-scaled FP8 (activations and gradients 1x128, weights 128x128)."""

    def __init__(self, in_features, out_features, device=None, dtype=torch.bfloat16):
        super().__init__()
        _check_dims(128, in_features, out_features)
        self.in_features = in_features
        self.out_features = out_features
        self.weight = torch.nn.Parameter(torch.empty((out_features, in_features), device=device, dtype=dtype))
        torch.nn.init.kaiming_uniform_(self.weight, a=5 ** 0.5)

    @classmethod
    def from_linear(cls, lin):
        """Same weights as a bias-free nn.Linear (converted to bf16)."""
        if lin.bias is not None:
            raise ValueError("Float8BlockwiseLinear has no bias")
        m = cls(lin.in_features, lin.out_features, device=lin.weight.device)
        with torch.no_grad():
            m.weight.copy_(lin.weight.to(torch.bfloat16))
        return m

    def forward(self, x):
        return float8_blockwise_linear(x, self.weight)

    def extra_repr(self):
        return f"in_features={self.in_features}, out_features={self.out_features}, blockwise fp8"


def swap_linear_layers(module):
    """Replace every bias-free nn.Linear under ``module`` (in place) by a
    Float8BlockwiseLinear with the same weights; returns ``module``."""
    for name, child in module.named_children():
        if isinstance(child, torch.nn.Linear) and child.bias is None:
            setattr(module, name, Float8BlockwiseLinear.from_linear(child))
        else:
            swap_linear_layers(child)
    return module
