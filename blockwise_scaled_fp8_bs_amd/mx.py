"""MXFP8 training layers: a dense linear layer and the MoE grouped GEMM, with
every GEMM in MXFP8 (E4M3 codes, one E8M0 scale per 32 values along the
contraction) on gfx950's block-scaled MFMA.

(The MXFP8 recipe of "[mxfp8 moe training] use new 3d colwise quantization
kernel", summary and microbenchmark table: grouped GEMMs of MoE training in
MXFP8, forward and forward + backward, with the expert weights quantized
along columns for the backward.  The pages name the recipe without defining
the format; the definition used is OCP MX v1.0.)

For y = x W^T, x [M, K], W [N, K]:

  forward   x  -> 32-blocks along K (rows) and along M (transposed, kept
                  for the weight gradient)            one quantizer pass
            W  -> 32-blocks along K (rows) and along N (transposed, kept
                  for the input gradient)             one quantizer pass
            y  = mx_mm(q(x), q(W))
  backward  dy -> 32-blocks along N (rows) and along M (transposed)
            dx = mx_mm(q(dy), q(W^T))                 contraction over N
            dW = mx_mm(q(dy^T), q(x^T))               contraction over M

The grouped form takes tokens sorted by expert (x [M, K], group g owns rows
[end_{g-1}, end_g)) and expert weights W [G, N, K].  Quantizing W as one
[G*N, K] matrix gives both layouts of every expert in one pass: its
32-row column blocks never cross an expert (N % 32 == 0), so the transposed
output [K, G*N] holds each W_g^T as a column slice -- the 3-D column-wise
quantization of the pages' kernel, with 32 x 1 blocks.  Forward and input
gradient are GROUP_M GEMMs over those per-expert views; the weight gradient
is a GROUP_K GEMM whose contraction groups are the token groups (their ends
must be multiples of 128).
"""

import torch

from . import binding as _b


def _check_mx_dims(**dims):
    for name, v in dims.items():
        if v % 128 != 0:
            raise ValueError(f"{name} = {v} must be a multiple of 128 for the MXFP8 layers "
                             "(128-wide tiles of 32-element blocks, transposed outputs)")


def _mx_rows_cols(x):
    """MX codes of x [R, C] in 32-blocks along rows and (transposed) along columns."""
    R, C = x.shape
    q = torch.empty((R, C), dtype=torch.uint8, device=x.device)
    s = _b.empty_mx_scales(C // 32, R, x.device)
    qt = torch.empty((C, R), dtype=torch.uint8, device=x.device)
    st = _b.empty_mx_scales(R // 32, C, x.device)
    _b.bs_mx_quant_1x32(x, q, s, qt, st)
    return q, s, qt, st


def _check_inputs(x, w, w_dims):
    for name, t in (("x", x), ("weight", w)):
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bfloat16, got {t.dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous (row-major); pass a contiguous tensor")
    if w.dim() != w_dims:
        raise ValueError(f"weight must be {w_dims}-D, got shape {tuple(w.shape)}")


class _Float8MXLinearFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x2, w):
        qx, sx, qxt, sxt = _mx_rows_cols(x2)
        qw, sw, qwt, swt = _mx_rows_cols(w)
        y = _b.bs_mx_scaled_mm(qx, sx, qw, sw, out_dtype=torch.bfloat16)
        ctx.save_for_backward(qxt, sxt, qwt, swt)
        ctx.w_dtype = w.dtype
        return y

    @staticmethod
    def backward(ctx, dy):
        qxt, sxt, qwt, swt = ctx.saved_tensors
        dy = dy.to(torch.bfloat16).contiguous()
        qg, sg, qgt, sgt = _mx_rows_cols(dy)
        dx = dw = None
        if ctx.needs_input_grad[0]:
            dx = _b.bs_mx_scaled_mm(qg, sg, qwt, swt, out_dtype=torch.bfloat16)
        if ctx.needs_input_grad[1]:
            dw = _b.bs_mx_scaled_mm(qgt, sgt, qxt, sxt, out_dtype=ctx.w_dtype)
        return dx, dw


def float8_mx_linear(x, weight):
    """y = x . weight^T with MXFP8 GEMMs in forward and backward.

    x [..., K] and weight [N, K]: contiguous bf16 GPU tensors; the token
    count, K and N multiples of 128.
    """
    _check_inputs(x, weight, 2)
    N, K = weight.shape
    if x.shape[-1] != K:
        raise ValueError(f"x has {x.shape[-1]} features, weight expects {K}")
    lead = x.shape[:-1]
    M = x.numel() // K if K else 0
    _check_mx_dims(tokens=M, in_features=K, out_features=N)
    if not (x.is_cuda and weight.is_cuda):
        raise ValueError("x and weight must be GPU tensors")
    y = _Float8MXLinearFn.apply(x.view(M, K), weight)
    return y.view(*lead, N)


class Float8MXLinear(torch.nn.Module):
    """Bias-free linear layer whose three GEMMs run in MXFP8."""

    def __init__(self, in_features, out_features, device=None, dtype=torch.bfloat16):
        super().__init__()
        _check_mx_dims(in_features=in_features, out_features=out_features)
        self.in_features, self.out_features = in_features, out_features
        self.weight = torch.nn.Parameter(torch.empty((out_features, in_features), device=device, dtype=dtype))
        torch.nn.init.kaiming_uniform_(self.weight, a=5 ** 0.5)

    @classmethod
    def from_linear(cls, lin):
        if getattr(lin, "bias", None) is not None:
            raise ValueError("Float8MXLinear has no bias")
        m = cls(lin.in_features, lin.out_features, device=lin.weight.device)
        with torch.no_grad():
            m.weight.copy_(lin.weight.to(torch.bfloat16))
        return m

    def forward(self, x):
        return float8_mx_linear(x, self.weight)

    def extra_repr(self):
        return f"in_features={self.in_features}, out_features={self.out_features}, mxfp8"


def _expert_views(w):
    """MX codes of W [G, N, K] as one [G*N, K] matrix, viewed per expert:
    forward operand [G, N, K] with scales [G, K/32, N], and the transposed
    (input-gradient) operand [G, K, N] with scales [G, N/32, K]."""
    G, N, K = w.shape
    q, s, qt, st = _mx_rows_cols(w.view(G * N, K))
    qf = q.view(G, N, K)
    sf = torch.as_strided(s, (G, K // 32, N), (N, s.stride(0), 1))
    qb = torch.as_strided(qt, (G, K, N), (N, qt.stride(0), 1))
    sbk = torch.as_strided(st, (G, N // 32, K), ((N // 32) * st.stride(0), st.stride(0), 1))
    return qf, sf, qb, sbk


class _MXGroupedMMFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, w, group_end):
        qx, sx, qxt, sxt = _mx_rows_cols(x)
        qf, sf, qb, sbk = _expert_views(w)
        y = _b.bs_mx_grouped_scaled_mm(_b.BS_GROUP_M, group_end, qx, sx, qf, sf, out_dtype=torch.bfloat16)
        ctx.save_for_backward(group_end, qxt, sxt, qb, sbk)
        ctx.w_dtype = w.dtype
        return y

    @staticmethod
    def backward(ctx, dy):
        group_end, qxt, sxt, qb, sbk = ctx.saved_tensors
        dy = dy.to(torch.bfloat16).contiguous()
        qg, sg, qgt, sgt = _mx_rows_cols(dy)
        dx = dw = None
        if ctx.needs_input_grad[0]:
            dx = _b.bs_mx_grouped_scaled_mm(_b.BS_GROUP_M, group_end, qg, sg, qb, sbk, out_dtype=torch.bfloat16)
        if ctx.needs_input_grad[1]:
            dw = _b.bs_mx_grouped_scaled_mm(_b.BS_GROUP_K, group_end, qgt, sgt, qxt, sxt, out_dtype=ctx.w_dtype)
        return dx, dw, None


def mx_grouped_mm(x, weight, group_end):
    """MoE expert GEMM y[rows of group g] = x[rows of group g] . weight[g]^T in
    MXFP8, forward and backward.

    x [M, K] bf16, tokens sorted by expert; weight [G, N, K] bf16; group_end
    an int32 GPU tensor [G] of cumulative row ends, each a multiple of 128
    (the weight gradient contracts over each group's tokens in 128-blocks;
    the ends are read on the device only, never checked on the host), the
    last equal to M.  M, K and N multiples of 128.
    """
    _check_inputs(x, weight, 3)
    G, N, K = weight.shape
    if x.dim() != 2 or x.shape[1] != K:
        raise ValueError(f"x must be [M, {K}], got {tuple(x.shape)}")
    if group_end.dtype != torch.int32 or tuple(group_end.shape) != (G,):
        raise ValueError(f"group_end must be an int32 tensor of shape [{G}] (one cumulative end per expert)")
    _check_mx_dims(tokens=x.shape[0], in_features=K, out_features=N)
    if not (x.is_cuda and weight.is_cuda and group_end.is_cuda):
        raise ValueError("x, weight and group_end must be GPU tensors")
    return _MXGroupedMMFn.apply(x, weight, group_end)
