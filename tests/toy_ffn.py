"""The toy FFN of the module-level parity tests, and an oracle linear layer.

("add FSDP and TP tests for Float8BlockwiseLinear", summary: a ToyModel FFN
with w1 and w2 split by output columns and out_proj by input rows under TP,
so w1 and w2 both read x and out_proj reads their combination.)  The reading
taken here is the gated FFN  out_proj(silu(w1 x) * w2 x)  with bias-free
layers.  Test code only.
"""

import numpy as np
import torch
import torch.nn.functional as F

from oracle import gemm, quant


class ToyFFN(torch.nn.Module):
    def __init__(self, dim, hidden, make_linear):
        super().__init__()
        self.w1 = make_linear(dim, hidden)
        self.w2 = make_linear(dim, hidden)
        self.out_proj = make_linear(hidden, dim)

    def forward(self, x):
        return self.out_proj(F.silu(self.w1(x)) * self.w2(x))


def _bits(t):
    return t.detach().contiguous().view(torch.int16).numpy().view(np.uint16)


def _bf16(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64)).to(torch.bfloat16)


class _OracleLinearFn(torch.autograd.Function):
    """The blockwise-FP8 recipe of one linear layer computed by the CPU oracle
    (codes and scales by the oracle quantizers, GEMMs in float64, results
    rounded to bf16 as the GPU writes them)."""

    @staticmethod
    def forward(ctx, x2, w):
        qx, sx = quant.quant_1x128_rowwise(_bits(x2))
        qw, sw = quant.quant_128x128(_bits(w))
        ctx.save_for_backward(x2, w)
        return _bf16(gemm.scaled_mm(qx, sx, qw, sw, 128))

    @staticmethod
    def backward(ctx, dy):
        x2, w = ctx.saved_tensors
        g = _bits(dy.to(torch.bfloat16))
        qg, sg = quant.quant_1x128_rowwise(g)
        qwt, swt = quant.quant_3d_colwise(_bits(w)[None])
        dx = _bf16(gemm.scaled_mm(qg, sg, qwt[0], swt[0], 128))
        qgt, sgt = quant.quant_1x128_colwise(g)
        qxt, sxt = quant.quant_1x128_colwise(_bits(x2))
        dw = _bf16(gemm.scaled_mm(qgt, sgt, qxt, sxt, 1))
        return dx, dw


class OracleLinear(torch.nn.Module):
    """CPU bf16 linear layer running the blockwise-FP8 recipe through the oracle."""

    def __init__(self, in_features, out_features):
        super().__init__()
        self.weight = torch.nn.Parameter(torch.zeros((out_features, in_features), dtype=torch.bfloat16))

    def forward(self, x):
        K = self.weight.shape[1]
        y = _OracleLinearFn.apply(x.reshape(-1, K), self.weight)
        return y.view(*x.shape[:-1], self.weight.shape[0])


class _OracleSwiGLUFn(torch.autograd.Function):
    """h = silu(a) * b rounded once to bf16 by the oracle; the backward is the
    oracle's (da = dh b silu'(a), db = dh silu(a), each rounded once to bf16
    from float64)."""

    @staticmethod
    def forward(ctx, a, b):
        from oracle import swiglu as oswiglu
        ctx.save_for_backward(a, b)
        h = oswiglu.swiglu(_bits(a), _bits(b))
        return torch.from_numpy(h.view(np.int16).copy()).view(torch.bfloat16).view(a.shape)

    @staticmethod
    def backward(ctx, dh):
        from oracle import swiglu as oswiglu
        a, b = ctx.saved_tensors
        da, db = oswiglu.swiglu_backward(_bits(a), _bits(b), _bits(dh.to(torch.bfloat16)))
        as_bf16 = lambda v: torch.from_numpy(v.view(np.int16).copy()).view(torch.bfloat16).view(a.shape)  # noqa: E731
        return as_bf16(da), as_bf16(db)


class OracleGatedFFN(torch.nn.Module):
    """The gated FFN with oracle-recipe layers and the oracle's once-rounded
    gated activation: the reference of the fused gated FFN module."""

    def __init__(self, dim, hidden):
        super().__init__()
        self.w1 = OracleLinear(dim, hidden)
        self.w2 = OracleLinear(dim, hidden)
        self.out_proj = OracleLinear(hidden, dim)

    def forward(self, x):
        return self.out_proj(_OracleSwiGLUFn.apply(self.w1(x), self.w2(x)))
