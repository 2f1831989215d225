"""Gated FFN  out_proj(silu(w1 x) * w2 x)  on blockwise-FP8 GEMMs, with the
gated activation fused into the quantizer that feeds out_proj.

("add FSDP and TP tests for Float8BlockwiseLinear", summary: the ToyModel FFN
with layers w1, w2 and out_proj, w1 and w2 both reading x; "[not for land]
float8 blockwise scaling training prototype using deep_gemm", description:
casting to FP8 as separate torch kernels costs extra passes over memory.)

Compared with three Float8BlockwiseLinear layers, the module saves passes
over HBM on both sides of the activation:

  forward   x is quantized once (rows for the GEMM, columns for the wgrad)
            instead of once per layer; w1 and w2 are quantized into one
            stacked [2H, D] operand, so  [a | b] = x [w1; w2]^T  is one GEMM;
            h = silu(a) * b is computed, rounded once to bf16 and quantized
            (rows and transposed columns) in one kernel, and never stored
  backward  da = dh * b * silu'(a) and db = dh * silu(a) are computed,
            rounded once and quantized (rows and columns of [da | db]) in
            one kernel from the saved [a | b] and dh, and never stored;
            dx = [da | db] . [w1; w2] is one GEMM whose contraction over 2H
            sums both branches in fp32; [dw1; dw2] is one wgrad GEMM

hidden must be a multiple of 512 (w2's block scales start 16-byte aligned
inside the stacked scale tensor), dim and the token count multiples of 128.
"""

import torch

from . import binding as _b
from .linear import _check_dims, _quant_rows_cols


def _quant_weight_into(w, q, s, qt, st):
    """128x128 codes of w [N, K] in both layouts, written into views."""
    _b.bs_quant_128x128_both(w, q, s, qt, st)


class _GatedFFNFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x2, w1, w2, wo):
        M, D = x2.shape
        H = w1.shape[0]
        hb = H // 128
        dev = x2.device
        qx, sx, qxt, sxt = _quant_rows_cols(x2)
        # w1 and w2 stacked: rows [0, H) and [H, 2H) of the forward operand,
        # columns [0, H) and [H, 2H) of the transposed (dgrad) operand
        q12 = torch.empty((2 * H, D), dtype=torch.uint8, device=dev)
        s12 = _b.empty_scales(D // 128, 2 * hb, dev)
        q12t = torch.empty((1, D, 2 * H), dtype=torch.uint8, device=dev)
        s12t = torch.empty((1, 2 * hb, _b._round4(D // 128)), dtype=torch.float32, device=dev)
        _quant_weight_into(w1, q12[:H], s12[:, :hb], q12t[:, :, :H], s12t[:, :hb])
        _quant_weight_into(w2, q12[H:], s12[:, hb:], q12t[:, :, H:], s12t[:, hb:])
        ab = _b.bs_scaled_mm(qx, sx, q12, s12, _b.BS_SCALE_128X128, out_dtype=torch.bfloat16)  # [a | b]
        # h = silu(a) * b, quantized for out_proj (rows) and its wgrad (columns)
        qh = torch.empty((M, H), dtype=torch.uint8, device=dev)
        sh = _b.empty_scales(hb, M, dev)
        qht = torch.empty((H, M), dtype=torch.uint8, device=dev)
        sht = _b.empty_scales(M // 128, H, dev)
        _b.bs_swiglu_quant_1x128(ab[:, :H], ab[:, H:], None, qh, sh, qht, sht)
        qo = torch.empty((D, H), dtype=torch.uint8, device=dev)
        so = _b.empty_scales(hb, D // 128, dev)
        qot = torch.empty((1, H, D), dtype=torch.uint8, device=dev)
        sot = torch.empty((1, D // 128, _b._round4(hb)), dtype=torch.float32, device=dev)
        _quant_weight_into(wo, qo, so, qot, sot)
        y = _b.bs_scaled_mm(qh, sh, qo, so, _b.BS_SCALE_128X128, out_dtype=torch.bfloat16)
        ctx.save_for_backward(ab, qxt, sxt, q12t, s12t, qht, sht, qot, sot)
        return y

    @staticmethod
    def backward(ctx, dy):
        ab, qxt, sxt, q12t, s12t, qht, sht, qot, sot = ctx.saved_tensors
        H = ab.shape[1] // 2
        dy = dy.to(torch.bfloat16).contiguous()
        qg, sg, qgt, sgt = _quant_rows_cols(dy)
        M = ab.shape[0]
        dev = ab.device
        dh = _b.bs_scaled_mm(qg, sg, qot[0], sot[0], _b.BS_SCALE_128X128, out_dtype=torch.bfloat16)
        dwo = _b.bs_scaled_mm_ws(qgt, sgt, qht, sht, _b.BS_SCALE_1X128, out_dtype=torch.bfloat16)
        # [da | db] (the activation's backward) quantized in one pass over a, b, dh
        qd = torch.empty((M, 2 * H), dtype=torch.uint8, device=dev)
        sd = _b.empty_scales(2 * H // 128, M, dev)
        qdt = torch.empty((2 * H, M), dtype=torch.uint8, device=dev)
        sdt = _b.empty_scales(M // 128, 2 * H, dev)
        _b.bs_swiglu_bwd_quant_1x128(ab[:, :H], ab[:, H:], dh, None, qd, sd, qdt, sdt)
        dx = dw1 = dw2 = None
        if ctx.needs_input_grad[0]:
            dx = _b.bs_scaled_mm(qd, sd, q12t[0], s12t[0], _b.BS_SCALE_128X128, out_dtype=torch.bfloat16)
        if ctx.needs_input_grad[1] or ctx.needs_input_grad[2]:
            dw12 = _b.bs_scaled_mm_ws(qdt, sdt, qxt, sxt, _b.BS_SCALE_1X128, out_dtype=torch.bfloat16)
            dw1, dw2 = dw12[:H], dw12[H:]
        return dx, dw1, dw2, dwo


def float8_blockwise_gated_ffn(x, w1, w2, out_proj):
    """y = (silu(x w1^T) * (x w2^T)) out_proj^T with every GEMM in blockwise
    FP8.  x [..., D]; w1, w2 [H, D]; out_proj [D, H]; all contiguous bf16
    GPU tensors."""
    for name, t in (("x", x), ("w1", w1), ("w2", w2), ("out_proj", out_proj)):
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bfloat16, got {t.dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous (row-major); pass a contiguous tensor")
    if w1.dim() != 2 or w2.shape != w1.shape:
        raise ValueError(f"w1 and w2 must both be [H, D], got {tuple(w1.shape)} and {tuple(w2.shape)}")
    H, D = w1.shape
    if tuple(out_proj.shape) != (D, H):
        raise ValueError(f"out_proj must be [{D}, {H}], got {tuple(out_proj.shape)}")
    if x.shape[-1] != D:
        raise ValueError(f"x has {x.shape[-1]} features, the FFN expects {D}")
    if H % 512 != 0:
        raise ValueError(f"hidden = {H} must be a multiple of 512 (w2's block scales sit 16-byte aligned "
                         "after w1's in the stacked operand)")
    lead = x.shape[:-1]
    M = x.numel() // D if D else 0
    _check_dims(M, D, H)
    if not all(t.is_cuda for t in (x, w1, w2, out_proj)):
        raise ValueError("x and the weights must be GPU tensors")
    y = _GatedFFNFn.apply(x.view(M, D), w1, w2, out_proj)
    return y.view(*lead, D)


class Float8BlockwiseGatedFFN(torch.nn.Module):
    """Bias-free gated FFN  out_proj(silu(w1 x) * w2 x)  in blockwise FP8,
    with parameters named like the ToyModel FFN (w1, w2, out_proj; each an
    [out, in] weight)."""

    def __init__(self, dim, hidden, device=None, dtype=torch.bfloat16):
        super().__init__()
        if hidden % 512 != 0:
            raise ValueError(f"hidden = {hidden} must be a multiple of 512")
        _check_dims(128, dim, hidden)
        self.dim, self.hidden = dim, hidden
        self.w1 = torch.nn.Parameter(torch.empty((hidden, dim), device=device, dtype=dtype))
        self.w2 = torch.nn.Parameter(torch.empty((hidden, dim), device=device, dtype=dtype))
        self.out_proj = torch.nn.Parameter(torch.empty((dim, hidden), device=device, dtype=dtype))
        for w in (self.w1, self.w2, self.out_proj):
            torch.nn.init.kaiming_uniform_(w, a=5 ** 0.5)

    @classmethod
    def from_linears(cls, w1, w2, out_proj):
        """Same weights as three bias-free linear layers (nn.Linear or
        Float8BlockwiseLinear) w1, w2 [dim -> hidden] and out_proj [hidden -> dim]."""
        for lin in (w1, w2, out_proj):
            if getattr(lin, "bias", None) is not None:
                raise ValueError("the gated FFN has no biases")
        hidden, dim = w1.weight.shape
        m = cls(dim, hidden, device=w1.weight.device)
        with torch.no_grad():
            m.w1.copy_(w1.weight.to(torch.bfloat16))
            m.w2.copy_(w2.weight.to(torch.bfloat16))
            m.out_proj.copy_(out_proj.weight.to(torch.bfloat16))
        return m

    def forward(self, x):
        return float8_blockwise_gated_ffn(x, self.w1, self.w2, self.out_proj)

    def extra_repr(self):
        return f"dim={self.dim}, hidden={self.hidden}, blockwise fp8, fused gated activation"
