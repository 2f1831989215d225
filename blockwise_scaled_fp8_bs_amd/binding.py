"""Thin Python binding of the C ABI (include/bs.h), same names, torch tensors in.

Argument marshalling only: shapes, strides and data pointers of torch tensors
are passed to the HIP library, whose kernels do all of the work; torch
provides device memory and the current stream.  Layout rules are checked here
and again in the library; a tensor in the wrong layout raises ``ValueError``
instead of being copied ("add FSDP and TP tests for Float8BlockwiseLinear",
review thread on the layout assertions: fail loudly, never silently copy).

Tensor conventions (all on one GPU):

* bf16 input ``x``: torch.bfloat16, 2-D (or 3-D for expert weights), unit
  stride along the last dimension; its row stride is the ``ld``.
* e4m3 codes: torch.uint8 with the same convention.
* scales: torch.float32, 2-D ``[K/128, ld]`` (3-D ``[G, K/128, ld]`` per
  expert): the contraction-block index is the outer index ("K-major"), the
  row stride is ``ld_s`` (a multiple of 4); entries past the logical count
  are padding and are never written.
"""

import ctypes

import torch

from . import _lib

BS_SCALE_1X128 = 4
BS_SCALE_128X128 = 5
BS_OUT_BF16 = 0
BS_OUT_F32 = 1
BS_GROUP_M = 0
BS_GROUP_K = 1


class BsError(RuntimeError):
    """A nonzero bs_status from the library."""

    def __init__(self, status, fn):
        lib = _lib.load()
        self.status = status
        self.name = lib.bs_status_string(status).decode()
        super().__init__(f"{fn} failed with {self.name}: {lib.bs_last_error().decode()}")


def _check(status, fn):
    if status != 0:
        raise BsError(status, fn)


def _ptr(t):
    # tensors without elements may have no storage: pass NULL (the ABI allows
    # NULL exactly for tensors with no elements)
    return None if t is None or t.data_ptr() == 0 else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _require(cond, msg):
    if not cond:
        raise ValueError(msg)


def _mat(t, name, dtype, dims=2):
    _require(t is not None, f"{name} is required")
    _require(t.dtype == dtype, f"{name} must be {dtype}, got {t.dtype}")
    _require(t.dim() == dims, f"{name} must be {dims}-D, got shape {tuple(t.shape)}")
    _require(t.is_cuda, f"{name} must be a GPU tensor")
    _require(t.shape[-1] <= 1 or t.stride(-1) == 1,
             f"{name} must have unit stride along its last dimension (row-major); got strides {t.stride()}"
             " -- pass a tensor in the required layout instead of relying on a copy")
    return t


def _ld(t):
    return t.stride(-2)


def _scale(t, name, nkb, count):
    _mat(t, name, torch.float32)
    _require(t.shape[0] == nkb, f"{name} must have {nkb} rows (one per 128-block of the contraction), got {t.shape[0]}")
    _require(t.shape[1] >= count, f"{name} must have at least {count} columns (K-major [K/128][>= {count}])")
    return t.stride(0)


def _round4(n):
    return (n + 3) // 4 * 4


def empty_scales(nkb, count, device, pad=0):
    """Allocate a K-major scale tensor [nkb, roundup4(count) + pad] (float32)."""
    return torch.empty((nkb, _round4(count) + pad), dtype=torch.float32, device=device)


# ----------------------------------------------------------------------------
# quantizers
# ----------------------------------------------------------------------------

def bs_quant_1x128(x, q_row=None, s_row=None, q_col=None, s_col=None, stream=None):
    """1x128 quantizer (rows and/or transposed columns) in one pass.

    x [R, C] bf16; q_row [R, C] uint8 with s_row [C/128, >= R];
    q_col [C, R] uint8 with s_col [R/128, >= C].
    """
    _check(_lib.load().bs_quant_1x128(*_quant_1x128_args(x, q_row, s_row, q_col, s_col), _stream(stream)),
           "bs_quant_1x128")


def _quant_1x128_args(x, q_row, s_row, q_col, s_col):
    """Checked C arguments of bs_quant_1x128 (without the stream)."""
    _mat(x, "x", torch.bfloat16)
    R, C = x.shape
    args = [_ptr(x), R, C, _ld(x)]
    if q_row is not None or s_row is not None:
        _mat(q_row, "q_row", torch.uint8)
        _require(tuple(q_row.shape) == (R, C), f"q_row must be [{R}, {C}]")
        ld_sr = _scale(s_row, "s_row", C // 128, R)
        args += [_ptr(q_row), _ld(q_row), _ptr(s_row), ld_sr]
    else:
        args += [None, 0, None, 0]
    if q_col is not None or s_col is not None:
        _mat(q_col, "q_col", torch.uint8)
        _require(tuple(q_col.shape) == (C, R), f"q_col must be the transpose [{C}, {R}]")
        ld_sc = _scale(s_col, "s_col", R // 128, C)
        args += [_ptr(q_col), _ld(q_col), _ptr(s_col), ld_sc]
    else:
        args += [None, 0, None, 0]
    return args


def bs_swiglu_quant_1x128(a, b, h=None, q_row=None, s_row=None, q_col=None, s_col=None, stream=None):
    """Gated activation h = silu(a) * b (rounded once to bf16) quantized 1x128
    along rows and/or transposed columns in one pass; h is written if given.

    a, b [R, C] bf16; h [R, C] bf16 or None; outputs as in bs_quant_1x128.
    """
    _mat(a, "a", torch.bfloat16)
    _mat(b, "b", torch.bfloat16)
    R, C = a.shape
    _require(tuple(b.shape) == (R, C), f"b must be [{R}, {C}] like a")
    args = [_ptr(a), _ptr(b), R, C, _ld(a), _ld(b)]
    if h is not None:
        _mat(h, "h", torch.bfloat16)
        _require(tuple(h.shape) == (R, C), f"h must be [{R}, {C}]")
        args += [_ptr(h), _ld(h)]
    else:
        args += [None, 0]
    if q_row is not None or s_row is not None:
        _mat(q_row, "q_row", torch.uint8)
        _require(tuple(q_row.shape) == (R, C), f"q_row must be [{R}, {C}]")
        ld_sr = _scale(s_row, "s_row", C // 128, R)
        args += [_ptr(q_row), _ld(q_row), _ptr(s_row), ld_sr]
    else:
        args += [None, 0, None, 0]
    if q_col is not None or s_col is not None:
        _mat(q_col, "q_col", torch.uint8)
        _require(tuple(q_col.shape) == (C, R), f"q_col must be the transpose [{C}, {R}]")
        ld_sc = _scale(s_col, "s_col", R // 128, C)
        args += [_ptr(q_col), _ld(q_col), _ptr(s_col), ld_sc]
    else:
        args += [None, 0, None, 0]
    _check(_lib.load().bs_swiglu_quant_1x128(*args, _stream(stream)), "bs_swiglu_quant_1x128")


def bs_swiglu_bwd_quant_1x128(a, b, dh, dab=None, q_row=None, s_row=None, q_col=None, s_col=None, stream=None):
    """Backward of h = silu(a) * b fused with the 1x128 quantizer: quantizes
    the [R, 2C] matrix [da | db] (da = dh b silu'(a), db = dh silu(a), each
    rounded once to bf16) along rows and/or transposed columns.

    a, b, dh [R, C] bf16; dab [R, 2C] bf16 or None; q_row [R, 2C] uint8 with
    s_row [2C/128, >= R]; q_col [2C, R] uint8 with s_col [R/128, >= 2C].
    """
    for t, name in ((a, "a"), (b, "b"), (dh, "dh")):
        _mat(t, name, torch.bfloat16)
    R, C = a.shape
    _require(tuple(b.shape) == (R, C) and tuple(dh.shape) == (R, C), f"b and dh must be [{R}, {C}] like a")
    args = [_ptr(a), _ptr(b), _ptr(dh), R, C, _ld(a), _ld(b), _ld(dh)]
    if dab is not None:
        _mat(dab, "dab", torch.bfloat16)
        _require(tuple(dab.shape) == (R, 2 * C), f"dab must be [{R}, {2 * C}]")
        args += [_ptr(dab), _ld(dab)]
    else:
        args += [None, 0]
    if q_row is not None or s_row is not None:
        _mat(q_row, "q_row", torch.uint8)
        _require(tuple(q_row.shape) == (R, 2 * C), f"q_row must be [{R}, {2 * C}]")
        ld_sr = _scale(s_row, "s_row", 2 * C // 128, R)
        args += [_ptr(q_row), _ld(q_row), _ptr(s_row), ld_sr]
    else:
        args += [None, 0, None, 0]
    if q_col is not None or s_col is not None:
        _mat(q_col, "q_col", torch.uint8)
        _require(tuple(q_col.shape) == (2 * C, R), f"q_col must be the transpose [{2 * C}, {R}]")
        ld_sc = _scale(s_col, "s_col", R // 128, 2 * C)
        args += [_ptr(q_col), _ld(q_col), _ptr(s_col), ld_sc]
    else:
        args += [None, 0, None, 0]
    _check(_lib.load().bs_swiglu_bwd_quant_1x128(*args, _stream(stream)), "bs_swiglu_bwd_quant_1x128")


def empty_mx_scales(nchunks, count, device, pad=0):
    """Allocate a K-major MX scale tensor [nchunks, roundup16(count) + pad] of E8M0 bytes (uint8)."""
    return torch.empty((nchunks, (count + 15) // 16 * 16 + pad), dtype=torch.uint8, device=device)


def _mx_scale(t, name, nch, count):
    _mat(t, name, torch.uint8)
    _require(t.shape[0] == nch, f"{name} must have {nch} rows (one per 32-block of the contraction), got {t.shape[0]}")
    _require(t.shape[1] >= count, f"{name} must have at least {count} columns (K-major [K/32][>= {count}] bytes)")
    return t.stride(0)


def bs_mx_quant_1x32(x, q_row=None, s_row=None, q_col=None, s_col=None, stream=None):
    """MXFP8 quantizer (32-element blocks, E8M0 scale bytes), rows and/or
    transposed columns in one pass.

    x [R, C] bf16; q_row [R, C] uint8 with s_row [C/32, >= R] uint8;
    q_col [C, R] uint8 with s_col [R/32, >= C] uint8.
    """
    _mat(x, "x", torch.bfloat16)
    R, C = x.shape
    args = [_ptr(x), R, C, _ld(x)]
    if q_row is not None or s_row is not None:
        _mat(q_row, "q_row", torch.uint8)
        _require(tuple(q_row.shape) == (R, C), f"q_row must be [{R}, {C}]")
        args += [_ptr(q_row), _ld(q_row), _ptr(s_row), _mx_scale(s_row, "s_row", C // 32, R)]
    else:
        args += [None, 0, None, 0]
    if q_col is not None or s_col is not None:
        _mat(q_col, "q_col", torch.uint8)
        _require(tuple(q_col.shape) == (C, R), f"q_col must be the transpose [{C}, {R}]")
        args += [_ptr(q_col), _ld(q_col), _ptr(s_col), _mx_scale(s_col, "s_col", R // 32, C)]
    else:
        args += [None, 0, None, 0]
    _check(_lib.load().bs_mx_quant_1x32(*args, _stream(stream)), "bs_mx_quant_1x32")


def bs_mx_scaled_mm(a, sa, b, sb, out=None, out_dtype=torch.bfloat16, stream=None):
    """D[M, N] = A [M, K] . B [N, K]^T with MX (E8M0, 32-element) scales
    sa [K/32, >= M] and sb [K/32, >= N] (uint8).  Returns ``out``."""
    _mat(a, "a", torch.uint8)
    _mat(b, "b", torch.uint8)
    M, K = a.shape
    N, Kb = b.shape
    _require(K == Kb, f"a is [M, {K}] but b is [N, {Kb}]: both must be contiguous along the same K")
    ld_sa = _mx_scale(sa, "sa", K // 32, M)
    ld_sb = _mx_scale(sb, "sb", K // 32, N)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    _mat(out, "out", out.dtype)
    _require(tuple(out.shape) == (M, N), f"out must be [{M}, {N}]")
    dt = {torch.bfloat16: BS_OUT_BF16, torch.float32: BS_OUT_F32}.get(out.dtype)
    _require(dt is not None, "out must be bfloat16 or float32")
    _check(_lib.load().bs_mx_scaled_mm(M, N, K, _ptr(a), _ld(a), _ptr(sa), ld_sa, _ptr(b), _ld(b), _ptr(sb), ld_sb,
                                       _ptr(out), _ld(out), dt, _stream(stream)),
           "bs_mx_scaled_mm")
    return out


def bs_mx_grouped_scaled_mm(mode, group_end, a, sa, b, sb, out=None, out_dtype=torch.bfloat16, stream=None):
    """Grouped (MoE) MX GEMM, group semantics as ``bs_grouped_scaled_mm``.

    BS_GROUP_M: a [M, K], sa [K/32, >= M]; b [G, N, K]; sb [G, K/32, >= N]
      (uint8, any 16-byte multiple stride between experts); out [M, N].
    BS_GROUP_K: a [M, T], sa [T/32, >= M]; b [N, T], sb [T/32, >= N];
      out [G, M, N]; group g contracts over tokens [end_{g-1}, end_g), ends
      multiples of 128.
    group_end: int32 GPU tensor [G] of cumulative ends.
    """
    _require(group_end is not None and group_end.dtype == torch.int32 and group_end.is_cuda
             and group_end.dim() == 1, "group_end must be a 1-D int32 GPU tensor")
    G = group_end.shape[0]
    _require(group_end.stride(0) == 1 or G <= 1, "group_end must be contiguous")
    _mat(a, "a", torch.uint8)
    M, K = a.shape
    ld_sa = _mx_scale(sa, "sa", K // 32, M)
    dt_map = {torch.bfloat16: BS_OUT_BF16, torch.float32: BS_OUT_F32}
    if mode == BS_GROUP_M:
        _mat(b, "b", torch.uint8, 3)
        _require(b.shape[0] == G and b.shape[2] == K, f"b must be [{G}, N, {K}]")
        N = b.shape[1]
        _mat(sb, "sb", torch.uint8, 3)
        _require(sb.shape[0] == G and sb.shape[1] == K // 32 and sb.shape[2] >= N,
                 f"sb must be [{G}, {K // 32}, >= {N}]")
        if out is None:
            out = torch.empty((M, N), dtype=out_dtype, device=a.device)
        _mat(out, "out", out.dtype)
        _require(tuple(out.shape) == (M, N), f"out must be [{M}, {N}]")
        args = [mode, G, M, N, K, _ptr(group_end), _ptr(a), _ld(a), _ptr(sa), ld_sa,
                _ptr(b), b.stride(0), b.stride(1), _ptr(sb), sb.stride(0), sb.stride(1),
                _ptr(out), 0, _ld(out)]
    else:
        _mat(b, "b", torch.uint8)
        N, Kb = b.shape
        _require(Kb == K, f"b must be [N, {K}] (tokens contiguous)")
        ld_sb = _mx_scale(sb, "sb", K // 32, N)
        if out is None:
            out = torch.empty((G, M, N), dtype=out_dtype, device=a.device)
        _mat(out, "out", out.dtype, 3)
        _require(tuple(out.shape) == (G, M, N), f"out must be [{G}, {M}, {N}]")
        args = [mode, G, M, N, K, _ptr(group_end), _ptr(a), _ld(a), _ptr(sa), ld_sa,
                _ptr(b), 0, _ld(b), _ptr(sb), 0, ld_sb,
                _ptr(out), out.stride(0), out.stride(1)]
    dt = dt_map.get(out.dtype)
    _require(dt is not None, "out must be bfloat16 or float32")
    _check(_lib.load().bs_mx_grouped_scaled_mm(*args, dt, _stream(stream)), "bs_mx_grouped_scaled_mm")
    return out


def bs_quant_128x128(x, q, s, stream=None):
    """128x128 quantizer: x [R, C] bf16 -> q [R, C] uint8, s [C/128, >= R/128]."""
    _mat(x, "x", torch.bfloat16)
    _mat(q, "q", torch.uint8)
    R, C = x.shape
    _require(tuple(q.shape) == (R, C), f"q must be [{R}, {C}]")
    ld_s = _scale(s, "s", C // 128, R // 128)
    _check(_lib.load().bs_quant_128x128(_ptr(x), R, C, _ld(x), _ptr(q), _ld(q), _ptr(s), ld_s, _stream(stream)),
           "bs_quant_128x128")


def bs_quant_3d_colwise(x, q, s, stream=None):
    """3-D colwise quantizer: x [G, R, C] bf16 -> q [G, C, R] uint8,
    s [G, R/128, >= C/128] (K-major for the transposed operand)."""
    _mat(x, "x", torch.bfloat16, 3)
    _mat(q, "q", torch.uint8, 3)
    _mat(s, "s", torch.float32, 3)
    G, R, C = x.shape
    _require(tuple(q.shape) == (G, C, R), f"q must be [{G}, {C}, {R}]")
    _require(s.shape[0] == G and s.shape[1] == R // 128 and s.shape[2] >= C // 128,
             f"s must be [{G}, {R // 128}, >= {C // 128}]")
    ld_s = s.stride(1)
    _check(_lib.load().bs_quant_3d_colwise(_ptr(x), G, R, C, x.stride(0), _ld(x), _ptr(q), q.stride(0), _ld(q),
                                           _ptr(s), s.stride(0), ld_s, _stream(stream)),
           "bs_quant_3d_colwise")


def bs_quant_128x128_both(x, q, s, qt, st, stream=None):
    """128x128 quantizer writing both weight layouts from one read of x.

    x [G, R, C] bf16 (or [R, C] for G = 1);
    q [G*R, C] uint8 with s [C/128, >= G*R/128]: the stacked forward layout;
    qt [G, C, R] uint8 with st [G, R/128, >= C/128]: the transposed (dgrad) layout.
    """
    _check(_lib.load().bs_quant_128x128_both(*_quant_128x128_both_args(x, q, s, qt, st), _stream(stream)),
           "bs_quant_128x128_both")


def _quant_128x128_both_args(x, q, s, qt, st):
    """Checked C arguments of bs_quant_128x128_both (without the stream)."""
    if x is not None and x.dim() == 2:
        x = x.unsqueeze(0)
    _mat(x, "x", torch.bfloat16, 3)
    _mat(q, "q", torch.uint8)
    _mat(qt, "qt", torch.uint8, 3)
    _mat(st, "st", torch.float32, 3)
    G, R, C = x.shape
    _require(tuple(q.shape) == (G * R, C), f"q must be [{G * R}, {C}] (the experts stacked)")
    ld_s = _scale(s, "s", C // 128, G * R // 128)
    _require(tuple(qt.shape) == (G, C, R), f"qt must be [{G}, {C}, {R}]")
    _require(st.shape[0] == G and st.shape[1] == R // 128 and st.shape[2] >= C // 128,
             f"st must be [{G}, {R // 128}, >= {C // 128}]")
    return [_ptr(x), G, R, C, x.stride(0), _ld(x), _ptr(q), _ld(q), _ptr(s), ld_s,
            _ptr(qt), qt.stride(0), _ld(qt), _ptr(st), st.stride(0), st.stride(1)]


def bs_quant_fwd_operands(x, q_row, s_row, q_col, s_col, w, qw, sw, qwt, swt, stream=None):
    """bs_quant_1x128 of the activation x (rows and transposed columns, all
    four outputs required) and bs_quant_128x128_both of the weights w in one
    launch; arguments as in those two calls.  Same results, byte for byte."""
    _require(all(t is not None for t in (q_row, s_row, q_col, s_col)),
             "q_row, s_row, q_col and s_col are all required")
    _check(_lib.load().bs_quant_fwd_operands(*_quant_1x128_args(x, q_row, s_row, q_col, s_col),
                                             *_quant_128x128_both_args(w, qw, sw, qwt, swt), _stream(stream)),
           "bs_quant_fwd_operands")


# ----------------------------------------------------------------------------
# GEMMs
# ----------------------------------------------------------------------------

def bs_scaled_mm(a, sa, b, sb, b_kind, out=None, out_dtype=torch.bfloat16, stream=None):
    """D[M, N] = blockwise-scaled A [M, K] . B [N, K]^T.

    sa [K/128, >= M] (1x128); sb [K/128, >= N/128] for BS_SCALE_128X128 or
    [K/128, >= N] for BS_SCALE_1X128.  Returns ``out`` ([M, N], bf16 or fp32).
    """
    _mat(a, "a", torch.uint8)
    _mat(b, "b", torch.uint8)
    M, K = a.shape
    N, Kb = b.shape
    _require(K == Kb, f"a is [M, {K}] but b is [N, {Kb}]: both must be contiguous along the same K")
    ld_sa = _scale(sa, "sa", K // 128, M)
    ld_sb = _scale(sb, "sb", K // 128, N if b_kind == BS_SCALE_1X128 else (N + 127) // 128)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    _mat(out, "out", out.dtype)
    _require(tuple(out.shape) == (M, N), f"out must be [{M}, {N}]")
    dt = {torch.bfloat16: BS_OUT_BF16, torch.float32: BS_OUT_F32}.get(out.dtype)
    _require(dt is not None, "out must be bfloat16 or float32")
    _check(_lib.load().bs_scaled_mm(M, N, K, _ptr(a), _ld(a), _ptr(sa), ld_sa, BS_SCALE_1X128, _ptr(b), _ld(b),
                                    _ptr(sb), ld_sb, b_kind, _ptr(out), _ld(out), dt, _stream(stream)),
           "bs_scaled_mm")
    return out


def bs_scaled_mm_quant(a, sa, b, sb, b_kind, out=None, q_row=None, s_row=None, q_col=None, s_col=None,
                       stream=None):
    """D = A . B^T (bf16) whose epilogue also writes the 1x128 quantization of
    D: q_row [M, N] uint8 with s_row [N/128, >= M], and/or q_col [N, M] with
    s_col [M/128, >= N] -- exactly what bs_quant_1x128(D, ...) writes.
    ``out`` (bf16 [M, N]) is optional; returns it (or None)."""
    _mat(a, "a", torch.uint8)
    _mat(b, "b", torch.uint8)
    M, K = a.shape
    N, Kb = b.shape
    _require(K == Kb, f"a is [M, {K}] but b is [N, {Kb}]: both must be contiguous along the same K")
    ld_sa = _scale(sa, "sa", K // 128, M)
    ld_sb = _scale(sb, "sb", K // 128, N if b_kind == BS_SCALE_1X128 else (N + 127) // 128)
    args = [M, N, K, _ptr(a), _ld(a), _ptr(sa), ld_sa, BS_SCALE_1X128, _ptr(b), _ld(b), _ptr(sb), ld_sb, b_kind]
    if out is not None:
        _mat(out, "out", torch.bfloat16)
        _require(tuple(out.shape) == (M, N), f"out must be [{M}, {N}]")
        args += [_ptr(out), _ld(out)]
    else:
        args += [None, N]
    if q_row is not None or s_row is not None:
        _mat(q_row, "q_row", torch.uint8)
        _require(tuple(q_row.shape) == (M, N), f"q_row must be [{M}, {N}]")
        args += [_ptr(q_row), _ld(q_row), _ptr(s_row), _scale(s_row, "s_row", N // 128, M)]
    else:
        args += [None, 0, None, 0]
    if q_col is not None or s_col is not None:
        _mat(q_col, "q_col", torch.uint8)
        _require(tuple(q_col.shape) == (N, M), f"q_col must be the transpose [{N}, {M}]")
        args += [_ptr(q_col), _ld(q_col), _ptr(s_col), _scale(s_col, "s_col", M // 128, N)]
    else:
        args += [None, 0, None, 0]
    _check(_lib.load().bs_scaled_mm_quant(*args, _stream(stream)), "bs_scaled_mm_quant")
    return out


def bs_scaled_mm_workspace_bytes(M, N, K, b_kind, out_dtype=torch.bfloat16):
    """Workspace bytes bs_scaled_mm_ws uses for this problem on the current device (0: no split)."""
    dt = {torch.bfloat16: BS_OUT_BF16, torch.float32: BS_OUT_F32}.get(out_dtype)
    _require(dt is not None, "out_dtype must be bfloat16 or float32")
    return int(_lib.load().bs_scaled_mm_workspace_bytes(M, N, K, b_kind, dt))


_WORKSPACES = {}


def streamk_workspace(nbytes, device=None):
    """A device workspace of at least ``nbytes`` for bs_scaled_mm_ws, cached
    per device and grown on demand (torch owns the memory).  Calls that share
    it must not overlap in time: use it from one stream."""
    device = torch.device("cuda" if device is None else device)
    if device.index is None:
        device = torch.device(device.type, torch.cuda.current_device())
    ws = _WORKSPACES.get(device)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(nbytes, 4096), dtype=torch.uint8, device=device)
        _WORKSPACES[device] = ws
    return ws


def bs_scaled_mm_ws(a, sa, b, sb, b_kind, workspace=None, out=None, out_dtype=torch.bfloat16, stream=None):
    """bs_scaled_mm with a device workspace (uint8 GPU tensor, 256-byte
    aligned) that lets the kernel split a ragged last round of tiles along
    K; see include/bs.h.  With
    ``workspace=None`` the per-device cached workspace (streamk_workspace)
    sized for this problem is used."""
    _mat(a, "a", torch.uint8)
    _mat(b, "b", torch.uint8)
    M, K = a.shape
    N, Kb = b.shape
    _require(K == Kb, f"a is [M, {K}] but b is [N, {Kb}]: both must be contiguous along the same K")
    ld_sa = _scale(sa, "sa", K // 128, M)
    ld_sb = _scale(sb, "sb", K // 128, N if b_kind == BS_SCALE_1X128 else (N + 127) // 128)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    if workspace is None:
        workspace = streamk_workspace(bs_scaled_mm_workspace_bytes(M, N, K, b_kind, out.dtype), a.device)
    _require(workspace.dtype == torch.uint8 and workspace.is_cuda and workspace.is_contiguous(),
             "workspace must be a contiguous uint8 GPU tensor")
    _mat(out, "out", out.dtype)
    _require(tuple(out.shape) == (M, N), f"out must be [{M}, {N}]")
    dt = {torch.bfloat16: BS_OUT_BF16, torch.float32: BS_OUT_F32}.get(out.dtype)
    _require(dt is not None, "out must be bfloat16 or float32")
    _check(_lib.load().bs_scaled_mm_ws(M, N, K, _ptr(a), _ld(a), _ptr(sa), ld_sa, BS_SCALE_1X128, _ptr(b), _ld(b),
                                       _ptr(sb), ld_sb, b_kind, _ptr(out), _ld(out), dt, _ptr(workspace),
                                       workspace.numel(), _stream(stream)),
           "bs_scaled_mm_ws")
    return out


def bs_grouped_scaled_mm(mode, group_end, a, sa, b, sb, b_kind, out=None, out_dtype=torch.bfloat16,
                         stream=None):
    """Grouped (MoE) scaled GEMM.

    BS_GROUP_M: a [M, K], sa [K/128, >= M]; b [G, N, K] (any stride between
      experts); sb [G, K/128, >= N/128] (any stride between experts, e.g. an
      interleaved view of one [K/128, G*N/128] scale matrix); out [M, N].
    BS_GROUP_K: a [M, T], sa [T/128, >= M]; b [N, T], sb [T/128, >= N];
      out [G, M, N]; group g contracts over tokens [end_{g-1}, end_g).
    group_end: int32 GPU tensor [G] of cumulative ends.
    """
    _require(group_end is not None and group_end.dtype == torch.int32 and group_end.is_cuda
             and group_end.dim() == 1, "group_end must be a 1-D int32 GPU tensor")
    G = group_end.shape[0]
    _require(group_end.stride(0) == 1 or G <= 1, "group_end must be contiguous")
    _mat(a, "a", torch.uint8)
    M, K = a.shape
    dt_map = {torch.bfloat16: BS_OUT_BF16, torch.float32: BS_OUT_F32}
    if mode == BS_GROUP_M:
        _mat(b, "b", torch.uint8, 3)
        _require(b.shape[0] == G and b.shape[2] == K, f"b must be [{G}, N, {K}]")
        N = b.shape[1]
        _mat(sb, "sb", torch.float32, 3)
        _require(sb.shape[0] == G and sb.shape[1] == K // 128 and sb.shape[2] >= N // 128,
                 f"sb must be [{G}, {K // 128}, >= {N // 128}]")
        ld_sa = _scale(sa, "sa", K // 128, M)
        if out is None:
            out = torch.empty((M, N), dtype=out_dtype, device=a.device)
        _mat(out, "out", out.dtype)
        _require(tuple(out.shape) == (M, N), f"out must be [{M}, {N}]")
        dt = dt_map.get(out.dtype)
        _require(dt is not None, "out must be bfloat16 or float32")
        ld_sb = sb.stride(1)
        args = [mode, G, M, N, K, _ptr(group_end), _ptr(a), _ld(a), _ptr(sa), ld_sa,
                _ptr(b), b.stride(0), b.stride(1), _ptr(sb), sb.stride(0), ld_sb, b_kind,
                _ptr(out), 0, _ld(out), dt]
    else:
        _mat(b, "b", torch.uint8)
        N, Kb = b.shape
        _require(Kb == K, f"b must be [N, {K}] (tokens contiguous)")
        ld_sa = _scale(sa, "sa", K // 128, M)
        ld_sb = _scale(sb, "sb", K // 128, N)
        if out is None:
            out = torch.empty((G, M, N), dtype=out_dtype, device=a.device)
        _mat(out, "out", out.dtype, 3)
        _require(tuple(out.shape) == (G, M, N), f"out must be [{G}, {M}, {N}]")
        dt = dt_map.get(out.dtype)
        _require(dt is not None, "out must be bfloat16 or float32")
        args = [mode, G, M, N, K, _ptr(group_end), _ptr(a), _ld(a), _ptr(sa), ld_sa,
                _ptr(b), 0, _ld(b), _ptr(sb), 0, ld_sb, b_kind,
                _ptr(out), out.stride(0), out.stride(1), dt]
    _check(_lib.load().bs_grouped_scaled_mm(*args, _stream(stream)), "bs_grouped_scaled_mm")
    return out


# ----------------------------------------------------------------------------
# diagnostics
# ----------------------------------------------------------------------------

def bs_diag_e4m3_census(device="cuda", stream=None):
    """(min_bits, max_bits, counts) per e4m3 code over all |y| <= 464 (CPU tensors)."""
    mn = torch.empty(256, dtype=torch.int32, device=device)
    mx = torch.empty(256, dtype=torch.int32, device=device)
    cnt = torch.empty(256, dtype=torch.int64, device=device)
    _check(_lib.load().bs_diag_e4m3_census(_ptr(mn), _ptr(mx), _ptr(cnt), _stream(stream)), "bs_diag_e4m3_census")
    torch.cuda.synchronize()
    return mn.cpu(), mx.cpu(), cnt.cpu()


def bs_diag_division(device="cuda", stream=None):
    """Counts of the quantizers' division vs IEEE (see include/bs.h):
    dict with pairs, scale_mismatch, code_mismatch, quotient_mismatch,
    tiny_quotient_mismatch."""
    res = torch.zeros(5, dtype=torch.int64, device=device)
    _check(_lib.load().bs_diag_division(_ptr(res), _stream(stream)), "bs_diag_division")
    torch.cuda.synchronize()
    v = [int(t) for t in res.cpu().tolist()]
    return dict(zip(["pairs", "scale_mismatch", "code_mismatch", "quotient_mismatch",
                     "tiny_quotient_mismatch"], v))


def bs_diag_stream(src, n_read, dst, n_write, stream=None):
    """Streaming reference: read n_read bytes of ``src`` and write n_write
    bytes of ``dst`` (uint8 GPU tensors) with the quantizers' access pattern."""
    _require(src.is_cuda and dst.is_cuda and src.dtype == torch.uint8 and dst.dtype == torch.uint8,
             "src and dst must be uint8 GPU tensors")
    _require(src.numel() >= n_read and dst.numel() >= n_write, "buffers too small")
    _check(_lib.load().bs_diag_stream(_ptr(src), n_read, _ptr(dst), n_write, _stream(stream)), "bs_diag_stream")
