"""Blockwise e4m3 quantizers, CPU oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definition followed (pages: "[not for land] float8 blockwise scaling training
prototype using deep_gemm", description -- activations scaled per 1x128 and
weights per 128x128 block; "add FSDP and TP tests for Float8BlockwiseLinear",
review thread on the kernel module -- ``EPS = 1e-12`` and fp32 ("_32F")
block scales).  For every block of 128 (1x128) or 128x128 (128x128) bf16
values ``x``:

1. ``amax = max |x|`` over the block (exact: |x| of a bf16 is a bf16);
2. ``amax_c = max(amax, EPS)`` with ``EPS`` the float32 nearest to 1e-12;
3. ``s = fl32(amax_c / 448)``, one IEEE float32 division, round to nearest
   even -- no power-of-two rounding of the scale;
4. ``y = fl32(x / s)`` for every element, IEEE float32 division (not
   ``x * (1/s)``, which differs in the last bit for some inputs);
5. ``q = e4m3(clamp(y, -448, 448))``, round to nearest even, sign kept.

Where the pages are silent these are the readings taken: the scale is
amax/448 in float32, EPS floors amax (a zero block gets a tiny positive scale
and all-zero codes), the element is divided by the stored scale, and the
quotient is rounded twice (to float32, then to e4m3).

Operand orientation of the outputs.  Every quantizer returns ``(q, s)`` in
the orientation of the GEMM operand it feeds: ``q`` has shape
``[rows, K]`` with K the contraction dimension, and ``s`` has one entry per
(row, 128-block of K) for 1x128 or per (128-block of rows, 128-block of K)
for 128x128.  These are logical arrays; the physical K-major layout of the
scales is a property of the library's boundary, not of the definition.

Two forms: ``*_scalar`` walks blocks and elements in Python loops (small
inputs only); the vectorized functions apply the same five steps with numpy
array operations on row chunks.
"""

import numpy as np

from . import e4m3

EPS = np.float32(1e-12)  # floor on amax; the kernel module's EPS = 1e-12
E4M3_MAX = np.float32(448.0)
BLOCK = 128


# ----------------------------------------------------------------------------
# bf16 <-> float32 (bf16 tensors travel as their uint16 bit patterns)
# ----------------------------------------------------------------------------

def bf16_bits_to_f32(bits):
    """Widen bf16 bit patterns (uint16) to float32; exact."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _check_finite(x):
    if not np.all(np.isfinite(x)):
        raise ValueError("oracle quantizer: inputs must be finite (bf16 Inf/NaN is outside the method)")


def _check_dims(*dims):
    for d in dims:
        if d % BLOCK:
            raise ValueError("oracle quantizer: every blocked dimension must be a multiple of 128")


# ----------------------------------------------------------------------------
# scalar form
# ----------------------------------------------------------------------------

def quantize_block_scalar(values):
    """Quantize one block given as a flat list of float32 values.

    Returns (codes as a list of ints, scale as np.float32).  Steps 1-5 of the
    module docstring, one element at a time.
    """
    amax = np.float32(0.0)
    for v in values:
        a = np.float32(abs(np.float32(v)))
        if a > amax:
            amax = a
    if amax < EPS:
        amax = EPS
    s = np.float32(amax / E4M3_MAX)          # float32 / float32 -> float32, RNE
    codes = []
    for v in values:
        y = np.float32(np.float32(v) / s)    # correctly rounded float32 quotient
        if y > E4M3_MAX:
            y = E4M3_MAX
        if y < -E4M3_MAX:
            y = -E4M3_MAX
        codes.append(e4m3.encode_scalar(y))
    return codes, s


def quant_1x128_rowwise_scalar(x_bits):
    """1x128 blocks along the last axis of a [R, C] bf16 array (scalar loops).

    Returns q uint8 [R, C] and s float32 [R, C/128].
    """
    x = bf16_bits_to_f32(x_bits)
    R, C = x.shape
    _check_dims(C)
    _check_finite(x)
    q = np.zeros((R, C), dtype=np.uint8)
    s = np.zeros((R, C // BLOCK), dtype=np.float32)
    for r in range(R):
        for kb in range(C // BLOCK):
            codes, sc = quantize_block_scalar(list(x[r, kb * BLOCK:(kb + 1) * BLOCK]))
            q[r, kb * BLOCK:(kb + 1) * BLOCK] = codes
            s[r, kb] = sc
    return q, s


def quant_1x128_colwise_scalar(x_bits):
    """Blocks of 128 consecutive rows of one column, written transposed.

    Returns q uint8 [C, R] (q[c, r] is the code of x[r, c]) and s float32
    [C, R/128] (s[c, rb] is the scale of column c, rows rb*128 .. +127).
    """
    x = bf16_bits_to_f32(x_bits)
    R, C = x.shape
    _check_dims(R)
    _check_finite(x)
    q = np.zeros((C, R), dtype=np.uint8)
    s = np.zeros((C, R // BLOCK), dtype=np.float32)
    for c in range(C):
        for rb in range(R // BLOCK):
            codes, sc = quantize_block_scalar(list(x[rb * BLOCK:(rb + 1) * BLOCK, c]))
            q[c, rb * BLOCK:(rb + 1) * BLOCK] = codes
            s[c, rb] = sc
    return q, s


def quant_128x128_scalar(x_bits):
    """128x128 tiles of a [R, C] bf16 array (scalar loops).

    Returns q uint8 [R, C] and s float32 [R/128, C/128].
    """
    x = bf16_bits_to_f32(x_bits)
    R, C = x.shape
    _check_dims(R, C)
    _check_finite(x)
    q = np.zeros((R, C), dtype=np.uint8)
    s = np.zeros((R // BLOCK, C // BLOCK), dtype=np.float32)
    for rb in range(R // BLOCK):
        for cb in range(C // BLOCK):
            tile = x[rb * BLOCK:(rb + 1) * BLOCK, cb * BLOCK:(cb + 1) * BLOCK]
            codes, sc = quantize_block_scalar(list(tile.reshape(-1)))
            q[rb * BLOCK:(rb + 1) * BLOCK, cb * BLOCK:(cb + 1) * BLOCK] = np.array(
                codes, dtype=np.uint8).reshape(BLOCK, BLOCK)
            s[rb, cb] = sc
    return q, s


# ----------------------------------------------------------------------------
# vectorized form (same five steps on whole arrays)
# ----------------------------------------------------------------------------

def _scale_from_amax(amax):
    amax = np.maximum(amax.astype(np.float32), EPS)
    return (amax / E4M3_MAX).astype(np.float32)


def _encode_quotient(x, s):
    y = (x / s).astype(np.float32)  # IEEE float32 division, broadcast
    y = np.clip(y, -E4M3_MAX, E4M3_MAX)
    return e4m3.encode(y)


def quant_1x128_rowwise(x_bits, chunk_rows=2048):
    """Vectorized 1x128 rowwise quantizer: q uint8 [R, C], s float32 [R, C/128]."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    R, C = x_bits.shape
    _check_dims(C)
    q = np.empty((R, C), dtype=np.uint8)
    s = np.empty((R, C // BLOCK), dtype=np.float32)
    for r0 in range(0, R, chunk_rows):
        x = bf16_bits_to_f32(x_bits[r0:r0 + chunk_rows])
        _check_finite(x)
        xb = x.reshape(x.shape[0], C // BLOCK, BLOCK)
        sc = _scale_from_amax(np.max(np.abs(xb), axis=2))
        q[r0:r0 + chunk_rows] = _encode_quotient(xb, sc[:, :, None]).reshape(x.shape[0], C)
        s[r0:r0 + chunk_rows] = sc
    return q, s


def quant_1x128_colwise(x_bits, chunk_cols=2048):
    """Vectorized colwise quantizer: q uint8 [C, R] (transposed), s [C, R/128].

    Defined as the rowwise quantizer applied to the transpose: a block is 128
    consecutive rows of one column.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    R, C = x_bits.shape
    _check_dims(R)
    q = np.empty((C, R), dtype=np.uint8)
    s = np.empty((C, R // BLOCK), dtype=np.float32)
    for c0 in range(0, C, chunk_cols):
        qt, st = quant_1x128_rowwise(np.ascontiguousarray(x_bits[:, c0:c0 + chunk_cols].T))
        q[c0:c0 + chunk_cols] = qt
        s[c0:c0 + chunk_cols] = st
    return q, s


def quant_128x128(x_bits, chunk_rowblocks=16):
    """Vectorized 128x128 quantizer: q uint8 [R, C], s float32 [R/128, C/128]."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    R, C = x_bits.shape
    _check_dims(R, C)
    q = np.empty((R, C), dtype=np.uint8)
    s = np.empty((R // BLOCK, C // BLOCK), dtype=np.float32)
    step = chunk_rowblocks * BLOCK
    for r0 in range(0, R, step):
        x = bf16_bits_to_f32(x_bits[r0:r0 + step])
        _check_finite(x)
        nrb = x.shape[0] // BLOCK
        xt = x.reshape(nrb, BLOCK, C // BLOCK, BLOCK)          # [rb, r, cb, c]
        sc = _scale_from_amax(np.max(np.abs(xt), axis=(1, 3)))  # [rb, cb]
        q[r0:r0 + step] = _encode_quotient(xt, sc[:, None, :, None]).reshape(x.shape[0], C)
        s[r0 // BLOCK:r0 // BLOCK + nrb] = sc
    return q, s


def quant_3d_colwise(w_bits):
    """3-D colwise quantizer of expert weights W[G, R, C] (R = out features).

    Reading taken: each expert's matrix is quantized in the same 128x128
    tiles as the weight quantizer and written transposed, so that it is the
    contraction-contiguous operand of the dgrad GEMM (grad_in = grad_out . W).
    Returns q uint8 [G, C, R] with q[g, c, r] the code of W[g, r, c], and
    s float32 [G, C/128, R/128] with s[g, cb, rb] the scale of tile (rb, cb).

    The pages name this kernel only for the MXFP8 recipe ("[mxfp8 moe
    training] use new 3d colwise quantization kernel", summary) and do not fix
    its block shape for 128x128 weight scaling; the 128x128 tile is the
    reading adopted.  Its arithmetic is that of :func:`quant_128x128`.
    """
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    G, R, C = w_bits.shape
    _check_dims(R, C)
    q = np.empty((G, C, R), dtype=np.uint8)
    s = np.empty((G, C // BLOCK, R // BLOCK), dtype=np.float32)
    for g in range(G):
        qg, sg = quant_128x128(w_bits[g])
        q[g] = qg.T
        s[g] = sg.T
    return q, s
