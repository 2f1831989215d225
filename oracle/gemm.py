"""Blockwise-scaled FP8 matmuls, CPU oracle: dequantize, then float64 matmul.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the scaled GEMM computes (pages: "[not for land] float8 blockwise
scaling training prototype using deep_gemm", description -- forward and
backward GEMMs of a dense linear, and grouped GEMMs for MoE; "add FSDP and TP
tests for Float8BlockwiseLinear", review thread on ``blockwise_scaled_mm`` --
A row-major, B column-major, i.e. both operands contiguous along the
contraction).  With ``A`` codes [M, K] and ``B`` codes [N, K]:

    D[m, n] = sum_k  dec(A[m, k]) * sa(m, k)  *  dec(B[n, k]) * sb(n, k)

where ``sa(m, k)`` is the 1x128 scale of row m, block k // 128 and
``sb(n, k)`` is the 128x128 scale of block (n // 128, k // 128) or the 1x128
scale of row n, block k // 128.  This is exactly the sum of per-128-block
partial products times the two block scales, which is how the kernels
evaluate it.

The oracle dequantizes both operands to float64 (each product of an e4m3
value and a float32 scale has at most 4 + 24 significant bits, so the
dequantized values are exact) and multiplies in float64 (numpy/BLAS).

Parity bar for an fp32-accumulating GPU result ``D`` (the recipe's per
element tolerance):  |D[m, n] - ref[m, n]| <= 2e-3 * ||a_m||_2 * ||b_n||_2,
with a_m and b_n the dequantized rows of A and B.
"""

import numpy as np

from . import e4m3

BLOCK = 128
REL_TOL = 2e-3


def dequant(q, s, row_block):
    """Dequantize codes ``q`` [rows, K] with logical scales ``s``.

    ``row_block`` is 1 for 1x128 scales (``s`` is [rows, K/128]) and 128 for
    128x128 scales (``s`` is [rows/128, K/128]).  Returns float64 [rows, K].
    """
    q = np.asarray(q, dtype=np.uint8)
    rows, K = q.shape
    if K % BLOCK or rows % row_block:
        raise ValueError("dequant: dimensions must be multiples of the block")
    vals = e4m3.decode(q)
    if np.isnan(vals).any():
        raise ValueError("dequant: NaN code in operand")
    s64 = np.asarray(s, dtype=np.float32).astype(np.float64)
    expected = (rows // row_block, K // BLOCK)
    if s64.shape != expected:
        raise ValueError(f"dequant: scale shape {s64.shape}, expected {expected}")
    full = np.repeat(np.repeat(s64, row_block, axis=0), BLOCK, axis=1)
    return vals * full


def scaled_mm(qa, sa, qb, sb, b_row_block):
    """D = A . B^T in float64 from codes and logical scales.

    ``qa`` [M, K] with 1x128 scales ``sa`` [M, K/128]; ``qb`` [N, K] with
    scales ``sb`` of row block ``b_row_block`` (128 or 1).
    """
    a = dequant(qa, sa, 1)
    b = dequant(qb, sb, b_row_block)
    return a @ b.T


def row_norms(x):
    """L2 norm of every row of a float64 matrix."""
    return np.sqrt(np.sum(np.asarray(x, dtype=np.float64) ** 2, axis=1))


def tolerance(a_deq, b_deq):
    """Per-element bound 2e-3 * ||a_m|| * ||b_n|| as an [M, N] array."""
    return REL_TOL * np.outer(row_norms(a_deq), row_norms(b_deq))


def check_close(d, ref, a_deq, b_deq):
    """Return (ok, worst ratio |d - ref| / bound) for a GPU result ``d``.

    A zero bound (an all-zero row) requires an exactly zero difference.
    """
    d = np.asarray(d, dtype=np.float64)
    err = np.abs(d - ref)
    bound = tolerance(a_deq, b_deq)
    if not np.all(np.isfinite(d)):
        return False, float("inf")
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0),
                         np.where(err > 0, np.inf, 0.0))
    worst = float(ratio.max()) if ratio.size else 0.0
    return worst <= 1.0, worst


# ----------------------------------------------------------------------------
# grouped (MoE) variants
# ----------------------------------------------------------------------------

def group_bounds(group_end):
    """[(start, end)] for cumulative group ends (each a multiple of 128)."""
    ends = [int(e) for e in group_end]
    out, start = [], 0
    for e in ends:
        if e < start or e % BLOCK:
            raise ValueError("group ends must be non-decreasing multiples of 128")
        out.append((start, e))
        start = e
    return out


def grouped_mm_group_m(group_end, qa, sa, qb, sb, b_row_block):
    """Grouped GEMM over row groups of A (MoE forward and dgrad).

    Rows [start_g, end_g) of A multiply expert g's B: qb [G, N, K] with
    scales sb [G, N/b_row_block, K/128].  Returns D float64 [M, N]; rows past
    the last group end are not defined by the method and are returned as NaN.
    """
    qa = np.asarray(qa, dtype=np.uint8)
    M = qa.shape[0]
    N = qb.shape[1]
    d = np.full((M, N), np.nan)
    for g, (start, end) in enumerate(group_bounds(group_end)):
        if end == start:
            continue
        d[start:end] = scaled_mm(qa[start:end], sa[start:end], qb[g], sb[g], b_row_block)
    return d


def grouped_mm_group_k(group_end, qa, sa, qb, sb):
    """Grouped GEMM over contraction groups (MoE wgrad).

    ``qa`` [N, T] and ``qb`` [K, T], both with 1x128 scales along T (the
    token axis): ``sa`` [N, T/128], ``sb`` [K, T/128].  Group g contracts over
    tokens [start_g, end_g).  Returns D float64 [G, N, K]; an empty group
    gives zeros.
    """
    qa = np.asarray(qa, dtype=np.uint8)
    qb = np.asarray(qb, dtype=np.uint8)
    bounds = group_bounds(group_end)
    N, K = qa.shape[0], qb.shape[0]
    d = np.zeros((len(bounds), N, K))
    for g, (start, end) in enumerate(bounds):
        if end == start:
            continue
        b0, b1 = start // BLOCK, end // BLOCK
        d[g] = scaled_mm(qa[:, start:end], sa[:, b0:b1], qb[:, start:end], sb[:, b0:b1], 1)
    return d
