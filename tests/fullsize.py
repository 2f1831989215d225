"""Thread-parallel drivers of the CPU oracle for full-size parity (test code only).

Blockwise quantization treats every block on its own, so the oracle applied
to row chunks (1x128 rows; 128x128 with chunks of whole 128-row tiles) or to
column chunks (1x128 columns) and concatenated is, by the definition, the
oracle applied to the whole array; the chunks only let numpy work on several
host cores at once (its array operations release the interpreter lock).  The
GEMM reference is the oracle's float64 product, formed in row panels so that
only one panel of the reference and of its tolerance is held at a time.
Nothing here does arithmetic of its own beyond slicing and concatenation.
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from oracle import gemm, quant

_POOL = ThreadPoolExecutor(max_workers=max(1, min(16, os.cpu_count() or 1)))


def _rows(fn, x, chunk):
    parts = list(_POOL.map(lambda r0: fn(x[r0:r0 + chunk]), range(0, x.shape[0], chunk)))
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def quant_rowwise(x_bits, chunk=256):
    """oracle.quant.quant_1x128_rowwise over row chunks: q [R, C], s [R, C/128]."""
    return _rows(quant.quant_1x128_rowwise, np.asarray(x_bits), chunk)


def quant_colwise(x_bits, chunk=256):
    """oracle.quant.quant_1x128_colwise over column chunks: q [C, R], s [C, R/128]."""
    x = np.asarray(x_bits)
    parts = list(_POOL.map(lambda c0: quant.quant_1x128_colwise(x[:, c0:c0 + chunk]),
                           range(0, x.shape[1], chunk)))
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def quant_128x128(x_bits, chunk=256):
    """oracle.quant.quant_128x128 over chunks of whole 128-row tiles."""
    assert chunk % 128 == 0
    return _rows(quant.quant_128x128, np.asarray(x_bits), chunk)


def dequant(q, s, row_block, chunk=256):
    """oracle.gemm.dequant over row chunks (row_block divides chunk)."""
    q = np.asarray(q)
    s = np.asarray(s)
    assert chunk % row_block == 0
    out = np.empty(q.shape, dtype=np.float64)

    def one(r0):
        out[r0:r0 + chunk] = gemm.dequant(q[r0:r0 + chunk], s[r0 // row_block:(r0 + chunk) // row_block], row_block)

    list(_POOL.map(one, range(0, q.shape[0], chunk)))
    return out


def check_gemm(d, a_deq, b_deq, rows=None, panel=1024, what="GEMM"):
    """Every element of the GPU result d[rows] (float64-convertible, [len(rows), N])
    against the oracle's float64 product a_deq[rows] . b_deq^T within
    2e-3 * ||a_m|| * ||b_n||.  Returns the worst |err| / bound."""
    rows = np.arange(a_deq.shape[0]) if rows is None else np.asarray(rows)
    worst = 0.0
    for p0 in range(0, len(rows), panel):
        r = rows[p0:p0 + panel]
        a = a_deq[r]
        ref = a @ b_deq.T
        ok, w = gemm.check_close(np.asarray(d[p0:p0 + panel], dtype=np.float64), ref, a, b_deq)
        assert ok, f"{what}: rows {r[0]}..{r[-1]} outside the tolerance (worst |err|/bound {w})"
        worst = max(worst, w)
    return worst
