"""Helpers shared by the GPU parity tests (test code only)."""

import numpy as np
import pytest
import torch

from blockwise_scaled_fp8_bs_amd import inputs

CANARY_U8 = 0xA5
CANARY_BF16_BITS = 0x7FBA     # a bf16 NaN pattern the kernels never produce
CANARY_F32_BITS = 0x7FBADBAD  # a float32 NaN pattern the kernels never produce

_INT_VIEW = {torch.uint8: (torch.uint8, np.uint8, CANARY_U8),
             torch.bfloat16: (torch.int16, np.uint16, CANARY_BF16_BITS),
             torch.float32: (torch.int32, np.uint32, CANARY_F32_BITS)}


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def bits16(t):
    """bf16 tensor -> numpy uint16 bit patterns (CPU copy)."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def bf16_from_bits(b):
    return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16)


def u8(t):
    return t.detach().contiguous().cpu().numpy()


def f32bits(t):
    return t.detach().contiguous().cpu().numpy().view(np.uint32)


def guarded(rows, cols, dtype, pad_cols=16, guard_rows=1, device="cuda"):
    """A [rows, cols] view of a larger buffer filled with a canary.

    The row stride is cols + pad_cols; one extra guard row follows.  Returns
    (full, view).
    """
    full = torch.empty((rows + guard_rows, cols + pad_cols), dtype=dtype, device=device)
    itype, _, canary = _INT_VIEW[dtype]
    full.view(itype).fill_(canary)
    return full, full[:rows, :cols]


def check_canaries(full, rows, cols):
    """Everything outside the [rows, cols] view must still hold the canary."""
    f = full.detach().cpu()
    itype, ntype, canary = _INT_VIEW[f.dtype]
    v = f.view(itype).numpy().view(ntype)
    mask = np.ones(v.shape, dtype=bool)
    mask[:rows, :cols] = False
    assert np.all(v[mask] == canary), "a kernel wrote outside its output (canary overwritten)"


def scale_buffer(nkb, count, pad=4, device="cuda"):
    """K-major scale tensor [nkb, roundup4(count) + pad] filled with the canary."""
    ld = (count + 3) // 4 * 4 + pad
    full = torch.empty((nkb + 1, ld), dtype=torch.float32, device=device)
    full.view(torch.int32).fill_(CANARY_F32_BITS)
    return full, full[:nkb]


def check_scale_canaries(full, nkb, count):
    v = full.detach().cpu().view(torch.int32).numpy().view(np.uint32)
    mask = np.ones(v.shape, dtype=bool)
    mask[:nkb, :count] = False
    assert np.all(v[mask] == CANARY_F32_BITS), "scale padding or guard row was written"


def special_input(R, C, seed, sigma=1.0):
    """bf16 [R, C] N(0, sigma) with edge-case blocks planted (CPU tensor).

    Planted (when the shape allows): a zero row block, a tiny row block
    (amax < EPS), an all-negative row block, a bf16-max element, bf16
    subnormals, negative zeros, an all-zero column over 128 rows, a tiny
    column, and an outlier column.
    """
    x = inputs.bf16_normal((R, C), sigma, seed)
    b = bits16(x).copy()
    rng = np.random.default_rng(seed + 1000)
    if R >= 8 and C >= 128:
        b[0, :128] = 0
        tiny = (rng.standard_normal(128) * 1e-20).astype(np.float32)
        b[1, :128] = bits16(torch.from_numpy(tiny).to(torch.bfloat16))
        b[2, :128] |= 0x8000
        b[3, 5] = 0x7F7F
        b[4, :128] = rng.integers(1, 0x7F, 128).astype(np.uint16) | (rng.integers(0, 2, 128) << 15).astype(np.uint16)
        b[5, 7] = 0x8000
        b[6, 130 % C] = 0x8000
    if R >= 128 and C >= 8:
        b[:128, 1] = 0
        tiny = (rng.standard_normal(128) * 1e-30).astype(np.float32)
        b[:128, 2] = bits16(torch.from_numpy(tiny).to(torch.bfloat16))
        b[17, 3] = bits16(torch.tensor([sigma * 4000.0]).to(torch.bfloat16))[0]
    return bf16_from_bits(b)
