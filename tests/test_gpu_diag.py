"""Exhaustive device checks of the quantizers' arithmetic, compared with the
oracle: the e4m3 encode step over every float32 |y| <= 448 (census of the
decision intervals) and the fma-based division over every reachable
(scale, bf16 element) pair."""

import numpy as np
import pytest

import blockwise_scaled_fp8_bs_amd as bs
from oracle import e4m3
from gpu_support import need_gpu

pytestmark = pytest.mark.gpu

BITS_464 = 0x43E80000  # the census covers |y| <= 464


def f32(u):
    return np.array([u], dtype=np.uint32).view(np.float32)


def test_division_matches_ieee_on_every_reachable_pair():
    need_gpu()
    r = bs.bs_diag_division()
    print(f"division check: {r}", flush=True)
    assert r["pairs"] > 1_000_000_000
    assert r["scale_mismatch"] == 0
    assert r["code_mismatch"] == 0
    assert r["quotient_mismatch"] == 0


def test_e4m3_encode_census_matches_oracle():
    """The kernels' encode step agrees with the oracle's encoder (which
    clamps to 448 first) on all ~2.2e9 float32 inputs |y| <= 464: both are
    monotone step functions, so equal decision intervals per code mean equal
    outputs everywhere."""
    need_gpu()
    mn, mx, cnt = bs.bs_diag_e4m3_census()
    mn = mn.numpy().view(np.uint32)
    mx = mx.numpy().view(np.uint32)
    cnt = cnt.numpy()
    produced = np.nonzero(cnt)[0]
    assert len(produced) == 254  # every finite code, none of the NaN codes
    assert 0x7F not in produced and 0xFF not in produced
    for sign in (0, 0x80):
        codes = sorted(c for c in produced if (c & 0x80) == sign)
        covered = 0
        for c in codes:
            lo, hi = int(mn[c]), int(mx[c])
            assert hi - lo + 1 == cnt[c], f"code {c:#x} is not an interval"
            covered += int(cnt[c])
            sgn = np.uint32(0x80000000 if sign else 0)
            assert e4m3.encode(f32(lo | sgn))[0] == c
            assert e4m3.encode(f32(hi | sgn))[0] == c
            if lo > 0:
                assert e4m3.encode(f32((lo - 1) | sgn))[0] != c
            if hi < BITS_464:
                assert e4m3.encode(f32((hi + 1) | sgn))[0] != c
        assert covered == BITS_464 + 1


def test_stream_reference_moves_the_bytes():
    """The streaming reference (a timing baseline) reads every input byte and
    writes every output byte: the first n_read written bytes are the input
    words XOR 1, the rest are written (canary gone)."""
    need_gpu()
    import torch
    n_read, n_write = 3 * 32768 + 4096, 3 * 32768 + 4096 + 3 * 1024 + 48
    src = torch.randint(0, 256, (n_read,), dtype=torch.uint8, device="cuda")
    dst = torch.full((n_write + 64,), 0xA5, dtype=torch.uint8, device="cuda")
    bs.bs_diag_stream(src, n_read, dst, n_write)
    torch.cuda.synchronize()
    s = src.cpu().numpy().view(np.uint32)
    d = dst.cpu().numpy()
    assert np.array_equal(d[:n_read].view(np.uint32), s ^ np.uint32(1))
    tail = d[n_read:n_write].view(np.uint32).reshape(-1, 4)
    assert np.all(tail[:, 1:] == np.array([1, 2, 3], dtype=np.uint32)), "tail bytes not written"
    assert np.all(d[n_write:] == 0xA5), "wrote past n_write"
