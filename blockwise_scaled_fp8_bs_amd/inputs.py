"""Seeded synthetic inputs shared by the tests, the bench and the oracle timing.

This module holds none of the method's arithmetic: it only draws normal
samples, casts them to bf16 (torch's round-to-nearest-even cast), multiplies a
chosen set of entries by an outlier factor and draws MoE group sizes.  Both
the HIP path and the CPU oracle receive the exact bf16 bytes made here.

Workloads (shapes from the grouped-GEMM microbenchmark table of the
"[mxfp8 moe training] use new 3d colwise quantization kernel" page; value
distributions as stated for the blockwise recipe's synthetic benchmarks):

* ``linear_fwd_256x512x256``   -- A [256, 512] N(0, 1), W [256, 512] N(0, 0.02),
  forward only;
* ``dense_8192x4096x4096``     -- M 8192, K 4096, N 4096; A N(0, 1) with 0.1 %
  of entries (exactly round(0.001 * M * K) distinct positions) multiplied by
  50; W N(0, 0.02); grad_out N(0, 0.01);
* ``ffn_up_16384x5120x8192``   -- M 16384, K 5120, N 8192; same distributions
  without outliers;
* ``ffn_down_16384x7168x2048`` -- M 16384, K 7168, N 2048; same;
* ``moe_128000x5120x8192_g8``  -- 128000 tokens, K 5120, N 8192, G = 8
  experts W [8, 8192, 5120]; group sizes are multiples of 128 cut from 1000
  blocks by 7 sorted uniform cut points in {0..1000} (sizes may be 0).

"N(0, s)" means standard deviation s.  Seeds: one base seed, with substreams
A = seed, W = seed + 1, grad_out = seed + 2, outlier positions = seed + 3,
group sizes = seed + 4.
"""

from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    M: int                 # tokens (rows of A and grad_out)
    K: int                 # in features
    N: int                 # out features
    G: int = 1             # experts (grouped only)
    fwd_only: bool = False
    sigma_a: float = 1.0
    sigma_w: float = 0.02
    sigma_g: float = 0.01
    outlier_frac: float = 0.0
    outlier_factor: float = 50.0
    tags: tuple = field(default_factory=tuple)


WORKLOADS = {
    w.name: w for w in [
        Workload("linear_fwd_256x512x256", M=256, K=512, N=256, fwd_only=True),
        Workload("dense_8192x4096x4096", M=8192, K=4096, N=4096, outlier_frac=0.001),
        Workload("ffn_up_16384x5120x8192", M=16384, K=5120, N=8192),
        Workload("ffn_down_16384x7168x2048", M=16384, K=7168, N=2048),
        Workload("moe_128000x5120x8192_g8", M=128000, K=5120, N=8192, G=8),
    ]
}

SEED_A, SEED_W, SEED_G, SEED_OUTLIER, SEED_GROUPS = 0, 1, 2, 3, 4


def bf16_normal(shape, sigma, seed, device="cpu"):
    """fp32 N(0, 1) draws times ``sigma``, cast to bf16 (round to nearest even)."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if sigma != 1.0:
        x.mul_(sigma)
    return x.to(torch.bfloat16)


def apply_outliers(x, frac, factor, seed):
    """Multiply exactly round(frac * numel) distinct entries of bf16 ``x`` by ``factor``.

    Positions come from a seeded random permutation; the product is formed in
    fp32 and cast back to bf16.  Modifies ``x`` in place and returns it.
    """
    count = int(round(frac * x.numel()))
    if count == 0:
        return x
    g = torch.Generator(device=x.device)
    g.manual_seed(int(seed))
    idx = torch.randperm(x.numel(), generator=g, device=x.device)[:count]
    flat = x.view(-1)
    flat[idx] = (flat[idx].float() * factor).to(torch.bfloat16)
    return x


def group_ends(total_rows, groups, seed, block=128):
    """Cumulative group ends for ``groups`` experts over ``total_rows`` rows.

    ``total_rows / block`` blocks are cut at ``groups - 1`` sorted uniform
    cut points drawn from {0 .. blocks}; sizes are multiples of ``block`` and
    may be zero.  Returns a list of ints whose last entry is ``total_rows``.
    """
    if total_rows % block:
        raise ValueError("total_rows must be a multiple of the block")
    blocks = total_rows // block
    g = torch.Generator()
    g.manual_seed(int(seed))
    cuts = torch.randint(0, blocks + 1, (groups - 1,), generator=g).sort().values.tolist()
    ends = [c * block for c in cuts] + [total_rows]
    return ends


def make_operands(w: Workload, seed=0, device="cpu", rows=None):
    """bf16 activations A [M, K], weights W [(G,) N, K] and grad_out [M, N].

    ``rows`` optionally truncates the token dimension (a sample of the same
    distributions, used for bounded CPU work); group ends then follow the
    truncated length.
    """
    M = w.M if rows is None else rows
    a = bf16_normal((M, w.K), w.sigma_a, seed + SEED_A, device)
    if w.outlier_frac:
        apply_outliers(a, w.outlier_frac, w.outlier_factor, seed + SEED_OUTLIER)
    wshape = (w.G, w.N, w.K) if w.G > 1 else (w.N, w.K)
    wt = bf16_normal(wshape, w.sigma_w, seed + SEED_W, device)
    gout = None if w.fwd_only else bf16_normal((M, w.N), w.sigma_g, seed + SEED_G, device)
    ends = group_ends(M, w.G, seed + SEED_GROUPS) if w.G > 1 else None
    return a, wt, gout, ends
