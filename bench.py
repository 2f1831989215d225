"""Benchmark of the blockwise-scaled FP8 training hot path on one MI355X.

One step = every kernel of one blockwise-FP8 linear layer's training pass
over one batch of seeded synthetic data already resident in HBM (by default
the MoE layer: 128000 tokens over 8 experts, K 5120, N 8192):

  quantize A [M, K] rows + transposed columns (1x128) and, in the same
    launch, W [N, K] (128x128) and W^T (3-D colwise layout) in one pass,
  quantize grad_out [M, N] rows + transposed columns (1x128),
  forward  out     = A . W^T          (1x128 x 128x128),
  dgrad    grad_in = grad_out . W     (1x128 x 128x128, via W^T),
  wgrad    grad_W  = grad_out^T . A   (1x128 x 1x128).

For the MoE workload the GEMMs are the grouped forms (GROUP_M forward and
dgrad, GROUP_K wgrad) and W is quantized per expert.

Prints ONE JSON line.  `value` is fwd+bwd GEMM FLOPs (3 * 2*M*N*K) divided
by the wall time of the whole step (quantizers included), over `steps` timed
steps in which only the dominant kernel is bracketed by HIP events (its
average duration gives `roofline`).  The per-kernel breakdown comes from a
separate pass of `steps` steps with events around every kernel (events
between kernels cost GPU time of their own).  The CPU oracle is timed on a
bounded sample of the same workload on the host (rank 0, N = 1).

The line also carries: the SHA-256 of the bf16 inputs (the bytes both the
GPU and the oracle consume), the shader and memory clocks read while the
timed steps ran (the driver updates them about once a second; where fewer
than two updates fall in the timed steps, the same steps keep running
untimed until two have come), a short record of each dense workload (forward, dgrad
and wgrad of one linear layer) timed the same way, and the smallest layer's
forward (256x512x256, launch-bound) as eager calls and as one HIP graph.
"""

import argparse
import json
import os
import statistics
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import blockwise_scaled_fp8_bs_amd as bs  # noqa: E402
from blockwise_scaled_fp8_bs_amd import inputs  # noqa: E402

FP8_PEAK_TFLOPS = 5000.0     # MI355X dense FP8 MFMA (no sparsity)
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
DEFAULT_WORKLOAD = "moe_128000x5120x8192_g8"
EXTRA_WORKLOADS = "dense_8192x4096x4096,ffn_up_16384x5120x8192,ffn_down_16384x7168x2048"


def r4(n):
    return (n + 3) // 4 * 4


# bench kernel name -> device kernel symbol (as rocprofv3 names it)
KERNEL_SYMBOL = {
    # (prefixes: the 1x128 kernels come in a one-tile-per-workgroup and a
    # persistent form, chosen by size)
    "quant_fwd_operands(A,W)": "quant_pair_kernel",
    "quant_1x128_rowcol(grad_out)": "quant_1x128_kernel<true, true, false,",
    "swiglu_quant": "quant_1x128_kernel<true, true, true,",
    "gemm_fwd": "gemm_kernel<0, false, false>",
    "gemm_dgrad": "gemm_kernel<0, false, false>",
    "gemm_wgrad": "gemm_kernel<0, true, false>",
    "gemm_wgrad_split": "gemm_sk_kernel<true, false>",
    "grouped_gemm_fwd": "gemm_kernel<1, false, false>",
    "grouped_gemm_dgrad": "gemm_kernel<1, false, false>",
    "grouped_gemm_wgrad": "gemm_kernel<2, true, false>",
}


# sources each device kernel is built from (a counter summary stays valid
# while these are unchanged)
KERNEL_SOURCES = {
    "gemm_kernel": ["bs_gemm.hip", "bs_kernels.h"],
    "gemm_sk_kernel": ["bs_gemm.hip", "bs_kernels.h"],
    "sk_reduce_kernel": ["bs_gemm.hip", "bs_kernels.h"],
    "mx_gemm_kernel": ["bs_gemm.hip", "bs_kernels.h"],
    "quant_": ["bs_quant.hip", "bs_device.h", "bs_kernels.h", "bs_mx.h"],
    "swiglu_bwd_quant_kernel": ["bs_quant.hip", "bs_device.h", "bs_kernels.h", "bs_mx.h"],
    "mx_quant_kernel": ["bs_quant.hip", "bs_device.h", "bs_kernels.h", "bs_mx.h"],
    "stream_kernel": ["bs_diag.hip", "bs_kernels.h"],
}


def _code_only(text):
    """C++ source with its comments removed and whitespace runs collapsed
    (string and character literals kept as written)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash(symbol):
    """sha256 prefix of the code of the sources of the device kernel
    `symbol`, comments and whitespace left out (editing a comment does not
    make counters taken on the same code stale)."""
    import hashlib
    src = os.path.join(ROOT, "blockwise_scaled_fp8_bs_amd", "csrc")
    files = next((fs for prefix, fs in KERNEL_SOURCES.items() if symbol.startswith(prefix)), None)
    if files is None:
        return None
    h = hashlib.sha256()
    for f in files:
        h.update(_code_only(open(os.path.join(src, f), encoding="utf-8").read()).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


def counter_traffic(workload, kernel, split=False):
    """HBM-side bytes per launch of `kernel` from the committed rocprofv3
    counter summary (FETCH_SIZE + WRITE_SIZE, each scaled by its reading of a
    known-size copy), or None when there is none or the kernel sources have
    changed since it was taken.  ``split``: the wgrad ran as its stream-K
    kernel."""
    path = os.path.join(ROOT, "profiles", f"{workload}_rocprof.txt")
    if not os.path.exists(path):
        return None
    sym = KERNEL_SYMBOL.get(kernel + "_split" if split else kernel)
    cur = kernel_source_hash(sym) if sym else None
    for line in open(path):
        if line.startswith("traffic_bytes ") and sym and sym in line:
            fields = line.split()
            src = fields[-1].split("=", 1)[1]
            if src == cur:
                return int(fields[-2])
    return None


class Step:
    """Buffers and launches of one training step of one workload."""

    def __init__(self, w: inputs.Workload, seed=0, device="cuda", scale_pad=0):
        """``scale_pad`` widens every scale tensor's row stride past
        roundup4(count) by that many floats (a multiple of 4; the padding is
        never written)."""
        self.w = w
        M, K, N, G = w.M, w.K, w.N, w.G
        dev = device
        self.scale_pad = scale_pad
        r4 = lambda n: (n + 3) // 4 * 4 + scale_pad  # noqa: E731
        a, wt, gout, ends = inputs.make_operands(w, seed=seed, device=dev)
        self.a, self.wt, self.gout = a, wt, gout
        self.grouped = G > 1
        u8 = torch.uint8
        # activations: rows (forward A operand) and transposed columns (wgrad B operand)
        self.qa = torch.empty((M, K), dtype=u8, device=dev)
        self.sa = torch.empty((K // 128, r4(M)), dtype=torch.float32, device=dev)
        self.qaT = torch.empty((K, M), dtype=u8, device=dev)
        self.saT = torch.empty((M // 128, r4(K)), dtype=torch.float32, device=dev)
        # grad_out: rows (dgrad A operand) and transposed columns (wgrad A operand)
        self.qg = torch.empty((M, N), dtype=u8, device=dev)
        self.sg = torch.empty((N // 128, r4(M)), dtype=torch.float32, device=dev)
        self.qgT = torch.empty((N, M), dtype=u8, device=dev)
        self.sgT = torch.empty((M // 128, r4(N)), dtype=torch.float32, device=dev)
        # weights: [G*N, K] 128x128 (forward) and [G, K, N] transposed (dgrad)
        wv = wt.view(G * N, K)
        self.wv = wv
        self.qw = torch.empty((G * N, K), dtype=u8, device=dev)
        self.sw = torch.empty((K // 128, r4(G * N // 128)), dtype=torch.float32, device=dev)
        self.qwT = torch.empty((G, K, N), dtype=u8, device=dev)
        self.swT = torch.empty((G, N // 128, r4(K // 128)), dtype=torch.float32, device=dev)
        self.w3 = wt.view(G, N, K)
        # outputs
        self.out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        self.gin = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        self.gw = torch.empty((G, N, K) if self.grouped else (N, K), dtype=torch.bfloat16, device=dev)
        if self.grouped:
            self.ends = torch.tensor(ends, dtype=torch.int32, device=dev)
            self.group_sizes = [e - s for s, e in zip([0] + ends[:-1], ends)]
            self.sw_view = torch.as_strided(self.sw, (G, K // 128, N // 128), (N // 128, self.sw.stride(0), 1))

    # (name, fn, algorithmic bytes or flops, kind)
    def kernels(self):
        w = self.w
        M, K, N, G = w.M, w.K, w.N, w.G
        gemm_flops = 2.0 * M * N * K
        q1_bytes = lambda R, C: R * C * (2 + 2) + 4 * (R * C // 128) * 2  # noqa: E731
        q128b_bytes = lambda R, C: R * C * (2 + 1 + 1) + 4 * (R * C // 16384) * 2  # noqa: E731
        # bf16 bytes each quantizer pass reads (the rest of its work is written)
        self.quant_read_bytes = {"quant_fwd_operands(A,W)": 2 * (M * K + G * N * K),
                                 "quant_1x128_rowcol(grad_out)": 2 * M * N}
        ks = [
            # the activation (1x128 rows + columns) and the weights (128x128,
            # both layouts) in one launch
            ("quant_fwd_operands(A,W)", lambda: bs.bs_quant_fwd_operands(
                self.a, self.qa, self.sa, self.qaT, self.saT, self.w3, self.qw, self.sw, self.qwT, self.swT),
             q1_bytes(M, K) + q128b_bytes(G * N, K), "GB/s"),
            ("quant_1x128_rowcol(grad_out)",
             lambda: bs.bs_quant_1x128(self.gout, self.qg, self.sg, self.qgT, self.sgT), q1_bytes(M, N), "GB/s"),
        ]
        if not self.grouped:
            ks += [
                ("gemm_fwd", lambda: bs.bs_scaled_mm(self.qa, self.sa, self.qw, self.sw, bs.BS_SCALE_128X128,
                                                     out=self.out), gemm_flops, "TFLOP/s"),
                ("gemm_dgrad", lambda: bs.bs_scaled_mm(self.qg, self.sg, self.qwT[0], self.swT[0],
                                                       bs.BS_SCALE_128X128, out=self.gin), gemm_flops, "TFLOP/s"),
                # stream-K form: splits a ragged last round of tiles along K
                # (and is the plain kernel when the tiles fill every round)
                ("gemm_wgrad", lambda: bs.bs_scaled_mm_ws(self.qgT, self.sgT, self.qaT, self.saT,
                                                          bs.BS_SCALE_1X128, out=self.gw), gemm_flops, "TFLOP/s"),
            ]
        else:
            ks += [
                ("grouped_gemm_fwd", lambda: bs.bs_grouped_scaled_mm(
                    bs.BS_GROUP_M, self.ends, self.qa, self.sa, self.qw.view(G, N, K), self.sw_view,
                    bs.BS_SCALE_128X128, out=self.out), gemm_flops, "TFLOP/s"),
                ("grouped_gemm_dgrad", lambda: bs.bs_grouped_scaled_mm(
                    bs.BS_GROUP_M, self.ends, self.qg, self.sg, self.qwT, self.swT, bs.BS_SCALE_128X128,
                    out=self.gin), gemm_flops, "TFLOP/s"),
                ("grouped_gemm_wgrad", lambda: bs.bs_grouped_scaled_mm(
                    bs.BS_GROUP_K, self.ends, self.qgT, self.sgT, self.qaT, self.saT, bs.BS_SCALE_1X128,
                    out=self.gw), gemm_flops, "TFLOP/s"),
            ]
        return ks


def cpu_oracle_sample(w: inputs.Workload, rows=2048, seed=0):
    """Time the CPU oracle on a bounded sample of the workload.

    The sample is the first `rows` tokens of the same seeded inputs (a
    [rows, K] activation and [rows, N] grad_out; the full weight, or one
    expert's weight): all seven steps (four quantizers, three GEMMs over the
    sampled tokens).  Returns (TFLOP/s of the sampled GEMMs over the whole
    sample time, seconds, description).
    """
    import numpy as np
    from oracle import gemm, quant

    a, wt, gout, _ = inputs.make_operands(w, seed=seed, device="cpu", rows=rows)
    if w.G > 1:
        wt = wt[0]
    bits = lambda t: t.contiguous().view(torch.int16).numpy().view(np.uint16)  # noqa: E731
    t0 = time.perf_counter()
    qa, sa = quant.quant_1x128_rowwise(bits(a))
    qaT, saT = quant.quant_1x128_colwise(bits(a))
    qw, sw = quant.quant_128x128(bits(wt))
    qwT, swT = quant.quant_3d_colwise(bits(wt)[None])
    qg, sg = quant.quant_1x128_rowwise(bits(gout))
    qgT, sgT = quant.quant_1x128_colwise(bits(gout))
    gemm.scaled_mm(qa, sa, qw, sw, 128)
    gemm.scaled_mm(qg, sg, qwT[0], swT[0], 128)
    gemm.scaled_mm(qgT, sgT, qaT, saT, 1)
    dt = time.perf_counter() - t0
    flops = 3 * 2.0 * rows * w.N * w.K
    desc = (f"first {rows} of {w.M} tokens of {w.name}{' (expert 0 weight)' if w.G > 1 else ''}: "
            f"4 quantizers + fwd/dgrad/wgrad GEMMs, {flops / 1e9:.1f} GFLOP")
    return flops / dt / 1e12, dt, desc


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads") for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return os.cpu_count()


def ffn_module_timing(M, D, H, interleaved_ms, seed):
    """Median fwd+bwd time of the fused gated FFN module and of the same FFN
    built from three Float8BlockwiseLinear layers (same weights and input)."""
    fused = bs.Float8BlockwiseGatedFFN(D, H, device="cuda")
    lin = [bs.Float8BlockwiseLinear(D, H, device="cuda"), bs.Float8BlockwiseLinear(D, H, device="cuda"),
           bs.Float8BlockwiseLinear(H, D, device="cuda")]
    with torch.no_grad():
        for k, name in enumerate(["w1", "w2", "out_proj"]):
            wt = inputs.bf16_normal(tuple(getattr(fused, name).shape), 0.02, seed + 10 + k).cuda()
            getattr(fused, name).copy_(wt)
            lin[k].weight.copy_(wt)
    x = inputs.bf16_normal((M, D), 1.0, seed + 20).cuda().requires_grad_()
    dy = inputs.bf16_normal((M, D), 0.01, seed + 21).cuda()
    params = [fused.w1, fused.w2, fused.out_proj] + [l.weight for l in lin]

    def clear():
        x.grad = None
        for p_ in params:
            p_.grad = None

    def run_fused():
        clear()
        fused(x).backward(dy)

    def run_unfused():
        clear()
        lin[2](torch.nn.functional.silu(lin[0](x)) * lin[1](x)).backward(dy)

    f_ms, u_ms = interleaved_ms([run_fused, run_unfused], 7)
    flops = 2.0 * M * D * H * 3 * 3
    return {"shape": {"tokens": M, "dim": D, "hidden": H}, "fused_ms": round(f_ms, 4),
            "unfused_ms": round(u_ms, 4), "speedup": round(u_ms / f_ms, 3),
            "fused_tflops": round(flops / (f_ms * 1e-3) / 1e12, 1)}


# MXFP8 grouped GEMM shapes (tokens M, out N, in K, experts G) and the pages'
# own MXFP8 and bf16 timings for them, in microseconds, forward and forward +
# backward ("[mxfp8 moe training] use new 3d colwise quantization kernel",
# microbenchmark table; another machine's numbers, quoted as context).
MX_SHAPES = [
    ((16384, 8192, 5120, 1), {"mxfp8_fwd": 790.56, "mxfp8_fwd_bwd": 2928.22, "bf16_fwd": 1236.03,
                              "bf16_fwd_bwd": 4257.76}),
    ((128000, 8192, 5120, 8), {"mxfp8_fwd": 5816.16, "mxfp8_fwd_bwd": 25204.8, "bf16_fwd": 10200.0,
                               "bf16_fwd_bwd": 44263.5}),
    ((16384, 2048, 7168, 1), {"mxfp8_fwd": 396.224, "mxfp8_fwd_bwd": 1436.51, "bf16_fwd": 425.248,
                              "bf16_fwd_bwd": 1458.74}),
]


# Dense GEMM shapes (M, N, K) at which the forward GEMM is timed next to two
# references: the vendor's plain FP8 GEMM (hipBLASLt through
# torch._scaled_mm, one scale per tensor, no blockwise scaling) and this
# build's MXFP8 GEMM (same kernel body, scales applied by the MFMA, no fold).
REFERENCE_SHAPES = [(8192, 4096, 4096), (16384, 8192, 5120), (16384, 5120, 8192), (32768, 8192, 8192)]


def launch_bound_timing(seed, n=300):
    """The smallest workload, the 256x512x256 linear forward (x quantized 1x128,
    W 128x128, the forward GEMM: three calls of a few microseconds each), is
    bound by launch overhead: time it as eager calls and as one replayed HIP
    graph of the same calls (the library enqueues only kernels and never
    synchronizes, so the calls capture as they are), and check that a replay
    writes the eager output bit for bit."""
    w = inputs.WORKLOADS["linear_fwd_256x512x256"]
    M, K, N = w.M, w.K, w.N
    x = inputs.bf16_normal((M, K), w.sigma_a, seed, device="cuda")
    wt = inputs.bf16_normal((N, K), w.sigma_w, seed + 1, device="cuda")
    qx = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sx = bs.empty_scales(K // 128, M, "cuda")
    qw = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    sw = bs.empty_scales(K // 128, N // 128, "cuda")
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def fwd():
        bs.bs_quant_1x128(x, q_row=qx, s_row=sx)
        bs.bs_quant_128x128(wt, qw, sw)
        bs.bs_scaled_mm(qx, sx, qw, sw, bs.BS_SCALE_128X128, out=out)

    for _ in range(10):
        fwd()
    torch.cuda.synchronize()
    ref = out.clone()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph):
            fwd()
    torch.cuda.current_stream().wait_stream(side)
    out.fill_(float("nan"))
    graph.replay()
    torch.cuda.synchronize()
    equal = bool(torch.equal(out.view(torch.int16), ref.view(torch.int16)))

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / n * 1e6

    eager_us, graph_us = [], []
    for _ in range(3):
        eager_us.append(timed(fwd))
        graph_us.append(timed(graph.replay))
    e, g = statistics.median(eager_us), statistics.median(graph_us)
    del graph
    return {"workload": w.name, "calls": 3, "eager_us_per_step": round(e, 1), "graph_us_per_step": round(g, 1),
            "speedup": round(e / g, 2), "graph_output_equal": equal}


def gemm_reference_timing(interleaved_ms, seed):
    """Median times of the 128-block forward GEMM, the MX GEMM and the
    vendor's plain FP8 GEMM on the same bf16 operands (each quantized its own
    way), the three alternating."""
    rows = []
    for (M, N, K) in REFERENCE_SHAPES:
        a = inputs.bf16_normal((M, K), 1.0, seed + 50, device="cuda")
        w = inputs.bf16_normal((N, K), 0.02, seed + 51, device="cuda")
        u8 = torch.uint8
        qa, sa = torch.empty((M, K), dtype=u8, device="cuda"), bs.empty_scales(K // 128, M, "cuda")
        qw, sw = torch.empty((N, K), dtype=u8, device="cuda"), bs.empty_scales(K // 128, N // 128, "cuda")
        bs.bs_quant_1x128(a, qa, sa)
        bs.bs_quant_128x128(w, qw, sw)
        ma, msa = torch.empty((M, K), dtype=u8, device="cuda"), bs.empty_mx_scales(K // 32, M, "cuda")
        mw, msw = torch.empty((N, K), dtype=u8, device="cuda"), bs.empty_mx_scales(K // 32, N, "cuda")
        bs.bs_mx_quant_1x32(a, ma, msa)
        bs.bs_mx_quant_1x32(w, mw, msw)
        # vendor operands: one scale per tensor, amax mapped to 448
        one = torch.ones((), device="cuda")
        a8 = (a.float() * (448.0 / a.float().abs().max())).to(torch.float8_e4m3fn)
        w8 = (w.float() * (448.0 / w.float().abs().max())).to(torch.float8_e4m3fn)
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

        def blockwise():
            bs.bs_scaled_mm(qa, sa, qw, sw, bs.BS_SCALE_128X128, out=out)

        def mx():
            bs.bs_mx_scaled_mm(ma, msa, mw, msw, out=out)

        def vendor():
            torch._scaled_mm(a8, w8.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16)

        t = dict(zip(("blockwise_128", "mxfp8", "vendor_plain_fp8"), interleaved_ms([blockwise, mx, vendor])))
        flops = 2.0 * M * N * K
        rows.append({"M": M, "N": N, "K": K, "us": {k: round(v * 1e3, 1) for k, v in t.items()},
                     "pflops": {k: round(flops / (v * 1e-3) / 1e15, 3) for k, v in t.items()}})
        del a, w, qa, qw, ma, mw, a8, w8, out
        torch.cuda.empty_cache()
    return rows


def mx_grouped_timing(median_ms, seed, which=None):
    """Median forward and forward + backward times of mx_grouped_mm (bf16 in,
    quantization included, as the pages' op) and of torch bf16 GEMMs per
    expert, at the pages' microbenchmark shapes with equal-size groups."""
    rows = []
    for i, ((M, N, K, G), pages) in enumerate(MX_SHAPES):
        if which is not None and i not in which:
            continue
        x = inputs.bf16_normal((M, K), 1.0, seed + 40, device="cuda").requires_grad_()
        wt = inputs.bf16_normal((G, N, K), 0.02, seed + 41, device="cuda").requires_grad_()
        dy = inputs.bf16_normal((M, N), 0.01, seed + 42, device="cuda")
        ends = torch.tensor([(g + 1) * M // G for g in range(G)], dtype=torch.int32, device="cuda")
        bounds = [0] + ends.tolist()

        def mx_fwd():
            with torch.no_grad():
                bs.mx_grouped_mm(x, wt, ends)

        def mx_fwd_bwd():
            x.grad = wt.grad = None
            bs.mx_grouped_mm(x, wt, ends).backward(dy)

        def bf16_fwd():
            with torch.no_grad():
                for g in range(G):
                    torch.mm(x[bounds[g]:bounds[g + 1]], wt[g].t())

        def bf16_fwd_bwd():
            x.grad = wt.grad = None
            y = torch.cat([torch.mm(x[bounds[g]:bounds[g + 1]], wt[g].t()) for g in range(G)])
            y.backward(dy)

        t = {name: median_ms(fn, 5) for name, fn in (("mxfp8_fwd", mx_fwd), ("mxfp8_fwd_bwd", mx_fwd_bwd),
                                                     ("bf16_fwd", bf16_fwd), ("bf16_fwd_bwd", bf16_fwd_bwd))}
        flops = 2.0 * M * N * K
        rows.append({"M": M, "N": N, "K": K, "G": G,
                     "us": {k: round(v * 1e3, 1) for k, v in t.items()},
                     "mxfp8_fwd_tflops": round(flops / (t["mxfp8_fwd"] * 1e-3) / 1e12, 1),
                     "mxfp8_fwd_bwd_tflops": round(3 * flops / (t["mxfp8_fwd_bwd"] * 1e-3) / 1e12, 1),
                     "speedup_vs_bf16": {"fwd": round(t["bf16_fwd"] / t["mxfp8_fwd"], 3),
                                         "fwd_bwd": round(t["bf16_fwd_bwd"] / t["mxfp8_fwd_bwd"], 3)},
                     "pages_us": pages})
        x.grad = wt.grad = None
        del x, wt, dy
        torch.cuda.empty_cache()
    return rows


def wgrad_split(w):
    """Whether the dense wgrad of workload w runs as the stream-K kernel."""
    return w.G == 1 and bs.bs_scaled_mm_workspace_bytes(w.N, w.K, w.M, bs.BS_SCALE_1X128) > 0


def input_digest(step):
    """SHA-256 of the bf16 inputs of a step (the exact bytes that both the
    GPU kernels and the CPU oracle consume) and of the group ends."""
    import hashlib
    out = {}
    for name, t in (("A", step.a), ("W", step.wt), ("grad_out", step.gout)):
        h = hashlib.sha256()
        h.update(t.contiguous().view(torch.int16).cpu().numpy())
        out[name] = h.hexdigest()
    if step.grouped:
        out["group_end"] = hashlib.sha256(step.ends.cpu().numpy().tobytes()).hexdigest()
    return out


class ClockSampler:
    """Shader (GFX) and memory (UCLK) clocks of the GPU, read from the driver
    through amdsmi in a background thread while timed work runs.  Records
    nothing (and says why) where the driver interface is not available."""

    def __init__(self, interval_s=0.005):
        import threading
        self.interval = interval_s
        self.samples = []
        self.error = None
        self.handle = None
        self.extra_steps = 0
        self._stop = threading.Event()
        self._thread = None
        try:
            import amdsmi
            self.smi = amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            props = torch.cuda.get_device_properties(torch.cuda.current_device())
            want = (props.pci_domain_id, props.pci_bus_id, props.pci_device_id)
            for h in handles:
                bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)          # "dddd:bb:dd.f"
                dom, bus, rest = bdf.split(":")
                if (int(dom, 16), int(bus, 16), int(rest.split(".")[0], 16)) == want:
                    self.handle = h
            if self.handle is None and len(handles) == 1:
                self.handle = handles[0]
            if self.handle is None:
                self.error = f"no amdsmi handle matches PCI {want}"
        except Exception as e:  # driver interface missing or not permitted
            self.error = f"{type(e).__name__}: {e}"

    def _read(self):
        """(table timestamp, mean GFX clock over the XCDs, UCLK).  The
        driver refreshes its metrics table about once a second, so reads in
        between repeat the last update; the timestamp tells updates apart."""
        m = self.smi.amdsmi_get_gpu_metrics_info(self.handle)
        ts = m.get("firmware_timestamp")
        if not isinstance(ts, int):
            ts = m.get("system_clock_counter")
        xcd = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, (int, float)) and 0 < c < 10000]
        g = sum(xcd) / len(xcd) if xcd else m.get("current_gfxclk")
        u = m.get("current_uclk")
        return (ts if isinstance(ts, int) else None,
                float(g) if isinstance(g, (int, float)) else None,
                float(u) if isinstance(u, (int, float)) else None)

    def _run(self):
        while not self._stop.is_set():
            try:
                self.samples.append(self._read())
            except Exception as e:
                self.error = f"{type(e).__name__}: {e}"
                return
            self._stop.wait(self.interval)

    def start(self):
        import threading
        if self.handle is None:
            return
        try:
            self.ts0 = self._read()[0]  # the update current before the work starts
        except Exception as e:
            self.error = f"{type(e).__name__}: {e}"
            return
        self._stop.clear()
        self._thread = threading.Thread(target=self._run, daemon=True)
        self._thread.start()

    def fresh(self):
        """Samples of metric-table updates made after start(), one per update
        (every sample when the driver gives no timestamp)."""
        out, seen = [], {getattr(self, "ts0", None)}
        for ts, g, u in self.samples:
            if ts is None:
                out.append((g, u))
            elif ts not in seen:
                seen.add(ts)
                out.append((g, u))
        return out

    def stop(self):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
            self._thread = None

    def summary(self, extra_steps=0):
        import statistics
        fresh = self.fresh()
        g = [x[0] for x in fresh if x[0]]
        u = [x[1] for x in fresh if x[1]]
        where = "the timed steps" + (f" and {extra_steps} further untimed steps" if extra_steps else "")
        src = ("amdsmi gpu metrics (current_gfxclks averaged over XCDs, current_uclk), one sample per update of "
               "the driver's metrics table (about once a second) during " + where)
        if not g:
            return {"sclk_mhz": None, "mclk_mhz": None, "samples": 0,
                    "error": self.error or "the metrics table was not updated while the work ran", "source": src}
        return {"sclk_mhz": round(statistics.median(g)), "sclk_min_mhz": round(min(g)),
                "sclk_max_mhz": round(max(g)), "mclk_mhz": round(statistics.median(u)) if u else None,
                "samples": len(g), "source": src}


def time_step(step, steps, warmup, stream, clocks=None):
    """Warm up, then (pass 1) time every kernel of `steps` steps with HIP
    events around each, and (pass 2) time exactly `steps` steps with events
    around the dominant kernel only.  Returns (per_kernel, dominant name,
    dominant kernel's average ms in pass 2, wall ms per step of pass 2)."""
    ks = step.kernels()

    def run_step(events=None, only=None):
        for i, (_, fn, _, _) in enumerate(ks):
            timed = events is not None and (only is None or i == only)
            if timed:
                events[0 if only is not None else i][0].record(stream)
            fn()
            if timed:
                events[0 if only is not None else i][1].record(stream)

    for _ in range(warmup):
        run_step()
    torch.cuda.synchronize()

    ev = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] for _ in ks]
          for _ in range(steps)]
    for s in range(steps):
        run_step(ev[s])
    torch.cuda.synchronize()
    per_kernel = {}
    for i, (name, _, work, unit) in enumerate(ks):
        ms = sum(ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(steps)) / steps
        rate = work / (ms * 1e-3) / (1e12 if unit == "TFLOP/s" else 1e9)
        peak = FP8_PEAK_TFLOPS if unit == "TFLOP/s" else HBM_PEAK_GBS
        per_kernel[name] = {"ms": round(ms, 4), "rate": round(rate, 1), "unit": unit,
                            "frac": round(rate / peak, 4), "work": work}
    dom_i = max(range(len(ks)), key=lambda i: per_kernel[ks[i][0]]["ms"])

    ev_dom = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]]
              for _ in range(steps)]
    torch.cuda.synchronize()
    if clocks is not None:
        clocks.start()
    t0 = time.perf_counter()
    for s in range(steps):
        run_step(ev_dom[s], only=dom_i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if clocks is not None:
        # the driver updates its clock readings about once a second: when the
        # timed steps were shorter than two updates, the same steps keep
        # running (untimed) until two more have come or 3 s have passed
        t_end = time.perf_counter() + 3.0
        while clocks.handle is not None and len(clocks.fresh()) < 2 and time.perf_counter() < t_end:
            run_step()
            torch.cuda.synchronize()
            clocks.extra_steps += 1
        clocks.stop()
    ms_per_step = (t1 - t0) * 1e3 / steps
    dom_ms = sum(e[0][0].elapsed_time(e[0][1]) for e in ev_dom) / steps
    return per_kernel, ks[dom_i][0], dom_ms, ms_per_step


def summarize(w, per_kernel, ms_per_step):
    gemm_flops = 3 * 2.0 * w.M * w.N * w.K
    gemm_ms = sum(v["ms"] for v in per_kernel.values() if v["unit"] == "TFLOP/s")
    quant_ms = sum(v["ms"] for v in per_kernel.values() if v["unit"] == "GB/s")
    quant_bytes = sum(v["work"] for v in per_kernel.values() if v["unit"] == "GB/s")
    return {
        "value": gemm_flops / (ms_per_step * 1e-3) / 1e12,
        "gemm_tflops": gemm_flops / (gemm_ms * 1e-3) / 1e12,
        "quant_gbs": quant_bytes / (quant_ms * 1e-3) / 1e9,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(inputs.WORKLOADS))
    ap.add_argument("--extra-workloads", default=EXTRA_WORKLOADS,
                    help="comma-separated dense workloads timed after the main one and reported per config "
                         "('' for none)")
    ap.add_argument("--scale-pad", type=int, default=0,
                    help="floats of padding past roundup4(count) in every scale tensor's row stride")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-digest", action="store_true", help="skip the SHA-256 of the inputs")
    ap.add_argument("--no-ffn-module", action="store_true", help="skip the gated FFN module timing")
    ap.add_argument("--no-mx", action="store_true", help="skip the MXFP8 grouped GEMM timings")
    ap.add_argument("--no-references", action="store_true",
                    help="skip the GEMM reference timings (vendor plain FP8 and MX GEMMs)")
    ap.add_argument("--mx-shapes", default=None,
                    help="comma-separated indices into the MXFP8 shape list (default: all)")
    ap.add_argument("--no-fusion", action="store_true",
                    help="skip the fused gated-activation timings (keeps per-kernel profiles to the step's shapes)")
    ap.add_argument("--no-cold", action="store_true", help="skip the copy reference and the cold-cache quantizers")
    ap.add_argument("--no-graph", action="store_true", help="skip the eager vs HIP-graph timing of the smallest layer")
    ap.add_argument("--cpu-rows", type=int, default=2048,
                    help="tokens of the workload the CPU oracle baseline runs on (capped at M)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="before the workload, run a plain device copy of this many MiB three times "
                         "(a known-size reference for hardware byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the blockwise FP8 hot path here is a single-GPU build "
              "(no collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    w = inputs.WORKLOADS[args.workload]
    if w.fwd_only:
        print("the forward-only workload is a parity case, not a bench line", file=sys.stderr)
        sys.exit(2)
    extras = [x for x in args.extra_workloads.split(",") if x and x != w.name]
    for x in extras:
        if x not in inputs.WORKLOADS or inputs.WORKLOADS[x].fwd_only:
            print(f"unknown or forward-only extra workload {x}", file=sys.stderr)
            sys.exit(2)
    torch.manual_seed(args.seed)
    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20)
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    stream = torch.cuda.current_stream()
    clocks = ClockSampler()

    step = Step(w, seed=args.seed, scale_pad=args.scale_pad)
    ks = step.kernels()
    per_kernel, dom, dom_ms, ms_per_step = time_step(step, args.steps, args.warmup, stream, clocks)
    summ = summarize(w, per_kernel, ms_per_step)
    d = per_kernel[dom]
    dom_rate = d["work"] / (dom_ms * 1e-3) / (1e12 if d["unit"] == "TFLOP/s" else 1e9)
    dom_peak = FP8_PEAK_TFLOPS if d["unit"] == "TFLOP/s" else HBM_PEAK_GBS
    roofline = {
        "kernel": dom,
        "bound": "mfma" if d["unit"] == "TFLOP/s" else "hbm",
        "achieved": round(dom_rate, 1),
        "peak": dom_peak,
        "unit": d["unit"],
        "frac": round(dom_rate / dom_peak, 4),
        "traffic": counter_traffic(w.name, dom, split=dom == "gemm_wgrad" and wgrad_split(w)),
        "avg_ms": round(dom_ms, 4),
        "work_per_launch": d["work"],
    }
    for v in per_kernel.values():
        v.pop("work")
    digest = None if args.no_digest else input_digest(step)
    if step.grouped:
        cfg_groups = step.group_sizes
    else:
        cfg_groups = None

    def median_ms(fn, n=7):
        fn()
        times = []
        for _ in range(n):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        return sorted(times)[n // 2]

    def interleaved_ms(fns, n=7):
        """Median times of several variants of one piece of work, taken in
        alternating order (a, b, ..., a, b, ...) so that the clock and heat
        of the chip, which drift over a run, weigh on each variant alike."""
        for fn in fns:
            fn()
        times = [[] for _ in fns]
        for _ in range(n):
            for i, fn in enumerate(fns):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                torch.cuda.synchronize()
                times[i].append(e0.elapsed_time(e1))
        return [sorted(t)[n // 2] for t in times]

    copy_gbs = cold_gbs = stream_gbs = None
    cold = {}
    stream_ceiling = {}
    if not args.no_cold:
        # Practical HBM reference: a plain device copy of 1 GiB (torch copy_),
        # timed the same way.  The fractions above use the published 8 TB/s peak.
        n_copy = 1 << 30
        src = torch.empty(n_copy, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        for _ in range(5):
            dst.copy_(src)
        c1.record(stream)
        torch.cuda.synchronize()
        copy_gbs = 2 * n_copy * 5 / (c0.elapsed_time(c1) * 1e-3) / 1e9

        # Quantizers on cold caches: before each timed call, reading the 1 GiB
        # scratch buffer evicts the inputs from L2 and the 256 MB last-level
        # cache, so the rate is the HBM-bound one (median of 5).  The flush
        # reads rather than writes: a written flush leaves the caches full of
        # dirty lines, and writing those back would be charged to the
        # quantizer.  Inside the step they may find part of their input cached.
        flush_src = src.view(torch.int32)
        flush_sink = torch.empty((), dtype=torch.int64, device="cuda")
        for name, fn, work, unit in ks:
            if unit != "GB/s":
                continue
            times = []
            for r in range(5):
                torch.sum(flush_src, dim=(0,), dtype=torch.int64, out=flush_sink)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1))
            ms = sorted(times)[len(times) // 2]
            rate = work / (ms * 1e-3) / 1e9
            cold[name] = {"ms": round(ms, 4), "rate": round(rate, 1), "unit": "GB/s",
                          "frac": round(rate / HBM_PEAK_GBS, 4), "work": work}
        cold_gbs = sum(v["work"] for v in cold.values()) / (sum(v["ms"] for v in cold.values()) * 1e-3) / 1e9
        for v in cold.values():
            v.pop("work")
        # The practical ceiling of each quantizer pass: the streaming
        # reference kernel (bs_diag_stream, the quantizers' access pattern)
        # moving the same bytes -- the bf16 input read, the codes and scales
        # written -- timed cold the same way.
        stream_ceiling = {}
        for name, _, work, unit in ks:
            if unit != "GB/s":
                continue
            n_read = step.quant_read_bytes[name] // 16 * 16
            n_write = int(work - step.quant_read_bytes[name]) // 16 * 16
            s_src = src[:n_read] if n_read <= src.numel() else torch.empty(n_read, dtype=torch.uint8, device="cuda")
            s_dst = torch.empty(max(n_write, n_read), dtype=torch.uint8, device="cuda")
            n_write = max(n_write, n_read)
            times = []
            for r in range(5):
                torch.sum(flush_src, dim=(0,), dtype=torch.int64, out=flush_sink)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                bs.bs_diag_stream(s_src, n_read, s_dst, n_write)
                e1.record(stream)
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1))
            ms = sorted(times)[len(times) // 2]
            stream_ceiling[name] = {"ms": round(ms, 4), "gbs": round((n_read + n_write) / (ms * 1e-3) / 1e9, 1),
                                    "bytes": n_read + n_write}
            del s_src, s_dst
        stream_gbs = sum(v["bytes"] for v in stream_ceiling.values()) / \
            (sum(v["ms"] for v in stream_ceiling.values()) * 1e-3) / 1e9
        del src, dst, flush_src
    del step, ks
    torch.cuda.empty_cache()

    # The dense workloads (one linear layer's forward, dgrad and wgrad): each
    # timed the same way, with fewer steps; the gated FFN module at the same
    # sizes (tokens M, dim K, hidden N) when asked for.
    extra = {}
    ffn = []
    fusion = fusion_bwd = None
    for x in extras:
        wx = inputs.WORKLOADS[x]
        sx = Step(wx, seed=args.seed, scale_pad=args.scale_pad)
        pk, dx, dmx, msx = time_step(sx, min(args.steps, 20), min(args.warmup, 3), stream)
        sm = summarize(wx, pk, msx)
        extra[x] = {"ms_per_step": round(msx, 4), "value": round(sm["value"], 1), "unit": "TFLOP/s",
                    "gemm_tflops": round(sm["gemm_tflops"], 1), "quant_gbs": round(sm["quant_gbs"], 1),
                    "kernels": {k: {kk: vv for kk, vv in v.items() if kk != "work"} for k, v in pk.items()}}
        if not args.no_fusion:
            # The forward GEMM's epilogue quantizing its own bf16 output for
            # the next layer (1x128 rows + transposed columns), against the
            # GEMM followed by the separate quantizer pass over D.
            Mx, Nx = wx.M, wx.N
            qr_ = torch.empty((Mx, Nx), dtype=torch.uint8, device="cuda")
            sr_ = bs.empty_scales(Nx // 128, Mx, "cuda")
            qc_ = torch.empty((Nx, Mx), dtype=torch.uint8, device="cuda")
            sc_ = bs.empty_scales(Mx // 128, Nx, "cuda")
            fargs = (sx.qa, sx.sa, sx.qw, sx.sw, bs.BS_SCALE_128X128)

            def sep():
                bs.bs_scaled_mm(*fargs, out=sx.out)
                bs.bs_quant_1x128(sx.out, qr_, sr_, qc_, sc_)

            def fused_q():
                bs.bs_scaled_mm_quant(*fargs, q_row=qr_, s_row=sr_, q_col=qc_, s_col=sc_)

            def fused_qd():
                bs.bs_scaled_mm_quant(*fargs, out=sx.out, q_row=qr_, s_row=sr_, q_col=qc_, s_col=sc_)

            s_ms, q_ms, qd_ms = interleaved_ms([sep, fused_q, fused_qd])
            extra[x]["gemm_quant_epilogue"] = {
                "separate_ms": round(s_ms, 4), "fused_ms": round(q_ms, 4), "fused_with_d_ms": round(qd_ms, 4),
                "speedup": round(s_ms / q_ms, 3), "speedup_with_d": round(s_ms / qd_ms, 3)}
            del qr_, sr_, qc_, sc_
        if not args.no_fusion and fusion is None:
            # Fusion next to the path: the FFN's gated activation h = silu(a) * b
            # quantized for the next layer (rows + transposed columns), fused in
            # one kernel versus torch's silu and mul followed by the quantizer.
            # a, b are [M, N] bf16 (the step's output and grad_out buffers).
            fa, fb = sx.out, sx.gout
            M_, N_ = fa.shape

            def fused():
                bs.bs_swiglu_quant_1x128(fa, fb, None, sx.qg, sx.sg, sx.qgT, sx.sgT)

            def unfused():
                h = torch.nn.functional.silu(fa) * fb
                bs.bs_quant_1x128(h, sx.qg, sx.sg, sx.qgT, sx.sgT)

            f_ms, u_ms = interleaved_ms([fused, unfused])
            f_bytes = M_ * N_ * (2 + 2 + 1 + 1) + 4 * (M_ * N_ // 128) * 2
            fusion = {"shape": [M_, N_], "fused_ms": round(f_ms, 4), "unfused_ms": round(u_ms, 4),
                      "fused_gbs": round(f_bytes / (f_ms * 1e-3) / 1e9, 1), "speedup": round(u_ms / f_ms, 2)}
            # ... and its backward: [da | db] from a, b, dh quantized (rows +
            # columns of the [M, 2N] matrix) in one kernel, versus the same
            # float32 arithmetic in torch followed by the quantizer.
            fd = inputs.bf16_normal((M_, N_), 0.01, args.seed + 30).cuda()
            qd = torch.empty((M_, 2 * N_), dtype=torch.uint8, device="cuda")
            sd = bs.empty_scales(2 * N_ // 128, M_, "cuda")
            qdt = torch.empty((2 * N_, M_), dtype=torch.uint8, device="cuda")
            sdt = bs.empty_scales(M_ // 128, 2 * N_, "cuda")
            dab = torch.empty((M_, 2 * N_), dtype=torch.bfloat16, device="cuda")

            def fused_bwd():
                bs.bs_swiglu_bwd_quant_1x128(fa, fb, fd, None, qd, sd, qdt, sdt)

            def unfused_bwd():
                a32, b32, d32 = fa.float(), fb.float(), fd.float()
                sig = torch.sigmoid(a32)
                dab[:, :N_] = d32 * b32 * sig * (1.0 + a32 * (1.0 - sig))
                dab[:, N_:] = d32 * a32 * sig
                bs.bs_quant_1x128(dab, qd, sd, qdt, sdt)

            fb_ms, ub_ms = interleaved_ms([fused_bwd, unfused_bwd])
            fb_bytes = M_ * N_ * (3 * 2 + 4 * 1) + 4 * (2 * M_ * N_ // 128) * 2
            fusion_bwd = {"shape": [M_, N_], "fused_ms": round(fb_ms, 4), "unfused_ms": round(ub_ms, 4),
                          "fused_gbs": round(fb_bytes / (fb_ms * 1e-3) / 1e9, 1),
                          "speedup": round(ub_ms / fb_ms, 2)}
            del qd, qdt, dab, fd
        del sx
        torch.cuda.empty_cache()
        # The gated FFN out_proj(silu(w1 x) * w2 x) as one module (shared
        # input quantization, stacked w1/w2 GEMMs, the fused activation
        # quantizers) against three Float8BlockwiseLinear layers with torch's
        # silu and mul: one forward + backward each.
        if not args.no_ffn_module and wx.N % 512 == 0:
            ffn.append(ffn_module_timing(wx.M, wx.K, wx.N, interleaved_ms, args.seed))
            torch.cuda.empty_cache()

    # MXFP8 grouped GEMMs (the pages' MoE recipe) at the pages' shapes,
    # forward and forward + backward with quantization, next to bf16
    mxfp8 = None
    if not args.no_mx:
        which = None if args.mx_shapes is None else {int(i) for i in args.mx_shapes.split(",")}
        mxfp8 = mx_grouped_timing(median_ms, args.seed, which)

    # the forward GEMM next to the vendor's plain FP8 GEMM and the MX GEMM
    references = None
    if not args.no_references:
        references = gemm_reference_timing(interleaved_ms, args.seed)

    graph = None
    if not args.no_graph:
        graph = launch_bound_timing(args.seed)

    cpu = None
    if not args.no_cpu_baseline:
        tflops, secs, desc = cpu_oracle_sample(w, rows=min(args.cpu_rows, w.M), seed=args.seed)
        cpu = {"value": round(tflops, 6), "unit": "TFLOP/s", "cores": blas_threads(), "kind": "oracle",
               "sample": desc, "seconds": round(secs, 2)}

    cfg = {"workload": w.name, "M": w.M, "K": w.K, "N": w.N, "G": w.G,
           "step": "quant A/W/W^T/grad_out + fwd, dgrad, wgrad GEMMs" +
                   (" (grouped: GROUP_M fwd/dgrad, GROUP_K wgrad)" if w.G > 1 else "")}
    if cfg_groups is not None:
        cfg["group_sizes"] = cfg_groups
    if args.scale_pad:
        cfg["scale_pad"] = args.scale_pad
    line = {
        "metric": "FP8 blockwise GEMM TFLOP/s fwd+bwd, % of FP8 MFMA peak; quantizer GB/s",
        "value": round(summ["value"], 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate)",
        "data": "synthetic (seeded N(0, s) bf16, resident in HBM)",
        "config": cfg,
        "gemm_tflops": round(summ["gemm_tflops"], 1),
        "gemm_frac_of_peak": round(summ["gemm_tflops"] / FP8_PEAK_TFLOPS, 4),
        "quant_gbs": round(summ["quant_gbs"], 1),
        "quant_frac_of_hbm": round(summ["quant_gbs"] / HBM_PEAK_GBS, 4),
        "clocks": clocks.summary(clocks.extra_steps),
        "inputs_sha256": digest,
        "hbm_copy_gbs": None if copy_gbs is None else round(copy_gbs, 1),
        "quant_frac_of_copy": None if copy_gbs is None else round(summ["quant_gbs"] / copy_gbs, 4),
        "quant_cold_gbs": None if cold_gbs is None else round(cold_gbs, 1),
        "quant_cold_frac_of_hbm": None if cold_gbs is None else round(cold_gbs / HBM_PEAK_GBS, 4),
        "quant_cold": cold,
        "stream_ceiling_gbs": None if stream_gbs is None else round(stream_gbs, 1),
        "quant_cold_frac_of_stream": None if stream_gbs is None else round(cold_gbs / stream_gbs, 4),
        "stream_ceiling": stream_ceiling,
        "kernels": per_kernel,
        "extra_configs": extra,
        "swiglu_quant_fusion": fusion,
        "swiglu_bwd_quant_fusion": fusion_bwd,
        "gated_ffn_module": ffn,
        "mxfp8_grouped_mm": mxfp8,
        "gemm_references": references,
        "launch_bound_graph": graph,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
