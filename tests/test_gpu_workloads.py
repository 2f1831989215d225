"""Parity at the full workload sizes, in the launch configuration bench.py times.

One training step of each workload runs on the GPU through bench.Step (the
same buffers and calls the bench times).  The oracle then recomputes sampled
pieces from the same bf16 inputs: whole quantization blocks (bit-exact codes
and scales) and individual GEMM outputs (within 2e-3 * ||a_m|| * ||b_n||),
each from its own quantization of exactly the rows/columns it needs.
"""

import numpy as np
import pytest
import torch

import bench
from blockwise_scaled_fp8_bs_amd import inputs
from oracle import gemm, quant
from gpu_support import bits16, need_gpu

pytestmark = [pytest.mark.gpu, pytest.mark.big]

N_SAMPLE = 24


def rows_cpu(t, idx):
    return t[torch.as_tensor(idx, device=t.device)].cpu()


def cols_cpu(t, idx):
    return t[:, torch.as_tensor(idx, device=t.device)].cpu()


def logical_rowscale(s_phys, row):
    """1x128 K-major scales of one row: s_phys[:, row] as a [1, nkb] array."""
    return s_phys[:, row].cpu().numpy()[None, :]


@pytest.fixture(scope="module", params=["dense_8192x4096x4096", "ffn_up_16384x5120x8192",
                                        "ffn_down_16384x7168x2048", "moe_128000x5120x8192_g8"])
def stepped(request):
    need_gpu()
    w = inputs.WORKLOADS[request.param]
    print(f"workload {w.name}: building inputs and running one step", flush=True)
    st = bench.Step(w, seed=0)
    for _, fn, _, _ in st.kernels():
        fn()
    torch.cuda.synchronize()
    yield st
    del st
    torch.cuda.empty_cache()


def group_of(st, m):
    if not st.grouped:
        return 0
    return int(np.searchsorted(np.asarray(st.ends.cpu()), m, side="right"))


def sample_rows(rng, M, st):
    base = list(rng.choice(M, N_SAMPLE, replace=False))
    if st.grouped:  # rows on both sides of every group boundary
        for e in st.ends.cpu().tolist()[:-1]:
            base += [max(e - 1, 0), min(e, M - 1)]
    return sorted(set(int(m) for m in base))


def test_activation_quantizers(stepped):
    st, w = stepped, stepped.w
    rng = np.random.default_rng(1)
    rows = sample_rows(rng, w.M, st)
    for x, q, s, name in [(st.a, st.qa, st.sa, "A"), (st.gout, st.qg, st.sg, "grad_out")]:
        xb = bits16(rows_cpu(x, rows))
        q_ref, s_ref = quant.quant_1x128_rowwise(xb)
        assert np.array_equal(rows_cpu(q, rows).numpy(), q_ref), f"{name} row codes"
        got_s = s[:, torch.as_tensor(rows, device=s.device)].cpu().numpy().T
        assert np.array_equal(got_s.view(np.uint32), s_ref.view(np.uint32)), f"{name} row scales"
    # transposed column outputs: whole 128-row blocks of a few columns
    for x, qT, sT, C, name in [(st.a, st.qaT, st.saT, w.K, "A^T"), (st.gout, st.qgT, st.sgT, w.N, "grad_out^T")]:
        cols = sorted(set(int(c) for c in rng.choice(C, 12, replace=False)) | {0, C - 1})
        for rb in sorted(set(int(r) for r in rng.choice(w.M // 128, 3, replace=False)) | {w.M // 128 - 1}):
            blk = x[rb * 128:(rb + 1) * 128][:, torch.as_tensor(cols, device=x.device)].cpu()
            q_ref, s_ref = quant.quant_1x128_colwise(bits16(blk))
            got_q = qT[torch.as_tensor(cols, device=qT.device), rb * 128:(rb + 1) * 128].cpu().numpy()
            assert np.array_equal(got_q, q_ref), f"{name} codes, row block {rb}"
            got_s = sT[rb, torch.as_tensor(cols, device=sT.device)].cpu().numpy()
            assert np.array_equal(got_s.view(np.uint32), s_ref[:, 0].view(np.uint32)), f"{name} scales"


def test_weight_quantizers(stepped):
    st, w = stepped, stepped.w
    rng = np.random.default_rng(2)
    G, N, K = w.G, w.N, w.K
    for rbg in sorted(set(int(r) for r in rng.choice(G * N // 128, 3, replace=False)) | {G * N // 128 - 1}):
        blk = st.wv[rbg * 128:(rbg + 1) * 128].cpu()
        q_ref, s_ref = quant.quant_128x128(bits16(blk))
        assert np.array_equal(st.qw[rbg * 128:(rbg + 1) * 128].cpu().numpy(), q_ref)
        assert np.array_equal(st.sw[:, rbg].cpu().numpy().view(np.uint32), s_ref[0].view(np.uint32))
        g, rb = divmod(rbg, N // 128)
        # transposed copy of the same tiles: q^T[g][:, rb*128 : +128], scales s^T[g][rb, :]
        assert np.array_equal(st.qwT[g][:, rb * 128:(rb + 1) * 128].cpu().numpy(), q_ref.T)
        assert np.array_equal(st.swT[g, rb, :K // 128].cpu().numpy().view(np.uint32), s_ref[0].view(np.uint32))


def _w_rows_deq(st, g, rows):
    """Dequantized rows of expert g's W (each from its whole 128-row tile)."""
    out = []
    for n in rows:
        rb = n // 128
        blk = st.w3[g, rb * 128:(rb + 1) * 128].cpu()
        q, s = quant.quant_128x128(bits16(blk))
        out.append(gemm.dequant(q, s, 128)[n % 128])
    return np.stack(out)


def _w_cols_deq(st, g, cols):
    """Dequantized columns of expert g's W, i.e. rows of W^T (128x128 tiles)."""
    out = []
    for k in cols:
        kb = k // 128
        blk = st.w3[g, :, kb * 128:(kb + 1) * 128].cpu()
        q, s = quant.quant_128x128(bits16(blk))
        out.append(gemm.dequant(q, s, 128)[:, k % 128])
    return np.stack(out)


def _check(d, ref, a, b, what):
    ok, worst = gemm.check_close(d, ref, a, b)
    assert ok, f"{what}: worst |err|/bound {worst}"
    return worst


def test_forward_and_dgrad_gemms(stepped):
    st, w = stepped, stepped.w
    rng = np.random.default_rng(3)
    ms = sample_rows(rng, w.M, st)
    ns = sorted(set(int(n) for n in rng.choice(w.N, 8, replace=False)) | {0, w.N - 1})
    ks = sorted(set(int(k) for k in rng.choice(w.K, 8, replace=False)) | {0, w.K - 1})
    a_q, a_s = quant.quant_1x128_rowwise(bits16(rows_cpu(st.a, ms)))
    g_q, g_s = quant.quant_1x128_rowwise(bits16(rows_cpu(st.gout, ms)))
    a_deq = gemm.dequant(a_q, a_s, 1)
    g_deq = gemm.dequant(g_q, g_s, 1)
    out = rows_cpu(st.out, ms).float().numpy().astype(np.float64)
    gin = rows_cpu(st.gin, ms).float().numpy().astype(np.float64)
    groups = [group_of(st, m) for m in ms]
    for g in sorted(set(groups)):
        sel = [i for i, gg in enumerate(groups) if gg == g]
        wn = _w_rows_deq(st, g, ns)                  # [len(ns), K]
        wk = _w_cols_deq(st, g, ks)                  # [len(ks), N]
        _check(out[np.ix_(sel, ns)], a_deq[sel] @ wn.T, a_deq[sel], wn, f"{w.name} forward, group {g}")
        _check(gin[np.ix_(sel, ks)], g_deq[sel] @ wk.T, g_deq[sel], wk, f"{w.name} dgrad, group {g}")


def test_wgrad_gemm(stepped):
    st, w = stepped, stepped.w
    rng = np.random.default_rng(4)
    ns = sorted(set(int(n) for n in rng.choice(w.N, 10, replace=False)) | {0, w.N - 1})
    ks = sorted(set(int(k) for k in rng.choice(w.K, 10, replace=False)) | {0, w.K - 1})
    gq, gs = quant.quant_1x128_colwise(bits16(cols_cpu(st.gout, ns)))   # [len(ns), M]
    aq, as_ = quant.quant_1x128_colwise(bits16(cols_cpu(st.a, ks)))     # [len(ks), M]
    ends = st.ends.cpu().tolist() if st.grouped else [w.M]
    start = 0
    for g, e in enumerate(ends):
        d = st.gw[g] if st.grouped else st.gw
        got = d[torch.as_tensor(ns, device=d.device)][:, torch.as_tensor(ks, device=d.device)]
        got = got.float().cpu().numpy().astype(np.float64)
        if e == start:
            assert np.all(got == 0), f"empty group {g} must be zero"
            continue
        a = gemm.dequant(gq[:, start:e], gs[:, start // 128:e // 128], 1)
        b = gemm.dequant(aq[:, start:e], as_[:, start // 128:e // 128], 1)
        _check(got, a @ b.T, a, b, f"{w.name} wgrad, group {g}")
        start = e


def test_linear_forward_256x512x256_full():
    """The small forward workload, every output element against the oracle
    (W scales K-major with ld 4, padded from 2)."""
    need_gpu()
    import blockwise_scaled_fp8_bs_amd as bs
    w = inputs.WORKLOADS["linear_fwd_256x512x256"]
    a, wt, _, _ = inputs.make_operands(w, seed=0)
    qa = torch.empty((256, 512), dtype=torch.uint8, device="cuda")
    sa = bs.empty_scales(4, 256, "cuda")
    qw = torch.empty((256, 512), dtype=torch.uint8, device="cuda")
    sw = bs.empty_scales(4, 2, "cuda")
    assert sw.stride(0) == 4
    bs.bs_quant_1x128(a.cuda(), qa, sa)
    bs.bs_quant_128x128(wt.cuda(), qw, sw)
    out = bs.bs_scaled_mm(qa, sa, qw, sw, bs.BS_SCALE_128X128)
    torch.cuda.synchronize()
    qa_r, sa_r = quant.quant_1x128_rowwise(bits16(a))
    qw_r, sw_r = quant.quant_128x128(bits16(wt))
    assert np.array_equal(qa.cpu().numpy(), qa_r) and np.array_equal(qw.cpu().numpy(), qw_r)
    assert np.array_equal(sw[:, :2].cpu().numpy(), sw_r.T)
    ad, wd = gemm.dequant(qa_r, sa_r, 1), gemm.dequant(qw_r, sw_r, 128)
    _check(out.float().cpu().numpy().astype(np.float64), ad @ wd.T, ad, wd, "linear forward")
