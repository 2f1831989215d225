"""Parity at the full workload sizes, in the launch configuration bench.py times.

One training step of each workload runs on the GPU through bench.Step (the
same buffers and calls the bench times).  The oracle then quantizes the same
bf16 inputs itself (tests/fullsize.py spreads its blocks over the host cores)
and:

* dense workloads (8192x4096x4096, 16384x5120x8192, 16384x7168x2048, and the
  last once more with every scale row stride padded 4 floats past
  roundup4(count)): EVERY code and EVERY scale of the four quantizer outputs
  bit-exact, scale padding untouched (NaN canary), and EVERY element of the
  forward, dgrad and wgrad outputs within 2e-3 * ||a_m|| * ||b_n|| of the
  oracle's float64 product of its own dequantized operands;
* the MoE workload (128000 tokens, 8 experts of 8192x5120, random group
  sizes): every weight code and scale in both layouts; 64 full 128-token
  panels of the activation and grad_out quantizers (rows, and the transposed
  columns of the same tokens) and of the forward and dgrad outputs (all
  columns) -- both sides of every group boundary, the first and last panel,
  the rest seeded at random -- and 64 full 128-row panels of the wgrad output
  (8 per non-empty expert, all columns), with every element of an empty
  expert's output checked to be zero.
"""

import numpy as np
import pytest
import torch

import bench
import fullsize
from blockwise_scaled_fp8_bs_amd import inputs
from gpu_support import CANARY_F32_BITS, bits16, need_gpu
from oracle import gemm, quant

pytestmark = [pytest.mark.gpu, pytest.mark.big]

DENSE = [("dense_8192x4096x4096", 0), ("ffn_up_16384x5120x8192", 0), ("ffn_down_16384x7168x2048", 0),
         ("ffn_down_16384x7168x2048", 4)]


def _canary(t):
    t.view(torch.int32).fill_(CANARY_F32_BITS)


def _f32bits(t):
    return t.contiguous().numpy().view(np.uint32)


def _check_scales(got, ref_logical, count, name):
    """got: K-major [nkb, ld] host tensor; ref_logical [count, nkb].  Every
    logical scale bit-exact, every padding entry still the canary."""
    g = _f32bits(got)
    assert np.array_equal(g[:, :count], np.ascontiguousarray(ref_logical.T).view(np.uint32)), f"{name} scales"
    assert np.all(g[:, count:] == CANARY_F32_BITS), f"{name}: scale padding was written"


class Run:
    """Host copies of one executed step: inputs (bf16 bits) and outputs."""


def _run_step(w, pad):
    print(f"full-size step: workload {w.name}, scale pad {pad}", flush=True)
    st = bench.Step(w, seed=0, scale_pad=pad)
    for t in (st.sa, st.saT, st.sg, st.sgT, st.sw, st.swT):
        _canary(t)
    for _, fn, _, _ in st.kernels():
        fn()
    torch.cuda.synchronize()
    return st


@pytest.fixture(scope="module", params=DENSE, ids=[f"{n}-pad{p}" for n, p in DENSE])
def dense_run(request):
    need_gpu()
    name, pad = request.param
    w = inputs.WORKLOADS[name]
    st = _run_step(w, pad)
    assert st.sa.stride(0) == (w.M + 3) // 4 * 4 + pad and st.swT.stride(1) == (w.K // 128 + 3) // 4 * 4 + pad
    r = Run()
    r.w, r.pad = w, pad
    r.a, r.wt, r.g = bits16(st.a), bits16(st.wt), bits16(st.gout)
    for k in ("qa", "sa", "qaT", "saT", "qg", "sg", "qgT", "sgT", "qw", "sw", "qwT", "swT"):
        setattr(r, k, getattr(st, k).cpu())
    r.out = st.out.float().cpu().numpy()
    r.gin = st.gin.float().cpu().numpy()
    r.gw = st.gw.float().cpu().numpy()
    del st
    torch.cuda.empty_cache()
    r.ref = {}
    yield r


def _oracle(r, key):
    """The oracle's own quantization of the run's bf16 inputs (memoized)."""
    if key not in r.ref:
        r.ref[key] = {
            "a_row": lambda: fullsize.quant_rowwise(r.a),
            "a_col": lambda: fullsize.quant_colwise(r.a),
            "g_row": lambda: fullsize.quant_rowwise(r.g),
            "g_col": lambda: fullsize.quant_colwise(r.g),
            "w": lambda: fullsize.quant_128x128(r.wt),
        }[key]()
    return r.ref[key]


def test_dense_quantizers_every_code_and_scale(dense_run):
    r, w = dense_run, dense_run.w
    M, K, N = w.M, w.K, w.N
    q, s = _oracle(r, "a_row")
    assert np.array_equal(r.qa.numpy(), q), "A row codes"
    _check_scales(r.sa, s, M, "A row")
    q, s = _oracle(r, "a_col")
    assert np.array_equal(r.qaT.numpy(), q), "A^T codes"
    _check_scales(r.saT, s, K, "A^T")
    q, s = _oracle(r, "g_row")
    assert np.array_equal(r.qg.numpy(), q), "grad_out row codes"
    _check_scales(r.sg, s, M, "grad_out row")
    q, s = _oracle(r, "g_col")
    assert np.array_equal(r.qgT.numpy(), q), "grad_out^T codes"
    _check_scales(r.sgT, s, N, "grad_out^T")
    q, s = _oracle(r, "w")
    assert np.array_equal(r.qw.numpy(), q), "W codes (forward layout)"
    _check_scales(r.sw, s, N // 128, "W")
    # the dgrad layout: q^T[0] = codes of W transposed, s^T[0][rb, cb] = scale of tile (rb, cb)
    assert np.array_equal(r.qwT[0].numpy(), q.T), "W^T codes (dgrad layout)"
    st = _f32bits(r.swT[0])
    assert np.array_equal(st[:, :K // 128], s.view(np.uint32)), "W^T scales"
    assert np.all(st[:, K // 128:] == CANARY_F32_BITS), "W^T scale padding was written"


def test_dense_forward_every_output(dense_run):
    r = dense_run
    qa, sa = _oracle(r, "a_row")
    qw, sw = _oracle(r, "w")
    worst = fullsize.check_gemm(r.out, fullsize.dequant(qa, sa, 1), fullsize.dequant(qw, sw, 128),
                                what=f"{r.w.name} forward")
    print(f"{r.w.name} forward: worst |err|/bound {worst:.3f}")


def test_dense_dgrad_every_output(dense_run):
    r = dense_run
    qg, sg = _oracle(r, "g_row")
    qw, sw = _oracle(r, "w")
    # the dgrad operand W^T holds W's codes and tile scales transposed (the
    # oracle's 3-D colwise quantizer is defined that way), so its dequantized
    # form is the transpose of W's
    wt_deq = np.ascontiguousarray(fullsize.dequant(qw, sw, 128).T)
    worst = fullsize.check_gemm(r.gin, fullsize.dequant(qg, sg, 1), wt_deq, what=f"{r.w.name} dgrad")
    print(f"{r.w.name} dgrad: worst |err|/bound {worst:.3f}")


def test_dense_wgrad_every_output(dense_run):
    r = dense_run
    qgt, sgt = _oracle(r, "g_col")
    qat, sat = _oracle(r, "a_col")
    worst = fullsize.check_gemm(r.gw, fullsize.dequant(qgt, sgt, 1), fullsize.dequant(qat, sat, 1),
                                what=f"{r.w.name} wgrad")
    print(f"{r.w.name} wgrad: worst |err|/bound {worst:.3f}")
    r.ref.clear()  # last test of this run: release the oracle's arrays


# ----------------------------------------------------------------------------
# MoE: 128000 tokens, 8 experts
# ----------------------------------------------------------------------------

N_PANELS = 64


@pytest.fixture(scope="module")
def moe_run():
    need_gpu()
    w = inputs.WORKLOADS["moe_128000x5120x8192_g8"]
    st = _run_step(w, 0)
    M, K, N, G = w.M, w.K, w.N, w.G
    r = Run()
    r.w = w
    r.ends = st.ends.cpu().tolist()
    starts = [0] + r.ends[:-1]
    r.bounds = list(zip(starts, r.ends))
    # token panels: both sides of every group boundary, first and last, the rest random
    npan = M // 128
    pick = {0, npan - 1}
    for e in r.ends[:-1]:
        pick |= {p for p in (e // 128 - 1, e // 128) if 0 <= p < npan}
    rng = np.random.default_rng(5)
    while len(pick) < N_PANELS:
        pick.add(int(rng.integers(0, npan)))
    r.panels = sorted(pick)
    idx = torch.as_tensor(np.concatenate([np.arange(p * 128, (p + 1) * 128) for p in r.panels]), device="cuda")
    r.rows = idx.cpu().numpy()
    r.a = bits16(st.a.index_select(0, idx))
    r.g = bits16(st.gout.index_select(0, idx))
    r.wt = bits16(st.wt)                                   # [G, N, K]
    r.qa = st.qa.index_select(0, idx).cpu().numpy()
    r.sa = st.sa.index_select(1, idx).cpu()                # [K/128, rows]
    r.qg = st.qg.index_select(0, idx).cpu().numpy()
    r.sg = st.sg.index_select(1, idx).cpu()
    r.qaT = st.qaT.index_select(1, idx).cpu().numpy()      # [K, rows]
    pidx = torch.as_tensor(r.panels, device="cuda")
    r.saT = st.saT.index_select(0, pidx).cpu()              # [panels, ld]
    r.qgT = st.qgT.index_select(1, idx).cpu().numpy()
    r.sgT = st.sgT.index_select(0, pidx).cpu()
    r.qw, r.sw, r.qwT, r.swT = st.qw.cpu().numpy(), st.sw.cpu(), st.qwT.cpu().numpy(), st.swT.cpu()
    r.out = st.out.index_select(0, idx).float().cpu().numpy()
    r.gin = st.gin.index_select(0, idx).float().cpu().numpy()
    # wgrad panels: the same 8 row panels (of N) of every non-empty expert;
    # empty experts whole.  Host copies of the wgrad inputs: all of A and the
    # panels' columns of grad_out.
    ps = sorted({0, N // 128 - 1} | {int(x) for x in rng.choice(np.arange(1, N // 128 - 1), 6, replace=False)})
    r.gw_panels = ps
    cols = torch.as_tensor(np.concatenate([np.arange(p * 128, (p + 1) * 128) for p in ps]), device="cuda")
    r.gw, r.gw_empty = {}, {}
    for g, (s0, e0) in enumerate(r.bounds):
        if e0 == s0:
            r.gw_empty[g] = st.gw[g].float().cpu().numpy()
        else:
            r.gw[g] = st.gw[g].index_select(0, cols).float().cpu().numpy()
    r.a_all = bits16(st.a)                                  # [M, K]
    r.g_cols = bits16(st.gout.index_select(1, cols))        # [M, 8 * 128]
    del st
    torch.cuda.empty_cache()
    yield r


def _group_of_row(r, m):
    for g, (s0, e0) in enumerate(r.bounds):
        if s0 <= m < e0:
            return g
    raise AssertionError(m)


def test_moe_weight_quantizers_every_code_and_scale(moe_run):
    r, w = moe_run, moe_run.w
    G, N, K = w.G, w.N, w.K
    q, s = fullsize.quant_128x128(r.wt.reshape(G * N, K))
    assert np.array_equal(r.qw, q), "expert weight codes (stacked forward layout)"
    _g = _f32bits(r.sw)
    assert np.array_equal(_g[:, :G * N // 128], np.ascontiguousarray(s.T).view(np.uint32)), "expert weight scales"
    for g in range(G):
        qg_ = q[g * N:(g + 1) * N]
        sg_ = s[g * N // 128:(g + 1) * N // 128]
        assert np.array_equal(r.qwT[g], qg_.T), f"expert {g} transposed codes"
        assert np.array_equal(_f32bits(r.swT[g])[:, :K // 128], sg_.view(np.uint32)), f"expert {g} transposed scales"
    r.w_ref = (q, s)


def test_moe_activation_quantizers_panels(moe_run):
    r, w = moe_run, moe_run.w
    for bits, qrow, srow, qcol, scol, C, name in ((r.a, r.qa, r.sa, r.qaT, r.saT, w.K, "A"),
                                                  (r.g, r.qg, r.sg, r.qgT, r.sgT, w.N, "grad_out")):
        q, s = fullsize.quant_rowwise(bits)
        assert np.array_equal(qrow, q), f"{name} row codes"
        assert np.array_equal(_f32bits(srow), np.ascontiguousarray(s.T).view(np.uint32)), f"{name} row scales"
        # transposed columns: each panel is one 128-token block of every column
        q, s = fullsize.quant_colwise(bits)            # [C, panels*128], [C, panels]
        assert np.array_equal(qcol, q), f"{name}^T codes"
        assert np.array_equal(_f32bits(scol)[:, :C], np.ascontiguousarray(s.T).view(np.uint32)), f"{name}^T scales"


def _w_deq(r, g):
    if not hasattr(r, "w_ref"):
        w = r.w
        r.w_ref = fullsize.quant_128x128(r.wt.reshape(w.G * w.N, w.K))
    q, s = r.w_ref
    N = r.w.N
    return fullsize.dequant(q[g * N:(g + 1) * N], s[g * N // 128:(g + 1) * N // 128], 128)


def test_moe_forward_and_dgrad_panels(moe_run):
    r = moe_run
    qa, sa = fullsize.quant_rowwise(r.a)
    qg, sg = fullsize.quant_rowwise(r.g)
    a_deq, g_deq = gemm.dequant(qa, sa, 1), gemm.dequant(qg, sg, 1)
    owner = np.array([_group_of_row(r, int(m)) for m in r.rows[::128]]).repeat(128)
    worst = 0.0
    for g in sorted(set(owner.tolist())):
        sel = np.flatnonzero(owner == g)
        wd = _w_deq(r, g)                                   # [N, K]
        worst = max(worst, fullsize.check_gemm(r.out[sel], a_deq, wd, rows=sel, what=f"MoE forward, expert {g}"))
        wtd = np.ascontiguousarray(wd.T)                    # [K, N]
        worst = max(worst, fullsize.check_gemm(r.gin[sel], g_deq, wtd, rows=sel, what=f"MoE dgrad, expert {g}"))
    print(f"MoE forward/dgrad, {len(r.panels)} panels: worst |err|/bound {worst:.3f}")


def test_moe_wgrad_panels_and_empty_experts(moe_run):
    r = moe_run
    for g, d in r.gw_empty.items():
        assert np.all(d == 0), f"empty expert {g}: wgrad output must be zero"
    assert len(r.gw_panels) * len(r.gw) + 8 * len(r.gw_empty) >= N_PANELS
    worst = 0.0
    for g, d in r.gw.items():
        s0, e0 = r.bounds[g]
        qgt, sgt = fullsize.quant_colwise(r.g_cols[s0:e0])   # [8*128, T_g]
        qat, sat = fullsize.quant_colwise(r.a_all[s0:e0])    # [K, T_g]
        worst = max(worst, fullsize.check_gemm(d, fullsize.dequant(qgt, sgt, 1), fullsize.dequant(qat, sat, 1),
                                               what=f"MoE wgrad, expert {g}"))
    print(f"MoE wgrad, {len(r.gw_panels)} panels of each of {len(r.gw)} experts: worst |err|/bound {worst:.3f}")


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
    assert np.array_equal(sa[:, :256].cpu().numpy(), sa_r.T)
    assert np.array_equal(sw[:, :2].cpu().numpy(), sw_r.T)
    ad, wd = gemm.dequant(qa_r, sa_r, 1), gemm.dequant(qw_r, sw_r, 128)
    ok, worst = gemm.check_close(out.float().cpu().numpy().astype(np.float64), ad @ wd.T, ad, wd)
    assert ok, f"linear forward: worst |err|/bound {worst}"
