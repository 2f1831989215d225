"""C-ABI boundary checks that need no GPU.

The library must load, export every function declared in include/bs.h, and
reject malformed arguments on the host with the documented status code and a
message naming the layout -- before anything is enqueued.  The pointers here
are fake (never dereferenced: validation fails first).
"""

import ctypes
import os
import re

import pytest

from blockwise_scaled_fp8_bs_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bs.h")

OK, NULL, SHAPE, LAYOUT, ALIGN, MODE = 0, 1, 2, 3, 4, 5
P = 0x10000  # a fake 16-byte aligned address
PU = 0x10004  # a fake misaligned address


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:bs_status|const char\*|int64_t)\s+(bs_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libbs.so is not built (python -m blockwise_scaled_fp8_bs_amd.build)")
    return _lib.load()


def test_header_declares_the_five_entry_points():
    names = declared_functions()
    for n in ["bs_quant_1x128", "bs_quant_128x128", "bs_quant_3d_colwise", "bs_scaled_mm",
              "bs_grouped_scaled_mm", "bs_status_string", "bs_last_error"]:
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, f"binding lacks a signature for {name}"


def test_status_strings(lib):
    assert lib.bs_status_string(0) == b"BS_OK"
    assert lib.bs_status_string(3) == b"BS_ERR_LAYOUT"
    assert lib.bs_status_string(99) == b"BS_ERR_UNKNOWN"


def _q1(lib, x=P, R=256, C=512, ld_x=512, q_row=P, ld_qr=512, s_row=P, ld_sr=256, q_col=None, ld_qc=0,
        s_col=None, ld_sc=0):
    return lib.bs_quant_1x128(x, R, C, ld_x, q_row, ld_qr, s_row, ld_sr, q_col, ld_qc, s_col, ld_sc, None)


@pytest.mark.parametrize("kw,code,frag", [
    (dict(x=None), NULL, "x is NULL"),
    (dict(q_row=None), NULL, "both"),
    (dict(q_row=None, s_row=None), NULL, "no output"),
    (dict(C=500, ld_x=512, ld_qr=512), SHAPE, "multiple of 128"),
    (dict(R=-1), SHAPE, ">= 0"),
    (dict(ld_x=256), LAYOUT, "row-major"),
    (dict(ld_sr=200), LAYOUT, "K-major"),
    (dict(ld_sr=258), LAYOUT, "multiple of 4"),
    (dict(x=PU), ALIGN, "aligned"),
    (dict(ld_qr=520), ALIGN, "ld_qr"),
    (dict(R=200, q_col=P, ld_qc=256, s_col=P, ld_sc=512), SHAPE, "column output"),
    (dict(q_col=P, ld_qc=100, s_col=P, ld_sc=512), LAYOUT, "transpose"),
])
def test_quant_1x128_validation(lib, kw, code, frag):
    assert _q1(lib, **kw) == code
    assert frag in lib.bs_last_error().decode()


def test_quant_1x128_empty_is_ok_without_launch(lib):
    assert _q1(lib, R=0) == OK
    assert lib.bs_last_error() == b""


def test_quant_128x128_validation(lib):
    f = lib.bs_quant_128x128
    assert f(P, 200, 512, 512, P, 512, P, 4, None) == SHAPE
    assert f(P, 256, 512, 512, P, 512, P, 1, None) == LAYOUT
    assert "K-major" in lib.bs_last_error().decode()
    assert f(P, 256, 512, 512, P, 512, P, 6, None) == LAYOUT
    assert "multiple of 4" in lib.bs_last_error().decode()
    assert f(P, 0, 512, 512, P, 512, P, 4, None) == OK


def test_quant_3d_colwise_validation(lib):
    f = lib.bs_quant_3d_colwise
    # G=2, R=256, C=384: q[g] is [384, 256]
    assert f(P, 2, 256, 384, 256 * 384, 384, P, 384 * 256, 100, P, 8, 4, None) == LAYOUT  # ld_q < R
    assert f(P, 2, 256, 384, 100, 384, P, 384 * 256, 256, P, 8, 4, None) == LAYOUT       # stride_xg
    assert f(P, 2, 256, 384, 256 * 384, 384, P, 384 * 256, 256, P, 4, 4, None) == LAYOUT  # stride_sg
    assert f(P, 0, 256, 384, 0, 384, P, 0, 256, P, 0, 4, None) == OK


def _mm(lib, M=256, N=256, K=512, a=P, lda=512, sa=P, ld_sa=256, a_kind=4, b=P, ldb=512, sb=P, ld_sb=4,
        b_kind=5, d=P, ldd=256, dt=0):
    return lib.bs_scaled_mm(M, N, K, a, lda, sa, ld_sa, a_kind, b, ldb, sb, ld_sb, b_kind, d, ldd, dt, None)


@pytest.mark.parametrize("kw,code,frag", [
    (dict(a=None), NULL, "non-NULL"),
    (dict(d=None), NULL, "d must be"),
    (dict(a_kind=5), MODE, "a_kind"),
    (dict(b_kind=7), MODE, "b_kind"),
    (dict(dt=3), MODE, "d_dtype"),
    (dict(K=500, lda=512, ldb=512), SHAPE, "multiple of 128"),
    (dict(N=200, ldd=256), SHAPE, "N=200"),
    (dict(lda=256), LAYOUT, "row-major [M, K]"),
    (dict(ldb=256), LAYOUT, "column-major"),
    (dict(ldd=128), LAYOUT, "row-major [M, N]"),
    (dict(ld_sa=128), LAYOUT, "K-major"),
    (dict(ld_sb=2), LAYOUT, "multiple of 4"),
    (dict(b_kind=4, ld_sb=4), LAYOUT, "ld_sb >= N"),
    (dict(a=PU), ALIGN, "aligned"),
    (dict(ldd=260), ALIGN, "16-byte rows"),
])
def test_scaled_mm_validation(lib, kw, code, frag):
    assert _mm(lib, **kw) == code
    assert frag in lib.bs_last_error().decode()


def test_scaled_mm_empty_is_ok(lib):
    assert _mm(lib, M=0) == OK


def _mm_ws(lib, ws=P * 16, ws_bytes=1 << 20, **kw):
    a = dict(M=256, N=256, K=512, a=P, lda=512, sa=P, ld_sa=256, a_kind=4, b=P, ldb=512, sb=P, ld_sb=4,
             b_kind=5, d=P, ldd=256, dt=0)
    a.update(kw)
    return lib.bs_scaled_mm_ws(a["M"], a["N"], a["K"], a["a"], a["lda"], a["sa"], a["ld_sa"], a["a_kind"], a["b"],
                               a["ldb"], a["sb"], a["ld_sb"], a["b_kind"], a["d"], a["ldd"], a["dt"], ws, ws_bytes,
                               None)


@pytest.mark.parametrize("kw,code,frag", [
    (dict(ws=None), NULL, "workspace is NULL"),
    (dict(ws=P + 16), ALIGN, "256-byte aligned"),
    (dict(ws_bytes=-1), LAYOUT, "workspace_bytes"),
    (dict(lda=256), LAYOUT, "row-major [M, K]"),
    (dict(a_kind=5), MODE, "a_kind"),
])
def test_scaled_mm_ws_validation(lib, kw, code, frag):
    assert _mm_ws(lib, **kw) == code
    assert frag in lib.bs_last_error().decode()


def test_scaled_mm_ws_empty_is_ok(lib):
    assert _mm_ws(lib, M=0) == OK
    assert _mm_ws(lib, M=0, ws=None, ws_bytes=0) == OK


def test_workspace_query_is_zero_for_invalid_problems(lib):
    f = lib.bs_scaled_mm_workspace_bytes
    assert f(0, 256, 512, 4, 0) == 0
    assert f(256, 200, 512, 4, 0) == 0     # N not a multiple of 128
    assert f(256, 256, 500, 4, 0) == 0     # K not a multiple of 128
    assert f(256, 256, 512, 7, 0) == 0     # unknown scale kind
    assert f(256, 256, 512, 4, 0) >= 0


def test_grouped_validation(lib):
    f = lib.bs_grouped_scaled_mm
    base = dict(mode=0, G=2, M=256, N=256, K=512, ge=P, a=P, lda=512, sa=P, ld_sa=256, b=P, sbg=256 * 512,
                ldb=512, sb=P, ssbg=2, ld_sb=4, b_kind=5, d=P, sdg=0, ldd=256, dt=0)

    def call(**kw):
        a = dict(base, **kw)
        return f(a["mode"], a["G"], a["M"], a["N"], a["K"], a["ge"], a["a"], a["lda"], a["sa"], a["ld_sa"],
                 a["b"], a["sbg"], a["ldb"], a["sb"], a["ssbg"], a["ld_sb"], a["b_kind"], a["d"], a["sdg"],
                 a["ldd"], a["dt"], None)

    assert call(mode=2) == MODE
    assert call(ge=None) == NULL
    assert call(b_kind=4) == MODE
    assert call(sdg=5) == MODE
    assert call(G=0) == OK
    # GROUP_K
    assert call(mode=1, b_kind=5) == MODE
    assert call(mode=1, b_kind=4, ld_sb=256, sbg=0, ssbg=0, sdg=10) == LAYOUT
    assert call(mode=1, b_kind=4, ld_sb=256, sbg=0, ssbg=0, sdg=256 * 256, G=0) == OK
    assert call(mode=1, b_kind=4, ld_sb=256, sbg=7, ssbg=0, sdg=256 * 256) == MODE


def _q128b(lib, x=P, G=2, R=256, C=384, stride_xg=256 * 384, ld_x=384, q=P, ld_q=384, s=P, ld_s=4,
           qt=P, stride_qtg=384 * 256, ld_qt=256, st=P, stride_stg=2 * 4, ld_st=4):
    return lib.bs_quant_128x128_both(x, G, R, C, stride_xg, ld_x, q, ld_q, s, ld_s, qt, stride_qtg, ld_qt, st,
                                     stride_stg, ld_st, None)


@pytest.mark.parametrize("kw,code,frag", [
    (dict(qt=None), NULL, "non-NULL"),
    (dict(R=200), SHAPE, "multiples of 128"),
    (dict(ld_q=256), LAYOUT, "ld_q"),
    (dict(ld_s=2), LAYOUT, "ld_s"),        # G*R/128 = 4 scale columns needed
    (dict(ld_s=6), LAYOUT, "multiple of 4"),
    (dict(ld_qt=128), LAYOUT, "ld_qt"),
    (dict(stride_qtg=1000), LAYOUT, "stride_qtg"),
    (dict(stride_stg=4), LAYOUT, "stride_stg"),
    (dict(stride_xg=100), LAYOUT, "stride_xg"),
    (dict(q=PU), ALIGN, "q must be 16-byte aligned"),
])
def test_quant_128x128_both_validation(lib, kw, code, frag):
    assert _q128b(lib, **kw) == code
    assert frag in lib.bs_last_error().decode()


def test_quant_128x128_both_empty_is_ok(lib):
    assert _q128b(lib, G=0, x=None, q=None, s=None, qt=None, st=None) == OK


def _qfwd(lib, x=P, R=256, C=384, ld_x=384, q_row=P, ld_qr=384, s_row=P, ld_sr=256, q_col=P, ld_qc=256,
          s_col=P, ld_sc=384, w=P, G=2, N=256, K=384, stride_wg=256 * 384, ld_w=384, qw=P, ld_qw=384, sw=P,
          ld_sw=4, qwt=P, stride_qwtg=384 * 256, ld_qwt=256, swt=P, stride_swtg=2 * 4, ld_swt=4):
    return lib.bs_quant_fwd_operands(x, R, C, ld_x, q_row, ld_qr, s_row, ld_sr, q_col, ld_qc, s_col, ld_sc,
                                     w, G, N, K, stride_wg, ld_w, qw, ld_qw, sw, ld_sw, qwt, stride_qwtg, ld_qwt,
                                     swt, stride_swtg, ld_swt, None)


@pytest.mark.parametrize("kw,code,frag", [
    (dict(q_col=None), NULL, "all be set"),
    (dict(s_row=None), NULL, "all be set"),
    (dict(x=None), NULL, "x is NULL"),
    (dict(C=500, ld_x=512, ld_qr=512), SHAPE, "multiple of 128"),
    (dict(ld_sr=258), LAYOUT, "multiple of 4"),
    (dict(x=PU), ALIGN, "aligned"),
    (dict(qwt=None), NULL, "non-NULL"),
    (dict(N=200), SHAPE, "multiples of 128"),
    (dict(ld_sw=2), LAYOUT, "ld_s"),
    (dict(stride_swtg=4), LAYOUT, "stride_stg"),
    (dict(qw=PU), ALIGN, "q must be 16-byte aligned"),
])
def test_quant_fwd_operands_validation(lib, kw, code, frag):
    """Each operand's checks are those of its own call, under this call's name."""
    assert _qfwd(lib, **kw) == code
    msg = lib.bs_last_error().decode()
    assert frag in msg and "bs_quant_fwd_operands" in msg


def test_quant_fwd_operands_empty_is_ok(lib):
    assert _qfwd(lib, R=0, G=0, x=None, q_row=None, s_row=None, q_col=None, s_col=None, w=None, qw=None,
                 sw=None, qwt=None, swt=None) == OK
    assert lib.bs_last_error() == b""


def test_leading_dimensions_are_bounded(lib):
    big = 1 << 22
    assert _q1(lib, ld_x=big) == LAYOUT and b"ld_x" in lib.bs_last_error()
    assert _q1(lib, ld_qr=big) == LAYOUT and b"ld_qr" in lib.bs_last_error()
    assert lib.bs_quant_128x128(P, 256, 512, 512, P, big, P, 4, None) == LAYOUT
    assert _q128b(lib, ld_x=big, stride_xg=256 * big) == LAYOUT
    assert _q128b(lib, ld_qt=big, stride_qtg=384 * big) == LAYOUT


def _sw(lib, a=P, b=P, R=256, C=512, ld_a=512, ld_b=512, h=None, ld_h=0, q_row=P, ld_qr=512, s_row=P, ld_sr=256,
        q_col=None, ld_qc=0, s_col=None, ld_sc=0):
    return lib.bs_swiglu_quant_1x128(a, b, R, C, ld_a, ld_b, h, ld_h, q_row, ld_qr, s_row, ld_sr, q_col, ld_qc,
                                     s_col, ld_sc, None)


@pytest.mark.parametrize("kw,code,frag", [
    (dict(b=None), NULL, "b is NULL"),
    (dict(a=None), NULL, "a is NULL"),
    (dict(ld_b=256), LAYOUT, "ld_b"),
    (dict(b=PU), ALIGN, "b must be 16-byte aligned"),
    (dict(h=P, ld_h=256), LAYOUT, "ld_h"),
    (dict(h=PU, ld_h=512), ALIGN, "h must be 16-byte aligned"),
    (dict(C=200, ld_a=200, ld_b=200), SHAPE, "multiple of 128"),
    (dict(q_row=None, s_row=None), NULL, "no output requested"),
])
def test_swiglu_quant_validation(lib, kw, code, frag):
    assert _sw(lib, **kw) == code
    assert frag in lib.bs_last_error().decode()


def _swb(lib, a=P, b=P, dh=P, R=256, C=512, ld_a=512, ld_b=512, ld_dh=512, dab=None, ld_dab=0, q_row=P,
         ld_qr=1024, s_row=P, ld_sr=256, q_col=P, ld_qc=256, s_col=P, ld_sc=1024):
    return lib.bs_swiglu_bwd_quant_1x128(a, b, dh, R, C, ld_a, ld_b, ld_dh, dab, ld_dab, q_row, ld_qr, s_row, ld_sr,
                                         q_col, ld_qc, s_col, ld_sc, None)


@pytest.mark.parametrize("kw,code,frag", [
    (dict(dh=None), NULL, "a, b and dh"),
    (dict(ld_dh=256), LAYOUT, "ld of dh"),
    (dict(b=PU), ALIGN, "b must be 16-byte aligned"),
    (dict(dab=P, ld_dab=512), LAYOUT, "ld_dab"),
    (dict(ld_qr=512), LAYOUT, "ld_qr"),
    (dict(ld_sc=512), LAYOUT, "ld_sc"),
    (dict(ld_sr=255), LAYOUT, "ld_sr"),
    (dict(R=200), SHAPE, "multiple of 128 for the column output"),
    (dict(C=200, ld_a=200, ld_b=200, ld_dh=200), SHAPE, "multiple of 128"),
    (dict(q_row=None, s_row=None, q_col=None, s_col=None), NULL, "no output requested"),
    (dict(s_col=None), NULL, "q_col and s_col"),
])
def test_swiglu_bwd_quant_validation(lib, kw, code, frag):
    assert _swb(lib, **kw) == code
    assert frag in lib.bs_last_error().decode()


def test_swiglu_bwd_quant_empty_is_ok(lib):
    assert _swb(lib, R=0, a=None, b=None, dh=None) == OK


def _mxq(lib, x=P, R=256, C=512, ld_x=512, q_row=P, ld_qr=512, s_row=P, ld_sr=256, q_col=P, ld_qc=256, s_col=P,
         ld_sc=512):
    return lib.bs_mx_quant_1x32(x, R, C, ld_x, q_row, ld_qr, s_row, ld_sr, q_col, ld_qc, s_col, ld_sc, None)


@pytest.mark.parametrize("kw,code,frag", [
    (dict(x=None), NULL, "x is NULL"),
    (dict(s_row=None), NULL, "q_row and s_row"),
    (dict(q_col=None), NULL, "q_col and s_col"),
    (dict(q_row=None, s_row=None, q_col=None, s_col=None), NULL, "no output requested"),
    (dict(C=96, ld_x=96, ld_qr=96, ld_sc=96), SHAPE, "multiple of 128"),
    (dict(R=200, ld_sr=208), SHAPE, "multiple of 128 for the column output"),
    (dict(ld_x=256), LAYOUT, "ld_x"),
    (dict(ld_qr=384), LAYOUT, "ld_qr"),
    (dict(ld_sr=248), LAYOUT, "ld_sr"),
    (dict(ld_sr=264 + 4), LAYOUT, "multiple of 16"),
    (dict(ld_qc=128), LAYOUT, "ld_qc"),
    (dict(ld_sc=500), LAYOUT, "ld_sc"),
    (dict(x=PU), ALIGN, "x must be 16-byte aligned"),
    (dict(s_col=PU), ALIGN, "q_col and s_col must be 16-byte aligned"),
])
def test_mx_quant_validation(lib, kw, code, frag):
    assert _mxq(lib, **kw) == code
    assert frag in lib.bs_last_error().decode()


def test_mx_quant_rows_only_skip_the_row_multiple_check(lib):
    # with only the row output, R=200 passes the shape check and is stopped
    # by the scale layout (ld_sr not a multiple of 16) before any launch
    assert _mxq(lib, R=0, x=None, q_col=None, s_col=None) == OK
    assert _mxq(lib, R=200, ld_sr=200, q_col=None, s_col=None) == LAYOUT   # 200 is not a multiple of 16


def _mxmm(lib, M=256, N=512, K=384, a=P, lda=384, sa=P, ld_sa=256, b=P, ldb=384, sb=P, ld_sb=512, d=P, ldd=512,
          dt=0):
    return lib.bs_mx_scaled_mm(M, N, K, a, lda, sa, ld_sa, b, ldb, sb, ld_sb, d, ldd, dt, None)


@pytest.mark.parametrize("kw,code,frag", [
    (dict(a=None), NULL, "a and sa"),
    (dict(sb=None), NULL, "b and sb"),
    (dict(d=None), NULL, "d must be non-NULL"),
    (dict(dt=7), MODE, "d_dtype"),
    (dict(N=200, ldd=200, ld_sb=208), SHAPE, "N=200"),
    (dict(K=96, lda=96, ldb=96), SHAPE, "K=96"),
    (dict(lda=256), LAYOUT, "lda"),
    (dict(ldd=256), LAYOUT, "ldd"),
    (dict(ld_sa=128), LAYOUT, "ld_sa"),
    (dict(ld_sb=520), LAYOUT, "ld_sb"),
    (dict(a=PU), ALIGN, "a and b must be 16-byte aligned"),
    (dict(sa=PU), ALIGN, "sa and sb"),
    (dict(d=PU), ALIGN, "d must be 16-byte aligned"),
])
def test_mx_scaled_mm_validation(lib, kw, code, frag):
    assert _mxmm(lib, **kw) == code
    assert frag in lib.bs_last_error().decode()


def test_mx_scaled_mm_empty_is_ok(lib):
    assert _mxmm(lib, M=0, a=None, sa=None) == OK
    assert _mxmm(lib, N=0, ldd=0, b=None, sb=None, d=None) == OK


def _mxg(lib, mode=0, G=2, M=256, N=512, K=384, ge=P, a=P, lda=384, sa=P, ld_sa=256, b=P, stride_bg=512 * 384,
         ldb=384, sb=P, stride_sbg=12 * 512, ld_sb=512, d=P, stride_dg=0, ldd=512, dt=0):
    return lib.bs_mx_grouped_scaled_mm(mode, G, M, N, K, ge, a, lda, sa, ld_sa, b, stride_bg, ldb, sb, stride_sbg,
                                       ld_sb, d, stride_dg, ldd, dt, None)


@pytest.mark.parametrize("kw,code,frag", [
    (dict(mode=7), MODE, "mode=7"),
    (dict(ge=None), NULL, "group_end is NULL"),
    (dict(G=-1), SHAPE, "G=-1"),
    (dict(ld_sa=200), LAYOUT, "ld_sa"),
    (dict(stride_dg=4096), MODE, "stride_dg must be 0"),
    (dict(stride_sbg=-16), LAYOUT, "stride_bg and stride_sbg must be >= 0"),
    (dict(stride_sbg=520), ALIGN, "multiples of 16"),
    (dict(mode=1, stride_bg=0, stride_sbg=0, M=200, ld_sa=208, stride_dg=200 * 512), SHAPE, "M=200"),
    (dict(mode=1, stride_sbg=0, stride_dg=256 * 512), MODE, "shares one B"),
    (dict(mode=1, stride_bg=0, stride_sbg=0, stride_dg=1024), LAYOUT, "stride_dg"),
])
def test_mx_grouped_validation(lib, kw, code, frag):
    assert _mxg(lib, **kw) == code
    assert frag in lib.bs_last_error().decode()


def test_mx_grouped_empty_is_ok(lib):
    assert _mxg(lib, G=0) == OK
    assert _mxg(lib, mode=1, G=0, stride_bg=0, stride_sbg=0) == OK
