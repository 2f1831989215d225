"""ctypes loader of the in-tree HIP library libbs.so (declarations: include/bs.h)."""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbs.so")

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_E = ctypes.c_int  # C enums

# name -> (restype, argtypes); mirrors include/bs.h
SIGNATURES = {
    "bs_quant_1x128": (_E, [_P, _I64, _I64, _I64, _P, _I64, _P, _I64, _P, _I64, _P, _I64, _P]),
    "bs_swiglu_quant_1x128": (_E, [_P, _P, _I64, _I64, _I64, _I64, _P, _I64, _P, _I64, _P, _I64, _P, _I64, _P, _I64,
                                   _P]),
    "bs_swiglu_bwd_quant_1x128": (_E, [_P, _P, _P, _I64, _I64, _I64, _I64, _I64, _P, _I64, _P, _I64, _P, _I64, _P,
                                       _I64, _P, _I64, _P]),
    "bs_mx_quant_1x32": (_E, [_P, _I64, _I64, _I64, _P, _I64, _P, _I64, _P, _I64, _P, _I64, _P]),
    "bs_mx_scaled_mm": (_E, [_I64, _I64, _I64, _P, _I64, _P, _I64, _P, _I64, _P, _I64, _P, _I64, _E, _P]),
    "bs_mx_grouped_scaled_mm": (_E, [_E, _I64, _I64, _I64, _I64, _P, _P, _I64, _P, _I64, _P, _I64, _I64, _P, _I64,
                                     _I64, _P, _I64, _I64, _E, _P]),
    "bs_quant_128x128": (_E, [_P, _I64, _I64, _I64, _P, _I64, _P, _I64, _P]),
    "bs_quant_3d_colwise": (_E, [_P, _I64, _I64, _I64, _I64, _I64, _P, _I64, _I64, _P, _I64, _I64, _P]),
    "bs_quant_128x128_both": (_E, [_P, _I64, _I64, _I64, _I64, _I64, _P, _I64, _P, _I64, _P, _I64, _I64, _P, _I64,
                                   _I64, _P]),
    "bs_quant_fwd_operands": (_E, [_P, _I64, _I64, _I64, _P, _I64, _P, _I64, _P, _I64, _P, _I64,
                                   _P, _I64, _I64, _I64, _I64, _I64, _P, _I64, _P, _I64, _P, _I64, _I64, _P, _I64,
                                   _I64, _P]),
    "bs_scaled_mm": (_E, [_I64, _I64, _I64, _P, _I64, _P, _I64, _E, _P, _I64, _P, _I64, _E, _P, _I64, _E, _P]),
    "bs_scaled_mm_quant": (_E, [_I64, _I64, _I64, _P, _I64, _P, _I64, _E, _P, _I64, _P, _I64, _E, _P, _I64,
                                _P, _I64, _P, _I64, _P, _I64, _P, _I64, _P]),
    "bs_scaled_mm_ws": (_E, [_I64, _I64, _I64, _P, _I64, _P, _I64, _E, _P, _I64, _P, _I64, _E, _P, _I64, _E, _P,
                             _I64, _P]),
    "bs_scaled_mm_workspace_bytes": (_I64, [_I64, _I64, _I64, _E, _E]),
    "bs_scaled_mm_noalloc": (_E, [_I64, _I64, _I64, _P, _I64, _P, _I64, _E, _P, _I64, _P, _I64, _E, _P, _I64, _E,
                                  _P]),
    "bs_grouped_scaled_mm": (_E, [_E, _I64, _I64, _I64, _I64, _P, _P, _I64, _P, _I64, _P, _I64, _I64, _P, _I64,
                                  _I64, _E, _P, _I64, _I64, _E, _P]),
    "bs_status_string": (ctypes.c_char_p, [_E]),
    "bs_last_error": (ctypes.c_char_p, []),
    "bs_diag_e4m3_census": (_E, [_P, _P, _P, _P]),
    "bs_diag_division": (_E, [_P, _P]),
    "bs_diag_stream": (_E, [_P, _I64, _P, _I64, _P]),
}

_lib = None


def load():
    """Load libbs.so once; raise loudly if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"HIP library not found at {LIB_PATH}; build it with "
                "`python -m blockwise_scaled_fp8_bs_amd.build` (hipcc, gfx950)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib
