"""Blockwise-scaled FP8 linear-layer training kernels for AMD MI355X (gfx950).

The compute path is the HIP library ``libbs.so`` (C ABI in include/bs.h);
``binding`` marshals torch tensors into it.  Importing this package does not
load the library; the first call does, and raises if it has not been built.
"""

from .binding import (  # noqa: F401
    BS_GROUP_K,
    BS_GROUP_M,
    BS_OUT_BF16,
    BS_OUT_F32,
    BS_SCALE_128X128,
    BS_SCALE_1X128,
    BsError,
    bs_diag_division,
    bs_diag_e4m3_census,
    bs_diag_stream,
    bs_grouped_scaled_mm,
    bs_mx_grouped_scaled_mm,
    bs_mx_quant_1x32,
    bs_mx_scaled_mm,
    bs_quant_128x128,
    bs_quant_128x128_both,
    bs_quant_1x128,
    bs_quant_3d_colwise,
    bs_quant_fwd_operands,
    bs_swiglu_bwd_quant_1x128,
    bs_swiglu_quant_1x128,
    bs_scaled_mm,
    bs_scaled_mm_quant,
    bs_scaled_mm_workspace_bytes,
    bs_scaled_mm_ws,
    empty_mx_scales,
    empty_scales,
    streamk_workspace,
)
from .linear import Float8BlockwiseLinear, float8_blockwise_linear, swap_linear_layers  # noqa: F401,E402
from .ffn import Float8BlockwiseGatedFFN, float8_blockwise_gated_ffn  # noqa: F401,E402
from .mx import Float8MXLinear, float8_mx_linear, mx_grouped_mm  # noqa: F401,E402
