// MXFP8 (OCP Microscaling reading of the pages' MXFP8 recipe) quantizer
// arguments and launcher: 32-element blocks along the contraction with one
// E8M0 exponent byte each, E4M3 elements.  (The MX GEMMs are a scale mode
// of launch_gemm.)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bs {

// Quantizer: rows (32-element blocks along each row) and/or columns (32
// consecutive rows of each column, written transposed).
struct MxQuantArgs {
    const uint16_t* x;
    int64_t R, C, ld_x;
    uint8_t* q_row;  // [R, C]
    int64_t ld_qr;
    uint8_t* s_row;  // [C/32][ld_sr >= R]
    int64_t ld_sr;
    uint8_t* q_col;  // [C, R]
    int64_t ld_qc;
    uint8_t* s_col;  // [R/32][ld_sc >= C]
    int64_t ld_sc;
    int64_t col_tiles;  // C / 128
};

hipError_t launch_mx_quant(const MxQuantArgs& a, bool row, bool col, hipStream_t stream);

}  // namespace bs
