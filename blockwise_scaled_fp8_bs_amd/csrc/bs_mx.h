// MXFP8 (OCP Microscaling reading of the pages' MXFP8 recipe) kernel
// arguments and launchers: 32-element blocks along the contraction with one
// E8M0 exponent byte each, E4M3 elements.
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

// GEMM D[M, N] = A[M, K] . B[N, K]^T, both operands with E8M0 scales
// [K/32][ld >= rows] (bytes).
struct MxGemmArgs {
    int64_t M, N, K;
    const uint8_t* a;
    int64_t lda;
    const uint8_t* sa;
    int64_t ld_sa;
    const uint8_t* b;
    int64_t ldb;
    const uint8_t* sb;
    int64_t ld_sb;
    void* d;
    int64_t ldd;
    int64_t tiles_m, tiles_n, num_tiles;  // set by the launcher
};

hipError_t launch_mx_quant(const MxQuantArgs& a, bool row, bool col, hipStream_t stream);
hipError_t launch_mx_gemm(const MxGemmArgs& a, bool out_f32, hipStream_t stream);

}  // namespace bs
