// Internal interface between the C ABI layer (bs_api.hip) and the kernel
// translation units.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bs {

struct Quant1x128Args {
    const uint16_t* x;
    int64_t R, C, ld_x;
    uint8_t* q_row;
    int64_t ld_qr;
    float* s_row;
    int64_t ld_sr;
    uint8_t* q_col;
    int64_t ld_qc;
    float* s_col;
    int64_t ld_sc;
    int64_t col_tiles;  // C / 128
    // gated form (bs_swiglu_quant_1x128): the quantized tensor is
    // h = bf16(silu(x) * y), optionally also written to h
    const uint16_t* y;
    int64_t ld_y;
    uint16_t* h;
    int64_t ld_h;
};

// Backward of the gated activation fused with the 1x128 quantizer: inputs
// a, b, dh are [R, C]; the quantized matrix is [da | db], [R, 2C].
struct SwigluBwdArgs {
    const uint16_t *a, *b, *dh;
    int64_t R, C, ld_a, ld_b, ld_dh;
    uint16_t* dab;  // optional [R, 2C] bf16 output of [da | db]
    int64_t ld_dab;
    uint8_t* q_row;  // [R, 2C]
    int64_t ld_qr;
    float* s_row;    // [2C/128][ld_sr >= R]
    int64_t ld_sr;
    uint8_t* q_col;  // [2C, R]
    int64_t ld_qc;
    float* s_col;    // [R/128][ld_sc >= 2C]
    int64_t ld_sc;
    int64_t col_tiles;  // C / 128
};

struct Quant128Args {
    const uint16_t* x;
    int64_t G, R, C, stride_xg, ld_x;
    uint8_t* q;
    int64_t stride_qg, ld_q;
    float* s;
    int64_t stride_sg, ld_s;
    int64_t row_tiles, col_tiles;  // R / 128, C / 128
    // second (transposed) output of the fused pass: qt[g] [C, R], st[g] [R/128][ld_st]
    uint8_t* qt;
    int64_t stride_qtg, ld_qt;
    float* st;
    int64_t stride_stg, ld_st;
};

// Which outputs a 128x128 pass writes.
enum Quant128Mode { kQ128Rows = 0, kQ128Transposed = 1, kQ128Both = 2 };

enum GroupKind { kDense = 0, kGroupM = 1, kGroupK = 2 };

// Scales of a GEMM's operands: A 1x128 with B 128x128 or B 1x128 (fp32,
// folded per 128-block), or MX on both (E8M0 per 32 elements, applied by
// the scaled MFMA).
enum ScaleMode { kScale128x128 = 0, kScale1x128 = 1, kScaleMx = 2 };

struct GemmArgs {
    int64_t M, N, K;
    const uint8_t* a;
    int64_t lda;
    const void* sa;  // fp32 1x128 scales, or E8M0 bytes [K/32][ld_sa] (kScaleMx)
    int64_t ld_sa;
    const uint8_t* b;
    int64_t ldb;
    const void* sb;  // fp32 128x128 or 1x128 scales, or E8M0 bytes [K/32][ld_sb] (kScaleMx)
    int64_t ld_sb;
    void* d;
    int64_t ldd;
    // grouped forms
    int64_t G;
    const int32_t* group_end;
    int64_t stride_bg, stride_sbg, stride_dg;
    // launch geometry
    int64_t tiles_m, tiles_n;  // tiles of the dense problem (GROUP_K: per group)
    int64_t num_tiles;         // grid size (an upper bound for GROUP_M)
    // stream-K split of a dense problem (set by launch_gemm_streamk): the
    // first sk_dp_tiles tiles are whole work items dealt round-robin over the
    // grid; the K iterations of the remaining sk_tiles tiles are divided
    // evenly over sk_wgs workgroups; sk_partial + v * 256 * 256 holds
    // workgroup v's partial tile for its owner (workspace)
    int64_t sk_dp_tiles, sk_tiles, sk_wgs;
    float* sk_partial;
    // quantized output (bs_scaled_mm_quant): the 1x128 codes and scales of
    // the bf16 D, rows and/or transposed columns, as bs_quant_1x128 writes them
    uint8_t* q_row;
    int64_t ld_qr;
    float* s_row;
    int64_t ld_sr;
    uint8_t* q_col;
    int64_t ld_qc;
    float* s_col;
    int64_t ld_sc;
};

// Stream-K decomposition of a dense GEMM for a given grid.
struct StreamK {
    int64_t grid;      // persistent workgroups
    int64_t dp_tiles;  // whole tiles (a multiple of grid)
    int64_t sk_tiles;  // tiles split over workgroups (0: no split)
    int64_t sk_wgs;    // workgroups sharing the split tiles' K iterations
};

hipError_t launch_quant_1x128(const Quant1x128Args& a, bool row, bool col, bool swiglu, hipStream_t stream);
hipError_t launch_quant_128x128(const Quant128Args& a, Quant128Mode mode, hipStream_t stream);
// launch_quant_1x128 (rows and columns) of xa and launch_quant_128x128
// (kQ128Both) of wa in one launch
hipError_t launch_quant_pair(const Quant1x128Args& xa, const Quant128Args& wa, hipStream_t stream);
hipError_t launch_swiglu_bwd_quant(const SwigluBwdArgs& a, bool row, bool col, hipStream_t stream);

hipError_t launch_gemm(const GemmArgs& a, GroupKind kind, ScaleMode scales, bool out_f32, hipStream_t stream);

// Dense GEMM whose epilogue also writes the 1x128 quantization of its bf16
// output (q_row / q_col of the arguments; d may be NULL).
hipError_t launch_gemm_quant(const GemmArgs& a, ScaleMode scales, hipStream_t stream);

// Dense GEMM with the ragged last round of tiles split along K (stream-K,
// two launches) when the workspace holds the partial tiles; otherwise as
// launch_gemm.
StreamK plan_streamk(const GemmArgs& a, ScaleMode scales, bool out_f32);
int64_t streamk_workspace_bytes(const StreamK& sk);
hipError_t launch_gemm_streamk(const GemmArgs& a, ScaleMode scales, bool out_f32, void* workspace,
                               int64_t workspace_bytes, hipStream_t stream);

// CUs of the current device and resident workgroups of `kernel` (`threads`
// per workgroup) per CU, for sizing persistent grids.  Queried once per
// (device, kernel, threads) and kept: the two runtime queries cost several
// microseconds per launch and their answers never change.  A failed query
// falls back to 256 CUs and `default_per_cu`.
struct DeviceFit {
    int cus;
    int per_cu;
};
DeviceFit device_fit(const void* kernel, int threads, int default_per_cu);

hipError_t launch_diag_e4m3_census(uint32_t* min_bits, uint32_t* max_bits, unsigned long long* counts,
                                   hipStream_t stream);
hipError_t launch_diag_division(unsigned long long* result, hipStream_t stream);
hipError_t launch_diag_stream(const void* src, int64_t n_read, void* dst, int64_t n_write, hipStream_t stream);

}  // namespace bs
