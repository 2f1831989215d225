/*
 * bs.h -- C ABI of the blockwise-scaled FP8 training kernels for AMD gfx950.
 *
 * The method (pages: "[not for land] float8 blockwise scaling training
 * prototype using deep_gemm", description; "[mxfp8 moe training] use new 3d
 * colwise quantization kernel", summary; "add FSDP and TP tests for
 * Float8BlockwiseLinear", summary and review threads):
 *
 *   - activations and gradients are quantized to e4m3 with one fp32 scale
 *     per 1x128 block along the GEMM contraction dimension;
 *   - weights are quantized with one fp32 scale per 128x128 block;
 *   - a scaled GEMM multiplies the e4m3 codes on the matrix cores and applies
 *     the two block scales of every 128-wide contraction block to the fp32
 *     partial sum before adding it to an fp32 accumulator;
 *   - forward out = A.W^T, dgrad grad_in = grad_out.W, wgrad
 *     grad_W = grad_out^T.A (both operands 1x128 along the token axis), and a
 *     grouped (MoE) form of each, with the expert weights quantized
 *     column-wise in 3-D for the backward.
 *
 * Quantization of one block x (bf16 values):
 *     amax = max|x|;  s = fl32(max(amax, EPS) / 448);  EPS = fl32(1e-12)
 *     q    = e4m3_rne(clamp(fl32(x / s), -448, 448))      (sign of zero kept)
 * e4m3 is the OCP FP8 E4M3 encoding (bias 7, max 448, NaN 0x7F/0xFF, no Inf).
 * Inputs must be finite; the result for Inf/NaN inputs is unspecified.
 *
 * Conventions for every entry point
 *   - Dimensions and leading dimensions ("ld") are in ELEMENTS, int64_t.
 *     Leading dimensions of data matrices (bf16 inputs, e4m3 codes, GEMM
 *     operands) must be < 2^22: the kernels address within a tile with
 *     32-bit offsets.  Larger values are rejected with BS_ERR_LAYOUT.
 *   - bf16 tensors are passed as uint16_t bit patterns, e4m3 codes as uint8_t,
 *     scales as float.  All data pointers are DEVICE pointers.  A pointer may
 *     be NULL only when the tensor it points to has no elements.
 *   - Matrices are row-major with unit stride along the last dimension:
 *     element (i, j) of X is X[i * ld + j].  Both GEMM operands are
 *     contiguous along the contraction dimension (A stored by rows, B by
 *     columns: "add FSDP and TP tests for Float8BlockwiseLinear", review
 *     thread on the layout assertions).
 *   - Scales are K-major (same page, review thread on
 *     _pad_blockwise_128x128_scale_k_major): the contraction-block index is
 *     the outer index and the row (1x128) or row-block (128x128) index is
 *     contiguous, s[kb * ld_s + row] or s[kb * ld_s + row / 128], and ld_s is
 *     a multiple of 4 (16 bytes).  One layout serves every scale tensor.
 *     Scale padding entries (index >= the logical count) are never written.
 *   - Ownership: the caller owns every buffer.  The library allocates nothing
 *     and is thread-safe; between calls it keeps only a host-side cache of
 *     device properties (CU count, resident workgroups per kernel) and the
 *     static device array of bs_scaled_mm_noalloc.  Outputs must not alias
 *     inputs or each other.
 *   - Execution: every call validates its arguments on the host, then
 *     enqueues its kernels on `stream` (NULL = the default stream) and returns
 *     without synchronizing.  Nothing is enqueued when validation fails.
 *   - Errors: a nonzero bs_status; bs_last_error() returns a message for the
 *     calling thread that names the argument and the required layout.  A
 *     kernel launch failure returns BS_ERR_HIP.
 *   - Alignment: data pointers must be 16-byte aligned and leading dimensions
 *     must make every row start 16-byte aligned (bf16: ld % 8 == 0, e4m3:
 *     ld % 16 == 0, fp32: ld % 4 == 0).
 */
#ifndef BS_H
#define BS_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum bs_status {
    BS_OK = 0,
    BS_ERR_NULL = 1,    /* a required pointer is NULL                        */
    BS_ERR_SHAPE = 2,   /* a blocked dimension is not a multiple of 128, or <0 */
    BS_ERR_LAYOUT = 3,  /* a leading dimension / group stride is too small,
                           or a scale ld is not a multiple of 4              */
    BS_ERR_ALIGN = 4,   /* a pointer or row is not 16-byte aligned           */
    BS_ERR_MODE = 5,    /* unsupported scale kind, dtype or group mode       */
    BS_ERR_HIP = 6      /* the HIP runtime rejected a launch                 */
} bs_status;

/* Scale recipes.  The numbers are those of the recipe enum the pages use
 * ("add FSDP and TP tests for Float8BlockwiseLinear", review thread on
 * _SCALING_TYPE: BlockWise1x128 is 4, and 5 is the 128x128 recipe). */
typedef enum bs_scale_kind {
    BS_SCALE_1X128 = 4,
    BS_SCALE_128X128 = 5
} bs_scale_kind;

typedef enum bs_dtype {
    BS_OUT_BF16 = 0,    /* output rounded to bf16, nearest-even              */
    BS_OUT_F32 = 1
} bs_dtype;

typedef enum bs_group_mode {
    BS_GROUP_M = 0,     /* groups of rows of A, one B per group (MoE fwd/dgrad) */
    BS_GROUP_K = 1      /* groups along the contraction, one D per group (wgrad) */
} bs_group_mode;

/*
 * bs_quant_1x128 -- 1x128 quantizer of activations / gradients, one HBM pass
 * producing either or both of
 *   row output: blocks of 128 consecutive elements of a row of X
 *               q_row[r * ld_qr + c],  s_row[(c / 128) * ld_sr + r]
 *   col output: blocks of 128 consecutive rows of a column of X, written
 *               transposed so that the token axis is contiguous:
 *               q_col[c * ld_qc + r] (code of X[r][c]),
 *               s_col[(r / 128) * ld_sc + c]
 * The row output is the A operand of the forward (activations) and dgrad
 * (grad_out) GEMMs; the col output is an operand of the wgrad GEMM.
 * Pages: "[not for land] float8 blockwise scaling training prototype using
 * deep_gemm", description (1x128 activation scaling; the grad_weight GEMM).
 *
 *   x      [R, C] bf16, ld_x >= C.  C % 128 == 0.  R >= 0; R % 128 == 0 when
 *          the col output is requested (a ragged R is allowed for rows only).
 *   q_row, s_row   both NULL or both set.  ld_qr >= C, ld_sr >= R.
 *   q_col, s_col   both NULL or both set.  ld_qc >= R, ld_sc >= C.
 *   At least one output pair must be set.
 */
bs_status bs_quant_1x128(const uint16_t* x, int64_t R, int64_t C, int64_t ld_x,
                         uint8_t* q_row, int64_t ld_qr, float* s_row, int64_t ld_sr,
                         uint8_t* q_col, int64_t ld_qc, float* s_col, int64_t ld_sc,
                         hipStream_t stream);

/*
 * bs_swiglu_quant_1x128 -- the gated FFN activation fused with the 1x128
 * quantizer of its output: h = silu(a) * b (silu(a) = a / (1 + exp(-a)); the
 * value of this formula in float64, rounded once to bf16, nearest even) is
 * quantized exactly as bs_quant_1x128 would quantize the bf16 tensor h, from
 * one read of a and b.  h itself is written only when the h pointer is set.
 *   a, b   [R, C] bf16 (a = w1 x, b = w2 x of the FFN), ld_a, ld_b >= C
 *   h      optional [R, C] bf16, ld_h >= C
 *   q_row/s_row, q_col/s_col  as in bs_quant_1x128 (blocks of h).
 * The kernel evaluates in fp32 and switches to float64 for the rare values
 * whose fp32 result lies within its error bound of a bf16 rounding tie.
 * Finite a, b can give |silu(a) * b| above the bf16 maximum: h is then +-inf
 * (the rounding overflows, and h is written so when requested), which is
 * outside the quantizer's finite domain -- the codes and the scale of every
 * 1x128 block (row and column) holding such an h are unspecified; all other
 * blocks are exact.
 * Pages: "add FSDP and TP tests for Float8BlockwiseLinear", summary (the
 * ToyModel FFN: w1 and w2 feed out_proj); the prototype page, description
 * (quantization as separate kernels is the overhead to remove).
 */
bs_status bs_swiglu_quant_1x128(const uint16_t* a, const uint16_t* b, int64_t R, int64_t C,
                                int64_t ld_a, int64_t ld_b, uint16_t* h, int64_t ld_h,
                                uint8_t* q_row, int64_t ld_qr, float* s_row, int64_t ld_sr,
                                uint8_t* q_col, int64_t ld_qc, float* s_col, int64_t ld_sc,
                                hipStream_t stream);

/*
 * bs_swiglu_bwd_quant_1x128 -- the backward of the same activation fused with
 * the 1x128 quantizer of its result: from one read of a, b and the upstream
 * gradient dh it forms
 *   da = dh * b * silu'(a),  silu'(a) = s (1 + a (1 - s)),  s = 1 / (1 + exp(-a))
 *   db = dh * silu(a)
 * (each the float64 value of its formula, 1 - s evaluated as
 * 1 / (1 + exp(a)), rounded once to bf16) and quantizes the [R, 2C] matrix
 * [da | db] -- da in columns [0, C), db in [C, 2C) -- exactly as
 * bs_quant_1x128 would: its rows feed the dgrad GEMM of the stacked
 * [w1; w2] weight, its transposed columns that weight's wgrad GEMM.
 *   a, b, dh  [R, C] bf16, ld_a, ld_b, ld_dh >= C
 *   dab       optional [R, 2C] bf16 output of [da | db], ld_dab >= 2C
 *   q_row, s_row   both NULL or both set: [R, 2C] codes, ld_qr >= 2C;
 *                  s_row[(c / 128) * ld_sr + r], ld_sr >= R
 *   q_col, s_col   both NULL or both set: [2C, R] codes, ld_qc >= R;
 *                  s_col[(r / 128) * ld_sc + c], ld_sc >= 2C
 *   C % 128 == 0; R % 128 == 0 when the col output is requested.
 * As in the forward, a da or db that overflows bf16 is +-inf, and the codes
 * and scale of every block holding one are unspecified.
 * Errors as bs_quant_1x128.
 * Pages: "add FSDP and TP tests for Float8BlockwiseLinear", summary (the
 * ToyModel FFN and its backward); the prototype page, description.
 */
bs_status bs_swiglu_bwd_quant_1x128(const uint16_t* a, const uint16_t* b, const uint16_t* dh, int64_t R,
                                    int64_t C, int64_t ld_a, int64_t ld_b, int64_t ld_dh, uint16_t* dab,
                                    int64_t ld_dab, uint8_t* q_row, int64_t ld_qr, float* s_row, int64_t ld_sr,
                                    uint8_t* q_col, int64_t ld_qc, float* s_col, int64_t ld_sc,
                                    hipStream_t stream);

/*
 * MXFP8 variant (the pages' MXFP8 recipe -- "[mxfp8 moe training] use new 3d
 * colwise quantization kernel", summary and microbenchmark table -- which the
 * pages name but do not define; the definition used is the OCP Microscaling
 * v1.0 one): blocks of 32 consecutive values along the contraction, one E8M0
 * scale byte per block, 2^(byte - 127) with byte = floor(log2(amax)) - 8 + 127
 * clamped to [0, 254] (a zero block gets byte 0), elements
 * e4m3(clamp(x / 2^(byte - 127), -448, 448)).  Scale tensors are bytes,
 * K-major like the 1x128 ones: s[(k / 32) * ld_s + row], ld_s % 16 == 0
 * and 16-byte aligned.  The GEMMs read scale bytes in aligned 16-byte
 * blocks: in each scale row they may read (and never use) the bytes between
 * the last row (M or N) and the next multiple of 16, which a tensor of
 * ld_s >= roundup16(rows) holds.
 *
 * bs_mx_quant_1x32 -- one HBM pass producing either or both of
 *   row output: q_row[r * ld_qr + c], s_row[(c / 32) * ld_sr + r]
 *   col output: 32 consecutive rows of a column, transposed:
 *               q_col[c * ld_qc + r], s_col[(r / 32) * ld_sc + c]
 *   x [R, C] bf16, ld_x >= C; C % 128 == 0; R % 128 == 0 when the col
 *   output is requested.  ld_qr >= C, ld_sr >= R; ld_qc >= R, ld_sc >= C;
 *   ld_sr, ld_sc multiples of 16; at least one output pair set.
 */
bs_status bs_mx_quant_1x32(const uint16_t* x, int64_t R, int64_t C, int64_t ld_x,
                           uint8_t* q_row, int64_t ld_qr, uint8_t* s_row, int64_t ld_sr,
                           uint8_t* q_col, int64_t ld_qc, uint8_t* s_col, int64_t ld_sc,
                           hipStream_t stream);

/*
 * bs_mx_scaled_mm -- D[M, N] = A[M, K] . B[N, K]^T with MX scales on both
 * operands: D = sum_k 2^(sa(m, k/32) - 127) dec(a[m, k]) 2^(sb(n, k/32) - 127)
 * dec(b[n, k]), fp32 accumulation (gfx950's block-scaled MFMA applies the
 * scales), bf16 or fp32 output.
 *   a [M, K] row-major, lda >= K; sa [K/32][ld_sa >= M] bytes
 *   b [N, K] (contiguous along K), ldb >= K; sb [K/32][ld_sb >= N] bytes
 *   K % 128 == 0, N % 128 == 0; ld_sa, ld_sb multiples of 16; 16-byte
 *   aligned operands with lda, ldb multiples of 16.  Errors as bs_scaled_mm.
 */
bs_status bs_mx_scaled_mm(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, const uint8_t* sa,
                          int64_t ld_sa, const uint8_t* b, int64_t ldb, const uint8_t* sb, int64_t ld_sb, void* d,
                          int64_t ldd, bs_dtype d_dtype, hipStream_t stream);

/*
 * bs_mx_grouped_scaled_mm -- the MoE form of bs_mx_scaled_mm, with the group
 * semantics of bs_grouped_scaled_mm (pages: "[mxfp8 moe training] use new 3d
 * colwise quantization kernel", microbenchmark table -- MXFP8 grouped GEMMs
 * over (M, N, K, G)).  group_end as there: DEVICE int32[G], cumulative,
 * clamped on the device, never read on the host.
 *   BS_GROUP_M (forward, dgrad): rows [end_{g-1}, end_g) of A use expert g,
 *     whose B is b + g*stride_bg ([N, K], ldb) with scale bytes
 *     sb + g*stride_sbg ([K/32][ld_sb >= N]); stride_bg and stride_sbg
 *     multiples of 16; stride_dg must be 0; any group sizes.
 *   BS_GROUP_K (wgrad): contraction groups, ends multiples of 128; stride_bg
 *     and stride_sbg must be 0; D_g = d + g*stride_dg; M % 128 == 0; an
 *     empty group writes zeros.
 * Other arguments and errors as bs_mx_scaled_mm.
 */
bs_status bs_mx_grouped_scaled_mm(bs_group_mode mode, int64_t G, int64_t M, int64_t N, int64_t K,
                                  const int32_t* group_end,
                                  const uint8_t* a, int64_t lda, const uint8_t* sa, int64_t ld_sa,
                                  const uint8_t* b, int64_t stride_bg, int64_t ldb,
                                  const uint8_t* sb, int64_t stride_sbg, int64_t ld_sb,
                                  void* d, int64_t stride_dg, int64_t ldd, bs_dtype d_dtype,
                                  hipStream_t stream);

/*
 * bs_quant_128x128 -- weight quantizer, one scale per 128x128 tile.
 *   x [R, C] bf16 (R = out features, C = in features = contraction),
 *   q[r * ld_q + c], s[(c / 128) * ld_s + r / 128].
 *   R % 128 == 0, C % 128 == 0, ld_x >= C, ld_q >= C, ld_s >= R / 128.
 * Pages: prototype page, description (written with torch ops, 128x128
 * scaling of one tensor takes three kernels, and a hand-written single
 * kernel is the proposed fix); "add FSDP and TP tests ...", review thread on
 * the K-major scale padding.
 */
bs_status bs_quant_128x128(const uint16_t* x, int64_t R, int64_t C, int64_t ld_x,
                           uint8_t* q, int64_t ld_q, float* s, int64_t ld_s,
                           hipStream_t stream);

/*
 * bs_quant_3d_colwise -- expert weights W[G][R][C] quantized in 128x128
 * tiles and written transposed, giving the contraction-contiguous operand of
 * the dgrad GEMM (grad_in = grad_out . W) for every expert:
 *   q[g * stride_qg + c * ld_q + r]   = code of W[g][r][c]
 *   s[g * stride_sg + (r / 128) * ld_s + c / 128] = scale of tile (r/128, c/128)
 * (the scale index is K-major for the transposed operand, whose contraction
 * is r).  G >= 0, R % 128 == 0, C % 128 == 0; ld_x >= C, stride_xg >= R*ld_x;
 * ld_q >= R, stride_qg >= C*ld_q; ld_s >= C/128, stride_sg >= (R/128)*ld_s,
 * stride_sg % 4 == 0.  G = 1 is the dense linear's transposed weight.
 * Pages: "[mxfp8 moe training] use new 3d colwise quantization kernel",
 * summary (a kernel that quantizes a 3-D expert-weight tensor column-wise for
 * the scaled grouped GEMM backward).  The pages give that kernel for another
 * block format; the 128x128 tile here is this library's reading for the
 * 128x128 weight recipe.
 */
bs_status bs_quant_3d_colwise(const uint16_t* x, int64_t G, int64_t R, int64_t C,
                              int64_t stride_xg, int64_t ld_x,
                              uint8_t* q, int64_t stride_qg, int64_t ld_q,
                              float* s, int64_t stride_sg, int64_t ld_s,
                              hipStream_t stream);

/*
 * bs_quant_128x128_both -- bs_quant_128x128 and bs_quant_3d_colwise of the
 * same weights in one pass (one read of x; the two outputs hold the same
 * codes and scales, in the forward and the dgrad layouts).  For expert g of
 * x[G][R][C] (x[g] at x + g * stride_xg):
 *   rows, as one stacked [G*R, C] matrix (what the forward / GROUP_M GEMM
 *   reads):  q[(g*R + r) * ld_q + c],  s[(c/128) * ld_s + g*R/128 + r/128]
 *   transposed, per expert (what the dgrad GEMM reads):
 *            qt[g * stride_qtg + c * ld_qt + r],
 *            st[g * stride_stg + (r/128) * ld_st + c/128]
 * G >= 0, R % 128 == 0, C % 128 == 0; ld_x >= C, stride_xg >= R*ld_x;
 * ld_q >= C, ld_s >= G*R/128; ld_qt >= R, stride_qtg >= C*ld_qt;
 * ld_st >= C/128, stride_stg >= (R/128)*ld_st; ld_s, ld_st multiples of 4.
 * Pages: as for the two calls it fuses; the prototype page, description,
 * proposes a single hand-written kernel for 128x128 scaling.
 */
bs_status bs_quant_128x128_both(const uint16_t* x, int64_t G, int64_t R, int64_t C,
                                int64_t stride_xg, int64_t ld_x,
                                uint8_t* q, int64_t ld_q, float* s, int64_t ld_s,
                                uint8_t* qt, int64_t stride_qtg, int64_t ld_qt,
                                float* st, int64_t stride_stg, int64_t ld_st,
                                hipStream_t stream);

/*
 * bs_quant_fwd_operands -- the forward operands of a linear layer (or of the
 * experts of a grouped one) quantized in one launch: bs_quant_1x128 of the
 * activation x [R, C] along rows and transposed columns, and
 * bs_quant_128x128_both of the weights w [G][N][K] (x's arguments first,
 * then w's, each with exactly the meaning, layout and constraints of those
 * two calls; all four outputs of x are required).  The results equal those
 * of the two calls, byte for byte; one launch instead of two lets the two
 * passes share a ramp-up and a tail (the dense passes last tens of
 * microseconds).  Either operand may be empty.  Errors as the two calls.
 * Pages: the prototype page, description: quantizing with separate kernels
 * costs extra passes and launches; path forward: fast hand-written
 * quantization.
 */
bs_status bs_quant_fwd_operands(const uint16_t* x, int64_t R, int64_t C, int64_t ld_x,
                                uint8_t* q_row, int64_t ld_qr, float* s_row, int64_t ld_sr,
                                uint8_t* q_col, int64_t ld_qc, float* s_col, int64_t ld_sc,
                                const uint16_t* w, int64_t G, int64_t N, int64_t K,
                                int64_t stride_wg, int64_t ld_w,
                                uint8_t* qw, int64_t ld_qw, float* sw, int64_t ld_sw,
                                uint8_t* qwt, int64_t stride_qwtg, int64_t ld_qwt,
                                float* swt, int64_t stride_swtg, int64_t ld_swt,
                                hipStream_t stream);

/*
 * bs_scaled_mm -- D[M, N] = sum_kb sa(m, kb) * sb(n, kb) * P_kb[m, n],
 * P_kb = sum over k in block kb of dec(a[m][k]) * dec(b[n][k]) (fp32 MFMA),
 * accumulated in fp32 and written as bf16 (nearest-even) or fp32.
 * Pages: "add FSDP and TP tests for Float8BlockwiseLinear", summary and review
 * threads (blockwise_scaled_mm(a, scale_a, scale_recipe_a, b, scale_b,
 * scale_recipe_b); one scale layout; fail loudly on wrong layouts);
 * prototype page, description (fwd and bwd GEMMs of a dense linear; the
 * 1x128 x 1x128 grad_weight GEMM).
 *
 *   a  [M, K] e4m3, lda >= K;  sa 1x128: sa[(k/128) * ld_sa + m], ld_sa >= M.
 *      a_kind must be BS_SCALE_1X128.
 *   b  [N, K] e4m3, ldb >= K;
 *      b_kind BS_SCALE_128X128: sb[(k/128) * ld_sb + n/128], ld_sb >= ceil(N/128),
 *             N % 128 == 0  (forward: b = W; dgrad: b = W^T from
 *             bs_quant_3d_colwise with G = 1)
 *      b_kind BS_SCALE_1X128:  sb[(k/128) * ld_sb + n],      ld_sb >= N
 *             (wgrad: a = grad_out^T, b = A^T, both from the col output of
 *             bs_quant_1x128)
 *   d  [M, N], ldd >= N, d_dtype BS_OUT_BF16 (uint16 bits) or BS_OUT_F32.
 *   M >= 0 (any), N % 128 == 0, K % 128 == 0.  K == 0 writes zeros.
 */
bs_status bs_scaled_mm(int64_t M, int64_t N, int64_t K,
                       const uint8_t* a, int64_t lda, const float* sa, int64_t ld_sa,
                       bs_scale_kind a_kind,
                       const uint8_t* b, int64_t ldb, const float* sb, int64_t ld_sb,
                       bs_scale_kind b_kind,
                       void* d, int64_t ldd, bs_dtype d_dtype,
                       hipStream_t stream);

/*
 * bs_scaled_mm_quant -- bs_scaled_mm with a bf16 output whose epilogue also
 * quantizes that output for the next layer: the 1x128 codes and scales of
 * the bf16 D, exactly as bs_quant_1x128 would write them from D (rows: blocks
 * of 128 consecutive columns of a row, the next layer's forward operand;
 * transposed columns: blocks of 128 consecutive rows of a column, its wgrad
 * operand), from the GEMM's registers instead of a second pass over D in HBM
 * (pages: prototype page, description -- quantization written as separate
 * kernels is the overhead a hand-written path removes).
 *   a, sa, b, sb, kinds, M, N, K   as bs_scaled_mm
 *   d      optional [M, N] bf16 output (ldd >= N); NULL: D is not written
 *   q_row, s_row   both NULL or both set: q_row[m * ld_qr + n] (ld_qr >= N),
 *                  s_row[(n / 128) * ld_sr + m] (ld_sr >= M, multiple of 4)
 *   q_col, s_col   both NULL or both set: q_col[n * ld_qc + m] (ld_qc >= M),
 *                  s_col[(m / 128) * ld_sc + n] (ld_sc >= N, multiple of 4);
 *                  requires M % 128 == 0
 *   At least one of d, the row pair, the column pair must be set.
 * Scale padding entries are never written.  Errors as bs_scaled_mm and
 * bs_quant_1x128.
 */
bs_status bs_scaled_mm_quant(int64_t M, int64_t N, int64_t K,
                             const uint8_t* a, int64_t lda, const float* sa, int64_t ld_sa,
                             bs_scale_kind a_kind,
                             const uint8_t* b, int64_t ldb, const float* sb, int64_t ld_sb,
                             bs_scale_kind b_kind,
                             uint16_t* d, int64_t ldd,
                             uint8_t* q_row, int64_t ld_qr, float* s_row, int64_t ld_sr,
                             uint8_t* q_col, int64_t ld_qc, float* s_col, int64_t ld_sc,
                             hipStream_t stream);

/*
 * bs_scaled_mm_ws -- bs_scaled_mm with a caller-provided device workspace
 * that lets the GPU balance a ragged last round of output tiles: when the
 * tiles are not a multiple of the GPU's resident workgroups and the last
 * round is at most 3/4 full, the K blocks of the last round's tiles are
 * divided evenly over all workgroups ("stream-K").  Two kernels on `stream`:
 * the GEMM computes the whole tiles into D and leaves the fp32 partial tile
 * of every piece of a split tile in the workspace; a reduction kernel adds
 * each split tile's partials in a fixed order and writes D (results are
 * reproducible run to run; they may differ from bs_scaled_mm's in the last
 * bits, since a split tile's K blocks are added in a different grouping --
 * both within the recipe's tolerance).  Same result definition as
 * bs_scaled_mm (pages: as there; the wgrad GEMM of an FFN layer can leave
 * part of the GPU idle in its last round of tiles).
 *
 *   All arguments as bs_scaled_mm, plus
 *   workspace        DEVICE memory, 256-byte aligned, owned by the caller;
 *                    no initial contents are needed.  NULL with
 *                    workspace_bytes == 0 is allowed.
 *   workspace_bytes  its size; bs_scaled_mm_workspace_bytes() gives what a
 *                    problem needs on the current device (one 256 x 256
 *                    fp32 tile per piece: split tiles + splitting
 *                    workgroups, at most 112 MiB on MI355X).  With less (or
 *                    for problems whose last round is full or more than 3/4
 *                    full) the call runs as bs_scaled_mm and does not touch
 *                    the workspace.
 * Calls that share a workspace must not overlap in time (use one stream, or
 * one workspace per stream).  Errors as bs_scaled_mm, plus BS_ERR_ALIGN for a
 * misaligned workspace and BS_ERR_NULL for a NULL one with nonzero size.
 */
bs_status bs_scaled_mm_ws(int64_t M, int64_t N, int64_t K,
                          const uint8_t* a, int64_t lda, const float* sa, int64_t ld_sa,
                          bs_scale_kind a_kind,
                          const uint8_t* b, int64_t ldb, const float* sb, int64_t ld_sb,
                          bs_scale_kind b_kind,
                          void* d, int64_t ldd, bs_dtype d_dtype,
                          void* workspace, int64_t workspace_bytes, hipStream_t stream);

/*
 * bs_scaled_mm_noalloc -- bs_scaled_mm_ws for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same kernels, with the workspace
 * replaced by a static device array of the library, 112 MiB on each GPU the
 * library runs on (held until the process ends).  The call makes no
 * allocation of any kind; the caller passes inputs and outputs only.  Every
 * call on one GPU shares that GPU's array (no contents need to survive
 * between calls): calls that overlap in time on one GPU (different streams,
 * or several threads) race -- issue them on one stream.  A problem whose
 * split would need more than the array holds is rejected with BS_ERR_SHAPE
 * (not on a 256-CU GPU, which needs at most 112 MiB); problems that are not
 * split run as bs_scaled_mm.  Arguments, result and errors as bs_scaled_mm;
 * BS_ERR_HIP if the device array cannot be located.
 */
bs_status bs_scaled_mm_noalloc(int64_t M, int64_t N, int64_t K,
                               const uint8_t* a, int64_t lda, const float* sa, int64_t ld_sa,
                               bs_scale_kind a_kind,
                               const uint8_t* b, int64_t ldb, const float* sb, int64_t ld_sb,
                               bs_scale_kind b_kind,
                               void* d, int64_t ldd, bs_dtype d_dtype, hipStream_t stream);

/* Workspace bytes bs_scaled_mm_ws uses for this problem on the current
 * device (0: the problem's tiles fill every round, no split).  Invalid
 * arguments also give 0. */
int64_t bs_scaled_mm_workspace_bytes(int64_t M, int64_t N, int64_t K, bs_scale_kind b_kind, bs_dtype d_dtype);

/*
 * bs_grouped_scaled_mm -- the MoE form of bs_scaled_mm (pages: prototype page,
 * description, which lists grouped forward and backward GEMMs for MoE;
 * "[mxfp8 moe training] ...", microbenchmark table, shapes (M, N, K, G)).
 *
 * group_end: DEVICE int32[G], cumulative ends of the G groups along the
 * grouped axis, non-decreasing, last == the axis length; zero-size groups are
 * allowed.  Read on the device (no host synchronization).  Kernels clamp
 * every end into [0, axis length] and treat a decreasing end as an empty
 * group, so malformed ends can never cause an out-of-bounds access.
 *
 *   BS_GROUP_M (forward, dgrad): rows [end_{g-1}, end_g) of A use expert g:
 *     a [M, K] 1x128 scales as in bs_scaled_mm; b_kind BS_SCALE_128X128;
 *     expert g's B is b + g*stride_bg ([N, K], ldb) with scales
 *     sb + g*stride_sbg (sb[(k/128)*ld_sb + n/128]);  d [M, N], ldd;
 *     stride_dg must be 0.  Rows past the last end are not written.
 *   BS_GROUP_K (wgrad): contraction groups; the ends must be multiples of 128:
 *     a [M, K] and b [N, K] both with 1x128 scales along K (sa[(k/128)*ld_sa + m],
 *     sb[(k/128)*ld_sb + n]); b_kind BS_SCALE_1X128; stride_bg and stride_sbg
 *     must be 0; expert g's result is d + g*stride_dg ([M, N], ldd),
 *     D_g = sum over k in [end_{g-1}, end_g); an empty group writes zeros.
 *   M >= 0 (GROUP_M) or M % 128 == 0 (GROUP_K); N % 128 == 0; K % 128 == 0.
 */
bs_status bs_grouped_scaled_mm(bs_group_mode mode, int64_t G, int64_t M, int64_t N, int64_t K,
                               const int32_t* group_end,
                               const uint8_t* a, int64_t lda, const float* sa, int64_t ld_sa,
                               const uint8_t* b, int64_t stride_bg, int64_t ldb,
                               const float* sb, int64_t stride_sbg, int64_t ld_sb,
                               bs_scale_kind b_kind,
                               void* d, int64_t stride_dg, int64_t ldd, bs_dtype d_dtype,
                               hipStream_t stream);

/* Human-readable name of a status code (static storage). */
const char* bs_status_string(bs_status status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* bs_last_error(void);

/* ------------------------------------------------------------------------
 * Diagnostics: exhaustive self-checks of the quantizers' arithmetic.  They
 * run the same device routines as the quantizer kernels.
 * ------------------------------------------------------------------------ */

/*
 * bs_diag_e4m3_census -- applies the quantizers' encode step (round to e4m3,
 * nearest even) to EVERY float32 value y with |y| <= 464 of both signs and
 * records, per output code c (0..255), the smallest and largest |y| bit
 * pattern (sign bit cleared) that produced it and how many did.  (Quantizer
 * quotients stay within 448 * (1 + 2^-23); the range up to 464 shows the
 * step saturates there without a clamp.)  Outputs: device uint32
 * min_bits[256], max_bits[256], uint64 counts[256]; codes never produced
 * have count 0.  Monotone rounding gives max_bits - min_bits + 1 == count
 * for every produced code.
 */
bs_status bs_diag_e4m3_census(uint32_t* min_bits, uint32_t* max_bits,
                              unsigned long long* counts, hipStream_t stream);

/*
 * bs_diag_division -- checks the quantizers' element division fl32(x / s)
 * against the correctly rounded IEEE division for every pair reachable from
 * bf16 inputs: s = fl32(max(amax, EPS) / 448) for every finite bf16 amax
 * >= 0 (amax = 0 takes the EPS floor), and every finite bf16 x of either
 * sign with |x| <= max(amax, EPS).  Output: device uint64 result[5] =
 * {pairs checked, scale mismatches, e4m3 code mismatches, quotient
 * mismatches with |x/s| >= 2^-10, quotient mismatches with |x/s| < 2^-10}.
 * The last count is informational: such quotients encode to a zero of the
 * quotient's sign whatever their low bits.
 */
bs_status bs_diag_division(unsigned long long* result, hipStream_t stream);

/*
 * bs_diag_stream -- the streaming reference of the HBM-bound kernels: reads
 * n_read bytes of src and writes n_write bytes of dst (n_read <= n_write,
 * both multiples of 16, 16-byte aligned device pointers) with the
 * quantizers' access pattern (16-byte loads and stores per lane, coalesced,
 * one workgroup per 32 KiB of input).  Timed on the byte counts of a
 * quantizer pass (e.g. 2 bytes read and 2.0625 written per element for 1x128
 * rows + transposed columns) it gives the practical ceiling that pass can
 * reach on the GPU.  The bytes written are not meaningful.
 */
bs_status bs_diag_stream(const void* src, int64_t n_read, void* dst, int64_t n_write, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* BS_H */
