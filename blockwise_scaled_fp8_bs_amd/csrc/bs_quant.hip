// Blockwise e4m3 quantizer kernels for gfx950.
//
// Every kernel works on 128x128 tiles of a bf16 matrix with 256 threads
// (4 wave64s).  Thread t owns an 8x8 sub-block: rows 8*(t/16) .. +7 and
// columns 8*(t%16) .. +7 of the tile, loaded as eight 16-byte row chunks, so
// a wave reads four full 256-byte row segments per load instruction.
//
//  * 1x128 row blocks: the 16 threads sharing a row group sit in one DPP row
//    of their wave; the block amax is a 4-step DPP max.
//  * 1x128 column blocks (128 consecutive rows of a column): per-thread max
//    over its 8 rows, shuffle over the 4 row groups of a wave, LDS over the 4
//    waves.  The codes are written transposed through an XOR-swizzled LDS
//    tile so that the global stores are full 128-byte rows of q^T.
//  * 128x128 blocks: one amax per tile (thread -> DPP row -> wave -> LDS).
//
// Each tile reads HBM once and writes each requested output once.
#include "bs_kernels.h"
#include "bs_device.h"

namespace bs {

namespace {

constexpr int kTile = 128;
constexpr int kThreads = 256;

struct TileRegs {
    float f[8][8];  // f[i][j]: row 8*tr + i, column 8*tc + j of the tile
};

__device__ __forceinline__ void load_tile(const uint16_t* __restrict__ x, int64_t ld_x, int64_t r0,
                                          int64_t c0, int64_t R, int tr, int tc, TileRegs& t) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t row = r0 + 8 * tr + i;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (row < R) v = *reinterpret_cast<const uint4*>(x + row * ld_x + c0 + 8 * tc);
        unpack8(v, t.f[i]);
    }
}

// Transposed store of an 8x8 block of codes per thread through LDS.
// codes[j] holds the 8 codes of column 8*tc + j for rows 8*tr .. 8*tr + 7.
// LDS tile: row c (a column of the source) is 128 bytes = 16 chunks of 8
// bytes; chunk tr is stored at physical chunk tr ^ tc, which spreads the 16
// lanes of a DPP row over all banks.
__device__ __forceinline__ void store_transposed(uint8_t* lds, const uint2* codes, int tr, int tc,
                                                 uint8_t* __restrict__ out, int64_t ld_out,
                                                 int64_t out_row0, int64_t out_col0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int c = 8 * tc + j;
        *reinterpret_cast<uint2*>(lds + c * kTile + ((tr ^ tc) * 8)) = codes[j];
    }
    __syncthreads();
    const int t = threadIdx.x;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int c = p * 32 + (t >> 3);
        const int k = t & 7;          // 16-byte chunk of the output row
        const int sw = (c >> 3) & 15;  // swizzle of LDS row c
        const int phys = (2 * k) ^ sw;  // physical 8-byte chunk of logical chunk 2k
        uint4 v = *reinterpret_cast<const uint4*>(lds + c * kTile + (phys & ~1) * 8);
        if (sw & 1) {  // the pair is stored swapped
            v = make_uint4(v.z, v.w, v.x, v.y);
        }
        *reinterpret_cast<uint4*>(out + (out_row0 + c) * ld_out + out_col0 + 16 * k) = v;
    }
}

template <bool ROW, bool COL>
__global__ __launch_bounds__(kThreads) void quant_1x128_kernel(Quant1x128Args a) {
    __shared__ float s_colmax[4][kTile];
    __shared__ __attribute__((aligned(16))) uint8_t s_tr[COL ? kTile * kTile : 16];

    const int t = threadIdx.x;
    const int tr = t >> 4, tc = t & 15;
    const int wave = t >> 6;
    const int64_t ct = blockIdx.x % a.col_tiles;
    const int64_t rt = blockIdx.x / a.col_tiles;
    const int64_t r0 = rt * kTile, c0 = ct * kTile;

    TileRegs tile;
    load_tile(a.x, a.ld_x, r0, c0, a.R, tr, tc, tile);

    if (ROW) {
        float my_scale = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float m = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(tile.f[i][j]));
            const uint32_t amax_bits = row16_max(__float_as_uint(m));
            const Scale sc = block_scale(__uint_as_float(amax_bits));
            const int64_t row = r0 + 8 * tr + i;
            const uint2 q = quant8(tile.f[i], sc);
            if (row < a.R) *reinterpret_cast<uint2*>(a.q_row + row * a.ld_qr + c0 + 8 * tc) = q;
            if ((tc & 7) == i) my_scale = sc.s;
        }
        // lanes tc < 8 store the scale of row 8*tr + tc: 32 consecutive rows per wave
        const int64_t row = r0 + 8 * tr + tc;
        if (tc < 8 && row < a.R) a.s_row[(c0 / kTile) * a.ld_sr + row] = my_scale;
    }

    if (COL) {
        // column amax over the tile's 128 rows
        float cm[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float m = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(tile.f[i][j]));
            m = fmaxf(m, __shfl_xor(m, 16));
            m = fmaxf(m, __shfl_xor(m, 32));
            cm[j] = m;
        }
        if ((t & 63) < 16) {
#pragma unroll
            for (int j = 0; j < 8; ++j) s_colmax[wave][8 * tc + j] = cm[j];
        }
        __syncthreads();
        Scale sc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int c = 8 * tc + j;
            const float m = fmaxf(fmaxf(s_colmax[0][c], s_colmax[1][c]),
                                  fmaxf(s_colmax[2][c], s_colmax[3][c]));
            sc[j] = block_scale(m);
        }
        uint2 codes[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            codes[j].x = encode4(div_by_scale(tile.f[0][j], sc[j]), div_by_scale(tile.f[1][j], sc[j]),
                                 div_by_scale(tile.f[2][j], sc[j]), div_by_scale(tile.f[3][j], sc[j]));
            codes[j].y = encode4(div_by_scale(tile.f[4][j], sc[j]), div_by_scale(tile.f[5][j], sc[j]),
                                 div_by_scale(tile.f[6][j], sc[j]), div_by_scale(tile.f[7][j], sc[j]));
        }
        if (t < 16) {
            float* dst = a.s_col + (r0 / kTile) * a.ld_sc + c0 + 8 * tc;
            *reinterpret_cast<float4*>(dst) = make_float4(sc[0].s, sc[1].s, sc[2].s, sc[3].s);
            *reinterpret_cast<float4*>(dst + 4) = make_float4(sc[4].s, sc[5].s, sc[6].s, sc[7].s);
        }
        store_transposed(s_tr, codes, tr, tc, a.q_col, a.ld_qc, c0, r0);
    }
}

// 128x128 quantizer; TRANSPOSE writes the tile transposed (3-D colwise).
template <bool TRANSPOSE>
__global__ __launch_bounds__(kThreads) void quant_128x128_kernel(Quant128Args a) {
    __shared__ float s_wmax[4];
    __shared__ __attribute__((aligned(16))) uint8_t s_tr[TRANSPOSE ? kTile * kTile : 16];

    const int t = threadIdx.x;
    const int tr = t >> 4, tc = t & 15;
    const int wave = t >> 6;
    const int64_t per_g = a.row_tiles * a.col_tiles;
    const int64_t g = blockIdx.x / per_g;
    const int64_t rem = blockIdx.x % per_g;
    const int64_t rt = rem / a.col_tiles, ct = rem % a.col_tiles;
    const int64_t r0 = rt * kTile, c0 = ct * kTile;
    const uint16_t* x = a.x + g * a.stride_xg;

    TileRegs tile;
    load_tile(x, a.ld_x, r0, c0, a.R, tr, tc, tile);

    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(tile.f[i][j]));
    uint32_t mb = row16_max(__float_as_uint(m));
    mb = max(mb, (uint32_t)__shfl_xor((int)mb, 16));
    mb = max(mb, (uint32_t)__shfl_xor((int)mb, 32));
    if ((t & 63) == 0) s_wmax[wave] = __uint_as_float(mb);
    __syncthreads();
    const float amax = fmaxf(fmaxf(s_wmax[0], s_wmax[1]), fmaxf(s_wmax[2], s_wmax[3]));
    const Scale sc = block_scale(amax);

    uint8_t* q = a.q + g * a.stride_qg;
    if (!TRANSPOSE) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t row = r0 + 8 * tr + i;
            *reinterpret_cast<uint2*>(q + row * a.ld_q + c0 + 8 * tc) = quant8(tile.f[i], sc);
        }
        if (t == 0) a.s[g * a.stride_sg + ct * a.ld_s + rt] = sc.s;
    } else {
        uint2 codes[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            codes[j].x = encode4(div_by_scale(tile.f[0][j], sc), div_by_scale(tile.f[1][j], sc),
                                 div_by_scale(tile.f[2][j], sc), div_by_scale(tile.f[3][j], sc));
            codes[j].y = encode4(div_by_scale(tile.f[4][j], sc), div_by_scale(tile.f[5][j], sc),
                                 div_by_scale(tile.f[6][j], sc), div_by_scale(tile.f[7][j], sc));
        }
        if (t == 0) a.s[g * a.stride_sg + rt * a.ld_s + ct] = sc.s;
        store_transposed(s_tr, codes, tr, tc, q, a.ld_q, c0, r0);
    }
}

}  // namespace

hipError_t launch_quant_1x128(const Quant1x128Args& a, bool row, bool col, hipStream_t stream) {
    const int64_t row_tiles = (a.R + kTile - 1) / kTile;
    const int64_t blocks = row_tiles * a.col_tiles;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)blocks), block(kThreads);
    if (row && col)
        hipLaunchKernelGGL((quant_1x128_kernel<true, true>), grid, block, 0, stream, a);
    else if (row)
        hipLaunchKernelGGL((quant_1x128_kernel<true, false>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((quant_1x128_kernel<false, true>), grid, block, 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_quant_128x128(const Quant128Args& a, bool transpose, hipStream_t stream) {
    const int64_t blocks = a.G * a.row_tiles * a.col_tiles;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)blocks), block(kThreads);
    if (transpose)
        hipLaunchKernelGGL((quant_128x128_kernel<true>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((quant_128x128_kernel<false>), grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace bs
