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
// Workgroups are persistent: each walks the tiles with a grid stride and
// loads the next tile's bf16 data into registers before working on the
// current one, so HBM reads overlap the arithmetic and no partly filled last
// wave of workgroups is left (passes over large operands launch one
// workgroup per tile instead: persistent_blocks).  LDS buffers alternate
// between consecutive tiles, so one barrier per LDS exchange suffices.  Each
// tile reads HBM once and writes each requested output once.
#include "bs_kernels.h"
#include "bs_device.h"
#include "bs_mx.h"

namespace bs {

namespace {

constexpr int kTile = 128;
constexpr int kThreads = 256;

struct Raw {
    uint4 v[8];  // v[i]: row 8*tr + i, columns 8*tc .. +7 (bf16)
};

struct TileRegs {
    float f[8][8];  // f[i][j]: row 8*tr + i, column 8*tc + j of the tile
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Raw buffer over [base, base + bytes): loads past the end read zero and
// stores past the end are dropped, which handles ragged tiles without
// per-lane bounds checks; the tile origin lives in the (scalar) descriptor
// and lanes keep 32-bit offsets.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
    const int32_t n = bytes > 0x7fffffff ? 0x7fffffff : (bytes < 0 ? 0 : (int32_t)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

// Rows [r0, r0 + 128) of a tile whose first column is c0; rows >= R read as 0.
__device__ __forceinline__ void load_raw(const uint16_t* __restrict__ x, int64_t ld_x, int64_t r0, int64_t c0,
                                         int64_t R, int voff, Raw& raw) {
    const int64_t rows = (R - r0) < kTile ? (R - r0) : kTile;
    const __amdgpu_buffer_rsrc_t rx = rsrc(x + r0 * ld_x + c0, rows * ld_x * 2);
    const int row_bytes = (int)(ld_x * 2);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, voff, i * row_bytes, 0));
        raw.v[i] = make_uint4(v[0], v[1], v[2], v[3]);
    }
}

__device__ __forceinline__ void unpack_tile(const Raw& raw, TileRegs& t) {
#pragma unroll
    for (int i = 0; i < 8; ++i) unpack8(raw.v[i], t.f[i]);
}

// Transposed store of an 8x8 block of codes per thread through LDS.
// codes[j] holds the 8 codes of column 8*tc + j for rows 8*tr .. 8*tr + 7.
// LDS tile: row c (a column of the source) is 128 bytes = 16 chunks of 8
// bytes; chunk tr is stored at physical chunk tr ^ tc, which spreads the 16
// lanes of a DPP row over all banks.  `out` points at output row 0, column 0
// of the tile; 8 lanes write each 128-byte output row.
__device__ __forceinline__ void store_transposed(uint8_t* lds, const uint2* codes, int tr, int tc,
                                                 uint8_t* __restrict__ out, int64_t ld_out) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int c = 8 * tc + j;
        *reinterpret_cast<uint2*>(lds + c * kTile + ((tr ^ tc) * 8)) = codes[j];
    }
    __syncthreads();
    const int t = threadIdx.x;
    const __amdgpu_buffer_rsrc_t ro = rsrc(out, (kTile - 1) * ld_out + kTile);
    const int voff = (t >> 3) * (int)ld_out + 16 * (t & 7);
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
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{v.x, v.y, v.z, v.w}, ro, voff, p * 32 * (int)ld_out, 0);
    }
}

__device__ __forceinline__ void col_codes(const TileRegs& tile, const Scale* sc, uint2* codes) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        codes[j].x = encode4(div_by_scale(tile.f[0][j], sc[j]), div_by_scale(tile.f[1][j], sc[j]),
                             div_by_scale(tile.f[2][j], sc[j]), div_by_scale(tile.f[3][j], sc[j]));
        codes[j].y = encode4(div_by_scale(tile.f[4][j], sc[j]), div_by_scale(tile.f[5][j], sc[j]),
                             div_by_scale(tile.f[6][j], sc[j]), div_by_scale(tile.f[7][j], sc[j]));
    }
}

// ---- the FFN's gated activation h = silu(a) * b and its derivative ----
// The value quantized is the float64 formula rounded once to bf16 (nearest
// even).  Each kernel evaluates it in fp32 (relative error below 2^-20 where
// no intermediate leaves the normal range) and takes that value's bf16
// rounding unless it lies within the error bound of a rounding tie, where
// (rarely) the float64 formula is evaluated instead.

// Distance of r from the nearest bf16 rounding tie, in fp32 units in the last
// place (the low 16 bits of r against the half step 0x8000).
__device__ __forceinline__ float tie_distance(float r) {
    // in float: the low half-word and its distance to 0x8000 are small
    // integers, exact in fp32 (4 instructions with the caller's - 16, against
    // 7 for the integer form)
    return fabsf((float)(__float_as_uint(r) & 0xFFFFu) - 32768.0f);
}

// float64 -> bf16 (as float), nearest even, one rounding: the fp64 -> fp32
// step rounds to odd (truncate, set the last bit if inexact), which keeps 16
// more bits than bf16, so the final fp32 -> bf16 rounding is the correct one.
__device__ __forceinline__ float bf16_from_double(double d) {
    float f = (float)d;
    if ((double)f != d) {
        uint32_t u = __float_as_uint(f);
        if (fabs((double)f) > fabs(d)) u -= 1u;  // step toward zero (inf -> FLT_MAX)
        f = __uint_as_float(u | 1u);
    }
    return (float)(__bf16)f;
}

constexpr float kTieWindow = 16.0f;   // fp32 ulps; the fp32 paths err by < 8

// tie_distance(r) > kTieWindow in two 16-bit integer instructions: the low
// half-word of r shifted so that the window [0x8000 - 16, 0x8000 + 16] maps
// to [0, 32].
__device__ __forceinline__ bool off_tie(float r) {
    return (uint16_t)(__float_as_uint(r) - (0x8000u - 16u)) > 32u;
}
constexpr float kMinNormal = 1.17549435e-38f;  // 2^-126

// The float64 evaluations, for the few elements in a thousand the fp32 paths
// leave undecided; each kernel calls them from one per-lane loop, outside its
// unrolled fp32 code.
__device__ __forceinline__ float swiglu_bf16_f64(float a, float b) {
    const double ad = a;
    return bf16_from_double(ad / (1.0 + exp(-ad)) * (double)b);
}

// da and db in float64 for the elements the fp32 path leaves undecided.
__device__ __forceinline__ float2 swiglu_grad_bf16_f64(float a, float b, float dh) {
    const double ad = a, bd = b, dd = dh;
    const double sd = 1.0 / (1.0 + exp(-ad));
    const double snd = 1.0 / (1.0 + exp(ad));
    return make_float2(bf16_from_double(dd * bd * sd * (1.0 + ad * snd)), bf16_from_double(dd * (ad * sd)));
}

// Undecided elements come out as +inf (bf16 0x7F80), which marks them for the
// float64 pass (the fp32 paths never return a true infinity: it is undecided).
constexpr uint32_t kRedoBits = 0x7F80u;

// exp(-a) in fp32 from the hardware base-2 exponential: -a log2(e) is
// formed as a rounded head ph plus its tail pl (the product's rounding error,
// exact by fma, and the part of log2(e) below fp32), and 2^(ph + pl) is taken
// as 2^ph (1 + pl ln 2).  On every bf16 value a with a normal result this is
// within 1.12 fp32 ulps of exp(-a) (the library expf: 0.76 ulps), at 6
// instructions instead of 13; results below the normal range come out as 0,
// where 1 + exp(-a) is 1 anyway.
constexpr float kLog2e = 1.44269502162933349609375f;  // log2(e) rounded to fp32
constexpr float kLog2eTail = 1.925963e-08f;           // log2(e) - kLog2e
constexpr float kLn2 = 0.693147180559945309f;
__device__ __forceinline__ float exp_neg(float a) {
    const float ph = -a * kLog2e;
    const float pl = __builtin_fmaf(-a, kLog2eTail, __builtin_fmaf(-a, kLog2e, -ph));
    const float e = __builtin_amdgcn_exp2f(ph);
    return __builtin_fmaf(e, pl * kLn2, e);
}

// h = silu(a) * b in fp32, to be rounded once to bf16 (nearest even) by the
// caller's packing; +inf (to be redone in float64) where a <= -69 (exp(-a)
// near fp32 overflow), silu(a) is subnormal,
// the product is not finite, or it lies near a rounding tie.  The quotient is
// a times the hardware reciprocal of 1 + exp(-a) (1 ulp; 1 + exp(-a) >= 1 is
// never subnormal); with exp_neg's 1.12 ulps the fp32 value errs by < 8 ulps,
// half the tie window.
__device__ __forceinline__ float swiglu_fast(float a, float b) {
    const float silu = a * __builtin_amdgcn_rcpf(1.0f + exp_neg(a));
    const float r = silu * b;
    const bool normal = silu == 0.0f || fabsf(silu) >= kMinNormal;
    const bool ok = a > -69.0f && normal && __builtin_isfinite(r) && off_tie(r);
    return ok ? r : __builtin_inff();
}

// da = dh * b * silu'(a) and db = dh * silu(a), silu'(a) = s (1 + a (1 - s)),
// s = 1 / (1 + exp(-a)), in fp32, each to be rounded once to bf16 by the
// caller's packing; da = +inf where
// either rounding is not certain to be the float64 formula's (a <= -69,
// an intermediate outside the normal range, or a value near a tie).  One
// exponential serves both sigmoids: 1 - s = exp(-a) s (within 2.3 ulps of
// 1 / (1 + exp(a)) on every bf16 a, as s is of its value).  Near
// silu'(a) = 0 the sum t = 1 + a (1 - s) cancels, so da's window adds
// 8 |a (1 - s)| / |t| ulps (infinite at t = 0), written without a division.
// The reciprocal is the hardware's (1 ulp; its argument is >= 1, never
// subnormal), inside both windows' margins.
__device__ __forceinline__ void swiglu_grad_fast(float a, float b, float dh, float& da, float& db) {
    const float e = exp_neg(a);
    const float s = __builtin_amdgcn_rcpf(1.0f + e);
    const float sn = e * s;
    const float t = __builtin_fmaf(a, sn, 1.0f);
    const float p1 = dh * b, p2 = p1 * s;
    const float rda = p2 * t;
    const float silu = a * s;
    const float rdb = dh * silu;
    // bitwise & of the conditions: all are cheap to evaluate, and
    // short-circuit && would make the compiler branch per element
    const bool ok_a = __builtin_isfinite(rda) &
                      ((p1 == 0.0f) | ((fabsf(p1) >= kMinNormal) & (fabsf(p2) >= kMinNormal))) &
                      ((tie_distance(rda) - kTieWindow) * fabsf(t) > 8.0f * fabsf(a * sn));
    const bool ok_b = __builtin_isfinite(rdb) & ((silu == 0.0f) | (fabsf(silu) >= kMinNormal)) & off_tie(rdb);
    const bool ok = (a > -69.0f) & ok_a & ok_b;
    da = ok ? rda : __builtin_inff();
    db = rdb;
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lo) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hi) << 16);
}

// Word k (0..31, static) of a thread's packed 8x8 block: row k / 4,
// columns 2 (k % 4) and 2 (k % 4) + 1.
__device__ __forceinline__ uint32_t raw_word(const Raw& r, int k) {
    const uint4 v = r.v[k >> 2];
    return (k & 3) == 0 ? v.x : (k & 3) == 1 ? v.y : (k & 3) == 2 ? v.z : v.w;
}

// Replaces element e (per lane: row e / 8, column e % 8) of a packed block by
// a bf16-exact value (rare path).  Branch-free blends: every word is rewritten
// with a mask that is zero except at the target half-word, so the block stays
// in registers (per-word conditional stores can be turned into an indexed
// store, which puts the block in private memory).
__device__ __forceinline__ void raw_set(Raw& r, int e, float v) {
    const uint32_t w = (uint32_t)e >> 1;
    const uint32_t h16 = __float_as_uint(v) >> 16;
    const uint32_t field = (e & 1) ? 0xFFFF0000u : 0x0000FFFFu;
    const uint32_t put = (e & 1) ? (h16 << 16) : h16;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t mx = (4u * i + 0u == w) ? field : 0u, my = (4u * i + 1u == w) ? field : 0u;
        const uint32_t mz = (4u * i + 2u == w) ? field : 0u, mw = (4u * i + 3u == w) ? field : 0u;
        r.v[i].x = (r.v[i].x & ~mx) | (put & mx);
        r.v[i].y = (r.v[i].y & ~my) | (put & my);
        r.v[i].z = (r.v[i].z & ~mz) | (put & mz);
        r.v[i].w = (r.v[i].w & ~mw) | (put & mw);
    }
}

// Re-evaluates, in float64, the elements of a thread's packed block that the
// fp32 path marked (+inf); fn(e) does element e.  The marks are found with
// integer arithmetic only (per-element compares would keep 64 lane masks
// alive), and the loop runs per lane: a wave spends one pass per marked
// element of its busiest lane (usually none or one per tile).
template <typename F>
__device__ __forceinline__ void fixup_block(const Raw& marked, F&& fn) {
    uint32_t m[2] = {0u, 0u};  // elements 0..31, 32..63
#pragma unroll
    for (int k = 0; k < 32; ++k) {
        const uint32_t w = raw_word(marked, k);
        const uint32_t lo = ((w & 0xFFFFu) ^ kRedoBits) - 1u, hi = ((w >> 16) ^ kRedoBits) - 1u;
        m[k >> 4] |= ((lo >> 31) << ((2 * k) & 31)) | ((hi >> 31) << ((2 * k + 1) & 31));
    }
    for (int h = 0; h < 2; ++h) {
        uint32_t mask = m[h];
        while (mask != 0) {
            const int e = 32 * h + __builtin_ctz(mask);
            mask &= mask - 1;
            fn(e);
        }
    }
}

// 1x128 row blocks of one tile: codes to q (the tile's first element; rows
// past `rows` are dropped), scales to s (the tile's entries of one K-major
// scale row).
__device__ __forceinline__ void quant_tile_rows(const TileRegs& tl, int64_t rows, uint8_t* q, int64_t ld_q,
                                                float* s, int tr, int tc) {
    const __amdgpu_buffer_rsrc_t rq = rsrc(q, rows * ld_q);
    const int voff_q = (8 * tr) * (int)ld_q + 8 * tc;
    float my_scale = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float m = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(tl.f[i][j]));
        const uint32_t amax_bits = row16_max(__float_as_uint(m));
        const Scale sc = block_scale(__uint_as_float(amax_bits));
        const uint2 qv = quant8(tl.f[i], sc);
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{qv.x, qv.y}, rq, voff_q, i * (int)ld_q, 0);
        if ((tc & 7) == i) my_scale = sc.s;
    }
    // lanes tc < 8 store the scale of row 8*tr + tc: 32 consecutive rows per wave
    const __amdgpu_buffer_rsrc_t rs = rsrc(s, rows * 4);
    if (tc < 8) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(my_scale), rs, (8 * tr + tc) * 4, 0, 0);
}

// 1x128 column blocks (the tile's 128 rows) of one tile: codes written
// transposed to qt (row c0 of q^T, column r0), scales to s (128 consecutive
// entries of one K-major scale row).  colmax and tr_lds are this call's LDS
// buffers (alternate between consecutive calls); it holds barriers, so every
// thread of the workgroup calls it.
__device__ __forceinline__ void quant_tile_cols(const TileRegs& tl, uint8_t* qt, int64_t ld_qt, float* s,
                                                float (*colmax)[kTile], uint8_t* tr_lds, int tr, int tc, int wave) {
    float cm[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        float m = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(tl.f[i][j]));
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        cm[j] = m;
    }
    if ((threadIdx.x & 63) < 16) {
#pragma unroll
        for (int j = 0; j < 8; ++j) colmax[wave][8 * tc + j] = cm[j];
    }
    __syncthreads();
    Scale sc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int c = 8 * tc + j;
        const float m = fmaxf(fmaxf(colmax[0][c], colmax[1][c]), fmaxf(colmax[2][c], colmax[3][c]));
        sc[j] = block_scale(m);
    }
    uint2 codes[8];
    col_codes(tl, sc, codes);
    if (threadIdx.x < 16) {
        const __amdgpu_buffer_rsrc_t rs = rsrc(s, kTile * 4);
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4{__float_as_uint(sc[0].s), __float_as_uint(sc[1].s), __float_as_uint(sc[2].s),
                  __float_as_uint(sc[3].s)}, rs, 32 * tc, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4{__float_as_uint(sc[4].s), __float_as_uint(sc[5].s), __float_as_uint(sc[6].s),
                  __float_as_uint(sc[7].s)}, rs, 32 * tc + 16, 0, 0);
    }
    store_transposed(tr_lds, codes, tr, tc, qt, ld_qt);
}

// bf16 values of a tile's rows (already bf16-exact floats) -> packed rows.
__device__ __forceinline__ void pack_tile(const TileRegs& tl, Raw& raw) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
        raw.v[i] = make_uint4(pack_bf16(tl.f[i][0], tl.f[i][1]), pack_bf16(tl.f[i][2], tl.f[i][3]),
                              pack_bf16(tl.f[i][4], tl.f[i][5]), pack_bf16(tl.f[i][6], tl.f[i][7]));
}

// Packed rows of a tile to out (the tile's first element; rows past `rows`
// are dropped).
__device__ __forceinline__ void store_raw(const Raw& raw, uint16_t* out, int64_t ld_out, int64_t rows, int tr,
                                          int tc) {
    const __amdgpu_buffer_rsrc_t ro = rsrc(out, rows * ld_out * 2);
    const int voff = (8 * tr) * (int)(ld_out * 2) + 16 * tc;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{raw.v[i].x, raw.v[i].y, raw.v[i].z, raw.v[i].w}, ro, voff,
                                               i * (int)(ld_out * 2), 0);
}

// 1x128 quantizer (rows and/or transposed columns).  SWIGLU quantizes
// h = bf16(silu(x) * y) instead of x, from one read of x and y, and writes
// h too when a.h is set.  ONE: the form for a grid of one workgroup per tile
// (the loop then runs once): each tile's inputs are loaded where they are
// used, with no registers held for the next tile's, so that more waves fit
// on a SIMD.
template <bool ROW, bool COL, bool SWIGLU, bool ONE>
__global__ __launch_bounds__(kThreads) void quant_1x128_kernel(Quant1x128Args a) {
    // ONE: a single LDS set (18 KiB instead of 36), a barrier between tiles
    // in the rare case that the grid is smaller than the tile count
    constexpr int kSets = ONE ? 1 : 2;
    __shared__ float s_colmax[kSets][4][kTile];
    __shared__ __attribute__((aligned(16))) uint8_t s_tr[COL ? kSets : 1][COL ? kTile * kTile : 16];

    const int t = threadIdx.x;
    const int tr = t >> 4, tc = t & 15;
    const int wave = t >> 6;
    const int64_t ntiles = ((a.R + kTile - 1) / kTile) * a.col_tiles;

    int64_t tile = blockIdx.x;
    if (tile >= ntiles) return;
    const int voff_x = (8 * tr) * (int)(a.ld_x * 2) + 16 * tc;
    const int voff_y = SWIGLU ? (8 * tr) * (int)(a.ld_y * 2) + 16 * tc : 0;
    Raw raw, raw_y;
    if (!ONE) {
        load_raw(a.x, a.ld_x, (tile / a.col_tiles) * kTile, (tile % a.col_tiles) * kTile, a.R, voff_x, raw);
        if (SWIGLU)
            load_raw(a.y, a.ld_y, (tile / a.col_tiles) * kTile, (tile % a.col_tiles) * kTile, a.R, voff_y, raw_y);
    }

    for (int parity = 0; tile < ntiles; tile += gridDim.x, parity ^= 1) {
        const int64_t r0 = (tile / a.col_tiles) * kTile, c0 = (tile % a.col_tiles) * kTile;
        const int64_t rows = (a.R - r0) < kTile ? (a.R - r0) : kTile;
        if (ONE) {
            load_raw(a.x, a.ld_x, r0, c0, a.R, voff_x, raw);
            if (SWIGLU) load_raw(a.y, a.ld_y, r0, c0, a.R, voff_y, raw_y);
        }
        TileRegs tl;
        Raw ph;  // gated form: h packed as bf16, +inf where the fp32 path left it undecided
        if (SWIGLU) {
            // row by row from the packed inputs, so that no float tile is live
            // while the next tile's inputs are loaded
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float fa[8], fb[8], g[8];
                unpack8(raw.v[i], fa);
                unpack8(raw_y.v[i], fb);
#pragma unroll
                for (int j = 0; j < 8; ++j) g[j] = swiglu_fast(fa[j], fb[j]);
                ph.v[i] = make_uint4(pack_bf16(g[0], g[1]), pack_bf16(g[2], g[3]), pack_bf16(g[4], g[5]),
                                     pack_bf16(g[6], g[7]));
            }
        } else {
            unpack_tile(raw, tl);
        }
        const int64_t next = tile + gridDim.x;
        if (!ONE && next < ntiles) {
            load_raw(a.x, a.ld_x, (next / a.col_tiles) * kTile, (next % a.col_tiles) * kTile, a.R, voff_x, raw);
            if (SWIGLU)
                load_raw(a.y, a.ld_y, (next / a.col_tiles) * kTile, (next % a.col_tiles) * kTile, a.R, voff_y,
                         raw_y);
        }
        if (SWIGLU) {
            // undecided elements: their inputs are read again (a few per tile)
            // and h is recomputed in float64
            fixup_block(ph, [&](int e) {
                const int64_t r = r0 + 8 * tr + (e >> 3), c = c0 + 8 * tc + (e & 7);
                if (r >= a.R) return;  // rows past the end read as zeros and are never marked
                raw_set(ph, e, swiglu_bf16_f64(__uint_as_float((uint32_t)a.x[r * a.ld_x + c] << 16),
                                                     __uint_as_float((uint32_t)a.y[r * a.ld_y + c] << 16)));
            });
            if (a.h != nullptr) store_raw(ph, a.h + r0 * a.ld_h + c0, a.ld_h, rows, tr, tc);
            unpack_tile(ph, tl);
        }
        if (ROW) quant_tile_rows(tl, rows, a.q_row + r0 * a.ld_qr + c0, a.ld_qr, a.s_row + (c0 / kTile) * a.ld_sr + r0, tr, tc);
        if (COL) {
            quant_tile_cols(tl, a.q_col + c0 * a.ld_qc + r0, a.ld_qc, a.s_col + (r0 / kTile) * a.ld_sc + c0,
                            s_colmax[ONE ? 0 : parity], s_tr[ONE ? 0 : parity], tr, tc, wave);
            if (ONE && tile + gridDim.x < ntiles) __syncthreads();
        }
    }
}

// Backward of the gated activation fused with the 1x128 quantizer: from one
// read of a, b and dh ([R, C] bf16) it forms da and db (each rounded once to
// bf16) and quantizes the [R, 2C] matrix [da | db] along rows and/or its
// transposed columns; [da | db] itself is written when a.dab is set.  Each
// input tile gives two output tiles: da's at columns c0, db's at C + c0.
template <bool ROW, bool COL>
__global__ __launch_bounds__(kThreads) void swiglu_bwd_quant_kernel(SwigluBwdArgs a) {
    __shared__ float s_colmax[2][4][kTile];
    __shared__ __attribute__((aligned(16))) uint8_t s_tr[COL ? 2 : 1][COL ? kTile * kTile : 16];

    const int t = threadIdx.x;
    const int tr = t >> 4, tc = t & 15;
    const int wave = t >> 6;
    const int64_t ntiles = ((a.R + kTile - 1) / kTile) * a.col_tiles;

    int64_t tile = blockIdx.x;
    if (tile >= ntiles) return;
    const int voff_a = (8 * tr) * (int)(a.ld_a * 2) + 16 * tc;
    const int voff_b = (8 * tr) * (int)(a.ld_b * 2) + 16 * tc;
    const int voff_d = (8 * tr) * (int)(a.ld_dh * 2) + 16 * tc;
    auto load3 = [&](int64_t tl_id, Raw& ra, Raw& rb, Raw& rd) {
        const int64_t r0 = (tl_id / a.col_tiles) * kTile, c0 = (tl_id % a.col_tiles) * kTile;
        load_raw(a.a, a.ld_a, r0, c0, a.R, voff_a, ra);
        load_raw(a.b, a.ld_b, r0, c0, a.R, voff_b, rb);
        load_raw(a.dh, a.ld_dh, r0, c0, a.R, voff_d, rd);
    };
    int parity = 0;
    for (; tile < ntiles; tile += gridDim.x) {
        const int64_t r0 = (tile / a.col_tiles) * kTile, c0 = (tile % a.col_tiles) * kTile;
        const int64_t rows = (a.R - r0) < kTile ? (a.R - r0) : kTile;
        const int64_t C = a.col_tiles * kTile;
        // No prefetch of the next tile: a, b and dh of two tiles would not fit
        // beside the outputs; two workgroups per SIMD hide the latency instead.
        Raw ra, rb, rd;
        load3(tile, ra, rb, rd);
        Raw pda, pdb;  // da and db of the tile, packed bf16 (da marked where undecided)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float fa[8], fb[8], fd[8], ga[8], gb[8];
            unpack8(ra.v[i], fa);
            unpack8(rb.v[i], fb);
            unpack8(rd.v[i], fd);
#pragma unroll
            for (int j = 0; j < 8; ++j) swiglu_grad_fast(fa[j], fb[j], fd[j], ga[j], gb[j]);
            pda.v[i] = make_uint4(pack_bf16(ga[0], ga[1]), pack_bf16(ga[2], ga[3]), pack_bf16(ga[4], ga[5]),
                                  pack_bf16(ga[6], ga[7]));
            pdb.v[i] = make_uint4(pack_bf16(gb[0], gb[1]), pack_bf16(gb[2], gb[3]), pack_bf16(gb[4], gb[5]),
                                  pack_bf16(gb[6], gb[7]));
        }
        // undecided elements: their inputs are read again (a few per tile)
        fixup_block(pda, [&](int e) {
            const int64_t r = r0 + 8 * tr + (e >> 3), c = c0 + 8 * tc + (e & 7);
            if (r >= a.R) return;  // rows past the end read as zeros and are never marked
            const float2 g = swiglu_grad_bf16_f64(__uint_as_float((uint32_t)a.a[r * a.ld_a + c] << 16),
                                                  __uint_as_float((uint32_t)a.b[r * a.ld_b + c] << 16),
                                                  __uint_as_float((uint32_t)a.dh[r * a.ld_dh + c] << 16));
            raw_set(pda, e, g.x);
            raw_set(pdb, e, g.y);
        });
        if (a.dab != nullptr) {
            store_raw(pda, a.dab + r0 * a.ld_dab + c0, a.ld_dab, rows, tr, tc);
            store_raw(pdb, a.dab + r0 * a.ld_dab + C + c0, a.ld_dab, rows, tr, tc);
        }
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int64_t co = (half ? C : 0) + c0;  // output column of the tile
            TileRegs tl;
            unpack_tile(half ? pdb : pda, tl);
            if (ROW)
                quant_tile_rows(tl, rows, a.q_row + r0 * a.ld_qr + co, a.ld_qr, a.s_row + (co / kTile) * a.ld_sr + r0,
                                tr, tc);
            if (COL) {
                quant_tile_cols(tl, a.q_col + co * a.ld_qc + r0, a.ld_qc, a.s_col + (r0 / kTile) * a.ld_sc + co,
                                s_colmax[parity], s_tr[parity], tr, tc, wave);
                parity ^= 1;
            }
        }
    }
}

// ---- MXFP8 (OCP Microscaling reading): 32-element blocks, E8M0 scales ----
// E8M0 byte of a block, floor(log2(amax)) - 8 + 127, from amax's exponent
// field; an amax below 2^-119 (scale exponent under -127), a subnormal amax
// or zero gives the smallest scale, byte 0.
__device__ __forceinline__ uint32_t mx_scale_byte(float amax) {
    const uint32_t ex = (__float_as_uint(amax) >> 23) & 0xFFu;
    return ex > 8u ? ex - 8u : 0u;
}

// Four elements divided by 2^(byte - 127) (exact: a power-of-two scaling),
// saturated at +-448, encoded (round to nearest even, sign kept).
__device__ __forceinline__ uint32_t mx_encode4(float x0, float x1, float x2, float x3, uint32_t byte) {
    const int ne = 127 - (int)byte;
    return encode4(clamp448(__builtin_amdgcn_ldexpf(x0, ne)), clamp448(__builtin_amdgcn_ldexpf(x1, ne)),
                   clamp448(__builtin_amdgcn_ldexpf(x2, ne)), clamp448(__builtin_amdgcn_ldexpf(x3, ne)));
}

// MX quantizer over 128x128 tiles: ROW writes 32-element blocks along each
// row (q_row [R, C], s_row[(c / 32) * ld_sr + r]); COL writes blocks of 32
// consecutive rows of each column, transposed (q_col [C, R],
// s_col[(r / 32) * ld_sc + c]).  A row block spans the 4 threads of a lane
// quad (8 columns each); a column block spans the 4 row groups of one wave.
template <bool ROW, bool COL>
__global__ __launch_bounds__(kThreads) void mx_quant_kernel(MxQuantArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t s_tr[COL ? 2 : 1][COL ? kTile * kTile : 16];

    const int t = threadIdx.x;
    const int tr = t >> 4, tc = t & 15;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int64_t ntiles = ((a.R + kTile - 1) / kTile) * a.col_tiles;

    int64_t tile = blockIdx.x;
    if (tile >= ntiles) return;
    const int voff_x = (8 * tr) * (int)(a.ld_x * 2) + 16 * tc;
    Raw raw;
    load_raw(a.x, a.ld_x, (tile / a.col_tiles) * kTile, (tile % a.col_tiles) * kTile, a.R, voff_x, raw);

    for (int parity = 0; tile < ntiles; tile += gridDim.x, parity ^= 1) {
        const int64_t r0 = (tile / a.col_tiles) * kTile, c0 = (tile % a.col_tiles) * kTile;
        const int64_t rows = (a.R - r0) < kTile ? (a.R - r0) : kTile;
        TileRegs tl;
        unpack_tile(raw, tl);
        const int64_t next = tile + gridDim.x;
        if (next < ntiles)
            load_raw(a.x, a.ld_x, (next / a.col_tiles) * kTile, (next % a.col_tiles) * kTile, a.R, voff_x, raw);

        if (ROW) {
            const __amdgpu_buffer_rsrc_t rq = rsrc(a.q_row + r0 * a.ld_qr + c0, rows * a.ld_qr);
            const int voff_q = (8 * tr) * (int)a.ld_qr + 8 * tc;
            // scale bytes of the tile's 4 column blocks (the lane quad of columns 8tc.. shares block tc / 4):
            // uniform descriptor over the 4 scale rows, the block in the lane offset, rows checked explicitly
            const __amdgpu_buffer_rsrc_t rs = rsrc(a.s_row + (c0 / 32) * a.ld_sr + r0, 3 * a.ld_sr + rows);
            const int voff_s = (tc / 4) * (int)a.ld_sr;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float m = 0.f;
#pragma unroll
                for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(tl.f[i][j]));
                uint32_t mb = __float_as_uint(m);
                mb = max(mb, (uint32_t)__builtin_amdgcn_mov_dpp((int)mb, 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
                mb = max(mb, (uint32_t)__builtin_amdgcn_mov_dpp((int)mb, 0x4E, 0xF, 0xF, false));  // quad_perm 2,3,0,1
                const uint32_t byte = mx_scale_byte(__uint_as_float(mb));
                const uint32_t lo = mx_encode4(tl.f[i][0], tl.f[i][1], tl.f[i][2], tl.f[i][3], byte);
                const uint32_t hi = mx_encode4(tl.f[i][4], tl.f[i][5], tl.f[i][6], tl.f[i][7], byte);
                __builtin_amdgcn_raw_buffer_store_b64(u32x2{lo, hi}, rq, voff_q, i * (int)a.ld_qr, 0);
                // one byte store per row: rows past the end are dropped, nothing beyond is written
                if ((tc & 3) == 0 && 8 * tr + i < rows)
                    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)byte, rs, voff_s + 8 * tr + i, 0, 0);
            }
        }
        if (COL) {
            uint2 codes[8];
            uint32_t bytes[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float m = 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(tl.f[i][j]));
                m = fmaxf(m, __shfl_xor(m, 16));
                m = fmaxf(m, __shfl_xor(m, 32));
                bytes[j] = mx_scale_byte(m);
                codes[j].x = mx_encode4(tl.f[0][j], tl.f[1][j], tl.f[2][j], tl.f[3][j], bytes[j]);
                codes[j].y = mx_encode4(tl.f[4][j], tl.f[5][j], tl.f[6][j], tl.f[7][j], bytes[j]);
            }
            if ((t & 63) < 16) {  // row group 0 of each wave: the 8 columns' scale bytes of the wave's 32 rows
                const __amdgpu_buffer_rsrc_t rs = rsrc(a.s_col + (r0 / 32 + wave) * a.ld_sc + c0, kTile);
                const uint32_t w0 = bytes[0] | (bytes[1] << 8) | (bytes[2] << 16) | (bytes[3] << 24);
                const uint32_t w1 = bytes[4] | (bytes[5] << 8) | (bytes[6] << 16) | (bytes[7] << 24);
                __builtin_amdgcn_raw_buffer_store_b64(u32x2{w0, w1}, rs, 8 * tc, 0, 0);
            }
            store_transposed(s_tr[parity], codes, tr, tc, a.q_col + c0 * a.ld_qc + r0, a.ld_qc);
        }
    }
}

// 128x128 quantizer.  MODE kQ128Rows writes the codes in place (q, s),
// kQ128Transposed writes each tile transposed (3-D colwise: q, s), kQ128Both
// writes both from one read of x (rows to q, s; transposed to qt, st).
// One 128x128 tile of expert g (tile row rt, column ct) from its values tl:
// the block amax (through wmax, 4 floats of LDS), the scale, and the codes in
// the requested layouts (the transposed ones staged through tr_lds).
template <int MODE>
__device__ __forceinline__ void quant_128_tile(const Quant128Args& a, int64_t g, int64_t rt, int64_t ct,
                                               const TileRegs& tl, float* wmax, uint8_t* tr_lds, int t, int tr,
                                               int tc, int wave) {
    constexpr bool ROWS = MODE != kQ128Transposed;
    constexpr bool TRANSPOSE = MODE != kQ128Rows;
    const int64_t r0 = rt * kTile, c0 = ct * kTile;
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(tl.f[i][j]));
    uint32_t mb = row16_max(__float_as_uint(m));
    mb = max(mb, (uint32_t)__shfl_xor((int)mb, 16));
    mb = max(mb, (uint32_t)__shfl_xor((int)mb, 32));
    if ((t & 63) == 0) wmax[wave] = __uint_as_float(mb);
    __syncthreads();
    const float amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    const Scale sc = block_scale(amax);

    if (ROWS) {
        uint8_t* q = a.q + g * a.stride_qg;
        const __amdgpu_buffer_rsrc_t rq = rsrc(q + r0 * a.ld_q + c0, (kTile - 1) * a.ld_q + kTile);
        const int voff_q = (8 * tr) * (int)a.ld_q + 8 * tc;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint2 c8 = quant8(tl.f[i], sc);
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{c8.x, c8.y}, rq, voff_q, i * (int)a.ld_q, 0);
        }
        if (t == 0) a.s[g * a.stride_sg + ct * a.ld_s + rt] = sc.s;
    }
    if (TRANSPOSE) {
        uint8_t* const qt = MODE == kQ128Both ? a.qt + g * a.stride_qtg : a.q + g * a.stride_qg;
        float* const st = MODE == kQ128Both ? a.st + g * a.stride_stg : a.s + g * a.stride_sg;
        const int64_t ld_qt = MODE == kQ128Both ? a.ld_qt : a.ld_q;
        const int64_t ld_st = MODE == kQ128Both ? a.ld_st : a.ld_s;
        Scale scs[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) scs[j] = sc;
        uint2 codes[8];
        col_codes(tl, scs, codes);
        if (t == 0) st[rt * ld_st + ct] = sc.s;
        store_transposed(tr_lds, codes, tr, tc, qt + c0 * ld_qt + r0, ld_qt);
    }
}

template <int MODE>
__global__ __launch_bounds__(kThreads) void quant_128x128_kernel(Quant128Args a) {
    constexpr bool TRANSPOSE = MODE != kQ128Rows;
    __shared__ float s_wmax[2][4];
    __shared__ __attribute__((aligned(16))) uint8_t s_tr[TRANSPOSE ? 2 : 1][TRANSPOSE ? kTile * kTile : 16];

    const int t = threadIdx.x;
    const int tr = t >> 4, tc = t & 15;
    const int wave = t >> 6;
    const int64_t per_g = a.row_tiles * a.col_tiles;
    const int64_t ntiles = a.G * per_g;

    auto coords = [&](int64_t tl_id, int64_t& g, int64_t& rt, int64_t& ct) {
        g = tl_id / per_g;
        const int64_t rem = tl_id % per_g;
        rt = rem / a.col_tiles;
        ct = rem % a.col_tiles;
    };

    int64_t tile = blockIdx.x;
    if (tile >= ntiles) return;
    const int voff_x = (8 * tr) * (int)(a.ld_x * 2) + 16 * tc;
    int64_t g, rt, ct;
    coords(tile, g, rt, ct);
    Raw raw;
    load_raw(a.x + g * a.stride_xg, a.ld_x, rt * kTile, ct * kTile, a.R, voff_x, raw);

    for (int parity = 0; tile < ntiles; tile += gridDim.x, parity ^= 1) {
        coords(tile, g, rt, ct);
        TileRegs tl;
        unpack_tile(raw, tl);
        const int64_t next = tile + gridDim.x;
        if (next < ntiles) {
            int64_t ng, nrt, nct;
            coords(next, ng, nrt, nct);
            load_raw(a.x + ng * a.stride_xg, a.ld_x, nrt * kTile, nct * kTile, a.R, voff_x, raw);
        }
        quant_128_tile<MODE>(a, g, rt, ct, tl, s_wmax[parity], s_tr[TRANSPOSE ? parity : 0], t, tr, tc, wave);
    }
}

// The forward operands of a linear layer in one launch: workgroups
// [0, tiles_w) take the 128x128 tiles of the weights w (both layouts, as
// quant_128x128_kernel<kQ128Both>), the rest the 128x128 tiles of x, whose
// rows and transposed columns are quantized 1x128 (as quant_1x128_kernel).
// One workgroup per tile (a grid-stride loop covers the rest if the grid is
// capped), so the two passes share one ramp-up and one tail.
__global__ __launch_bounds__(kThreads, 4) void quant_pair_kernel(Quant1x128Args xa, Quant128Args wa) {
    __shared__ float s_colmax[4][kTile];
    __shared__ __attribute__((aligned(16))) uint8_t s_tr[kTile * kTile];

    const int t = threadIdx.x;
    const int tr = t >> 4, tc = t & 15;
    const int wave = t >> 6;
    const int64_t per_g = wa.row_tiles * wa.col_tiles;
    const int64_t tiles_w = wa.G * per_g;
    const int64_t ntiles = tiles_w + ((xa.R + kTile - 1) / kTile) * xa.col_tiles;
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        Raw raw;
        TileRegs tl;
        if (tile < tiles_w) {
            const int64_t g = tile / per_g, rem = tile % per_g;
            const int64_t rt = rem / wa.col_tiles, ct = rem % wa.col_tiles;
            load_raw(wa.x + g * wa.stride_xg, wa.ld_x, rt * kTile, ct * kTile, wa.R,
                     (8 * tr) * (int)(wa.ld_x * 2) + 16 * tc, raw);
            unpack_tile(raw, tl);
            quant_128_tile<kQ128Both>(wa, g, rt, ct, tl, s_colmax[0], s_tr, t, tr, tc, wave);
        } else {
            const int64_t xt = tile - tiles_w;
            const int64_t r0 = (xt / xa.col_tiles) * kTile, c0 = (xt % xa.col_tiles) * kTile;
            const int64_t rows = (xa.R - r0) < kTile ? (xa.R - r0) : kTile;
            load_raw(xa.x, xa.ld_x, r0, c0, xa.R, (8 * tr) * (int)(xa.ld_x * 2) + 16 * tc, raw);
            unpack_tile(raw, tl);
            quant_tile_rows(tl, rows, xa.q_row + r0 * xa.ld_qr + c0, xa.ld_qr,
                            xa.s_row + (c0 / kTile) * xa.ld_sr + r0, tr, tc);
            quant_tile_cols(tl, xa.q_col + c0 * xa.ld_qc + r0, xa.ld_qc, xa.s_col + (r0 / kTile) * xa.ld_sc + c0,
                            s_colmax, s_tr, tr, tc, wave);
        }
        if (tile + gridDim.x < ntiles) __syncthreads();  // LDS reused by the next tile
    }
}

// Persistent grid: as many workgroups as fit on the device at once (per the
// kernel's occupancy), never more than the tiles.  A problem of at least 2
// such grids' worth of tiles launches one workgroup per tile instead (the
// tile loop then runs once and never prefetches): every quantizer runs
// 4-15 % faster that way from there up to the MoE sizes (likely because
// in-order dispatch keeps the tiles in flight within one contiguous window
// of rows, where persistent workgroups drift apart), while a smaller problem
// (the 4096 x 4096 weight pass: 1024 tiles) was 12 % slower and stays
// persistent.
template <typename K>
int64_t persistent_blocks(K kernel, int64_t tiles) {
    const DeviceFit fit = device_fit(reinterpret_cast<const void*>(kernel), kThreads, 2);
    const int64_t cap = (int64_t)fit.cus * fit.per_cu;
    // (capped at 2^23 workgroups, 2^31 threads; the grid-stride loop takes the rest)
    constexpr int64_t kMaxBlocks = (int64_t)1 << 23;
    if (tiles >= 2 * cap) return tiles < kMaxBlocks ? tiles : kMaxBlocks;
    return tiles < cap ? tiles : cap;
}

}  // namespace

template <typename K, typename A>
hipError_t launch_persistent(K kernel, const A& a, int64_t tiles, hipStream_t stream) {
    dim3 grid((unsigned)persistent_blocks(kernel, tiles)), block(kThreads);
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, a);
    return hipGetLastError();
}

// persistent_blocks' choice between the two forms of a kernel: `one` (no
// prefetch) when the grid is one workgroup per tile, `persist` otherwise.
template <typename K1, typename KP, typename A>
hipError_t launch_one_or_persistent(K1 one, KP persist, const A& a, int64_t tiles, hipStream_t stream) {
    const int64_t blocks = persistent_blocks(persist, tiles);
    dim3 block(kThreads);
    if (blocks == tiles) {
        hipLaunchKernelGGL(one, dim3((unsigned)blocks), block, 0, stream, a);
    } else {
        hipLaunchKernelGGL(persist, dim3((unsigned)blocks), block, 0, stream, a);
    }
    return hipGetLastError();
}

hipError_t launch_quant_1x128(const Quant1x128Args& a, bool row, bool col, bool swiglu, hipStream_t stream) {
    const int64_t tiles = ((a.R + kTile - 1) / kTile) * a.col_tiles;
    if (tiles == 0) return hipSuccess;
#define BS_Q1X128(R, C, S) \
    launch_one_or_persistent(quant_1x128_kernel<R, C, S, true>, quant_1x128_kernel<R, C, S, false>, a, tiles, stream)
    if (swiglu) {
        if (row && col) return BS_Q1X128(true, true, true);
        if (row) return BS_Q1X128(true, false, true);
        return BS_Q1X128(false, true, true);
    }
    if (row && col) return BS_Q1X128(true, true, false);
    if (row) return BS_Q1X128(true, false, false);
    return BS_Q1X128(false, true, false);
#undef BS_Q1X128
}

hipError_t launch_swiglu_bwd_quant(const SwigluBwdArgs& a, bool row, bool col, hipStream_t stream) {
    const int64_t tiles = ((a.R + kTile - 1) / kTile) * a.col_tiles;
    if (tiles == 0) return hipSuccess;
    if (row && col) return launch_persistent(swiglu_bwd_quant_kernel<true, true>, a, tiles, stream);
    if (row) return launch_persistent(swiglu_bwd_quant_kernel<true, false>, a, tiles, stream);
    return launch_persistent(swiglu_bwd_quant_kernel<false, true>, a, tiles, stream);
}

hipError_t launch_mx_quant(const MxQuantArgs& a, bool row, bool col, hipStream_t stream) {
    const int64_t tiles = ((a.R + kTile - 1) / kTile) * a.col_tiles;
    if (tiles == 0) return hipSuccess;
    if (row && col) return launch_persistent(mx_quant_kernel<true, true>, a, tiles, stream);
    if (row) return launch_persistent(mx_quant_kernel<true, false>, a, tiles, stream);
    return launch_persistent(mx_quant_kernel<false, true>, a, tiles, stream);
}

hipError_t launch_quant_pair(const Quant1x128Args& xa, const Quant128Args& wa, hipStream_t stream) {
    const int64_t tiles = wa.G * wa.row_tiles * wa.col_tiles + ((xa.R + kTile - 1) / kTile) * xa.col_tiles;
    if (tiles == 0) return hipSuccess;
    constexpr int64_t kMaxBlocks = (int64_t)1 << 23;
    hipLaunchKernelGGL(quant_pair_kernel, dim3((unsigned)(tiles < kMaxBlocks ? tiles : kMaxBlocks)),
                       dim3(kThreads), 0, stream, xa, wa);
    return hipGetLastError();
}

hipError_t launch_quant_128x128(const Quant128Args& a, Quant128Mode mode, hipStream_t stream) {
    const int64_t tiles = a.G * a.row_tiles * a.col_tiles;
    if (tiles == 0) return hipSuccess;
    if (mode == kQ128Both) return launch_persistent(quant_128x128_kernel<kQ128Both>, a, tiles, stream);
    if (mode == kQ128Transposed) return launch_persistent(quant_128x128_kernel<kQ128Transposed>, a, tiles, stream);
    return launch_persistent(quant_128x128_kernel<kQ128Rows>, a, tiles, stream);
}

}  // namespace bs
