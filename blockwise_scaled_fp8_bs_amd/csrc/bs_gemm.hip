// Blockwise-scaled FP8 GEMM kernels for gfx950 (dense and grouped).
//
//   D[m, n] = sum_kb sa(m, kb) * sb(n, kb) * P_kb[m, n],
//   P_kb[m, n] = sum_{k in block kb} dec(A[m, k]) * dec(B[n, k])
//
// (pages: "[not for land] float8 blockwise scaling training prototype using
// deep_gemm", description -- forward/backward GEMMs with 1x128 activation and
// 128x128 weight scales, and the "1x128 by 1x128" grad_weight GEMM; "add FSDP
// and TP tests for Float8BlockwiseLinear", review threads -- both operands
// contiguous along the contraction, fp32 K-major scales.)
//
// Design for CDNA4:
//  * v_mfma_f32_16x16x128_f8f6f4 contracts exactly one 128-wide scale block
//    per instruction, so every MFMA result is a complete partial P_kb of a
//    16x16 tile; it is folded into the fp32 accumulator with one VALU fma
//    per element (acc += P_kb * sa * sb) while later MFMAs run.
//  * Workgroup tile 256 x 256 x 128, 8 wave64s as 2 (M) x 4 (N), wave tile
//    128 x 64 = 8 x 4 MFMA tiles, 128 fp32 accumulators per lane.
//  * Operand tiles are staged in LDS, double buffered (2 x 64 KiB), with a
//    16-byte-chunk XOR swizzle (chunk ^ (row & 7)) so that the 16 lanes of
//    an MFMA operand read hit distinct banks.  The 1x128 A scales (and B
//    scales) of the current K block are staged next to them.
//  * Workgroup ids are remapped so that each of the 8 XCDs works on a
//    contiguous range of tiles, ordered in groups of 8 tile rows for L2 reuse.
#include "bs_kernels.h"

namespace bs {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int NT = 512;
constexpr int WAVES_N = 4;
constexpr int WM = 128, WN = 64;
constexpr int TM = WM / 16, TN = WN / 16;
constexpr int kGroupRows = 8;  // tile rows per L2 group

struct __attribute__((aligned(16))) Smem {
    uint8_t a[2][BM * BK];
    uint8_t b[2][BN * BK];
    float sa[2][BM];
    float sb[2][BN];
};

__device__ __forceinline__ int64_t xcd_remap(int64_t i, int64_t n) {
    // Workgroup i is dispatched to XCD i % 8; give XCD x the contiguous
    // logical range [x*q + min(x, r), ...) of n = 8q + r tiles (a bijection).
    const int64_t q = n / 8, r = n % 8;
    const int64_t x = i % 8, j = i / 8;
    return x * q + (x < r ? x : r) + j;
}

__device__ __forceinline__ void grouped_order(int64_t L, int64_t tiles_m, int64_t tiles_n, int64_t& tm,
                                              int64_t& tn) {
    const int64_t per_group = kGroupRows * tiles_n;
    const int64_t first = (L / per_group) * kGroupRows;
    const int64_t gm = (tiles_m - first) < kGroupRows ? (tiles_m - first) : kGroupRows;
    const int64_t r = L % per_group;
    tm = first + r % gm;
    tn = r / gm;
}

struct Tile {
    int64_t m0, m_end;   // rows [m0, m_end) of A and D belong to this tile's problem
    int64_t n0;
    int64_t kb0, kb1;    // K blocks [kb0, kb1)
    int64_t g;           // group (GROUP_K: which D to write)
    const uint8_t* b;
    const float* sb;
};

template <int KIND>
__device__ __forceinline__ bool resolve_tile(const GemmArgs& p, Tile& t) {
    t.b = p.b;
    t.sb = p.sb;
    t.g = 0;
    t.kb0 = 0;
    t.kb1 = p.K / BK;
    if (KIND == kDense) {
        const int64_t L = xcd_remap(blockIdx.x, p.num_tiles);
        int64_t tm, tn;
        grouped_order(L, p.tiles_m, p.tiles_n, tm, tn);
        t.m0 = tm * BM;
        t.m_end = p.M;
        t.n0 = tn * BN;
        return true;
    } else if (KIND == kGroupM) {
        // count tile rows over the groups (ends clamped to be monotone in [0, M])
        int64_t rows = 0, prev = 0;
        for (int64_t g = 0; g < p.G; ++g) {
            int64_t e = p.group_end[g];
            e = e < prev ? prev : (e > p.M ? p.M : e);
            rows += (e - prev + BM - 1) / BM;
            prev = e;
        }
        const int64_t total = rows * p.tiles_n;
        if ((int64_t)blockIdx.x >= total) return false;
        const int64_t L = xcd_remap(blockIdx.x, total);
        int64_t tr, tn;
        grouped_order(L, rows, p.tiles_n, tr, tn);
        int64_t before = 0;
        prev = 0;
        for (int64_t g = 0; g < p.G; ++g) {
            int64_t e = p.group_end[g];
            e = e < prev ? prev : (e > p.M ? p.M : e);
            const int64_t cnt = (e - prev + BM - 1) / BM;
            if (tr < before + cnt) {
                t.m0 = prev + (tr - before) * BM;
                t.m_end = e;
                t.n0 = tn * BN;
                t.b = p.b + g * p.stride_bg;
                t.sb = p.sb + g * p.stride_sbg;
                return true;
            }
            before += cnt;
            prev = e;
        }
        return false;
    } else {  // kGroupK
        const int64_t per_g = p.tiles_m * p.tiles_n;
        const int64_t L = xcd_remap(blockIdx.x, p.num_tiles);
        const int64_t g = L / per_g;
        int64_t tm, tn;
        grouped_order(L % per_g, p.tiles_m, p.tiles_n, tm, tn);
        int64_t s = 0, e = 0;
        for (int64_t h = 0; h <= g; ++h) {
            s = e;
            int64_t v = p.group_end[h];
            e = v < s ? s : (v > p.K ? p.K : v);
        }
        t.m0 = tm * BM;
        t.m_end = p.M;
        t.n0 = tn * BN;
        t.kb0 = s / BK;
        t.kb1 = e / BK;
        t.g = g;
        return true;
    }
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource (gfx9 layout): offsets at or beyond `bytes` read as zero.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, int64_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const int32_t n = bytes > 0x7fffffff ? 0x7fffffff : (bytes < 0 ? 0 : (int32_t)bytes);
    return i32x4{(int32_t)(uint32_t)a, (int32_t)((a >> 32) & 0xffffu), n, 0x00020000};
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(size_t)(__attribute__((address_space(3))) const char*)p;
}

// Global -> LDS copies (buffer_load ... lds): lane i's bytes land at
// lds_base + i * size.  Issued through inline asm so that the compiler does
// not wait for them before every LDS read of the other stage (it cannot tell
// the two stages apart); the kernel waits for them explicitly (vmcnt(0))
// before the barrier that publishes the stage.
// Byte address = buffer base + voffset (per lane) + soffset (uniform).
__device__ __forceinline__ void dma16(i32x4 rs, uint32_t lds_base, int voffset, int soffset) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voffset), "s"(rs),
                    "s"(__builtin_amdgcn_readfirstlane(soffset)) : "memory");
}

__device__ __forceinline__ void dma4(i32x4 rs, uint32_t lds_base, int voffset, int soffset) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                 :: "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voffset), "s"(rs),
                    "s"(__builtin_amdgcn_readfirstlane(soffset)) : "memory");
}

__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// 16-byte-chunk swizzle of a 128-byte LDS row: physical chunk = logical ^ swz(row).
// The 8 lanes of each 128-byte group of an MFMA operand read sit on 8
// consecutive rows at one logical chunk and land on 8 distinct chunks.
// (On gfx950's 64-bank LDS, (row ^ row >> 3) & 7 also removes the remaining
// two-way conflicts between 16-lane groups, but measured no faster here.)
__device__ __forceinline__ int swz(int row) { return row & 7; }

template <int KIND, bool B1X128, bool OUT_F32>
__global__ __launch_bounds__(NT) void gemm_kernel(GemmArgs p) {
    __shared__ Smem sm;

    Tile tile;
    if (!resolve_tile<KIND>(p, tile)) return;
    char* const dbase = static_cast<char*>(p.d) + tile.g * p.stride_dg * (OUT_F32 ? 4 : 2);

    const int t = threadIdx.x;
    const int lane = t & 63, w = t >> 6;
    const int wm = w / WAVES_N, wn = w % WAVES_N;
    const int lr = lane & 15, lg = lane >> 4;

    // ---- buffer descriptors: rows past the tile's problem read as zero ----
    const int64_t rows_a = (tile.m_end - tile.m0) < BM ? (tile.m_end - tile.m0) : BM;
    const int64_t rows_b = (p.N - tile.n0) < BN ? (p.N - tile.n0) : BN;
    const int64_t nkb_all = p.K / BK;
    const i32x4 rs_a = make_rsrc(p.a + tile.m0 * p.lda, rows_a * p.lda);
    const i32x4 rs_b = make_rsrc(tile.b + tile.n0 * p.ldb, rows_b * p.ldb);
    const i32x4 rs_sa = make_rsrc(p.sa + tile.m0, ((nkb_all - 1) * p.ld_sa + (p.M - tile.m0)) * 4);
    const int64_t nb_count = (p.N + BK - 1) / BK;
    const i32x4 rs_sb =
        B1X128 ? make_rsrc(tile.sb + tile.n0, ((nkb_all - 1) * p.ld_sb + (p.N - tile.n0)) * 4)
               : make_rsrc(tile.sb, ((nkb_all - 1) * p.ld_sb + nb_count) * 4);

    // Wave w fills LDS rows [(8i + w) * 8, +8) of each operand in round i
    // (1 KiB: lane l -> physical chunk l % 8 of row l / 8, which holds the
    // logical chunk (l % 8) ^ swz(row); swz sees bits 0..3 of the row, i.e.
    // l / 8 and the parity of w).
    const int ld_lrow = lane >> 3;
    const int ld_lchunk = (lane & 7) ^ swz(w * 8 + ld_lrow);
    const int sb_nb = (int)(tile.n0 / BK);

    // Loop-invariant lane offsets; the K block and the round's 64-row step
    // enter through the uniform soffset.
    const int voff_a = (int)((w * 8 + ld_lrow) * p.lda) + ld_lchunk * 16;
    const int voff_b = (int)((w * 8 + ld_lrow) * p.ldb) + ld_lchunk * 16;
    const int voff_s = B1X128 ? lane * 16 : (sb_nb + lane) * 4;

    auto issue_loads = [&](int64_t kb, int s) {
        const int k_off = (int)(kb * BK);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            dma16(rs_a, lds_addr(&sm.a[s][(8 * i + w) * 1024]), voff_a, k_off + (int)(64 * i * p.lda));
            dma16(rs_b, lds_addr(&sm.b[s][(8 * i + w) * 1024]), voff_b, k_off + (int)(64 * i * p.ldb));
        }
        if (w == 0) {
            dma16(rs_sa, lds_addr(&sm.sa[s][0]), lane * 16, (int)(kb * p.ld_sa * 4));
        } else if (w == 1) {
            if (B1X128)
                dma16(rs_sb, lds_addr(&sm.sb[s][0]), voff_s, (int)(kb * p.ld_sb * 4));
            else if (lane < 2)
                dma4(rs_sb, lds_addr(&sm.sb[s][0]), voff_s, (int)(kb * p.ld_sb * 4));
        }
    };
    auto frag = [&](const uint8_t* base, int row) -> v8i {
        const int sw = swz(row);
        const uint4 lo = *reinterpret_cast<const uint4*>(base + row * BK + (((2 * lg) ^ sw) * 16));
        const uint4 hi = *reinterpret_cast<const uint4*>(base + row * BK + (((2 * lg + 1) ^ sw) * 16));
        v8i r;
        r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
        r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
        return r;
    };

    // The MFMA computes the transposed tile (B rows as its first operand), so
    // lane l holds, for MFMA tile (i, j), row  wm*WM + 16i + (l % 16)  and the
    // four consecutive columns  wn*WN + 16j + 4(l / 16) + r,  r = 0..3.
    v4f acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    const int64_t nkb = tile.kb1 > tile.kb0 ? tile.kb1 - tile.kb0 : 0;
    if (nkb > 0) issue_loads(tile.kb0, 0);
    wait_dma();
    __syncthreads();

    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    // One K block on LDS stage s (a compile-time constant at both call sites).
    auto step = [&](int64_t it, const int s) {
        if (it + 1 < nkb) issue_loads(tile.kb0 + it + 1, s ^ 1);
        // Operand reads in the order the MFMAs consume them, so that the
        // first MFMA waits for two fragments only (every wave reads right
        // after the barrier); the scales are needed later, by the fmas.
        v8i af_next = frag(sm.a[s], wm * WM + lr);
        v8i bf[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) bf[j] = frag(sm.b[s], wn * WN + j * 16 + lr);
        v4f sbv[TN];  // B scale of each of the lane's output columns
        if (B1X128) {
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const float4 t4 = *reinterpret_cast<const float4*>(&sm.sb[s][wn * WN + j * 16 + 4 * lg]);
                sbv[j] = v4f{t4.x, t4.y, t4.z, t4.w};
            }
        }
        const float sbw = B1X128 ? 0.f : sm.sb[s][wn >> 1];
        float sa_i[TM];
#pragma unroll
        for (int i = 0; i < TM; ++i) sa_i[i] = sm.sa[s][wm * WM + i * 16 + lr];

        // Software pipeline at MFMA granularity: the scale fmas of tile
        // (i, j) run while the MFMA of the next tile executes.
        v4f pbuf[2];
        int pi = 0, pj = 0;
        auto fold = [&](const v4f& pk, int i, int j) {
            if (B1X128) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[i][j][r] = __builtin_fmaf(pk[r], sa_i[i] * sbv[j][r], acc[i][j][r]);
            } else {
                const float sc = sa_i[i] * sbw;
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(pk[r], sc, acc[i][j][r]);
            }
        };
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const v8i af = af_next;
            if (i + 1 < TM) af_next = frag(sm.a[s], wm * WM + (i + 1) * 16 + lr);
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int t = i * TN + j;
                pbuf[t & 1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], af, zero, 0, 0, 0, 0, 0, 0);
                if (t > 0) fold(pbuf[(t - 1) & 1], pi, pj);
                pi = i;
                pj = j;
            }
        }
        fold(pbuf[(TM * TN - 1) & 1], TM - 1, TN - 1);
        wait_dma();
        __syncthreads();
    };
    for (int64_t it = 0; it < nkb; ++it) step(it, (int)(it & 1));

    // ---- epilogue: four consecutive columns per lane and tile ----
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int64_t m = tile.m0 + wm * WM + i * 16 + lr;
        if (m >= tile.m_end) continue;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int64_t n = tile.n0 + wn * WN + j * 16 + 4 * lg;
            if (n >= p.N) continue;
            const v4f v = acc[i][j];
            if (OUT_F32) {
                *reinterpret_cast<float4*>(reinterpret_cast<float*>(dbase) + m * p.ldd + n) =
                    make_float4(v[0], v[1], v[2], v[3]);
            } else {
                const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[0]) |
                                    ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[1]) << 16);
                const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[2]) |
                                    ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[3]) << 16);
                *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(dbase) + m * p.ldd + n) = make_uint2(lo, hi);
            }
        }
    }
}

template <int KIND>
hipError_t launch_kind(const GemmArgs& a, bool b_1x128, bool out_f32, hipStream_t stream) {
    if (a.num_tiles <= 0) return hipSuccess;
    if (a.num_tiles > 0x7fffffff) return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)a.num_tiles), block(NT);
    if (b_1x128) {
        if (out_f32) hipLaunchKernelGGL((gemm_kernel<KIND, true, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((gemm_kernel<KIND, true, false>), grid, block, 0, stream, a);
    } else {
        if (out_f32) hipLaunchKernelGGL((gemm_kernel<KIND, false, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((gemm_kernel<KIND, false, false>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& a, GroupKind kind, bool b_1x128, bool out_f32, hipStream_t stream) {
    switch (kind) {
        case kDense: return launch_kind<kDense>(a, b_1x128, out_f32, stream);
        case kGroupM: return launch_kind<kGroupM>(a, b_1x128, out_f32, stream);
        default: return launch_kind<kGroupK>(a, b_1x128, out_f32, stream);
    }
}

}  // namespace bs
