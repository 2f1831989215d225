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

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ lds_void* to_lds(void* p) {
    return (lds_void*)(__attribute__((address_space(3))) char*)p;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    // Raw buffer: offsets at or beyond `bytes` read as zero.
    const int32_t n = bytes > 0x7fffffff ? 0x7fffffff : (bytes < 0 ? 0 : (int32_t)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

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
    const __amdgpu_buffer_rsrc_t rs_a = make_rsrc(p.a + tile.m0 * p.lda, rows_a * p.lda);
    const __amdgpu_buffer_rsrc_t rs_b = make_rsrc(tile.b + tile.n0 * p.ldb, rows_b * p.ldb);
    const __amdgpu_buffer_rsrc_t rs_sa =
        make_rsrc(p.sa + tile.m0, ((nkb_all - 1) * p.ld_sa + (p.M - tile.m0)) * 4);
    const int64_t nb_count = (p.N + BK - 1) / BK;
    const __amdgpu_buffer_rsrc_t rs_sb =
        B1X128 ? make_rsrc(tile.sb + tile.n0, ((nkb_all - 1) * p.ld_sb + (p.N - tile.n0)) * 4)
               : make_rsrc(tile.sb, ((nkb_all - 1) * p.ld_sb + nb_count) * 4);

    // Wave w fills LDS rows [(8i + w) * 8, +8) of each operand in round i
    // (1 KiB: lane l -> physical chunk l % 8 of row l / 8, which holds the
    // logical chunk (l % 8) ^ (l / 8) under the row-XOR swizzle).
    const int ld_lrow = lane >> 3;
    const int ld_lchunk = (lane & 7) ^ ld_lrow;
    const int sb_nb = (int)(tile.n0 / BK);

    auto issue_loads = [&](int64_t kb, int s) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = (8 * i + w) * 8 + ld_lrow;
            const int off_a = (int)(row * p.lda + kb * BK) + ld_lchunk * 16;
            const int off_b = (int)(row * p.ldb + kb * BK) + ld_lchunk * 16;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_a, to_lds(&sm.a[s][(8 * i + w) * 1024]), 16, off_a, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_b, to_lds(&sm.b[s][(8 * i + w) * 1024]), 16, off_b, 0, 0, 0);
        }
        if (w == 0) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_sa, to_lds(&sm.sa[s][0]), 16,
                                                     (int)(kb * p.ld_sa * 4) + lane * 16, 0, 0, 0);
        } else if (w == 1) {
            if (B1X128) {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_sb, to_lds(&sm.sb[s][0]), 16,
                                                         (int)(kb * p.ld_sb * 4) + lane * 16, 0, 0, 0);
            } else if (lane < 2) {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_sb, to_lds(&sm.sb[s][0]), 4,
                                                         (int)((kb * p.ld_sb + sb_nb) * 4) + lane * 4, 0, 0, 0);
            }
        }
    };
    auto frag = [&](const uint8_t* base, int row) -> v8i {
        const int sw = row & 7;
        const uint4 lo = *reinterpret_cast<const uint4*>(base + row * BK + (((2 * lg) ^ sw) * 16));
        const uint4 hi = *reinterpret_cast<const uint4*>(base + row * BK + (((2 * lg + 1) ^ sw) * 16));
        v8i r;
        r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
        r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
        return r;
    };

    v4f acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    const int64_t nkb = tile.kb1 > tile.kb0 ? tile.kb1 - tile.kb0 : 0;
    if (nkb > 0) issue_loads(tile.kb0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    for (int64_t it = 0; it < nkb; ++it) {
        const int s = (int)(it & 1);
        if (it + 1 < nkb) issue_loads(tile.kb0 + it + 1, s ^ 1);

        v8i bf[TN];
        float sbj[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int nrow = wn * WN + j * 16 + lr;
            bf[j] = frag(sm.b[s], nrow);
            sbj[j] = B1X128 ? sm.sb[s][nrow] : sm.sb[s][wn >> 1];
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const v8i af = frag(sm.a[s], wm * WM + i * 16 + lr);
            const float4 sa4 = *reinterpret_cast<const float4*>(&sm.sa[s][wm * WM + i * 16 + 4 * lg]);
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const v4f pk = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[j], zero, 0, 0, 0, 0,
                                                                                  0, 0);
                acc[i][j][0] = __builtin_fmaf(pk[0], sa4.x * sbj[j], acc[i][j][0]);
                acc[i][j][1] = __builtin_fmaf(pk[1], sa4.y * sbj[j], acc[i][j][1]);
                acc[i][j][2] = __builtin_fmaf(pk[2], sa4.z * sbj[j], acc[i][j][2]);
                acc[i][j][3] = __builtin_fmaf(pk[3], sa4.w * sbj[j], acc[i][j][3]);
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }

    // ---- epilogue: D[m, n] for m < m_end, n < N ----
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int64_t n = tile.n0 + wn * WN + j * 16 + lr;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t m = tile.m0 + wm * WM + i * 16 + 4 * lg + r;
                if (m < tile.m_end && n < p.N) {
                    if (OUT_F32) {
                        reinterpret_cast<float*>(dbase)[m * p.ldd + n] = acc[i][j][r];
                    } else {
                        const __bf16 h = (__bf16)acc[i][j][r];
                        reinterpret_cast<uint16_t*>(dbase)[m * p.ldd + n] = __builtin_bit_cast(uint16_t, h);
                    }
                }
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
