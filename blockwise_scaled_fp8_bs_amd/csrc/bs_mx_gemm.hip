// MXFP8 GEMM for gfx950 (OCP Microscaling reading of the pages' MXFP8 recipe):
//
//   D[m, n] = sum_k 2^ea(m, k/32) dec(A[m, k]) * 2^eb(n, k/32) dec(B[n, k])
//
// with one E8M0 exponent byte per 32 consecutive K values of each row of A
// and of B.  v_mfma_scale_f32_16x16x128_f8f6f4 applies those scales itself:
// lane (row r, K chunk c) of each operand supplies the scale byte of its 32
// K values, so one MFMA consumes one 128-wide K block with its four scales
// per row and accumulates into the fp32 tile directly -- no per-block fold on
// the VALU, which bounds the 128-block GEMMs.  Everything else (256x256x128
// tiles, 8 waves as 2 x 4, LDS-DMA double buffering with the swizzle, group
// alternating copy issue, persistent XCD-aware tile order, LDS-staged
// epilogue) is the 128-block GEMM's design; the scale bytes of a K block
// (4 chunks x 256 rows per operand, 1 KiB) ride along with its operands.
//
// (pages: "[mxfp8 moe training] use new 3d colwise quantization kernel",
// summary and microbenchmark table -- the MXFP8 scaled GEMMs; the format
// itself is the OCP MX v1.0 definition, which the pages do not state.)
#include "bs_mx.h"

namespace bs {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int NT = 512;
constexpr int WAVES_N = 4;
constexpr int WM = 128, WN = 64;
constexpr int TM = WM / 16, TN = WN / 16;
constexpr int kGroupRows = 8;  // tile rows per L2 group
constexpr int kChunks = BK / 32;  // MX blocks per K block

struct __attribute__((aligned(16))) MxSmem {
    uint8_t a[2][BM * BK];
    uint8_t b[2][BN * BK];
    uint8_t sa[2][kChunks * BM];  // [chunk][row] E8M0 bytes of the K block
    uint8_t sb[2][kChunks * BN];
};

__device__ __forceinline__ int64_t xcd_remap(int64_t i, int64_t n) {
    // Tile i is taken by a workgroup on XCD i % 8 (workgroups are dispatched
    // round-robin over the XCDs and the persistent stride is a multiple of
    // 8); give XCD x the contiguous logical range [x*q + min(x, r), ...) of
    // n = 8q + r tiles (a bijection).
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

__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// 16-byte-chunk swizzle of a 128-byte LDS row: physical chunk = logical ^ swz(row).
// An MFMA operand read has 16 lanes on 16 consecutive rows at one logical
// chunk; with this swizzle they cover all 64 banks exactly once, and since
// swz depends on row % 16 only, every fragment of a wave uses the same
// lane offsets.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

struct MxOperands {
    i32x4 a, b, sa, sb;
};

// Descriptors of one tile's operands.  Scale reads stay inside the scale
// tensors (rows past the tile's valid rows read other rows' bytes or zero,
// and only feed outputs that are never stored).
__device__ __forceinline__ MxOperands mx_operands(const MxGemmArgs& p, int64_t m0, int64_t n0) {
    const int64_t rows_a = (p.M - m0) < BM ? (p.M - m0) : BM;
    const int64_t rows_b = (p.N - n0) < BN ? (p.N - n0) : BN;
    const int64_t nch = p.K / 32;
    MxOperands o;
    o.a = make_rsrc(p.a + m0 * p.lda, rows_a * p.lda);
    o.b = make_rsrc(p.b + n0 * p.ldb, rows_b * p.ldb);
    o.sa = make_rsrc(p.sa + m0, nch * p.ld_sa - m0);
    o.sb = make_rsrc(p.sb + n0, nch * p.ld_sb - n0);
    return o;
}

template <bool OUT_F32>
__global__ __launch_bounds__(NT) void mx_gemm_kernel(MxGemmArgs p) {
    __shared__ MxSmem sm;

    const int t = threadIdx.x;
    const int lane = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = w / WAVES_N, wn = w % WAVES_N;
    const int lr = lane & 15, lg = lane >> 4;

    const int64_t total = p.num_tiles;
    int64_t idx = blockIdx.x;
    if (idx >= total) return;

    // Operand copies as in the 128-block GEMM: wave w fills LDS rows
    // (8i + w) * 8 of each operand in round i (all waves), or rows
    // (4i + w % 4) * 8 in round i when one group of four waves issues a K
    // block alone.  Scale copies: lane l -> chunk l / 16 of the block, bytes
    // 16 (l % 16) .. of the tile's 256 rows.
    const int ld_lrow = lane >> 3;
    const int ld_lchunk = (lane & 7) ^ swz(w * 8 + ld_lrow);
    const int voff_a = (int)((w * 8 + ld_lrow) * p.lda) + ld_lchunk * 16;
    const int voff_b = (int)((w * 8 + ld_lrow) * p.ldb) + ld_lchunk * 16;
    const int wq = w & 3;
    const int voff_a4 = (int)((wq * 8 + ld_lrow) * p.lda) + ld_lchunk * 16;
    const int voff_b4 = (int)((wq * 8 + ld_lrow) * p.ldb) + ld_lchunk * 16;
    const int voff_sa = (lane >> 4) * (int)p.ld_sa + (lane & 15) * 16;
    const int voff_sb = (lane >> 4) * (int)p.ld_sb + (lane & 15) * 16;

    auto issue_scales = [&](const MxOperands& o, int32_t kb, int s, int first_wave) {
        if (w == first_wave) dma16(o.sa, lds_addr(&sm.sa[s][0]), voff_sa, (int)((int64_t)kb * kChunks * p.ld_sa));
        else if (w == first_wave + 1)
            dma16(o.sb, lds_addr(&sm.sb[s][0]), voff_sb, (int)((int64_t)kb * kChunks * p.ld_sb));
    };
    auto issue_loads = [&](const MxOperands& o, int32_t kb, int s) {
        const int k_off = kb * BK;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            dma16(o.a, lds_addr(&sm.a[s][(8 * i + w) * 1024]), voff_a, k_off + (int)(64 * i * p.lda));
            dma16(o.b, lds_addr(&sm.b[s][(8 * i + w) * 1024]), voff_b, k_off + (int)(64 * i * p.ldb));
        }
        issue_scales(o, kb, s, 0);
    };
    auto issue_loads_group = [&](const MxOperands& o, int32_t kb, int s, int g) {
        if ((w >> 2) != g) return;
        const int k_off = kb * BK;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            dma16(o.a, lds_addr(&sm.a[s][(4 * i + wq) * 1024]), voff_a4, k_off + (int)(32 * i * p.lda));
            dma16(o.b, lds_addr(&sm.b[s][(4 * i + wq) * 1024]), voff_b4, k_off + (int)(32 * i * p.ldb));
        }
        issue_scales(o, kb, s, 4 * g);
    };
    // The MFMA reads a lane's first four registers as K = 16 lg .. 16 lg + 15
    // and its last four as K = 64 + 16 lg .. (measured on gfx950 with one
    // nonzero byte per call), while the scale of lane group c covers K
    // = 32 c .. 32 c + 31: so lane group lg loads logical chunks lg and 4 + lg
    // of the row, and K in the MFMA is K in memory.
    auto frag = [&](const uint8_t* base, int row) -> v8i {
        const int sw = swz(row);
        const uint4 lo = *reinterpret_cast<const uint4*>(base + row * BK + ((lg ^ sw) * 16));
        const uint4 hi = *reinterpret_cast<const uint4*>(base + row * BK + (((lg + 4) ^ sw) * 16));
        v8i r;
        r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
        r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
        return r;
    };
    auto tile_origin = [&](int64_t i, int64_t& m0, int64_t& n0) {
        int64_t tm, tn;
        grouped_order(xcd_remap(i, total), p.tiles_m, p.tiles_n, tm, tn);
        m0 = tm * BM;
        n0 = tn * BN;
    };

    const int32_t nkb = (int32_t)(p.K / BK);
    int64_t m0, n0;
    tile_origin(idx, m0, n0);
    MxOperands ops = mx_operands(p, m0, n0);
    int s = 0;
    if (nkb > 0) issue_loads(ops, 0, 0);
    wait_dma();
    __syncthreads();

    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    for (;;) {
        const int64_t nidx = idx + gridDim.x;
        const bool has_next = nidx < total;
        int64_t nm0 = m0, nn0 = n0;
        MxOperands nops = ops;
        bool next_issued = false;
        auto load_next = [&](int stage) {
            tile_origin(nidx, nm0, nn0);
            nops = mx_operands(p, nm0, nn0);
            if (nkb > 0) issue_loads(nops, 0, stage);
            next_issued = true;
        };

        // lane l holds, for MFMA tile (i, j), row wm*WM + 16i + (l % 16) and
        // columns wn*WN + 16j + 4(l / 16) + r (B rows are the first operand)
        v4f acc[TM][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = zero;

        for (int32_t it = 0; it < nkb; ++it) {
            if (it + 1 < nkb) issue_loads_group(ops, it + 1, s ^ 1, it & 1);
            else if (has_next) load_next(s ^ 1);
            const uint8_t* const la = sm.a[s];
            const uint8_t* const lb = sm.b[s];
            v8i af_next = frag(la, wm * WM + lr);
            v8i bf[TN];
            int scb[TN];  // E8M0 byte of B row wn*WN + 16j + lr, K chunk lg
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                bf[j] = frag(lb, wn * WN + j * 16 + lr);
                scb[j] = sm.sb[s][lg * BN + wn * WN + j * 16 + lr];
            }
            int sca[TM];  // E8M0 byte of A row wm*WM + 16i + lr, K chunk lg
#pragma unroll
            for (int i = 0; i < TM; ++i) sca[i] = sm.sa[s][lg * BM + wm * WM + i * 16 + lr];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const v8i af = af_next;
                if (i + 1 < TM) af_next = frag(la, wm * WM + (i + 1) * 16 + lr);
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], af, acc[i][j], 0, 0, 0,
                                                                                  scb[j], 0, sca[i]);
            }
            wait_dma();
            __syncthreads();
            s ^= 1;
        }

        // ---- epilogue (as in the 128-block GEMM): stage each 16 x 64 block
        // of the wave's tile in the free LDS stage, store whole 16-byte row chunks ----
        {
            constexpr int ESZ = OUT_F32 ? 4 : 2;
            constexpr int PITCH = WN * ESZ + 16;
            constexpr int CPR = WN * ESZ / 16;
            constexpr int RPI = 64 / CPR;
            uint8_t* const stg = (w < 4 ? sm.a[s ^ 1] : sm.b[s ^ 1]) + (w & 3) * 8192;
            char* const dbase = static_cast<char*>(p.d);
            const int rrow = lane / CPR, rch = lane % CPR;
            const int64_t n = n0 + wn * WN + rch * (16 / ESZ);
#pragma unroll
            for (int i = 0; i < TM; ++i) {
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const v4f v = acc[i][j];
                    uint8_t* const dst = stg + lr * PITCH + (j * 16 + 4 * lg) * ESZ;
                    if (OUT_F32) {
                        *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
                    } else {
                        const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[0]) |
                                            ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[1]) << 16);
                        const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[2]) |
                                            ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[3]) << 16);
                        *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
                    }
                }
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
                for (int q = 0; q < 16 / RPI; ++q) {
                    const int row = q * RPI + rrow;
                    const uint4 v = *reinterpret_cast<const uint4*>(stg + row * PITCH + rch * 16);
                    const int64_t m = m0 + wm * WM + i * 16 + row;
                    if (m < p.M && n < p.N)
                        __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v),
                                                    reinterpret_cast<u32x4*>(dbase + (m * p.ldd + n) * ESZ));
                }
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            }
        }

        if (!has_next) break;
        if (!next_issued) load_next(s);
        wait_dma();
        __syncthreads();
        m0 = nm0;
        n0 = nn0;
        ops = nops;
        idx = nidx;
    }
}

// Persistent grid: as many workgroups as fit on the device at once, never
// more than the tiles.
template <typename Kern>
unsigned persistent_grid(Kern kernel, int64_t tiles) {
    int dev = 0, cus = 256, per_cu = 1;
    if (hipGetDevice(&dev) == hipSuccess) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
    }
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, NT, 0) == hipSuccess && occ > 0) per_cu = occ;
    const int64_t cap = (int64_t)cus * per_cu;
    return (unsigned)(tiles < cap ? tiles : cap);
}

template <bool F32>
hipError_t launch_mx_one(const MxGemmArgs& a, hipStream_t stream) {
    const unsigned grid = persistent_grid(mx_gemm_kernel<F32>, a.num_tiles);
    hipLaunchKernelGGL((mx_gemm_kernel<F32>), dim3(grid), dim3(NT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mx_gemm(const MxGemmArgs& args, bool out_f32, hipStream_t stream) {
    MxGemmArgs a = args;
    a.tiles_m = (a.M + BM - 1) / BM;
    a.tiles_n = (a.N + BN - 1) / BN;
    a.num_tiles = a.tiles_m * a.tiles_n;
    if (a.num_tiles <= 0) return hipSuccess;
    return out_f32 ? launch_mx_one<true>(a, stream) : launch_mx_one<false>(a, stream);
}

}  // namespace bs
