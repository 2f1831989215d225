// Blockwise-scaled FP8 GEMM kernels for gfx950 (dense and grouped).
//
//   D[m, n] = sum_kb sa(m, kb) * sb(n, kb) * P_kb[m, n],
//   P_kb[m, n] = sum_{k in block kb} dec(A[m, k]) * dec(B[n, k])
//
// and the MXFP8 form (E8M0 scales per 32 K values of each row of A and B):
//
//   D[m, n] = sum_k 2^ea(m, k/32) dec(A[m, k]) * 2^eb(n, k/32) dec(B[n, k])
//
// (pages: "[not for land] float8 blockwise scaling training prototype using
// deep_gemm", description -- forward/backward GEMMs with 1x128 activation and
// 128x128 weight scales, and the 1x128 x 1x128 grad_weight GEMM; "add FSDP
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
//    16-byte-chunk XOR swizzle so that MFMA operand reads are free of bank
//    conflicts.  The 1x128 A scales (and B scales) of the current K block
//    are staged next to them.
//  * Persistent workgroups (one per CU) walk the tiles; the first K block
//    of the next tile is loaded during the last K block of the current one,
//    and the output tile is staged through LDS so that every store writes
//    whole 128-byte rows while those loads land.  Output stores are
//    non-temporal.
//  * Tile ids are remapped so that each of the 8 XCDs works on a contiguous
//    range of tiles, ordered in groups of 8 tile rows for L2 reuse.
//  * MX (pages: "[mxfp8 moe training] use new 3d colwise quantization
//    kernel", summary and microbenchmark table; the format is the OCP MX
//    v1.0 definition, which the pages do not state): the same kernel with
//    v_mfma_scale applying the E8M0 bytes itself -- each lane supplies the
//    byte of its operand row and of one 32-wide K chunk -- so the MFMA
//    accumulates straight into the fp32 tile and there is no VALU fold.
//    The scale bytes of a K block (4 chunks x 256 rows per operand, 1 KiB)
//    ride along with its operand tiles.
#include "bs_kernels.h"

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
constexpr int kMxPitch = BM + 16;  // MX scale bytes staged per chunk: 256 rows from a 16-byte aligned start

constexpr int kMaxRankedGroups = 256;  // GROUP_K: groups ordered by size up to this count (<= NT)
constexpr int kMaxSlicedGroups = 64;   // GROUP_M: XCD-sliced tile-row order up to this count (8 x 64 <= NT)

// Scales of one operand for one K block: fp32 per row (1x128), the two
// 128x128 block scales of a B tile (f[0], f[1]), or MX bytes [chunk][row]
// with a pitch of 272: a tile of a grouped A may start at any row, and its
// bytes are copied from the 16-byte boundary at or below it.
union ScaleStage {
    float f[BM];
    uint8_t e8[kChunks * kMxPitch];
};
static_assert(BM == BN, "one scale stage layout serves both operands");

struct __attribute__((aligned(16))) Smem {
    uint8_t a[2][BM * BK];
    uint8_t b[2][BN * BK];
    ScaleStage sa[2];
    ScaleStage sb[2];
    int32_t group_by_rank[kMaxRankedGroups];  // GROUP_K: group index of the r-th largest group
    int32_t group_tmp[kMaxRankedGroups];
    // GROUP_M slice order: tile rows before slot k = (slice k / G of group
    // k % G), and each group's first row, end row and tile rows
    int32_t slice_start[8 * kMaxSlicedGroups + 1];
    int32_t g_start[kMaxSlicedGroups], g_end[kMaxSlicedGroups], g_rows[kMaxSlicedGroups];
    int32_t wave_sum[NT / 64];
};

// Read-only views of the GROUP_M slice tables (LDS).
struct SliceTables {
    const int32_t *slice_start, *g_start, *g_end, *g_rows;
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

struct Tile {
    int32_t m0, m_end;   // rows [m0, m_end) of A and D belong to this tile's problem
    int32_t n0;
    int32_t kb0, kb1;    // K blocks [kb0, kb1)
    int32_t g;           // group: whose B (GROUP_M) or which D (GROUP_K)
    int32_t role;        // stream-K: 0 whole tile, 1 later K blocks (partial for the owner), 2 owner
    int32_t sk_last;     // owner: the last workgroup holding a part of this tile
};

// Stream-K work item q of this workgroup (dense problems): first the whole
// tiles q * grid + blockIdx.x of the leading rounds, then the pieces of the
// split tiles that fall into this workgroup's share [i0, i1) of their K
// iterations, in order.  Shares are dealt by a virtual index v that gives the
// workgroups of one XCD consecutive shares (so an XCD works on a few
// neighbouring tiles and shares their operand panels in its L2).  A piece
// that starts a tile's K range is its owner: it adds the partial tiles of
// the later pieces (virtual workgroups v + 1 .. sk_last, each of which has
// that piece as its first) before storing D.
__device__ __forceinline__ int64_t sk_virtual(const GemmArgs& p) {
    return (int64_t)blockIdx.x < p.sk_wgs ? xcd_remap(blockIdx.x, p.sk_wgs) : (int64_t)blockIdx.x;
}

__device__ __forceinline__ bool sk_has_work(const GemmArgs& p, int64_t q) {
    const int64_t P = gridDim.x, w = sk_virtual(p);
    const int64_t dp_rounds = p.sk_dp_tiles / P;
    if (q < dp_rounds) return true;
    if (w >= p.sk_wgs) return false;
    const int64_t nkb = p.K / BK, I = p.sk_tiles * nkb;
    const int64_t i0 = w * I / p.sk_wgs, i1 = (w + 1) * I / p.sk_wgs;
    return (i0 / nkb + (q - dp_rounds)) * nkb < i1;
}

__device__ __forceinline__ bool sk_work(const GemmArgs& p, int64_t q, Tile& t) {
    const int64_t P = gridDim.x, w = sk_virtual(p);
    const int64_t nkb = p.K / BK;
    const int64_t dp_rounds = p.sk_dp_tiles / P;
    int64_t L;
    t.g = 0;
    t.role = 0;
    t.sk_last = 0;
    t.m_end = (int32_t)p.M;
    if (q < dp_rounds) {
        L = xcd_remap(q * P + blockIdx.x, p.sk_dp_tiles);
        t.kb0 = 0;
        t.kb1 = (int32_t)nkb;
    } else {
        if (w >= p.sk_wgs) return false;
        const int64_t I = p.sk_tiles * nkb;
        const int64_t i0 = w * I / p.sk_wgs, i1 = (w + 1) * I / p.sk_wgs;
        const int64_t tt = i0 / nkb + (q - dp_rounds);
        const int64_t s = i0 > tt * nkb ? i0 : tt * nkb;
        const int64_t e = i1 < (tt + 1) * nkb ? i1 : (tt + 1) * nkb;
        if (s >= e) return false;
        L = p.sk_dp_tiles + tt;
        t.kb0 = (int32_t)(s - tt * nkb);
        t.kb1 = (int32_t)(e - tt * nkb);
        if (t.kb0 > 0) {
            t.role = 1;
        } else if (t.kb1 < nkb) {
            t.role = 2;
            t.sk_last = (int32_t)(((tt + 1) * nkb * p.sk_wgs - 1) / I);
        }
    }
    int64_t tm, tn;
    grouped_order(L, p.tiles_m, p.tiles_n, tm, tn);
    t.m0 = (int32_t)(tm * BM);
    t.n0 = (int32_t)(tn * BN);
    return true;
}

// Number of tiles; for GROUP_M also the tile rows summed over the groups
// (group ends clamped to be monotone in [0, M]).
template <int KIND>
__device__ __forceinline__ int64_t tile_total(const GemmArgs& p, int64_t& rows) {
    rows = p.tiles_m;
    if (KIND != kGroupM) return p.num_tiles;
    int64_t prev = 0;
    rows = 0;
    for (int64_t g = 0; g < p.G; ++g) {
        int64_t e = p.group_end[g];
        e = e < prev ? prev : (e > p.M ? p.M : e);
        rows += (e - prev + BM - 1) / BM;
        prev = e;
    }
    return rows * p.tiles_n;
}

template <int KIND>
__device__ __forceinline__ void resolve_tile(const GemmArgs& p, int64_t idx, int64_t total, int64_t rows,
                                             const int32_t* group_by_rank, const SliceTables& st, Tile& t) {
    t.g = 0;
    t.role = 0;
    t.sk_last = 0;
    t.kb0 = 0;
    t.kb1 = (int32_t)(p.K / BK);
    const int64_t L = KIND == kGroupK ? 0 : xcd_remap(idx, total);
    if (KIND == kDense) {
        int64_t tm, tn;
        grouped_order(L, p.tiles_m, p.tiles_n, tm, tn);
        t.m0 = (int32_t)(tm * BM);
        t.m_end = (int32_t)p.M;
        t.n0 = (int32_t)(tn * BN);
    } else if (KIND == kGroupM && p.G <= kMaxSlicedGroups) {
        // slice order: the largest slot k with slice_start[k] <= tr holds
        // tile row tr (empty slots share their successor's start).  LDS
        // reads land in vector registers: readfirstlane keeps the tile
        // (and the buffer descriptors built from it) in scalar registers.
        auto lds = [](const int32_t* a, int i) { return __builtin_amdgcn_readfirstlane(a[i]); };
        int64_t tr, tn;
        grouped_order(L, rows, p.tiles_n, tr, tn);
        int lo = 0, hi = 8 * (int)p.G - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (lds(st.slice_start, mid) <= tr) lo = mid;
            else hi = mid - 1;
        }
        const int x = lo / (int)p.G, g = lo - x * (int)p.G;
        const int64_t row = x * (int64_t)lds(st.g_rows, g) / 8 + (tr - lds(st.slice_start, lo));
        t.m0 = (int32_t)(lds(st.g_start, g) + row * BM);
        t.m_end = lds(st.g_end, g);
        t.n0 = (int32_t)(tn * BN);
        t.g = g;
    } else if (KIND == kGroupM) {
        int64_t tr, tn;
        grouped_order(L, rows, p.tiles_n, tr, tn);
        int64_t before = 0, prev = 0;
        t.m0 = (int32_t)p.M;
        t.m_end = (int32_t)p.M;
        t.n0 = (int32_t)(tn * BN);
        for (int64_t g = 0; g < p.G; ++g) {
            int64_t e = p.group_end[g];
            e = e < prev ? prev : (e > p.M ? p.M : e);
            const int64_t cnt = (e - prev + BM - 1) / BM;
            if (tr < before + cnt) {
                t.m0 = (int32_t)(prev + (tr - before) * BM);
                t.m_end = (int32_t)e;
                t.g = (int32_t)g;
                break;
            }
            before += cnt;
            prev = e;
        }
    } else {  // kGroupK
        // Tiles of a group cost its K blocks, which differ widely between
        // groups.  Logical order: groups by decreasing size (tiles of one
        // group in the L2-grouped order); dealt round by round over the
        // persistent workgroups, each XCD taking 32 consecutive tiles of a
        // round, alternating direction between rounds (a workgroup that got
        // one of a round's larger tiles gets a smaller one next).
        const int64_t per_g = p.tiles_m * p.tiles_n;
        const int64_t nw = gridDim.x, round = idx / nw, slot = idx % nw;
        int64_t Lk = idx;
        if ((round + 1) * nw <= total) {  // full round: permute within it
            int64_t pos = (nw % 8 == 0) ? (slot % 8) * (nw / 8) + slot / 8 : slot;
            if (round & 1) pos = nw - 1 - pos;
            Lk = round * nw + pos;
        }
        const int64_t rank = Lk / per_g;
        const int64_t g = p.G <= kMaxRankedGroups ? group_by_rank[rank] : rank;
        int64_t tm, tn;
        grouped_order(Lk % per_g, p.tiles_m, p.tiles_n, tm, tn);
        int64_t s = 0, e = 0;
        for (int64_t h = 0; h <= g; ++h) {
            s = e;
            int64_t v = p.group_end[h];
            e = v < s ? s : (v > p.K ? p.K : v);
        }
        t.m0 = (int32_t)(tm * BM);
        t.m_end = (int32_t)p.M;
        t.n0 = (int32_t)(tn * BN);
        t.kb0 = (int32_t)(s / BK);
        t.kb1 = (int32_t)(e / BK);
        t.g = (int32_t)g;
    }
    if (t.kb1 < t.kb0) t.kb1 = t.kb0;
}

// Raw buffer resource (gfx9 layout): offsets at or beyond `bytes` read as zero.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, int64_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const int32_t n = bytes > 0x7fffffff ? 0x7fffffff : (bytes < 0 ? 0 : (int32_t)bytes);
    return i32x4{(int32_t)(uint32_t)a, (int32_t)((a >> 32) & 0xffffu), n, 0x00020000};
}

// The four descriptors of one tile's operands.
struct Operands {
    i32x4 a, b, sa, sb;
};

template <int KIND, int SC>
__device__ __forceinline__ Operands make_operands(const GemmArgs& p, const Tile& t) {
    const int64_t rows_a = (t.m_end - t.m0) < BM ? (t.m_end - t.m0) : BM;
    const int64_t rows_b = (p.N - t.n0) < BN ? (p.N - t.n0) : BN;
    const int64_t nkb_all = p.K / BK;
    const uint8_t* const b = KIND == kGroupM ? p.b + t.g * p.stride_bg : p.b;
    Operands o;
    o.a = make_rsrc(p.a + (int64_t)t.m0 * p.lda, rows_a * p.lda);
    o.b = make_rsrc(b + (int64_t)t.n0 * p.ldb, rows_b * p.ldb);
    if (SC == kScaleMx) {
        // bytes of the tile's rows in every chunk row; the last chunk row is
        // read up to the 16-byte boundary at or above column M (N): the range
        // check drops whole dwords, so a limit inside a dword would also drop
        // the valid bytes before it, and an aligned 16-byte block holding a
        // valid byte cannot cross a page.  Reads past the tile's valid rows
        // see other rows' bytes or zero and feed only outputs that are never
        // stored.
        const int64_t nch = p.K / 32;
        const int64_t ma = t.m0 & ~15;  // 16-byte aligned start (ld_sa and the tensor are)
        const uint8_t* const sa = static_cast<const uint8_t*>(p.sa);
        const uint8_t* const sb = static_cast<const uint8_t*>(p.sb) + (KIND == kGroupM ? t.g * p.stride_sbg : 0);
        o.sa = make_rsrc(sa + ma, (nch - 1) * p.ld_sa + ((p.M + 15) & ~15) - ma);
        o.sb = make_rsrc(sb + t.n0, (nch - 1) * p.ld_sb + ((p.N + 15) & ~15) - t.n0);
        return o;
    }
    const float* const sb = static_cast<const float*>(p.sb) + (KIND == kGroupM ? t.g * p.stride_sbg : 0);
    o.sa = make_rsrc(static_cast<const float*>(p.sa) + t.m0, ((nkb_all - 1) * p.ld_sa + (p.M - t.m0)) * 4);
    if (SC == kScale1x128) {
        o.sb = make_rsrc(sb + t.n0, ((nkb_all - 1) * p.ld_sb + (p.N - t.n0)) * 4);
    } else {
        const int64_t nb = t.n0 / BK, nb_count = (p.N + BK - 1) / BK;
        o.sb = make_rsrc(sb + nb, ((nkb_all - 1) * p.ld_sb + nb_count - nb) * 4);
    }
    return o;
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
// An MFMA operand read has 16 lanes on 16 consecutive rows at one logical
// chunk; with this swizzle they cover all 64 banks exactly once, and since
// swz depends on row % 16 only, every fragment of a wave uses the same
// lane offsets.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

template <int KIND, int SC, bool OUT_F32, bool SK = false>
__device__ __forceinline__ void gemm_body(const GemmArgs& p) {
    __shared__ Smem sm;  // one per instantiation; each kernel below uses one
    constexpr bool B1X128 = SC == kScale1x128;
    constexpr bool MX = SC == kScaleMx;
    static_assert(!SK || KIND == kDense, "stream-K splits dense problems only");
    const int t = threadIdx.x;
    const int lane = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = w / WAVES_N, wn = w % WAVES_N;
    const int lr = lane & 15, lg = lane >> 4;

    int64_t rows_total;
    const int64_t total = tile_total<KIND>(p, rows_total);
    int64_t idx = blockIdx.x;  // tile index (stream-K: work item counter q)
    if (SK) {
        Tile t0;
        idx = 0;
        if (!sk_work(p, 0, t0)) return;
    } else if (idx >= total) {
        return;
    }

    if (KIND == kGroupM && p.G <= kMaxSlicedGroups) {
        // Tile-row order for GROUP_M: slice x (of 8) of every group in turn,
        // x-major.  Each XCD walks a contiguous eighth of the order, so the
        // 8 XCDs go through the groups together and read one or two
        // experts' B at a time from the shared last-level cache -- rather
        // than 8 experts' B at once, which does not fit and streams from
        // HBM.  Slot k = x * G + g holds rows [x r_g / 8, (x + 1) r_g / 8)
        // of group g's r_g tile rows.
        const int t0 = threadIdx.x;
        if (t0 < p.G) {
            int64_t s0 = 0, e = 0;
            for (int h = 0; h <= t0; ++h) {
                s0 = e;
                const int64_t v = p.group_end[h];
                e = v < s0 ? s0 : (v > p.M ? p.M : v);
            }
            sm.g_start[t0] = (int32_t)s0;
            sm.g_end[t0] = (int32_t)e;
            sm.g_rows[t0] = (int32_t)((e - s0 + BM - 1) / BM);
        }
        __syncthreads();
        const int nslots = 8 * (int)p.G;
        int32_t v = 0;
        if (t0 < nslots) {
            const int x = t0 / (int)p.G, g = t0 - x * (int)p.G;
            const int64_t r = sm.g_rows[g];
            v = (int32_t)((x + 1) * r / 8 - x * r / 8);
        }
        // block-wide inclusive scan: within each wave, then across waves
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int32_t u = __shfl_up(v, d);
            if (lane >= d) v += u;
        }
        if (lane == 63) sm.wave_sum[w] = v;
        __syncthreads();
        int32_t off = 0;
        for (int i = 0; i < w; ++i) off += sm.wave_sum[i];
        if (t0 < nslots) sm.slice_start[t0 + 1] = v + off;
        if (t0 == 0) sm.slice_start[0] = 0;
        __syncthreads();
    }
    const SliceTables slices{sm.slice_start, sm.g_start, sm.g_end, sm.g_rows};

    if (KIND == kGroupK && p.G <= kMaxRankedGroups) {
        // Rank the groups by size, largest first (ties: lower index first);
        // thread g handles group g.  Sizes come from the clamped cumulative
        // ends e_g = max(e_{g-1}, min(end_g, K)), e_{-1} = 0.
        const int t0 = threadIdx.x;
        if (t0 < p.G) {
            const int64_t v = p.group_end[t0];
            sm.group_tmp[t0] = (int32_t)(v < 0 ? 0 : (v > p.K ? p.K : v));
        }
        __syncthreads();
        int32_t sz = 0;
        if (t0 < p.G) {
            int32_t e = 0, st = 0;
            for (int h = 0; h <= t0; ++h) {
                st = e;
                e = sm.group_tmp[h] > e ? sm.group_tmp[h] : e;
            }
            sz = e - st;
        }
        __syncthreads();
        if (t0 < p.G) sm.group_tmp[t0] = sz;
        __syncthreads();
        if (t0 < p.G) {
            int r = 0;
            for (int h = 0; h < p.G; ++h) {
                const int32_t sh = sm.group_tmp[h];
                r += (sh > sz || (sh == sz && h < t0)) ? 1 : 0;
            }
            sm.group_by_rank[r] = t0;
        }
        __syncthreads();
    }

    // Wave w fills LDS rows [(8i + w) * 8, +8) of each operand in round i
    // (1 KiB: lane l -> physical chunk l % 8 of row l / 8, which holds the
    // logical chunk (l % 8) ^ swz(row); swz sees bits 0..3 of the row, i.e.
    // l / 8 and the parity of w).  Loop-invariant lane offsets; the K block
    // and the round's 64-row step enter through the uniform soffset.
    // Logical chunk c holds the row's 16-byte chunk c of K, except for MX:
    // the MFMA reads a lane's first four registers as K = 16 lg .. 16 lg + 15
    // and its last four as K = 64 + 16 lg .. (measured on gfx950 with one
    // nonzero byte per call), and the scale of lane group c covers
    // K = 32 c .. 32 c + 31, so for MX logical chunk c holds K chunk
    // (c >> 1) + 4 (c & 1): the fragment reads (logical chunks 2 lg, 2 lg + 1)
    // then hand the MFMA K in memory order.  (Reading chunks lg and lg + 4
    // instead costs 3-5 % on every GEMM.)
    const int ld_lrow = lane >> 3;
    const int ld_lchunk = (lane & 7) ^ swz(w * 8 + ld_lrow);
    const int ld_kchunk = MX ? (ld_lchunk >> 1) + 4 * (ld_lchunk & 1) : ld_lchunk;
    const int voff_a = (int)((w * 8 + ld_lrow) * p.lda) + ld_kchunk * 16;
    const int voff_b = (int)((w * 8 + ld_lrow) * p.ldb) + ld_kchunk * 16;
    const int voff_s = B1X128 ? lane * 16 : lane * 4;
    // MX scale copies: 4 chunks x 17 pieces of 16 bytes per operand; piece
    // q of the 68 lands at stage byte 16 q (chunk q / 17 at 272 (q / 17)).
    // Lanes 0..63 copy pieces 0..63, lanes 0..3 of a second copy pieces 64..67.
    const int mx_q0 = lane, mx_q1 = 64 + (lane & 3);
    const int voff_mxa0 = (mx_q0 / 17) * (int)p.ld_sa + (mx_q0 % 17) * 16;
    const int voff_mxa1 = (mx_q1 / 17) * (int)p.ld_sa + (mx_q1 % 17) * 16;
    const int voff_mxb0 = (mx_q0 / 17) * (int)p.ld_sb + (mx_q0 % 17) * 16;
    const int voff_mxb1 = (mx_q1 / 17) * (int)p.ld_sb + (mx_q1 % 17) * 16;

    // The K block's scales, copied by waves w0 (A) and w0 + 1 (B).
    auto issue_scales = [&](const Operands& o, int32_t kb, int s, int w0) {
        if (MX) {
            if (w == w0) {
                const int so = (int)((int64_t)kb * kChunks * p.ld_sa);
                dma16(o.sa, lds_addr(&sm.sa[s].e8[0]), voff_mxa0, so);
                if (lane < 4) dma16(o.sa, lds_addr(&sm.sa[s].e8[1024]), voff_mxa1, so);
            } else if (w == w0 + 1) {
                const int so = (int)((int64_t)kb * kChunks * p.ld_sb);
                dma16(o.sb, lds_addr(&sm.sb[s].e8[0]), voff_mxb0, so);
                if (lane < 4) dma16(o.sb, lds_addr(&sm.sb[s].e8[1024]), voff_mxb1, so);
            }
        } else if (w == w0) {
            dma16(o.sa, lds_addr(&sm.sa[s].f[0]), lane * 16, (int)((int64_t)kb * p.ld_sa * 4));
        } else if (w == w0 + 1) {
            if (B1X128)
                dma16(o.sb, lds_addr(&sm.sb[s].f[0]), voff_s, (int)((int64_t)kb * p.ld_sb * 4));
            else if (lane < 2)
                dma4(o.sb, lds_addr(&sm.sb[s].f[0]), voff_s, (int)((int64_t)kb * p.ld_sb * 4));
        }
    };
    auto issue_loads = [&](const Operands& o, int32_t kb, int s) {
        const int k_off = kb * BK;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            dma16(o.a, lds_addr(&sm.a[s][(8 * i + w) * 1024]), voff_a, k_off + (int)(64 * i * p.lda));
            dma16(o.b, lds_addr(&sm.b[s][(8 * i + w) * 1024]), voff_b, k_off + (int)(64 * i * p.ldb));
        }
        issue_scales(o, kb, s, 0);
    };
    // The same copies issued by the four waves of group g alone (rows
    // [(4i + w % 4) * 8, +8) in round i = 0..7).  Copies stall the issuing
    // wave while the CU's address unit works through them (about 1 KiB per
    // 16 cycles); with one group issuing per K block, the other group's
    // waves go straight to their MFMAs and keep the matrix pipes busy.
    const int wq = w & 3;
    const int voff_a4 = (int)((wq * 8 + ld_lrow) * p.lda) + ld_kchunk * 16;
    const int voff_b4 = (int)((wq * 8 + ld_lrow) * p.ldb) + ld_kchunk * 16;
    auto issue_loads_group = [&](const Operands& o, int32_t kb, int s, int g) {
        if ((w >> 2) != g) return;
        const int k_off = kb * BK;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            dma16(o.a, lds_addr(&sm.a[s][(4 * i + wq) * 1024]), voff_a4, k_off + (int)(32 * i * p.lda));
            dma16(o.b, lds_addr(&sm.b[s][(4 * i + wq) * 1024]), voff_b4, k_off + (int)(32 * i * p.ldb));
        }
        issue_scales(o, kb, s, 4 * g);
    };
    // Piece k of issue_loads_group's copies for wave group g: k < 16 one
    // operand copy (A for even k, B for odd k, round k / 2), k == 16 the scales.
    auto issue_piece = [&](const Operands& o, int32_t kb, int s, int g, int k) {
        const int k_off = kb * BK;
        const int i = k >> 1;
        if (k == 16)
            issue_scales(o, kb, s, 4 * g);
        else if ((k & 1) == 0)
            dma16(o.a, lds_addr(&sm.a[s][(4 * i + wq) * 1024]), voff_a4, k_off + (int)(32 * i * p.lda));
        else
            dma16(o.b, lds_addr(&sm.b[s][(4 * i + wq) * 1024]), voff_b4, k_off + (int)(32 * i * p.ldb));
    };
    // With 128x128 B scales (forward and dgrad) the issuing group spreads
    // its copies over its first 9 MFMAs, two per MFMA, instead of issuing
    // all 17 before them: its waves then join the matrix pipes early, and
    // every copy is still issued in the first quarter of the K block (3-4 %
    // faster on the dense and FFN shapes).  The 1x128 x 1x128 kernel needs
    // its registers for the per-element fold and keeps the block issue; so
    // does the MX kernel (no gain measured).
    constexpr bool kSpread = !MX && !B1X128 && KIND != kGroupK;
    // An MFMA operand fragment: logical chunks 2 lg and 2 lg + 1 of the row
    // (for MX, K chunks lg and lg + 4: see the copies above).
    auto frag = [&](const uint8_t* base, int row) -> v8i {
        const int sw = swz(row);
        const uint4 lo = *reinterpret_cast<const uint4*>(base + row * BK + (((2 * lg) ^ sw) * 16));
        const uint4 hi = *reinterpret_cast<const uint4*>(base + row * BK + (((2 * lg + 1) ^ sw) * 16));
        v8i r;
        r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
        r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
        return r;
    };

    Tile cur;
    if (SK)
        sk_work(p, idx, cur);
    else
        resolve_tile<KIND>(p, idx, total, rows_total, sm.group_by_rank, slices, cur);
    Operands ops = make_operands<KIND, SC>(p, cur);
    int32_t nkb = cur.kb1 - cur.kb0;
    int s = 0;  // LDS stage holding the current K block
    if (nkb > 0) issue_loads(ops, cur.kb0, 0);
    wait_dma();
    __syncthreads();

    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    for (;;) {
        // The next tile of this workgroup: its first K block is loaded
        // during the last K block of this one.
        const int64_t nidx = SK ? idx + 1 : idx + gridDim.x;
        const bool has_next = SK ? sk_has_work(p, nidx) : nidx < total;
        Tile nxt = cur;
        Operands nops = ops;
        bool next_resolved = false;
        auto load_next = [&](int stage) {
            if (SK)
                sk_work(p, nidx, nxt);
            else
                resolve_tile<KIND>(p, nidx, total, rows_total, sm.group_by_rank, slices, nxt);
            nops = make_operands<KIND, SC>(p, nxt);
            if (nxt.kb1 > nxt.kb0) issue_loads(nops, nxt.kb0, stage);
            next_resolved = true;
        };

        // The MFMA computes the transposed tile (B rows as its first operand),
        // so lane l holds, for MFMA tile (i, j), row  wm*WM + 16i + (l % 16)
        // and the four consecutive columns  wn*WN + 16j + 4(l / 16) + r.
        v4f acc[TM][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = zero;

        for (int32_t it = 0; it < nkb; ++it) {
            const bool spread = kSpread && it + 1 < nkb && (w >> 2) == (it & 1);
            if (it + 1 < nkb) {
                if (!kSpread) issue_loads_group(ops, cur.kb0 + it + 1, s ^ 1, it & 1);
            } else if (has_next) {
                load_next(s ^ 1);
            }
            // Operand reads in the order the MFMAs consume them, so that the
            // first MFMA waits for two fragments only; the scales are needed
            // later, by the fmas.
            const uint8_t* const la = sm.a[s];
            const uint8_t* const lb = sm.b[s];
            v8i af_next = frag(la, wm * WM + lr);
            v8i bf[TN];
#pragma unroll
            for (int j = 0; j < TN; ++j) bf[j] = frag(lb, wn * WN + j * 16 + lr);
            if (MX) {
                // E8M0 bytes of the lane's operand rows in K chunk lg (A's
                // tile rows start cur.m0 % 16 bytes into the staged chunk)
                const uint8_t* const ea = &sm.sa[s].e8[lg * kMxPitch + (cur.m0 & 15) + wm * WM + lr];
                const uint8_t* const eb = &sm.sb[s].e8[lg * kMxPitch + wn * WN + lr];
                int scb[TN], sca[TM];
#pragma unroll
                for (int j = 0; j < TN; ++j) scb[j] = eb[j * 16];
#pragma unroll
                for (int i = 0; i < TM; ++i) sca[i] = ea[i * 16];
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    const v8i af = af_next;
                    if (i + 1 < TM) af_next = frag(la, wm * WM + (i + 1) * 16 + lr);
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], af, acc[i][j], 0, 0, 0,
                                                                                      scb[j], 0, sca[i]);
                }
            } else {
                v4f sbv[TN];  // B scale of each of the lane's output columns
                if (B1X128) {
#pragma unroll
                    for (int j = 0; j < TN; ++j) {
                        const float4 t4 = *reinterpret_cast<const float4*>(&sm.sb[s].f[wn * WN + j * 16 + 4 * lg]);
                        sbv[j] = v4f{t4.x, t4.y, t4.z, t4.w};
                    }
                }
                const float sbw = B1X128 ? 0.f : sm.sb[s].f[wn >> 1];
                float sa_i[TM];
#pragma unroll
                for (int i = 0; i < TM; ++i) sa_i[i] = sm.sa[s].f[wm * WM + i * 16 + lr];

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
                    if (i + 1 < TM) af_next = frag(la, wm * WM + (i + 1) * 16 + lr);
#pragma unroll
                    for (int j = 0; j < TN; ++j) {
                        const int q = i * TN + j;
                        pbuf[q & 1] =
                            __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], af, zero, 0, 0, 0, 0, 0, 0);
                        if (kSpread && q <= 8 && spread) {
                            issue_piece(ops, cur.kb0 + it + 1, s ^ 1, it & 1, 2 * q);
                            if (q < 8) issue_piece(ops, cur.kb0 + it + 1, s ^ 1, it & 1, 2 * q + 1);
                        }
                        if (q > 0) fold(pbuf[(q - 1) & 1], pi, pj);
                        pi = i;
                        pj = j;
                    }
                }
                fold(pbuf[(TM * TN - 1) & 1], TM - 1, TN - 1);
            }
            wait_dma();
            __syncthreads();
            s ^= 1;
        }

        // ---- stream-K: a piece after a tile's first K blocks leaves its
        // partial tile (lane-major, as the registers hold it) in this
        // workgroup's slot and raises its flag; the owner adds the partials of
        // virtual workgroups v + 1 .. sk_last, in that order, and clears their
        // flags ----
        bool store_d = true;
        // The slot is addressed through a buffer descriptor: lane offset in one
        // VGPR, the MFMA tile's 1 KiB step as the uniform offset.  Partial
        // tiles are written and read at device scope (cache policy SC1: the
        // stores go through this XCD's L2 to memory, the loads fetch from
        // there), so that no cache-wide write-back or invalidate is needed
        // -- other workgroups on the same XCD keep their cached operands.
        const int sk_voff = (w * TM * TN * 64 + lane) * 16;
        constexpr int kDeviceScope = 16;  // SC1
        const int sk_v = SK ? (int)sk_virtual(p) : 0;
        if (SK && cur.role == 1) {
            const __amdgpu_buffer_rsrc_t slot = __builtin_amdgcn_make_buffer_rsrc(
                p.sk_partial + (int64_t)sk_v * (BM * BN), (short)0, BM * BN * 4, 0x00020000);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[i][j]), slot, sk_voff,
                                                           (i * TN + j) * 1024, kDeviceScope);
            // every store of the partial has reached device scope before the
            // flag is raised
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (t == 0) __hip_atomic_store(&p.sk_flag[sk_v], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            store_d = false;
        } else if (SK && cur.role == 2) {
            bool lost = false;
            for (int c = sk_v + 1; c <= cur.sk_last; ++c) {
                // the flag is raised by a workgroup that has already finished
                // its piece (pieces are its first work after the whole tiles);
                // the bound only guards against a workspace whose flags were
                // not zero on entry
                int n = 0;
                while (__hip_atomic_load(&p.sk_flag[c], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u &&
                       n < (1 << 22)) {
                    __builtin_amdgcn_s_sleep(2);
                    ++n;
                }
                lost = lost || n >= (1 << 22);
                // the loads below are issued after the flag was seen set
                asm volatile("" ::: "memory");
                const __amdgpu_buffer_rsrc_t slot = __builtin_amdgcn_make_buffer_rsrc(
                    p.sk_partial + (int64_t)c * (BM * BN), (short)0, BM * BN * 4, 0x00020000);
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] += __builtin_bit_cast(
                            v4f, __builtin_amdgcn_raw_buffer_load_b128(slot, sk_voff, (i * TN + j) * 1024,
                                                                       kDeviceScope));
            }
            if (lost) {  // never expected: make the tile visibly wrong rather than silently short
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j) acc[i][j] = v4f{NAN, NAN, NAN, NAN};
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();  // every wave has read the partials
            if (t == 0)
                for (int c = sk_v + 1; c <= cur.sk_last; ++c)
                    __hip_atomic_store(&p.sk_flag[c], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }

        // ---- epilogue: stage each 16 x 64 block of the wave's tile in the
        // free LDS stage (s ^ 1: read for the last time before the barrier
        // above), then store whole 16-byte chunks of rows ----
        if (store_d) {
            constexpr int ESZ = OUT_F32 ? 4 : 2;
            constexpr int PITCH = WN * ESZ + 16;     // padded row: 16 lanes of a write hit distinct banks
            constexpr int CPR = WN * ESZ / 16;       // 16-byte chunks per row
            constexpr int RPI = 64 / CPR;            // rows per read / store instruction
            uint8_t* const stg = (w < 4 ? sm.a[s ^ 1] : sm.b[s ^ 1]) + (w & 3) * 8192;
            char* const dbase = static_cast<char*>(p.d) + (KIND == kGroupK ? (int64_t)cur.g * p.stride_dg * ESZ : 0);
            const int rrow = lane / CPR, rch = lane % CPR;
            const int64_t n = (int64_t)cur.n0 + wn * WN + rch * (16 / ESZ);
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
                // the reads below take other lanes' writes: wait for them
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
                for (int q = 0; q < 16 / RPI; ++q) {
                    const int row = q * RPI + rrow;
                    const uint4 v = *reinterpret_cast<const uint4*>(stg + row * PITCH + rch * 16);
                    const int64_t m = (int64_t)cur.m0 + wm * WM + i * 16 + row;
                    // non-temporal: the output is not read again here, and
                    // keeping it out of the caches leaves them to the operand
                    // tiles (and to the inputs of whatever runs next)
                    if (m < cur.m_end && n < p.N)
                        __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v),
                                                    reinterpret_cast<u32x4*>(dbase + (m * p.ldd + n) * ESZ));
                }
                // the next block's writes reuse the staging rows
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            }
        }

        if (!has_next) break;
        if (!next_resolved) load_next(s);  // this tile had no K blocks
        wait_dma();
        __syncthreads();  // staging reads done before stage s ^ 1 is refilled; next tile's block visible
        cur = nxt;
        ops = nops;
        nkb = nxt.kb1 - nxt.kb0;
        idx = nidx;
    }
}

template <int KIND, bool B1X128, bool OUT_F32>
__global__ __launch_bounds__(NT) void gemm_kernel(GemmArgs p) {
    gemm_body<KIND, B1X128 ? kScale1x128 : kScale128x128, OUT_F32>(p);
}

template <int KIND, bool OUT_F32>
__global__ __launch_bounds__(NT) void mx_gemm_kernel(GemmArgs p) {
    gemm_body<KIND, kScaleMx, OUT_F32>(p);
}

template <bool B1X128, bool OUT_F32>
__global__ __launch_bounds__(NT) void gemm_sk_kernel(GemmArgs p) {
    gemm_body<kDense, B1X128 ? kScale1x128 : kScale128x128, OUT_F32, true>(p);
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

template <typename Kern>
hipError_t launch_persistent_gemm(Kern kernel, const GemmArgs& a, hipStream_t stream) {
    const unsigned grid = persistent_grid(kernel, a.num_tiles);
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(NT), 0, stream, a);
    return hipGetLastError();
}

template <int KIND>
hipError_t launch_kind(const GemmArgs& a, ScaleMode scales, bool out_f32, hipStream_t stream) {
    if (a.num_tiles <= 0) return hipSuccess;
    switch (scales) {
        case kScaleMx:
            return out_f32 ? launch_persistent_gemm(mx_gemm_kernel<KIND, true>, a, stream)
                           : launch_persistent_gemm(mx_gemm_kernel<KIND, false>, a, stream);
        case kScale1x128:
            return out_f32 ? launch_persistent_gemm(gemm_kernel<KIND, true, true>, a, stream)
                           : launch_persistent_gemm(gemm_kernel<KIND, true, false>, a, stream);
        default:
            return out_f32 ? launch_persistent_gemm(gemm_kernel<KIND, false, true>, a, stream)
                           : launch_persistent_gemm(gemm_kernel<KIND, false, false>, a, stream);
    }
}

template <typename Kern>
hipError_t launch_grid(Kern kernel, unsigned grid, const GemmArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(NT), 0, stream, a);
    return hipGetLastError();
}

// Smallest K share of a stream-K workgroup, in K blocks.
constexpr int64_t kSkMinBlocks = 4;

template <typename Kern>
StreamK plan_for(Kern kernel, const GemmArgs& a) {
    StreamK sk{0, 0, 0, 0};
    const int64_t tiles = a.tiles_m * a.tiles_n;
    const int64_t P = persistent_grid(kernel, (int64_t)1 << 40);  // every resident workgroup
    const int64_t nkb = a.K / BK;
    sk.grid = tiles < P ? tiles : P;
    if (tiles <= 0 || P <= 1 || nkb < 2 * kSkMinBlocks) return sk;
    const int64_t rest = tiles % P;
    // A last round at least 3/4 full is left as it is: the split costs each
    // of its workgroups a second prologue and epilogue and a partial tile
    // through memory, and with a quarter of the CUs idle the busy ones run
    // at a higher clock (measured: 224 tiles on 256 CUs ran 11 % slower
    // split; 128 tiles over a full round ran 5 % faster).
    if (rest == 0 || 4 * rest > 3 * P) return sk;
    const int64_t iters = rest * nkb;
    int64_t wgs = iters / kSkMinBlocks;
    wgs = wgs < P ? wgs : P;
    if (wgs <= rest) return sk;  // no more workgroups than split tiles: no gain
    sk.grid = P;
    sk.dp_tiles = tiles - rest;
    sk.sk_tiles = rest;
    sk.sk_wgs = wgs;
    return sk;
}

template <bool B1X128>
StreamK plan_kind(const GemmArgs& a, bool out_f32) {
    return out_f32 ? plan_for(gemm_sk_kernel<B1X128, true>, a) : plan_for(gemm_sk_kernel<B1X128, false>, a);
}

constexpr int64_t kSkFlagBytes = 4096;  // flag words, one per workgroup (room for 1024)

}  // namespace

StreamK plan_streamk(const GemmArgs& a, ScaleMode scales, bool out_f32) {
    return scales == kScale1x128 ? plan_kind<true>(a, out_f32) : plan_kind<false>(a, out_f32);
}

int64_t streamk_workspace_bytes(const StreamK& sk) {
    if (sk.sk_tiles == 0) return 0;
    return kSkFlagBytes + sk.sk_wgs * (int64_t)(BM * BN) * 4;
}

hipError_t launch_gemm_streamk(const GemmArgs& a, ScaleMode scales, bool out_f32, void* workspace,
                               int64_t workspace_bytes, hipStream_t stream) {
    const StreamK sk = plan_streamk(a, scales, out_f32);
    const int64_t need = streamk_workspace_bytes(sk);
    if (sk.sk_tiles == 0 || sk.sk_wgs * 4 > kSkFlagBytes || workspace == nullptr || workspace_bytes < need)
        return launch_gemm(a, kDense, scales, out_f32, stream);
    GemmArgs g = a;
    g.sk_dp_tiles = sk.dp_tiles;
    g.sk_tiles = sk.sk_tiles;
    g.sk_wgs = sk.sk_wgs;
    g.sk_flag = static_cast<uint32_t*>(workspace);
    g.sk_partial = reinterpret_cast<float*>(static_cast<char*>(workspace) + kSkFlagBytes);
    const unsigned grid = (unsigned)sk.grid;
    if (scales == kScale1x128)
        return out_f32 ? launch_grid(gemm_sk_kernel<true, true>, grid, g, stream)
                       : launch_grid(gemm_sk_kernel<true, false>, grid, g, stream);
    return out_f32 ? launch_grid(gemm_sk_kernel<false, true>, grid, g, stream)
                   : launch_grid(gemm_sk_kernel<false, false>, grid, g, stream);
}

namespace {
__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0u;
}
}  // namespace

hipError_t launch_zero_words(uint32_t* p, int64_t n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256), 0, stream, p,
                       n);
    return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& a, GroupKind kind, ScaleMode scales, bool out_f32, hipStream_t stream) {
    switch (kind) {
        case kDense: return launch_kind<kDense>(a, scales, out_f32, stream);
        case kGroupM: return launch_kind<kGroupM>(a, scales, out_f32, stream);
        default: return launch_kind<kGroupK>(a, scales, out_f32, stream);
    }
}

}  // namespace bs
