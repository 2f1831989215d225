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
#include "bs_device.h"
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
// Tile rows per L2 group (tiles are walked down the group's rows first).
// Dense and GROUP_M: 4.  An XCD's rows of a small expert can be a slice of
// 0-3 tile rows, so an 8-row group often spans three experts and its 32
// concurrent tiles need the B panels of all three; with 4 rows, over the
// random group sizes of the 128000-token MoE layer, the forward fetched 15.1
// instead of 18.5 GB and ran 1-3 % faster, the dgrad 7 % faster (equal
// groups: both unchanged within 1 %).  On the dense layers 4 rows are 2-7 %
// faster than 8 for the forward and dgrad (16384x5120x8192 forward 7 %,
// 16384x7168x2048 forward 1 % slower), 2 rows mixed, 16 no better.
// GROUP_K and stream-K: 8 (GROUP_K with 4: same time, with 2: 3 % slower).
constexpr int kGroupRows = 4;
constexpr int kGroupRowsK = 8;
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
    // quantizing epilogue: each wave's half-row amaxes [wm][wn][i][lane % 16]
    float row_amax[2][WAVES_N][TM][16];
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

template <int ROWS = kGroupRows>
__device__ __forceinline__ void grouped_order(int64_t L, int64_t tiles_m, int64_t tiles_n, int64_t& tm,
                                              int64_t& tn) {
    const int64_t per_group = ROWS * tiles_n;
    const int64_t first = (L / per_group) * ROWS;
    const int64_t gm = (tiles_m - first) < ROWS ? (tiles_m - first) : ROWS;
    const int64_t r = L % per_group;
    tm = first + r % gm;
    tn = r / gm;
}

struct Tile {
    int32_t m0, m_end;   // rows [m0, m_end) of A and D belong to this tile's problem
    int32_t n0;
    int32_t kb0, kb1;    // K blocks [kb0, kb1)
    int32_t g;           // group: whose B (GROUP_M) or which D (GROUP_K)
    int32_t role;        // stream-K: 0 whole tile, 1 a piece (its partial goes to the workspace)
    int32_t sk_last;     // stream-K piece: its workspace slot
};

// Stream-K split of a dense problem.  The K iterations of the split tiles
// (the ragged last round) are divided evenly over sk_wgs workgroups, whose
// shares are dealt by a virtual index v that gives the workgroups of one XCD
// consecutive shares (an XCD then works on a few neighbouring tiles and
// shares their operand panels in its L2).  Work item q of a workgroup: first
// the whole tiles q * grid + blockIdx.x of the leading rounds, then the
// pieces of its share, one per split tile it touches, in order.  Every piece
// leaves its fp32 partial tile in slot v + t of the workspace (tile t, share
// v: the pairs (t, v) of all pieces form a staircase, so v + t is unique);
// a second kernel adds each tile's partials in share order and writes D.
struct SkPlan {
    int32_t v;          // virtual workgroup index (share order)
    int32_t dp_rounds;  // rounds of whole tiles
    int32_t nkb;        // K blocks per tile
    int32_t t0;         // first split tile of this share
    int32_t i0, i1;     // this share of the split tiles' K iterations (i1 <= i0: none)
};

// Wave-uniform values in scalar registers.
__device__ __forceinline__ int32_t uni(int64_t x) { return __builtin_amdgcn_readfirstlane((int32_t)x); }

__device__ __forceinline__ SkPlan sk_plan(const GemmArgs& p) {
    SkPlan s;
    const int64_t P = gridDim.x, b = blockIdx.x;
    s.v = uni(b < p.sk_wgs ? xcd_remap(b, p.sk_wgs) : b);
    s.dp_rounds = uni(p.sk_dp_tiles / P);
    s.nkb = uni(p.K / BK);
    const int64_t I = p.sk_tiles * (int64_t)s.nkb;
    if (s.v < p.sk_wgs) {
        s.i0 = uni(s.v * I / p.sk_wgs);
        s.i1 = uni((s.v + 1) * I / p.sk_wgs);
    } else {
        s.i0 = s.i1 = 0;
    }
    s.t0 = uni(s.i0 / s.nkb);
    return s;
}

__device__ __forceinline__ bool sk_has_work(const SkPlan& s, int64_t q) {
    if (q < s.dp_rounds) return true;
    return (s.t0 + (q - s.dp_rounds)) * (int64_t)s.nkb < s.i1;
}

__device__ __forceinline__ void sk_work(const GemmArgs& p, const SkPlan& s, int64_t q, Tile& t) {
    int64_t L;
    t.g = 0;
    t.role = 0;
    t.sk_last = 0;
    t.m_end = (int32_t)p.M;
    if (q < s.dp_rounds) {
        L = xcd_remap(q * gridDim.x + blockIdx.x, p.sk_dp_tiles);
        t.kb0 = 0;
        t.kb1 = s.nkb;
    } else {
        const int32_t tt = s.t0 + (int32_t)(q - s.dp_rounds);
        const int32_t lo = tt * s.nkb, hi = lo + s.nkb;
        L = p.sk_dp_tiles + tt;
        t.kb0 = (s.i0 > lo ? s.i0 : lo) - lo;
        t.kb1 = (s.i1 < hi ? s.i1 : hi) - lo;
        t.role = 1;
        t.sk_last = s.v + tt;  // the piece's slot
    }
    int64_t tm, tn;
    grouped_order<kGroupRowsK>(L, p.tiles_m, p.tiles_n, tm, tn);
    t.m0 = uni(tm * BM);
    t.n0 = uni(tn * BN);
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
        grouped_order<kGroupRowsK>(Lk % per_g, p.tiles_m, p.tiles_n, tm, tn);
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

// Quantizing epilogue: the wave's 128 x 64 block of the output as bf16 (hb:
// two values per word, columns 4 lg + {0, 1} and {2, 3} of MFMA tile (i, j),
// the rounding the bf16 output gets), quantized in 1x128 blocks exactly as
// bs_quant_1x128 quantizes a bf16 tensor.  The packed form halves the
// registers the epilogue holds, which keeps the K loop free of spills.
//  * rows: a block is 128 columns of one row, held by a pair of waves (wn,
//    wn ^ 1); each lane reduces its 16 values, the 4 lanes of a row exchange
//    maxima by shuffles, the pair through LDS.  Codes are staged in the
//    wave's 8 KiB of the free LDS stage ([row][64 B], 16-byte chunks XOR-ed
//    with row bits 2..3: conflict-free) and stored as whole 16-byte chunks;
//  * columns: a block is the wave's 128 rows of one column: each lane
//    reduces its 8 values, the 16 lanes of a DPP row hold one column's rows.
//    Each lane encodes 4 columns of one row per dword; a 4 x 4 byte
//    transpose across the lanes of a quad (two DPP exchanges, two byte
//    permutes) turns them into 4 rows of one column, staged as [col][128 B]
//    (16-byte chunks XOR-ed with column bits 1..3) and stored transposed.
__device__ __forceinline__ float hb_val(const uint32_t (&hb)[TM][TN][2], int i, int j, int r) {
    return (r & 1) ? bf16_hi(hb[i][j][r >> 1]) : bf16_lo(hb[i][j][r >> 1]);
}

// The lane index passed through an opaque move: address arithmetic derived
// from it is then computed where it is used, in each tile's epilogue,
// instead of being hoisted out of the tile loop and held (and spilled) across
// the K loop.
__device__ __forceinline__ int opaque_lane(int lane) {
    int v;
    asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "v"(lane));
    return v;
}

__device__ __forceinline__ void quant_epilogue(const GemmArgs& p, const uint32_t (&hb)[TM][TN][2], uint8_t* stq,
                                               float (*row_amax)[WAVES_N][TM][16], int64_t m_wave, int64_t m_end,
                                               int64_t n_wave, int wm, int wn, int lane_in) {
    const int lane = opaque_lane(lane_in);
    const int lr = lane & 15, lg = lane >> 4;
    const bool n_ok = n_wave < p.N;  // N % 128 == 0: a wave pair is wholly in or out
    if (p.q_row) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            float m = 0.f;
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) m = fmaxf(m, fabsf(hb_val(hb, i, j, r)));
            m = fmaxf(m, __shfl_xor(m, 16));
            m = fmaxf(m, __shfl_xor(m, 32));
            if (lg == 0) row_amax[wm][wn][i][lr] = m;
        }
        __syncthreads();
        const int64_t scol = (n_wave / 128) * p.ld_sr;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const Scale sc = block_scale(fmaxf(row_amax[wm][wn][i][lr], row_amax[wm][wn ^ 1][i][lr]));
            const int row = 16 * i + lr;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const uint32_t x = encode4(div_by_scale(hb_val(hb, i, j, 0), sc), div_by_scale(hb_val(hb, i, j, 1), sc),
                                           div_by_scale(hb_val(hb, i, j, 2), sc), div_by_scale(hb_val(hb, i, j, 3), sc));
                *reinterpret_cast<uint32_t*>(stq + row * 64 + ((j ^ ((row >> 2) & 3)) * 16) + 4 * lg) = x;
            }
            if (n_ok && (wn & 1) == 0 && lg == 0 && m_wave + row < m_end) p.s_row[scol + m_wave + row] = sc.s;
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // other lanes' staging writes
        if (n_ok) {
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int row = q * 16 + (lane >> 2), c = lane & 3;
                const uint4 v = *reinterpret_cast<const uint4*>(stq + row * 64 + ((c ^ ((row >> 2) & 3)) * 16));
                if (m_wave + row < m_end)
                    *reinterpret_cast<uint4*>(p.q_row + (m_wave + row) * p.ld_qr + n_wave + c * 16) = v;
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // staging reads done before reuse
    }
    if (p.q_col && n_ok && m_wave < m_end) {  // M % 128 == 0: the wave's 128 rows are all valid
        const int t4 = lane & 3, q4 = (lane >> 2) & 3;
        const uint32_t sel1 = (t4 & 1) ? 0x03070105u : 0x06020400u;
        const uint32_t sel2 = (t4 & 2) ? 0x03020706u : 0x05040100u;
        const int64_t srow = (m_wave / 128) * p.ld_sc + n_wave;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            Scale cs[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float m = 0.f;
#pragma unroll
                for (int i = 0; i < TM; ++i) m = fmaxf(m, fabsf(hb_val(hb, i, j, r)));
                cs[r] = block_scale(__uint_as_float(row16_max(__float_as_uint(m))));
            }
            const int col = 16 * j + 4 * lg + t4;
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const uint32_t x =
                    encode4(div_by_scale(hb_val(hb, i, j, 0), cs[0]), div_by_scale(hb_val(hb, i, j, 1), cs[1]),
                            div_by_scale(hb_val(hb, i, j, 2), cs[2]), div_by_scale(hb_val(hb, i, j, 3), cs[3]));
                // x: columns 4 lg .. + 3 of row 16 i + lane % 16; after the
                // transpose: rows 16 i + 4 q4 .. + 3 of column col
                const uint32_t px = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);
                const uint32_t z = __builtin_amdgcn_perm(px, x, sel1);
                const uint32_t pz = (uint32_t)__builtin_amdgcn_mov_dpp((int)z, 0x4E, 0xF, 0xF, false);
                const uint32_t y = __builtin_amdgcn_perm(pz, z, sel2);
                *reinterpret_cast<uint32_t*>(stq + col * 128 + 16 * (i ^ ((col >> 1) & 7)) + 4 * q4) = y;
            }
            if (lr == 0)
                *reinterpret_cast<float4*>(p.s_col + srow + 16 * j + 4 * lg) =
                    make_float4(cs[0].s, cs[1].s, cs[2].s, cs[3].s);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int col = k * 8 + (lane >> 3), c = lane & 7;
            const uint4 v = *reinterpret_cast<const uint4*>(stq + col * 128 + 16 * (c ^ ((col >> 1) & 7)));
            *reinterpret_cast<uint4*>(p.q_col + (n_wave + col) * p.ld_qc + m_wave + c * 16) = v;
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
}

template <int KIND, int SC, bool OUT_F32, bool SK = false, bool QEPI = false>
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
    SkPlan skp{};
    if (SK) {
        skp = sk_plan(p);
        idx = 0;
        if (!sk_has_work(skp, 0)) return;
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
    // Copy c = 0..7 of this wave's share: A for even c, B for odd c, rows
    // [(8i + w) * 8, +8) of round i = c / 2.
    auto issue_copy = [&](const Operands& o, int32_t kb, int s, int c) {
        const int k_off = kb * BK;
        const int i = c >> 1;
        if ((c & 1) == 0)
            dma16(o.a, lds_addr(&sm.a[s][(8 * i + w) * 1024]), voff_a, k_off + (int)(64 * i * p.lda));
        else
            dma16(o.b, lds_addr(&sm.b[s][(8 * i + w) * 1024]), voff_b, k_off + (int)(64 * i * p.ldb));
    };
    auto issue_loads = [&](const Operands& o, int32_t kb, int s) {
#pragma unroll
        for (int c = 0; c < 8; ++c) issue_copy(o, kb, s, c);
        issue_scales(o, kb, s, 0);
    };
    // The same copies issued by the four waves of group g alone (rows
    // [(4i + w % 4) * 8, +8) in round i = 0..7).  Copies stall the issuing
    // wave while the CU's address unit works through them (about 1 KiB per
    // 16 cycles); with one group issuing per K block, the other group's
    // waves go straight to their MFMAs and keep the matrix pipes busy.  The
    // MX kernel issues this way at the start of each block, the others but
    // GROUP_M in two halves after the first MFMAs (kLateIssue): every wave
    // issuing its share at the block start was 1.5-3 % slower, and so was
    // splitting the wgrad's copies (A by the group at the block start, B by
    // every wave after one of its first MFMAs).
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
    // Half h of issue_loads_group's copies (rounds 4h .. 4h + 3; the scales
    // with the first half).
    auto issue_loads_group_half = [&](const Operands& o, int32_t kb, int s, int g, int h) {
        if ((w >> 2) != g) return;
        const int k_off = kb * BK;
#pragma unroll
        for (int i = 4 * h; i < 4 * h + 4; ++i) {
            dma16(o.a, lds_addr(&sm.a[s][(4 * i + wq) * 1024]), voff_a4, k_off + (int)(32 * i * p.lda));
            dma16(o.b, lds_addr(&sm.b[s][(4 * i + wq) * 1024]), voff_b4, k_off + (int)(32 * i * p.ldb));
        }
        if (h == 0) issue_scales(o, kb, s, 4 * g);
    };
    // GROUP_M (MoE forward and dgrad, 128x128 B scales) has all eight waves
    // share the next K block's copies instead: wave w issues its issue_copy
    // pieces, one after each of its third to tenth MFMAs (waves 0 and 1 the
    // scales with the first piece), so every copy is still issued in the
    // first third of the block.  Both waves of a SIMD then carry the same
    // load and reach the block-end barrier together: with one group issuing,
    // the other group spent 16-24 % of its time waiting there.  The shared
    // spread is 3-5 % faster than one group spreading its copies over its
    // first MFMAs (itself 3-4 % faster than issuing every copy before the
    // first MFMA) and 1.2 % faster on the MoE forward than one group's
    // copies in two bursts (kLateIssue); starting it after the first MFMA
    // was 1 % slower, after the fourth or fifth 1-2 % slower.  The MX kernel
    // keeps the one-group issue at the block start (its shared spread was
    // 4 % slower).
    constexpr bool kSpread = !MX && !B1X128 && KIND == kGroupM;
    constexpr int kSpreadAt = 2;
    // The other kernels' issuing group takes its copies after its first
    // MFMAs instead of before them, so the matrix pipes start on both waves'
    // work at the block start: half after its third MFMA, half after its
    // fifth.  For the 1x128 x 1x128 wgrad (whose per-element fold leaves no
    // registers for a spread: one copy per MFMA spills), against all copies
    // before the first MFMA: MoE wgrad about 3 %, FFN-up wgrad 2 % faster;
    // measured alternatives, all slower: all copies after the first, second,
    // third or fifth MFMA; halves after the second and fourth, third and
    // fourth, fourth and fifth, or second and fifth MFMAs; quarters after
    // the second to fifth; a half after the sixth MFMA made the compiler
    // spill.  For the dense forward and dgrad (128x128 B scales), against
    // the shared spread from the first MFMA: 8192x4096x4096 and
    // 16384x5120x8192 forward 3.3-3.6 % faster, dgrads and the
    // 16384x7168x2048 GEMMs within 0.7 %.
    constexpr bool kLateIssue = !kSpread && !MX;
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
        sk_work(p, skp, idx, cur);
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
        const bool has_next = SK ? sk_has_work(skp, nidx) : nidx < total;
        Tile nxt = cur;
        Operands nops = ops;
        bool next_resolved = false;
        auto load_next = [&](int stage) {
            if (SK)
                sk_work(p, skp, nidx, nxt);
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
            const bool spread = kSpread && it + 1 < nkb;
            if (it + 1 < nkb) {
                if (!kSpread && !kLateIssue) issue_loads_group(ops, cur.kb0 + it + 1, s ^ 1, it & 1);
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
                        if (kSpread && q >= kSpreadAt && q < kSpreadAt + 8 && spread) {
                            if (q == kSpreadAt) issue_scales(ops, cur.kb0 + it + 1, s ^ 1, 0);
                            issue_copy(ops, cur.kb0 + it + 1, s ^ 1, q - kSpreadAt);
                        }
                        if (q > 0) fold(pbuf[(q - 1) & 1], pi, pj);
                        if (kLateIssue && (q == 2 || q == 4) && it + 1 < nkb)
                            issue_loads_group_half(ops, cur.kb0 + it + 1, s ^ 1, it & 1, q == 2 ? 0 : 1);
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

        // ---- stream-K: a piece leaves its partial tile in its slot,
        // lane-major as the registers hold it (the reduction kernel reads it
        // back in the same layout) ----
        bool store_d = true;
        if (SK && cur.role == 1) {
            const int sk_voff = (w * TM * TN * 64 + opaque_lane(lane)) * 16;
            const __amdgpu_buffer_rsrc_t slot = __builtin_amdgcn_make_buffer_rsrc(
                p.sk_partial + (int64_t)cur.sk_last * (BM * BN), (short)0, BM * BN * 4, 0x00020000);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[i][j]), slot, sk_voff,
                                                           (i * TN + j) * 1024, 0);
            store_d = false;
        }

        if (QEPI) {
            // the quantized values are those of the bf16 output: pack them
            // (round to nearest even) and let the fp32 tile go
            uint32_t hb[TM][TN][2];
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        hb[i][j][h] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)acc[i][j][2 * h]) |
                                      ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)acc[i][j][2 * h + 1]) << 16);
            uint8_t* const stq = (w < 4 ? sm.a[s ^ 1] : sm.b[s ^ 1]) + (w & 3) * 8192;
            quant_epilogue(p, hb, stq, sm.row_amax, (int64_t)cur.m0 + wm * WM, cur.m_end, (int64_t)cur.n0 + wn * WN,
                           wm, wn, lane);
            if (p.d) {
                // D from the packed values, staged as the plain epilogue does
                constexpr int PITCH = WN * 2 + 16;
                const int ln = opaque_lane(lane);
                const int rrow = ln / 8, rch = ln % 8, lr = ln & 15, lg = ln >> 4;
                const int64_t n = (int64_t)cur.n0 + wn * WN + rch * 8;
                uint16_t* const dbase = static_cast<uint16_t*>(p.d);
#pragma unroll
                for (int i = 0; i < TM; ++i) {
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        *reinterpret_cast<uint2*>(stq + lr * PITCH + (j * 16 + 4 * lg) * 2) =
                            make_uint2(hb[i][j][0], hb[i][j][1]);
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        const int row = q * 8 + rrow;
                        const uint4 v = *reinterpret_cast<const uint4*>(stq + row * PITCH + rch * 16);
                        const int64_t m = (int64_t)cur.m0 + wm * WM + i * 16 + row;
                        if (m < cur.m_end && n < p.N)
                            __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v),
                                                        reinterpret_cast<u32x4*>(dbase + m * p.ldd + n));
                    }
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                }
            }
            store_d = false;
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
            const int ln = SK ? opaque_lane(lane) : lane;
            const int rrow = ln / CPR, rch = ln % CPR, lr_e = ln & 15, lg_e = ln >> 4;
            const int64_t n = (int64_t)cur.n0 + wn * WN + rch * (16 / ESZ);
#pragma unroll
            for (int i = 0; i < TM; ++i) {
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const v4f v = acc[i][j];
                    uint8_t* const dst = stg + lr_e * PITCH + (j * 16 + 4 * lg_e) * ESZ;
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

// Stream-K reduction: workgroup (t, w) adds, for wave slice w of split tile
// t, the partial tiles of the shares v_first(t) .. v_last(t) in share order
// and writes D (rows < M, columns < N).  A thread takes 8 of the slice's 32
// MFMA tiles, one float4 (4 consecutive columns of one row) each.
template <bool OUT_F32>
__global__ __launch_bounds__(256) void sk_reduce_kernel(GemmArgs p) {
    const int64_t t = blockIdx.x / 8;
    const int w = blockIdx.x % 8, wm = w / WAVES_N, wn = w % WAVES_N;
    const int lane = threadIdx.x & 63, part = threadIdx.x >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int64_t nkb = p.K / BK, I = p.sk_tiles * nkb;
    // share holding iteration i: the largest v with v * I / sk_wgs <= i
    const int64_t v0 = ((t * nkb + 1) * p.sk_wgs - 1) / I, v1 = (((t + 1) * nkb) * p.sk_wgs - 1) / I;
    int64_t tm, tn;
    grouped_order<kGroupRowsK>(p.sk_dp_tiles + t, p.tiles_m, p.tiles_n, tm, tn);
#pragma unroll
    for (int k = 0; k < TM * TN / 4; ++k) {
        const int q = part * (TM * TN / 4) + k, i = q / TN, j = q % TN;
        float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int64_t v = v0; v <= v1; ++v) {
            const float4 x = reinterpret_cast<const float4*>(p.sk_partial + (v + t) * (BM * BN))[(w * TM * TN + q) * 64 + lane];
            if (v == v0) {
                s = x;
            } else {
                s.x += x.x;
                s.y += x.y;
                s.z += x.z;
                s.w += x.w;
            }
        }
        const int64_t m = tm * BM + wm * WM + i * 16 + lr;
        const int64_t n = tn * BN + wn * WN + j * 16 + 4 * lg;
        if (m < p.M && n < p.N) {
            if (OUT_F32) {
                *reinterpret_cast<float4*>(static_cast<float*>(p.d) + m * p.ldd + n) = s;
            } else {
                const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)s.x) |
                                    ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)s.y) << 16);
                const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)s.z) |
                                    ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)s.w) << 16);
                *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.d) + m * p.ldd + n) = make_uint2(lo, hi);
            }
        }
    }
}

template <bool B1X128>
__global__ __launch_bounds__(NT) void gemm_quant_kernel(GemmArgs p) {
    gemm_body<kDense, B1X128 ? kScale1x128 : kScale128x128, false, 0, true>(p);
}

// Persistent grid: as many workgroups as fit on the device at once, never
// more than the tiles.
template <typename Kern>
unsigned persistent_grid(Kern kernel, int64_t tiles) {
    const DeviceFit fit = device_fit(reinterpret_cast<const void*>(kernel), NT, 1);
    const int64_t cap = (int64_t)fit.cus * fit.per_cu;
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

}  // namespace

StreamK plan_streamk(const GemmArgs& a, ScaleMode scales, bool out_f32) {
    return scales == kScale1x128 ? plan_kind<true>(a, out_f32) : plan_kind<false>(a, out_f32);
}

int64_t streamk_workspace_bytes(const StreamK& sk) {
    if (sk.sk_tiles == 0) return 0;
    return (sk.sk_tiles + sk.sk_wgs) * (int64_t)(BM * BN) * 4;  // slots v + t
}

hipError_t launch_gemm_streamk(const GemmArgs& a, ScaleMode scales, bool out_f32, void* workspace,
                               int64_t workspace_bytes, hipStream_t stream) {
    const StreamK sk = plan_streamk(a, scales, out_f32);
    const int64_t need = streamk_workspace_bytes(sk);
    if (sk.sk_tiles == 0 || workspace == nullptr || workspace_bytes < need)
        return launch_gemm(a, kDense, scales, out_f32, stream);
    GemmArgs g = a;
    g.sk_dp_tiles = sk.dp_tiles;
    g.sk_tiles = sk.sk_tiles;
    g.sk_wgs = sk.sk_wgs;
    g.sk_partial = static_cast<float*>(workspace);
    const unsigned grid = (unsigned)sk.grid, rgrid = (unsigned)(sk.sk_tiles * 8);
    hipError_t e;
    if (scales == kScale1x128)
        e = out_f32 ? launch_grid(gemm_sk_kernel<true, true>, grid, g, stream)
                    : launch_grid(gemm_sk_kernel<true, false>, grid, g, stream);
    else
        e = out_f32 ? launch_grid(gemm_sk_kernel<false, true>, grid, g, stream)
                    : launch_grid(gemm_sk_kernel<false, false>, grid, g, stream);
    if (e != hipSuccess) return e;
    if (out_f32)
        hipLaunchKernelGGL(sk_reduce_kernel<true>, dim3(rgrid), dim3(256), 0, stream, g);
    else
        hipLaunchKernelGGL(sk_reduce_kernel<false>, dim3(rgrid), dim3(256), 0, stream, g);
    return hipGetLastError();
}

hipError_t launch_gemm_quant(const GemmArgs& a, ScaleMode scales, hipStream_t stream) {
    if (a.num_tiles <= 0) return hipSuccess;
    return scales == kScale1x128 ? launch_persistent_gemm(gemm_quant_kernel<true>, a, stream)
                                 : launch_persistent_gemm(gemm_quant_kernel<false>, a, stream);
}

hipError_t launch_gemm(const GemmArgs& a, GroupKind kind, ScaleMode scales, bool out_f32, hipStream_t stream) {
    switch (kind) {
        case kDense: return launch_kind<kDense>(a, scales, out_f32, stream);
        case kGroupM: return launch_kind<kGroupM>(a, scales, out_f32, stream);
        default: return launch_kind<kGroupK>(a, scales, out_f32, stream);
    }
}

}  // namespace bs
