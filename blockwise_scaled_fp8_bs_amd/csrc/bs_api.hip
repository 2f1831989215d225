// C ABI of the blockwise-scaled FP8 library: host-side validation, then one
// launch on the caller's stream.  Declarations and contracts: include/bs.h.
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/bs.h"
#include "bs_kernels.h"
#include "bs_mx.h"

namespace {

// Leading dimensions (elements) stay below 2^22 so that the kernels' lane
// and in-tile offsets (up to 256 rows of a tile) fit in 32 bits.
constexpr int64_t kMaxLd = (int64_t)1 << 22;

thread_local std::string g_last_error;

bs_status fail(bs_status st, const char* fn, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = std::string(fn) + ": " + buf;
    return st;
}

bs_status ok() {
    g_last_error.clear();
    return BS_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bs_status hip_status(hipError_t e, const char* fn) {
    if (e == hipSuccess) return ok();
    return fail(BS_ERR_HIP, fn, "kernel launch failed: %s", hipGetErrorString(e));
}

// Leading dimension checks, in elements.
#define REQUIRE(cond, code, ...)                           \
    do {                                                   \
        if (!(cond)) return fail(code, fn, __VA_ARGS__);   \
    } while (0)

}  // namespace

namespace bs {

DeviceFit device_fit(const void* kernel, int threads, int default_per_cu) {
    struct Entry {
        int dev;
        const void* kernel;
        int threads;
        DeviceFit fit;
    };
    static std::mutex mu;
    static std::vector<Entry> cache;
    int dev = -1;
    const bool have_dev = hipGetDevice(&dev) == hipSuccess;
    {
        std::lock_guard<std::mutex> lock(mu);
        for (const Entry& e : cache)
            if (have_dev && e.dev == dev && e.kernel == kernel && e.threads == threads) return e.fit;
    }
    DeviceFit fit{256, default_per_cu};
    bool complete = have_dev;
    int v = 0;
    if (have_dev && hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
        fit.cus = v;
    else
        complete = false;
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, threads, 0) == hipSuccess && occ > 0)
        fit.per_cu = occ;
    else
        complete = false;
    if (complete) {  // only answers from the runtime are kept
        std::lock_guard<std::mutex> lock(mu);
        cache.push_back(Entry{dev, kernel, threads, fit});
    }
    return fit;
}

}  // namespace bs

extern "C" {

const char* bs_status_string(bs_status st) {
    switch (st) {
        case BS_OK: return "BS_OK";
        case BS_ERR_NULL: return "BS_ERR_NULL";
        case BS_ERR_SHAPE: return "BS_ERR_SHAPE";
        case BS_ERR_LAYOUT: return "BS_ERR_LAYOUT";
        case BS_ERR_ALIGN: return "BS_ERR_ALIGN";
        case BS_ERR_MODE: return "BS_ERR_MODE";
        case BS_ERR_HIP: return "BS_ERR_HIP";
    }
    return "BS_ERR_UNKNOWN";
}

const char* bs_last_error(void) { return g_last_error.c_str(); }

namespace {

// Argument checks of the 1x128 quantizers (y, h already checked); fills *out.
bs_status check_quant_1x128(const char* fn, const uint16_t* x, const uint16_t* y, int64_t ld_y, uint16_t* h,
                            int64_t ld_h, int64_t R, int64_t C, int64_t ld_x, uint8_t* q_row, int64_t ld_qr,
                            float* s_row, int64_t ld_sr, uint8_t* q_col, int64_t ld_qc, float* s_col,
                            int64_t ld_sc, bs::Quant1x128Args* out) {
    const bool row = q_row || s_row, col = q_col || s_col;
    const bool empty = R == 0 || C == 0;
    REQUIRE(x || empty, BS_ERR_NULL, y ? "a is NULL" : "x is NULL");
    REQUIRE(!row || (q_row && s_row) || empty, BS_ERR_NULL, "q_row and s_row must both be set or both NULL");
    REQUIRE(!col || (q_col && s_col) || empty, BS_ERR_NULL, "q_col and s_col must both be set or both NULL");
    REQUIRE(row || col || empty, BS_ERR_NULL, "no output requested (q_row/s_row and q_col/s_col are all NULL)");
    REQUIRE(R >= 0 && C >= 0, BS_ERR_SHAPE, "R=%lld C=%lld must be >= 0", (long long)R, (long long)C);
    REQUIRE(C % 128 == 0, BS_ERR_SHAPE, "C=%lld must be a multiple of 128 (1x128 blocks along rows)",
            (long long)C);
    REQUIRE(!col || R % 128 == 0, BS_ERR_SHAPE,
            "R=%lld must be a multiple of 128 for the column output (128-row blocks)", (long long)R);
    REQUIRE(ld_x >= C, BS_ERR_LAYOUT, "ld_x=%lld < C=%lld: x must be row-major [R, C]", (long long)ld_x,
            (long long)C);
    REQUIRE(ld_x < kMaxLd, BS_ERR_LAYOUT, "ld_x=%lld must be < 2^22 (32-bit offsets inside a tile)", (long long)ld_x);
    REQUIRE(aligned16(x) && ld_x % 8 == 0, BS_ERR_ALIGN, "x must be 16-byte aligned with ld_x %% 8 == 0");
    if (row) {
        REQUIRE(ld_qr >= C, BS_ERR_LAYOUT, "ld_qr=%lld < C=%lld: q_row is row-major [R, C]", (long long)ld_qr,
                (long long)C);
        REQUIRE(ld_sr >= R, BS_ERR_LAYOUT, "ld_sr=%lld < R=%lld: s_row is K-major [C/128][ld_sr >= R]",
                (long long)ld_sr, (long long)R);
        REQUIRE(ld_sr % 4 == 0, BS_ERR_LAYOUT, "ld_sr=%lld must be a multiple of 4 (16-byte scale rows)",
                (long long)ld_sr);
        REQUIRE(ld_qr < kMaxLd, BS_ERR_LAYOUT, "ld_qr=%lld must be < 2^22", (long long)ld_qr);
        REQUIRE(aligned16(q_row) && ld_qr % 16 == 0, BS_ERR_ALIGN,
                "q_row must be 16-byte aligned with ld_qr %% 16 == 0");
        REQUIRE(aligned16(s_row), BS_ERR_ALIGN, "s_row must be 16-byte aligned");
    }
    if (col) {
        REQUIRE(ld_qc >= R, BS_ERR_LAYOUT, "ld_qc=%lld < R=%lld: q_col is the transpose [C, R]",
                (long long)ld_qc, (long long)R);
        REQUIRE(ld_sc >= C, BS_ERR_LAYOUT, "ld_sc=%lld < C=%lld: s_col is K-major [R/128][ld_sc >= C]",
                (long long)ld_sc, (long long)C);
        REQUIRE(ld_sc % 4 == 0, BS_ERR_LAYOUT, "ld_sc=%lld must be a multiple of 4 (16-byte scale rows)",
                (long long)ld_sc);
        REQUIRE(ld_qc < kMaxLd, BS_ERR_LAYOUT, "ld_qc=%lld must be < 2^22", (long long)ld_qc);
        REQUIRE(aligned16(q_col) && ld_qc % 16 == 0, BS_ERR_ALIGN,
                "q_col must be 16-byte aligned with ld_qc %% 16 == 0");
        REQUIRE(aligned16(s_col), BS_ERR_ALIGN, "s_col must be 16-byte aligned");
    }
    *out = bs::Quant1x128Args{x,    R,     C,     ld_x,  q_row, ld_qr, s_row, ld_sr, q_col, ld_qc,
                              s_col, ld_sc, C / 128, y,     ld_y,  h,     ld_h};
    return ok();
}

// Shared by bs_quant_1x128 and bs_swiglu_quant_1x128 (y, h already checked).
bs_status quant_1x128_common(const char* fn, const uint16_t* x, const uint16_t* y, int64_t ld_y, uint16_t* h,
                             int64_t ld_h, int64_t R, int64_t C, int64_t ld_x, uint8_t* q_row, int64_t ld_qr,
                             float* s_row, int64_t ld_sr, uint8_t* q_col, int64_t ld_qc, float* s_col,
                             int64_t ld_sc, hipStream_t stream) {
    bs::Quant1x128Args a{};
    const bs_status st = check_quant_1x128(fn, x, y, ld_y, h, ld_h, R, C, ld_x, q_row, ld_qr, s_row, ld_sr, q_col,
                                           ld_qc, s_col, ld_sc, &a);
    if (st != BS_OK || R == 0 || C == 0) return st;
    return hip_status(bs::launch_quant_1x128(a, q_row || s_row, q_col || s_col, y != nullptr, stream), fn);
}

}  // namespace

bs_status bs_quant_1x128(const uint16_t* x, int64_t R, int64_t C, int64_t ld_x, uint8_t* q_row, int64_t ld_qr,
                         float* s_row, int64_t ld_sr, uint8_t* q_col, int64_t ld_qc, float* s_col, int64_t ld_sc,
                         hipStream_t stream) {
    return quant_1x128_common("bs_quant_1x128", x, nullptr, 0, nullptr, 0, R, C, ld_x, q_row, ld_qr, s_row, ld_sr,
                              q_col, ld_qc, s_col, ld_sc, stream);
}

bs_status bs_swiglu_quant_1x128(const uint16_t* a, const uint16_t* b, int64_t R, int64_t C, int64_t ld_a,
                                int64_t ld_b, uint16_t* h, int64_t ld_h, uint8_t* q_row, int64_t ld_qr,
                                float* s_row, int64_t ld_sr, uint8_t* q_col, int64_t ld_qc, float* s_col,
                                int64_t ld_sc, hipStream_t stream) {
    static const char* fn = "bs_swiglu_quant_1x128";
    const bool empty = R == 0 || C == 0;
    REQUIRE(b || empty, BS_ERR_NULL, "b is NULL");
    REQUIRE(ld_b >= C, BS_ERR_LAYOUT, "ld_b=%lld < C=%lld: b must be row-major [R, C]", (long long)ld_b,
            (long long)C);
    REQUIRE(ld_b < kMaxLd, BS_ERR_LAYOUT, "ld_b=%lld must be < 2^22", (long long)ld_b);
    REQUIRE(aligned16(b) && ld_b % 8 == 0, BS_ERR_ALIGN, "b must be 16-byte aligned with ld_b %% 8 == 0");
    if (h) {
        REQUIRE(ld_h >= C, BS_ERR_LAYOUT, "ld_h=%lld < C=%lld: h is row-major [R, C]", (long long)ld_h,
                (long long)C);
        REQUIRE(ld_h < kMaxLd, BS_ERR_LAYOUT, "ld_h=%lld must be < 2^22", (long long)ld_h);
        REQUIRE(aligned16(h) && ld_h % 8 == 0, BS_ERR_ALIGN, "h must be 16-byte aligned with ld_h %% 8 == 0");
    }
    // a takes the place of x in the shared checks
    return quant_1x128_common(fn, a, empty ? nullptr : b, ld_b, h, ld_h, R, C, ld_a, q_row, ld_qr, s_row, ld_sr,
                              q_col, ld_qc, s_col, ld_sc, stream);
}

bs_status bs_swiglu_bwd_quant_1x128(const uint16_t* a, const uint16_t* b, const uint16_t* dh, int64_t R,
                                    int64_t C, int64_t ld_a, int64_t ld_b, int64_t ld_dh, uint16_t* dab,
                                    int64_t ld_dab, uint8_t* q_row, int64_t ld_qr, float* s_row, int64_t ld_sr,
                                    uint8_t* q_col, int64_t ld_qc, float* s_col, int64_t ld_sc,
                                    hipStream_t stream) {
    static const char* fn = "bs_swiglu_bwd_quant_1x128";
    const bool row = q_row || s_row, col = q_col || s_col;
    const bool empty = R == 0 || C == 0;
    REQUIRE((a && b && dh) || empty, BS_ERR_NULL, "a, b and dh must be non-NULL");
    REQUIRE(!row || (q_row && s_row) || empty, BS_ERR_NULL, "q_row and s_row must both be set or both NULL");
    REQUIRE(!col || (q_col && s_col) || empty, BS_ERR_NULL, "q_col and s_col must both be set or both NULL");
    REQUIRE(row || col || empty, BS_ERR_NULL, "no output requested (q_row/s_row and q_col/s_col are all NULL)");
    REQUIRE(R >= 0 && C >= 0, BS_ERR_SHAPE, "R=%lld C=%lld must be >= 0", (long long)R, (long long)C);
    REQUIRE(C % 128 == 0, BS_ERR_SHAPE, "C=%lld must be a multiple of 128 (1x128 blocks along rows)",
            (long long)C);
    REQUIRE(!col || R % 128 == 0, BS_ERR_SHAPE,
            "R=%lld must be a multiple of 128 for the column output (128-row blocks)", (long long)R);
    const struct { const uint16_t* p; int64_t ld; const char* name; } ins[3] = {{a, ld_a, "a"}, {b, ld_b, "b"},
                                                                             {dh, ld_dh, "dh"}};
    for (const auto& in : ins) {
        REQUIRE(in.ld >= C && in.ld < kMaxLd, BS_ERR_LAYOUT, "ld of %s = %lld must be >= C=%lld and < 2^22",
                in.name, (long long)in.ld, (long long)C);
        REQUIRE(aligned16(in.p) && in.ld % 8 == 0, BS_ERR_ALIGN, "%s must be 16-byte aligned with ld %% 8 == 0",
                in.name);
    }
    if (dab) {
        REQUIRE(ld_dab >= 2 * C && ld_dab < kMaxLd, BS_ERR_LAYOUT, "ld_dab=%lld must be >= 2C=%lld and < 2^22",
                (long long)ld_dab, (long long)(2 * C));
        REQUIRE(aligned16(dab) && ld_dab % 8 == 0, BS_ERR_ALIGN, "dab must be 16-byte aligned with ld_dab %% 8 == 0");
    }
    if (row) {
        REQUIRE(ld_qr >= 2 * C && ld_qr < kMaxLd, BS_ERR_LAYOUT,
                "ld_qr=%lld must be >= 2C=%lld (q_row is [R, 2C]) and < 2^22", (long long)ld_qr, (long long)(2 * C));
        REQUIRE(ld_sr >= R && ld_sr % 4 == 0, BS_ERR_LAYOUT,
                "ld_sr=%lld must be >= R=%lld and a multiple of 4 (s_row is K-major [2C/128][ld_sr])",
                (long long)ld_sr, (long long)R);
        REQUIRE(aligned16(q_row) && ld_qr % 16 == 0 && aligned16(s_row), BS_ERR_ALIGN,
                "q_row and s_row must be 16-byte aligned with ld_qr %% 16 == 0");
    }
    if (col) {
        REQUIRE(ld_qc >= R && ld_qc < kMaxLd, BS_ERR_LAYOUT,
                "ld_qc=%lld must be >= R=%lld (q_col is the transpose [2C, R]) and < 2^22", (long long)ld_qc,
                (long long)R);
        REQUIRE(ld_sc >= 2 * C && ld_sc % 4 == 0, BS_ERR_LAYOUT,
                "ld_sc=%lld must be >= 2C=%lld and a multiple of 4 (s_col is K-major [R/128][ld_sc])",
                (long long)ld_sc, (long long)(2 * C));
        REQUIRE(aligned16(q_col) && ld_qc % 16 == 0 && aligned16(s_col), BS_ERR_ALIGN,
                "q_col and s_col must be 16-byte aligned with ld_qc %% 16 == 0");
    }
    if (empty) return ok();
    bs::SwigluBwdArgs args{a,     b,     dh,    R,     C,     ld_a,  ld_b,  ld_dh, dab,   ld_dab,
                           q_row, ld_qr, s_row, ld_sr, q_col, ld_qc, s_col, ld_sc, C / 128};
    return hip_status(bs::launch_swiglu_bwd_quant(args, row, col, stream), fn);
}

bs_status bs_mx_quant_1x32(const uint16_t* x, int64_t R, int64_t C, int64_t ld_x, uint8_t* q_row, int64_t ld_qr,
                           uint8_t* s_row, int64_t ld_sr, uint8_t* q_col, int64_t ld_qc, uint8_t* s_col,
                           int64_t ld_sc, hipStream_t stream) {
    static const char* fn = "bs_mx_quant_1x32";
    const bool row = q_row || s_row, col = q_col || s_col;
    const bool empty = R == 0 || C == 0;
    REQUIRE(x || empty, BS_ERR_NULL, "x is NULL");
    REQUIRE(!row || (q_row && s_row) || empty, BS_ERR_NULL, "q_row and s_row must both be set or both NULL");
    REQUIRE(!col || (q_col && s_col) || empty, BS_ERR_NULL, "q_col and s_col must both be set or both NULL");
    REQUIRE(row || col || empty, BS_ERR_NULL, "no output requested (q_row/s_row and q_col/s_col are all NULL)");
    REQUIRE(R >= 0 && C >= 0, BS_ERR_SHAPE, "R=%lld C=%lld must be >= 0", (long long)R, (long long)C);
    REQUIRE(C % 128 == 0, BS_ERR_SHAPE, "C=%lld must be a multiple of 128 (128-column tiles of 32-element blocks)",
            (long long)C);
    REQUIRE(!col || R % 128 == 0, BS_ERR_SHAPE, "R=%lld must be a multiple of 128 for the column output",
            (long long)R);
    REQUIRE(ld_x >= C && ld_x < kMaxLd, BS_ERR_LAYOUT, "ld_x=%lld must be >= C=%lld and < 2^22", (long long)ld_x,
            (long long)C);
    REQUIRE(aligned16(x) && ld_x % 8 == 0, BS_ERR_ALIGN, "x must be 16-byte aligned with ld_x %% 8 == 0");
    if (row) {
        REQUIRE(ld_qr >= C && ld_qr < kMaxLd, BS_ERR_LAYOUT, "ld_qr=%lld must be >= C=%lld and < 2^22",
                (long long)ld_qr, (long long)C);
        REQUIRE(ld_sr >= R && ld_sr % 16 == 0, BS_ERR_LAYOUT,
                "ld_sr=%lld must be >= R=%lld and a multiple of 16 (s_row is K-major [C/32][ld_sr] bytes)",
                (long long)ld_sr, (long long)R);
        REQUIRE(aligned16(q_row) && ld_qr % 16 == 0 && aligned16(s_row), BS_ERR_ALIGN,
                "q_row and s_row must be 16-byte aligned with ld_qr %% 16 == 0");
    }
    if (col) {
        REQUIRE(ld_qc >= R && ld_qc < kMaxLd, BS_ERR_LAYOUT, "ld_qc=%lld must be >= R=%lld and < 2^22",
                (long long)ld_qc, (long long)R);
        REQUIRE(ld_sc >= C && ld_sc % 16 == 0, BS_ERR_LAYOUT,
                "ld_sc=%lld must be >= C=%lld and a multiple of 16 (s_col is K-major [R/32][ld_sc] bytes)",
                (long long)ld_sc, (long long)C);
        REQUIRE(aligned16(q_col) && ld_qc % 16 == 0 && aligned16(s_col), BS_ERR_ALIGN,
                "q_col and s_col must be 16-byte aligned with ld_qc %% 16 == 0");
    }
    if (empty) return ok();
    bs::MxQuantArgs a{x, R, C, ld_x, q_row, ld_qr, s_row, ld_sr, q_col, ld_qc, s_col, ld_sc, C / 128};
    return hip_status(bs::launch_mx_quant(a, row, col, stream), fn);
}

namespace {

// Argument checks shared by the MX GEMMs (dense and grouped).
bs_status check_mx_gemm_common(const char* fn, int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda,
                               const uint8_t* sa, int64_t ld_sa, const uint8_t* b, int64_t ldb, const uint8_t* sb,
                               int64_t ld_sb, void* d, int64_t ldd, bs_dtype d_dtype) {
    REQUIRE((a && sa) || M == 0 || K == 0, BS_ERR_NULL, "a and sa must be non-NULL");
    REQUIRE((b && sb) || N == 0 || K == 0, BS_ERR_NULL, "b and sb must be non-NULL");
    REQUIRE(d || M == 0 || N == 0, BS_ERR_NULL, "d must be non-NULL");
    REQUIRE(d_dtype == BS_OUT_BF16 || d_dtype == BS_OUT_F32, BS_ERR_MODE, "d_dtype=%d must be BF16 or F32",
            (int)d_dtype);
    REQUIRE(M >= 0 && N >= 0 && K >= 0, BS_ERR_SHAPE, "M, N, K must be >= 0");
    REQUIRE(N % 128 == 0, BS_ERR_SHAPE, "N=%lld must be a multiple of 128", (long long)N);
    REQUIRE(K % 128 == 0, BS_ERR_SHAPE, "K=%lld must be a multiple of 128 (four 32-element blocks per K step)",
            (long long)K);
    REQUIRE(lda >= K && ldb >= K, BS_ERR_LAYOUT,
            "lda=%lld, ldb=%lld must be >= K=%lld: a [M, K] and b [N, K] contiguous along the contraction",
            (long long)lda, (long long)ldb, (long long)K);
    REQUIRE(ldd >= N, BS_ERR_LAYOUT, "ldd=%lld < N=%lld: d is row-major [M, N]", (long long)ldd, (long long)N);
    REQUIRE(ld_sa >= M && ld_sa % 16 == 0, BS_ERR_LAYOUT,
            "ld_sa=%lld must be >= M=%lld and a multiple of 16 (sa is K-major [K/32][ld_sa] bytes)",
            (long long)ld_sa, (long long)M);
    REQUIRE(ld_sb >= N && ld_sb % 16 == 0, BS_ERR_LAYOUT,
            "ld_sb=%lld must be >= N=%lld and a multiple of 16 (sb is K-major [K/32][ld_sb] bytes)",
            (long long)ld_sb, (long long)N);
    REQUIRE(lda < (1ll << 22) && ldb < (1ll << 22), BS_ERR_LAYOUT,
            "lda and ldb must be < 2^22 elements (32-bit tile offsets)");
    REQUIRE((K / 32 + 1) * (ld_sa > ld_sb ? ld_sa : ld_sb) < (1ll << 31), BS_ERR_LAYOUT,
            "scale tensors must be smaller than 2 GiB (32-bit offsets)");
    REQUIRE(aligned16(a) && lda % 16 == 0 && aligned16(b) && ldb % 16 == 0, BS_ERR_ALIGN,
            "a and b must be 16-byte aligned with lda, ldb %% 16 == 0");
    REQUIRE(aligned16(sa) && aligned16(sb), BS_ERR_ALIGN, "sa and sb must be 16-byte aligned");
    REQUIRE(aligned16(d) && ldd % (d_dtype == BS_OUT_F32 ? 4 : 8) == 0, BS_ERR_ALIGN,
            "d must be 16-byte aligned with 16-byte rows");
    return ok();
}

}  // namespace

bs_status bs_mx_scaled_mm(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, const uint8_t* sa,
                          int64_t ld_sa, const uint8_t* b, int64_t ldb, const uint8_t* sb, int64_t ld_sb, void* d,
                          int64_t ldd, bs_dtype d_dtype, hipStream_t stream) {
    static const char* fn = "bs_mx_scaled_mm";
    bs_status st = check_mx_gemm_common(fn, M, N, K, a, lda, sa, ld_sa, b, ldb, sb, ld_sb, d, ldd, d_dtype);
    if (st != BS_OK) return st;
    if (M == 0 || N == 0) return ok();
    bs::GemmArgs g{};
    g.M = M; g.N = N; g.K = K;
    g.a = a; g.lda = lda; g.sa = sa; g.ld_sa = ld_sa;
    g.b = b; g.ldb = ldb; g.sb = sb; g.ld_sb = ld_sb;
    g.d = d; g.ldd = ldd;
    g.G = 1;
    g.tiles_m = (M + 255) / 256;
    g.tiles_n = (N + 255) / 256;
    g.num_tiles = g.tiles_m * g.tiles_n;
    return hip_status(bs::launch_gemm(g, bs::kDense, bs::kScaleMx, d_dtype == BS_OUT_F32, stream), fn);
}

bs_status bs_mx_grouped_scaled_mm(bs_group_mode mode, int64_t G, int64_t M, int64_t N, int64_t K,
                                  const int32_t* group_end, const uint8_t* a, int64_t lda, const uint8_t* sa,
                                  int64_t ld_sa, const uint8_t* b, int64_t stride_bg, int64_t ldb, const uint8_t* sb,
                                  int64_t stride_sbg, int64_t ld_sb, void* d, int64_t stride_dg, int64_t ldd,
                                  bs_dtype d_dtype, hipStream_t stream) {
    static const char* fn = "bs_mx_grouped_scaled_mm";
    REQUIRE(mode == BS_GROUP_M || mode == BS_GROUP_K, BS_ERR_MODE, "mode=%d must be BS_GROUP_M or BS_GROUP_K",
            (int)mode);
    REQUIRE(group_end, BS_ERR_NULL, "group_end is NULL");
    REQUIRE(G >= 0, BS_ERR_SHAPE, "G=%lld must be >= 0", (long long)G);
    bs_status st = check_mx_gemm_common(fn, M, N, K, a, lda, sa, ld_sa, b, ldb, sb, ld_sb, d, ldd, d_dtype);
    if (st != BS_OK) return st;
    bs::GemmArgs g{};
    g.M = M; g.N = N; g.K = K;
    g.a = a; g.lda = lda; g.sa = sa; g.ld_sa = ld_sa;
    g.b = b; g.ldb = ldb; g.sb = sb; g.ld_sb = ld_sb;
    g.d = d; g.ldd = ldd;
    g.G = G; g.group_end = group_end;
    g.tiles_n = (N + 255) / 256;
    if (mode == BS_GROUP_M) {
        REQUIRE(stride_dg == 0, BS_ERR_MODE, "BS_GROUP_M writes one D [M, N]: stride_dg must be 0");
        REQUIRE(stride_bg >= 0 && stride_sbg >= 0, BS_ERR_LAYOUT, "stride_bg and stride_sbg must be >= 0");
        REQUIRE(stride_bg % 16 == 0 && stride_sbg % 16 == 0, BS_ERR_ALIGN,
                "stride_bg and stride_sbg must be multiples of 16 bytes");
        if (G == 0 || M == 0 || N == 0) return ok();
        g.stride_bg = stride_bg;
        g.stride_sbg = stride_sbg;
        g.tiles_m = (M + 255) / 256;
        g.num_tiles = (g.tiles_m + G) * g.tiles_n;  // upper bound on the sum of per-group tile rows
        return hip_status(bs::launch_gemm(g, bs::kGroupM, bs::kScaleMx, d_dtype == BS_OUT_F32, stream), fn);
    }
    REQUIRE(stride_bg == 0 && stride_sbg == 0, BS_ERR_MODE,
            "BS_GROUP_K shares one B over the groups: stride_bg and stride_sbg must be 0");
    REQUIRE(M % 128 == 0, BS_ERR_SHAPE, "M=%lld must be a multiple of 128 for BS_GROUP_K", (long long)M);
    REQUIRE(G <= 1 || stride_dg >= M * ldd, BS_ERR_LAYOUT, "stride_dg=%lld < M*ldd", (long long)stride_dg);
    REQUIRE(stride_dg % (d_dtype == BS_OUT_F32 ? 4 : 8) == 0, BS_ERR_ALIGN,
            "stride_dg must keep every D[g] 16-byte aligned");
    if (G == 0 || M == 0 || N == 0) return ok();
    g.stride_dg = stride_dg;
    g.tiles_m = (M + 255) / 256;
    g.num_tiles = G * g.tiles_m * g.tiles_n;
    return hip_status(bs::launch_gemm(g, bs::kGroupK, bs::kScaleMx, d_dtype == BS_OUT_F32, stream), fn);
}

bs_status bs_quant_128x128(const uint16_t* x, int64_t R, int64_t C, int64_t ld_x, uint8_t* q, int64_t ld_q,
                           float* s, int64_t ld_s, hipStream_t stream) {
    static const char* fn = "bs_quant_128x128";
    REQUIRE((x && q && s) || R == 0 || C == 0, BS_ERR_NULL, "x, q and s must be non-NULL");
    REQUIRE(R >= 0 && C >= 0 && R % 128 == 0 && C % 128 == 0, BS_ERR_SHAPE,
            "R=%lld C=%lld must be non-negative multiples of 128 (128x128 blocks)", (long long)R, (long long)C);
    REQUIRE(ld_x >= C, BS_ERR_LAYOUT, "ld_x=%lld < C=%lld: x must be row-major [R, C]", (long long)ld_x,
            (long long)C);
    REQUIRE(ld_q >= C, BS_ERR_LAYOUT, "ld_q=%lld < C=%lld: q is row-major [R, C]", (long long)ld_q, (long long)C);
    REQUIRE(ld_s >= R / 128, BS_ERR_LAYOUT, "ld_s=%lld < R/128=%lld: s is K-major [C/128][ld_s >= R/128]",
            (long long)ld_s, (long long)(R / 128));
    REQUIRE(ld_s % 4 == 0, BS_ERR_LAYOUT, "ld_s=%lld must be a multiple of 4 (K stride padded to 16 bytes)",
            (long long)ld_s);
    REQUIRE(ld_x < kMaxLd, BS_ERR_LAYOUT, "ld_x=%lld must be < 2^22 (32-bit offsets inside a tile)", (long long)ld_x);
    REQUIRE(ld_q < kMaxLd, BS_ERR_LAYOUT, "ld_q=%lld must be < 2^22", (long long)ld_q);
    REQUIRE(aligned16(x) && ld_x % 8 == 0, BS_ERR_ALIGN, "x must be 16-byte aligned with ld_x %% 8 == 0");
    REQUIRE(aligned16(q) && ld_q % 16 == 0, BS_ERR_ALIGN, "q must be 16-byte aligned with ld_q %% 16 == 0");
    REQUIRE(aligned16(s), BS_ERR_ALIGN, "s must be 16-byte aligned");
    if (R == 0 || C == 0) return ok();
    bs::Quant128Args a{x, 1, R, C, 0, ld_x, q, 0, ld_q, s, 0, ld_s, R / 128, C / 128};
    return hip_status(bs::launch_quant_128x128(a, bs::kQ128Rows, stream), fn);
}

bs_status bs_quant_3d_colwise(const uint16_t* x, int64_t G, int64_t R, int64_t C, int64_t stride_xg, int64_t ld_x,
                              uint8_t* q, int64_t stride_qg, int64_t ld_q, float* s, int64_t stride_sg, int64_t ld_s,
                              hipStream_t stream) {
    static const char* fn = "bs_quant_3d_colwise";
    REQUIRE((x && q && s) || G == 0 || R == 0 || C == 0, BS_ERR_NULL, "x, q and s must be non-NULL");
    REQUIRE(G >= 0 && R >= 0 && C >= 0 && R % 128 == 0 && C % 128 == 0, BS_ERR_SHAPE,
            "G=%lld R=%lld C=%lld: G >= 0 and R, C non-negative multiples of 128", (long long)G, (long long)R,
            (long long)C);
    REQUIRE(ld_x >= C, BS_ERR_LAYOUT, "ld_x=%lld < C=%lld: x[g] must be row-major [R, C]", (long long)ld_x,
            (long long)C);
    REQUIRE(G <= 1 || stride_xg >= R * ld_x, BS_ERR_LAYOUT, "stride_xg=%lld < R*ld_x", (long long)stride_xg);
    REQUIRE(ld_q >= R, BS_ERR_LAYOUT, "ld_q=%lld < R=%lld: q[g] is the transpose [C, R]", (long long)ld_q,
            (long long)R);
    REQUIRE(G <= 1 || stride_qg >= C * ld_q, BS_ERR_LAYOUT, "stride_qg=%lld < C*ld_q", (long long)stride_qg);
    REQUIRE(ld_s >= C / 128, BS_ERR_LAYOUT, "ld_s=%lld < C/128=%lld: s[g] is K-major [R/128][ld_s >= C/128]",
            (long long)ld_s, (long long)(C / 128));
    REQUIRE(ld_s % 4 == 0, BS_ERR_LAYOUT, "ld_s=%lld must be a multiple of 4", (long long)ld_s);
    REQUIRE(G <= 1 || stride_sg >= (R / 128) * ld_s, BS_ERR_LAYOUT, "stride_sg=%lld < (R/128)*ld_s",
            (long long)stride_sg);
    REQUIRE(stride_sg % 4 == 0 && stride_qg % 16 == 0 && stride_xg % 8 == 0, BS_ERR_ALIGN,
            "group strides must keep 16-byte alignment (stride_sg %% 4, stride_qg %% 16, stride_xg %% 8)");
    REQUIRE(ld_x < kMaxLd, BS_ERR_LAYOUT, "ld_x=%lld must be < 2^22 (32-bit offsets inside a tile)", (long long)ld_x);
    REQUIRE(ld_q < kMaxLd, BS_ERR_LAYOUT, "ld_q=%lld must be < 2^22", (long long)ld_q);
    REQUIRE(aligned16(x) && ld_x % 8 == 0, BS_ERR_ALIGN, "x must be 16-byte aligned with ld_x %% 8 == 0");
    REQUIRE(aligned16(q) && ld_q % 16 == 0, BS_ERR_ALIGN, "q must be 16-byte aligned with ld_q %% 16 == 0");
    REQUIRE(aligned16(s), BS_ERR_ALIGN, "s must be 16-byte aligned");
    if (G == 0 || R == 0 || C == 0) return ok();
    bs::Quant128Args a{x, G, R, C, stride_xg, ld_x, q, stride_qg, ld_q, s, stride_sg, ld_s, R / 128, C / 128};
    return hip_status(bs::launch_quant_128x128(a, bs::kQ128Transposed, stream), fn);
}

namespace {

// Argument checks of the two-layout 128x128 quantizer; fills *out.
bs_status check_quant_128x128_both(const char* fn, const uint16_t* x, int64_t G, int64_t R, int64_t C,
                                   int64_t stride_xg, int64_t ld_x, uint8_t* q, int64_t ld_q, float* s,
                                   int64_t ld_s, uint8_t* qt, int64_t stride_qtg, int64_t ld_qt, float* st,
                                   int64_t stride_stg, int64_t ld_st, bs::Quant128Args* out) {
    REQUIRE((x && q && s && qt && st) || G == 0 || R == 0 || C == 0, BS_ERR_NULL,
            "x, q, s, qt and st must be non-NULL");
    REQUIRE(G >= 0 && R >= 0 && C >= 0 && R % 128 == 0 && C % 128 == 0, BS_ERR_SHAPE,
            "G=%lld R=%lld C=%lld: G >= 0 and R, C non-negative multiples of 128", (long long)G, (long long)R,
            (long long)C);
    REQUIRE(ld_x >= C, BS_ERR_LAYOUT, "ld_x=%lld < C=%lld: x[g] must be row-major [R, C]", (long long)ld_x,
            (long long)C);
    REQUIRE(G <= 1 || stride_xg >= R * ld_x, BS_ERR_LAYOUT, "stride_xg=%lld < R*ld_x", (long long)stride_xg);
    REQUIRE(ld_q >= C, BS_ERR_LAYOUT, "ld_q=%lld < C=%lld: q is row-major [G*R, C]", (long long)ld_q, (long long)C);
    REQUIRE(ld_s >= G * (R / 128), BS_ERR_LAYOUT,
            "ld_s=%lld < G*R/128=%lld: s is K-major [C/128][ld_s >= G*R/128]", (long long)ld_s,
            (long long)(G * (R / 128)));
    REQUIRE(ld_s % 4 == 0, BS_ERR_LAYOUT, "ld_s=%lld must be a multiple of 4", (long long)ld_s);
    REQUIRE(ld_qt >= R, BS_ERR_LAYOUT, "ld_qt=%lld < R=%lld: qt[g] is the transpose [C, R]", (long long)ld_qt,
            (long long)R);
    REQUIRE(G <= 1 || stride_qtg >= C * ld_qt, BS_ERR_LAYOUT, "stride_qtg=%lld < C*ld_qt", (long long)stride_qtg);
    REQUIRE(ld_st >= C / 128, BS_ERR_LAYOUT, "ld_st=%lld < C/128=%lld: st[g] is K-major [R/128][ld_st >= C/128]",
            (long long)ld_st, (long long)(C / 128));
    REQUIRE(ld_st % 4 == 0, BS_ERR_LAYOUT, "ld_st=%lld must be a multiple of 4", (long long)ld_st);
    REQUIRE(G <= 1 || stride_stg >= (R / 128) * ld_st, BS_ERR_LAYOUT, "stride_stg=%lld < (R/128)*ld_st",
            (long long)stride_stg);
    REQUIRE(stride_stg % 4 == 0 && stride_qtg % 16 == 0 && stride_xg % 8 == 0, BS_ERR_ALIGN,
            "group strides must keep 16-byte alignment (stride_stg %% 4, stride_qtg %% 16, stride_xg %% 8)");
    REQUIRE(ld_x < kMaxLd, BS_ERR_LAYOUT, "ld_x=%lld must be < 2^22 (32-bit offsets inside a tile)", (long long)ld_x);
    REQUIRE(ld_q < kMaxLd && ld_qt < kMaxLd, BS_ERR_LAYOUT, "ld_q=%lld and ld_qt=%lld must be < 2^22",
            (long long)ld_q, (long long)ld_qt);
    REQUIRE(aligned16(x) && ld_x % 8 == 0, BS_ERR_ALIGN, "x must be 16-byte aligned with ld_x %% 8 == 0");
    REQUIRE(aligned16(q) && ld_q % 16 == 0, BS_ERR_ALIGN, "q must be 16-byte aligned with ld_q %% 16 == 0");
    REQUIRE(aligned16(qt) && ld_qt % 16 == 0, BS_ERR_ALIGN, "qt must be 16-byte aligned with ld_qt %% 16 == 0");
    REQUIRE(aligned16(s) && aligned16(st), BS_ERR_ALIGN, "s and st must be 16-byte aligned");
    // rows of expert g are rows g*R .. of the stacked q; its scale columns
    // start at g*R/128 of each K-major row of s
    *out = bs::Quant128Args{x, G, R, C, stride_xg, ld_x, q, R * ld_q, ld_q, s, R / 128, ld_s, R / 128, C / 128,
                            qt, stride_qtg, ld_qt, st, stride_stg, ld_st};
    return ok();
}

}  // namespace

bs_status bs_quant_128x128_both(const uint16_t* x, int64_t G, int64_t R, int64_t C, int64_t stride_xg,
                                int64_t ld_x, uint8_t* q, int64_t ld_q, float* s, int64_t ld_s, uint8_t* qt,
                                int64_t stride_qtg, int64_t ld_qt, float* st, int64_t stride_stg, int64_t ld_st,
                                hipStream_t stream) {
    static const char* fn = "bs_quant_128x128_both";
    bs::Quant128Args a{};
    const bs_status status = check_quant_128x128_both(fn, x, G, R, C, stride_xg, ld_x, q, ld_q, s, ld_s, qt,
                                                      stride_qtg, ld_qt, st, stride_stg, ld_st, &a);
    if (status != BS_OK || G == 0 || R == 0 || C == 0) return status;
    return hip_status(bs::launch_quant_128x128(a, bs::kQ128Both, stream), fn);
}

bs_status bs_quant_fwd_operands(const uint16_t* x, int64_t R, int64_t C, int64_t ld_x, uint8_t* q_row,
                                int64_t ld_qr, float* s_row, int64_t ld_sr, uint8_t* q_col, int64_t ld_qc,
                                float* s_col, int64_t ld_sc, const uint16_t* w, int64_t G, int64_t N, int64_t K,
                                int64_t stride_wg, int64_t ld_w, uint8_t* qw, int64_t ld_qw, float* sw,
                                int64_t ld_sw, uint8_t* qwt, int64_t stride_qwtg, int64_t ld_qwt, float* swt,
                                int64_t stride_swtg, int64_t ld_swt, hipStream_t stream) {
    static const char* fn = "bs_quant_fwd_operands";
    const bool x_empty = R == 0 || C == 0;
    REQUIRE((q_row && s_row && q_col && s_col) || x_empty, BS_ERR_NULL,
            "q_row, s_row, q_col and s_col must all be set (x is quantized along rows and columns)");
    bs::Quant1x128Args xa{};
    bs_status status = check_quant_1x128(fn, x, nullptr, 0, nullptr, 0, R, C, ld_x, q_row, ld_qr, s_row, ld_sr,
                                         q_col, ld_qc, s_col, ld_sc, &xa);
    if (status != BS_OK) return status;
    bs::Quant128Args wa{};
    status = check_quant_128x128_both(fn, w, G, N, K, stride_wg, ld_w, qw, ld_qw, sw, ld_sw, qwt, stride_qwtg,
                                      ld_qwt, swt, stride_swtg, ld_swt, &wa);
    if (status != BS_OK) return status;
    if (x_empty) xa.R = 0, xa.col_tiles = 0;
    if (G == 0 || N == 0 || K == 0) wa.G = 0;
    return hip_status(bs::launch_quant_pair(xa, wa, stream), fn);
}

namespace {

bs_status check_gemm_common(const char* fn, int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda,
                            const float* sa, int64_t ld_sa, const uint8_t* b, int64_t ldb, const float* sb,
                            int64_t ld_sb, bs_scale_kind b_kind, void* d, int64_t ldd, bs_dtype d_dtype) {
    REQUIRE((a && sa) || M == 0 || K == 0, BS_ERR_NULL, "a and sa must be non-NULL");
    REQUIRE((b && sb) || N == 0 || K == 0, BS_ERR_NULL, "b and sb must be non-NULL");
    REQUIRE(d || M == 0 || N == 0, BS_ERR_NULL, "d must be non-NULL");
    REQUIRE(b_kind == BS_SCALE_1X128 || b_kind == BS_SCALE_128X128, BS_ERR_MODE,
            "b_kind=%d must be BS_SCALE_1X128 (4) or BS_SCALE_128X128 (5)", (int)b_kind);
    REQUIRE(d_dtype == BS_OUT_BF16 || d_dtype == BS_OUT_F32, BS_ERR_MODE, "d_dtype=%d must be BF16 or F32",
            (int)d_dtype);
    REQUIRE(M >= 0 && N >= 0 && K >= 0, BS_ERR_SHAPE, "M, N, K must be >= 0");
    REQUIRE(N % 128 == 0, BS_ERR_SHAPE, "N=%lld must be a multiple of 128", (long long)N);
    REQUIRE(K % 128 == 0, BS_ERR_SHAPE, "K=%lld must be a multiple of 128 (1x128 blocks along K)", (long long)K);
    REQUIRE(lda >= K, BS_ERR_LAYOUT,
            "lda=%lld < K=%lld: a must be row-major [M, K] (contiguous along the contraction)", (long long)lda,
            (long long)K);
    REQUIRE(ldb >= K, BS_ERR_LAYOUT,
            "ldb=%lld < K=%lld: b must be [N, K] contiguous along K (column-major B of D = A.B)", (long long)ldb,
            (long long)K);
    REQUIRE(ldd >= N, BS_ERR_LAYOUT, "ldd=%lld < N=%lld: d is row-major [M, N]", (long long)ldd, (long long)N);
    REQUIRE(ld_sa % 4 == 0, BS_ERR_LAYOUT, "ld_sa=%lld must be a multiple of 4", (long long)ld_sa);
    REQUIRE(ld_sb % 4 == 0, BS_ERR_LAYOUT, "ld_sb=%lld must be a multiple of 4", (long long)ld_sb);
    // Operand tiles and scale rows are addressed with 32-bit buffer offsets.
    REQUIRE(lda < (1ll << 22) && ldb < (1ll << 22), BS_ERR_LAYOUT,
            "lda and ldb must be < 2^22 elements (32-bit tile offsets)");
    REQUIRE((K / 128 + 1) * (ld_sa > ld_sb ? ld_sa : ld_sb) < (1ll << 29), BS_ERR_LAYOUT,
            "scale tensors must be smaller than 2 GiB (32-bit offsets)");
    REQUIRE(aligned16(a) && lda % 16 == 0, BS_ERR_ALIGN, "a must be 16-byte aligned with lda %% 16 == 0");
    REQUIRE(aligned16(b) && ldb % 16 == 0, BS_ERR_ALIGN, "b must be 16-byte aligned with ldb %% 16 == 0");
    REQUIRE(aligned16(sa) && aligned16(sb), BS_ERR_ALIGN, "sa and sb must be 16-byte aligned");
    REQUIRE(aligned16(d) && ldd % (d_dtype == BS_OUT_F32 ? 4 : 8) == 0, BS_ERR_ALIGN,
            "d must be 16-byte aligned with 16-byte rows");
    return ok();
}

}  // namespace

bs_status bs_scaled_mm(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, const float* sa,
                       int64_t ld_sa, bs_scale_kind a_kind, const uint8_t* b, int64_t ldb, const float* sb,
                       int64_t ld_sb, bs_scale_kind b_kind, void* d, int64_t ldd, bs_dtype d_dtype,
                       hipStream_t stream) {
    static const char* fn = "bs_scaled_mm";
    REQUIRE(a_kind == BS_SCALE_1X128, BS_ERR_MODE, "a_kind=%d: A takes 1x128 scales (BS_SCALE_1X128 = 4)",
            (int)a_kind);
    bs_status st = check_gemm_common(fn, M, N, K, a, lda, sa, ld_sa, b, ldb, sb, ld_sb, b_kind, d, ldd, d_dtype);
    if (st != BS_OK) return st;
    REQUIRE(ld_sa >= M, BS_ERR_LAYOUT, "ld_sa=%lld < M=%lld: sa is K-major [K/128][ld_sa >= M]",
            (long long)ld_sa, (long long)M);
    const int64_t nrows_sb = b_kind == BS_SCALE_1X128 ? N : N / 128;
    REQUIRE(ld_sb >= nrows_sb, BS_ERR_LAYOUT, "ld_sb=%lld < %lld: sb is K-major [K/128][ld_sb >= %s]",
            (long long)ld_sb, (long long)nrows_sb, b_kind == BS_SCALE_1X128 ? "N" : "N/128");
    if (M == 0 || N == 0) return ok();
    bs::GemmArgs g{};
    g.M = M; g.N = N; g.K = K;
    g.a = a; g.lda = lda; g.sa = sa; g.ld_sa = ld_sa;
    g.b = b; g.ldb = ldb; g.sb = sb; g.ld_sb = ld_sb;
    g.d = d; g.ldd = ldd;
    g.G = 1;
    g.tiles_m = (M + 255) / 256;
    g.tiles_n = (N + 255) / 256;
    g.num_tiles = g.tiles_m * g.tiles_n;
    return hip_status(bs::launch_gemm(g, bs::kDense, b_kind == BS_SCALE_1X128 ? bs::kScale1x128 : bs::kScale128x128,
                                      d_dtype == BS_OUT_F32, stream), fn);
}

namespace {

// The dense problem of bs_scaled_mm as kernel arguments (validated).
bs::GemmArgs dense_args(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, const float* sa,
                        int64_t ld_sa, const uint8_t* b, int64_t ldb, const float* sb, int64_t ld_sb, void* d,
                        int64_t ldd) {
    bs::GemmArgs g{};
    g.M = M; g.N = N; g.K = K;
    g.a = a; g.lda = lda; g.sa = sa; g.ld_sa = ld_sa;
    g.b = b; g.ldb = ldb; g.sb = sb; g.ld_sb = ld_sb;
    g.d = d; g.ldd = ldd;
    g.G = 1;
    g.tiles_m = (M + 255) / 256;
    g.tiles_n = (N + 255) / 256;
    g.num_tiles = g.tiles_m * g.tiles_n;
    return g;
}

}  // namespace

bs_status bs_scaled_mm_quant(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, const float* sa,
                             int64_t ld_sa, bs_scale_kind a_kind, const uint8_t* b, int64_t ldb, const float* sb,
                             int64_t ld_sb, bs_scale_kind b_kind, uint16_t* d, int64_t ldd, uint8_t* q_row,
                             int64_t ld_qr, float* s_row, int64_t ld_sr, uint8_t* q_col, int64_t ld_qc, float* s_col,
                             int64_t ld_sc, hipStream_t stream) {
    static const char* fn = "bs_scaled_mm_quant";
    const bool row = q_row || s_row, col = q_col || s_col;
    const bool empty = M == 0 || N == 0;
    REQUIRE(a_kind == BS_SCALE_1X128, BS_ERR_MODE, "a_kind=%d: A takes 1x128 scales (BS_SCALE_1X128 = 4)",
            (int)a_kind);
    REQUIRE(!row || (q_row && s_row) || empty, BS_ERR_NULL, "q_row and s_row must both be set or both NULL");
    REQUIRE(!col || (q_col && s_col) || empty, BS_ERR_NULL, "q_col and s_col must both be set or both NULL");
    REQUIRE(d || row || col || empty, BS_ERR_NULL, "no output requested (d, q_row/s_row and q_col/s_col all NULL)");
    // d is checked as bs_scaled_mm's bf16 output when given (a stand-in pointer otherwise)
    bs_status st = check_gemm_common(fn, M, N, K, a, lda, sa, ld_sa, b, ldb, sb, ld_sb, b_kind,
                                     d ? static_cast<void*>(d) : reinterpret_cast<void*>(16), d ? ldd : N,
                                     BS_OUT_BF16);
    if (st != BS_OK) return st;
    REQUIRE(ld_sa >= M, BS_ERR_LAYOUT, "ld_sa=%lld < M=%lld: sa is K-major [K/128][ld_sa >= M]",
            (long long)ld_sa, (long long)M);
    const int64_t nrows_sb = b_kind == BS_SCALE_1X128 ? N : N / 128;
    REQUIRE(ld_sb >= nrows_sb, BS_ERR_LAYOUT, "ld_sb=%lld < %lld: sb is K-major [K/128][ld_sb >= %s]",
            (long long)ld_sb, (long long)nrows_sb, b_kind == BS_SCALE_1X128 ? "N" : "N/128");
    REQUIRE(!col || M % 128 == 0, BS_ERR_SHAPE,
            "M=%lld must be a multiple of 128 for the column output (128-row blocks)", (long long)M);
    if (row) {
        REQUIRE(ld_qr >= N && ld_qr < kMaxLd, BS_ERR_LAYOUT, "ld_qr=%lld must be >= N=%lld (q_row is [M, N]) and < 2^22",
                (long long)ld_qr, (long long)N);
        REQUIRE(ld_sr >= M && ld_sr % 4 == 0, BS_ERR_LAYOUT,
                "ld_sr=%lld must be >= M=%lld and a multiple of 4 (s_row is K-major [N/128][ld_sr])",
                (long long)ld_sr, (long long)M);
        REQUIRE(aligned16(q_row) && ld_qr % 16 == 0 && aligned16(s_row), BS_ERR_ALIGN,
                "q_row and s_row must be 16-byte aligned with ld_qr %% 16 == 0");
    }
    if (col) {
        REQUIRE(ld_qc >= M && ld_qc < kMaxLd, BS_ERR_LAYOUT,
                "ld_qc=%lld must be >= M=%lld (q_col is the transpose [N, M]) and < 2^22", (long long)ld_qc,
                (long long)M);
        REQUIRE(ld_sc >= N && ld_sc % 4 == 0, BS_ERR_LAYOUT,
                "ld_sc=%lld must be >= N=%lld and a multiple of 4 (s_col is K-major [M/128][ld_sc])",
                (long long)ld_sc, (long long)N);
        REQUIRE(aligned16(q_col) && ld_qc % 16 == 0 && aligned16(s_col), BS_ERR_ALIGN,
                "q_col and s_col must be 16-byte aligned with ld_qc %% 16 == 0");
    }
    if (empty) return ok();
    bs::GemmArgs g = dense_args(M, N, K, a, lda, sa, ld_sa, b, ldb, sb, ld_sb, d, ldd);
    g.q_row = row ? q_row : nullptr;
    g.ld_qr = ld_qr;
    g.s_row = row ? s_row : nullptr;
    g.ld_sr = ld_sr;
    g.q_col = col ? q_col : nullptr;
    g.ld_qc = ld_qc;
    g.s_col = col ? s_col : nullptr;
    g.ld_sc = ld_sc;
    return hip_status(
        bs::launch_gemm_quant(g, b_kind == BS_SCALE_1X128 ? bs::kScale1x128 : bs::kScale128x128, stream), fn);
}

int64_t bs_scaled_mm_workspace_bytes(int64_t M, int64_t N, int64_t K, bs_scale_kind b_kind, bs_dtype d_dtype) {
    if (M <= 0 || N <= 0 || K <= 0 || N % 128 || K % 128) return 0;
    if (b_kind != BS_SCALE_1X128 && b_kind != BS_SCALE_128X128) return 0;
    const bs::GemmArgs g = dense_args(M, N, K, nullptr, K, nullptr, M, nullptr, K, nullptr, N, nullptr, N);
    return bs::streamk_workspace_bytes(bs::plan_streamk(
        g, b_kind == BS_SCALE_1X128 ? bs::kScale1x128 : bs::kScale128x128, d_dtype == BS_OUT_F32));
}

bs_status bs_scaled_mm_ws(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, const float* sa,
                          int64_t ld_sa, bs_scale_kind a_kind, const uint8_t* b, int64_t ldb, const float* sb,
                          int64_t ld_sb, bs_scale_kind b_kind, void* d, int64_t ldd, bs_dtype d_dtype,
                          void* workspace, int64_t workspace_bytes, hipStream_t stream) {
    static const char* fn = "bs_scaled_mm_ws";
    REQUIRE(a_kind == BS_SCALE_1X128, BS_ERR_MODE, "a_kind=%d: A takes 1x128 scales (BS_SCALE_1X128 = 4)",
            (int)a_kind);
    bs_status st = check_gemm_common(fn, M, N, K, a, lda, sa, ld_sa, b, ldb, sb, ld_sb, b_kind, d, ldd, d_dtype);
    if (st != BS_OK) return st;
    REQUIRE(ld_sa >= M, BS_ERR_LAYOUT, "ld_sa=%lld < M=%lld: sa is K-major [K/128][ld_sa >= M]",
            (long long)ld_sa, (long long)M);
    const int64_t nrows_sb = b_kind == BS_SCALE_1X128 ? N : N / 128;
    REQUIRE(ld_sb >= nrows_sb, BS_ERR_LAYOUT, "ld_sb=%lld < %lld: sb is K-major [K/128][ld_sb >= %s]",
            (long long)ld_sb, (long long)nrows_sb, b_kind == BS_SCALE_1X128 ? "N" : "N/128");
    REQUIRE(workspace_bytes >= 0, BS_ERR_LAYOUT, "workspace_bytes=%lld must be >= 0", (long long)workspace_bytes);
    REQUIRE(workspace || workspace_bytes == 0, BS_ERR_NULL, "workspace is NULL but workspace_bytes=%lld",
            (long long)workspace_bytes);
    REQUIRE(workspace == nullptr || ((reinterpret_cast<uintptr_t>(workspace) & 255u) == 0), BS_ERR_ALIGN,
            "workspace must be 256-byte aligned");
    if (M == 0 || N == 0) return ok();
    const bs::GemmArgs g = dense_args(M, N, K, a, lda, sa, ld_sa, b, ldb, sb, ld_sb, d, ldd);
    return hip_status(bs::launch_gemm_streamk(g, b_kind == BS_SCALE_1X128 ? bs::kScale1x128 : bs::kScale128x128,
                                              d_dtype == BS_OUT_F32, workspace, workspace_bytes, stream),
                      fn);
}

}  // extern "C"

// Device scratch of bs_scaled_mm_noalloc: one 256 x 256 fp32 partial tile
// per stream-K piece -- split tiles + splitting workgroups, at most
// 192 + 256 = 448 on a 256-CU GPU (a split last round is at most 3/4 full)
// -- 112 MiB per GPU, held until the process ends.  Host code never uses the
// array's name as an address: each device's copy is looked up once with
// hipGetSymbolAddress (scratch_on_device).
static constexpr int64_t kScratchBytes = (int64_t)448 * 256 * 256 * 4;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's scratch address (set up on the first call on the device,
// with that device current).
hipError_t scratch_on_device(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

bs_status bs_scaled_mm_noalloc(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, const float* sa,
                               int64_t ld_sa, bs_scale_kind a_kind, const uint8_t* b, int64_t ldb, const float* sb,
                               int64_t ld_sb, bs_scale_kind b_kind, void* d, int64_t ldd, bs_dtype d_dtype,
                               hipStream_t stream) {
    static const char* fn = "bs_scaled_mm_noalloc";
    REQUIRE(a_kind == BS_SCALE_1X128, BS_ERR_MODE, "a_kind=%d: A takes 1x128 scales (BS_SCALE_1X128 = 4)",
            (int)a_kind);
    bs_status st = check_gemm_common(fn, M, N, K, a, lda, sa, ld_sa, b, ldb, sb, ld_sb, b_kind, d, ldd, d_dtype);
    if (st != BS_OK) return st;
    REQUIRE(ld_sa >= M, BS_ERR_LAYOUT, "ld_sa=%lld < M=%lld: sa is K-major [K/128][ld_sa >= M]",
            (long long)ld_sa, (long long)M);
    const int64_t nrows_sb = b_kind == BS_SCALE_1X128 ? N : N / 128;
    REQUIRE(ld_sb >= nrows_sb, BS_ERR_LAYOUT, "ld_sb=%lld < %lld: sb is K-major [K/128][ld_sb >= %s]",
            (long long)ld_sb, (long long)nrows_sb, b_kind == BS_SCALE_1X128 ? "N" : "N/128");
    if (M == 0 || N == 0) return ok();
    const bs::GemmArgs g = dense_args(M, N, K, a, lda, sa, ld_sa, b, ldb, sb, ld_sb, d, ldd);
    const bs::ScaleMode sc = b_kind == BS_SCALE_1X128 ? bs::kScale1x128 : bs::kScale128x128;
    const int64_t need = bs::streamk_workspace_bytes(bs::plan_streamk(g, sc, d_dtype == BS_OUT_F32));
    REQUIRE(need <= kScratchBytes, BS_ERR_SHAPE,
            "the split of this problem needs %lld bytes of scratch; the static scratch holds %lld "
            "(use bs_scaled_mm_ws with a larger workspace)", (long long)need, (long long)kScratchBytes);
    if (need == 0) return hip_status(bs::launch_gemm(g, bs::kDense, sc, d_dtype == BS_OUT_F32, stream), fn);
    void* ws = nullptr;
    hipError_t e = scratch_on_device(&ws);
    if (e != hipSuccess) return fail(BS_ERR_HIP, fn, "device scratch lookup failed: %s", hipGetErrorString(e));
    return hip_status(bs::launch_gemm_streamk(g, sc, d_dtype == BS_OUT_F32, ws, kScratchBytes, stream), fn);
}

bs_status bs_grouped_scaled_mm(bs_group_mode mode, int64_t G, int64_t M, int64_t N, int64_t K,
                               const int32_t* group_end, const uint8_t* a, int64_t lda, const float* sa,
                               int64_t ld_sa, const uint8_t* b, int64_t stride_bg, int64_t ldb, const float* sb,
                               int64_t stride_sbg, int64_t ld_sb, bs_scale_kind b_kind, void* d, int64_t stride_dg,
                               int64_t ldd, bs_dtype d_dtype, hipStream_t stream) {
    static const char* fn = "bs_grouped_scaled_mm";
    REQUIRE(mode == BS_GROUP_M || mode == BS_GROUP_K, BS_ERR_MODE, "mode=%d must be BS_GROUP_M or BS_GROUP_K",
            (int)mode);
    REQUIRE(group_end, BS_ERR_NULL, "group_end is NULL");
    REQUIRE(G >= 0, BS_ERR_SHAPE, "G=%lld must be >= 0", (long long)G);
    bs_status st = check_gemm_common(fn, M, N, K, a, lda, sa, ld_sa, b, ldb, sb, ld_sb, b_kind, d, ldd, d_dtype);
    if (st != BS_OK) return st;
    REQUIRE(ld_sa >= M, BS_ERR_LAYOUT, "ld_sa=%lld < M=%lld: sa is K-major [K/128][ld_sa >= M]",
            (long long)ld_sa, (long long)M);
    bs::GemmArgs g{};
    g.M = M; g.N = N; g.K = K;
    g.a = a; g.lda = lda; g.sa = sa; g.ld_sa = ld_sa;
    g.b = b; g.ldb = ldb; g.sb = sb; g.ld_sb = ld_sb;
    g.d = d; g.ldd = ldd;
    g.G = G; g.group_end = group_end;
    g.tiles_n = (N + 255) / 256;
    if (mode == BS_GROUP_M) {
        REQUIRE(b_kind == BS_SCALE_128X128, BS_ERR_MODE,
                "BS_GROUP_M takes 128x128 expert-weight scales (b_kind = BS_SCALE_128X128)");
        REQUIRE(stride_dg == 0, BS_ERR_MODE, "BS_GROUP_M writes one D [M, N]: stride_dg must be 0");
        REQUIRE(ld_sb >= N / 128, BS_ERR_LAYOUT, "ld_sb=%lld < N/128: sb[g] is K-major [K/128][ld_sb >= N/128]",
                (long long)ld_sb);
        // Expert operands are inputs: their regions may interleave (e.g. the
        // scales of W quantized as one [G*N, K] matrix, stride_sbg = N/128).
        REQUIRE(stride_bg >= 0 && stride_sbg >= 0, BS_ERR_LAYOUT, "stride_bg and stride_sbg must be >= 0");
        REQUIRE(stride_bg % 16 == 0, BS_ERR_ALIGN, "stride_bg must be a multiple of 16 bytes");
        if (G == 0 || M == 0 || N == 0) return ok();
        g.stride_bg = stride_bg;
        g.stride_sbg = stride_sbg;
        g.tiles_m = (M + 255) / 256;
        g.num_tiles = (g.tiles_m + G) * g.tiles_n;  // upper bound on the sum of per-group tile rows
        return hip_status(bs::launch_gemm(g, bs::kGroupM, bs::kScale128x128, d_dtype == BS_OUT_F32, stream), fn);
    }
    REQUIRE(b_kind == BS_SCALE_1X128, BS_ERR_MODE,
            "BS_GROUP_K contracts two 1x128-scaled operands (b_kind = BS_SCALE_1X128)");
    REQUIRE(stride_bg == 0 && stride_sbg == 0, BS_ERR_MODE,
            "BS_GROUP_K shares one B over the groups: stride_bg and stride_sbg must be 0");
    REQUIRE(M % 128 == 0, BS_ERR_SHAPE, "M=%lld must be a multiple of 128 for BS_GROUP_K", (long long)M);
    REQUIRE(ld_sb >= N, BS_ERR_LAYOUT, "ld_sb=%lld < N=%lld: sb is K-major [K/128][ld_sb >= N]", (long long)ld_sb,
            (long long)N);
    REQUIRE(G <= 1 || stride_dg >= M * ldd, BS_ERR_LAYOUT, "stride_dg=%lld < M*ldd", (long long)stride_dg);
    REQUIRE(stride_dg % (d_dtype == BS_OUT_F32 ? 4 : 8) == 0, BS_ERR_ALIGN,
            "stride_dg must keep every D[g] 16-byte aligned");
    if (G == 0 || M == 0 || N == 0) return ok();
    g.stride_dg = stride_dg;
    g.tiles_m = (M + 255) / 256;
    g.num_tiles = G * g.tiles_m * g.tiles_n;
    return hip_status(bs::launch_gemm(g, bs::kGroupK, bs::kScale1x128, d_dtype == BS_OUT_F32, stream), fn);
}

bs_status bs_diag_e4m3_census(uint32_t* min_bits, uint32_t* max_bits, unsigned long long* counts,
                              hipStream_t stream) {
    static const char* fn = "bs_diag_e4m3_census";
    REQUIRE(min_bits && max_bits && counts, BS_ERR_NULL, "outputs must be non-NULL");
    return hip_status(bs::launch_diag_e4m3_census(min_bits, max_bits, counts, stream), fn);
}

bs_status bs_diag_stream(const void* src, int64_t n_read, void* dst, int64_t n_write, hipStream_t stream) {
    static const char* fn = "bs_diag_stream";
    REQUIRE((src && dst) || n_read == 0, BS_ERR_NULL, "src and dst must be non-NULL");
    REQUIRE(n_read >= 0 && n_write >= n_read, BS_ERR_SHAPE, "need 0 <= n_read <= n_write (got %lld, %lld)",
            (long long)n_read, (long long)n_write);
    REQUIRE(n_read % 16 == 0 && n_write % 16 == 0, BS_ERR_SHAPE, "n_read and n_write must be multiples of 16");
    REQUIRE(aligned16(src) && aligned16(dst), BS_ERR_ALIGN, "src and dst must be 16-byte aligned");
    if (n_read == 0) return ok();
    return hip_status(bs::launch_diag_stream(src, n_read, dst, n_write, stream), fn);
}

bs_status bs_diag_division(unsigned long long* result, hipStream_t stream) {
    static const char* fn = "bs_diag_division";
    REQUIRE(result, BS_ERR_NULL, "result must be non-NULL");
    return hip_status(bs::launch_diag_division(result, stream), fn);
}

}  // extern "C"
