// gq_api.cpp -- the C ABI of libgq: argument checks, error reporting, launches.
//
// Every check runs on the host before anything is launched; a failed check
// returns its status and leaves a sentence naming the argument and the
// condition in a per-thread buffer.  Unsupported shapes are refused rather
// than computed on a subset (page "Frink Inference: the Rust alternative to
// llama.cpp", section "The goal, stated once", first point: load or refuse
// with a sentence naming what is missing, never compute something else).
#include "gq.h"

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "gq_internal.h"

namespace {

thread_local char g_err[512] = "";

gq_status fail(gq_status s, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

gq_status check_ptr(const char *fn, const char *name, const void *p)
{
    if (!p)
        return fail(GQ_EINVAL, "%s: %s is NULL", fn, name);
    if (!aligned16(p))
        return fail(GQ_EALIGN, "%s: %s (%p) is not 16-byte aligned", fn, name, p);
    return GQ_OK;
}

// Sizes the kernels index with 32-bit row/column counts.
constexpr int64_t kMaxDim = (int64_t)1 << 30;

gq_status check_dim(const char *fn, const char *name, int64_t v, bool allow_zero)
{
    if (v < 0 || (!allow_zero && v == 0))
        return fail(GQ_EINVAL, "%s: %s = %lld must be %s", fn, name, (long long)v,
                    allow_zero ? "non-negative" : "positive");
    if (v > kMaxDim)
        return fail(GQ_ESHAPE, "%s: %s = %lld exceeds the supported maximum %lld", fn, name,
                    (long long)v, (long long)kMaxDim);
    return GQ_OK;
}

gq_status check_k(const char *fn, const char *name, int64_t K, int64_t block)
{
    gq_status st = check_dim(fn, name, K, false);
    if (st != GQ_OK)
        return st;
    if (K % block != 0)
        return fail(GQ_ESHAPE, "%s: %s = %lld is not a multiple of the %lld-weight block", fn,
                    name, (long long)K, (long long)block);
    return GQ_OK;
}

gq_status launched(const char *fn, hipError_t e)
{
    if (e != hipSuccess)
        return fail(GQ_EHIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return GQ_OK;
}

#define GQ_TRY(expr)                                                                           \
    do {                                                                                       \
        gq_status st_ = (expr);                                                                \
        if (st_ != GQ_OK)                                                                      \
            return st_;                                                                        \
    } while (0)

gq_status gemv_checks(const char *fn, const void *w, const float *x, float *y, int64_t M,
                      int64_t K, int64_t B, int64_t block)
{
    GQ_TRY(check_dim(fn, "M", M, true));
    GQ_TRY(check_k(fn, "K", K, block));
    if (B < 0 || B > GQ_GEMV_MAX_BATCH)
        return fail(GQ_EINVAL, "%s: B = %lld is outside [0, %d]", fn, (long long)B,
                    GQ_GEMV_MAX_BATCH);
    if (M == 0 || B == 0)
        return GQ_OK;
    GQ_TRY(check_ptr(fn, "w", w));
    GQ_TRY(check_ptr(fn, "x", x));
    GQ_TRY(check_ptr(fn, "y", y));
    return GQ_OK;
}

constexpr size_t kAlign = 256;
size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

gq_status moe_layout(const char *fn, int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk,
                     size_t off[7])
{
    GQ_TRY(check_dim(fn, "T", T, true));
    GQ_TRY(check_k(fn, "H", H, 256));
    GQ_TRY(check_k(fn, "I", I, 256));
    if (E < 1 || E > 256)
        return fail(GQ_ESHAPE, "%s: E = %lld is outside the supported range [1, 256]", fn,
                    (long long)E);
    if (topk < 1 || topk > E)
        return fail(GQ_EINVAL, "%s: topk = %lld is outside [1, E = %lld]", fn, (long long)topk,
                    (long long)E);
    const int64_t A = T * topk;
    if (A > ((int64_t)1 << 20))
        return fail(GQ_ESHAPE, "%s: T*topk = %lld exceeds the supported maximum %lld", fn,
                    (long long)A, (long long)1 << 20);
    size_t o = 0;
    off[0] = o;
    o = up(o + (size_t)(E + 3) * 4);
    off[1] = o;
    o = up(o + (size_t)A * 4);
    off[2] = o;
    o = up(o + (size_t)A * 4);
    off[3] = o;
    o = up(o + (size_t)2 * (A + E) * 4);
    off[4] = o;
    o = up(o + (size_t)A * I * 2);
    off[5] = o;
    o = up(o + (size_t)A * H * 4);
    off[6] = o;
    return GQ_OK;
}

} // namespace

extern "C" {

gq_status gq_gemv_q8_0(const void *w, const float *x, float *y, int64_t M, int64_t K, int64_t B,
                       void *stream)
{
    static const char fn[] = "gq_gemv_q8_0";
    GQ_TRY(gemv_checks(fn, w, x, y, M, K, B, 32));
    if (M == 0 || B == 0)
        return GQ_OK;
    return launched(fn, gq::launch_gemv_q8_0(w, x, y, M, K, (int)B, (hipStream_t)stream));
}

// The matrix-core small-batch kernel addresses a matrix and its activations
// with 32-bit byte offsets.
static bool gemv_mfma_fits(int64_t M, int64_t K, int64_t B)
{
    return M * (K / 256) * 144 < ((int64_t)1 << 32) && B * K * 4 < ((int64_t)1 << 31);
}

gq_status gq_gemv_q4k(const void *w, const float *x, float *y, int64_t M, int64_t K, int64_t B,
                      void *stream)
{
    static const char fn[] = "gq_gemv_q4k";
    GQ_TRY(gemv_checks(fn, w, x, y, M, K, B, 256));
    if (M == 0 || B == 0)
        return GQ_OK;
    if (B == 1 && K <= gq::GemvStreamMaxK) {
        gq::GemvEntry e{(const uint8_t *)w, x, y, (int)M, (int)K, 0, 0};
        const long long total = (long long)M * gq::gemv_row_work(K);
        const int grid = gq::gemv_stream_grid(total, gq::gemv_stream_tiles(M, K));
        return launched(fn, gq::launch_gemv_stream(nullptr, e, 1, total, grid, (hipStream_t)stream));
    }
    // batch 2..16: whole-K blocks of 64 rows (the table kernel) once they
    // fill half the chip, else the K-split binary32 form, which is also
    // faster at batch 2, at batch 3-4 below 12288 rows (its one-tile
    // launches), and takes matrices past the table kernel's 32-bit offsets
    // (measured, kernel durations: 4096x14336 at batch 4 84 -> 29 us,
    // 4096x4096 25 -> 13 us, 14336x4096 at batch 2 26.9 -> 24.5 us,
    // 11008x4096 at batch 4 25.8 -> 23.2 us, 9216x4096 25.6 -> 22.5 us;
    // 14336x4096 at batch 4 26.5 us on the table kernel against 31.7)
    if (B >= 2) {
        if (B == 2 || M <= 32LL * gq::device_cus() || (B <= 4 && M < 12288) ||
            !gemv_mfma_fits(M, K, B))
            return launched(fn,
                            gq::launch_gemv_q4k_f32(w, x, y, M, K, (int)B, (hipStream_t)stream));
        gq::GemvEntry e{(const uint8_t *)w, x, y, (int)M, (int)K, 0, 0};
        const long long total = (long long)M * (K / 256) * 144;
        return launched(fn, gq::launch_gemv_mfma(nullptr, e, 1, total, gq::gemv_mfma_blocks(M, 1),
                                                 gq::gemv_mfma_blocks(M, 2),
                                                 gq::gemv_mfma_blocks(M, 3), (int)B,
                                                 (hipStream_t)stream));
    }
    return launched(fn, gq::launch_gemv_q4k(w, x, y, M, K, (int)B, (hipStream_t)stream));
}

// Table of a multi-product: a 40-byte header, then n entries laid out as
// gq::GemvEntry (48 bytes).  The same bytes are read on the host (checks, launch
// shape) and on the device (the kernel).
namespace {
constexpr uint32_t kTableMagic = 0x544D5147u; // "GQMT"
constexpr uint32_t kTableVersion = 2;
struct TableHeader {
    uint32_t magic, version;
    int64_t n;
    int64_t total_bytes; // weight bytes of all entries
    int64_t total_tiles;
    int64_t total_work; // gemv_row_work of all entries
};
static_assert(sizeof(TableHeader) == 40, "table header layout");
} // namespace

size_t gq_gemv_q4k_multi_table_bytes(int64_t n)
{
    if (n < 1 || n > ((int64_t)1 << 20))
        return 0;
    return sizeof(TableHeader) + (size_t)n * sizeof(gq::GemvEntry);
}

gq_status gq_gemv_q4k_multi_plan(const gq_gemv_desc *descs, int64_t n, void *table,
                                 size_t table_bytes)
{
    static const char fn[] = "gq_gemv_q4k_multi_plan";
    if (!descs)
        return fail(GQ_EINVAL, "%s: descs is NULL", fn);
    if (n < 1 || n > ((int64_t)1 << 20))
        return fail(GQ_EINVAL, "%s: n = %lld is outside [1, 2^20]", fn, (long long)n);
    if (!table)
        return fail(GQ_EINVAL, "%s: table is NULL", fn);
    if (table_bytes < gq_gemv_q4k_multi_table_bytes(n))
        return fail(GQ_EWORKSPACE, "%s: table_bytes = %zu is below the required %zu", fn,
                    table_bytes, gq_gemv_q4k_multi_table_bytes(n));
    int64_t total = 0, tiles = 0, work = 0;
    for (int64_t i = 0; i < n; ++i) {
        const gq_gemv_desc &d = descs[i];
        char name[64];
        snprintf(name, sizeof name, "descs[%lld].M", (long long)i);
        GQ_TRY(check_dim(fn, name, d.M, false));
        snprintf(name, sizeof name, "descs[%lld].K", (long long)i);
        GQ_TRY(check_k(fn, name, d.K, 256));
        if (d.K > gq::GemvStreamMaxK)
            return fail(GQ_ESHAPE, "%s: descs[%lld].K = %lld exceeds %d", fn, (long long)i,
                        (long long)d.K, gq::GemvStreamMaxK);
        snprintf(name, sizeof name, "descs[%lld].w", (long long)i);
        GQ_TRY(check_ptr(fn, name, d.w));
        snprintf(name, sizeof name, "descs[%lld].x", (long long)i);
        GQ_TRY(check_ptr(fn, name, d.x));
        snprintf(name, sizeof name, "descs[%lld].y", (long long)i);
        GQ_TRY(check_ptr(fn, name, d.y));
        total += d.M * (d.K / 256) * 144;
        work += d.M * gq::gemv_row_work(d.K);
        tiles += gq::gemv_stream_tiles(d.M, d.K);
    }
    TableHeader h{kTableMagic, kTableVersion, n, total, tiles, work};
    memcpy(table, &h, sizeof h);
    gq::GemvEntry *ent = reinterpret_cast<gq::GemvEntry *>((uint8_t *)table + sizeof h);
    int64_t begin = 0, wbegin = 0;
    for (int64_t i = 0; i < n; ++i) {
        const gq_gemv_desc &d = descs[i];
        gq::GemvEntry e{(const uint8_t *)d.w, d.x, d.y, (int)d.M, (int)d.K, begin, wbegin};
        memcpy(&ent[i], &e, sizeof e);
        begin += d.M * (d.K / 256) * 144;
        wbegin += d.M * gq::gemv_row_work(d.K);
    }
    return GQ_OK;
}

gq_status gq_gemv_q4k_multi(const void *table, const void *table_dev, void *stream)
{
    static const char fn[] = "gq_gemv_q4k_multi";
    if (!table)
        return fail(GQ_EINVAL, "%s: table is NULL", fn);
    TableHeader h;
    memcpy(&h, table, sizeof h);
    if (h.magic != kTableMagic || h.version != kTableVersion || h.n < 1)
        return fail(GQ_EINVAL, "%s: table was not written by gq_gemv_q4k_multi_plan", fn);
    GQ_TRY(check_ptr(fn, "table_dev", table_dev));
    const gq::GemvEntry *dev = reinterpret_cast<const gq::GemvEntry *>(
        (const uint8_t *)table_dev + sizeof(TableHeader));
    const gq::GemvEntry none{};
    const int grid = gq::gemv_stream_grid(h.total_work, h.total_tiles);
    return launched(fn, gq::launch_gemv_stream(dev, none, (int)h.n, h.total_work, grid,
                                               (hipStream_t)stream));
}

gq_status gq_gemv_q4k_multi_batched(const void *table, const void *table_dev, int64_t B,
                                    void *stream)
{
    static const char fn[] = "gq_gemv_q4k_multi_batched";
    if (!table)
        return fail(GQ_EINVAL, "%s: table is NULL", fn);
    TableHeader h;
    memcpy(&h, table, sizeof h);
    if (h.magic != kTableMagic || h.version != kTableVersion || h.n < 1)
        return fail(GQ_EINVAL, "%s: table was not written by gq_gemv_q4k_multi_plan", fn);
    if (B < 1 || B > GQ_GEMV_MAX_BATCH)
        return fail(GQ_EINVAL, "%s: B = %lld is outside [1, %d]", fn, (long long)B,
                    GQ_GEMV_MAX_BATCH);
    GQ_TRY(check_ptr(fn, "table_dev", table_dev));
    const gq::GemvEntry *dev = reinterpret_cast<const gq::GemvEntry *>(
        (const uint8_t *)table_dev + sizeof(TableHeader));
    const gq::GemvEntry none{};
    if (B == 1) {
        const int grid = gq::gemv_stream_grid(h.total_work, h.total_tiles);
        return launched(fn, gq::launch_gemv_stream(dev, none, (int)h.n, h.total_work, grid,
                                                   (hipStream_t)stream));
    }
    const gq::GemvEntry *ent =
        reinterpret_cast<const gq::GemvEntry *>((const uint8_t *)table + sizeof h);
    long long blocks1 = 0, blocks2 = 0, blocks3 = 0;
    for (int64_t i = 0; i < h.n; ++i) {
        gq::GemvEntry e;
        memcpy(&e, &ent[i], sizeof e);
        if (!gemv_mfma_fits(e.M, e.K, B))
            return fail(GQ_ESHAPE, "%s: entry %lld (M = %d, K = %d) is too large for batch %lld",
                        fn, (long long)i, e.M, e.K, (long long)B);
        blocks1 += gq::gemv_mfma_blocks(e.M, 1);
        blocks2 += gq::gemv_mfma_blocks(e.M, 2);
        blocks3 += gq::gemv_mfma_blocks(e.M, 3);
    }
    return launched(fn, gq::launch_gemv_mfma(dev, none, (int)h.n, h.total_bytes, blocks1, blocks2,
                                             blocks3,
                                             (int)B, (hipStream_t)stream));
}

// Table checks shared by the batched multi-product forms: header, B, every
// entry within the matrix-core path's limits; block and record counts.
static gq_status batched_table(const char *fn, const void *table, int64_t B, TableHeader &h,
                               long long &blocks1, long long &blocks2, long long &blocks3,
                               long long &records)
{
    if (!table)
        return fail(GQ_EINVAL, "%s: table is NULL", fn);
    memcpy(&h, table, sizeof h);
    if (h.magic != kTableMagic || h.version != kTableVersion || h.n < 1)
        return fail(GQ_EINVAL, "%s: table was not written by gq_gemv_q4k_multi_plan", fn);
    if (B < 1 || B > GQ_GEMV_MAX_BATCH)
        return fail(GQ_EINVAL, "%s: B = %lld is outside [1, %d]", fn, (long long)B,
                    GQ_GEMV_MAX_BATCH);
    const gq::GemvEntry *ent =
        reinterpret_cast<const gq::GemvEntry *>((const uint8_t *)table + sizeof h);
    blocks1 = blocks2 = blocks3 = records = 0;
    for (int64_t i = 0; i < h.n; ++i) {
        gq::GemvEntry e;
        memcpy(&e, &ent[i], sizeof e);
        if (B >= 2 && !gemv_mfma_fits(e.M, e.K, B))
            return fail(GQ_ESHAPE, "%s: entry %lld (M = %d, K = %d) is too large for batch %lld",
                        fn, (long long)i, e.M, e.K, (long long)B);
        blocks1 += gq::gemv_mfma_blocks(e.M, 1);
        blocks2 += gq::gemv_mfma_blocks(e.M, 2);
        blocks3 += gq::gemv_mfma_blocks(e.M, 3);
        records += e.K / 256;
    }
    return GQ_OK;
}

size_t gq_gemv_q4k_multi_batched_ws_bytes(const void *table, int64_t B)
{
    char saved[sizeof g_err];
    memcpy(saved, g_err, sizeof g_err);
    TableHeader h;
    long long b1 = 0, b2 = 0, b3 = 0, recs = 0;
    const gq_status st = batched_table("gq_gemv_q4k_multi_batched_ws_bytes", table, B, h, b1, b2,
                                       b3, recs);
    memcpy(g_err, saved, sizeof g_err);
    if (st != GQ_OK)
        return 0;
    if (B == 1)
        return 1; // no workspace used; 1 so that 0 keeps meaning "invalid"
    return (size_t)gq::gemv_mfma_prestaged_bytes(h.n, recs, (int)B);
}

gq_status gq_gemv_q4k_multi_batched_ws(const void *table, const void *table_dev, int64_t B,
                                       void *ws, size_t ws_bytes, void *stream)
{
    static const char fn[] = "gq_gemv_q4k_multi_batched_ws";
    TableHeader h;
    long long blocks1 = 0, blocks2 = 0, blocks3 = 0, records = 0;
    GQ_TRY(batched_table(fn, table, B, h, blocks1, blocks2, blocks3, records));
    GQ_TRY(check_ptr(fn, "table_dev", table_dev));
    if (B == 1)
        return gq_gemv_q4k_multi(table, table_dev, stream);
    const size_t need = (size_t)gq::gemv_mfma_prestaged_bytes(h.n, records, (int)B);
    if (!ws)
        return fail(GQ_EWORKSPACE, "%s: ws is NULL (needs %zu bytes)", fn, need);
    if (!aligned16(ws))
        return fail(GQ_EALIGN, "%s: ws (%p) is not 16-byte aligned", fn, ws);
    if (ws_bytes < need)
        return fail(GQ_EWORKSPACE, "%s: ws_bytes = %zu is below the required %zu", fn, ws_bytes,
                    need);
    if (records > ((long long)1 << 31) - 1)
        return fail(GQ_ESHAPE, "%s: %lld super-blocks in the table exceed 2^31", fn, records);
    const gq::GemvEntry *dev = reinterpret_cast<const gq::GemvEntry *>(
        (const uint8_t *)table_dev + sizeof(TableHeader));
    return launched(fn, gq::launch_gemv_mfma_prestaged(dev, (int)h.n, h.total_bytes, blocks1,
                                                       blocks2, blocks3, records, (int)B, ws,
                                                       (hipStream_t)stream));
}

static gq_status gemm_common(const char *fn, const void *w, const uint16_t *x, uint16_t *y,
                             int64_t M, int64_t K, int64_t N, int64_t tile_rows, bool q8,
                             void *stream)
{
    GQ_TRY(check_dim(fn, "M", M, true));
    // Q8_0: the small-tile kernel takes two blocks per step, the large tiles
    // whole runs of 256 weights
    GQ_TRY(check_k(fn, "K", K, q8 && (tile_rows == 0 || tile_rows == 64) ? 64 : 256));
    GQ_TRY(check_dim(fn, "N", N, true));
    if (N > ((int64_t)1 << 21))
        return fail(GQ_ESHAPE, "%s: N = %lld exceeds the supported maximum %lld", fn,
                    (long long)N, (long long)1 << 21);
    if (M == 0 || N == 0)
        return GQ_OK;
    GQ_TRY(check_ptr(fn, "w", w));
    GQ_TRY(check_ptr(fn, "x", x));
    GQ_TRY(check_ptr(fn, "y", y));
    if (tile_rows == 0) {
        // too few 256 x 256 tiles for the device: K groups where they are
        // estimated fastest
        const int kg = K % 256 == 0 ? gq::gemm_kgroups_choice(M, K, N) : 0;
        if (kg)
            return launched(fn, gq::launch_gemm_kgroups(w, x, y, M, K, N, kg, q8,
                                                        (hipStream_t)stream));
        tile_rows = K % 256 == 0 ? gq::gemm_big_choice(M, K, N) : 0;
    }
    if (tile_rows == 0 || tile_rows == 64)
        return launched(fn, q8 ? gq::launch_gemm_q8_0(w, x, y, M, K, N, (hipStream_t)stream)
                               : gq::launch_gemm_q4k(w, x, y, M, K, N, (hipStream_t)stream));
    if (!gq::gemm_big_fits(M, K, N))
        return fail(GQ_ESHAPE, "%s: N*K = %lld is too large for the %lld-row tiles", fn,
                    (long long)(N * K), (long long)tile_rows);
    return launched(fn, gq::launch_gemm_big(w, x, y, M, K, N, (int)tile_rows, q8,
                                            (hipStream_t)stream));
}

gq_status gq_gemm_q4k(const void *w, const uint16_t *x, uint16_t *y, int64_t M, int64_t K,
                      int64_t N, void *stream)
{
    return gemm_common("gq_gemm_q4k", w, x, y, M, K, N, 0, false, stream);
}

gq_status gq_gemm_q8_0(const void *w, const uint16_t *x, uint16_t *y, int64_t M, int64_t K,
                       int64_t N, void *stream)
{
    return gemm_common("gq_gemm_q8_0", w, x, y, M, K, N, 0, true, stream);
}

gq_status gq_gemm_q8_0_tiles(const void *w, const uint16_t *x, uint16_t *y, int64_t M, int64_t K,
                             int64_t N, int64_t tile_rows, void *stream)
{
    static const char fn[] = "gq_gemm_q8_0_tiles";
    if (tile_rows != 0 && tile_rows != 64 && tile_rows != 128 && tile_rows != 256)
        return fail(GQ_EINVAL, "%s: tile_rows = %lld must be 0, 64, 128 or 256", fn,
                    (long long)tile_rows);
    return gemm_common(fn, w, x, y, M, K, N, tile_rows, true, stream);
}

gq_status gq_gemm_q4k_tiles(const void *w, const uint16_t *x, uint16_t *y, int64_t M, int64_t K,
                            int64_t N, int64_t tile_rows, void *stream)
{
    static const char fn[] = "gq_gemm_q4k_tiles";
    if (tile_rows != 0 && tile_rows != 64 && tile_rows != 128 && tile_rows != 256)
        return fail(GQ_EINVAL, "%s: tile_rows = %lld must be 0, 64, 128 or 256", fn,
                    (long long)tile_rows);
    return gemm_common(fn, w, x, y, M, K, N, tile_rows, false, stream);
}

gq_status gq_gemm_q4k_kgroups(const void *w, const uint16_t *x, uint16_t *y, int64_t M, int64_t K,
                              int64_t N, int64_t groups, void *stream)
{
    static const char fn[] = "gq_gemm_q4k_kgroups";
    GQ_TRY(check_dim(fn, "M", M, true));
    GQ_TRY(check_k(fn, "K", K, 256));
    GQ_TRY(check_dim(fn, "N", N, true));
    if (groups != 2 && groups != 4)
        return fail(GQ_EINVAL, "%s: groups = %lld must be 2 or 4", fn, (long long)groups);
    if ((K / 256) % groups != 0)
        return fail(GQ_ESHAPE, "%s: groups = %lld does not divide the %lld super-blocks of K", fn,
                    (long long)groups, (long long)(K / 256));
    if (N > ((int64_t)1 << 21) || !gq::gemm_big_fits(M > 0 ? M : 1, K, N > 0 ? N : 1))
        return fail(GQ_ESHAPE, "%s: N*K = %lld is too large for the large tiles", fn,
                    (long long)(N * K));
    if (M == 0 || N == 0)
        return GQ_OK;
    GQ_TRY(check_ptr(fn, "w", w));
    GQ_TRY(check_ptr(fn, "x", x));
    GQ_TRY(check_ptr(fn, "y", y));
    return launched(fn, gq::launch_gemm_kgroups(w, x, y, M, K, N, (int)groups, false,
                                                (hipStream_t)stream));
}

// Split count of the split-K product: `splits` as given, or the automatic choice.
static gq_status splitk_count(const char *fn, int64_t M, int64_t K, int64_t N, int64_t splits,
                              int *out)
{
    GQ_TRY(check_dim(fn, "M", M, false));
    GQ_TRY(check_k(fn, "K", K, 256));
    GQ_TRY(check_dim(fn, "N", N, false));
    if (!gq::gemm_big_fits(M, K, N) || M * (K / 256) * 144 >= ((int64_t)1 << 32))
        return fail(GQ_ESHAPE, "%s: M = %lld, K = %lld, N = %lld is too large for the split tiles",
                    fn, (long long)M, (long long)K, (long long)N);
    if (splits == 0)
        splits = gq::gemm_splitk_choice(M, K, N);
    if (splits < 1 || splits > 64)
        return fail(GQ_EINVAL, "%s: splits = %lld is outside [1, 64] (0: automatic)", fn,
                    (long long)splits);
    if ((K / 256) % splits != 0)
        return fail(GQ_ESHAPE, "%s: splits = %lld does not divide the %lld super-blocks of K", fn,
                    (long long)splits, (long long)(K / 256));
    *out = (int)splits;
    return GQ_OK;
}

size_t gq_gemm_q4k_splitk_workspace_bytes(int64_t M, int64_t K, int64_t N, int64_t splits)
{
    char saved[sizeof g_err];
    memcpy(saved, g_err, sizeof g_err);
    int s = 0;
    const gq_status st = splitk_count("gq_gemm_q4k_splitk_workspace_bytes", M, K, N, splits, &s);
    memcpy(g_err, saved, sizeof g_err);
    if (st != GQ_OK)
        return 0;
    return (size_t)s * (size_t)N * (size_t)M * sizeof(float);
}

gq_status gq_gemm_q4k_splitk(const void *w, const uint16_t *x, uint16_t *y, int64_t M, int64_t K,
                             int64_t N, int64_t splits, void *ws, size_t ws_bytes, void *stream)
{
    static const char fn[] = "gq_gemm_q4k_splitk";
    int s = 0;
    GQ_TRY(splitk_count(fn, M, K, N, splits, &s));
    GQ_TRY(check_ptr(fn, "w", w));
    GQ_TRY(check_ptr(fn, "x", x));
    GQ_TRY(check_ptr(fn, "y", y));
    const size_t need = (size_t)s * (size_t)N * (size_t)M * sizeof(float);
    if (!ws)
        return fail(GQ_EWORKSPACE, "%s: ws is NULL (needs %zu bytes)", fn, need);
    if (!aligned16(ws))
        return fail(GQ_EALIGN, "%s: ws (%p) is not 16-byte aligned", fn, ws);
    if (ws_bytes < need)
        return fail(GQ_EWORKSPACE, "%s: ws_bytes = %zu is below the required %zu (splits = %d)", fn,
                    ws_bytes, need, s);
    return launched(fn, gq::launch_gemm_splitk(w, x, y, M, K, N, s, (float *)ws,
                                               (hipStream_t)stream));
}

gq_status gq_gemm_q4k_splitk_static(const void *w, const uint16_t *x, uint16_t *y, int64_t M,
                                    int64_t K, int64_t N, int64_t splits, void *stream)
{
    static const char fn[] = "gq_gemm_q4k_splitk_static";
    int s = 0;
    GQ_TRY(splitk_count(fn, M, K, N, splits, &s));
    GQ_TRY(check_ptr(fn, "w", w));
    GQ_TRY(check_ptr(fn, "x", x));
    GQ_TRY(check_ptr(fn, "y", y));
    const size_t need = (size_t)s * (size_t)N * (size_t)M * sizeof(float);
    if (need > gq::kSplitkScratchBytes)
        return fail(GQ_EWORKSPACE,
                    "%s: %d runs of binary32 partials need %zu bytes, above the static scratch "
                    "of %zu bytes (fewer splits, or gq_gemm_q4k_splitk with a workspace)",
                    fn, s, need, gq::kSplitkScratchBytes);
    float *ws = nullptr;
    const hipError_t e = gq::splitk_scratch(&ws);
    if (e != hipSuccess)
        return fail(GQ_EHIP, "%s: device address of the static scratch: %s", fn,
                    hipGetErrorString(e));
    return launched(fn, gq::launch_gemm_splitk(w, x, y, M, K, N, s, ws, (hipStream_t)stream));
}

size_t gq_gemm_q4k_splitk_static_max_bytes(void) { return gq::kSplitkScratchBytes; }

size_t gq_moe_workspace_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk)
{
    size_t off[7];
    char saved[sizeof g_err];
    memcpy(saved, g_err, sizeof g_err);
    const gq_status st = moe_layout("gq_moe_workspace_bytes", T, H, I, E, topk, off);
    if (st != GQ_OK)
        return 0;
    memcpy(g_err, saved, sizeof g_err);
    return off[6];
}

gq_status gq_moe_workspace_offsets(int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk,
                                   size_t off[7])
{
    if (!off)
        return fail(GQ_EINVAL, "gq_moe_workspace_offsets: off is NULL");
    return moe_layout("gq_moe_workspace_offsets", T, H, I, E, topk, off);
}

static gq_status moe_common(const char *fn, const void *w_gate, const void *w_up,
                            const void *w_down, const uint16_t *x, const int32_t *topk_ids,
                            const float *topk_w, uint16_t *out, int64_t T, int64_t H, int64_t I,
                            int64_t E, int64_t topk, void *ws, size_t ws_bytes, void *stream,
                            int weight_input, int q8_0)
{
    gq::MoeArgs a;
    a.weight_input = weight_input;
    a.q8_0 = q8_0;
    GQ_TRY(moe_layout(fn, T, H, I, E, topk, a.off));
    if (T == 0)
        return GQ_OK;
    GQ_TRY(check_ptr(fn, "w_gate", w_gate));
    GQ_TRY(check_ptr(fn, "w_up", w_up));
    GQ_TRY(check_ptr(fn, "w_down", w_down));
    GQ_TRY(check_ptr(fn, "x", x));
    GQ_TRY(check_ptr(fn, "topk_ids", topk_ids));
    GQ_TRY(check_ptr(fn, "topk_w", topk_w));
    GQ_TRY(check_ptr(fn, "out", out));
    if (!ws)
        return fail(GQ_EWORKSPACE, "%s: ws is NULL (needs %zu bytes)", fn, a.off[6]);
    if (!aligned16(ws))
        return fail(GQ_EALIGN, "%s: ws (%p) is not 16-byte aligned", fn, ws);
    if (ws_bytes < a.off[6])
        return fail(GQ_EWORKSPACE, "%s: ws_bytes = %zu is below the required %zu", fn, ws_bytes,
                    a.off[6]);
    a.w_gate = (const uint8_t *)w_gate;
    a.w_up = (const uint8_t *)w_up;
    a.w_down = (const uint8_t *)w_down;
    a.x = x;
    a.ids = topk_ids;
    a.wts = topk_w;
    a.out = out;
    a.T = T;
    a.H = H;
    a.I = I;
    a.E = E;
    a.topk = topk;
    a.ws = (uint8_t *)ws;
    return launched(fn, gq::launch_moe(a, (hipStream_t)stream));
}

gq_status gq_moe_gemm_q4k(const void *w_gate, const void *w_up, const void *w_down,
                          const uint16_t *x, const int32_t *topk_ids, const float *topk_w,
                          uint16_t *out, int64_t T, int64_t H, int64_t I, int64_t E,
                          int64_t topk, void *ws, size_t ws_bytes, void *stream)
{
    return moe_common("gq_moe_gemm_q4k", w_gate, w_up, w_down, x, topk_ids, topk_w, out, T, H, I,
                      E, topk, ws, ws_bytes, stream, 0, 0);
}

gq_status gq_moe_gemm_q4k_input_weighted(const void *w_gate, const void *w_up,
                                         const void *w_down, const uint16_t *x,
                                         const int32_t *topk_ids, const float *topk_w,
                                         uint16_t *out, int64_t T, int64_t H, int64_t I,
                                         int64_t E, int64_t topk, void *ws, size_t ws_bytes,
                                         void *stream)
{
    return moe_common("gq_moe_gemm_q4k_input_weighted", w_gate, w_up, w_down, x, topk_ids, topk_w,
                      out, T, H, I, E, topk, ws, ws_bytes, stream, 1, 0);
}

gq_status gq_moe_gemm_q8_0(const void *w_gate, const void *w_up, const void *w_down,
                           const uint16_t *x, const int32_t *topk_ids, const float *topk_w,
                           uint16_t *out, int64_t T, int64_t H, int64_t I, int64_t E,
                           int64_t topk, void *ws, size_t ws_bytes, void *stream)
{
    return moe_common("gq_moe_gemm_q8_0", w_gate, w_up, w_down, x, topk_ids, topk_w, out, T, H, I,
                      E, topk, ws, ws_bytes, stream, 0, 1);
}

gq_status gq_moe_gemm_q8_0_input_weighted(const void *w_gate, const void *w_up,
                                          const void *w_down, const uint16_t *x,
                                          const int32_t *topk_ids, const float *topk_w,
                                          uint16_t *out, int64_t T, int64_t H, int64_t I,
                                          int64_t E, int64_t topk, void *ws, size_t ws_bytes,
                                          void *stream)
{
    return moe_common("gq_moe_gemm_q8_0_input_weighted", w_gate, w_up, w_down, x, topk_ids,
                      topk_w, out, T, H, I, E, topk, ws, ws_bytes, stream, 1, 1);
}

gq_status gq_gemv_q4k_swiglu(const void *w_gate, const void *w_up, const float *x, float *h,
                             int64_t M, int64_t K, void *stream)
{
    static const char fn[] = "gq_gemv_q4k_swiglu";
    GQ_TRY(check_dim(fn, "M", M, true));
    GQ_TRY(check_k(fn, "K", K, 256));
    if (K > gq::GemvStreamMaxK)
        return fail(GQ_ESHAPE, "%s: K = %lld exceeds %d", fn, (long long)K, gq::GemvStreamMaxK);
    if (M > ((int64_t)1 << 29))
        return fail(GQ_ESHAPE, "%s: M = %lld exceeds 2^29 rows", fn, (long long)M);
    if (M == 0)
        return GQ_OK;
    GQ_TRY(check_ptr(fn, "w_gate", w_gate));
    GQ_TRY(check_ptr(fn, "w_up", w_up));
    GQ_TRY(check_ptr(fn, "x", x));
    GQ_TRY(check_ptr(fn, "h", h));
    return launched(fn, gq::launch_gemv_swiglu(w_gate, w_up, x, h, M, K, (hipStream_t)stream));
}

gq_status gq_gemv_q4k_swiglu_batched(const void *w_gate, const void *w_up, const float *x,
                                     float *h, int64_t M, int64_t K, int64_t B, void *stream)
{
    static const char fn[] = "gq_gemv_q4k_swiglu_batched";
    GQ_TRY(check_dim(fn, "M", M, true));
    GQ_TRY(check_k(fn, "K", K, 256));
    if (B < 1 || B > 16)
        return fail(GQ_EINVAL, "%s: B = %lld is outside [1, 16]", fn, (long long)B);
    if (B == 1)
        return gq_gemv_q4k_swiglu(w_gate, w_up, x, h, M, K, stream);
    if (!gemv_mfma_fits(M, K, B))
        return fail(GQ_ESHAPE, "%s: M = %lld, K = %lld is too large for batch %lld", fn,
                    (long long)M, (long long)K, (long long)B);
    if (M == 0)
        return GQ_OK;
    GQ_TRY(check_ptr(fn, "w_gate", w_gate));
    GQ_TRY(check_ptr(fn, "w_up", w_up));
    GQ_TRY(check_ptr(fn, "x", x));
    GQ_TRY(check_ptr(fn, "h", h));
    return launched(fn, gq::launch_gemv_swiglu_mfma(w_gate, w_up, x, h, M, K, (int)B,
                                                    (hipStream_t)stream));
}

gq_status gq_moe_route(const float *logits, int32_t *topk_ids, float *topk_w, int64_t T,
                       int64_t E, int64_t topk, int64_t renormalize, void *stream)
{
    static const char fn[] = "gq_moe_route";
    GQ_TRY(check_dim(fn, "T", T, true));
    if (E < 1 || E > 256)
        return fail(GQ_EINVAL, "%s: E = %lld is outside [1, 256]", fn, (long long)E);
    if (topk < 1 || topk > E)
        return fail(GQ_EINVAL, "%s: topk = %lld is outside [1, E = %lld]", fn, (long long)topk,
                    (long long)E);
    if (T > ((int64_t)1 << 24))
        return fail(GQ_ESHAPE, "%s: T = %lld exceeds 2^24 tokens", fn, (long long)T);
    if (T == 0)
        return GQ_OK;
    GQ_TRY(check_ptr(fn, "logits", logits));
    GQ_TRY(check_ptr(fn, "topk_ids", topk_ids));
    GQ_TRY(check_ptr(fn, "topk_w", topk_w));
    return launched(fn, gq::launch_moe_route(logits, topk_ids, topk_w, T, E, topk,
                                             renormalize != 0, (hipStream_t)stream));
}

gq_status gq_quantize_q8k(const float *x, int8_t *q, float *d, int32_t *bsum, int64_t B,
                          int64_t K, void *stream)
{
    static const char fn[] = "gq_quantize_q8k";
    GQ_TRY(check_dim(fn, "B", B, true));
    GQ_TRY(check_k(fn, "K", K, 256));
    if (B * K > ((int64_t)1 << 34))
        return fail(GQ_ESHAPE, "%s: B*K = %lld exceeds 2^34 activations", fn, (long long)(B * K));
    if (B == 0)
        return GQ_OK;
    GQ_TRY(check_ptr(fn, "x", x));
    GQ_TRY(check_ptr(fn, "q", q));
    GQ_TRY(check_ptr(fn, "d", d));
    GQ_TRY(check_ptr(fn, "bsum", bsum));
    return launched(fn, gq::launch_quantize_q8k(x, q, d, bsum, B, K, (hipStream_t)stream));
}

gq_status gq_gemv_q4k_q8k(const void *w, const int8_t *q, const float *d, const int32_t *bsum,
                          float *y, int64_t M, int64_t K, int64_t B, void *stream)
{
    static const char fn[] = "gq_gemv_q4k_q8k";
    GQ_TRY(check_dim(fn, "M", M, true));
    GQ_TRY(check_k(fn, "K", K, 256));
    if (B < 0 || B > GQ_GEMV_MAX_BATCH)
        return fail(GQ_EINVAL, "%s: B = %lld is outside [0, %d]", fn, (long long)B,
                    GQ_GEMV_MAX_BATCH);
    if (M == 0 || B == 0)
        return GQ_OK;
    GQ_TRY(check_ptr(fn, "w", w));
    GQ_TRY(check_ptr(fn, "q", q));
    GQ_TRY(check_ptr(fn, "d", d));
    GQ_TRY(check_ptr(fn, "bsum", bsum));
    GQ_TRY(check_ptr(fn, "y", y));
    return launched(fn, gq::launch_gemv_q4k_q8k(w, q, d, bsum, y, M, K, (int)B,
                                                (hipStream_t)stream));
}

gq_status gq_gemm_q4k_q8k(const void *w, const int8_t *q, const float *d, float *y, int64_t M,
                          int64_t K, int64_t N, void *stream)
{
    static const char fn[] = "gq_gemm_q4k_q8k";
    GQ_TRY(check_dim(fn, "M", M, true));
    GQ_TRY(check_k(fn, "K", K, 256));
    GQ_TRY(check_dim(fn, "N", N, true));
    if (M * (K / 256) * 144 >= ((int64_t)1 << 40) || N * K > ((int64_t)1 << 34) ||
        (M + 127) / 128 * ((N + 63) / 64) > 0x7fffffff || M > 0x7fffffff || N > 0x7fffffff)
        return fail(GQ_ESHAPE, "%s: M = %lld, K = %lld, N = %lld is too large", fn, (long long)M,
                    (long long)K, (long long)N);
    if (M == 0 || N == 0)
        return GQ_OK;
    GQ_TRY(check_ptr(fn, "w", w));
    GQ_TRY(check_ptr(fn, "q", q));
    GQ_TRY(check_ptr(fn, "d", d));
    GQ_TRY(check_ptr(fn, "y", y));
    return launched(fn, gq::launch_gemm_q4k_q8k(w, q, d, y, M, K, N, (hipStream_t)stream));
}

gq_status gq_dequant_q8_0(const void *w, float *out32, uint16_t *out16, int64_t M, int64_t K,
                          void *stream)
{
    static const char fn[] = "gq_dequant_q8_0";
    GQ_TRY(check_dim(fn, "M", M, true));
    GQ_TRY(check_k(fn, "K", K, 32));
    if (M == 0)
        return GQ_OK;
    GQ_TRY(check_ptr(fn, "w", w));
    if (!out32 && !out16)
        return fail(GQ_EINVAL, "%s: out32 and out16 are both NULL", fn);
    if (out32)
        GQ_TRY(check_ptr(fn, "out32", out32));
    if (out16)
        GQ_TRY(check_ptr(fn, "out16", out16));
    return launched(fn, gq::launch_dequant_q8_0(w, out32, out16, M, K, (hipStream_t)stream));
}

gq_status gq_dequant_q4k(const void *w, float *out32, uint16_t *out16, int64_t M, int64_t K,
                         void *stream)
{
    static const char fn[] = "gq_dequant_q4k";
    GQ_TRY(check_dim(fn, "M", M, true));
    GQ_TRY(check_k(fn, "K", K, 256));
    if (M == 0)
        return GQ_OK;
    GQ_TRY(check_ptr(fn, "w", w));
    if (!out32 && !out16)
        return fail(GQ_EINVAL, "%s: out32 and out16 are both NULL", fn);
    if (out32)
        GQ_TRY(check_ptr(fn, "out32", out32));
    if (out16)
        GQ_TRY(check_ptr(fn, "out16", out16));
    return launched(fn, gq::launch_dequant_q4k(w, out32, out16, M, K, (hipStream_t)stream));
}

const char *gq_last_error(void) { return g_err; }

const char *gq_status_str(gq_status s)
{
    switch (s) {
    case GQ_OK: return "GQ_OK";
    case GQ_EINVAL: return "GQ_EINVAL";
    case GQ_ESHAPE: return "GQ_ESHAPE";
    case GQ_EALIGN: return "GQ_EALIGN";
    case GQ_EWORKSPACE: return "GQ_EWORKSPACE";
    case GQ_EHIP: return "GQ_EHIP";
    }
    return "GQ_UNKNOWN";
}

int gq_version(void) { return 100; }

} // extern "C"
