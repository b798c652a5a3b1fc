// Drives every entry point of the C ABI (gq.h) on the host, with valid
// arguments (the launchers are counting stubs) and with each refusal, under
// AddressSanitizer and UndefinedBehaviorSanitizer.  Buffers are host memory
// standing in for device pointers: the ABI layer never dereferences them.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "gq.h"

extern int g_launches;
static int g_fail = 0;

#define CHECK(cond)                                                                               \
    do {                                                                                         \
        if (!(cond)) {                                                                           \
            fprintf(stderr, "%s:%d: check failed: %s (last error: %s)\n", __FILE__, __LINE__,    \
                    #cond, gq_last_error());                                                     \
            g_fail = 1;                                                                          \
        }                                                                                        \
    } while (0)

// a refused call launches nothing and names its reason
#define REFUSED(call, code)                                                                       \
    do {                                                                                         \
        const int before = g_launches;                                                           \
        const gq_status st = (call);                                                             \
        if (st != (code))                                                                        \
            fprintf(stderr, "status %d, expected %d\n", (int)st, (int)(code));                  \
        CHECK(st == (code));                                                                     \
        CHECK(g_launches == before);                                                             \
        CHECK(strlen(gq_last_error()) > 0);                                                      \
    } while (0)

#define LAUNCHED(call)                                                                            \
    do {                                                                                         \
        const int before = g_launches;                                                           \
        CHECK((call) == GQ_OK);                                                                  \
        CHECK(g_launches > before);                                                              \
    } while (0)

int main()
{
    alignas(256) static unsigned char buf[1 << 16];
    void *p = buf;
    void *mis = buf + 4; // 4-byte, not 16-byte, aligned
    const float *xf = (const float *)p;
    float *yf = (float *)(buf + 4096);
    const uint16_t *x16 = (const uint16_t *)p;
    uint16_t *y16 = (uint16_t *)(buf + 4096);

    // matrix-vector products
    LAUNCHED(gq_gemv_q4k(p, xf, yf, 64, 512, 1, nullptr));
    LAUNCHED(gq_gemv_q4k(p, xf, yf, 64, 512, 16, nullptr));
    LAUNCHED(gq_gemv_q4k(p, xf, yf, 64, 16640, 1, nullptr));
    LAUNCHED(gq_gemv_q8_0(p, xf, yf, 64, 96, 3, nullptr));
    CHECK(gq_gemv_q4k(p, xf, yf, 0, 512, 1, nullptr) == GQ_OK);
    REFUSED(gq_gemv_q4k(p, xf, yf, 64, 500, 1, nullptr), GQ_ESHAPE);
    REFUSED(gq_gemv_q4k(p, xf, yf, 64, 512, 17, nullptr), GQ_EINVAL);
    REFUSED(gq_gemv_q4k(nullptr, xf, yf, 64, 512, 1, nullptr), GQ_EINVAL);
    REFUSED(gq_gemv_q4k(mis, xf, yf, 64, 512, 1, nullptr), GQ_EALIGN);
    REFUSED(gq_gemv_q4k(p, xf, yf, -1, 512, 1, nullptr), GQ_EINVAL);
    REFUSED(gq_gemv_q8_0(p, xf, yf, 64, 100, 1, nullptr), GQ_ESHAPE);

    // multi-product tables
    std::vector<gq_gemv_desc> d(5);
    for (int i = 0; i < 5; ++i)
        d[i] = gq_gemv_desc{p, xf, yf, 17 + 100 * i, 256 * (i + 1)};
    const size_t tb = gq_gemv_q4k_multi_table_bytes(5);
    CHECK(tb > 0 && gq_gemv_q4k_multi_table_bytes(0) == 0);
    std::vector<unsigned char> table(tb);
    CHECK(gq_gemv_q4k_multi_plan(d.data(), 5, table.data(), tb) == GQ_OK);
    LAUNCHED(gq_gemv_q4k_multi(table.data(), p, nullptr));
    LAUNCHED(gq_gemv_q4k_multi_batched(table.data(), p, 4, nullptr));
    REFUSED(gq_gemv_q4k_multi_batched(table.data(), p, 17, nullptr), GQ_EINVAL);
    {
        const size_t nws = gq_gemv_q4k_multi_batched_ws_bytes(table.data(), 4);
        CHECK(nws > 0 && gq_gemv_q4k_multi_batched_ws_bytes(table.data(), 17) == 0);
        LAUNCHED(gq_gemv_q4k_multi_batched_ws(table.data(), p, 4, p, nws, nullptr));
        REFUSED(gq_gemv_q4k_multi_batched_ws(table.data(), p, 4, p, nws - 1, nullptr), GQ_EWORKSPACE);
        REFUSED(gq_gemv_q4k_multi_batched_ws(table.data(), p, 4, nullptr, nws, nullptr), GQ_EWORKSPACE);
    }
    REFUSED(gq_gemv_q4k_multi_plan(d.data(), 5, table.data(), tb - 1), GQ_EWORKSPACE);
    d[2].K = 16640; // above the one-launch limit
    REFUSED(gq_gemv_q4k_multi_plan(d.data(), 5, table.data(), tb), GQ_ESHAPE);
    d[2].K = 768;
    d[3].x = (const float *)mis;
    REFUSED(gq_gemv_q4k_multi_plan(d.data(), 5, table.data(), tb), GQ_EALIGN);
    std::vector<unsigned char> junk(tb, 0xAB);
    REFUSED(gq_gemv_q4k_multi(junk.data(), p, nullptr), GQ_EINVAL);
    LAUNCHED(gq_gemv_q4k_swiglu(p, p, xf, yf, 128, 4096, nullptr));
    REFUSED(gq_gemv_q4k_swiglu(p, p, xf, yf, 128, 32768, nullptr), GQ_ESHAPE);
    LAUNCHED(gq_gemv_q4k_swiglu_batched(p, p, xf, yf, 128, 4096, 4, nullptr));
    LAUNCHED(gq_gemv_q4k_swiglu_batched(p, p, xf, yf, 128, 4096, 1, nullptr));
    REFUSED(gq_gemv_q4k_swiglu_batched(p, p, xf, yf, 128, 4096, 17, nullptr), GQ_EINVAL);
    REFUSED(gq_gemv_q4k_swiglu_batched(p, p, xf, yf, 1 << 22, 16384, 2, nullptr), GQ_ESHAPE);

    // matrix products
    LAUNCHED(gq_gemm_q4k(p, x16, y16, 256, 1024, 512, nullptr));
    LAUNCHED(gq_gemm_q8_0(p, x16, y16, 256, 1024, 512, nullptr));
    LAUNCHED(gq_gemm_q4k_tiles(p, x16, y16, 256, 1024, 512, 128, nullptr));
    REFUSED(gq_gemm_q4k_tiles(p, x16, y16, 256, 1024, 512, 100, nullptr), GQ_EINVAL);
    LAUNCHED(gq_gemm_q8_0_tiles(p, x16, y16, 256, 1024, 512, 256, nullptr));
    LAUNCHED(gq_gemm_q8_0(p, x16, y16, 256, 1024, 128, nullptr)); // the K-group path
    LAUNCHED(gq_gemm_q8_0_tiles(p, x16, y16, 256, 320, 512, 64, nullptr));
    REFUSED(gq_gemm_q8_0_tiles(p, x16, y16, 256, 320, 512, 128, nullptr), GQ_ESHAPE);
    REFUSED(gq_gemm_q8_0_tiles(p, x16, y16, 256, 1024, 512, 100, nullptr), GQ_EINVAL);
    LAUNCHED(gq_gemm_q4k(p, x16, y16, 256, 1024, 128, nullptr)); // the K-group path
    LAUNCHED(gq_gemm_q4k_kgroups(p, x16, y16, 256, 1024, 512, 4, nullptr));
    LAUNCHED(gq_gemm_q4k_kgroups(p, x16, y16, 256, 512, 512, 2, nullptr));
    REFUSED(gq_gemm_q4k_kgroups(p, x16, y16, 256, 512, 512, 4, nullptr), GQ_ESHAPE);
    REFUSED(gq_gemm_q4k_kgroups(p, x16, y16, 256, 1024, 512, 3, nullptr), GQ_EINVAL);
    REFUSED(gq_gemm_q8_0(p, x16, y16, 256, 96, 512, nullptr), GQ_ESHAPE);
    const size_t wsb = gq_gemm_q4k_splitk_workspace_bytes(4096, 14336, 512, 8);
    CHECK(wsb == (size_t)8 * 512 * 4096 * 4);
    LAUNCHED(gq_gemm_q4k_splitk(p, x16, y16, 4096, 14336, 512, 8, p, wsb, nullptr));
    REFUSED(gq_gemm_q4k_splitk(p, x16, y16, 4096, 14336, 512, 8, p, wsb - 4, nullptr),
            GQ_EWORKSPACE);
    REFUSED(gq_gemm_q4k_splitk(p, x16, y16, 4096, 14336, 512, 5, p, wsb, nullptr), GQ_ESHAPE);
    LAUNCHED(gq_gemm_q4k_splitk_static(p, x16, y16, 4096, 14336, 512, 8, nullptr));
    REFUSED(gq_gemm_q4k_splitk_static(p, x16, y16, 4096, 14336, 4096, 8, nullptr),
            GQ_EWORKSPACE);
    CHECK(gq_gemm_q4k_splitk_static_max_bytes() == (size_t)64 << 20);

    // mixture of experts
    const int64_t T = 37, H = 512, I = 256, E = 8, k = 2;
    const size_t mwb = gq_moe_workspace_bytes(T, H, I, E, k);
    size_t off[7];
    CHECK(mwb > 0 && gq_moe_workspace_offsets(T, H, I, E, k, off) == GQ_OK);
    for (int i = 0; i < 7; ++i)
        CHECK(off[i] % 16 == 0 && off[i] <= mwb);
    std::vector<unsigned char> ws(mwb + 16);
    void *wsp = ws.data() + (16 - (uintptr_t)ws.data() % 16) % 16;
    LAUNCHED(gq_moe_gemm_q4k(p, p, p, x16, (const int32_t *)p, xf, y16, T, H, I, E, k, wsp, mwb,
                             nullptr));
    LAUNCHED(gq_moe_gemm_q4k_input_weighted(p, p, p, x16, (const int32_t *)p, xf, y16, T, H, I, E,
                                            k, wsp, mwb, nullptr));
    LAUNCHED(gq_moe_gemm_q8_0(p, p, p, x16, (const int32_t *)p, xf, y16, T, H, I, E, k, wsp, mwb,
                              nullptr));
    LAUNCHED(gq_moe_gemm_q8_0_input_weighted(p, p, p, x16, (const int32_t *)p, xf, y16, T, H, I, E,
                                             k, wsp, mwb, nullptr));
    REFUSED(gq_moe_gemm_q4k(p, p, p, x16, (const int32_t *)p, xf, y16, T, H, I, E, k, wsp, mwb - 1,
                            nullptr),
            GQ_EWORKSPACE);
    REFUSED(gq_moe_gemm_q4k(p, p, p, x16, (const int32_t *)p, xf, y16, T, H, I, E, E + 1, wsp,
                            mwb, nullptr),
            GQ_EINVAL);
    REFUSED(gq_moe_gemm_q4k(p, p, p, x16, (const int32_t *)p, xf, y16, T, 500, I, E, k, wsp, mwb,
                            nullptr),
            GQ_ESHAPE);
    LAUNCHED(gq_moe_route(xf, (int32_t *)yf, yf, T, 64, 8, 0, nullptr));
    REFUSED(gq_moe_route(xf, (int32_t *)yf, yf, T, 300, 8, 0, nullptr), GQ_EINVAL);
    CHECK(gq_moe_workspace_bytes(T, H, I, E, E + 1) == 0);

    // integer-dot path, dequantization probes, diagnostics
    LAUNCHED(gq_quantize_q8k(xf, (int8_t *)yf, yf, (int32_t *)yf, 5, 512, nullptr));
    LAUNCHED(gq_gemv_q4k_q8k(p, (const int8_t *)p, xf, (const int32_t *)p, yf, 64, 512, 7, nullptr));
    LAUNCHED(gq_gemm_q4k_q8k(p, (const int8_t *)p, xf, yf, 300, 1024, 200, nullptr));
    REFUSED(gq_gemm_q4k_q8k(p, (const int8_t *)p, xf, yf, 300, 1000, 200, nullptr), GQ_ESHAPE);
    REFUSED(gq_gemm_q4k_q8k(p, (const int8_t *)mis, xf, yf, 300, 1024, 200, nullptr), GQ_EALIGN);
    LAUNCHED(gq_dequant_q4k(p, yf, nullptr, 8, 512, nullptr));
    LAUNCHED(gq_dequant_q8_0(p, nullptr, y16, 8, 64, nullptr));
    REFUSED(gq_dequant_q4k(p, nullptr, nullptr, 8, 512, nullptr), GQ_EINVAL);
    for (int s = 0; s <= 6; ++s)
        CHECK(gq_status_str((gq_status)s) != nullptr);
    CHECK(gq_version() > 0);

    if (g_fail)
        return 1;
    printf("api driver: %d launches, all checks passed\n", g_launches);
    return 0;
}
