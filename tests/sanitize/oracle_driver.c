/* Runs every function of the C oracle on small random inputs, exact-size
 * buffers, under AddressSanitizer and UndefinedBehaviorSanitizer; checks a few
 * identities on the way (fused product equals dequantize-then-dot, one-hot
 * reads a column, binary16 round trip). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

double orc_half_to_double(uint16_t h);
uint16_t orc_double_to_half(double v);
void orc_half_array_to_double(const uint16_t *h, int64_t n, double *out);
void orc_double_array_to_half(const double *v, int64_t n, uint16_t *out);
void orc_q4k_fields(const uint8_t *blk, double *d, double *dmin, int32_t *sc, int32_t *m, int32_t *q);
void orc_dequant(int fmt, const uint8_t *w, int64_t M, int64_t K, float *out32, uint16_t *out16);
void orc_gemv(int fmt, const uint8_t *w, const float *x, int64_t M, int64_t K, int64_t B,
              const int64_t *rows, int64_t nr, double *y, double *S);
void orc_gemv_separate(int fmt, const uint8_t *w, const float *x, int64_t M, int64_t K, int64_t B,
                       double *y);
void orc_gemm(int fmt, const uint8_t *w, const uint16_t *x16, int64_t M, int64_t K, int64_t N,
              const int64_t *rows, int64_t nrows, const int64_t *toks, int64_t ntoks, double *y,
              double *S);
void orc_moe_route(const float *logits, int64_t T, int64_t E, int64_t topk, int32_t *ids,
                   double *wts, int renorm);
void orc_swiglu(const double *g, const double *u, int64_t n, double *h);
void orc_moe_ffn(int fmt, const uint8_t *w_gate, const uint8_t *w_up, const uint8_t *w_down,
                 const uint16_t *x16, const int32_t *ids, const float *wts, int64_t T, int64_t H,
                 int64_t I, int64_t E, int64_t topk, double *g, double *u, double *h, double *d,
                 double *out, double *Sg, double *Su, double *Sd, int weight_input);
void orc_quantize_q8k(const float *x, int64_t B, int64_t K, int8_t *q, float *d, int32_t *bsum);
void orc_gemv_q4k_q8k(const uint8_t *w, const int8_t *q, const float *d, int64_t M, int64_t K,
                      int64_t B, const int64_t *rows, int64_t nr, double *y, double *S);
void orc_q4k_terms(const uint8_t *w, int64_t M, int64_t K, double *a, double *c);

static uint64_t st = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void)
{
    st ^= st << 13;
    st ^= st >> 7;
    st ^= st << 17;
    return (uint32_t)(st >> 16);
}
static float nrm(void) { return ((float)(rnd() % 20001) - 10000.f) / 5000.f; }

static void *xmalloc(size_t n)
{
    void *p = malloc(n ? n : 1);
    if (!p)
        exit(2);
    return p;
}

/* packed weights with small finite binary16 scales */
static uint8_t *weights(int fmt, int64_t M, int64_t K)
{
    const int64_t bb = fmt == 0 ? 34 : 144, wb = fmt == 0 ? 32 : 256;
    const int64_t n = M * (K / wb);
    uint8_t *w = (uint8_t *)xmalloc((size_t)(n * bb));
    for (int64_t i = 0; i < n * bb; i++)
        w[i] = (uint8_t)rnd();
    for (int64_t b = 0; b < n; b++) {
        const uint16_t d = orc_double_to_half(1e-3 * (1 + rnd() % 1000) / 500.0);
        w[b * bb] = (uint8_t)d;
        w[b * bb + 1] = (uint8_t)(d >> 8);
        if (fmt == 1) {
            const uint16_t dm = orc_double_to_half(1e-3 * (1 + rnd() % 1000) / 500.0);
            w[b * bb + 2] = (uint8_t)dm;
            w[b * bb + 3] = (uint8_t)(dm >> 8);
        }
    }
    return w;
}

int main(void)
{
    int fail = 0;
    for (uint32_t h = 0; h < 65536; h++) {
        const double v = orc_half_to_double((uint16_t)h);
        if (v == v && orc_double_to_half(v) != h && !(v == 0.0))
            fail = 1;
    }
    for (int fmt = 0; fmt < 2; fmt++) {
        const int64_t M = 7, K = 512, B = 3, N = 5;
        uint8_t *w = weights(fmt, M, K);
        float *x = (float *)xmalloc(sizeof(float) * B * K);
        uint16_t *x16 = (uint16_t *)xmalloc(2 * N * K);
        for (int64_t i = 0; i < B * K; i++)
            x[i] = nrm();
        for (int64_t i = 0; i < N * K; i++)
            x16[i] = orc_double_to_half(nrm());
        float *w32 = (float *)xmalloc(sizeof(float) * M * K);
        uint16_t *w16 = (uint16_t *)xmalloc(2 * M * K);
        orc_dequant(fmt, w, M, K, w32, w16);
        double *y = (double *)xmalloc(sizeof(double) * B * M), *S = (double *)xmalloc(sizeof(double) * B * M);
        double *y2 = (double *)xmalloc(sizeof(double) * B * M);
        orc_gemv(fmt, w, x, M, K, B, NULL, M, y, S);
        orc_gemv_separate(fmt, w, x, M, K, B, y2);
        for (int64_t i = 0; i < B * M; i++)
            if (y[i] != y2[i])
                fail = 1;
        const int64_t rows[2] = {6, 1}, toks[3] = {4, 0, 2};
        double *yr = (double *)xmalloc(sizeof(double) * B * 2), *Sr = (double *)xmalloc(sizeof(double) * B * 2);
        orc_gemv(fmt, w, x, M, K, B, rows, 2, yr, Sr);
        double *yg = (double *)xmalloc(sizeof(double) * 3 * 2), *Sg = (double *)xmalloc(sizeof(double) * 3 * 2);
        orc_gemm(fmt, w, x16, M, K, N, rows, 2, toks, 3, yg, Sg);
        /* one-hot column */
        float *oh = (float *)xmalloc(sizeof(float) * K);
        for (int64_t k = 0; k < K; k++)
            oh[k] = k == 77 ? 1.f : 0.f;
        orc_gemv(fmt, w, oh, M, K, 1, NULL, M, y, S);
        for (int64_t r = 0; r < M; r++)
            if (y[r] != (double)w32[r * K + 77])
                fail = 1;
        free(oh); free(yg); free(Sg); free(yr); free(Sr);
        free(y); free(y2); free(S); free(w16); free(w32); free(x16); free(x); free(w);
    }
    {
        const int64_t M = 5, K = 768, B = 4;
        uint8_t *w = weights(1, M, K);
        double dd, dm;
        int32_t sc[8], m[8], q[256];
        orc_q4k_fields(w, &dd, &dm, sc, m, q);
        float *x = (float *)xmalloc(sizeof(float) * B * K);
        for (int64_t i = 0; i < B * K; i++)
            x[i] = nrm();
        int8_t *qq = (int8_t *)xmalloc(B * K);
        float *d = (float *)xmalloc(sizeof(float) * B * (K / 256));
        int32_t *bs = (int32_t *)xmalloc(sizeof(int32_t) * B * (K / 32));
        orc_quantize_q8k(x, B, K, qq, d, bs);
        double *y = (double *)xmalloc(sizeof(double) * B * M), *S = (double *)xmalloc(sizeof(double) * B * M);
        orc_gemv_q4k_q8k(w, qq, d, M, K, B, NULL, M, y, S);
        double *a = (double *)xmalloc(sizeof(double) * M * K), *c = (double *)xmalloc(sizeof(double) * M * K);
        orc_q4k_terms(w, M, K, a, c);
        free(a); free(c); free(y); free(S); free(bs); free(d); free(qq); free(x); free(w);
    }
    {
        const int64_t T = 6, E = 8, k = 3, H = 256, I = 256;
        float *lg = (float *)xmalloc(sizeof(float) * T * E);
        for (int64_t i = 0; i < T * E; i++)
            lg[i] = nrm();
        int32_t *ids = (int32_t *)xmalloc(sizeof(int32_t) * T * k);
        double *wts = (double *)xmalloc(sizeof(double) * T * k);
        orc_moe_route(lg, T, E, k, ids, wts, 0);
        orc_moe_route(lg, T, E, k, ids, wts, 1);
        float *wf = (float *)xmalloc(sizeof(float) * T * k);
        for (int64_t i = 0; i < T * k; i++)
            wf[i] = (float)wts[i];
        for (int fmt = 0; fmt < 2; fmt++) {
            uint8_t *wg = weights(fmt, E * I, H), *wu = weights(fmt, E * I, H), *wd = weights(fmt, E * H, I);
            uint16_t *x16 = (uint16_t *)xmalloc(2 * T * H);
            for (int64_t i = 0; i < T * H; i++)
                x16[i] = orc_double_to_half(nrm());
            const int64_t A = T * k;
            double *g = (double *)xmalloc(8 * A * I), *u = (double *)xmalloc(8 * A * I), *hh = (double *)xmalloc(8 * A * I);
            double *dd2 = (double *)xmalloc(8 * A * H), *out = (double *)xmalloc(8 * T * H);
            double *Sg = (double *)xmalloc(8 * A * I), *Su = (double *)xmalloc(8 * A * I), *Sd = (double *)xmalloc(8 * A * H);
            for (int wi = 0; wi < 2; wi++)
                orc_moe_ffn(fmt, wg, wu, wd, x16, ids, wf, T, H, I, E, k, g, u, hh, dd2, out, Sg, Su, Sd, wi);
            orc_swiglu(g, u, A * I, hh);
            free(g); free(u); free(hh); free(dd2); free(out); free(Sg); free(Su); free(Sd);
            free(x16); free(wg); free(wu); free(wd);
        }
        free(wf); free(wts); free(ids); free(lg);
    }
    double hv[3] = {1.0, -0.0, 65504.0};
    uint16_t hb[3];
    double back[3];
    orc_double_array_to_half(hv, 3, hb);
    orc_half_array_to_double(hb, 3, back);
    if (back[0] != 1.0 || back[2] != 65504.0)
        fail = 1;
    if (fail) {
        fprintf(stderr, "oracle driver: an identity failed\n");
        return 1;
    }
    printf("oracle driver: all checks passed\n");
    return 0;
}
