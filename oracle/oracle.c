/*
 * oracle.c -- plain, slow reference for the fused block-dequant matmul.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke
 * check and the CPU-baseline leg of the benchmark load this file's library.
 * It shares no code, header, table or constant with the HIP library, and the
 * HIP library never calls it.
 *
 * What is computed (page "Building a Rust Inference Engine That Matches
 * Llama.cpp", section "Where the wins came from"): a matrix product whose
 * weights are stored as GGUF quantized blocks and are turned back into real
 * numbers at the moment they enter the dot product.  Because that fusion is
 * exact up to rounding order, this oracle is the plain definition written out:
 * dequantize every weight per the block format, then accumulate the dot
 * product in binary64.  Activations stay binary32 (page "Frink Inference: the
 * Rust alternative to llama.cpp", section "Where llama.cpp is still ahead",
 * the item on K-quant logits: activations are kept in f32, never quantized to
 * an 8-bit format before the dot).
 *
 * Block formats (the GGUF format the pages load; page "Building a Rust
 * Inference Engine That Matches Llama.cpp", sections "What Ferrox actually is"
 * and "Further resources"), little-endian:
 *
 *   Q8_0, 34 bytes per 32 weights:
 *     bytes 0-1  d      binary16 scale
 *     bytes 2-33 q[32]  two's-complement int8
 *     weight i = d * q[i]
 *
 *   Q4_K, 144 bytes per 256-weight super-block:
 *     bytes 0-1    d      binary16 super-block scale
 *     bytes 2-3    dmin   binary16 super-block min scale
 *     bytes 4-15   s[12]  eight 6-bit sub-block scales sc[j] and eight 6-bit
 *                         sub-block mins m[j] (packing in q4k_scale_min)
 *     bytes 16-143 qs[128] 256 unsigned 4-bit quants (order in q4k_quant)
 *     weight k (sub-block j = k / 32) = d * sc[j] * q[k] - dmin * m[j]
 *
 * A row of K weights is K/32 Q8_0 blocks or K/256 Q4_K super-blocks stored
 * back to back; rows follow each other with no padding.
 *
 * Rounding: d*sc*q and dmin*m are exact in binary64, and so is their
 * difference (every term is an integer multiple of 2^-24 below 2^27), so each
 * weight is the exact value rounded once to binary32 (round to nearest even,
 * C's default conversion).  The binary16 weight used by half-precision matrix
 * products is that binary32 value rounded once more to binary16.
 *
 * Results are binary64 sums; alongside each output y this file returns the
 * bound S = sum |w * x| that parity tolerances are scaled by.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary16, written from the format definition.                   */
/* ------------------------------------------------------------------------ */

/* binary16 bits -> value: sign bit 15, 5-bit exponent (bias 15), 10-bit
 * fraction; exponent 0 is the subnormal range (no implicit 1, scale 2^-24). */
double orc_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return sign ? -v : v;
}

/* Round-half-to-even of a non-negative value v to an integer, computed from
 * the definition (v holds at most 53 significant bits, so this is exact). */
static double round_half_even(double v)
{
    double n = floor(v);
    double frac = v - n;
    if (frac > 0.5 || (frac == 0.5 && fmod(n, 2.0) != 0.0))
        n += 1.0;
    return n;
}

/* value -> binary16 bits, round to nearest, ties to even. */
uint16_t orc_double_to_half(double v)
{
    uint16_t sign = 0;
    if (isnan(v))
        return 0x7e00;
    if (signbit(v)) {
        sign = 0x8000;
        v = -v;
    }
    if (v >= 65520.0) /* halfway between 65504 and 2^16 rounds to even: inf */
        return sign | 0x7c00;
    if (v < ldexp(1.0, -14)) {
        /* subnormal range: integer multiples of 2^-24; 1024 is the smallest
         * normal and its encoding 0x0400 follows on naturally */
        double n = round_half_even(ldexp(v, 24));
        return sign | (uint16_t)n;
    }
    int e; /* v = fr * 2^e with 0.5 <= fr < 1 */
    double fr = frexp(v, &e);
    double n = round_half_even(ldexp(fr, 11)); /* 1024 <= n <= 2048 */
    int ex = e - 1;                              /* v ~ n * 2^(ex - 10) */
    if (n == 2048.0) {
        n = 1024.0;
        ex += 1;
    }
    if (ex + 15 >= 31)
        return sign | 0x7c00;
    return sign | (uint16_t)(((ex + 15) << 10) | ((int)n - 1024));
}

void orc_half_array_to_double(const uint16_t *h, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = orc_half_to_double(h[i]);
}

void orc_double_array_to_half(const double *v, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = orc_double_to_half(v[i]);
}

static uint16_t le16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* ------------------------------------------------------------------------ */
/* Q8_0                                                                      */
/* ------------------------------------------------------------------------ */

#define Q8_0_BLOCK 32
#define Q8_0_BYTES 34

/* Weight k of row r, as the exact product d * q (binary64). */
static double q8_0_weight_exact(const uint8_t *w, int64_t K, int64_t r, int64_t k)
{
    int64_t nb = K / Q8_0_BLOCK;
    const uint8_t *blk = w + (r * nb + k / Q8_0_BLOCK) * Q8_0_BYTES;
    double d = orc_half_to_double(le16(blk));
    int q = (int8_t)blk[2 + k % Q8_0_BLOCK];
    return d * (double)q;
}

/* ------------------------------------------------------------------------ */
/* Q4_K                                                                      */
/* ------------------------------------------------------------------------ */

#define QK_K 256
#define Q4_K_BYTES 144

/* Sub-block j's 6-bit scale and min from the 12 packed bytes s[0..11].
 * Sub-blocks 0-3 keep both values whole in the low six bits of s[j] (scale)
 * and s[j+4] (min).  Sub-blocks 4-7 take their low four bits from s[j+4]
 * (scale in the low nibble, min in the high nibble) and their top two bits
 * from the otherwise unused top bits of s[j-4] (scale) and s[j] (min). */
static void q4k_scale_min(const uint8_t *s, int j, int *sc, int *m)
{
    if (j < 4) {
        *sc = s[j] & 63;
        *m = s[j + 4] & 63;
    } else {
        *sc = (s[j + 4] & 0x0f) | ((s[j - 4] >> 6) << 4);
        *m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
    }
}

/* Quant k (0..255) of a super-block: the 128 quant bytes form four groups of
 * 32; group g serves weights 64g..64g+63, the low nibble of byte 32g+i holding
 * weight 64g+i and the high nibble holding weight 64g+32+i. */
static int q4k_quant(const uint8_t *qs, int k)
{
    int g = k / 64, r = k % 64;
    uint8_t b = qs[32 * g + r % 32];
    return r < 32 ? (b & 0x0f) : (b >> 4);
}

static double q4k_weight_exact(const uint8_t *w, int64_t K, int64_t r, int64_t k)
{
    int64_t nb = K / QK_K;
    const uint8_t *blk = w + (r * nb + k / QK_K) * Q4_K_BYTES;
    double d = orc_half_to_double(le16(blk));
    double dmin = orc_half_to_double(le16(blk + 2));
    int kk = (int)(k % QK_K);
    int sc, m;
    q4k_scale_min(blk + 4, kk / 32, &sc, &m);
    int q = q4k_quant(blk + 16, kk);
    return d * (double)sc * (double)q - dmin * (double)m;
}

/* Decoded fields of one Q4_K super-block, for tests that inspect them. */
void orc_q4k_fields(const uint8_t *blk, double *d, double *dmin, int32_t *sc, int32_t *m,
                    int32_t *q)
{
    *d = orc_half_to_double(le16(blk));
    *dmin = orc_half_to_double(le16(blk + 2));
    for (int j = 0; j < 8; j++) {
        int a, b;
        q4k_scale_min(blk + 4, j, &a, &b);
        sc[j] = a;
        m[j] = b;
    }
    for (int k = 0; k < QK_K; k++)
        q[k] = q4k_quant(blk + 16, k);
}

/* ------------------------------------------------------------------------ */
/* Dequantization (fmt 0 = Q8_0, 1 = Q4_K)                                   */
/* ------------------------------------------------------------------------ */

static double weight_exact(int fmt, const uint8_t *w, int64_t K, int64_t r, int64_t k)
{
    return fmt == 0 ? q8_0_weight_exact(w, K, r, k) : q4k_weight_exact(w, K, r, k);
}

/* out32[r*K+k] = weight rounded once to binary32; out16 (optional) = that
 * binary32 value rounded to binary16.  Either output may be NULL. */
void orc_dequant(int fmt, const uint8_t *w, int64_t M, int64_t K, float *out32, uint16_t *out16)
{
    for (int64_t r = 0; r < M; r++)
        for (int64_t k = 0; k < K; k++) {
            float w32 = (float)weight_exact(fmt, w, K, r, k);
            if (out32)
                out32[r * K + k] = w32;
            if (out16)
                out16[r * K + k] = orc_double_to_half((double)w32);
        }
}

/* ------------------------------------------------------------------------ */
/* Matrix-vector products with binary32 activations                          */
/* ------------------------------------------------------------------------ */

/* y[b][i] = sum_k w32[rows[i]][k] * x[b][k] in binary64, S likewise of |.|.
 * The weight is produced inside the dot loop (the fused form).  rows == NULL
 * means all M rows in order (nrows = M). */
void orc_gemv(int fmt, const uint8_t *w, const float *x, int64_t M, int64_t K, int64_t B,
              const int64_t *rows, int64_t nrows, double *y, double *S)
{
    if (!rows)
        nrows = M;
    for (int64_t b = 0; b < B; b++)
        for (int64_t i = 0; i < nrows; i++) {
            int64_t r = rows ? rows[i] : i;
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < K; k++) {
                double w32 = (double)(float)weight_exact(fmt, w, K, r, k);
                double p = w32 * (double)x[b * K + k];
                acc += p;
                mag += fabs(p);
            }
            y[b * nrows + i] = acc;
            S[b * nrows + i] = mag;
        }
}

/* The same product computed in two separate passes: the whole row is
 * dequantized into a binary32 buffer first, then dotted in the same order. */
void orc_gemv_separate(int fmt, const uint8_t *w, const float *x, int64_t M, int64_t K,
                       int64_t B, double *y)
{
    float *row = (float *)malloc((size_t)K * sizeof(float));
    for (int64_t r = 0; r < M; r++) {
        for (int64_t k = 0; k < K; k++)
            row[k] = (float)weight_exact(fmt, w, K, r, k);
        for (int64_t b = 0; b < B; b++) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; k++)
                acc += (double)row[k] * (double)x[b * K + k];
            y[b * M + r] = acc;
        }
    }
    free(row);
}

/* ------------------------------------------------------------------------ */
/* Matrix products with binary16 activations: Y = X * W^T                    */
/* ------------------------------------------------------------------------ */

/* y[t][i] = sum_k w32[rows[i]][k] * x16[toks[t]][k] in binary64 (x16 holds
 * binary16 bit patterns, taken exactly).  NULL rows/toks mean all, in order. */
void orc_gemm(int fmt, const uint8_t *w, const uint16_t *x16, int64_t M, int64_t K, int64_t N,
              const int64_t *rows, int64_t nrows, const int64_t *toks, int64_t ntoks, double *y,
              double *S)
{
    if (!rows)
        nrows = M;
    if (!toks)
        ntoks = N;
    double *wrow = (double *)malloc((size_t)K * sizeof(double));
    double *xrow = (double *)malloc((size_t)K * sizeof(double));
    for (int64_t i = 0; i < nrows; i++) {
        int64_t r = rows ? rows[i] : i;
        for (int64_t k = 0; k < K; k++)
            wrow[k] = (double)(float)weight_exact(fmt, w, K, r, k);
        for (int64_t t = 0; t < ntoks; t++) {
            int64_t n = toks ? toks[t] : t;
            for (int64_t k = 0; k < K; k++)
                xrow[k] = orc_half_to_double(x16[n * K + k]);
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < K; k++) {
                double p = wrow[k] * xrow[k];
                acc += p;
                mag += fabs(p);
            }
            y[t * nrows + i] = acc;
            S[t * nrows + i] = mag;
        }
    }
    free(wrow);
    free(xrow);
}

/* ------------------------------------------------------------------------ */
/* Mixture-of-experts feed-forward                                           */
/* ------------------------------------------------------------------------ */

/* Routing of one token: p = softmax(logits) in binary64; ids = the topk
 * largest p in descending order, equal values going to the lower expert
 * index; wts = those p as they are (renorm == 0), or each divided by the sum
 * of the topk chosen p (renorm != 0). */
void orc_moe_route(const float *logits, int64_t T, int64_t E, int64_t topk, int32_t *ids,
                   double *wts, int renorm)
{
    double *p = (double *)malloc((size_t)E * sizeof(double));
    char *taken = (char *)malloc((size_t)E);
    for (int64_t t = 0; t < T; t++) {
        const float *l = logits + t * E;
        double mx = -INFINITY, sum = 0.0;
        for (int64_t e = 0; e < E; e++)
            if ((double)l[e] > mx)
                mx = (double)l[e];
        for (int64_t e = 0; e < E; e++) {
            p[e] = exp((double)l[e] - mx);
            sum += p[e];
        }
        for (int64_t e = 0; e < E; e++) {
            p[e] /= sum;
            taken[e] = 0;
        }
        for (int64_t s = 0; s < topk; s++) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; e++)
                if (!taken[e] && (best < 0 || p[e] > p[best]))
                    best = e;
            taken[best] = 1;
            ids[t * topk + s] = (int32_t)best;
            wts[t * topk + s] = p[best];
        }
        if (renorm) {
            double chosen = 0.0;
            for (int64_t s = 0; s < topk; s++)
                chosen += wts[t * topk + s];
            for (int64_t s = 0; s < topk; s++)
                wts[t * topk + s] /= chosen;
        }
    }
    free(p);
    free(taken);
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* SwiGLU of a feed-forward layer's gate and up products: h = silu(g) * u,
 * silu(z) = z / (1 + e^-z), in binary64, elementwise over n values. */
void orc_swiglu(const double *g, const double *u, int64_t n, double *h)
{
    for (int64_t i = 0; i < n; i++)
        h[i] = silu(g[i]) * u[i];
}

/* Dense product of one expert's weight matrix (R rows of C columns, format
 * fmt) with a binary64 vector. */
static void expert_matvec(int fmt, const uint8_t *w, int64_t R, int64_t C, const double *v,
                          double *out, double *mag)
{
    for (int64_t r = 0; r < R; r++) {
        double acc = 0.0, s = 0.0;
        for (int64_t c = 0; c < C; c++) {
            double p = (double)(float)weight_exact(fmt, w, C, r, c) * v[c];
            acc += p;
            s += fabs(p);
        }
        out[r] = acc;
        if (mag)
            mag[r] = s;
    }
}

/* The MoE feed-forward of every token, entirely in binary64.
 *   weights: w_gate, w_up are E stacked [I rows][H cols] matrices;
 *            w_down is E stacked [H rows][I cols] matrices, all of format
 *            fmt (0 = Q8_0, 1 = Q4_K).
 *   x16 [T][H] binary16 bits; ids/wts [T][topk] routing (binary32 weights).
 * For each (token t, slot s) with expert e = ids[t][s]:
 *   g = Wg_e x, u = Wu_e x, h = silu(g) * u, d = Wd_e h   (assignment a = t*topk+s)
 * and out[t] = sum over slots of wts[t][s] * d.  With weight_input != 0 the
 * slot weight scales the expert's input instead: x' = wts[t][s] * x feeds
 * g and u, and out[t] = sum over slots of d.  Outputs (any may be NULL):
 *   g, u, h [T*topk][I], d [T*topk][H], out [T][H], Sg, Su [T*topk][I], Sd [T*topk][H]. */
void orc_moe_ffn(int fmt, const uint8_t *w_gate, const uint8_t *w_up, const uint8_t *w_down,
                 const uint16_t *x16, const int32_t *ids, const float *wts, int64_t T, int64_t H,
                 int64_t I, int64_t E, int64_t topk, double *g, double *u, double *h, double *d,
                 double *out, double *Sg, double *Su, double *Sd, int weight_input)
{
    size_t gu_bytes = fmt == 0 ? (size_t)I * (size_t)(H / Q8_0_BLOCK) * Q8_0_BYTES
                               : (size_t)I * (size_t)(H / QK_K) * Q4_K_BYTES;
    size_t dn_bytes = fmt == 0 ? (size_t)H * (size_t)(I / Q8_0_BLOCK) * Q8_0_BYTES
                               : (size_t)H * (size_t)(I / QK_K) * Q4_K_BYTES;
    double *xv = (double *)malloc((size_t)H * sizeof(double));
    double *xw = (double *)malloc((size_t)H * sizeof(double));
    double *gv = (double *)malloc((size_t)I * sizeof(double));
    double *uv = (double *)malloc((size_t)I * sizeof(double));
    double *hv = (double *)malloc((size_t)I * sizeof(double));
    double *dv = (double *)malloc((size_t)H * sizeof(double));
    double *sg = (double *)malloc((size_t)I * sizeof(double));
    double *su = (double *)malloc((size_t)I * sizeof(double));
    double *sd = (double *)malloc((size_t)H * sizeof(double));
    for (int64_t t = 0; t < T; t++) {
        for (int64_t c = 0; c < H; c++)
            xv[c] = orc_half_to_double(x16[t * H + c]);
        if (out)
            for (int64_t c = 0; c < H; c++)
                out[t * H + c] = 0.0;
        for (int64_t s = 0; s < topk; s++) {
            int64_t a = t * topk + s;
            int64_t e = ids[a];
            const double *xin = xv;
            if (weight_input) {
                for (int64_t c = 0; c < H; c++)
                    xw[c] = (double)wts[a] * xv[c];
                xin = xw;
            }
            expert_matvec(fmt, w_gate + (size_t)e * gu_bytes, I, H, xin, gv, sg);
            expert_matvec(fmt, w_up + (size_t)e * gu_bytes, I, H, xin, uv, su);
            for (int64_t i = 0; i < I; i++)
                hv[i] = silu(gv[i]) * uv[i];
            expert_matvec(fmt, w_down + (size_t)e * dn_bytes, H, I, hv, dv, sd);
            for (int64_t i = 0; i < I; i++) {
                if (g)
                    g[a * I + i] = gv[i];
                if (u)
                    u[a * I + i] = uv[i];
                if (h)
                    h[a * I + i] = hv[i];
                if (Sg)
                    Sg[a * I + i] = sg[i];
                if (Su)
                    Su[a * I + i] = su[i];
            }
            for (int64_t c = 0; c < H; c++) {
                if (d)
                    d[a * H + c] = dv[c];
                if (Sd)
                    Sd[a * H + c] = sd[c];
                if (out)
                    out[t * H + c] += (weight_input ? 1.0 : (double)wts[a]) * dv[c];
            }
        }
    }
    free(xv);
    free(xw);
    free(gv);
    free(uv);
    free(hv);
    free(dv);
    free(sg);
    free(su);
    free(sd);
}

/* ------------------------------------------------------------------------ */
/* Activations as 8-bit blocks (the Q8_K form of the integer-dot path)       */
/* ------------------------------------------------------------------------ */

/* The pages name llama.cpp's practice of quantizing the activations to Q8_K
 * before the dot product (page "Frink Inference: the Rust alternative to
 * llama.cpp", the item on K-quant logits drifting) without defining the
 * block.  Reading: per 256 consecutive activations of a row, amax = max |x|,
 * code q = x * (127 / amax) rounded to nearest (ties to even) and clamped to
 * [-127, 127], scale d = amax / 127; every step in binary32.  A block of zeros
 * has d = 0 and q = 0.  bsum[j] is the sum of the 32 codes of sub-block j.
 *   x [B][K] binary32; q [B][K]; d [B][K/256]; bsum [B][K/32]. */
void orc_quantize_q8k(const float *x, int64_t B, int64_t K, int8_t *q, float *d, int32_t *bsum)
{
    int64_t nsb = K / QK_K;
    for (int64_t b = 0; b < B; b++) {
        for (int64_t s = 0; s < nsb; s++) {
            const float *v = x + b * K + s * QK_K;
            int8_t *qo = q + b * K + s * QK_K;
            float amax = 0.0f;
            for (int i = 0; i < QK_K; i++) {
                float a = fabsf(v[i]);
                if (a > amax)
                    amax = a;
            }
            float iscale = amax > 0.0f ? 127.0f / amax : 0.0f;
            d[b * nsb + s] = amax / 127.0f;
            for (int i = 0; i < QK_K; i++) {
                float t = v[i] * iscale;
                float r = rintf(t);
                if (r > 127.0f)
                    r = 127.0f;
                if (r < -127.0f)
                    r = -127.0f;
                qo[i] = (int8_t)r;
            }
            for (int j = 0; j < QK_K / 32; j++) {
                int32_t acc = 0;
                for (int i = 0; i < 32; i++)
                    acc += qo[32 * j + i];
                bsum[b * (K / 32) + s * (QK_K / 32) + j] = acc;
            }
        }
    }
}

/* y[b][i] = sum_k w(r, k) * (d_b[k / 256] * q_b[k]) for r = rows[i] (all rows
 * if rows is NULL), in binary64, with w the exact Q4_K weight
 * d * sc * q - dmin * m (not rounded to binary32: the integer-dot form scales
 * exact integer sums).  S[b][i] = sum_k (|d sc q| + |dmin m|) * |d_b q_b[k]|,
 * the magnitude against which the kernel's binary32 scaling rounds. */
void orc_gemv_q4k_q8k(const uint8_t *w, const int8_t *q, const float *d, int64_t M, int64_t K,
                      int64_t B, const int64_t *rows, int64_t nr, double *y, double *S)
{
    int64_t nsb = K / QK_K;
    (void)M;
    for (int64_t i = 0; i < nr; i++) {
        int64_t r = rows ? rows[i] : i;
        for (int64_t b = 0; b < B; b++) {
            double acc = 0.0, mag = 0.0;
            for (int64_t s = 0; s < nsb; s++) {
                const uint8_t *blk = w + (r * nsb + s) * Q4_K_BYTES;
                double dd = orc_half_to_double(le16(blk));
                double dm = orc_half_to_double(le16(blk + 2));
                double xs = (double)d[b * nsb + s];
                for (int k = 0; k < QK_K; k++) {
                    int sc, m;
                    q4k_scale_min(blk + 4, k / 32, &sc, &m);
                    double a = dd * (double)sc * (double)q4k_quant(blk + 16, k);
                    double c = dm * (double)m;
                    double xv = xs * (double)q[b * K + s * QK_K + k];
                    acc += (a - c) * xv;
                    mag += (fabs(a) + fabs(c)) * fabs(xv);
                }
            }
            y[b * nr + i] = acc;
            if (S)
                S[b * nr + i] = mag;
        }
    }
}

/* The two exact terms of every Q4_K weight, w = a - c with a = d * sc_j * q
 * and c = dmin * m_j, in binary64 (both products are exact there), for an
 * M x K matrix: a[r][k], c[r][k].  The integer-dot product scales exact
 * integer sums, so its reference uses these terms unrounded (as in
 * orc_gemv_q4k_q8k), and its error bound weighs |a| + |c|. */
void orc_q4k_terms(const uint8_t *w, int64_t M, int64_t K, double *a, double *c)
{
    int64_t nsb = K / QK_K;
    for (int64_t r = 0; r < M; r++) {
        for (int64_t s = 0; s < nsb; s++) {
            const uint8_t *blk = w + (r * nsb + s) * Q4_K_BYTES;
            double dd = orc_half_to_double(le16(blk));
            double dm = orc_half_to_double(le16(blk + 2));
            for (int k = 0; k < QK_K; k++) {
                int sc, m;
                q4k_scale_min(blk + 4, k / 32, &sc, &m);
                a[r * K + s * QK_K + k] = dd * (double)sc * (double)q4k_quant(blk + 16, k);
                c[r * K + s * QK_K + k] = dm * (double)m;
            }
        }
    }
}
