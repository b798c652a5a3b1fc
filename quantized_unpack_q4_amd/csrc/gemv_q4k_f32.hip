// gemv_q4k_f32.hip -- single Q4_K matrix-vector products for 2..16 activation
// rows on the binary32 matrix cores, K split over the waves of a workgroup.
//
// y[b][r] = sum_k w[r][k] * x[b][k] with w = d*sc*q - dmin*m per 32-weight
// sub-block, binary32 activations and results (the pages' fused dequant-dot,
// page "Building a Rust Inference Engine That Matches Llama.cpp", section
// "Where the wins came from"; activations stay binary32, page "Frink
// Inference: the Rust alternative to llama.cpp", the item on K-quant logits).
// Each lane dequantizes its weights itself: d*sc and dmin*m are exact in
// binary32 (an 11-bit significand times a 6-bit integer), so w comes from one
// fused multiply-add, fma(q, d*sc, -dmin*m), with one rounding; the products
// w*x and their sums are binary32 on v_mfma_f32_4x4x1f32 (B <= 4; its 16
// blocks of 4x4 either as rows 4g .. 4g+3 of a 16-row tile over 8-weight
// slice s of a sub-block, or as the 4 weights 4s .. 4s+3 of a unit for one
// 4-row group, which loads each activation by one lane instead of four) or
// v_mfma_f32_16x16x4f32 (the batch rows fill the 16 rows of the activation
// operand), accumulated in the matrix-core accumulator over all of the wave's
// K.  No activation split and no factored form: every term keeps a relative
// error of a few 2^-24 whatever the spread of x.
//
// Work split.  A workgroup of W waves owns T 16-row tiles over all of K; the
// unit of work is 64 weights of a row (sub-blocks 2p and 2p+1 of a
// super-block: the 4-bit quants of both share the 32 bytes 32p .. 32p+31 of
// the quant area), and wave w takes units u = w, w + W, ...  The weights go
// through LDS a chunk (W units, W/4 whole super-blocks of every row) at a
// time, loaded as the row's contiguous 16-byte pieces (two chunk buffers, one
// barrier per chunk); each lane then reads its row's 16-byte header (an LDS
// broadcast) and its 8 quant bytes.  The W partial results meet in LDS in
// wave order at the end.  This is the form for a single product whose rows
// alone cannot fill the chip with whole-K blocks of 64 rows or more.
#include "gq_device.h"
#include "gq_internal.h"

namespace gq {

namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// FORM: kWide (16x16x4), kGroups (4x4x1, block 4g + s = 4-row group g over
// 8-weight slice s of each sub-block) or kSlices (4x4x1, block s = the 4
// weights 4s .. 4s+3 of a unit for every 4-row group: each activation loaded
// by one lane instead of four).
enum { kWide = 0, kGroups = 1, kSlices = 2 };
template <int T, int W, int FORM>
__global__ __launch_bounds__(64 * W) void gemv_q4k_f32_kernel(
    const uint8_t *__restrict__ w, const float *__restrict__ x, float *__restrict__ y, int M,
    int K, int B)
{
    constexpr int kRows = 16 * T;
    constexpr bool SMALL = FORM != kWide, SLICES = FORM == kSlices;
    constexpr int kBatch = SMALL ? 4 : 16;
    static_assert(W % 4 == 0, "a chunk of W units is whole super-blocks");
    // a chunk of a row: W/4 super-blocks = 36W bytes = 9W/4 pieces of 16
    // bytes; LDS row stride 9W + 4 dwords (16-byte aligned, rows spread over
    // the banks)
    constexpr int kPieces = 9 * W / 4;
    constexpr int kStride = 9 * W + 4; // dwords
    constexpr int kPer = (kRows * kPieces + 64 * W - 1) / (64 * W);
    __shared__ u32x4_t wbuf4[2][kRows * kStride / 4];
    __shared__ float red[W][kBatch][kRows]; // [wave][batch row][weight row]
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = tid >> 6;
    // 16x16x4: lane l takes activation row l % 16 and weight row l % 16, slice
    // l / 16 (weights 8s .. 8s+7 of each sub-block); 4x4x1: block 4g + s, lane
    // 4(4g + s) + i takes activation row i, weight row 4g + i, slice s.  Either
    // way the lane's results belong to its own weight row.
    const int wr = SMALL ? ((lane >> 4) << 2) | (lane & 3) : lane & 15;
    const int ks = SMALL ? (lane >> 2) & 3 : lane >> 4;
    const int xb = SMALL ? lane & 3 : lane & 15;
    // kSlices: lane l = 4s + j takes activation row j and weight row 4g + j of
    // every 4-row group g, for the weights 4s .. 4s+3 of a unit: sub-block
    // 2p + s/8 (low or high nibbles), elements 4(s%8) .. 4(s%8)+3
    const int sl = lane >> 2, jl = lane & 3, sh = sl >> 3;
    const int r0 = (int)blockIdx.x * kRows;
    const int nunit = K >> 6;
    const int nchunk = (nunit + W - 1) / W;
    const int64_t row_bytes = (int64_t)(K >> 8) * kQ4kBytes;
    const bool xrow_ok = xb < B;
    const float *xrow = x + (int64_t)(xrow_ok ? xb : 0) * K;

    // staging: piece p = tid + 64W*n is 16 bytes of row p / kPieces at byte
    // 16 * (p % kPieces) of the chunk; rows are whole pieces, so a piece is
    // either inside its row or past its end (not loaded: no wave reads it)
    const uint8_t *src[kPer];
    int dst[kPer], pj[kPer];
    bool pok[kPer];
#pragma unroll
    for (int n = 0; n < kPer; ++n) {
        const int p = tid + 64 * W * n;
        pok[n] = p < kRows * kPieces;
        const int row = pok[n] ? p / kPieces : 0, j = p % kPieces;
        src[n] = w + (int64_t)min(r0 + row, M - 1) * row_bytes;
        dst[n] = (row * kStride) / 4 + j;
        pj[n] = 16 * j;
    }
    u32x4_t stg[kPer];
    auto stage_load = [&](int c) {
        const int64_t base = (int64_t)c * (W / 4 * kQ4kBytes);
#pragma unroll
        for (int n = 0; n < kPer; ++n)
            if (pok[n] && base + pj[n] < row_bytes)
                stg[n] = *(const u32x4_t *)(src[n] + base + pj[n]);
    };
    auto stage_store = [&](int buf) {
#pragma unroll
        for (int n = 0; n < kPer; ++n)
            if (pok[n])
                wbuf4[buf][dst[n]] = stg[n];
    };

    struct Xs {
        float4 x0, x1, x2, x3; // x[b][64u + 8s .. +7], x[b][64u + 32 + 8s .. +7]
    };
    auto load_x = [&](int u, Xs &p) {
        if (SLICES) {
            p.x0 = xrow_ok && u < nunit ? ldf4(xrow + 64 * u + 4 * sl)
                                        : make_float4(0.f, 0.f, 0.f, 0.f);
        } else if (xrow_ok && u < nunit) {
            const float *xp = xrow + 64 * u + 8 * ks;
            p.x0 = ldf4(xp);
            p.x1 = ldf4(xp + 4);
            p.x2 = ldf4(xp + 32);
            p.x3 = ldf4(xp + 36);
        } else {
            p.x0 = p.x1 = p.x2 = p.x3 = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };

    constexpr int G = SLICES ? 4 : 1; // 4-row groups held apart (kSlices)
    float4_t acc[T][G];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int g = 0; g < G; ++g)
            acc[t][g] = float4_t{0.f, 0.f, 0.f, 0.f};
    // this wave's unit of the chunk in buffer buf: super-block wave / 4 of the
    // chunk, sub-blocks 2p and 2p+1 with p = wave % 4
    const int p = wave & 3;
    auto compute = [&](int buf, const Xs &xs) {
        const uint32_t *wb = reinterpret_cast<const uint32_t *>(wbuf4[buf]);
        if constexpr (SLICES) {
            const float xv[4] = {xs.x0.x, xs.x0.y, xs.x0.z, xs.x0.w};
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const uint32_t *pr =
                        wb + (16 * t + 4 * g + jl) * kStride + 36 * (wave >> 2);
                    const uint32_t h0 = pr[0], h1 = pr[1], h2 = pr[2], h3 = pr[3];
                    const uint32_t q = (pr[4 + 8 * p + (sl & 7)] >> (4 * sh)) & 0x0f0f0f0fu;
                    uint32_t sc, m;
                    q4k_scale_min(h1, h2, h3, 2 * p + sh, sc, m);
                    const float dsc = half_to_float(h0 & 0xffffu) * (float)sc;
                    const float ndmm = -(half_to_float(h0 >> 16) * (float)m);
                    acc[t][g] = __builtin_amdgcn_mfma_f32_4x4x1f32(
                        xv[0], fmaf(ubyte_to_float<0>(q), dsc, ndmm), acc[t][g], 0, 0, 0);
                    acc[t][g] = __builtin_amdgcn_mfma_f32_4x4x1f32(
                        xv[1], fmaf(ubyte_to_float<1>(q), dsc, ndmm), acc[t][g], 0, 0, 0);
                    acc[t][g] = __builtin_amdgcn_mfma_f32_4x4x1f32(
                        xv[2], fmaf(ubyte_to_float<2>(q), dsc, ndmm), acc[t][g], 0, 0, 0);
                    acc[t][g] = __builtin_amdgcn_mfma_f32_4x4x1f32(
                        xv[3], fmaf(ubyte_to_float<3>(q), dsc, ndmm), acc[t][g], 0, 0, 0);
                }
            return;
        }
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const uint32_t *pr = wb + (16 * t + wr) * kStride + 36 * (wave >> 2);
            const uint32_t h0 = pr[0], h1 = pr[1], h2 = pr[2], h3 = pr[3];
            const uint32_t qa = pr[4 + 8 * p + 2 * ks], qb = pr[5 + 8 * p + 2 * ks];
            const float d = half_to_float(h0 & 0xffffu), dmin = half_to_float(h0 >> 16);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                // sub-block 2p + h: the low (h = 0) or high nibbles
                uint32_t sc, m;
                q4k_scale_min(h1, h2, h3, 2 * p + h, sc, m);
                const float dsc = d * (float)sc, ndmm = -(dmin * (float)m);
                const uint32_t a = (qa >> (4 * h)) & 0x0f0f0f0fu;
                const uint32_t b = (qb >> (4 * h)) & 0x0f0f0f0fu;
                const float wv[8] = {
                    fmaf(ubyte_to_float<0>(a), dsc, ndmm), fmaf(ubyte_to_float<1>(a), dsc, ndmm),
                    fmaf(ubyte_to_float<2>(a), dsc, ndmm), fmaf(ubyte_to_float<3>(a), dsc, ndmm),
                    fmaf(ubyte_to_float<0>(b), dsc, ndmm), fmaf(ubyte_to_float<1>(b), dsc, ndmm),
                    fmaf(ubyte_to_float<2>(b), dsc, ndmm), fmaf(ubyte_to_float<3>(b), dsc, ndmm)};
                const float4 u = h ? xs.x2 : xs.x0, v = h ? xs.x3 : xs.x1;
                const float xv[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    acc[t][0] = SMALL ? __builtin_amdgcn_mfma_f32_4x4x1f32(xv[j], wv[j], acc[t][0],
                                                                           0, 0, 0)
                                      : __builtin_amdgcn_mfma_f32_16x16x4f32(xv[j], wv[j],
                                                                             acc[t][0], 0, 0, 0);
            }
        }
    };

    // chunk c is computed from LDS buffer c % 2 while the loaded chunk c + 1
    // is stored into the other and the loads of chunk c + 2 go out
    // (kSlices, one float4 of activations per unit, loads them two chunks
    // ahead)
    constexpr int XA = SLICES ? 2 : 1;
    Xs xc, xn, xnn;
    stage_load(0);
    load_x(wave, xc);
    if (XA == 2)
        load_x(W + wave, xn);
    stage_store(0);
    __syncthreads();
    if (nchunk > 1)
        stage_load(1);
    for (int c = 0; c < nchunk; ++c) {
        load_x((c + XA) * W + wave, XA == 2 ? xnn : xn);
        if (c * W + wave < nunit)
            compute(c & 1, xc);
        if (c + 1 < nchunk) {
            stage_store((c + 1) & 1);
            if (c + 2 < nchunk)
                stage_load(c + 2);
        }
        __syncthreads();
        xc = xn;
        if (XA == 2)
            xn = xnn;
    }
    if constexpr (SLICES) {
        // sum the 16 slices of a unit (lanes 4, 8, 16 and 32 apart)
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float v = acc[t][g][i];
                    v += __shfl_xor(v, 4, 64);
                    v += __shfl_xor(v, 8, 64);
                    v += __shfl_xor(v, 16, 64);
                    v += __shfl_xor(v, 32, 64);
                    acc[t][g][i] = v;
                }
        if (sl == 0)
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int g = 0; g < G; ++g)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        red[wave][i][16 * t + 4 * g + jl] = acc[t][g][i];
    } else if constexpr (SMALL) {
        // sum the four weight slices (lanes 4 and 8 apart)
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[t][0][i] += __shfl_xor(acc[t][0][i], 4, 64);
                acc[t][0][i] += __shfl_xor(acc[t][0][i], 8, 64);
            }
        if (ks == 0)
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    red[wave][i][16 * t + wr] = acc[t][0][i];
    } else {
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                red[wave][4 * (lane >> 4) + i][16 * t + wr] = acc[t][0][i];
    }
    __syncthreads();
    for (int o = tid; o < kBatch * kRows; o += 64 * W) {
        const int b = o / kRows, r = o % kRows;
        float s = 0.f;
#pragma unroll
        for (int wv = 0; wv < W; ++wv)
            s += red[wv][b][r];
        if (b < B && r0 + r < M)
            y[(int64_t)b * M + r0 + r] = s;
    }
}

template <int T, int W>
hipError_t go(const void *w, const float *x, float *y, int64_t M, int64_t K, int B, hipStream_t s)
{
    const unsigned grid = (unsigned)((M + 16 * T - 1) / (16 * T));
    // batch 4, and 3 with K of 8192 or more, on the slice form, whose
    // activation loads do not repeat per 4-row group (measured, kernel
    // durations, group -> slice form: 4096x14336 batch 4 35.4 -> 28.6 us,
    // batch 3 30.1 -> 28.1; 6144x14336 batch 4 54.8 -> 47.9; 4096x4096 batch
    // 3 11.2 -> 12.4, batch 4 12.7 -> 12.5)
    if (B == 4 || (B == 3 && K >= 8192))
        hipLaunchKernelGGL((gemv_q4k_f32_kernel<T, W, kSlices>), dim3(grid), dim3(64 * W), 0, s,
                           static_cast<const uint8_t *>(w), x, y, (int)M, (int)K, B);
    else if (B <= 4)
        hipLaunchKernelGGL((gemv_q4k_f32_kernel<T, W, kGroups>), dim3(grid), dim3(64 * W), 0, s,
                           static_cast<const uint8_t *>(w), x, y, (int)M, (int)K, B);
    else
        hipLaunchKernelGGL((gemv_q4k_f32_kernel<T, W, kWide>), dim3(grid), dim3(64 * W), 0, s,
                           static_cast<const uint8_t *>(w), x, y, (int)M, (int)K, B);
    return hipGetLastError();
}

} // namespace

hipError_t launch_gemv_q4k_f32(const void *w, const float *x, float *y, int64_t M, int64_t K,
                               int B, hipStream_t s)
{
#ifdef LAB_T
    return go<LAB_T, LAB_W>(w, x, y, M, K, B, s);
#else
    const int64_t blocks2 = (M + 31) / 32, blocks1 = (M + 15) / 16;
    if (blocks2 >= 384)
        return go<2, 8>(w, x, y, M, K, B, s);
    if (blocks1 > device_cus())
        return go<1, 8>(w, x, y, M, K, B, s);
    return go<1, 16>(w, x, y, M, K, B, s);
#endif
}

} // namespace gq
