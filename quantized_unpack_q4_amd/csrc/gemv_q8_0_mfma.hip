// gemv_q8_0_mfma.hip -- Q8_0 matrix-vector products for 2..16 activation rows
// on the matrix cores.
//
// y[b][r] = sum_k w[r][k] * x[b][k], w = d * q per 32-weight block, binary32
// activations and results (the pages' fused dequant-dot, page "Building a Rust
// Inference Engine That Matches Llama.cpp", section "Where the wins came
// from"; Q8_0 is the format whose results the pages report as matching
// llama.cpp's, page "Frink Inference: the Rust alternative to llama.cpp", the
// item on K-quant logits).  Per block the sum is taken in factored form,
//     d * sum_k q_k x_k,
// with sum_k q_k x_k on v_mfma_f32_16x16x32_f16, one block per instruction
// pair: the quant is an exact binary16 integer, the activation enters as two
// binary16 halves hi + lo of x * 2^e, where 2^e (per activation row and
// block) brings the block's largest |x| to [2^14, 2^15).  The products are
// exact and the sums binary32, so every value at least 2^-17 of its block's
// largest |x| keeps 22 significant bits and every value at least 2^-20 of it
// a relative error below 2^-19; d and 2^-e are applied in binary32 per block.
// A block of an activation row whose non-zero |x| span more than 2^20 (the
// split would lose its small values) is left out of the split and
// computed exactly instead: d*q (exact) times the binary32 activation, summed
// in binary32 over the four lanes that hold the block.
//
// Work split.  A workgroup of 16 waves owns T 16-row tiles of weight rows (T
// = 2 when that still gives at least 384 workgroups, else 1; the tiles share
// each activation operand) over all of K; wave w takes the
// 64-weight pairs of blocks m = w, w + 16, ... (a pair is 68 bytes starting
// 4-byte aligned when K % 64 == 0), and the 16 partial results are summed in
// wave order through LDS at the end.  The batch rows fill the 16 rows of the
// activation operand (rows past B are zero).
#include "gq_device.h"
#include "gq_internal.h"

namespace gq {

namespace {

constexpr int kWaves = 16;
constexpr int kMaxTiles = 2; // 16-row weight tiles per workgroup, at most

typedef __attribute__((address_space(1))) const uint32_t g_u32;

// The registers one pair of blocks needs: this lane's weight dwords (its
// quarter's quants of both blocks and the two scales) and its activation row's
// 2 x 8 binary32 values.
struct Pair {
    // per tile: block 0 dwords 2q .. 2q+2 (quants 8q .. 8q+7 at byte shift 2),
    // dword 0 (scale 0, low half), dword 8 (scale 1, high half), block 1
    // dwords 9+2q, 10+2q (quants 8q .. 8q+7, aligned)
    uint32_t wa0[kMaxTiles], wa1[kMaxTiles], wa2[kMaxTiles], d0w[kMaxTiles], d1w[kMaxTiles],
        wb0[kMaxTiles], wb1[kMaxTiles];
    float4 x0, x1, x2, x3; // x[b][64m + 8q .. +7], x[b][64m + 32 + 8q .. +7]
};

__device__ __forceinline__ half8_t quants8(uint32_t q0, uint32_t q1)
{
    // signed bytes as exact binary16 integers: (q ^ 0x80) - 128 through the
    // unsigned byte conversion
    const uint32_t a = q0 ^ 0x80808080u, b = q1 ^ 0x80808080u;
    const uint4 v = make_uint4(
        pack_half2(ubyte_to_float<0>(a) - 128.f, ubyte_to_float<1>(a) - 128.f),
        pack_half2(ubyte_to_float<2>(a) - 128.f, ubyte_to_float<3>(a) - 128.f),
        pack_half2(ubyte_to_float<0>(b) - 128.f, ubyte_to_float<1>(b) - 128.f),
        pack_half2(ubyte_to_float<2>(b) - 128.f, ubyte_to_float<3>(b) - 128.f));
    return __builtin_bit_cast(half8_t, v);
}

// hi and lo binary16 halves of x * 2^e for 8 values.
__device__ __forceinline__ void split8(float4 u, float4 v, int e, half8_t &hi, half8_t &lo)
{
    const float s[8] = {ldexpf(u.x, e), ldexpf(u.y, e), ldexpf(u.z, e), ldexpf(u.w, e),
                        ldexpf(v.x, e), ldexpf(v.y, e), ldexpf(v.z, e), ldexpf(v.w, e)};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const _Float16 h = (_Float16)s[i];
        hi[i] = h;
        lo[i] = (_Float16)(s[i] - (float)h); // exact difference, one rounding
    }
}

// Exponent e with max|x| * 2^e in [2^14, 2^15) over the 32 values of one
// block of this lane's activation row (its 8 and those of the 3 other lanes
// of the row: lanes b, b+16, b+32, b+48); 0 for an all-zero block.  exact: the
// block's non-zero |x| span more than 2^20.
__device__ __forceinline__ int block_exp(float4 u, float4 v, bool &exact)
{
    const float a[8] = {fabsf(u.x), fabsf(u.y), fabsf(u.z), fabsf(u.w),
                        fabsf(v.x), fabsf(v.y), fabsf(v.z), fabsf(v.w)};
    float m = 0.f, mn = INFINITY;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        m = fmaxf(m, a[i]);
        mn = a[i] > 0.f ? fminf(mn, a[i]) : mn;
    }
    m = fmaxf(m, __shfl_xor(m, 16, 64));
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    mn = fminf(mn, __shfl_xor(mn, 16, 64));
    mn = fminf(mn, __shfl_xor(mn, 32, 64));
    exact = m > 1048576.f * mn; // 2^20
    if (m == 0.f)
        return 0;
    int E;
    (void)frexpf(m, &E); // m = f * 2^E, f in [0.5, 1)
    return 15 - E;
}

template <int T>
__global__ __launch_bounds__(64 * kWaves) void gemv_q8_0_mfma_kernel(
    const uint8_t *__restrict__ w, const float *__restrict__ x, float *__restrict__ y, int M,
    int K, int B)
{
    constexpr int kRows = 16 * T;
    __shared__ float red[kWaves][16][kRows]; // [wave][batch row][weight row]
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 15, q = lane >> 4;
    const int r0 = (int)blockIdx.x * kRows;
    const int npair = K >> 6;
    const int64_t row_bytes = (int64_t)(K >> 5) * kQ80Bytes;
    // rows past M read row M - 1 and are not written
    const uint8_t *wrow[T];
#pragma unroll
    for (int t = 0; t < T; ++t)
        wrow[t] = w + (int64_t)min(r0 + 16 * t + col, M - 1) * row_bytes;
    const bool xrow_ok = col < B;
    const float *xrow = x + (int64_t)(xrow_ok ? col : 0) * K;

    auto load = [&](int m, Pair &p) {
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const uint8_t *pp = wrow[t] + (int64_t)m * (2 * kQ80Bytes);
            p.wa0[t] = *(g_u32 *)(pp + 8 * q);
            p.wa1[t] = *(g_u32 *)(pp + 8 * q + 4);
            p.wa2[t] = *(g_u32 *)(pp + 8 * q + 8);
            p.d0w[t] = *(g_u32 *)(pp);
            p.d1w[t] = *(g_u32 *)(pp + 32);
            p.wb0[t] = *(g_u32 *)(pp + 36 + 8 * q);
            p.wb1[t] = *(g_u32 *)(pp + 40 + 8 * q);
        }
        if (xrow_ok) {
            const float *xp = xrow + 64 * m + 8 * q;
            p.x0 = ldf4(xp);
            p.x1 = ldf4(xp + 4);
            p.x2 = ldf4(xp + 32);
            p.x3 = ldf4(xp + 36);
        } else {
            p.x0 = p.x1 = p.x2 = p.x3 = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };

    // tile t: batch row 4q + i, weight row 16t + col
    float acc[T][4];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc[t][i] = 0.f;
    auto compute = [&](const Pair &p) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            const float4 u = blk ? p.x2 : p.x0, v = blk ? p.x3 : p.x1;
            bool exact;
            const int e = block_exp(u, v, exact);
            half8_t xh, xl;
            split8(u, v, e, xh, xl);
            if (exact) {
                xh = half8_t{0, 0, 0, 0, 0, 0, 0, 0};
                xl = xh;
            }
            int eb[4]; // exponents of batch rows 4q + i
#pragma unroll
            for (int i = 0; i < 4; ++i)
                eb[i] = __shfl(e, 4 * q + i, 64);
            float dq[T];
            half8_t wqv[T];
#pragma unroll
            for (int t = 0; t < T; ++t) {
                wqv[t] = blk ? quants8(p.wb0[t], p.wb1[t])
                             : quants8(__builtin_amdgcn_alignbyte(p.wa1[t], p.wa0[t], 2),
                                       __builtin_amdgcn_alignbyte(p.wa2[t], p.wa1[t], 2));
                dq[t] = half_to_float(blk ? (p.d1w[t] >> 16) : (p.d0w[t] & 0xffffu));
                float4_t c = float4_t{0.f, 0.f, 0.f, 0.f};
                c = __builtin_amdgcn_mfma_f32_16x16x32_f16(xh, wqv[t], c, 0, 0, 0);
                c = __builtin_amdgcn_mfma_f32_16x16x32_f16(xl, wqv[t], c, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[t][i] = fmaf(dq[t], ldexpf(c[i], -eb[i]), acc[t][i]);
            }
            // batch rows whose block is computed exactly (bit b: row b)
            uint64_t rows_exact = __ballot(exact && q == 0 && col < B);
            while (rows_exact) {
                const int b = __builtin_ctzll(rows_exact);
                rows_exact &= rows_exact - 1;
                // row b's 8 activations of this lane's quarter, from lane b + 16q
                const int src = b + 16 * q;
                const float xv[8] = {__shfl(u.x, src, 64), __shfl(u.y, src, 64),
                                     __shfl(u.z, src, 64), __shfl(u.w, src, 64),
                                     __shfl(v.x, src, 64), __shfl(v.y, src, 64),
                                     __shfl(v.z, src, 64), __shfl(v.w, src, 64)};
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    float part = 0.f;
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        part = fmaf(dq[t] * (float)wqv[t][i], xv[i], part);
                    part += __shfl_xor(part, 16, 64);
                    part += __shfl_xor(part, 32, 64);
                    if (q == (b >> 2)) {
                        const int i = b & 3;
                        acc[t][0] += i == 0 ? part : 0.f;
                        acc[t][1] += i == 1 ? part : 0.f;
                        acc[t][2] += i == 2 ? part : 0.f;
                        acc[t][3] += i == 3 ? part : 0.f;
                    }
                }
            }
        }
    };

    int m = wave;
    if (m < npair) {
        Pair cur, nxt;
        load(m, cur);
        for (; m < npair; m += kWaves) {
            if (m + kWaves < npair)
                load(m + kWaves, nxt);
            compute(cur);
            cur = nxt;
        }
    }
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            red[wave][4 * q + i][16 * t + col] = acc[t][i];
    __syncthreads();
    if (tid < 16 * kRows) {
        const int b = tid / kRows, r = tid % kRows;
        float s = 0.f;
#pragma unroll
        for (int wv = 0; wv < kWaves; ++wv)
            s += red[wv][b][r];
        if (b < B && r0 + r < M)
            y[(int64_t)b * M + r0 + r] = s;
    }
}

} // namespace

hipError_t launch_gemv_q8_0_mfma(const void *w, const float *x, float *y, int64_t M, int64_t K,
                                 int B, hipStream_t s)
{
    // two tiles per workgroup halve the activation reads per weight row, but
    // only pay while the grid still covers the chip (measured: 14336 rows
    // 63 -> 53 us at batch 16; 4096 rows slower with 128 workgroups)
    const int64_t blocks2 = (M + 31) / 32;
    if (blocks2 >= 384)
        hipLaunchKernelGGL((gemv_q8_0_mfma_kernel<2>), dim3((unsigned)blocks2), dim3(64 * kWaves),
                           0, s, static_cast<const uint8_t *>(w), x, y, (int)M, (int)K, B);
    else
        hipLaunchKernelGGL((gemv_q8_0_mfma_kernel<1>), dim3((unsigned)((M + 15) / 16)),
                           dim3(64 * kWaves), 0, s, static_cast<const uint8_t *>(w), x, y, (int)M,
                           (int)K, B);
    return hipGetLastError();
}

} // namespace gq
