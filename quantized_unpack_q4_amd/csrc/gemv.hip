// gemv.hip -- fused dequant matrix-vector products (Q4_K, Q8_0) for gfx950.
//
// y[b][r] = sum_k w[r][k] x[b][k] with binary32 activations that are never
// quantized (page "Frink Inference: the Rust alternative to llama.cpp",
// section "Where llama.cpp is still ahead", K-quant item), and each weight
// dequantized inside the dot product rather than in a separate pass (page
// "Building a Rust Inference Engine That Matches Llama.cpp", section "Where
// the wins came from").
//
// Q4_K arithmetic (the general kernel: batch 1 with K above the streaming
// kernel's limit, and matrices too large for the matrix-core kernel's 32-bit
// offsets).  Each weight is dequantized once to its binary32 value,
// w = d*sc_j*q - dmin*m_j with one rounding (d*sc_j*q is exact, so a fused
// multiply-add gives it), and multiplied by each of the B activation rows in
// binary32; the dequantization is shared by the batch rows.  Unlike the
// factored form sum(q*x)*d*sc - sum(x)*dmin*m, whose rounding error follows
// the two terms, the error here follows sum |w*x| however w's terms cancel.
// High nibbles are used as 16*q (masking without a shift) and the factor 1/16
// goes into d*sc (exact).
#include "gq_device.h"
#include "gq_internal.h"

namespace gq {

// ---------------------------------------------------------------------------
// Q4_K
// ---------------------------------------------------------------------------
// Lane mapping: four lanes per super-block, lane quarter g = lane & 3 owns the
// 32 quant bytes of group g (weights 64g..64g+63, sub-blocks 2g and 2g+1), so
// one wave covers 16 super-blocks per step along K.  Each wave handles R rows
// at once and reuses every activation load across them.
template <int B, int R>
__global__ __launch_bounds__(256) void gemv_q4k_kernel(const uint8_t *__restrict__ w,
                                                       const float *__restrict__ x,
                                                       float *__restrict__ y, int M, int K)
{
    const int lane = threadIdx.x & 63;
    const int row0 = ((int)blockIdx.x * 4 + ((int)threadIdx.x >> 6)) * R;
    if (row0 >= M)
        return;
    const int nsb = K >> 8;
    const size_t row_bytes = (size_t)nsb * kQ4kBytes;
    const int g = lane & 3;

    float acc[R][B];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int b = 0; b < B; ++b)
            acc[r][b] = 0.f;

    for (int s = lane >> 2; s < nsb; s += 16) {
        uint4 hd[R], qa[R], qb[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (row0 + r < M) {
                const uint8_t *blk = w + (size_t)(row0 + r) * row_bytes + (size_t)s * kQ4kBytes;
                hd[r] = ld16(blk);
                qa[r] = ld16(blk + 16 + 32 * g);
                qb[r] = ld16(blk + 32 + 32 * g);
            } else {
                hd[r] = make_uint4(0, 0, 0, 0);
                qa[r] = hd[r];
                qb[r] = hd[r];
            }
        }
        const float *xs = x + (size_t)s * 256 + 64 * g;
        float dsl[R], dsh[R], dml[R], dmh[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            uint32_t scl, ml, sch, mh;
            q4k_scale_min(hd[r].y, hd[r].z, hd[r].w, 2 * g, scl, ml);
            q4k_scale_min(hd[r].y, hd[r].z, hd[r].w, 2 * g + 1, sch, mh);
            const float d = half_to_float(hd[r].x);
            const float dmin = half_to_float(hd[r].x >> 16);
            dsl[r] = d * (float)scl;
            dsh[r] = d * (float)sch * 0.0625f;
            dml[r] = dmin * (float)ml;
            dmh[r] = dmin * (float)mh;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float wl[R][4], wh[R][4];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint32_t D = i == 0 ? qa[r].x : i == 1 ? qa[r].y : i == 2 ? qa[r].z
                                 : i == 3 ? qa[r].w : i == 4 ? qb[r].x : i == 5 ? qb[r].y
                                 : i == 6 ? qb[r].z : qb[r].w;
                const uint32_t lo = D & 0x0f0f0f0fu;
                const uint32_t hi = D & 0xf0f0f0f0u;
                wl[r][0] = fmaf(dsl[r], ubyte_to_float<0>(lo), -dml[r]);
                wl[r][1] = fmaf(dsl[r], ubyte_to_float<1>(lo), -dml[r]);
                wl[r][2] = fmaf(dsl[r], ubyte_to_float<2>(lo), -dml[r]);
                wl[r][3] = fmaf(dsl[r], ubyte_to_float<3>(lo), -dml[r]);
                wh[r][0] = fmaf(dsh[r], ubyte_to_float<0>(hi), -dmh[r]);
                wh[r][1] = fmaf(dsh[r], ubyte_to_float<1>(hi), -dmh[r]);
                wh[r][2] = fmaf(dsh[r], ubyte_to_float<2>(hi), -dmh[r]);
                wh[r][3] = fmaf(dsh[r], ubyte_to_float<3>(hi), -dmh[r]);
            }
#pragma unroll
            for (int b = 0; b < B; ++b) {
                const float4 xl = ldf4(xs + (size_t)b * K + 4 * i);
                const float4 xh = ldf4(xs + (size_t)b * K + 32 + 4 * i);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    float a = acc[r][b];
                    a = fmaf(wl[r][0], xl.x, a);
                    a = fmaf(wl[r][1], xl.y, a);
                    a = fmaf(wl[r][2], xl.z, a);
                    a = fmaf(wl[r][3], xl.w, a);
                    a = fmaf(wh[r][0], xh.x, a);
                    a = fmaf(wh[r][1], xh.y, a);
                    a = fmaf(wh[r][2], xh.z, a);
                    a = fmaf(wh[r][3], xh.w, a);
                    acc[r][b] = a;
                }
            }
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const float v = wave_sum(acc[r][b]);
            if (lane == 0 && row0 + r < M)
                y[(size_t)b * M + row0 + r] = v;
        }
}

template <int B, int R>
static hipError_t gemv_q4k_go(const void *w, const float *x, float *y, int64_t M, int64_t K,
                              hipStream_t s)
{
    const int64_t waves = (M + R - 1) / R;
    const int64_t grid = (waves + 3) / 4;
    hipLaunchKernelGGL((gemv_q4k_kernel<B, R>), dim3((unsigned)grid), dim3(256), 0, s,
                       (const uint8_t *)w, x, y, (int)M, (int)K);
    return hipGetLastError();
}

hipError_t launch_gemv_q4k(const void *w, const float *x, float *y, int64_t M, int64_t K, int B,
                           hipStream_t s)
{
    switch (B) {
    case 1: return gemv_q4k_go<1, 4>(w, x, y, M, K, s);
    case 2: return gemv_q4k_go<2, 2>(w, x, y, M, K, s);
    case 3: return gemv_q4k_go<3, 2>(w, x, y, M, K, s);
    case 4: return gemv_q4k_go<4, 2>(w, x, y, M, K, s);
    case 5: return gemv_q4k_go<5, 1>(w, x, y, M, K, s);
    case 6: return gemv_q4k_go<6, 1>(w, x, y, M, K, s);
    case 7: return gemv_q4k_go<7, 1>(w, x, y, M, K, s);
    case 8: return gemv_q4k_go<8, 1>(w, x, y, M, K, s);
    case 9: return gemv_q4k_go<9, 1>(w, x, y, M, K, s);
    case 10: return gemv_q4k_go<10, 1>(w, x, y, M, K, s);
    case 11: return gemv_q4k_go<11, 1>(w, x, y, M, K, s);
    case 12: return gemv_q4k_go<12, 1>(w, x, y, M, K, s);
    case 13: return gemv_q4k_go<13, 1>(w, x, y, M, K, s);
    case 14: return gemv_q4k_go<14, 1>(w, x, y, M, K, s);
    case 15: return gemv_q4k_go<15, 1>(w, x, y, M, K, s);
    case 16: return gemv_q4k_go<16, 1>(w, x, y, M, K, s);
    default: return hipErrorInvalidValue;
    }
}

// ---------------------------------------------------------------------------
// Q8_0
// ---------------------------------------------------------------------------
// One lane per 34-byte block.  A block starts on an even byte: its position p
// is either 0 or 2 modulo 4.  The lane reads the aligned dwords covering the
// block and takes the 32 quants out with a byte shift of 2 (p % 4 == 0) or 4
// (p % 4 == 2); it never reads outside the block's own dwords except the two
// bytes before it, which belong to the same buffer.
template <int B, int R>
__global__ __launch_bounds__(256) void gemv_q8_0_kernel(const uint8_t *__restrict__ w,
                                                        const float *__restrict__ x,
                                                        float *__restrict__ y, int M, int K)
{
    const int lane = threadIdx.x & 63;
    const int row0 = ((int)blockIdx.x * 4 + ((int)threadIdx.x >> 6)) * R;
    if (row0 >= M)
        return;
    const int nb = K >> 5;
    const size_t row_bytes = (size_t)nb * kQ80Bytes;

    float acc[R][B];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int b = 0; b < B; ++b)
            acc[r][b] = 0.f;

    for (int blk = lane; blk < nb; blk += 64) {
        float part[R][B];
        float dd[R];
        uint32_t q[R][8];
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int b = 0; b < B; ++b)
                part[r][b] = 0.f;
            if (row0 + r >= M) {
                dd[r] = 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    q[r][i] = 0;
                continue;
            }
            const size_t p = (size_t)(row0 + r) * row_bytes + (size_t)blk * kQ80Bytes;
            const uint32_t *base = reinterpret_cast<const uint32_t *>(w + (p & ~(size_t)3));
            uint32_t W[9];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                W[i] = base[i];
            const bool odd = (p & 2) != 0; // block begins 2 bytes into a dword
            if (odd)
                W[8] = base[8];
            else
                W[8] = *reinterpret_cast<const uint16_t *>(reinterpret_cast<const uint8_t *>(base) + 32);
            dd[r] = half_to_float(odd ? (W[0] >> 16) : W[0]);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                q[r][i] = odd ? W[i + 1] : __builtin_amdgcn_alignbyte(W[i + 1], W[i], 2);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
#pragma unroll
            for (int b = 0; b < B; ++b) {
                const float4 xv = ldf4(x + (size_t)b * K + (size_t)blk * 32 + 4 * i);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const uint32_t v = q[r][i];
                    part[r][b] = fmaf((float)(int8_t)(v & 0xff), xv.x, part[r][b]);
                    part[r][b] = fmaf((float)(int8_t)((v >> 8) & 0xff), xv.y, part[r][b]);
                    part[r][b] = fmaf((float)(int8_t)((v >> 16) & 0xff), xv.z, part[r][b]);
                    part[r][b] = fmaf((float)(int8_t)(v >> 24), xv.w, part[r][b]);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < B; ++b)
                acc[r][b] = fmaf(dd[r], part[r][b], acc[r][b]);
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const float v = wave_sum(acc[r][b]);
            if (lane == 0 && row0 + r < M)
                y[(size_t)b * M + row0 + r] = v;
        }
}

template <int B, int R>
static hipError_t gemv_q8_0_go(const void *w, const float *x, float *y, int64_t M, int64_t K,
                               hipStream_t s)
{
    const int64_t waves = (M + R - 1) / R;
    const int64_t grid = (waves + 3) / 4;
    hipLaunchKernelGGL((gemv_q8_0_kernel<B, R>), dim3((unsigned)grid), dim3(256), 0, s,
                       (const uint8_t *)w, x, y, (int)M, (int)K);
    return hipGetLastError();
}

hipError_t launch_gemv_q8_0(const void *w, const float *x, float *y, int64_t M, int64_t K,
                            int B, hipStream_t s)
{
    // 2..16 activation rows: matrix cores, when rows are whole pairs of blocks
    if (B >= 2 && K % 64 == 0)
        return launch_gemv_q8_0_mfma(w, x, y, M, K, B, s);
    // batch 1: four rows per wave share the activation loads on tall matrices
    // (measured: 14336 x 4096 26.7 -> 22.5 us; 4096-row matrices lose waves and
    // are faster at two)
    if (B == 1 && M >= 8192)
        return gemv_q8_0_go<1, 4>(w, x, y, M, K, s);
    switch (B) {
    case 1: return gemv_q8_0_go<1, 2>(w, x, y, M, K, s);
    case 2: return gemv_q8_0_go<2, 2>(w, x, y, M, K, s);
    case 3: return gemv_q8_0_go<3, 1>(w, x, y, M, K, s);
    case 4: return gemv_q8_0_go<4, 1>(w, x, y, M, K, s);
    case 5: return gemv_q8_0_go<5, 1>(w, x, y, M, K, s);
    case 6: return gemv_q8_0_go<6, 1>(w, x, y, M, K, s);
    case 7: return gemv_q8_0_go<7, 1>(w, x, y, M, K, s);
    case 8: return gemv_q8_0_go<8, 1>(w, x, y, M, K, s);
    case 9: return gemv_q8_0_go<9, 1>(w, x, y, M, K, s);
    case 10: return gemv_q8_0_go<10, 1>(w, x, y, M, K, s);
    case 11: return gemv_q8_0_go<11, 1>(w, x, y, M, K, s);
    case 12: return gemv_q8_0_go<12, 1>(w, x, y, M, K, s);
    case 13: return gemv_q8_0_go<13, 1>(w, x, y, M, K, s);
    case 14: return gemv_q8_0_go<14, 1>(w, x, y, M, K, s);
    case 15: return gemv_q8_0_go<15, 1>(w, x, y, M, K, s);
    case 16: return gemv_q8_0_go<16, 1>(w, x, y, M, K, s);
    default: return hipErrorInvalidValue;
    }
}

} // namespace gq
