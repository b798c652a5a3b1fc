// gemv_q8k.hip -- the opt-in integer-dot matrix-vector product: activations
// quantized to 8-bit blocks, Q4_K quants multiplied against them with 8-bit
// dot products.
//
// This is llama.cpp's way of evaluating K-quant products, which the pages set
// against keeping the activations in binary32 (page "Frink Inference: the Rust
// alternative to llama.cpp", the item on K-quant logits drifting): the
// activations lose precision to 8-bit codes, so results move by up to
// sum_k |w_k| |x_k - d q_k|.  The binary32 products elsewhere in this library
// are the default; this path is separate and opt-in.
//
// The activation block (the pages name it Q8_K and do not define it) is read
// as: 256 consecutive activations of a row, scale d = max|x| / 127 and codes
// q = x * (127 / max|x|) rounded to nearest even, clamped to [-127, 127], in
// binary32; a zero block has d = 0.  With it the 32-weight sub-block j of a
// Q4_K super-block contributes
//   d_x * ( d * sc_j * sum_i q4_i q_i  -  dmin * m_j * sum_i q_i )
// where both sums are exact integers (sum_i q_i is the block's precomputed
// sub-block sum), taken by v_dot4_i32_i8 on four code pairs at a time.
#include "gq_device.h"
#include "gq_internal.h"

namespace gq {

namespace {

constexpr int kWaves = 4; // waves per workgroup, both kernels

// One wave per 256-activation block (blocks in row-major order over [B][K]):
// lane l takes activations 4l..4l+3.
__global__ __launch_bounds__(64 * kWaves) void quantize_q8k_kernel(
    const float *__restrict__ x, int8_t *__restrict__ q, float *__restrict__ d,
    int32_t *__restrict__ bsum, int64_t nblk)
{
    const int lane = threadIdx.x & 63;
    const int64_t blk = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (blk >= nblk) // the whole wave leaves together
        return;
    const float4 v = ldf4(x + blk * 256 + 4 * lane);
    float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    const float iscale = amax > 0.f ? 127.f / amax : 0.f;
    auto code = [&](float xv) {
        const float t = xv * iscale;
        return (int)fminf(fmaxf(rintf(t), -127.f), 127.f);
    };
    const int c0 = code(v.x), c1 = code(v.y), c2 = code(v.z), c3 = code(v.w);
    reinterpret_cast<uint32_t *>(q + blk * 256)[lane] =
        (uint32_t)(c0 & 255) | ((uint32_t)(c1 & 255) << 8) | ((uint32_t)(c2 & 255) << 16) |
        ((uint32_t)(c3 & 255) << 24);
    // sub-block j is lanes 8j..8j+7
    int s = c0 + c1 + c2 + c3;
    s += __shfl_xor(s, 1, 64);
    s += __shfl_xor(s, 2, 64);
    s += __shfl_xor(s, 4, 64);
    if ((lane & 7) == 0)
        bsum[blk * 8 + (lane >> 3)] = s;
    if (lane == 0)
        d[blk] = amax / 127.f;
}

// One wave per R consecutive weight rows, all B activation rows at once.  A
// lane takes one (super-block, 32-byte quant group) pair at a time: the group
// holds the low nibbles of sub-block 2g and the high nibbles of sub-block
// 2g + 1, 64 weights per row, whose 64 activation codes are four 16-byte
// loads per batch row, loaded once for the R rows.
template <int B, int R>
__global__ __launch_bounds__(64 * kWaves) void gemv_q4k_q8k_kernel(
    const uint8_t *__restrict__ w, const int8_t *__restrict__ q, const float *__restrict__ xd,
    const int32_t *__restrict__ bsum, float *__restrict__ y, int M, int K)
{
    const int lane = threadIdx.x & 63;
    const int r0 = ((int)blockIdx.x * kWaves + (threadIdx.x >> 6)) * R;
    if (r0 >= M) // the whole wave leaves together
        return;
    const int nsb = K >> 8;
    const int ntask = 4 * nsb;
    const int64_t row_bytes = (int64_t)nsb * kQ4kBytes;
    // rows past M (last wave of a ragged M) read row M - 1 and are not written
    const uint8_t *wr[R];
#pragma unroll
    for (int j = 0; j < R; ++j)
        wr[j] = w + (int64_t)min(r0 + j, M - 1) * row_bytes;
    float acc[R][B];
#pragma unroll
    for (int j = 0; j < R; ++j)
#pragma unroll
        for (int b = 0; b < B; ++b)
            acc[j][b] = 0.f;

    for (int t = lane; t < ntask; t += 64) {
        const int s = t >> 2, g = t & 3;
        uint32_t W[R][8], sl[R], ml[R], sh[R], mh[R];
        float d[R], dmin[R];
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const uint8_t *blk = wr[j] + (int64_t)s * kQ4kBytes;
            const uint4 h = ld16(blk);
            const uint4 qa = ld16(blk + 16 + 32 * g), qb = ld16(blk + 32 + 32 * g);
            q4k_scale_min(h.y, h.z, h.w, 2 * g, sl[j], ml[j]);
            q4k_scale_min(h.y, h.z, h.w, 2 * g + 1, sh[j], mh[j]);
            d[j] = half_to_float(h.x);
            dmin[j] = half_to_float(h.x >> 16);
            W[j][0] = qa.x; W[j][1] = qa.y; W[j][2] = qa.z; W[j][3] = qa.w;
            W[j][4] = qb.x; W[j][5] = qb.y; W[j][6] = qb.z; W[j][7] = qb.w;
        }
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const int8_t *xq = q + (int64_t)b * K + (int64_t)s * 256 + 64 * g;
            const uint4 x0 = ld16(xq), x1 = ld16(xq + 16), x2 = ld16(xq + 32), x3 = ld16(xq + 48);
            const uint32_t X[16] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w,
                                    x2.x, x2.y, x2.z, x2.w, x3.x, x3.y, x3.z, x3.w};
            const int2 bs =
                *reinterpret_cast<const int2 *>(bsum + (int64_t)b * (K >> 5) + 8 * s + 2 * g);
            const float dx = xd[(int64_t)b * nsb + s];
#pragma unroll
            for (int j = 0; j < R; ++j) {
                int lo = 0, hi = 0;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    lo = __builtin_amdgcn_sdot4((int)(W[j][i] & 0x0f0f0f0fu), (int)X[i], lo, false);
                    hi = __builtin_amdgcn_sdot4((int)((W[j][i] >> 4) & 0x0f0f0f0fu), (int)X[8 + i],
                                                hi, false);
                }
                // |isum| < 2^23 and |msum| < 2^19: both convert to binary32 exactly
                const int isum = (int)sl[j] * lo + (int)sh[j] * hi;
                const int msum = (int)ml[j] * bs.x + (int)mh[j] * bs.y;
                acc[j][b] = fmaf(dx, d[j] * (float)isum - dmin[j] * (float)msum, acc[j][b]);
            }
        }
    }
#pragma unroll
    for (int j = 0; j < R; ++j)
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const float v = wave_sum(acc[j][b]);
            if (lane == 0 && r0 + j < M)
                y[(int64_t)b * M + r0 + j] = v;
        }
}

// Rows per wave: the activation codes are loaded once per lane task for R
// rows, so their cache traffic per weight byte falls as 1/R (measured on
// 14336 x 4096: batch 16 69 -> 52 us from R = 1 to 4, batch 4 23 -> 21 us;
// batch 1 is fastest at R = 1).
template <int B>
hipError_t gemv_go(const void *w, const int8_t *q, const float *xd, const int32_t *bsum, float *y,
                   int64_t M, int64_t K, hipStream_t s)
{
    constexpr int R = B == 1 ? 1 : B <= 3 ? 2 : 4;
    const int64_t blocks = (M + R * kWaves - 1) / (R * kWaves);
    hipLaunchKernelGGL((gemv_q4k_q8k_kernel<B, R>), dim3((unsigned)blocks), dim3(64 * kWaves), 0,
                       s, static_cast<const uint8_t *>(w), q, xd, bsum, y, (int)M, (int)K);
    return hipGetLastError();
}

typedef int v4i_t __attribute__((ext_vector_type(4)));
constexpr int kMWaves = 16; // waves per workgroup of the matrix-core form

// Batch 2..16 on the int8 matrix cores.  A workgroup of 16 waves owns 16
// weight rows and splits K by super-blocks over its waves.  Per 32-weight
// sub-block j one v_mfma_i32_16x16x32_i8 gives the exact sums sum_i q4_i q_i
// for the 16 batch rows x 16 weight rows (codes as the first operand, the
// 4-bit quants as bytes 0..15 as the second), and a second one accumulates
// m_j * sum_i q_i over the super-block (the second operand is m_j in every
// byte).  sc_j * (first sum) is summed over j in int32 (|.| < 2^25), and per
// super-block d_x * (d * that - dmin * (second sum)) is applied in binary32.
// The 16 waves' partial results are summed in wave order through LDS.
__global__ __launch_bounds__(64 * kMWaves) void gemv_q4k_q8k_mfma_kernel(
    const uint8_t *__restrict__ w, const int8_t *__restrict__ q, const float *__restrict__ xd,
    float *__restrict__ y, int M, int K, int B)
{
    __shared__ float red[kMWaves][16][16]; // [wave][batch row][weight row]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, qq = lane >> 4;
    const int r0 = (int)blockIdx.x * 16;
    const int nsb = K >> 8;
    const int64_t rowb = (int64_t)nsb * kQ4kBytes;
    // rows past M read row M - 1 and are not written; batch rows past B are zero
    const uint8_t *wrow = w + (int64_t)min(r0 + col, M - 1) * rowb;
    const bool xok = col < B;
    const int8_t *xrow = q + (int64_t)(xok ? col : 0) * K;

    float acc[4] = {0.f, 0.f, 0.f, 0.f}; // batch row 4qq + i, weight row col
    for (int s = wave; s < nsb; s += kMWaves) {
        const uint8_t *blk = wrow + (int64_t)s * kQ4kBytes;
        const uint4 h = ld16(blk);
        uint2 qw[4];
#pragma unroll
        for (int g = 0; g < 4; ++g)
            qw[g] = *reinterpret_cast<const uint2 *>(blk + 16 + 32 * g + 8 * qq);
        long xa[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            xa[j] = xok ? *reinterpret_cast<const long *>(xrow + (int64_t)s * 256 + 32 * j + 8 * qq)
                        : 0L;
        v4i_t c2 = v4i_t{0, 0, 0, 0};
        int ai[4] = {0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int g = j >> 1, hh = j & 1;
            const uint32_t lo = hh ? (qw[g].x >> 4) & 0x0f0f0f0fu : qw[g].x & 0x0f0f0f0fu;
            const uint32_t hi = hh ? (qw[g].y >> 4) & 0x0f0f0f0fu : qw[g].y & 0x0f0f0f0fu;
            const long wb = (long)(((unsigned long)hi << 32) | lo);
            uint32_t sc, m;
            q4k_scale_min(h.y, h.z, h.w, j, sc, m);
            const long mb = (long)((unsigned long)m * 0x0101010101010101ull);
            const v4i_t c1 = __builtin_amdgcn_mfma_i32_16x16x32_i8(xa[j], wb, v4i_t{0, 0, 0, 0}, 0,
                                                                   0, 0);
            c2 = __builtin_amdgcn_mfma_i32_16x16x32_i8(xa[j], mb, c2, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                ai[i] += (int)sc * c1[i];
        }
        const float d = half_to_float(h.x), dmin = half_to_float(h.x >> 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int b = 4 * qq + i;
            const float dx = b < B ? xd[(int64_t)b * nsb + s] : 0.f;
            acc[i] = fmaf(dx, d * (float)ai[i] - dmin * (float)c2[i], acc[i]);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
        red[wave][4 * qq + i][col] = acc[i];
    __syncthreads();
    if (tid < 256) {
        const int b = tid >> 4, r = tid & 15;
        float v = 0.f;
#pragma unroll
        for (int wv = 0; wv < kMWaves; ++wv)
            v += red[wv][b][r];
        if (b < B && r0 + r < M)
            y[(int64_t)b * M + r0 + r] = v;
    }
}

} // namespace

hipError_t launch_quantize_q8k(const float *x, int8_t *q, float *d, int32_t *bsum, int64_t B,
                               int64_t K, hipStream_t s)
{
    const int64_t nblk = B * (K / 256);
    const int64_t blocks = (nblk + kWaves - 1) / kWaves;
    hipLaunchKernelGGL(quantize_q8k_kernel, dim3((unsigned)blocks), dim3(64 * kWaves), 0, s, x, q,
                       d, bsum, nblk);
    return hipGetLastError();
}

hipError_t launch_gemv_q4k_q8k(const void *w, const int8_t *q, const float *d,
                               const int32_t *bsum, float *y, int64_t M, int64_t K, int B,
                               hipStream_t s)
{
    // batch 6..16 on the int8 matrix cores (measured on 14336 x 4096, rotated
    // weights: batch 8 31.2 -> 26.2 us, batch 16 52 -> 31.6 us; at batch 2 and 4
    // the vector kernel below is faster, 15.2 and 20.7 us against 21.6 and 23.6)
    if (B >= 6) {
        hipLaunchKernelGGL(gemv_q4k_q8k_mfma_kernel, dim3((unsigned)((M + 15) / 16)),
                           dim3(64 * kMWaves), 0, s, static_cast<const uint8_t *>(w), q, d, y,
                           (int)M, (int)K, B);
        return hipGetLastError();
    }
    switch (B) {
    case 1: return gemv_go<1>(w, q, d, bsum, y, M, K, s);
    case 2: return gemv_go<2>(w, q, d, bsum, y, M, K, s);
    case 3: return gemv_go<3>(w, q, d, bsum, y, M, K, s);
    case 4: return gemv_go<4>(w, q, d, bsum, y, M, K, s);
    case 5: return gemv_go<5>(w, q, d, bsum, y, M, K, s);
    case 6: return gemv_go<6>(w, q, d, bsum, y, M, K, s);
    case 7: return gemv_go<7>(w, q, d, bsum, y, M, K, s);
    case 8: return gemv_go<8>(w, q, d, bsum, y, M, K, s);
    case 9: return gemv_go<9>(w, q, d, bsum, y, M, K, s);
    case 10: return gemv_go<10>(w, q, d, bsum, y, M, K, s);
    case 11: return gemv_go<11>(w, q, d, bsum, y, M, K, s);
    case 12: return gemv_go<12>(w, q, d, bsum, y, M, K, s);
    case 13: return gemv_go<13>(w, q, d, bsum, y, M, K, s);
    case 14: return gemv_go<14>(w, q, d, bsum, y, M, K, s);
    case 15: return gemv_go<15>(w, q, d, bsum, y, M, K, s);
    default: return gemv_go<16>(w, q, d, bsum, y, M, K, s);
    }
}

} // namespace gq
