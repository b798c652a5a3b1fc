// gemm_q8k.hip -- the opt-in integer-dot matrix product (prefill) over 8-bit
// activation codes: Y[n][r] = sum_k w(r, k) * d_x[n][k/256] * q_x[n][k].
//
// llama.cpp quantizes activations to 8-bit blocks before its K-quant
// products; the pages name that as the reason its logits drift from Frink's
// binary32 path (page "Frink Inference: the Rust alternative to llama.cpp",
// section "Where llama.cpp is still ahead", K-quant item).  Here it is an
// opt-in entry point beside the binary16 dequant product: the activation
// codes come from gq_quantize_q8k (per 256 values one binary32 scale d_x).
//
// Arithmetic.  Per Q4_K super-block the result is
//     d_x * ( d * sum_j sc_j * sum_{k in j} q4_k * q_k  -  dmin * sum_j m_j * sum_{k in j} q_k ),
// and the inner sums are exact integers.  They run on the int8 matrix cores
// (v_mfma_i32_32x32x32_i8, one 32-weight sub-block per instruction) with the
// sub-block's 6-bit scale folded into the weight operand, so that the
// accumulators never need a per-sub-block vector multiply: sc = 8*sc_hi +
// sc_lo (each 0..7) makes q4*sc_lo and q4*sc_hi bytes of at most 105, and the
// min term takes m_j (at most 63) in every byte of its operand.  Three int32
// accumulators per output fragment collect, over the 8 sub-blocks,
//     P_lo = sum q4 sc_lo q,  P_hi = sum q4 sc_hi q,  P_m = sum m q,
// all exact (|P| < 2^25), and once per super-block
//     total += d_x * (d * (8 P_hi + P_lo) - dmin * P_m)
// in binary32.  Bytes of q4 * sc come from one packed 16-bit multiply per 4
// quants (no byte product exceeds 8 bits, so no carry crosses a byte).
//
// Work split.  A workgroup of 4 waves owns 128 weight rows x 64 tokens; wave w
// takes rows 32w..32w+31 against both 32-token fragments.  Per super-block
// the 64 tokens' codes (16 KB) and scales are staged in LDS (double-buffered,
// one barrier per super-block; 16-byte chunks of a token at chunk ^ (token &
// 15), so that 16 lanes reading one chunk of 16 tokens hit 16 bank groups);
// each lane loads its own weight row's header and 4 x 16 quant bytes, one
// super-block ahead.  The activation fragment is the matrix instruction's
// first operand (rows = tokens) and the weights its second (columns = weight
// rows), so each lane's 16 results share one weight row's d and dmin.
#include "gq_device.h"
#include "gq_internal.h"

namespace gq {

namespace {

typedef int int4v __attribute__((ext_vector_type(4)));
typedef int int16v __attribute__((ext_vector_type(16)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4 g_u32x4;

constexpr int BM = 128; // weight rows per workgroup
constexpr int BN = 64;  // tokens per workgroup
constexpr int NT = 256;

__device__ __forceinline__ uint4 gload16(const void *p)
{
    const u32x4 v = *(g_u32x4 *)(p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// four bytes (each at most 15) times a small integer, bytewise
__device__ __forceinline__ uint32_t bytes_times(uint32_t v, uint32_t s)
{
    const u16x2 a = __builtin_bit_cast(u16x2, v);
    const u16x2 b = {(unsigned short)s, (unsigned short)s};
    return __builtin_bit_cast(uint32_t, (u16x2)(a * b));
}

struct WBlk {
    uint4 h;    // header: d | dmin << 16, then the 12 scale/min bytes
    uint4 q[4]; // quant bytes 32g + 16h .. 32g + 16h + 15 of group g
};

struct Lds {
    uint4 act[2][BN][16]; // [buffer][token][chunk ^ (token & 15)]
    float dx[2][BN];
};

} // namespace

__global__ __launch_bounds__(NT, 2) void gemm_q4k_q8k_kernel(const uint8_t *__restrict__ w,
                                                             const int8_t *__restrict__ qx,
                                                             const float *__restrict__ dxs,
                                                             float *__restrict__ y, int M, int K,
                                                             int N, int tiles_m)
{
    __shared__ Lds sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 31, h = lane >> 5;
    const int tm = (int)blockIdx.x % tiles_m, tn = (int)blockIdx.x / tiles_m;
    const int m0 = tm * BM, n0 = tn * BN;
    const int nsb = K >> 8;

    // this lane's weight row (rows past M read row M - 1, never stored)
    const int row = m0 + 32 * wave + r;
    const uint8_t *wrow = w + (size_t)min(row, M - 1) * (size_t)nsb * kQ4kBytes;
    auto load_w = [&](int s, WBlk &b) {
        const uint8_t *blk = wrow + (size_t)s * kQ4kBytes;
        b.h = gload16(blk);
#pragma unroll
        for (int g = 0; g < 4; ++g)
            b.q[g] = gload16(blk + 16 + 32 * g + 16 * h);
    };

    // staging: thread tid moves chunk c of tokens tid/16 + 16p (p = 0..3)
    const int sc_c = tid & 15, sc_t = tid >> 4;
    uint4 ar[4];
    float dxr = 0.f;
    auto load_act = [&](int s) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int n = n0 + sc_t + 16 * p;
            ar[p] = n < N ? gload16(qx + (size_t)n * K + 256 * s + 16 * sc_c)
                          : make_uint4(0, 0, 0, 0);
        }
        if (tid < BN)
            dxr = n0 + tid < N ? dxs[(size_t)(n0 + tid) * nsb + s] : 0.f;
    };
    auto store_act = [&](int buf) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int t = sc_t + 16 * p;
            sm.act[buf][t][sc_c ^ (t & 15)] = ar[p];
        }
        if (tid < BN)
            sm.dx[buf][tid] = dxr;
    };

    float total[2][16];
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int v = 0; v < 16; ++v)
            total[f][v] = 0.f;

    auto compute = [&](int buf, const WBlk &b) {
        int16v plo[2], phi[2], pm[2];
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            plo[f] = int16v{};
            phi[f] = int16v{};
            pm[f] = int16v{};
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint32_t sc, m;
            q4k_scale_min(b.h.y, b.h.z, b.h.w, j, sc, m);
            const uint4 qq = b.q[j >> 1];
            const int sh = 4 * (j & 1);
            const uint32_t n0w = (qq.x >> sh) & 0x0F0F0F0Fu, n1w = (qq.y >> sh) & 0x0F0F0F0Fu;
            const uint32_t n2w = (qq.z >> sh) & 0x0F0F0F0Fu, n3w = (qq.w >> sh) & 0x0F0F0F0Fu;
            const uint32_t slo = sc & 7u, shi = sc >> 3;
            const int4v blo = {(int)bytes_times(n0w, slo), (int)bytes_times(n1w, slo),
                               (int)bytes_times(n2w, slo), (int)bytes_times(n3w, slo)};
            const int4v bhi = {(int)bytes_times(n0w, shi), (int)bytes_times(n1w, shi),
                               (int)bytes_times(n2w, shi), (int)bytes_times(n3w, shi)};
            const int mb = (int)(m * 0x01010101u);
            const int4v bm = {mb, mb, mb, mb};
#pragma unroll
            for (int f = 0; f < 2; ++f) {
                const int t = 32 * f + r;
                const int4v a = __builtin_bit_cast(int4v, sm.act[buf][t][(2 * j + h) ^ (t & 15)]);
                plo[f] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, blo, plo[f], 0, 0, 0);
                phi[f] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bhi, phi[f], 0, 0, 0);
                pm[f] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bm, pm[f], 0, 0, 0);
            }
        }
        const float d = half_to_float(b.h.x), dmin = half_to_float(b.h.x >> 16);
#pragma unroll
        for (int f = 0; f < 2; ++f) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                // element v = 4g + i is token 32f + 8g + 4h + i of this fragment
                const float4 xs = *reinterpret_cast<const float4 *>(&sm.dx[buf][32 * f + 8 * g + 4 * h]);
                const float xv[4] = {xs.x, xs.y, xs.z, xs.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int v = 4 * g + i;
                    const int ti = (phi[f][v] << 3) + plo[f][v];
                    const float val = fmaf(d, (float)ti, -dmin * (float)pm[f][v]);
                    total[f][v] = fmaf(xv[i], val, total[f][v]);
                }
            }
        }
    };

    WBlk wa, wb;
    load_act(0);
    load_w(0, wa);
    store_act(0);
    __syncthreads();
    for (int s = 0; s < nsb; s += 2) {
        const bool more = s + 1 < nsb;
        if (more) {
            load_act(s + 1);
            load_w(s + 1, wb);
        }
        compute(0, wa);
        if (more)
            store_act(1);
        __syncthreads();
        if (!more)
            break;
        const bool more2 = s + 2 < nsb;
        if (more2) {
            load_act(s + 2);
            load_w(s + 2, wa);
        }
        compute(1, wb);
        if (more2)
            store_act(0);
        __syncthreads();
    }

    if (row < M) {
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int n = n0 + 32 * f + 8 * (v >> 2) + 4 * h + (v & 3);
                if (n < N)
                    y[(size_t)n * M + row] = total[f][v];
            }
    }
}

hipError_t launch_gemm_q4k_q8k(const void *w, const int8_t *q, const float *d, float *y, int64_t M,
                               int64_t K, int64_t N, hipStream_t s)
{
    const int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const int64_t grid = tiles_m * tiles_n;
    if (grid > 0x7fffffff)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(gemm_q4k_q8k_kernel, dim3((unsigned)grid), dim3(NT), 0, s,
                       (const uint8_t *)w, q, d, y, (int)M, (int)K, (int)N, (int)tiles_m);
    return hipGetLastError();
}

} // namespace gq
