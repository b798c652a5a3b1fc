// gemv_q8_0_mfma.hip -- Q8_0 matrix-vector products for 2..16 activation rows
// on the matrix cores, in binary32.
//
// y[b][r] = sum_k w[r][k] * x[b][k], w = d * q per 32-weight block, binary32
// activations and results (the pages' fused dequant-dot, page "Building a Rust
// Inference Engine That Matches Llama.cpp", section "Where the wins came
// from"; Q8_0 is the format whose results the pages report as matching
// llama.cpp's, page "Frink Inference: the Rust alternative to llama.cpp", the
// item on K-quant logits).  Per block the sum is taken in factored form,
//     d * sum_k q_k x_k,
// with sum_k q_k x_k on the binary32 matrix-core products: the quant is an
// exact binary32 integer and the activation goes in as it is, so nothing is
// split, rescaled or routed around (binary32 products and sums throughout,
// subnormals kept, as a binary32 dot product in another order would give);
// d is applied in binary32 once per block.  B <= 4 runs the 16-block
// v_mfma_f32_4x4x1f32 in one of two layouts: block 4g + s as rows 4g .. 4g+3
// of a 16-row tile against the batch rows over 8-weight slice s of the block
// (eight instructions per block and tile), or block s as the 4 weights
// 4s .. 4s+3 of a pair for one 4-row group (four instructions per group and
// pair, each activation loaded by one lane instead of four); larger batches
// run v_mfma_f32_16x16x4f32 (the batch rows fill the 16 rows of the
// activation operand, rows past B are zero).  An instruction takes one
// weight and one activation per lane.
//
// Work split.  A workgroup of W waves owns T 16-row tiles of weight rows over
// all of K; wave w takes the 64-weight pairs of blocks m = w, w + W, ... (a
// pair is 68 bytes starting 4-byte aligned when K % 64 == 0), and the W
// partial results are summed in wave order through LDS at the end.  The
// weights go through LDS a chunk (W pairs of every row) at a time: the
// workgroup loads each row's 68W contiguous bytes as 16-byte pieces, so a
// load instruction covers whole cache lines of one or two rows, where loading
// each lane's own dwords straight from memory touched a line per row and
// dword and left the L1 cache, not memory, as the limit; the waves then read
// their lanes' dwords from LDS.  Two chunk buffers, one barrier per chunk.
#include "gq_device.h"
#include "gq_internal.h"

namespace gq {

namespace {

typedef __attribute__((address_space(1))) const uint32_t g_u32;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
// 16 bytes at a 4-byte aligned address
typedef unsigned int u32x4a4_t __attribute__((ext_vector_type(4), aligned(4)));

// signed byte k of v as binary32 (exact)
template <int k> __device__ __forceinline__ float sbyte(uint32_t v)
{
    return (float)((int32_t)(v << (24 - 8 * k)) >> 24);
}

// FORM: kWide (batch rows 0..15 on 16x16x4), kGroups (0..3 on 4x4x1, block
// 4g + s = 4-row group g of a tile over 8-weight slice s of a block), kSlices
// (0..3 on 4x4x1, block s = the 4 weights 4s .. 4s+3 of a pair for every
// 4-row group, so each activation is loaded by one lane, not four).
enum { kWide = 0, kGroups = 1, kSlices = 2 };
template <int T, int W, int FORM>
__global__ __launch_bounds__(64 * W) void gemv_q8_0_mfma_kernel(
    const uint8_t *__restrict__ w, const float *__restrict__ x, float *__restrict__ y, int M,
    int K, int B)
{
    constexpr int kRows = 16 * T;
    constexpr bool SMALL = FORM != kWide, SLICES = FORM == kSlices;
    constexpr int kBatch = SMALL ? 4 : 16;
    static_assert(kBatch * kRows <= 64 * W, "the reduction needs a thread per output");
    static_assert(W % 4 == 0, "a chunk of W pairs is whole 16-byte pieces");
    // weights of a chunk (W pairs of every row of the workgroup) in LDS: row
    // stride 17W + 4 dwords keeps 16-byte pieces aligned and spreads the rows
    // of a tile over the banks
    constexpr int kPieces = 17 * W / 4;       // 16-byte pieces of a row's chunk
    constexpr int kStride = 17 * W + 4;       // dwords
    constexpr int kPer = (kRows * kPieces + 64 * W - 1) / (64 * W); // pieces per thread
    __shared__ u32x4_t wbuf4[2][kRows * kStride / 4];
    __shared__ float red[W][kBatch][kRows]; // [wave][batch row][weight row]
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = tid >> 6;
    const int wr = SMALL ? ((lane >> 4) << 2) | (lane & 3) : lane & 15;
    const int ks = SMALL ? (lane >> 2) & 3 : lane >> 4;
    const int xb = SMALL ? lane & 3 : lane & 15;
    // kSlices: lane l = 4s + j takes activation row j and weight row 4g + j of
    // every 4-row group g, for the weights 4s .. 4s+3 of a pair (block s / 8,
    // quants from byte 34(s/8) + 2 + 4(s%8); the scale in the low or high
    // half of dword 8(s/8))
    const int sl = lane >> 2, jl = lane & 3;
    const int sblk = sl >> 3;
    const int qd = sblk ? 9 + (sl & 7) : (sl & 7), qsh = sblk ? 0 : 2;
    const int dd = 8 * sblk, dsh = 16 * sblk;
    const int r0 = (int)blockIdx.x * kRows;
    const int npair = K >> 6;
    const int nchunk = (npair + W - 1) / W;
    const int64_t row_bytes = (int64_t)(K >> 5) * kQ80Bytes;
    const bool xrow_ok = xb < B;
    const float *xrow = x + (int64_t)(xrow_ok ? xb : 0) * K;

    // staging: piece p = tid + 64W*n is 16 bytes of row p / kPieces at byte
    // 16 * (p % kPieces) of the chunk.  Pieces past the row's end are not
    // loaded (no wave reads those pairs); one that straddles it reads on into
    // the next row, or, on the matrix's last row, dword by dword up to its end.
    const uint8_t *src[kPer]; // row start
    int dst[kPer], pj[kPer];
    bool pok[kPer], plast[kPer];
#pragma unroll
    for (int n = 0; n < kPer; ++n) {
        const int p = tid + 64 * W * n;
        pok[n] = p < kRows * kPieces;
        const int row = pok[n] ? p / kPieces : 0, j = p % kPieces;
        src[n] = w + (int64_t)min(r0 + row, M - 1) * row_bytes;
        plast[n] = r0 + row >= M - 1;
        dst[n] = (row * kStride) / 4 + j;
        pj[n] = 16 * j;
    }
    u32x4_t stg[kPer];
    auto stage_load = [&](int c) {
        const int64_t base = (int64_t)c * (W * 2 * kQ80Bytes);
#pragma unroll
        for (int n = 0; n < kPer; ++n)
            if (pok[n]) {
                const int64_t pos = base + pj[n];
                if (pos + 16 <= row_bytes || (pos < row_bytes && !plast[n])) {
                    stg[n] = *(const u32x4a4_t *)(src[n] + pos);
                } else if (pos < row_bytes) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        stg[n][i] = pos + 4 * i < row_bytes ? *(g_u32 *)(src[n] + pos + 4 * i) : 0u;
                }
            }
    };
    auto stage_store = [&](int buf) {
#pragma unroll
        for (int n = 0; n < kPer; ++n)
            if (pok[n])
                wbuf4[buf][dst[n]] = stg[n];
    };

    struct Xs {
        float4 x0, x1, x2, x3;
    };
    auto load_x = [&](int m, Xs &p) {
        if (SLICES) {
            p.x0 = xrow_ok && m < npair ? ldf4(xrow + 64 * m + 4 * sl)
                                        : make_float4(0.f, 0.f, 0.f, 0.f);
        } else if (xrow_ok && m < npair) {
            const float *xp = xrow + 64 * m + 8 * ks;
            p.x0 = ldf4(xp);
            p.x1 = ldf4(xp + 4);
            p.x2 = ldf4(xp + 32);
            p.x3 = ldf4(xp + 36);
        } else {
            p.x0 = p.x1 = p.x2 = p.x3 = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };

    constexpr int G = SLICES ? 4 : 1; // 4-row groups held apart (kSlices)
    float acc[T][G][4];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[t][g][i] = 0.f;
    // this wave's pair of the chunk in buffer buf against activations p
    auto compute = [&](int buf, const Xs &p) {
        const uint32_t *wb = reinterpret_cast<const uint32_t *>(wbuf4[buf]);
        if constexpr (SLICES) {
            const float xv[4] = {p.x0.x, p.x0.y, p.x0.z, p.x0.w};
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const uint32_t *pr = wb + (16 * t + 4 * g + jl) * kStride + 17 * wave;
                    const uint32_t q = __builtin_amdgcn_alignbyte(pr[qd + 1], pr[qd], qsh);
                    const uint32_t dw = (pr[dd] >> dsh) & 0xffffu;
                    float4_t c = float4_t{0.f, 0.f, 0.f, 0.f};
                    c = __builtin_amdgcn_mfma_f32_4x4x1f32(xv[0], sbyte<0>(q), c, 0, 0, 0);
                    c = __builtin_amdgcn_mfma_f32_4x4x1f32(xv[1], sbyte<1>(q), c, 0, 0, 0);
                    c = __builtin_amdgcn_mfma_f32_4x4x1f32(xv[2], sbyte<2>(q), c, 0, 0, 0);
                    c = __builtin_amdgcn_mfma_f32_4x4x1f32(xv[3], sbyte<3>(q), c, 0, 0, 0);
                    const float d = half_to_float(dw);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[t][g][i] = fmaf(d, c[i], acc[t][g][i]);
                }
            return;
        }
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            const float4 u = blk ? p.x2 : p.x0, v = blk ? p.x3 : p.x1;
            const float xv[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const uint32_t *pr = wb + (16 * t + wr) * kStride + 17 * wave;
                uint32_t q0, q1, dw;
                if (blk == 0) {
                    const uint32_t a0 = pr[2 * ks], a1 = pr[2 * ks + 1], a2 = pr[2 * ks + 2];
                    q0 = __builtin_amdgcn_alignbyte(a1, a0, 2);
                    q1 = __builtin_amdgcn_alignbyte(a2, a1, 2);
                    dw = pr[0] & 0xffffu;
                } else {
                    q0 = pr[9 + 2 * ks];
                    q1 = pr[10 + 2 * ks];
                    dw = pr[8] >> 16;
                }
                const float wv[8] = {sbyte<0>(q0), sbyte<1>(q0), sbyte<2>(q0), sbyte<3>(q0),
                                     sbyte<0>(q1), sbyte<1>(q1), sbyte<2>(q1), sbyte<3>(q1)};
                float4_t c = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    c = SMALL ? __builtin_amdgcn_mfma_f32_4x4x1f32(xv[j], wv[j], c, 0, 0, 0)
                              : __builtin_amdgcn_mfma_f32_16x16x4f32(xv[j], wv[j], c, 0, 0, 0);
                const float d = half_to_float(dw);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[t][0][i] = fmaf(d, c[i], acc[t][0][i]);
            }
        }
    };

    // chunk c is computed from LDS buffer c % 2 while the loaded chunk c + 1
    // is stored into the other and the loads of chunk c + 2 go out
    // (kSlices, one float4 of activations per pair, loads them two chunks
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
        if (c * W + wave < npair)
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
        // sum the 16 slices of a pair (lanes 4, 8, 16 and 32 apart)
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
        // sum the four weight slices of a block (lanes 4 and 8 apart)
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
    if (tid < kBatch * kRows) {
        const int b = tid / kRows, r = tid % kRows;
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
    // batch 4 (and 3 on one-tile launches) on the slice form, whose
    // activation loads do not repeat per 4-row group; batch 2 on the group
    // form, which spends half the scaling FMAs (measured, kernel durations,
    // group -> slice form: 4096x14336 batch 4 37.4 -> 28.5 us, 11008x4096
    // 31.0 -> 23.5, 4096x4096 13.7 -> 12.0; batch 2 14336x4096 23.8 -> 28.0,
    // 4096x4096 10.7 -> 12.1; batch 3 14336x4096 25.5 -> 28.0)
    if (B == 4 || (B == 3 && T == 1))
        hipLaunchKernelGGL((gemv_q8_0_mfma_kernel<T, W, kSlices>), dim3(grid), dim3(64 * W), 0,
                           s, static_cast<const uint8_t *>(w), x, y, (int)M, (int)K, B);
    else if (B <= 4)
        hipLaunchKernelGGL((gemv_q8_0_mfma_kernel<T, W, kGroups>), dim3(grid), dim3(64 * W), 0,
                           s, static_cast<const uint8_t *>(w), x, y, (int)M, (int)K, B);
    else
        hipLaunchKernelGGL((gemv_q8_0_mfma_kernel<T, W, kWide>), dim3(grid), dim3(64 * W), 0, s,
                           static_cast<const uint8_t *>(w), x, y, (int)M, (int)K, B);
    return hipGetLastError();
}

} // namespace

hipError_t launch_gemv_q8_0_mfma(const void *w, const float *x, float *y, int64_t M, int64_t K,
                                 int B, hipStream_t s)
{
#ifdef LAB_T
    return go<LAB_T, LAB_W>(w, x, y, M, K, B, s);
#else
    // two tiles per workgroup halve the activation reads per weight row while
    // the grid still covers the chip twice over; eight-wave workgroups fit
    // two to a CU, which pays when there are more workgroups than CUs
    // (measured, kernel durations: 14336x4096 batch 2 23.8 us with two tiles
    // of eight waves; 11008x4096 one tile 24.6 us with eight waves, 28.6 with
    // sixteen; 4096-row matrices 10.5 us with sixteen waves, 15 with eight)
    const int64_t blocks2 = (M + 31) / 32, blocks1 = (M + 15) / 16;
    if (blocks2 >= 384)
        return go<2, 8>(w, x, y, M, K, B, s);
    if (blocks1 > device_cus())
        return go<1, 8>(w, x, y, M, K, B, s);
    return go<1, 16>(w, x, y, M, K, B, s);
#endif
}

} // namespace gq
