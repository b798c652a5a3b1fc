// dequant.hip -- bit-exact dequantization probes (Q8_0, Q4_K) for gfx950.
//
// Each weight is the exact block value rounded once to binary32: for Q4_K,
// d*sc and dmin*m are exact binary32 products (at most 17 significant bits)
// and one fused multiply-add forms d*sc*q - dmin*m with a single rounding.
// The binary16 copy is that binary32 value rounded to nearest even
// (page "Building a Rust Inference Engine That Matches Llama.cpp", section
// "Where the wins came from": the same values the fused products consume).
#include "gq_device.h"
#include "gq_internal.h"

namespace gq {

// One thread per 4 consecutive weights of a Q4_K super-block; 64 threads per
// super-block, 4 super-blocks per 256-thread workgroup.
__global__ __launch_bounds__(256) void dequant_q4k_kernel(const uint8_t *__restrict__ w,
                                                          float *__restrict__ out32,
                                                          uint16_t *__restrict__ out16,
                                                          int64_t nsb)
{
    const int64_t sb = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (sb >= nsb)
        return;
    const int t = threadIdx.x & 63;
    const int k = 4 * t;          // first of this thread's 4 weights
    const int j = k >> 5;         // sub-block
    const int g = k >> 6;         // 32-byte quant group
    const int hi = (k >> 5) & 1;  // high nibbles for the second half of the group
    const uint8_t *blk = w + sb * kQ4kBytes;
    const uint4 h = ld16(blk);
    uint32_t sc, m;
    q4k_scale_min(h.y, h.z, h.w, j, sc, m);
    const float dsc = half_to_float(h.x) * (float)sc;
    const float dmm = half_to_float(h.x >> 16) * (float)m;
    const uint32_t q4 = *reinterpret_cast<const uint32_t *>(blk + 16 + 32 * g + (k & 31));
    const uint32_t nib = hi ? (q4 >> 4) & 0x0f0f0f0fu : q4 & 0x0f0f0f0fu;
    float v[4];
    v[0] = fmaf(dsc, ubyte_to_float<0>(nib), -dmm);
    v[1] = fmaf(dsc, ubyte_to_float<1>(nib), -dmm);
    v[2] = fmaf(dsc, ubyte_to_float<2>(nib), -dmm);
    v[3] = fmaf(dsc, ubyte_to_float<3>(nib), -dmm);
    const int64_t o = sb * kQ4kWeights + k;
    if (out32)
        *reinterpret_cast<float4 *>(out32 + o) = make_float4(v[0], v[1], v[2], v[3]);
    if (out16)
        *reinterpret_cast<uint2 *>(out16 + o) = make_uint2(pack_half2(v[0], v[1]),
                                                           pack_half2(v[2], v[3]));
}

// One thread per 2 weights of a Q8_0 block; 16 threads per block.  Blocks are
// 34 bytes, so a block starts on an even byte; quants are read in pairs.
__global__ __launch_bounds__(256) void dequant_q8_0_kernel(const uint8_t *__restrict__ w,
                                                           float *__restrict__ out32,
                                                           uint16_t *__restrict__ out16,
                                                           int64_t nblk)
{
    const int64_t b = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    if (b >= nblk)
        return;
    const int t = threadIdx.x & 15;
    const uint8_t *blk = w + b * kQ80Bytes;
    const float d = half_to_float(*reinterpret_cast<const uint16_t *>(blk));
    const uint16_t qq = *reinterpret_cast<const uint16_t *>(blk + 2 + 2 * t);
    const float v0 = d * (float)(int8_t)(qq & 0xff);
    const float v1 = d * (float)(int8_t)(qq >> 8);
    const int64_t o = b * kQ80Weights + 2 * t;
    if (out32)
        *reinterpret_cast<float2 *>(out32 + o) = make_float2(v0, v1);
    if (out16)
        *reinterpret_cast<uint32_t *>(out16 + o) = pack_half2(v0, v1);
}

hipError_t launch_dequant_q4k(const void *w, float *out32, uint16_t *out16, int64_t M,
                              int64_t K, hipStream_t s)
{
    const int64_t nsb = M * (K / kQ4kWeights);
    const int64_t grid = (nsb + 3) / 4;
    hipLaunchKernelGGL(dequant_q4k_kernel, dim3((unsigned)grid), dim3(256), 0, s,
                       (const uint8_t *)w, out32, out16, nsb);
    return hipGetLastError();
}

hipError_t launch_dequant_q8_0(const void *w, float *out32, uint16_t *out16, int64_t M,
                               int64_t K, hipStream_t s)
{
    const int64_t nblk = M * (K / kQ80Weights);
    const int64_t grid = (nblk + 15) / 16;
    hipLaunchKernelGGL(dequant_q8_0_kernel, dim3((unsigned)grid), dim3(256), 0, s,
                       (const uint8_t *)w, out32, out16, nblk);
    return hipGetLastError();
}

} // namespace gq
