// gq_device.h -- device-side helpers shared by the gfx950 kernels of libgq.
//
// Block formats (GGUF, as loaded by the engines on the page "Building a Rust
// Inference Engine That Matches Llama.cpp", section "What Ferrox actually
// is"):
//   Q8_0  34 B / 32 weights: binary16 d, 32 x int8 q            w = d*q
//   Q4_K 144 B / 256 weights: binary16 d, binary16 dmin, 12 B of 6-bit
//         scales/mins, 128 B of 4-bit quants               w = d*sc*q - dmin*m
// A Q4_K super-block is read as nine 16-byte words: word 0 is the header
// (dword 0 = d | dmin << 16, dwords 1..3 = the 12 scale/min bytes) and words
// 1..8 are the quants; quant byte 32g+i carries weight 64g+i in its low nibble
// and weight 64g+32+i in its high nibble.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gq {

constexpr int kQ4kBytes = 144;
constexpr int kQ4kWeights = 256;
constexpr int kQ80Bytes = 34;
constexpr int kQ80Weights = 32;

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float half_to_float(uint32_t bits16)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits16 & 0xffffu));
}

// Two binary32 values rounded to binary16 (nearest even) and packed lo | hi << 16.
__device__ __forceinline__ uint32_t pack_half2(float lo, float hi)
{
    typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
    half2_t v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// Byte n (0..3) of a dword as a float (v_cvt_f32_ubyte{n}).
template <int n>
__device__ __forceinline__ float ubyte_to_float(uint32_t v)
{
    return (float)((v >> (8 * n)) & 0xffu);
}

// 6-bit scale and min of sub-block j from header dwords h1 = s[0..3],
// h2 = s[4..7], h3 = s[8..11].  Sub-blocks 0..3 hold both values in the low
// six bits of s[j] and s[j+4]; sub-blocks 4..7 take the low four bits from
// the nibbles of s[j+4] and the top two bits from bits 6..7 of s[j-4] (scale)
// and s[j] (min).
__device__ __forceinline__ void q4k_scale_min(uint32_t h1, uint32_t h2, uint32_t h3, int j,
                                              uint32_t &sc, uint32_t &m)
{
    if (j < 4) {
        sc = (h1 >> (8 * j)) & 63u;
        m = (h2 >> (8 * j)) & 63u;
    } else {
        const int s = 8 * (j - 4);
        sc = ((h3 >> s) & 15u) | (((h1 >> (s + 6)) & 3u) << 4);
        m = ((h3 >> (s + 4)) & 15u) | (((h2 >> (s + 6)) & 3u) << 4);
    }
}

// SwiGLU gate activation silu(z) = z / (1 + e^-z) in binary32 (the mixture-of-
// experts gate/up epilogues; the oracle evaluates it in binary64).
__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        v += __shfl_xor(v, off, 64);
    return v;
}

__device__ __forceinline__ uint4 ld16(const void *p)
{
    return *reinterpret_cast<const uint4 *>(p);
}

__device__ __forceinline__ float4 ldf4(const float *p)
{
    return *reinterpret_cast<const float4 *>(p);
}

} // namespace gq
