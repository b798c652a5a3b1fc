// probes.hip -- measurement probes, built into their own library
// (libgq_probe.so) and used only to measure the achievable ceilings that the
// kernels are compared with on the same device; not part of the gq C ABI.
//
//   gqp_stream_read  every 16-byte word of a buffer is read once and folded
//                    into one word per wave, so that the loads stay: either
//                    grid-stride with four 16-byte loads per thread in flight
//                    (kind 0) or each workgroup streaming its own contiguous
//                    range with eight loads per thread in flight (kind 1);
//                    kinds 2 and 3: the range form with non-temporal loads
//                    (every instruction reads whole cache lines), 256 or 512
//                    threads per workgroup;
//   gqp_mfma_f16     a register-only loop of v_mfma_f32_32x32x16_f16 on eight
//                    independent accumulators per wave, eight waves (two per
//                    SIMD) per workgroup.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));

constexpr int kReadThreads = 256;
constexpr int kMfmaThreads = 512;
constexpr int kMfmaChains = 8;

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const uint4 *__restrict__ p,
                                                                   long long n16,
                                                                   uint32_t *__restrict__ sink)
{
    const long long stride = (long long)gridDim.x * kReadThreads;
    long long i = (long long)blockIdx.x * kReadThreads + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
        acc ^= (a.x ^ a.y ^ a.z ^ a.w) ^ (b.x ^ b.y ^ b.z ^ b.w) ^ (c.x ^ c.y ^ c.z ^ c.w) ^
               (d.x ^ d.y ^ d.z ^ d.w);
    }
    for (; i < n16; i += stride) {
        const uint4 a = p[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        acc ^= (uint32_t)__shfl_xor((int)acc, off, 64);
    if ((threadIdx.x & 63) == 0)
        sink[(long long)blockIdx.x * (kReadThreads / 64) + threadIdx.x / 64] = acc;
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4 g_u32x4;

template <bool NT = false, int T = kReadThreads>
__global__ __launch_bounds__(T) void range_read_kernel(const uint4 *__restrict__ p, long long n16,
                                                       uint32_t *__restrict__ sink)
{
    constexpr int U = 8;
    const long long lo = n16 * blockIdx.x / gridDim.x, hi = n16 * (blockIdx.x + 1) / gridDim.x;
    long long i = lo + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (U - 1) * T < hi; i += U * T) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const g_u32x4 *a = (const g_u32x4 *)(p + i + u * T);
            const u32x4 t = NT ? __builtin_nontemporal_load(a) : *a;
            v[u] = make_uint4(t.x, t.y, t.z, t.w);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < hi; i += T) {
        const uint4 a = p[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        acc ^= (uint32_t)__shfl_xor((int)acc, off, 64);
    if ((threadIdx.x & 63) == 0)
        sink[(long long)blockIdx.x * (T / 64) + threadIdx.x / 64] = acc;
}

__global__ __launch_bounds__(kMfmaThreads, 1) void mfma_f16_kernel(float *__restrict__ sink,
                                                                   int iters)
{
    half8_t a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (_Float16)(0.001f * (float)(threadIdx.x & 63));
        b[i] = (_Float16)(0.01f * (float)i);
    }
    float16_t c[kMfmaChains];
#pragma unroll
    for (int j = 0; j < kMfmaChains; ++j)
        c[j] = float16_t{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < kMfmaChains; ++j)
            c[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c[j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kMfmaChains; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v)
            s += c[j][v];
    sink[(long long)blockIdx.x * kMfmaThreads + threadIdx.x] = s;
}

} // namespace

// Reads `bytes` (a multiple of 16) from buf with `grid` workgroups of 256
// threads, in form `kind` (0 or 1, see above); sink holds grid * 4 words.
// Returns the hipError_t of the launch.
extern "C" int gqp_stream_read(const void *buf, long long bytes, uint32_t *sink, int grid,
                               int kind, void *stream)
{
    if (!buf || !sink || bytes <= 0 || bytes % 16 != 0 || grid <= 0 || kind < 0 || kind > 3)
        return (int)hipErrorInvalidValue;
    const uint4 *p = (const uint4 *)buf;
    const hipStream_t s = (hipStream_t)stream;
    if (kind == 0)
        hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(kReadThreads), 0, s, p,
                           bytes / 16, sink);
    else if (kind == 1)
        hipLaunchKernelGGL((range_read_kernel<false>), dim3((unsigned)grid), dim3(kReadThreads),
                           0, s, p, bytes / 16, sink);
    else if (kind == 2)
        hipLaunchKernelGGL((range_read_kernel<true>), dim3((unsigned)grid), dim3(kReadThreads), 0,
                           s, p, bytes / 16, sink);
    else
        hipLaunchKernelGGL((range_read_kernel<true, 512>), dim3((unsigned)grid), dim3(512), 0, s,
                           p, bytes / 16, sink);
    return (int)hipGetLastError();
}

// grid workgroups of 512 threads, each wave `iters` rounds of 8 matrix
// instructions; sink holds grid * 512 floats.  Floating-point operations per
// launch: grid * 8 waves * iters * 8 * 2 * 32 * 32 * 16.
extern "C" int gqp_mfma_f16(float *sink, int iters, int grid, void *stream)
{
    if (!sink || iters <= 0 || grid <= 0)
        return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(mfma_f16_kernel, dim3((unsigned)grid), dim3(kMfmaThreads), 0,
                       (hipStream_t)stream, sink, iters);
    return (int)hipGetLastError();
}

extern "C" long long gqp_mfma_f16_flops(int iters, int grid)
{
    return (long long)grid * (kMfmaThreads / 64) * iters * kMfmaChains * 2LL * 32 * 32 * 16;
}
