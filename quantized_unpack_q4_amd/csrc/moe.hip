// moe.hip -- grouping and combine steps of the mixture-of-experts layer.
//
// The pages' engines run mixture-of-experts checkpoints with their own expert
// routing (page "Frink Inference: the Rust alternative to llama.cpp", opening
// paragraph; page "Building a Rust Inference Engine That Matches
// Llama.cpp", section "Utility": OLMoE-1B-7B).  Given each token's top-k
// expert ids and weights, the layer here is four launches on one stream:
//   1. group    one workgroup counts assignments per expert, scans the counts,
//               lists the token tiles of every expert and gives each
//               (token, slot) assignment a stable position in expert order
//               (ties keep assignment order, so the result is deterministic);
//   2. gate/up  grouped matrix product with the SwiGLU epilogue (gemm.hip, or
//               moe_skinny.hip when the experts average 48 tokens or fewer);
//   3. down     grouped matrix product into binary32 rows (likewise);
//   4. combine  out[t] = sum over slots, in slot order, of weight * row.
// No atomics touch the outputs and nothing waits on the host.
#include "gq_device.h"
#include "gq_internal.h"

namespace gq {

constexpr int kMaxExperts = 256;
constexpr int kGroupThreads = 1024;
constexpr int kGroupWaves = kGroupThreads / 64;

hipError_t launch_moe_gemms(const MoeArgs &a, int bn, int max_tiles, hipStream_t s);

int moe_token_tile(int64_t assignments, int64_t experts)
{
    const int64_t mean = assignments / (experts > 0 ? experts : 1);
    return mean <= 48 ? 32 : mean <= 96 ? 64 : 128;
}

// offsets[0..E-1]: first sorted position of each expert; offsets[E]: number of
// valid assignments; offsets[E+1]: number of token tiles; offsets[E+2]:
// assignments dropped because their id lies outside [0, E).
__global__ __launch_bounds__(kGroupThreads) void moe_group_kernel(
    const int32_t *__restrict__ ids, int A, int E, int BN, int max_tiles,
    int32_t *__restrict__ offsets, int32_t *__restrict__ sorted, int32_t *__restrict__ pos_of,
    int32_t *__restrict__ tiles)
{
    __shared__ int cnt[kMaxExperts];
    __shared__ int base[kMaxExperts];
    __shared__ int wcnt[kGroupWaves][kMaxExperts];
    __shared__ int ndrop;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    for (int e = tid; e < E; e += kGroupThreads)
        cnt[e] = 0;
    if (tid == 0)
        ndrop = 0;
    __syncthreads();
    for (int a = tid; a < A; a += kGroupThreads) {
        const int e = ids[a];
        if (e >= 0 && e < E)
            atomicAdd(&cnt[e], 1);
        else
            atomicAdd(&ndrop, 1);
    }
    __syncthreads();
    if (tid == 0) {
        int off = 0, nt = 0;
        for (int e = 0; e < E; ++e) {
            base[e] = off;
            offsets[e] = off;
            for (int p = off; p < off + cnt[e]; p += BN) {
                tiles[nt] = e;
                tiles[max_tiles + nt] = p;
                ++nt;
            }
            off += cnt[e];
        }
        offsets[E] = off;
        offsets[E + 1] = nt;
        offsets[E + 2] = ndrop;
    }
    __syncthreads();

    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int c0 = 0; c0 < A; c0 += kGroupThreads) {
        const int a = c0 + tid;
        const int e = a < A ? ids[a] : -1;
        const bool valid = e >= 0 && e < E;
        // lanes of this wave holding the same expert id
        uint64_t peers = __ballot(valid);
#pragma unroll
        for (int bit = 0; bit < 8; ++bit) {
            const bool set = valid && ((e >> bit) & 1);
            const uint64_t b = __ballot(set);
            peers &= set ? b : ~b;
        }
        const int rank = __popcll(peers & below);
        for (int i = tid; i < kGroupWaves * E; i += kGroupThreads)
            wcnt[i / E][i % E] = 0;
        __syncthreads();
        if (valid && rank == 0)
            wcnt[wave][e] = __popcll(peers);
        __syncthreads();
        for (int x = tid; x < E; x += kGroupThreads) {
            int run = base[x];
            for (int w = 0; w < kGroupWaves; ++w) {
                const int t = wcnt[w][x];
                wcnt[w][x] = run;
                run += t;
            }
            base[x] = run;
        }
        __syncthreads();
        if (valid) {
            const int pos = wcnt[wave][e] + rank;
            sorted[pos] = a;
            pos_of[a] = pos;
        } else if (a < A) {
            pos_of[a] = -1;
        }
        __syncthreads();
    }
}

// One thread per 4 output columns of one token.
__global__ __launch_bounds__(256) void moe_combine_kernel(const float *__restrict__ D,
                                                          const int32_t *__restrict__ pos_of,
                                                          const float *__restrict__ wts,
                                                          uint16_t *__restrict__ out, int H,
                                                          int topk, int col_blocks)
{
    const int t = blockIdx.x / col_blocks;
    const int c = ((blockIdx.x % col_blocks) * 256 + threadIdx.x) * 4;
    if (c >= H)
        return;
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    for (int s = 0; s < topk; ++s) {
        const int pos = pos_of[(int64_t)t * topk + s];
        if (pos < 0)
            continue;
        const float wgt = wts[(int64_t)t * topk + s];
        const float4 d = ldf4(D + (int64_t)pos * H + c);
        a0 = fmaf(wgt, d.x, a0);
        a1 = fmaf(wgt, d.y, a1);
        a2 = fmaf(wgt, d.z, a2);
        a3 = fmaf(wgt, d.w, a3);
    }
    *reinterpret_cast<uint2 *>(out + (int64_t)t * H + c) =
        make_uint2(pack_half2(a0, a1), pack_half2(a2, a3));
}

hipError_t launch_moe(const MoeArgs &a, hipStream_t s)
{
    const int64_t A = a.T * a.topk;
    const int bn = moe_token_tile(A, a.E);
    const int max_tiles = (int)((A + bn - 1) / bn + a.E);
    int32_t *offsets = reinterpret_cast<int32_t *>(a.ws + a.off[0]);
    int32_t *sorted = reinterpret_cast<int32_t *>(a.ws + a.off[1]);
    int32_t *pos_of = reinterpret_cast<int32_t *>(a.ws + a.off[2]);
    int32_t *tiles = reinterpret_cast<int32_t *>(a.ws + a.off[3]);
    hipLaunchKernelGGL(moe_group_kernel, dim3(1), dim3(kGroupThreads), 0, s, a.ids, (int)A,
                       (int)a.E, bn, max_tiles, offsets, sorted, pos_of, tiles);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    err = moe_skinny_applies(A, a.E) ? launch_moe_skinny(a, s)
                                     : launch_moe_gemms(a, bn, max_tiles, s);
    if (err != hipSuccess)
        return err;
    const int col_blocks = (int)((a.H / 4 + 255) / 256);
    hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)(a.T * col_blocks)), dim3(256), 0, s,
                       reinterpret_cast<const float *>(a.ws + a.off[5]), pos_of, a.wts, a.out,
                       (int)a.H, (int)a.topk, col_blocks);
    return hipGetLastError();
}

} // namespace gq
