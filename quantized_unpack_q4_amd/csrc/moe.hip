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
//   2. gate/up  grouped matrix product with the SwiGLU epilogue (gemm.hip;
//               moe_skinny.hip when the experts average 48 tokens or fewer,
//               the 256 x 256 tiles of gemm_big.hip from 160 on);
//   3. down     grouped matrix product into binary32 rows (likewise);
//   4. combine  out[t] = sum over slots, in slot order, of weight * row.
// No atomics touch the outputs and nothing waits on the host.
#include "gq_device.h"
#include "gq_internal.h"

namespace gq {

constexpr int kMaxExperts = 256;
constexpr int kGroupThreads = 1024;
constexpr int kGroupWaves = kGroupThreads / 64;
constexpr int kGroupBatch = 16;

hipError_t launch_moe_gemms(const MoeArgs &a, int bn, int max_tiles, hipStream_t s);

int moe_token_tile(int64_t assignments, int64_t experts)
{
    const int64_t mean = assignments / (experts > 0 ? experts : 1);
    return mean <= 48 ? 32 : mean <= 96 ? 64 : 128;
}

// Lanes of this wave whose valid expert id equals this lane's (8 ballots over
// the id bits, E <= 256).
__device__ __forceinline__ uint64_t same_expert_lanes(bool valid, int e)
{
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
        const bool set = valid && ((e >> bit) & 1);
        const uint64_t b = __ballot(set);
        peers &= set ? b : ~b;
    }
    return peers;
}

// Exclusive prefix sum of v over threads 0 .. 64*nw - 1 (nw <= 4 waves);
// every thread of the workgroup must call it.  Returns the exclusive prefix
// and sets *total.
__device__ __forceinline__ int block_exclusive_scan(int v, int nw, int *scratch, int *total)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int inc = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int u = __shfl_up(inc, off, 64);
        if (lane >= off)
            inc += u;
    }
    if (wave < nw && lane == 63)
        scratch[wave] = inc;
    __syncthreads();
    int before = 0, all = 0;
    for (int w = 0; w < nw; ++w) {
        before += w < wave ? scratch[w] : 0;
        all += scratch[w];
    }
    __syncthreads();
    *total = all;
    return before + inc - v;
}

// offsets[0..E-1]: first sorted position of each expert; offsets[E]: number of
// valid assignments; offsets[E+1]: number of token tiles; offsets[E+2]:
// assignments dropped because their id lies outside [0, E).
//
// Wave w owns the contiguous slice [w*S, (w+1)*S) of the assignments: it
// counts its slice per expert (LDS adds into its own counters), one scan
// across waves and experts turns the counts into starting positions, and a
// second walk of the slice hands out positions in assignment order (ballot
// ranking among the lanes of a chunk with the same expert), so the order is
// stable by (expert, assignment index) and no atomic touches a position.  Both walks load the ids of up to
// kGroupBatch 64-id chunks at once before processing them in order, so a
// walk waits for one load latency per batch rather than one per chunk.
__global__ __launch_bounds__(kGroupThreads) void moe_group_kernel(
    const int32_t *__restrict__ ids, int A, int E, int BN, int max_tiles,
    int32_t *__restrict__ offsets, int32_t *__restrict__ sorted, int32_t *__restrict__ pos_of,
    int32_t *__restrict__ tiles)
{
    __shared__ int wstart[kGroupWaves][kMaxExperts]; // per wave: count, then first position
    __shared__ int wdrop[kGroupWaves];
    __shared__ int scratch[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int S = (A + kGroupWaves - 1) / kGroupWaves;
    const int a_begin = wave * S, a_end = min(A, a_begin + S);
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

    for (int i = tid; i < kGroupWaves * kMaxExperts; i += kGroupThreads)
        wstart[i / kMaxExperts][i % kMaxExperts] = 0;
    __syncthreads();

    // ids of chunks c0, c0 + 64, ... (kGroupBatch of them), -1 past the slice
    auto load_batch = [&](int c0, int (&ev)[kGroupBatch]) {
#pragma unroll
        for (int u = 0; u < kGroupBatch; ++u) {
            const int a = c0 + 64 * u + lane;
            ev[u] = a < a_end ? ids[a] : -1;
        }
    };

    // 1. per-wave counts
    int drop = 0;
    for (int c0 = a_begin; c0 < a_end; c0 += 64 * kGroupBatch) {
        int ev[kGroupBatch];
        load_batch(c0, ev);
#pragma unroll
        for (int u = 0; u < kGroupBatch; ++u) {
            const int a = c0 + 64 * u + lane;
            if (c0 + 64 * u >= a_end)
                break; // wave-uniform
            const int e = ev[u];
            const bool valid = e >= 0 && e < E;
            // counts only: one LDS add per assignment (a sum, so the order
            // of the adds does not matter)
            if (valid)
                atomicAdd(&wstart[wave][e], 1);
            drop += __popcll(__ballot(a < a_end && !valid));
        }
    }
    if (lane == 0)
        wdrop[wave] = drop;
    __syncthreads();

    // 2. per expert: total count, then expert bases and token tiles (scans
    // over experts, E <= 256 = 4 waves of threads)
    const int nw = (E + 63) / 64;
    int cnt = 0;
    if (tid < E) {
        for (int w = 0; w < kGroupWaves; ++w)
            cnt += wstart[w][tid];
    }
    int total_valid = 0, total_big = 0, total_small = 0;
    const int base = block_exclusive_scan(tid < E ? cnt : 0, nw, scratch, &total_valid);
    const int ntile = tid < E ? (cnt + BN - 1) / BN : 0;
    // tiles of 64 tokens or fewer (an expert's remainder when BN > 64) are
    // the cheapest: they go after every other tile, so that they fill the
    // last round of workgroups instead of leaving large tiles for it
    const int rem = tid < E ? cnt % BN : 0;
    const int nsmall = BN > 64 && rem > 0 && rem <= 64 ? 1 : 0;
    const int nbig = ntile - nsmall;
    const int tbase = block_exclusive_scan(nbig, nw, scratch, &total_big);
    const int sbase = block_exclusive_scan(nsmall, nw, scratch, &total_small);
    const int total_tiles = total_big + total_small;
    if (tid < E) {
        offsets[tid] = base;
        int run = base;
        for (int w = 0; w < kGroupWaves; ++w) {
            const int t = wstart[w][tid];
            wstart[w][tid] = run;
            run += t;
        }
        for (int i = 0; i < nbig; ++i) {
            tiles[tbase + i] = tid;
            tiles[max_tiles + tbase + i] = base + i * BN;
        }
        if (nsmall) {
            tiles[total_big + sbase] = tid;
            tiles[max_tiles + total_big + sbase] = base + nbig * BN;
        }
    }
    if (tid == 0) {
        int nd = 0;
        for (int w = 0; w < kGroupWaves; ++w)
            nd += wdrop[w];
        offsets[E] = total_valid;
        offsets[E + 1] = total_tiles;
        offsets[E + 2] = nd;
    }
    __syncthreads();

    // 3. positions, in assignment order within each wave's slice
    for (int c0 = a_begin; c0 < a_end; c0 += 64 * kGroupBatch) {
        int ev[kGroupBatch];
        load_batch(c0, ev);
#pragma unroll
        for (int u = 0; u < kGroupBatch; ++u) {
            const int a = c0 + 64 * u + lane;
            if (c0 + 64 * u >= a_end)
                break; // wave-uniform
            const int e = ev[u];
            const bool valid = e >= 0 && e < E;
            const uint64_t peers = same_expert_lanes(valid, e);
            const int rank = __popcll(peers & below);
            const int pos = valid ? wstart[wave][e] + rank : -1;
            if (valid && rank == 0)
                wstart[wave][e] += __popcll(peers);
            if (valid)
                sorted[pos] = a;
            if (a < a_end)
                pos_of[a] = pos;
        }
    }
}

// One thread per 4 output columns of one token.
__global__ __launch_bounds__(256) void moe_combine_kernel(const float *__restrict__ D,
                                                          const int32_t *__restrict__ pos_of,
                                                          const float *__restrict__ wts,
                                                          uint16_t *__restrict__ out, int H,
                                                          int topk, int col_blocks, int unit)
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
        const float wgt = unit ? 1.f : wts[(int64_t)t * topk + s];
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
    // the 256 x 256 tiles take whole runs of 256 weights: Q8_0 stacks whose
    // H or I is not a multiple of 256 use the 128-row tile kernel instead
    const bool big = moe_big_applies(A, a.E, a.H, a.I) && (!a.q8_0 || a.I % 256 == 0);
    const int bn = big ? moe_big_token_tile() : moe_token_tile(A, a.E);
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
    err = big ? launch_moe_big(a, max_tiles, s)
              : moe_skinny_applies(A, a.E) ? launch_moe_skinny(a, s)
                                           : launch_moe_gemms(a, bn, max_tiles, s);
    if (err != hipSuccess)
        return err;
    const int col_blocks = (int)((a.H / 4 + 255) / 256);
    hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)(a.T * col_blocks)), dim3(256), 0, s,
                       reinterpret_cast<const float *>(a.ws + a.off[5]), pos_of, a.wts, a.out,
                       (int)a.H, (int)a.topk, col_blocks, a.weight_input);
    return hipGetLastError();
}

} // namespace gq
