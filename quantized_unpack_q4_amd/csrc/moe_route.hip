// moe_route.hip -- expert routing of the mixture-of-experts layer on the device.
//
// The pages' engine does its own expert routing natively, next to the loader
// and the quantized kernels (page "Frink Inference: the Rust alternative to
// llama.cpp", opening paragraph).  Here each token's router logits pick its
// top-k experts and their weights: the softmax probabilities of the chosen
// experts, optionally renormalised to sum to one over them.
//
// One 16-lane row per token when E <= 64, one wave per token up to E = 256
// (four logits per lane either way); the reductions over a token's lanes are
// DPP moves inside a row plus, for whole waves, two wave permutes.  Softmax is
// strictly increasing, so the top-k experts are the top-k logits: they are
// chosen by exact comparison of the binary32 logits, equal logits going to the
// lower expert index, which keeps the ids independent of how the
// probabilities are rounded.  The probabilities are exp(l - max) / sum in
// binary32 (expf; the max and the sum are butterfly reductions over the
// token's lanes, the same order on every call).
#include "gq_device.h"
#include "gq_internal.h"

namespace gq {

namespace {

constexpr int kRouteWaves = 4; // waves per workgroup
constexpr int kPerLane = 4;    // logits per lane

// One cross-lane step of a reduction: row-local DPP moves for offsets 1, 2
// (quad permutes) and 4, 8 (row rotates), a full-wave permute for 16 and 32.
template <int STEP>
__device__ __forceinline__ int xlane(int v)
{
    if constexpr (STEP == 0)
        return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, true); // quad_perm [1,0,3,2]
    else if constexpr (STEP == 1)
        return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, true); // quad_perm [2,3,0,1]
    else if constexpr (STEP == 2)
        return __builtin_amdgcn_update_dpp(0, v, 0x124, 0xF, 0xF, true); // row_ror:4
    else if constexpr (STEP == 3)
        return __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, true); // row_ror:8
    else
        return __shfl_xor(v, STEP == 4 ? 16 : 32, 64);
}
template <int STEP>
__device__ __forceinline__ float xlanef(float v)
{
    return __builtin_bit_cast(float, xlane<STEP>(__builtin_bit_cast(int, v)));
}

// (value, index, probability) of the larger logit; equal values go to the
// lower index.  Empty slots carry -inf and an index of E or more, so a real
// expert always wins over them.
__device__ __forceinline__ void better(float &v, int &i, float &q, float v2, int i2, float q2)
{
    if (v2 > v || (v2 == v && i2 < i)) {
        v = v2;
        i = i2;
        q = q2;
    }
}

// Reductions over the L lanes of one token (L = 16: one DPP row; L = 64:
// the wave); every lane of the token ends with the result.
template <int L>
__device__ __forceinline__ float token_max(float v)
{
    v = fmaxf(v, xlanef<0>(v));
    v = fmaxf(v, xlanef<1>(v));
    v = fmaxf(v, xlanef<2>(v));
    v = fmaxf(v, xlanef<3>(v));
    if constexpr (L == 64) {
        v = fmaxf(v, xlanef<4>(v));
        v = fmaxf(v, xlanef<5>(v));
    }
    return v;
}
template <int L>
__device__ __forceinline__ float token_sum(float v)
{
    v += xlanef<0>(v);
    v += xlanef<1>(v);
    v += xlanef<2>(v);
    v += xlanef<3>(v);
    if constexpr (L == 64) {
        v += xlanef<4>(v);
        v += xlanef<5>(v);
    }
    return v;
}
template <int STEP>
__device__ __forceinline__ void argmax_step(float &v, int &i, float &q)
{
    better(v, i, q, xlanef<STEP>(v), xlane<STEP>(i), xlanef<STEP>(q));
}

// L lanes per token (16 for E <= 64, else 64); expert e = lane + L*j of the
// token sits in slot j of lane `lane` (its lane within the token).
template <int L>
__global__ __launch_bounds__(64 * kRouteWaves) void moe_route_kernel(
    const float *__restrict__ logits, int32_t *__restrict__ ids, float *__restrict__ wts, int T,
    int E, int topk, int renorm)
{
    const int lane = threadIdx.x & (L - 1);
    const int t = ((int)blockIdx.x * kRouteWaves * 64 + (int)threadIdx.x) / L;
    // a token's lanes are one DPP row (L = 16) or the whole wave (L = 64):
    // tokens past T leave together and no other token reads their lanes
    if (t >= T)
        return;
    const float *l = logits + (size_t)t * E;

    float v[kPerLane];
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
        const int e = lane + L * j;
        v[j] = e < E ? l[e] : -INFINITY;
    }
    float mx = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
    mx = token_max<L>(mx);
    float p[kPerLane], part = 0.f;
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
        p[j] = lane + L * j < E ? expf(v[j] - mx) : 0.f;
        part += p[j];
    }
    const float inv = 1.f / token_sum<L>(part);

    // k rounds of an arg-max over the logits not yet taken; slot s (expert id
    // and probability) is kept by lane s % L in register s / L
    bool taken[kPerLane] = {false, false, false, false};
    float mp[kPerLane] = {0.f, 0.f, 0.f, 0.f};
    int mid[kPerLane] = {0, 0, 0, 0};
    float chosen = 0.f; // sum of the chosen probabilities (the same on every lane)
    for (int s = 0; s < topk; ++s) {
        float bv = -INFINITY, bq = 0.f;
        int bi = 1 << 30;
#pragma unroll
        for (int j = 0; j < kPerLane; ++j)
            if (!taken[j])
                better(bv, bi, bq, v[j], lane + L * j, p[j]);
        argmax_step<0>(bv, bi, bq);
        argmax_step<1>(bv, bi, bq);
        argmax_step<2>(bv, bi, bq);
        argmax_step<3>(bv, bi, bq);
        if constexpr (L == 64) {
            argmax_step<4>(bv, bi, bq);
            argmax_step<5>(bv, bi, bq);
        }
        // every lane of the token now holds the winner (bi, its probability bq)
#pragma unroll
        for (int j = 0; j < kPerLane; ++j) {
            if (bi == lane + L * j)
                taken[j] = true;
            if (s == lane + L * j) {
                mp[j] = bq;
                mid[j] = bi;
            }
        }
        chosen += bq;
    }
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
        const int s = lane + L * j;
        if (s < topk) {
            ids[(size_t)t * topk + s] = mid[j];
            wts[(size_t)t * topk + s] = renorm ? mp[j] / chosen : mp[j] * inv;
        }
    }
}

} // namespace

hipError_t launch_moe_route(const float *logits, int32_t *ids, float *wts, int64_t T, int64_t E,
                            int64_t topk, bool renorm, hipStream_t s)
{
    const int per_block = 64 * kRouteWaves;
    if (E <= 64) {
        const int64_t blocks = (T * 16 + per_block - 1) / per_block;
        hipLaunchKernelGGL(moe_route_kernel<16>, dim3((unsigned)blocks), dim3(per_block), 0, s,
                           logits, ids, wts, (int)T, (int)E, (int)topk, renorm ? 1 : 0);
    } else {
        const int64_t blocks = (T * 64 + per_block - 1) / per_block;
        hipLaunchKernelGGL(moe_route_kernel<64>, dim3((unsigned)blocks), dim3(per_block), 0, s,
                           logits, ids, wts, (int)T, (int)E, (int)topk, renorm ? 1 : 0);
    }
    return hipGetLastError();
}

} // namespace gq
