// moe_skinny.hip -- the grouped expert products of the mixture-of-experts layer
// when each expert sees few tokens.
//
// With 256 tokens, top-8 routing and 64 experts (the OLMoE-shaped layer the
// pages run, page "Building a Rust Inference Engine That Matches Llama.cpp",
// section "Utility"), an expert gets about 32 tokens: the expert products are
// skinny and the layer is bound by streaming the 226 MB of packed expert
// weights, not by the matrix cores.  This kernel streams each weight once per
// chunk of up to 64 tokens of its expert:
//   * a workgroup (4 waves) owns 64 rows of one expert's matrix (64 rows of
//     gate and the same 64 rows of up in the gate/up product), all of K;
//   * per super-block, the token slices it needs (up to 64 rows x 256 binary16
//     activations, gathered through the expert's sorted assignment list) are
//     copied global -> LDS by direct-to-LDS loads, one super-block ahead, into
//     a bank-swizzled layout;
//   * each lane dequantizes its own weights straight into the operand of
//     v_mfma_f32_16x16x32_f16, w16 = binary16(binary32(d*sc*q - dmin*m)) by one
//     mixed-precision FMA per weight from the quant taken as the binary16
//     subnormal q*2^-24 (the same binary16 weights as the tiled products), no
//     LDS round trip;
//   * binary32 accumulation over all of K, then the SwiGLU epilogue
//     h = binary16(silu(g) * u) (gate/up) or binary32 rows (down), written in
//     the expert-sorted order the combine step reads.
// Q8_0 expert stacks take the same schedule: 256 weights of a row are eight
// 34-byte blocks, 272 bytes starting 16-byte aligned, and each lane owns two
// whole blocks (its quarter's 64 weights, 68 bytes, four 16-byte and one
// 4-byte load).  The matrix-core k order inside each 32-weight step is
// permuted alike for weights and activations, so that step j takes weights
// 8j .. 8j+7 of every quarter; w16 = binary16(d * q), exact before the one
// rounding.
#include "gq_device.h"
#include "gq_internal.h"

namespace gq {

namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4 g_u32x4;
typedef __attribute__((address_space(1))) const u32x2 g_u32x2;
typedef unsigned int u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef __attribute__((address_space(1))) const u32x4a4 g_u32x4a4;
typedef __attribute__((address_space(1))) const unsigned int g_u32;

constexpr int kQ8Step = 8 * kQ80Bytes; // 272 bytes: 256 weights of a Q8_0 row

constexpr int SR = 64;  // weight rows per workgroup
constexpr int ST = 64;  // tokens per chunk (up to 4 groups of 16)
constexpr int NT = 256; // threads per workgroup

struct SkinnyParams {
    const uint8_t *w, *w2;  // stacked Q4_K expert matrices (w2: up, gate/up product only)
    const uint16_t *x;      // gate/up: x [T][K]; down: h [A][K] in sorted order
    // (w, w2: Q8_0 stacks in the Q8 instances)
    void *y;                // gate/up: h [A][M] binary16; down: d [A][M] binary32
    const int32_t *offsets; // expert start positions in sorted order, [E] = total
    const int32_t *sorted;  // assignment t*topk + s at each sorted position
    int M, K, topk;
    int64_t expert_bytes;
    const float *wts; // gate/up with weight_input: the slot weights, [T*topk]
    int weight_input;
};

// 16 bytes per lane, global -> LDS; lane l lands at lds_base + 16*l (lds_base
// wave-uniform).  Inline assembly keeps it out of the compiler's wait
// insertion: the kernel retires it with an explicit vmcnt(0) before the
// barrier that publishes the data.
__device__ __forceinline__ void dma16(const void *gsrc, const void *lds_base)
{
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(
        (uint32_t)(size_t)(const __attribute__((address_space(3))) void *)lds_base);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gsrc), "s"(m0)
                 : "memory", "m0");
}

// Two binary16 weights from two quants taken as binary16 subnormals and the
// binary32 scale s and offset o: binary16(binary32(s*q + o)) each, packed.
// Two binary32 mixed-precision FMAs and one packed round-to-nearest
// conversion, written out: the fused binary16-result forms of the FMA take
// about twice the issue time of either.
__device__ __forceinline__ uint32_t deq2(uint32_t qa, int sela, uint32_t qb, int selb, float s,
                                         float o)
{
    const h2_t a = __builtin_bit_cast(h2_t, qa), b = __builtin_bit_cast(h2_t, qb);
    const float lo = fmaf((float)(sela ? a.y : a.x), s, o);
    const float hi = fmaf((float)(selb ? b.y : b.x), s, o);
    uint32_t r;
    asm("v_cvt_pk_f16_f32 %0, %1, %2" : "=v"(r) : "v"(lo), "v"(hi));
    return r;
}

// This lane's packed weights of one super-block: the header of its row and
// the 32 bytes of quant group `quarter`, i.e. sub-blocks 2*quarter (low
// nibbles) and 2*quarter + 1 (high nibbles).
struct WSb {
    uint4 h, qa, qb;
};

__device__ __forceinline__ uint4 gload16(const uint8_t *p)
{
    const u32x4 v = *(g_u32x4 *)p;
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void load_wsb(const uint8_t *row, int sb, int quarter, WSb &w)
{
    const uint8_t *blk = row + (size_t)sb * kQ4kBytes;
    w.h = gload16(blk);
    w.qa = gload16(blk + 16 + 32 * quarter);
    w.qb = gload16(blk + 32 + 32 * quarter);
}

// Q8_0: this lane's two blocks (2*quarter, 2*quarter + 1) of one 256-weight
// step, as 17 dwords: D[0] = scale 0 and quants 0, 1; quants 2..31 of block 0
// end in the low half of D[8], whose high half is scale 1; D[9..16] are the
// 32 quants of block 1.
struct WSb8 {
    uint32_t D[17];
};

__device__ __forceinline__ void load_wsb8(const uint8_t *row, int sb, int quarter, WSb8 &w)
{
    const uint8_t *p = row + (size_t)sb * kQ8Step + 68 * quarter;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const u32x4a4 v = *(g_u32x4a4 *)(p + 16 * i);
        w.D[4 * i] = v.x;
        w.D[4 * i + 1] = v.y;
        w.D[4 * i + 2] = v.z;
        w.D[4 * i + 3] = v.w;
    }
    w.D[16] = *(g_u32 *)(p + 64);
}

// Eight binary16 weights binary16(d * q) from eight signed quant bytes; the
// byte is converted as (q ^ 0x80) - 128 through an unsigned conversion, and
// d * u - 128 d is exact in binary32 (at most 19 significant bits).
__device__ __forceinline__ half8_t deq8(uint32_t q0, uint32_t q1, float d)
{
    const uint32_t a = q0 ^ 0x80808080u, b = q1 ^ 0x80808080u;
    const float o = -128.f * d;
    const uint4 v = make_uint4(
        pack_half2(fmaf(d, ubyte_to_float<0>(a), o), fmaf(d, ubyte_to_float<1>(a), o)),
        pack_half2(fmaf(d, ubyte_to_float<2>(a), o), fmaf(d, ubyte_to_float<3>(a), o)),
        pack_half2(fmaf(d, ubyte_to_float<0>(b), o), fmaf(d, ubyte_to_float<1>(b), o)),
        pack_half2(fmaf(d, ubyte_to_float<2>(b), o), fmaf(d, ubyte_to_float<3>(b), o)));
    return __builtin_bit_cast(half8_t, v);
}

template <bool Q8> struct WeightSet {
    typedef WSb type;
};
template <> struct WeightSet<true> {
    typedef WSb8 type;
};

// One chunk of up to 16*NG tokens of expert e: positions [p0, p0 + nc) of the
// sorted list.
template <int MODE, int NG, bool Q8>
__device__ __forceinline__ void run_chunk(const SkinnyParams &p, int e, int p0, int nc,
                                          _Float16 *xs0, _Float16 *xs1)
{
    typedef typename WeightSet<Q8>::type WS;
    constexpr int NMAT = MODE == 0 ? 2 : 1;
    constexpr int NDMA = NG * 2; // direct-to-LDS copies per wave per super-block
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, quarter = lane >> 4;
    const int K = p.K, M = p.M, nsb = K >> 8;
    const size_t rowb = (size_t)(K >> 8) * (Q8 ? kQ8Step : kQ4kBytes);
    const int row = (int)blockIdx.x * SR + wave * 16 + col;

    const uint8_t *wrow[NMAT];
    wrow[0] = p.w + (size_t)e * p.expert_bytes + (size_t)row * rowb;
    if constexpr (NMAT == 2)
        wrow[1] = p.w2 + (size_t)e * p.expert_bytes + (size_t)row * rowb;

    // copy i of this wave fills LDS bytes [1 KB * (NDMA*wave + i), +1 KB):
    // tokens t = 2*(NDMA*wave + i) + lane/32, slot lane%32, holding 16-byte
    // chunk (lane%32) ^ (t%32) of the token's 512-byte super-block slice
    const uint16_t *src[NDMA];
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
        const int t = 2 * (NDMA * wave + i) + (lane >> 5);
        const int tc = t < nc ? t : nc - 1;
        const int64_t xrow =
            MODE == 0 ? (int64_t)(p.sorted[p0 + tc] / p.topk) : (int64_t)(p0 + tc);
        src[i] = p.x + xrow * K + 8 * ((lane & 31) ^ (t & 31));
    }
    auto issue_x = [&](int sb, _Float16 *buf) {
#pragma unroll
        for (int i = 0; i < NDMA; ++i)
            dma16(src[i] + 256 * sb, buf + 512 * (NDMA * wave + i));
    };

    float4_t acc[NMAT][NG];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int g = 0; g < NG; ++g)
            acc[m][g] = float4_t{0.f, 0.f, 0.f, 0.f};

    // Q8_0: step j pairs weights 64*quarter + 8j .. +7 of every row with the
    // activations of the same k, 16-byte chunk 8*quarter + j of the slice
    auto compute8 = [&](const _Float16 *buf, const WSb8 (&w)[NMAT]) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            half8_t bop[NMAT];
#pragma unroll
            for (int m = 0; m < NMAT; ++m) {
                const uint32_t *D = w[m].D;
                if (j < 4)
                    bop[m] = deq8(__builtin_amdgcn_alignbyte(D[2 * j + 1], D[2 * j], 2),
                                  __builtin_amdgcn_alignbyte(D[2 * j + 2], D[2 * j + 1], 2),
                                  half_to_float(D[0] & 0xffffu));
                else
                    bop[m] = deq8(D[2 * j + 1], D[2 * j + 2], half_to_float(D[8] >> 16));
            }
            const int c = 8 * quarter + j;
#pragma unroll
            for (int tg = 0; tg < NG; ++tg) {
                const int t = 16 * tg + col;
                const half8_t a =
                    *reinterpret_cast<const half8_t *>(buf + 256 * t + 8 * (c ^ (t & 31)));
#pragma unroll
                for (int m = 0; m < NMAT; ++m)
                    acc[m][tg] =
                        __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bop[m], acc[m][tg], 0, 0, 0);
            }
        }
    };

    // Q4_K: the 32 weights of matrix-core step (p, hh) in quarter q are
    // positions 8p .. 8p+7 of sub-blocks 2q + hh (the lane's quant group q,
    // low nibbles for hh = 0, high for hh = 1), paired with activation chunk
    // 4(2q + hh) + p of the slice, so that a lane needs the scales of two
    // sub-blocks only
    auto compute = [&](const _Float16 *buf, const WSb (&w)[NMAT]) {
        float sl[NMAT], ol[NMAT], sh[NMAT], oh[NMAT];
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
            const uint4 h = w[m].h;
            const float d = half_to_float(h.x), dmin = half_to_float(h.x >> 16);
            const float d24 = d * 16777216.f, d20 = d * 1048576.f;
            // scale and min bytes of sub-blocks 0-3 (q < 2) or 4-7; sub-blocks
            // 2q and 2q + 1 are bytes 2(q & 1) and 2(q & 1) + 1 of them
            const uint32_t scw = quarter < 2 ? (h.y & 0x3F3F3F3Fu)
                                             : ((h.w & 0x0F0F0F0Fu) | ((h.y >> 2) & 0x30303030u));
            const uint32_t mnw = quarter < 2
                                     ? (h.z & 0x3F3F3F3Fu)
                                     : (((h.w >> 4) & 0x0F0F0F0Fu) | ((h.z >> 2) & 0x30303030u));
            const uint32_t b0 = 16u * (uint32_t)(quarter & 1);
            sl[m] = (float)__builtin_amdgcn_ubfe(scw, b0, 8) * d24;
            sh[m] = (float)__builtin_amdgcn_ubfe(scw, b0 + 8, 8) * d20;
            ol[m] = -dmin * (float)__builtin_amdgcn_ubfe(mnw, b0, 8);
            oh[m] = -dmin * (float)__builtin_amdgcn_ubfe(mnw, b0 + 8, 8);
        }
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
            half8_t bop[NMAT][2]; // [matrix][hh], positions 8pp .. 8pp+7 in order
#pragma unroll
            for (int m = 0; m < NMAT; ++m) {
                const uint4 &qv = pp < 2 ? w[m].qa : w[m].qb;
                const uint32_t D0 = (pp & 1) ? qv.z : qv.x, D1 = (pp & 1) ? qv.w : qv.y;
                const uint32_t t0 = D0 >> 8, t1 = D1 >> 8;
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const uint32_t mk = hh ? 0x00F000F0u : 0x000F000Fu;
                    const uint32_t a0 = D0 & mk, a1 = t0 & mk; // bytes (0,2), (1,3)
                    const uint32_t a2 = D1 & mk, a3 = t1 & mk; // bytes (4,6), (5,7)
                    const float s = hh ? sh[m] : sl[m], o = hh ? oh[m] : ol[m];
                    const uint4 v = make_uint4(deq2(a0, 0, a1, 0, s, o), deq2(a0, 1, a1, 1, s, o),
                                               deq2(a2, 0, a3, 0, s, o), deq2(a2, 1, a3, 1, s, o));
                    bop[m][hh] = __builtin_bit_cast(half8_t, v);
                }
            }
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int c = 4 * (2 * quarter + hh) + pp; // 16-byte chunk of the 512-byte slice
#pragma unroll
                for (int tg = 0; tg < NG; ++tg) {
                    const int t = 16 * tg + col;
                    const half8_t a =
                        *reinterpret_cast<const half8_t *>(buf + 256 * t + 8 * (c ^ (t & 31)));
#pragma unroll
                    for (int m = 0; m < NMAT; ++m)
                        acc[m][tg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bop[m][hh],
                                                                            acc[m][tg], 0, 0, 0);
                }
            }
        }
    };

    // the previous chunk's readers are done with both buffers
    __syncthreads();
    auto load_w = [&](int sb, WS(&w)[NMAT]) {
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
            if constexpr (Q8)
                load_wsb8(wrow[m], sb, quarter, w[m]);
            else
                load_wsb(wrow[m], sb, quarter, w[m]);
        }
    };
    auto compute_w = [&](const _Float16 *buf, const WS(&w)[NMAT]) {
        if constexpr (Q8)
            compute8(buf, w);
        else
            compute(buf, w);
    };
    WS wa[NMAT], wb[NMAT];
    issue_x(0, xs0);
    load_w(0, wa);
    // two super-blocks per iteration so that buffers and register sets stay fixed
    for (int sb = 0; sb < nsb; sb += 2) {
        // retire this wave's copies and weight loads of super-block sb, then
        // publish the copies of every wave
        __builtin_amdgcn_s_waitcnt(0); // vmcnt(0) expcnt(0) lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        if (sb + 1 < nsb) {
            issue_x(sb + 1, xs1);
            load_w(sb + 1, wb);
        }
        compute_w(xs0, wa);
        if (sb + 1 >= nsb)
            break;
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_s_barrier();
        if (sb + 2 < nsb) {
            issue_x(sb + 2, xs0);
            load_w(sb + 2, wa);
        }
        compute_w(xs1, wb);
    }

    // element i of group tg: token 16*tg + 4*quarter + i, weight row `row`
#pragma unroll
    for (int tg = 0; tg < NG; ++tg)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 16 * tg + 4 * quarter + i;
            if (t >= nc)
                continue;
            const int64_t pos = p0 + t;
            if constexpr (MODE == 0) {
                // the slot weight on the expert's input scales g and u alike
                const float pw = p.weight_input ? p.wts[p.sorted[pos]] : 1.f;
                const float v = silu(pw * acc[0][tg][i]) * (pw * acc[1][tg][i]);
                reinterpret_cast<uint16_t *>(p.y)[pos * M + row] = (uint16_t)pack_half2(v, 0.f);
            } else {
                reinterpret_cast<float *>(p.y)[pos * M + row] = acc[0][tg][i];
            }
        }
}

template <int MODE, bool Q8>
__global__ __launch_bounds__(NT, 2) void moe_skinny_kernel(SkinnyParams p)
{
    __shared__ __attribute__((aligned(16))) _Float16 xs0[ST * 256];
    __shared__ __attribute__((aligned(16))) _Float16 xs1[ST * 256];
    const int e = blockIdx.y;
    const int begin = p.offsets[e], end = p.offsets[e + 1];
    for (int c0 = begin; c0 < end; c0 += ST) {
        const int nc = end - c0 < ST ? end - c0 : ST;
        switch ((nc + 15) >> 4) {
        case 1: run_chunk<MODE, 1, Q8>(p, e, c0, nc, xs0, xs1); break;
        case 2: run_chunk<MODE, 2, Q8>(p, e, c0, nc, xs0, xs1); break;
        case 3: run_chunk<MODE, 3, Q8>(p, e, c0, nc, xs0, xs1); break;
        default: run_chunk<MODE, 4, Q8>(p, e, c0, nc, xs0, xs1); break;
        }
    }
}

} // namespace

bool moe_skinny_applies(int64_t assignments, int64_t experts)
{
    return assignments <= 48 * experts;
}

hipError_t launch_moe_skinny(const MoeArgs &a, hipStream_t s)
{
    SkinnyParams p{};
    p.offsets = reinterpret_cast<const int32_t *>(a.ws + a.off[0]);
    p.sorted = reinterpret_cast<const int32_t *>(a.ws + a.off[1]);
    p.topk = (int)a.topk;
    p.wts = a.wts;
    p.weight_input = a.weight_input;

    // gate/up with the SwiGLU epilogue: h[pos][0..I) in binary16
    p.w = a.w_gate;
    p.w2 = a.w_up;
    p.x = a.x;
    p.y = a.ws + a.off[4];
    p.M = (int)a.I;
    p.K = (int)a.H;
    p.expert_bytes = a.q8_0 ? a.I * (a.H / kQ80Weights) * kQ80Bytes
                            : a.I * (a.H / kQ4kWeights) * kQ4kBytes;
    if (a.q8_0)
        hipLaunchKernelGGL((moe_skinny_kernel<0, true>), dim3((unsigned)(a.I / SR), (unsigned)a.E),
                           dim3(NT), 0, s, p);
    else
        hipLaunchKernelGGL((moe_skinny_kernel<0, false>), dim3((unsigned)(a.I / SR), (unsigned)a.E),
                           dim3(NT), 0, s, p);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;

    // down: d[pos][0..H) in binary32
    p.w = a.w_down;
    p.w2 = nullptr;
    p.x = reinterpret_cast<const uint16_t *>(a.ws + a.off[4]);
    p.y = a.ws + a.off[5];
    p.M = (int)a.H;
    p.K = (int)a.I;
    p.expert_bytes = a.q8_0 ? a.H * (a.I / kQ80Weights) * kQ80Bytes
                            : a.H * (a.I / kQ4kWeights) * kQ4kBytes;
    if (a.q8_0)
        hipLaunchKernelGGL((moe_skinny_kernel<1, true>), dim3((unsigned)(a.H / SR), (unsigned)a.E),
                           dim3(NT), 0, s, p);
    else
        hipLaunchKernelGGL((moe_skinny_kernel<1, false>), dim3((unsigned)(a.H / SR), (unsigned)a.E),
                           dim3(NT), 0, s, p);
    return hipGetLastError();
}

} // namespace gq
