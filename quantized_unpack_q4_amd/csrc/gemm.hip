// gemm.hip -- fused dequant matrix products on the gfx950 matrix cores.
//
// Y = X * W^T with W in Q4_K blocks and X, Y in binary16, accumulated in
// binary32: the prefill product and the two grouped products of the
// mixture-of-experts layer.  The page "Building a Rust Inference Engine That
// Matches Llama.cpp" (section "Where the wins came from") fuses the
// dequantization into the matmul so the weights are never expanded into a
// full-precision buffer in memory; here each workgroup expands only the
// 64-weight slice of its W tile that the current step needs, into LDS, and
// the matrix cores read it from there.  The binary16 weight is the binary32
// weight (one fused multiply-add, one rounding) rounded to nearest even.
//
// Structure: a 256-thread workgroup owns a BM x BN output tile (BM weight
// rows, BN activation rows) and walks K in steps of 64 weights (a quarter of
// a super-block: sub-blocks 2g and 2g+1 of super-block s).  Steps are double
// buffered in LDS: the global loads of step k+1 are issued before the matrix
// instructions of step k and are dequantized into the other buffer after
// them, one barrier per step.  Four waves split the tile WM x WN; each wave
// issues v_mfma_f32_16x16x32_f16 on 16 x 16 fragments.
#include "gq_device.h"
#include "gq_internal.h"

namespace gq {

enum { kModeGemm = 0, kModeGateUp = 1, kModeDown = 2 };
// weight formats: Q4_K super-blocks, or Q8_0 blocks (plain product only; a
// 64-weight step is two 34-byte blocks, 68 bytes that start 4-byte aligned in
// every row when K % 64 == 0)
enum { kFmtQ4K = 0, kFmtQ8 = 1 };

struct GemmParams {
    const uint8_t *w;      // Q4_K weights (gate for the gate/up product); experts stacked
    const uint8_t *w2;     // up weights (gate/up product only)
    const uint16_t *x;     // binary16 activations, rows of K
    void *y;               // output (see the epilogues)
    int M, K, N;           // weight rows, reduction length, activation rows (plain product)
    const int32_t *sorted; // grouped products: assignment at each sorted position
    const int32_t *tiles;  // grouped products: [2][max_tiles] (expert, first position)
    const int32_t *offsets;// grouped products: expert start positions, [E] = total, [E+1] = tiles
    int max_tiles;
    int topk;
    int E;
    int64_t expert_bytes;  // bytes of one expert's weight matrix
    const float *wts;      // gate/up with weight_input: the slot weights, [T*topk]
    int weight_input;
};


template <int BM, int BN, int WM, int WN, int MODE, int FMT = kFmtQ4K>
__global__ __launch_bounds__(256) void gemm_q4k_kernel(GemmParams p)
{
    constexpr int KS = 64;        // weights per K step
    constexpr int LDR = KS + 8;   // LDS row stride in halves (144 bytes, keeps 16-byte alignment)
    constexpr int NW = MODE == kModeGateUp ? 2 : 1;
    constexpr int TPR = 256 / BM; // threads per weight row in the dequant step
    constexpr int QB = 32 / TPR;  // quant bytes per thread per step
    constexpr int XU = BN / 32;   // 16-byte activation chunks per thread per step
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 16, FN = TN / 16;
    static_assert(BM * TPR == 256 && QB % 8 == 0, "tile rows");
    static_assert(XU >= 1 && FM >= 1 && FN >= 1 && WM * WN == 4, "tile shape");

    __shared__ __attribute__((aligned(16))) _Float16 sW[2][NW][BM][LDR];
    __shared__ __attribute__((aligned(16))) _Float16 sX[2][BN][LDR];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int K = p.K;
    const int nsb = K >> 8;
    const int64_t row_bytes = FMT == kFmtQ8 ? (int64_t)(K / 32) * 34 : (int64_t)nsb * kQ4kBytes;
    // Q8_0: this thread's 64/TPR weights of a step start at weight w8 of the
    // step, inside block w8/32; their quant bytes start at byte q8 of the
    // step's 68 bytes (dword q8/4, byte shift q8%4, 0 or 2), the block scale
    // sits in the low or high half of dword d8w
    constexpr int QB8 = 64 / TPR;
    const int w8 = (tid % TPR) * QB8;
    const int q8 = 34 * (w8 >> 5) + 2 + (w8 & 31);
    const int d8w = (34 * (w8 >> 5)) >> 2, d8hi = (34 * (w8 >> 5)) & 3 ? 16 : 0;

    // ---- tile coordinates ----
    const int m0 = blockIdx.x * BM;
    int n0 = 0, nvalid = 0;
    const uint8_t *wA = p.w;
    const uint8_t *wB = p.w2;
    if (MODE == kModeGemm) {
        n0 = blockIdx.y * BN;
        nvalid = min(BN, p.N - n0);
    } else {
        const int t = blockIdx.y;
        if (t >= p.offsets[p.E + 1]) // tiles beyond this routing's count
            return;
        const int e = p.tiles[t];
        n0 = p.tiles[p.max_tiles + t];
        nvalid = min(BN, p.offsets[e + 1] - n0);
        wA += (int64_t)e * p.expert_bytes;
        if (MODE == kModeGateUp)
            wB += (int64_t)e * p.expert_bytes;
    }

    // ---- per-thread roles ----
    const int drow = tid / TPR;               // weight row this thread dequantizes
    const int dpart = tid % TPR;              // which QB-byte slice of the 32-byte group
    const bool drow_ok = m0 + drow < p.M;
    const uint8_t *wrowA = wA + (int64_t)(m0 + drow) * row_bytes;
    const uint8_t *wrowB = NW == 2 ? wB + (int64_t)(m0 + drow) * row_bytes : nullptr;

    const uint16_t *xrow[XU];
    int xchunk[XU], xr[XU];
#pragma unroll
    for (int u = 0; u < XU; ++u) {
        const int idx = tid + 256 * u;
        xr[u] = idx >> 3;
        xchunk[u] = idx & 7;
        xrow[u] = nullptr;
        if (xr[u] < nvalid) {
            int64_t src;
            if (MODE == kModeGemm)
                src = n0 + xr[u];
            else if (MODE == kModeGateUp)
                src = p.sorted[n0 + xr[u]] / p.topk;
            else
                src = n0 + xr[u];
            xrow[u] = p.x + src * (int64_t)K;
        }
    }

    // ---- staging registers ----
    uint4 rh[NW];
    uint32_t rq[NW][QB / 4];
    uint4 rx[XU];
    uint32_t r8[NW][QB8 / 4 + 1], r8d[NW]; // Q8_0: quant dwords (one extra for the shift), scale dword

    auto load_step = [&](int kt) {
        if constexpr (FMT == kFmtQ8) {
#pragma unroll
            for (int v = 0; v < NW; ++v) {
                if (drow_ok) {
                    const uint32_t *st =
                        reinterpret_cast<const uint32_t *>((v == 0 ? wrowA : wrowB) + (int64_t)kt * 68);
#pragma unroll
                    for (int i = 0; i <= QB8 / 4; ++i)
                        r8[v][i] = st[min((q8 >> 2) + i, 16)]; // dword 16: the step's last
                    r8d[v] = st[d8w];
                } else {
#pragma unroll
                    for (int i = 0; i <= QB8 / 4; ++i)
                        r8[v][i] = 0u;
                    r8d[v] = 0u;
                }
            }
#pragma unroll
            for (int u = 0; u < XU; ++u)
                rx[u] = xrow[u] ? ld16(xrow[u] + kt * KS + 8 * xchunk[u]) : make_uint4(0, 0, 0, 0);
            return;
        }
        const int s = kt >> 2, g = kt & 3;
#pragma unroll
        for (int v = 0; v < NW; ++v) {
            const uint8_t *blk = (v == 0 ? wrowA : wrowB) + (int64_t)s * kQ4kBytes;
            if (drow_ok) {
                rh[v] = ld16(blk);
                const uint8_t *q = blk + 16 + 32 * g + dpart * QB;
#pragma unroll
                for (int i = 0; i < QB / 16; ++i) {
                    const uint4 a = ld16(q + 16 * i);
                    rq[v][4 * i] = a.x;
                    rq[v][4 * i + 1] = a.y;
                    rq[v][4 * i + 2] = a.z;
                    rq[v][4 * i + 3] = a.w;
                }
                if constexpr (QB == 8) {
                    const uint2 a = *reinterpret_cast<const uint2 *>(q);
                    rq[v][0] = a.x;
                    rq[v][1] = a.y;
                }
            } else {
                rh[v] = make_uint4(0, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < QB / 4; ++i)
                    rq[v][i] = 0;
            }
        }
#pragma unroll
        for (int u = 0; u < XU; ++u)
            rx[u] = xrow[u] ? ld16(xrow[u] + kt * KS + 8 * xchunk[u]) : make_uint4(0, 0, 0, 0);
    };

    auto store_step = [&](int kt, int buf) {
        if constexpr (FMT == kFmtQ8) {
            // w = binary16(d * q): exact in binary32, one rounding to binary16.
            // The signed byte q is taken as (q ^ 0x80) - 128 from an unsigned
            // byte conversion (exact), not as a sign-extended integer: the
            // compiler folds the latter into an unsigned conversion of the
            // sign-extended byte here, which turns negative quants into ~2^32.
#pragma unroll
            for (int v = 0; v < NW; ++v) {
                const float d = half_to_float((r8d[v] >> d8hi) & 0xffffu);
                uint32_t hw[QB8 / 2];
#pragma unroll
                for (int i = 0; i < QB8 / 4; ++i) {
                    const uint32_t D =
                        __builtin_amdgcn_alignbyte(r8[v][i + 1], r8[v][i], q8 & 3) ^ 0x80808080u;
                    hw[2 * i] = pack_half2(d * (ubyte_to_float<0>(D) - 128.f),
                                           d * (ubyte_to_float<1>(D) - 128.f));
                    hw[2 * i + 1] = pack_half2(d * (ubyte_to_float<2>(D) - 128.f),
                                               d * (ubyte_to_float<3>(D) - 128.f));
                }
                _Float16 *dst = &sW[buf][v][drow][w8];
#pragma unroll
                for (int i = 0; i < QB8 / 8; ++i)
                    *reinterpret_cast<uint4 *>(dst + 8 * i) =
                        make_uint4(hw[4 * i], hw[4 * i + 1], hw[4 * i + 2], hw[4 * i + 3]);
            }
#pragma unroll
            for (int u = 0; u < XU; ++u)
                *reinterpret_cast<uint4 *>(&sX[buf][xr[u]][8 * xchunk[u]]) = rx[u];
            return;
        }
        const int g = kt & 3;
#pragma unroll
        for (int v = 0; v < NW; ++v) {
            uint32_t scl, ml, sch, mh;
            q4k_scale_min(rh[v].y, rh[v].z, rh[v].w, 2 * g, scl, ml);
            q4k_scale_min(rh[v].y, rh[v].z, rh[v].w, 2 * g + 1, sch, mh);
            const float d = half_to_float(rh[v].x), dmin = half_to_float(rh[v].x >> 16);
            const float dsl = d * (float)scl, dml = dmin * (float)ml;
            const float dsh = d * (float)sch, dmh = dmin * (float)mh;
            uint32_t lo[QB / 2], hi[QB / 2];
#pragma unroll
            for (int i = 0; i < QB / 4; ++i) {
                const uint32_t D = rq[v][i];
                const uint32_t a = D & 0x0f0f0f0fu, b = (D >> 4) & 0x0f0f0f0fu;
                lo[2 * i] = pack_half2(fmaf(dsl, ubyte_to_float<0>(a), -dml),
                                       fmaf(dsl, ubyte_to_float<1>(a), -dml));
                lo[2 * i + 1] = pack_half2(fmaf(dsl, ubyte_to_float<2>(a), -dml),
                                           fmaf(dsl, ubyte_to_float<3>(a), -dml));
                hi[2 * i] = pack_half2(fmaf(dsh, ubyte_to_float<0>(b), -dmh),
                                       fmaf(dsh, ubyte_to_float<1>(b), -dmh));
                hi[2 * i + 1] = pack_half2(fmaf(dsh, ubyte_to_float<2>(b), -dmh),
                                           fmaf(dsh, ubyte_to_float<3>(b), -dmh));
            }
            _Float16 *dst = &sW[buf][v][drow][0];
#pragma unroll
            for (int i = 0; i < QB / 8; ++i) {
                *reinterpret_cast<uint4 *>(dst + dpart * QB + 8 * i) =
                    make_uint4(lo[4 * i], lo[4 * i + 1], lo[4 * i + 2], lo[4 * i + 3]);
                *reinterpret_cast<uint4 *>(dst + 32 + dpart * QB + 8 * i) =
                    make_uint4(hi[4 * i], hi[4 * i + 1], hi[4 * i + 2], hi[4 * i + 3]);
            }
        }
#pragma unroll
        for (int u = 0; u < XU; ++u)
            *reinterpret_cast<uint4 *>(&sX[buf][xr[u]][8 * xchunk[u]]) = rx[u];
    };

    float4_t acc[NW][FM][FN];
#pragma unroll
    for (int v = 0; v < NW; ++v)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[v][i][j] = float4_t{0.f, 0.f, 0.f, 0.f};

    const int wm = wave / WN, wn = wave % WN;
    const int frow = lane & 15, fk = 8 * (lane >> 4);

    const int nk = K / KS;
    load_step(0);
    store_step(0, 0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk)
            load_step(kt + 1);
#pragma unroll
        for (int ks = 0; ks < KS / 32; ++ks) {
            half8_t bf[FN];
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bf[j] = *reinterpret_cast<const half8_t *>(&sX[buf][wn * TN + 16 * j + frow][32 * ks + fk]);
#pragma unroll
            for (int v = 0; v < NW; ++v)
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    const half8_t af = *reinterpret_cast<const half8_t *>(
                        &sW[buf][v][wm * TM + 16 * i + frow][32 * ks + fk]);
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[v][i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[j], acc[v][i][j], 0, 0, 0);
                }
        }
        if (kt + 1 < nk)
            store_step(kt + 1, buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: fragment element (reg c) is weight row 4*(lane>>4)+c, activation row lane&15 ----
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int m = m0 + wm * TM + 16 * i + 4 * (lane >> 4);
            const int nl = wn * TN + 16 * j + (lane & 15);
            if (nl >= nvalid)
                continue;
            const int64_t n = n0 + nl;
            if (MODE == kModeGemm) {
                uint16_t *yr = reinterpret_cast<uint16_t *>(p.y) + n * p.M;
                const float4_t a = acc[0][i][j];
                if (m + 3 < p.M && (p.M & 3) == 0) {
                    *reinterpret_cast<uint2 *>(yr + m) = make_uint2(pack_half2(a[0], a[1]), pack_half2(a[2], a[3]));
                } else {
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        if (m + c < p.M)
                            yr[m + c] = (uint16_t)pack_half2(a[c], 0.f);
                }
            } else if (MODE == kModeGateUp) {
                uint16_t *hr = reinterpret_cast<uint16_t *>(p.y) + n * p.M;
                // the slot weight on the expert's input scales g and u alike
                const float pw = p.weight_input ? p.wts[p.sorted[n]] : 1.f;
                const float4_t gg = pw * acc[0][i][j];
                const float4_t uu = pw * acc[NW - 1][i][j];
                *reinterpret_cast<uint2 *>(hr + m) =
                    make_uint2(pack_half2(silu(gg[0]) * uu[0], silu(gg[1]) * uu[1]),
                               pack_half2(silu(gg[2]) * uu[2], silu(gg[3]) * uu[3]));
            } else {
                float *dr = reinterpret_cast<float *>(p.y) + n * p.M;
                const float4_t a = acc[0][i][j];
                *reinterpret_cast<float4 *>(dr + m) = make_float4(a[0], a[1], a[2], a[3]);
            }
        }
}

template <int BM, int BN, int WM, int WN, int FMT = kFmtQ4K>
static hipError_t gemm_go(const GemmParams &p, hipStream_t s)
{
    dim3 grid((p.M + BM - 1) / BM, (p.N + BN - 1) / BN);
    hipLaunchKernelGGL((gemm_q4k_kernel<BM, BN, WM, WN, kModeGemm, FMT>), grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_gemm_q8_0(const void *w, const uint16_t *x, uint16_t *y, int64_t M, int64_t K,
                            int64_t N, hipStream_t s)
{
    GemmParams p{};
    p.w = (const uint8_t *)w;
    p.x = x;
    p.y = y;
    p.M = (int)M;
    p.K = (int)K;
    p.N = (int)N;
    if (N <= 64)
        return gemm_go<128, 32, 4, 1, kFmtQ8>(p, s);
    const int64_t t128 = ((M + 127) / 128) * ((N + 127) / 128);
    const int64_t t64x128 = ((M + 63) / 64) * ((N + 127) / 128);
    if (t128 >= 448)
        return gemm_go<128, 128, 2, 2, kFmtQ8>(p, s);
    if (t64x128 >= 384)
        return gemm_go<64, 128, 1, 4, kFmtQ8>(p, s);
    return gemm_go<64, 64, 2, 2, kFmtQ8>(p, s);
}

hipError_t launch_gemm_q4k(const void *w, const uint16_t *x, uint16_t *y, int64_t M, int64_t K,
                           int64_t N, hipStream_t s)
{
    GemmParams p{};
    p.w = (const uint8_t *)w;
    p.x = x;
    p.y = y;
    p.M = (int)M;
    p.K = (int)K;
    p.N = (int)N;
    if (N <= 64)
        return gemm_go<128, 32, 4, 1>(p, s);
    // smaller tiles when the large ones would leave CUs idle: 128 x 128 from
    // 448 tiles (1.75 per CU of a 256-CU part), 64 x 128 from 384, else 64 x 64
    const int64_t t128 = ((M + 127) / 128) * ((N + 127) / 128);
    const int64_t t64x128 = ((M + 63) / 64) * ((N + 127) / 128);
    if (t128 >= 448)
        return gemm_go<128, 128, 2, 2>(p, s);
    if (t64x128 >= 384)
        return gemm_go<64, 128, 1, 4>(p, s);
    return gemm_go<64, 64, 2, 2>(p, s);
}

// ---- grouped products of the mixture-of-experts layer ----

template <int BN, int FMT>
static hipError_t moe_gemms(const MoeArgs &a, int max_tiles, hipStream_t s)
{
    const int32_t *offsets = reinterpret_cast<const int32_t *>(a.ws + a.off[0]);
    GemmParams p{};
    p.sorted = reinterpret_cast<const int32_t *>(a.ws + a.off[1]);
    p.tiles = reinterpret_cast<const int32_t *>(a.ws + a.off[3]);
    p.offsets = offsets;
    p.max_tiles = max_tiles;
    p.topk = (int)a.topk;
    p.E = (int)a.E;
    p.wts = a.wts;
    p.weight_input = a.weight_input;

    // gate/up with the SwiGLU epilogue: h[pos][0..I) in binary16
    p.w = a.w_gate;
    p.w2 = a.w_up;
    p.x = a.x;
    p.y = a.ws + a.off[4];
    p.M = (int)a.I;
    p.K = (int)a.H;
    p.expert_bytes = FMT == kFmtQ8 ? a.I * (a.H / 32) * 34 : a.I * (a.H / kQ4kWeights) * kQ4kBytes;
    constexpr int WM = BN >= 64 ? 2 : 4, WN = 4 / WM;
    hipLaunchKernelGGL((gemm_q4k_kernel<128, BN, WM, WN, kModeGateUp, FMT>),
                       dim3((unsigned)(a.I / 128), (unsigned)max_tiles), dim3(256), 0, s, p);
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
    p.expert_bytes = FMT == kFmtQ8 ? a.H * (a.I / 32) * 34 : a.H * (a.I / kQ4kWeights) * kQ4kBytes;
    hipLaunchKernelGGL((gemm_q4k_kernel<128, BN, WM, WN, kModeDown, FMT>),
                       dim3((unsigned)(a.H / 128), (unsigned)max_tiles), dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_moe_gemms(const MoeArgs &a, int bn, int max_tiles, hipStream_t s)
{
    if (a.q8_0) {
        switch (bn) {
        case 32: return moe_gemms<32, kFmtQ8>(a, max_tiles, s);
        case 64: return moe_gemms<64, kFmtQ8>(a, max_tiles, s);
        default: return moe_gemms<128, kFmtQ8>(a, max_tiles, s);
        }
    }
    switch (bn) {
    case 32: return moe_gemms<32, kFmtQ4K>(a, max_tiles, s);
    case 64: return moe_gemms<64, kFmtQ4K>(a, max_tiles, s);
    default: return moe_gemms<128, kFmtQ4K>(a, max_tiles, s);
    }
}

} // namespace gq
