// gemm_big.hip -- large-tile fused dequant matrix product for prefill.
//
// Y[N][M] = X[N][K] * W[M][K]^T, W in Q4_K blocks, X and Y binary16, binary32
// accumulation on the gfx950 matrix cores.  The dequantization happens when
// the weights are needed, once per workgroup tile, and never lands in global
// memory (page "Building a Rust Inference Engine That Matches Llama.cpp",
// section "Where the wins came from").
//
// Tiling.  One 512-thread workgroup (eight waves, two per SIMD) owns a
// 256 x 256 tile of Y (256 weight rows by 256 activation rows); wave (wm, wn)
// of the 2 x 4 wave grid owns a 128 x 64 sub-tile held in accumulation
// registers as 4 x 2 fragments of v_mfma_f32_32x32x16_f16.  K advances 64
// weights per step (sub-blocks 2g and 2g+1 of one super-block).  Per step:
//   * the activation slice (256 rows x 64 halves) is copied global -> LDS by
//     direct-to-LDS loads one step ahead (no registers involved);
//   * the packed weight slice (header + 32 quant bytes per row, two threads
//     per row) is loaded into registers two steps ahead and dequantized into
//     LDS one step ahead: w16 = binary16(binary32(d*sc*q - dmin*m)) by one
//     mixed-precision FMA per weight (the quant enters as the binary16
//     subnormal q*2^-24, exactly);
//   * the matrix cores consume the current step from LDS; the fragments of
//     the next 16-wide sub-step are read while the current one multiplies,
//     and the last sub-step's matrix instructions are issued after the
//     barrier that ends the step, where they cover the LDS latency of the
//     next step's first fragments.
// With two waves per SIMD and the matrix instructions at raised priority, one
// wave's dequantization and LDS traffic overlap the other's matrix work.  The
// barrier that ends a step waits only for this step's LDS writes and copies,
// never for the weight loads still in flight for the step after next.
//
// LDS rows are 128 bytes (64 halves = eight 16-byte chunks); chunk j of row r
// sits in slot j ^ (r & 7) so that the rows one fragment read touches spread
// over the banks.  Two buffers of each operand: 4 x 32 KB.
//
// Workgroups are numbered so that each XCD (blockIdx mod 8) receives a
// contiguous run of tiles in activation-panel-major order: the workgroups an
// XCD runs at once share one activation panel in that XCD's L2.
#include "gq_device.h"
#include "gq_internal.h"

namespace gq {

namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x3 __attribute__((ext_vector_type(3)));
typedef __attribute__((address_space(1))) const u32x4 g_u32x4;
typedef __attribute__((address_space(1))) const u32x3 g_u32x3;

__device__ __forceinline__ uint4 gload16(const void *p)
{
    const u32x4 v = *(g_u32x4 *)(p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// 16 bytes per lane, global -> LDS: lane l reads gbase + voff (gbase
// wave-uniform, voff a 32-bit byte offset) and lands at lds_base + 16*l
// (lds_base wave-uniform).  Issued as inline assembly so that the compiler's
// wait insertion does not see it: the kernel waits for these copies itself,
// with an explicit vmcnt before the barrier that publishes them.  The compiler
// then counts fewer outstanding loads than there are, so every wait it
// inserts for its own loads errs on the safe side.
__device__ __forceinline__ void load_lds16(const void *gbase, uint32_t voff, const void *lds_base)
{
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(
        (uint32_t)(size_t)(const __attribute__((address_space(3))) void *)lds_base);
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(gbase),
                 "s"(m0)
                 : "memory", "m0");
}

// Two weights from two binary16 quants (subnormal q*2^-24 or 16q*2^-24) and
// the binary32 scale/offset: binary16(binary32(s*q + o)) each, packed.
__device__ __forceinline__ uint32_t deq2(uint32_t qa, int sela, uint32_t qb, int selb, float s,
                                         float o)
{
    const h2_t a = __builtin_bit_cast(h2_t, qa), b = __builtin_bit_cast(h2_t, qb);
    const _Float16 lo = (_Float16)fmaf((float)(sela ? a.y : a.x), s, o);
    const _Float16 hi = (_Float16)fmaf((float)(selb ? b.y : b.x), s, o);
    return __builtin_bit_cast(uint32_t, h2_t{lo, hi});
}

template <int V>
struct IC {
    static constexpr int value = V;
};

constexpr int KS = 64;  // weights per K step
constexpr int BM = 256; // weight rows per tile
constexpr int BN = 256; // activation rows per tile
constexpr int NT = 512; // threads per workgroup
constexpr int WAVES_N = 4;
constexpr int TM = 128, TN = 64;          // per wave
constexpr int FM = TM / 32, FN = TN / 32; // 32 x 32 fragments per wave

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt in
// 6:4, lgkmcnt in 11:8): vmcnt <= vm with lgkmcnt == 0 or left free.
constexpr int waitcnt_vm_lgkm0(int vm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4); }
constexpr int waitcnt_vm(int vm) { return waitcnt_vm_lgkm0(vm) | (15 << 8); }

enum { kBigDense = 0, kBigGateUp = 1, kBigDown = 2 };

struct BigParams {
    const uint8_t *w, *w2; // Q4_K weights (gate/up: gate, up; experts stacked)
    const uint16_t *x;     // binary16 activations, rows of K
    void *y;               // dense: Y [N][M] binary16; gate/up: h [A][M] binary16; down: d [A][M] binary32
    int M, K, N;           // weight rows (per expert), reduction length, activation rows (dense)
    int tiles_m, tiles_total;
    // grouped experts: token tiles of 256 sorted positions, one expert each
    const int32_t *sorted, *tiles, *offsets;
    int max_tiles, topk, E;
    int64_t expert_bytes;
};

} // namespace

// MODE kBigDense: Y = X W^T over 256 x 256 tiles.  MODE kBigGateUp: a tile is
// 128 rows of an expert's gate matrix and the same 128 rows of its up matrix
// (waves 0-3 and 4-7) against up to 256 of the expert's tokens, gathered
// through the sorted assignment list; the gate accumulators are passed to the
// up waves through LDS and h = binary16(silu(g) * u) is written.  MODE
// kBigDown: 256 rows of an expert's down matrix against its rows of h,
// binary32 outputs.
template <int MODE>
__global__ __launch_bounds__(NT, 1) void gemm_q4k_big_kernel(BigParams p)
{
    const int M = p.M, K = p.K;
    // four distinct LDS objects (not one array of buffers) so that the
    // compiler can tell the copies into one buffer from the reads of the other
    __shared__ __attribute__((aligned(16))) _Float16 sX0[BN * KS];
    __shared__ __attribute__((aligned(16))) _Float16 sX1[BN * KS];
    __shared__ __attribute__((aligned(16))) _Float16 sW0[BM * KS];
    __shared__ __attribute__((aligned(16))) _Float16 sW1[BM * KS];
    auto Xbuf = [&](int b) -> _Float16 * { return b ? sX1 : sX0; };
    auto Wbuf = [&](int b) -> _Float16 * { return b ? sW1 : sW0; };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6); // wave-uniform
    int m0, n0, nvalid, e = 0;
    if constexpr (MODE == kBigDense) {
        // XCD-aware tile order: the hardware deals consecutive workgroups to
        // the 8 XCDs in turn; give XCD x the contiguous tile run
        // [x*T/8, (x+1)*T/8).
        const int b = blockIdx.x;
        const int per = (p.tiles_total + 7) / 8;
        const int tile = (b % 8) * per + b / 8;
        if (tile >= p.tiles_total)
            return;
        const int n_t = tile / p.tiles_m, m_t = tile % p.tiles_m;
        m0 = m_t * BM;
        n0 = n_t * BN;
        nvalid = p.N - n0 < BN ? p.N - n0 : BN;
    } else {
        const int t = blockIdx.y;
        if (t >= p.offsets[p.E + 1])
            return;
        e = p.tiles[t];
        n0 = p.tiles[p.max_tiles + t]; // first sorted position of the tile
        const int end = p.offsets[e + 1];
        nvalid = end - n0 < BN ? end - n0 : BN;
        m0 = (int)blockIdx.x * (MODE == kBigGateUp ? BM / 2 : BM);
    }

    const int nsb = K >> 8;
    const size_t rowb = (size_t)nsb * kQ4kBytes;
    const int nk = K / KS;

    // dequantization: thread t handles weight row t/2 and quant bytes
    // 16p..16p+15 (p = t & 1) of the step's 32-byte group: their low nibbles
    // are chunks 2p, 2p+1 of the row's LDS slice, their high nibbles chunks
    // 4+2p, 5+2p
    const int drow = tid >> 1, dp = tid & 1;
    // this thread's weight row: dense and down rows m0 + drow; gate/up rows
    // m0 + drow of gate (waves 0-3) and m0 + drow - 128 of up (waves 4-7)
    const uint8_t *w = p.w;
    int wr_want = m0 + drow;
    if constexpr (MODE != kBigDense)
        w = ((MODE == kBigGateUp && wave >= 4) ? p.w2 : p.w) + (size_t)e * p.expert_bytes;
    if constexpr (MODE == kBigGateUp)
        wr_want = m0 + (drow & (BM / 2 - 1));
    const bool wrow_ok = wr_want < M;
    const int wr = wrow_ok ? wr_want : M - 1;
    // byte offset of this thread's row (+16 for the second half); the weight
    // matrix (one expert's) is below 2^31 bytes on this path
    const uint32_t woff = (uint32_t)wr * (uint32_t)rowb + 16u * dp;

    // activation copies: copy i of wave v fills LDS slots [(4v + i) * 64, +64),
    // i.e. row (4v + i) * 8 + lane / 8, slot lane % 8, holding chunk
    // (lane % 8) ^ (row & 7) = (lane % 8) ^ ((lane / 8) & 7)
    // (byte offsets below 2^31: the activation matrix is smaller on this path)
    uint32_t xoff[4];
    {
        const int xr0 = 32 * wave + (lane >> 3);
        const int xchunk = (lane & 7) ^ ((lane >> 3) & 7);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int nl = min(xr0 + 8 * i, nvalid - 1); // rows past the tile repeat its last
            int row = n0 + nl;
            if constexpr (MODE == kBigGateUp)
                row = p.sorted[row] / p.topk; // the token of that sorted position
            xoff[i] = ((uint32_t)row * (uint32_t)K + 8u * xchunk) * 2u;
        }
    }
    const uint16_t *x = p.x;
    auto issue_x = [&](int kt, auto buf_c) {
        constexpr int buf = decltype(buf_c)::value;
        const uint16_t *xk = x + (size_t)kt * KS; // wave-uniform
#pragma unroll
        for (int i = 0; i < 4; ++i)
            load_lds16(xk, xoff[i], Xbuf(buf) + (4 * wave + i) * 512);
    };

    uint4 rh[2], rq[2]; // packed weights of the two steps ahead (slot = step & 1)
    // the quant group g = kt % 4 is known at compile time; groups 0 and 1 need
    // only the first 12 header bytes (a register that is loaded but never
    // read would be reused while its load is still in flight)
    auto issue_w = [&](int kt, auto slot_c, auto g_c) {
        constexpr int slot = decltype(slot_c)::value;
        constexpr int g = decltype(g_c)::value;
        const uint8_t *blk = w + (size_t)(kt >> 2) * kQ4kBytes; // wave-uniform
        if constexpr (g < 2) {
            const u32x3 v = *(g_u32x3 *)(blk + (woff - 16u * dp));
            rh[slot] = make_uint4(v.x, v.y, v.z, 0u);
        } else {
            rh[slot] = gload16(blk + (woff - 16u * dp));
        }
        rq[slot] = gload16(blk + 16 + 32 * g + woff);
    };
    auto dequant_w = [&](auto slot_c, auto g_c, auto buf_c) {
        constexpr int slot = decltype(slot_c)::value;
        constexpr int g = decltype(g_c)::value;
        constexpr int buf = decltype(buf_c)::value;
        const uint4 h = rh[slot];
        uint32_t scl, ml, sch, mh;
        if constexpr (g < 2) {
            scl = (h.y >> (16 * g)) & 63u;
            ml = (h.z >> (16 * g)) & 63u;
            sch = (h.y >> (16 * g + 8)) & 63u;
            mh = (h.z >> (16 * g + 8)) & 63u;
        } else {
            constexpr int s0 = 16 * (g - 2), s1 = s0 + 8;
            scl = ((h.w >> s0) & 15u) | (((h.y >> (s0 + 6)) & 3u) << 4);
            ml = ((h.w >> (s0 + 4)) & 15u) | (((h.z >> (s0 + 6)) & 3u) << 4);
            sch = ((h.w >> s1) & 15u) | (((h.y >> (s1 + 6)) & 3u) << 4);
            mh = ((h.w >> (s1 + 4)) & 15u) | (((h.z >> (s1 + 6)) & 3u) << 4);
        }
        const float d = wrow_ok ? half_to_float(h.x) : 0.f;
        const float dmin = wrow_ok ? half_to_float(h.x >> 16) : 0.f;
        // quants enter as q*2^-24 (low nibbles) and 16q*2^-24 (high nibbles)
        const float sl = d * (float)scl * 16777216.f, ol = -dmin * (float)ml;
        const float sh = d * (float)sch * 1048576.f, oh = -dmin * (float)mh;
        const uint32_t q[4] = {rq[slot].x, rq[slot].y, rq[slot].z, rq[slot].w};
        _Float16 *dst = Wbuf(buf) + drow * KS;
        const int sw = drow & 7;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            // bytes 16p+8c..16p+8c+7: low nibbles are k = 16p+8c.. (chunk
            // 2p+c), high nibbles k = 32+16p+8c.. (chunk 4+2p+c)
            const uint32_t D0 = q[2 * c], D1 = q[2 * c + 1];
            const uint32_t t0 = D0 >> 8, t1 = D1 >> 8;
            const uint32_t l0 = D0 & 0x000F000Fu, l1 = t0 & 0x000F000Fu; // (q0,q2), (q1,q3)
            const uint32_t l2 = D1 & 0x000F000Fu, l3 = t1 & 0x000F000Fu; // (q4,q6), (q5,q7)
            const uint32_t h0 = D0 & 0x00F000F0u, h1 = t0 & 0x00F000F0u;
            const uint32_t h2 = D1 & 0x00F000F0u, h3 = t1 & 0x00F000F0u;
            const uint4 lo = make_uint4(deq2(l0, 0, l1, 0, sl, ol), deq2(l0, 1, l1, 1, sl, ol),
                                        deq2(l2, 0, l3, 0, sl, ol), deq2(l2, 1, l3, 1, sl, ol));
            const uint4 hi = make_uint4(deq2(h0, 0, h1, 0, sh, oh), deq2(h0, 1, h1, 1, sh, oh),
                                        deq2(h2, 0, h3, 0, sh, oh), deq2(h2, 1, h3, 1, sh, oh));
            *reinterpret_cast<uint4 *>(dst + 8 * ((2 * dp + c) ^ sw)) = lo;
            *reinterpret_cast<uint4 *>(dst + 8 * ((4 + 2 * dp + c) ^ sw)) = hi;
        }
    };

    float16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = float16_t{};

    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int frow = lane & 31, fchunk = lane >> 5;

    // v_mfma_f32_32x32x16_f16: operand lane l holds row l % 32, k 8*(l/32)..+7
    auto load_frags = [&](auto buf_c, int ks, half8_t(&af)[FM], half8_t(&bf)[FN]) {
        constexpr int buf = decltype(buf_c)::value;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int r = wn * TN + 32 * j + frow;
            const int c = (2 * ks + fchunk) ^ (r & 7);
            bf[j] = *reinterpret_cast<const half8_t *>(Xbuf(buf) + r * KS + 8 * c);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int r = wm * TM + 32 * i + frow;
            const int c = (2 * ks + fchunk) ^ (r & 7);
            af[i] = *reinterpret_cast<const half8_t *>(Wbuf(buf) + r * KS + 8 * c);
        }
    };
    // Fragments rotate through two register sets: sub-step ks of a step
    // multiplies from set ks & 1 while set (ks + 1) & 1 is read from LDS.  The
    // last sub-step's fragments are read before the barrier that ends the step
    // and multiplied after it, so that its matrix instructions cover the LDS
    // latency of the next step's first fragments (the set starts as zeros).
    half8_t a0[FM], b0[FN], a1[FM], b1[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
        a1[i] = half8_t{};
#pragma unroll
    for (int j = 0; j < FN; ++j)
        b1[j] = half8_t{};
    auto mfma = [&](const half8_t(&af)[FM], const half8_t(&bf)[FN]) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    };
    auto mfma_step = [&](auto buf_c) {
        load_frags(buf_c, 0, a0, b0);
        mfma(a1, b1); // last sub-step of the previous step
        load_frags(buf_c, 1, a1, b1);
        mfma(a0, b0);
        load_frags(buf_c, 2, a0, b0);
        mfma(a1, b1);
        load_frags(buf_c, 3, a1, b1);
        mfma(a0, b0);
    };

    // One K step kt with S = kt % 4 known at compile time: buffers alternate
    // with kt & 1, the packed weights of step s live in register slot s & 1
    // (loaded two steps ahead, dequantized one step ahead) and the quant group
    // of step s is s % 4.
    auto step = [&](int kt, auto S_c) {
        constexpr int S = decltype(S_c)::value;
        const int n1 = kt + 1 < nk ? kt + 1 : nk - 1;
        const int n2 = kt + 2 < nk ? kt + 2 : nk - 1;
        // the only loads still in flight are the packed weights of step kt+1,
        // issued a whole step ago: retire them before issuing new loads, so
        // that no wait inside the step can fall on the copies issued below
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        __builtin_amdgcn_sched_barrier(0);
        issue_x(n1, IC<(S + 1) & 1>{});
        issue_w(n2, IC<S & 1>{}, IC<(S + 2) & 3>{}); // step kt's slot is free again
        __builtin_amdgcn_sched_barrier(0); // keep the loads ahead of the matrix work
        // matrix instructions at raised priority: while one wave of a SIMD
        // dequantizes, the other keeps the matrix core busy
        __builtin_amdgcn_s_setprio(1);
        mfma_step(IC<S & 1>{});
        __builtin_amdgcn_s_setprio(0);
        dequant_w(IC<(S + 1) & 1>{}, IC<(S + 1) & 3>{}, IC<(S + 1) & 1>{});
        // this wave's LDS writes and copies for the next step are done; the two
        // weight loads for the step after next stay in flight
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2));
        __builtin_amdgcn_s_barrier();
    };

    // prologue: step 0 in LDS, step 1 packed weights in registers
    issue_x(0, IC<0>{});
    issue_w(0, IC<0>{}, IC<0>{});
    issue_w(1, IC<1>{}, IC<1>{}); // nk >= 4
    dequant_w(IC<0>{}, IC<0>{}, IC<0>{});
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2));
    __builtin_amdgcn_s_barrier();

    // nk = K / 64 is a multiple of 4 (K % 256 == 0)
    for (int kt = 0; kt < nk; kt += 4) {
        step(kt, IC<0>{});
        step(kt + 1, IC<1>{});
        step(kt + 2, IC<2>{});
        step(kt + 3, IC<3>{});
    }
    mfma(a1, b1); // last sub-step of the last step

    // epilogue: element v of fragment (i, j) is weight row
    // 8*(v/4) + 4*(lane/32) + v%4 and activation row lane % 32 of the wave's tile
    if constexpr (MODE == kBigGateUp) {
        // gate waves (wm = 0) hand their accumulators to the up waves with the
        // same wn through LDS buffer wn (32 KB: 64 lanes x 128 floats, in the
        // fragment layout both waves share); the K loop's last barrier has
        // released every buffer
        float4_t *xch = reinterpret_cast<float4_t *>(wn == 0 ? sX0 : wn == 1 ? sX1 : wn == 2 ? sW0 : sW1);
        if (wm == 0) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int v4 = 0; v4 < 4; ++v4) {
                        const float16_t a = acc[i][j];
                        xch[((i * FN + j) * 4 + v4) * 64 + lane] =
                            float4_t{a[4 * v4], a[4 * v4 + 1], a[4 * v4 + 2], a[4 * v4 + 3]};
                    }
        }
        __builtin_amdgcn_s_waitcnt(0xC07F); // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        if (wm == 1) {
            uint16_t *h = reinterpret_cast<uint16_t *>(p.y);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int nl = wn * TN + 32 * j + (lane & 31);
                    if (nl >= nvalid)
                        continue;
                    uint16_t *hr = h + (size_t)(n0 + nl) * M;
                    const float16_t u = acc[i][j];
#pragma unroll
                    for (int v4 = 0; v4 < 4; ++v4) {
                        const float4_t g = xch[((i * FN + j) * 4 + v4) * 64 + lane];
                        const int m = m0 + 32 * i + 8 * v4 + 4 * (lane >> 5);
                        *reinterpret_cast<uint2 *>(hr + m) = make_uint2(
                            pack_half2(silu(g[0]) * u[4 * v4], silu(g[1]) * u[4 * v4 + 1]),
                            pack_half2(silu(g[2]) * u[4 * v4 + 2], silu(g[3]) * u[4 * v4 + 3]));
                    }
                }
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int nl = wn * TN + 32 * j + (lane & 31);
            if (nl >= nvalid)
                continue;
            const float16_t a = acc[i][j];
            if constexpr (MODE == kBigDown) {
                float *dr = reinterpret_cast<float *>(p.y) + (size_t)(n0 + nl) * M;
#pragma unroll
                for (int v4 = 0; v4 < 4; ++v4) {
                    const int m = m0 + wm * TM + 32 * i + 8 * v4 + 4 * (lane >> 5);
                    *reinterpret_cast<float4_t *>(dr + m) =
                        float4_t{a[4 * v4], a[4 * v4 + 1], a[4 * v4 + 2], a[4 * v4 + 3]};
                }
                continue;
            }
            uint16_t *yr = reinterpret_cast<uint16_t *>(p.y) + (size_t)(n0 + nl) * M;
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) {
                const int m = m0 + wm * TM + 32 * i + 8 * v4 + 4 * (lane >> 5);
                if (m + 3 < M && (M & 3) == 0) {
                    *reinterpret_cast<uint2 *>(yr + m) =
                        make_uint2(pack_half2(a[4 * v4], a[4 * v4 + 1]),
                                   pack_half2(a[4 * v4 + 2], a[4 * v4 + 3]));
                } else {
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        if (m + c < M)
                            yr[m + c] = (uint16_t)pack_half2(a[4 * v4 + c], 0.f);
                }
            }
        }
}

bool gemm_big_applies(int64_t M, int64_t K, int64_t N)
{
    // enough 256 x 256 tiles to fill the chip once, and 32-bit byte offsets
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    return M >= 256 && N >= 256 && tiles >= 256 && M * (K / 256) * kQ4kBytes < (1ll << 31) &&
           N * K * 2 < (1ll << 31);
}

hipError_t launch_gemm_big(const void *w, const uint16_t *x, uint16_t *y, int64_t M, int64_t K,
                           int64_t N, hipStream_t s)
{
    BigParams p{};
    p.w = (const uint8_t *)w;
    p.x = x;
    p.y = y;
    p.M = (int)M;
    p.K = (int)K;
    p.N = (int)N;
    p.tiles_m = (int)((M + BM - 1) / BM);
    p.tiles_total = p.tiles_m * (int)((N + BN - 1) / BN);
    const int grid = (p.tiles_total + 7) / 8 * 8;
    hipLaunchKernelGGL(gemm_q4k_big_kernel<kBigDense>, dim3((unsigned)grid), dim3(NT), 0, s, p);
    return hipGetLastError();
}

int moe_big_token_tile() { return BN; }

bool moe_big_applies(int64_t assignments, int64_t experts, int64_t H, int64_t I)
{
    // about 160 or more tokens per expert on average, and 32-bit byte offsets
    // for one expert's matrices and for the activations and h
    return assignments >= 160 * experts && I * (H / 256) * kQ4kBytes < (1ll << 31) &&
           assignments * I * 2 < (1ll << 31) && assignments * H * 2 < (1ll << 31);
}

hipError_t launch_moe_big(const MoeArgs &a, int max_tiles, hipStream_t s)
{
    BigParams p{};
    p.offsets = reinterpret_cast<const int32_t *>(a.ws + a.off[0]);
    p.sorted = reinterpret_cast<const int32_t *>(a.ws + a.off[1]);
    p.tiles = reinterpret_cast<const int32_t *>(a.ws + a.off[3]);
    p.max_tiles = max_tiles;
    p.topk = (int)a.topk;
    p.E = (int)a.E;

    // gate/up with the SwiGLU epilogue: h[pos][0..I) in binary16
    p.w = a.w_gate;
    p.w2 = a.w_up;
    p.x = a.x;
    p.y = a.ws + a.off[4];
    p.M = (int)a.I;
    p.K = (int)a.H;
    p.expert_bytes = a.I * (a.H / kQ4kWeights) * kQ4kBytes;
    hipLaunchKernelGGL(gemm_q4k_big_kernel<kBigGateUp>,
                       dim3((unsigned)(a.I / (BM / 2)), (unsigned)max_tiles), dim3(NT), 0, s, p);
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
    p.expert_bytes = a.H * (a.I / kQ4kWeights) * kQ4kBytes;
    hipLaunchKernelGGL(gemm_q4k_big_kernel<kBigDown>, dim3((unsigned)(a.H / BM), (unsigned)max_tiles),
                       dim3(NT), 0, s, p);
    return hipGetLastError();
}

} // namespace gq
