// gemm_big.hip -- large-tile fused dequant matrix product for prefill and for
// expert products with many tokens per expert.
//
// Y[N][M] = X[N][K] * W[M][K]^T, W in Q4_K blocks, X and Y binary16, binary32
// accumulation on the gfx950 matrix cores.  The dequantization happens when
// the weights are needed, once per workgroup tile, and never lands in global
// or shared memory (page "Building a Rust Inference Engine That Matches
// Llama.cpp", section "Where the wins came from").
//
// Tiling.  Each wave owns 32 weight rows against 256 activation rows, held in
// accumulation registers as 8 fragments of v_mfma_f32_32x32x16_f16.  A
// workgroup is NW such waves (NW = 8: 256 x 256 tiles, one workgroup per CU;
// NW = 4: 128 x 256 tiles, two workgroups per CU).  Either way a SIMD runs two
// waves, which the matrix pipe needs to issue at its full rate.  Every weight
// is dequantized by exactly one lane, straight into the A operand registers:
// lane l holds row l % 32 and the 16 quant bytes 16h..16h+15 (h = l / 32) of
// the current 32-byte quant group, i.e. the 32 weights
//   k = 16h + b (low nibble of byte b) and 32 + 16h + b (high nibble),
// which the four 16-wide sub-steps of a 64-weight step take as
//   sub-step s: k = 32(s >> 1) + 16h + 8(s & 1) + 0..7.
// The activations are read from LDS in the same order (8-half chunk
// 4(s >> 1) + 2h + (s & 1)), so the k order inside a step is a permutation
// applied to both operands.
//
// Per 64-weight step:
//   * the activation slice (256 rows x 64 halves) is copied global -> LDS by
//     direct-to-LDS loads one step ahead, shared by all waves;
//   * the packed weights (16-byte header + 16 quant bytes per lane) are
//     loaded into registers three steps ahead and dequantized one step ahead:
//     w16 = binary16(binary32(d*sc*q - dmin*m)), one mixed-precision FMA per
//     weight (the quant enters as the binary16 subnormal q*2^-24, exactly)
//     and one packed round-to-nearest conversion per two weights;
//   * the matrix instructions consume the current step, each followed by one
//     LDS read of the next sub-step's fragments and a few dequantization
//     instructions (an explicit interleave: the compiler would otherwise
//     bunch the reads in front of their first use).
//
// LDS rows are 128 bytes (64 halves = eight 16-byte chunks); chunk c of row r
// sits in slot c ^ ((r >> 1) & 7): a 16-lane read phase touches 16 rows and,
// with this map, 16 distinct 16-byte bank groups.
//
// Gate/up (grouped experts): the 32 rows of a wave's A fragment are 16 rows
// of the gate matrix (fragment rows 0-15) and the same 16 rows of the up
// matrix (rows 16-31).  In the accumulator layout fragment rows r and r + 16
// sit in the same lane (elements v and v + 8), so h = silu(g) * u is formed
// in registers.
//
// Workgroups of the dense product are numbered so that each XCD (blockIdx
// mod 8) receives a contiguous run of tiles in activation-panel-major order:
// the workgroups an XCD runs at once share one activation panel in its L2.
#include <mutex>

#include "gq_device.h"
#include "gq_internal.h"
#include "gq_lds_dma.h"

namespace gq {

namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x3 __attribute__((ext_vector_type(3)));
typedef __attribute__((address_space(1))) const u32x4 g_u32x4;
typedef __attribute__((address_space(1))) const u32x3 g_u32x3;
typedef unsigned int u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef __attribute__((address_space(1))) const u32x4a4 g_u32x4a4;
typedef __attribute__((address_space(1))) const unsigned int g_u32;

__device__ __forceinline__ uint4 gload16(const uint8_t *p)
{
    const u32x4 v = *(g_u32x4 *)(p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Two weights from two binary16 quants (subnormal q*2^-24 or 16q*2^-24, the
// half selected by sel) and the binary32 scale/offset:
// binary16(binary32(s*q + o)) each, packed (first weight in the low half).
// The conversion is written out so that it stays one packed round-to-nearest
// instruction for both weights.
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

// Four binary16 weights binary16(d * q) from four signed quant bytes of a
// Q8_0 block (d its binary16 scale, in both halves of d2).  Each byte, offset
// to u = q + 128, becomes the binary16 1024 + u (exponent bits 0x64 above the
// byte), and subtracting 1152 leaves q exactly; one packed binary16 multiply
// then rounds the exact product d * q once.
__device__ __forceinline__ void deq4_q8(uint32_t q, h2_t d2, uint32_t &lo, uint32_t &hi)
{
    const uint32_t u = q ^ 0x80808080u;
    const h2_t off = {(_Float16)1152.f, (_Float16)1152.f};
    const h2_t a = __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u)) - off;
    const h2_t b = __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)) - off;
    lo = __builtin_bit_cast(uint32_t, a * d2);
    hi = __builtin_bit_cast(uint32_t, b * d2);
}

constexpr int KS = 64;  // weights per K step
constexpr int BN = 256; // activation rows per tile
constexpr int FN = BN / 32;

// s_waitcnt immediate (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt in
// 6:4, lgkmcnt in 11:8): vmcnt <= vm and lgkmcnt == 0.
constexpr int waitcnt_vm_lgkm0(int vm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4); }

enum { kBigDense = 0, kBigGateUp = 1, kBigDown = 2, kBigSplit = 3 };

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
    int splits; // kBigSplit: K is cut into this many equal runs of whole super-blocks
    const float *wts; // gate/up with weight_input: the slot weights, [T*topk]
    int weight_input;
};

} // namespace

// MODE kBigSplit: the dense tiles, each over one of p.splits equal runs of
// K; the binary32 partial tile goes to p.y as [split][N][M] for
// gemm_splitk_reduce_kernel.
// MODE kBigDense: Y = X W^T over (32 NW) x 256 tiles.  MODE kBigGateUp: a tile
// is 16 NW rows of an expert's gate matrix and the same rows of its up matrix
// against up to 256 of the expert's tokens, gathered through the sorted
// assignment list; h = binary16(silu(g) * u) is written.  MODE kBigDown:
// 32 NW rows of an expert's down matrix against its rows of h, binary32
// outputs.
// One tile: weight rows from m0 (BM = 32 NW / KG of them) against activation
// rows n0 .. n0 + 32 FNT - 1 (nvalid of them valid), over all of K (or split's
// run of it).  FNT = 8 (256 activation rows) for the full tiles; the expert
// products take FNT = 2 (64 rows) for a tile of 64 tokens or fewer, the
// remainder of an expert's tokens, whose matrix work would otherwise be mostly
// empty.
// KG > 1 (dense product only): the NW waves form KG groups of NW / KG; group g
// runs the whole tile over the g-th of KG equal runs of K with its own LDS
// buffers (KG (32 FNT x 64)-half slices per buffer), and at the end groups
// 1 .. KG-1 hand their binary32 partial tiles to group 0 through LDS, which
// adds them in group order (deterministic) and stores the tile.  The groups
// step in lockstep (same number of steps, one barrier per step for all).
template <int MODE, int NW, int FNT, int KG = 1, bool Q8 = false>
__device__ __forceinline__ void big_tile(const BigParams &p, int m0, int n0, int nvalid, int e,
                                         int split, _Float16 *sX0, _Float16 *sX1)
{
    constexpr int FN = FNT;
    constexpr int NWG = NW / KG;           // waves per K group
    constexpr int BM = 32 * NWG;           // weight rows per tile (gate/up: gate + up rows)
    constexpr int NQ = 4 * FN / NWG;       // 1 KB activation copies per wave per step
    constexpr int GX = 32 * FN * KS;       // halves of one group's slice of an LDS buffer
    constexpr int VPM = FN >= 8 ? 3 : 24 / FN; // dequant instructions placed after each matrix instruction
    static_assert(NQ >= 1, "each wave copies at least 1 KB per step");
    static_assert(KG == 1 || MODE == kBigDense, "K groups: dense product only");
    static_assert(NW % KG == 0, "whole waves per K group");
    const int M = p.M, K = p.K;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wall = __builtin_amdgcn_readfirstlane(tid >> 6); // wave-uniform
    const int kg = wall / NWG;   // K group
    const int wave = wall % NWG; // wave within its K group
    const int r = lane & 31, h = lane >> 5;
    const int nsb = K >> 8;
    // bytes per 256 weights of a row: one Q4_K super-block or eight Q8_0 blocks
    constexpr int kSbBytes = Q8 ? 8 * kQ80Bytes : kQ4kBytes;
    constexpr int NWL = Q8 ? 4 : 2; // weight loads per lane and step
    const size_t rowb = (size_t)nsb * kSbBytes;
    // split products: this workgroup's run of K starts at super-block sb0;
    // K groups: this group's run
    const int krun = MODE == kBigSplit ? K / p.splits : K / KG;
    const int sb0 = MODE == kBigSplit ? split * (krun >> 8) : kg * (krun >> 8);
    const int nk = krun / KS;

    // this lane's weight row
    int wr_want = m0 + 32 * wave + r;
    const uint8_t *wbase = p.w;
    if constexpr (MODE == kBigGateUp) {
        wr_want = m0 + 16 * wave + (r & 15);
        wbase = (r < 16 ? p.w : p.w2);
    }
    if constexpr (MODE != kBigDense)
        wbase += (size_t)e * p.expert_bytes;
    const bool wok = wr_want < M;
    const uint8_t *wrow =
        wbase + (size_t)(wok ? wr_want : M - 1) * rowb + (size_t)sb0 * kSbBytes;

    // activation copies: copy q of wave v fills LDS 16-byte units
    // [(NQ v + q) * 64, +64), i.e. row (NQ v + q) * 8 + lane / 8, slot lane % 8,
    // holding chunk (lane % 8) ^ swz(row) (byte offsets below 2^31: the
    // activation matrix is smaller on this path)
    auto swz = [](int row) { return (row >> 1) & 7; };
    uint32_t xoff[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int row = (NQ * wave + q) * 8 + (lane >> 3);
        const int nl = min(row, nvalid - 1); // rows past the tile repeat its last
        int grow = n0 + nl;
        if constexpr (MODE == kBigGateUp)
            grow = p.sorted[grow] / p.topk; // the token of that sorted position
        xoff[q] = ((uint32_t)grow * (uint32_t)K + 8u * (uint32_t)((lane & 7) ^ swz(row))) * 2u;
    }
    const uint32_t lds0 = (uint32_t)(size_t)(const __attribute__((address_space(3))) void *)sX0;
    const uint32_t lds1 = (uint32_t)(size_t)(const __attribute__((address_space(3))) void *)sX1;
    const uint32_t gofs = (uint32_t)kg * (2u * GX); // this group's slice, bytes
    const uint32_t mb0 = __builtin_amdgcn_readfirstlane(lds0 + gofs + (uint32_t)wave * (1024u * NQ));
    const uint32_t mb1 = __builtin_amdgcn_readfirstlane(lds1 + gofs + (uint32_t)wave * (1024u * NQ));
    const uint16_t *x = p.x + (size_t)sb0 * 256;
    auto issue_x = [&](int kt, int buf) {
        const uint16_t *xk = x + (size_t)kt * KS; // wave-uniform
#pragma unroll
        for (int q = 0; q < NQ; ++q)
            load_lds16(xk, xoff[q], (buf ? mb1 : mb0) + 1024u * q);
    };

    // packed weights of the steps ahead: slot = step & 3; step kt + 3 is
    // loaded during step kt and has until the end of step kt + 1 to land (the
    // wait that ends each step leaves only the newest step's NWL loads in
    // flight).  Quant groups 0 and 1 need only the first 12 header bytes (d,
    // dmin and scale/min bytes 0-7); loading 16 would leave the fourth
    // register of the load dead, and the compiler may then reuse it while the
    // load is in flight, which costs a wait for every load issued before it
    // (the activation copies included).
    uint4 rh[4], rq[4];
    uint32_t r8b[4], r8d[4]; // Q8_0: the 4-byte loads
    auto issue_w = [&](int kt, int slot, int g) {
        if constexpr (Q8) {
            // step kt is blocks 2kt and 2kt+1 (68 bytes from a 4-byte aligned
            // start): lane half h takes bytes 16h .. 16h+19 (its 16 quants of
            // the first block start at byte 2 + 16h), its 16 quants of the
            // second block (bytes 36 + 16h ..) and the dword holding the scale
            // it lacks (the second block's for h = 0, the first's for h = 1)
            const uint8_t *st = wrow + (size_t)kt * (2 * kQ80Bytes);
            const u32x4a4 a = *(g_u32x4a4 *)(st + 16 * h);
            rh[slot] = make_uint4(a.x, a.y, a.z, a.w);
            r8b[slot] = *(g_u32 *)(st + 16 + 16 * h);
            const u32x4a4 c = *(g_u32x4a4 *)(st + 36 + 16 * h);
            rq[slot] = make_uint4(c.x, c.y, c.z, c.w);
            r8d[slot] = *(g_u32 *)(st + (h ? 0 : 32));
            (void)g;
            return;
        }
        const uint8_t *blk = wrow + (size_t)(kt >> 2) * kQ4kBytes;
        if (g < 2) {
            const u32x3 v = *(g_u32x3 *)(blk);
            rh[slot] = make_uint4(v.x, v.y, v.z, 0u);
        } else {
            rh[slot] = gload16(blk);
        }
        rq[slot] = gload16(blk + 16 + 32 * g + 16 * h);
    };
    // A operands of one step from slot `slot`, quant group g
    auto dequant = [&](int slot, int g, half8_t(&dst)[4]) {
        if constexpr (Q8) {
            // sub-steps 0, 1: quants 16h .. 16h+15 of the first block; 2, 3:
            // of the second block
            const uint4 a = rh[slot], c = rq[slot];
            const uint32_t b = r8b[slot], dd = r8d[slot];
            // rows past M (read from row M - 1) get zero weights
            const uint32_t d0 = wok ? (h ? (dd & 0xFFFFu) : (a.x & 0xFFFFu)) : 0u;
            const uint32_t d1 = wok ? (h ? (b >> 16) : (dd >> 16)) : 0u;
            const h2_t d0v = __builtin_bit_cast(h2_t, d0 | (d0 << 16));
            const h2_t d1v = __builtin_bit_cast(h2_t, d1 | (d1 << 16));
            const uint32_t q0[4] = {__builtin_amdgcn_alignbyte(a.y, a.x, 2),
                                    __builtin_amdgcn_alignbyte(a.z, a.y, 2),
                                    __builtin_amdgcn_alignbyte(a.w, a.z, 2),
                                    __builtin_amdgcn_alignbyte(b, a.w, 2)};
            const uint32_t q1[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
            for (int v = 0; v < 2; ++v) {
                uint32_t w[4];
                deq4_q8(q0[2 * v], d0v, w[0], w[1]);
                deq4_q8(q0[2 * v + 1], d0v, w[2], w[3]);
                dst[v] = __builtin_bit_cast(half8_t, make_uint4(w[0], w[1], w[2], w[3]));
                deq4_q8(q1[2 * v], d1v, w[0], w[1]);
                deq4_q8(q1[2 * v + 1], d1v, w[2], w[3]);
                dst[2 + v] = __builtin_bit_cast(half8_t, make_uint4(w[0], w[1], w[2], w[3]));
            }
            (void)g;
            return;
        }
        const uint4 hd = rh[slot];
        uint32_t scl, ml, sch, mh;
        if (g < 2) {
            scl = (hd.y >> (16 * g)) & 63u;
            ml = (hd.z >> (16 * g)) & 63u;
            sch = (hd.y >> (16 * g + 8)) & 63u;
            mh = (hd.z >> (16 * g + 8)) & 63u;
        } else {
            const int s0 = 16 * (g - 2), s1 = s0 + 8;
            scl = ((hd.w >> s0) & 15u) | (((hd.y >> (s0 + 6)) & 3u) << 4);
            ml = ((hd.w >> (s0 + 4)) & 15u) | (((hd.z >> (s0 + 6)) & 3u) << 4);
            sch = ((hd.w >> s1) & 15u) | (((hd.y >> (s1 + 6)) & 3u) << 4);
            mh = ((hd.w >> (s1 + 4)) & 15u) | (((hd.z >> (s1 + 6)) & 3u) << 4);
        }
        const float d = wok ? half_to_float(hd.x) : 0.f;
        const float dmin = wok ? half_to_float(hd.x >> 16) : 0.f;
        // quants enter as q*2^-24 (low nibbles) and 16q*2^-24 (high nibbles)
        const float sl = d * (float)scl * 16777216.f, ol = -dmin * (float)ml;
        const float sh = d * (float)sch * 1048576.f, oh = -dmin * (float)mh;
        const uint32_t q[4] = {rq[slot].x, rq[slot].y, rq[slot].z, rq[slot].w};
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            // bytes 8c..8c+7 of the lane's slice: low nibbles feed sub-step c,
            // high nibbles sub-step 2 + c
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
            dst[c] = __builtin_bit_cast(half8_t, lo);
            dst[2 + c] = __builtin_bit_cast(half8_t, hi);
        }
    };

    float16_t acc[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j)
        acc[j] = float16_t{};

    // B fragment j of sub-step s: activation row 32j + r, chunk
    // 4(s >> 1) + 2h + (s & 1)
    half8_t bf0[FN], bf1[FN];
    auto read_b = [&](int buf, int s, half8_t(&bf)[FN]) {
        const int c = 2 * h + (s & 1) + 4 * (s >> 1);
        const _Float16 *X = (buf ? sX1 : sX0) + kg * GX;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int row = 32 * j + r;
            bf[j] = *reinterpret_cast<const half8_t *>(X + row * KS + 8 * (c ^ swz(row)));
        }
    };
    auto mfma = [&](const half8_t &a, const half8_t(&bf)[FN]) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, bf[j], acc[j], 0, 0, 0);
    };

    // One K step kt with S = kt % 4: the activations of step kt are in LDS
    // buffer S & 1, its A operands in `cur` (dequantized during step kt-1),
    // the packed weights of step kt+1 in slot (S+1) & 3 (arrived), those of
    // step kt+2 in slot (S+2) & 3 (in flight), and step kt+3's weight loads go
    // to slot (S+3) & 3.
    auto step = [&](int kt, int S, half8_t(&cur)[4], half8_t(&nxt)[4]) {
        const int buf = S & 1;
        const int n1 = kt + 1 < nk ? kt + 1 : nk - 1;
        const int n3 = kt + 3 < nk ? kt + 3 : nk - 1;
        read_b(buf, 0, bf0);
        // copies first: the wait that ends the step then leaves exactly this
        // step's NWL weight loads in flight
        issue_x(n1, buf ^ 1);
        issue_w(n3, (S + 3) & 3, (S + 3) & 3);
        read_b(buf, 1, bf1);
        mfma(cur[0], bf0);
        dequant((S + 1) & 3, (S + 1) & 3, nxt);
        read_b(buf, 2, bf0);
        mfma(cur[1], bf1);
        read_b(buf, 3, bf1);
        mfma(cur[2], bf0);
        mfma(cur[3], bf1);
        // schedule: the first sub-step's reads, the NWL weight loads, then
        // each matrix instruction followed by one LDS read and three VALU ops
        __builtin_amdgcn_sched_group_barrier(0x100, FN, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, NWL, 0);
#pragma unroll
        for (int u = 0; u < 4 * FN; ++u) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
        }
        // this wave's copies for the next step and the weights of step kt+2
        // have landed (loads complete in issue order; the NWL loads of step
        // kt+3 stay in flight); after the barrier every wave's copies have.
        // The compiler counts only the weight loads, so by its count too the
        // weights of step kt+2 are in and it inserts no wait of its own
        // before their dequantization in the next step.
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(NWL));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };

    // prologue: step 0's activations in LDS, A operands of step 0, packed
    // weights of step 1 in slot 1, step 2's on the way to slot 2
    half8_t a0[4], a1[4];
    // (Q8_0: fenced so that each step's four loads stay together, since the
    // wait below counts on step 2's being the newest; the compiler keeps the
    // Q4_K loads in order by itself)
    issue_x(0, 0);
    issue_w(0, 0, 0);
    if constexpr (Q8)
        __builtin_amdgcn_sched_barrier(0);
    issue_w(1, 1, 1); // nk >= 4
    if constexpr (Q8)
        __builtin_amdgcn_sched_barrier(0);
    issue_w(2, 2, 2);
    if constexpr (Q8)
        __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(NWL));
    dequant(0, 0, a0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);

    // nk = K / 64 is a multiple of 4 (K % 256 == 0)
    for (int kt = 0; kt < nk; kt += 4) {
        step(kt, 0, a0, a1);
        step(kt + 1, 1, a1, a0);
        step(kt + 2, 2, a0, a1);
        step(kt + 3, 3, a1, a0);
    }

    if constexpr (KG > 1) {
        // every wave's LDS reads and copies ended before the last step's
        // barrier; the partial tiles of groups 1.. go to [g-1][wave][j][v4]
        // (a float4 per lane), group 0 adds them in group order
        float4_t *red = reinterpret_cast<float4_t *>(sX0);
        if (kg > 0) {
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int v4 = 0; v4 < 4; ++v4)
                    red[(((kg - 1) * NWG + wave) * FN * 4 + 4 * j + v4) * 64 + lane] =
                        float4_t{acc[j][4 * v4], acc[j][4 * v4 + 1], acc[j][4 * v4 + 2],
                                 acc[j][4 * v4 + 3]};
        }
        __syncthreads();
        if (kg > 0)
            return;
#pragma unroll
        for (int g = 1; g < KG; ++g)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
#pragma unroll
                for (int v4 = 0; v4 < 4; ++v4) {
                    const float4_t v = red[(((g - 1) * NWG + wave) * FN * 4 + 4 * j + v4) * 64 + lane];
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        acc[j][4 * v4 + c] += v[c];
                }
                // the sums land here, before the next fragment's reads (the
                // compiler would otherwise sink the additions into the stores
                // and hold every read's registers until then: 256 VGPRs)
                asm volatile("" : "+v"(acc[j])::"memory");
            }
    }

    // epilogue: element v of fragment j is fragment row 8*(v/4) + 4*h + v%4
    // and activation row 32j + r of the tile
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int nl = 32 * j + r;
        if (nl >= nvalid)
            continue;
        const float16_t a = acc[j];
        if constexpr (MODE == kBigGateUp) {
            // elements v < 8 are gate rows 8*(v/4) + 4h + v%4 of the wave's 16,
            // elements v + 8 the same rows of up
            uint16_t *hr = reinterpret_cast<uint16_t *>(p.y) + (size_t)(n0 + nl) * M;
            // the slot weight on the expert's input scales g and u alike
            const float pw = p.weight_input ? p.wts[p.sorted[n0 + nl]] : 1.f;
#pragma unroll
            for (int v4 = 0; v4 < 2; ++v4) {
                const int m = m0 + 16 * wave + 8 * v4 + 4 * h;
                float o[4];
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    o[c] = silu(pw * a[4 * v4 + c]) * (pw * a[8 + 4 * v4 + c]);
                *reinterpret_cast<uint2 *>(hr + m) =
                    make_uint2(pack_half2(o[0], o[1]), pack_half2(o[2], o[3]));
            }
        } else if constexpr (MODE == kBigSplit) {
            float *dr = reinterpret_cast<float *>(p.y) + ((size_t)split * p.N + n0 + nl) * M;
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) {
                const int m = m0 + 32 * wave + 8 * v4 + 4 * h;
                if (m + 3 < M && (M & 3) == 0) {
                    *reinterpret_cast<float4_t *>(dr + m) =
                        float4_t{a[4 * v4], a[4 * v4 + 1], a[4 * v4 + 2], a[4 * v4 + 3]};
                } else {
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        if (m + c < M)
                            dr[m + c] = a[4 * v4 + c];
                }
            }
        } else if constexpr (MODE == kBigDown) {
            float *dr = reinterpret_cast<float *>(p.y) + (size_t)(n0 + nl) * M;
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) {
                const int m = m0 + 32 * wave + 8 * v4 + 4 * h;
                *reinterpret_cast<float4_t *>(dr + m) =
                    float4_t{a[4 * v4], a[4 * v4 + 1], a[4 * v4 + 2], a[4 * v4 + 3]};
            }
        } else {
            uint16_t *yr = reinterpret_cast<uint16_t *>(p.y) + (size_t)(n0 + nl) * M;
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) {
                const int m = m0 + 32 * wave + 8 * v4 + 4 * h;
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
}

// Q8: Q8_0 weights (rows of K/32 34-byte blocks) instead of Q4_K
template <int MODE, int NW, bool Q8 = false>
__global__ __launch_bounds__(64 * NW, 8 / NW) void gemm_q4k_big_kernel(BigParams p)
{
    constexpr int BM = 32 * NW; // weight rows per tile (gate/up: gate + up rows)
    __shared__ __attribute__((aligned(16))) _Float16 sX0[BN * KS];
    __shared__ __attribute__((aligned(16))) _Float16 sX1[BN * KS];
    int m0, n0, nvalid, e = 0, split = 0;
    if constexpr (MODE == kBigDense || MODE == kBigSplit) {
        // XCD-aware tile order: the hardware deals consecutive workgroups to
        // the 8 XCDs in turn; give XCD x the contiguous tile run
        // [x*T/8, (x+1)*T/8) (split products: units split-major, so an XCD's
        // run shares its splits' activation panels).
        const int b = blockIdx.x;
        const int units = p.tiles_total * (MODE == kBigSplit ? p.splits : 1);
        const int per = (units + 7) / 8;
        int tile = (b % 8) * per + b / 8;
        if (tile >= units)
            return;
        if constexpr (MODE == kBigSplit) {
            split = tile / p.tiles_total;
            tile -= split * p.tiles_total;
        }
        const int n_t = tile / p.tiles_m, m_t = tile % p.tiles_m;
        m0 = m_t * BM;
        n0 = n_t * BN;
        nvalid = p.N - n0 < BN ? p.N - n0 : BN;
        big_tile<MODE, NW, FN, 1, Q8>(p, m0, n0, nvalid, e, split, sX0, sX1);
    } else {
        // XCD-aware order: the hardware deals consecutive workgroups to the 8
        // XCDs in turn; XCD x takes token tiles x, x + 8, x + 16, ... each
        // with all its row tiles, so that a token tile's activations are read
        // into one XCD's L2 (gridDim.y is a multiple of 8, which makes the
        // map one-to-one)
        const int rt = (int)gridDim.x;
        const int b = (int)blockIdx.x + rt * (int)blockIdx.y;
        const int k = b >> 3;
        const int t = 8 * (k / rt) + (b & 7);
        if (t >= p.offsets[p.E + 1])
            return;
        e = p.tiles[t];
        n0 = p.tiles[p.max_tiles + t]; // first sorted position of the tile
        const int end = p.offsets[e + 1];
        nvalid = end - n0 < BN ? end - n0 : BN;
        m0 = (k % rt) * (MODE == kBigGateUp ? BM / 2 : BM);
        // the same for the whole workgroup
        if (__builtin_amdgcn_readfirstlane(nvalid) <= 64)
            big_tile<MODE, NW, 2, 1, Q8>(p, m0, n0, nvalid, e, split, sX0, sX1);
        else
            big_tile<MODE, NW, FN, 1, Q8>(p, m0, n0, nvalid, e, split, sX0, sX1);
    }
}

// The dense product on tiles of 256/KG weight rows x 128 activation rows, K
// split across KG groups of waves inside the workgroup (see big_tile); tiles
// in the same XCD-aware order as the dense kernel.
template <int KG, bool Q8 = false>
__global__ __launch_bounds__(512, 1) void gemm_q4k_kgroups_kernel(BigParams p)
{
    constexpr int FNT = 4, BM = 256 / KG, BNT = 32 * FNT, GX = BNT * KS;
    // two step buffers of KG group slices; after the last step the partial
    // tiles of groups 1..KG-1 reuse the space
    __shared__ __attribute__((aligned(16))) _Float16 sX[2 * KG * GX];
    static_assert((KG - 1) * BM * BNT * 4 <= (int)sizeof(sX), "partial tiles fit the step buffers");
    const int b = blockIdx.x;
    const int per = (p.tiles_total + 7) / 8;
    const int tile = (b % 8) * per + b / 8;
    if (tile >= p.tiles_total)
        return;
    const int n_t = tile / p.tiles_m, m_t = tile % p.tiles_m;
    const int m0 = m_t * BM, n0 = n_t * BNT;
    const int nvalid = p.N - n0 < BNT ? p.N - n0 : BNT;
    big_tile<kBigDense, 8, FNT, KG, Q8>(p, m0, n0, nvalid, 0, 0, sX, sX + KG * GX);
}

// Y[n][m] = binary16(sum over s = 0..splits-1 of part[s][n][m]), summed in
// binary32 in split order (deterministic), one rounding to binary16.
__global__ __launch_bounds__(256) void gemm_splitk_reduce_kernel(const float *__restrict__ part,
                                                                 uint16_t *__restrict__ y,
                                                                 int64_t count, int splits)
{
    // four outputs per thread (count is a multiple of 4: M % 4 == 0), else one
    const bool vec = (count & 3) == 0;
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * (vec ? 4 : 1);
    if (i >= count)
        return;
    if (vec) {
        float4_t s = *reinterpret_cast<const float4_t *>(part + i);
        for (int k = 1; k < splits; ++k)
            s += *reinterpret_cast<const float4_t *>(part + (int64_t)k * count + i);
        *reinterpret_cast<uint2 *>(y + i) = make_uint2(pack_half2(s[0], s[1]), pack_half2(s[2], s[3]));
    } else {
        float s = part[i];
        for (int k = 1; k < splits; ++k)
            s += part[(int64_t)k * count + i];
        y[i] = (uint16_t)pack_half2(s, 0.f);
    }
}

namespace {

int64_t dense_tiles(int64_t M, int64_t N, int bm) { return ((M + bm - 1) / bm) * ((N + BN - 1) / BN); }

} // namespace

int gemm_big_choice(int64_t M, int64_t K, int64_t N)
{
    // enough tiles to fill the chip: 256 x 256 tiles one per CU, else
    // 128 x 256 tiles two per CU
    if (M < 128 || N < 256 || !gemm_big_fits(M, K, N))
        return 0;
    if (dense_tiles(M, N, 256) >= 256)
        return 256;
    if (dense_tiles(M, N, 128) >= 192)
        return 128;
    return 0;
}

bool gemm_big_fits(int64_t M, int64_t K, int64_t N)
{
    // 32-bit activation offsets; K a positive multiple of 256
    return M >= 1 && N >= 1 && K >= 256 && K % 256 == 0 && N * K * 2 < (1ll << 31);
}

hipError_t launch_gemm_big(const void *w, const uint16_t *x, uint16_t *y, int64_t M, int64_t K,
                           int64_t N, int bm, bool q8, hipStream_t s)
{
    if ((bm != 256 && bm != 128) || !gemm_big_fits(M, K, N))
        return hipErrorInvalidValue;
    BigParams p{};
    p.w = (const uint8_t *)w;
    p.x = x;
    p.y = y;
    p.M = (int)M;
    p.K = (int)K;
    p.N = (int)N;
    p.tiles_m = (int)((M + bm - 1) / bm);
    p.tiles_total = (int)dense_tiles(M, N, bm);
    const int grid = (p.tiles_total + 7) / 8 * 8;
    if (q8 && bm == 256)
        hipLaunchKernelGGL((gemm_q4k_big_kernel<kBigDense, 8, true>), dim3((unsigned)grid),
                           dim3(512), 0, s, p);
    else if (q8)
        hipLaunchKernelGGL((gemm_q4k_big_kernel<kBigDense, 4, true>), dim3((unsigned)grid),
                           dim3(256), 0, s, p);
    else if (bm == 256)
        hipLaunchKernelGGL((gemm_q4k_big_kernel<kBigDense, 8>), dim3((unsigned)grid), dim3(512), 0, s, p);
    else
        hipLaunchKernelGGL((gemm_q4k_big_kernel<kBigDense, 4>), dim3((unsigned)grid), dim3(256), 0, s, p);
    return hipGetLastError();
}

int gemm_kgroups_choice(int64_t M, int64_t K, int64_t N)
{
    // Only where the 256 x 256 tiles do not fill the device.  Estimated time:
    // rounds of tiles on the device (one workgroup per CU at a time) times
    // the time of one such round per 1024 of K, measured on 4096 x 14336 and
    // 4096/6144/14336 x 4096 products with 128-1024 activation rows:
    // 128 x 256 tiles (two per CU) 18 us, K groups of 2 (128 x 128 tiles)
    // 10 us, K groups of 4 (64 x 128 tiles) 6.6 us.  The 128 x 256 tiles
    // count when the large-tile choice would take them; the small-tile
    // kernels otherwise, which the K groups beat wherever they apply.
    if (M < 1 || N < 1 || K < 256 || K % 256 != 0 || !gemm_big_fits(M, K, N))
        return 0;
    const int big = gemm_big_choice(M, K, N);
    if (big == 256)
        return 0;
    const int64_t cus = device_cus();
    auto rounds = [&](int64_t tiles) { return (double)((tiles + cus - 1) / cus); };
    const int64_t nsb = K / 256;
    const double inf = 1e300;
    const double t128 = big == 128 ? rounds(dense_tiles(M, N, 128)) * 18.0 : inf;
    const double kg2 = nsb % 2 == 0 ? rounds(((M + 127) / 128) * ((N + 127) / 128)) * 10.0 : inf;
    const double kg4 = nsb % 4 == 0 ? rounds(((M + 63) / 64) * ((N + 127) / 128)) * 6.6 : inf;
    if (kg4 < inf && kg4 <= kg2 && kg4 < t128)
        return 4;
    if (kg2 < inf && kg2 < t128)
        return 2;
    return 0;
}

hipError_t launch_gemm_kgroups(const void *w, const uint16_t *x, uint16_t *y, int64_t M,
                               int64_t K, int64_t N, int kg, bool q8, hipStream_t s)
{
    if ((kg != 2 && kg != 4) || (K / 256) % kg != 0 || !gemm_big_fits(M, K, N))
        return hipErrorInvalidValue;
    const int bm = 256 / kg;
    BigParams p{};
    p.w = (const uint8_t *)w;
    p.x = x;
    p.y = y;
    p.M = (int)M;
    p.K = (int)K;
    p.N = (int)N;
    p.tiles_m = (int)((M + bm - 1) / bm);
    p.tiles_total = (int)(p.tiles_m * ((N + 127) / 128));
    const int grid = (p.tiles_total + 7) / 8 * 8;
    if (kg == 4 && q8)
        hipLaunchKernelGGL((gemm_q4k_kgroups_kernel<4, true>), dim3((unsigned)grid), dim3(512), 0, s, p);
    else if (q8)
        hipLaunchKernelGGL((gemm_q4k_kgroups_kernel<2, true>), dim3((unsigned)grid), dim3(512), 0, s, p);
    else if (kg == 4)
        hipLaunchKernelGGL((gemm_q4k_kgroups_kernel<4>), dim3((unsigned)grid), dim3(512), 0, s, p);
    else
        hipLaunchKernelGGL((gemm_q4k_kgroups_kernel<2>), dim3((unsigned)grid), dim3(512), 0, s, p);
    return hipGetLastError();
}

int gemm_splitk_choice(int64_t M, int64_t K, int64_t N)
{
    // the divisor s of K/256 (s <= 32) with the least estimated time, in
    // units of one 64-weight step of a round of 256 x 256 tiles:
    //   ceil(tiles*s / CUs) * (K/64)/s   (rounds of tiles, each K/s long)
    // + 8*s*N*M / kBytesPerStep           (binary32 partials written and read)
    // with kBytesPerStep = 1e7 bytes: a step takes about 2 us, in which HBM
    // moves about 1e7 bytes.  Ties go to the smaller s.
    constexpr double kBytesPerStep = 1e7;
    if (M < 1 || N < 1 || K < 256 || K % 256 != 0)
        return 0;
    const int64_t tiles = dense_tiles(M, N, 256), nsb = K / 256;
    int64_t cus = 0;
    {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
            cus = v;
        if (cus <= 0)
            cus = 256;
    }
    const double nk = (double)(K / 64);
    auto cost = [&](int64_t s) {
        return (double)((tiles * s + cus - 1) / cus) * nk / (double)s +
               8.0 * (double)s * (double)N * (double)M / kBytesPerStep;
    };
    int best = 1;
    double best_cost = cost(1);
    for (int64_t s = 2; s <= 32 && s <= nsb; ++s) {
        if (nsb % s)
            continue;
        const double c = cost(s);
        if (c < best_cost - 1e-9) {
            best = (int)s;
            best_cost = c;
        }
    }
    return best;
}

hipError_t launch_gemm_splitk(const void *w, const uint16_t *x, uint16_t *y, int64_t M, int64_t K,
                              int64_t N, int splits, float *ws, hipStream_t s)
{
    if (splits < 1 || (K / 256) % splits != 0 || !gemm_big_fits(M, K, N))
        return hipErrorInvalidValue;
    BigParams p{};
    p.w = (const uint8_t *)w;
    p.x = x;
    p.y = ws;
    p.M = (int)M;
    p.K = (int)K;
    p.N = (int)N;
    p.splits = splits;
    p.tiles_m = (int)((M + 255) / 256);
    p.tiles_total = (int)dense_tiles(M, N, 256);
    const int64_t units = (int64_t)p.tiles_total * splits;
    const int grid = (int)((units + 7) / 8 * 8);
    hipLaunchKernelGGL((gemm_q4k_big_kernel<kBigSplit, 8>), dim3((unsigned)grid), dim3(512), 0, s, p);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    const int64_t count = M * N;
    const int64_t threads = (count & 3) == 0 ? count / 4 : count;
    hipLaunchKernelGGL(gemm_splitk_reduce_kernel, dim3((unsigned)((threads + 255) / 256)),
                       dim3(256), 0, s, ws, y, count, splits);
    return hipGetLastError();
}

// Split-K partials for callers that cannot allocate device memory: one array
// per device (each GPU the library runs on holds its own copy until the
// process ends).  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in): it uses the device address that
// hipGetSymbolAddress returns, looked up once per device.
static __device__ __align__(256) float scratch[kSplitkScratchBytes / sizeof(float)];

hipError_t splitk_scratch(float **out)
{
    static std::mutex mu;
    static float *addr[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= 64)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        if (!ptr)
            return hipErrorInvalidSymbol;
        addr[dev] = static_cast<float *>(ptr);
    }
    *out = addr[dev];
    return hipSuccess;
}

int moe_big_token_tile() { return BN; }

bool moe_big_applies(int64_t assignments, int64_t experts, int64_t H, int64_t I)
{
    // about 160 or more tokens per expert on average, and 32-bit byte offsets
    // for the activations and h
    return assignments >= 160 * experts && assignments * I * 2 < (1ll << 31) &&
           assignments * H * 2 < (1ll << 31) && I % 128 == 0 && H % 256 == 0;
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
    p.wts = a.wts;
    p.weight_input = a.weight_input;

    // gate/up with the SwiGLU epilogue: h[pos][0..I) in binary16, 128 rows of
    // I per workgroup
    p.w = a.w_gate;
    p.w2 = a.w_up;
    p.x = a.x;
    p.y = a.ws + a.off[4];
    p.M = (int)a.I;
    p.K = (int)a.H;
    p.expert_bytes = a.q8_0 ? a.I * (a.H / kQ80Weights) * kQ80Bytes
                            : a.I * (a.H / kQ4kWeights) * kQ4kBytes;
    // token tiles rounded up to a multiple of 8 for the XCD-aware order
    const unsigned ty = (unsigned)((max_tiles + 7) / 8 * 8);
    if (a.q8_0)
        hipLaunchKernelGGL((gemm_q4k_big_kernel<kBigGateUp, 8, true>), dim3((unsigned)(a.I / 128), ty),
                           dim3(512), 0, s, p);
    else
        hipLaunchKernelGGL((gemm_q4k_big_kernel<kBigGateUp, 8>), dim3((unsigned)(a.I / 128), ty),
                           dim3(512), 0, s, p);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;

    // down: d[pos][0..H) in binary32, 256 rows of H per workgroup
    p.w = a.w_down;
    p.w2 = nullptr;
    p.x = reinterpret_cast<const uint16_t *>(a.ws + a.off[4]);
    p.y = a.ws + a.off[5];
    p.M = (int)a.H;
    p.K = (int)a.I;
    p.expert_bytes = a.q8_0 ? a.H * (a.I / kQ80Weights) * kQ80Bytes
                            : a.H * (a.I / kQ4kWeights) * kQ4kBytes;
    if (a.q8_0)
        hipLaunchKernelGGL((gemm_q4k_big_kernel<kBigDown, 8, true>), dim3((unsigned)(a.H / 256), ty),
                           dim3(512), 0, s, p);
    else
        hipLaunchKernelGGL((gemm_q4k_big_kernel<kBigDown, 8>), dim3((unsigned)(a.H / 256), ty),
                           dim3(512), 0, s, p);
    return hipGetLastError();
}

} // namespace gq
