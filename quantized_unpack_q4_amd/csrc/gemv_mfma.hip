// gemv_mfma.hip -- small-batch Q4_K matrix-vector products on the matrix cores.
//
// y[b][r] = sum_k w[r][k] * x[b][k] for 2 <= B <= 16 activation rows, with
// binary32 activations and results (page "Building a Rust Inference Engine
// That Matches Llama.cpp", section "Where the wins came from": the dequant is
// fused into the dot product; page "Frink", the paragraph on K-quant logits:
// activations stay binary32, never requantized).  Each output is computed in
// the factored form of a Q4_K super-block,
//     sum over sub-blocks j of  (d*sc_j) * sum_k q_k x_k  -  (dmin*m_j) * sum_k x_k,
// with both sums exact or binary32-accurate:
//   * sum_j sc_j * sum_k q_k x_k runs on v_mfma_f32_16x16x32_f16 with one
//     accumulator over the super-block; the lanes of quarter q own quant group
//     q (sub-blocks 2q and 2q+1, 32 bytes), so an instruction takes 8 weights
//     of one sub-block from each quarter: the quant times its sub-block's
//     6-bit scale (at most 945)
//     enters as the binary16 subnormal (sc*q)*2^-24 (exact) and the
//     activation as two binary16 halves hi + lo of x * 2^e, where 2^e (per
//     activation row and super-block) brings the largest |x| of the slice to
//     [2^14, 2^15); the products are exact and the sums binary32, every value
//     at least 2^-17 of that maximum keeps 22 significant bits and every value
//     at least 2^-20 of it a relative error below 2^-19;
//   * d * 2^-e is applied in binary32 once per super-block;
//   * sum_j (dmin*m_j) * sum_k x_k is a 16 x 16 x 8 product per super-block on
//     v_mfma_f32_16x16x4f32 from the binary32 sub-block sums of x.
// A sub-block of an activation row holding a non-zero |x| below 2^-20 of the
// super-block's largest, or more than 1/16 of the row's sum of |x| over the
// super-block, is left out of the split (its staged values and sum are zero)
// and computed exactly instead: each weight dequantized to its binary32 value
// times the binary32 activation (staged in LDS for such sub-blocks), summed
// over the four lanes that hold the sub-block.  The reasons are those of the
// batch-1 kernel: the split would lose the small values, and a dominant
// activation would meet a near-cancelling d*sc*q - dmin*m through the
// factored form, whose error follows the two terms, not their difference.
//
// Gate/up pairs (PAIR): a block is 64 output rows r of the gate and up
// matrices (same shape); a wave's two 16-row tiles are gate rows and up rows
// r0 .. r0+15, so each lane holds g and u of the same (row, activation row)
// and writes h = silu(g) * u (binary32) instead of either product.
//
// Work split.  A block is 192 consecutive rows of one matrix (4 waves x 3
// tiles x 16 rows; 128 with two tiles when there are too few blocks of 192
// for the grid) over the whole K.  The 256 threads first stage the
// activations of one super-block (B rows x 256) into LDS in the matrix-core
// layout, then every wave multiplies its two 16-row tiles against them; the
// staging of super-block s+1 and the packed weight loads of s+2 overlap the
// work on s.  Blocks of all matrices of a table are dealt to the workgroups by
// byte ranges of packed weights, as in the batch-1 streaming kernel.
#include "gq_device.h"
#include "gq_internal.h"
#include "gq_lds_dma.h"

namespace gq {

namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// rows per block: 64 per 16-row tile of each wave (two or three tiles)
constexpr int rows_per_block(int tiles) { return 64 * tiles; }
constexpr int NT = 256; // threads per workgroup

struct Smem {
    // activations of one super-block, [buffer][sub-block j][quarter q][slot]:
    // the 8 binary16 values of quarter q (k = 32j + 8q + {0,2,1,3,4,6,5,7}) of
    // activation row b sit in slot b ^ swz(j, q)
    uint4 xh[2][8][4][16];
    uint4 xl[2][8][4][16];
    float sx[2][8][16]; // [buffer][j][b] binary32 sum of x over sub-block j (0: computed exactly)
    float inv[2][16];   // [buffer][b] 2^-e
    uint64_t exact[2][4]; // [buffer][wave]: bit 16i + 2j: row 4*wave + i, sub-block j exact
    float xf[2][8][16][32]; // [buffer][j][b][k]: binary32 x of the sub-blocks computed exactly
};

// a sub-block holding a non-zero |x| below 1/kSplitSpan of its super-block's
// largest is computed exactly
constexpr float kSplitSpan = 1048576.f; // 2^20
// ... and one holding more than this fraction of its super-block's sum of |x|
constexpr float kDominant = 0.0625f;

// Slot swizzle: the 16 staging threads of one activation row write 16
// different (j, q) pairs at once; xor-ing the row index with a function of
// (j, q) spreads those writes over the banks (the reads, 16 rows of one (j, q),
// stay a permutation of 16 consecutive slots).
__device__ __forceinline__ int swz(int j, int q) { return (2 * j + (q >> 1)) & 15; }

__device__ __forceinline__ float dpp_f(float v, int ctrl_sel)
{
    int r;
    const int iv = __builtin_bit_cast(int, v);
    switch (ctrl_sel) {
    case 0: r = __builtin_amdgcn_update_dpp(0, iv, 0xB1, 0xF, 0xF, false); break;  // quad [1,0,3,2]
    case 1: r = __builtin_amdgcn_update_dpp(0, iv, 0x4E, 0xF, 0xF, false); break;  // quad [2,3,0,1]
    case 2: r = __builtin_amdgcn_update_dpp(0, iv, 0x124, 0xF, 0xF, false); break; // row_ror:4
    default: r = __builtin_amdgcn_update_dpp(0, iv, 0x128, 0xF, 0xF, false); break; // row_ror:8
    }
    return __builtin_bit_cast(float, r);
}

__device__ __forceinline__ uint32_t pack_h2(_Float16 a, _Float16 b)
{
    return __builtin_bit_cast(uint32_t, h2_t{a, b});
}

// hi and lo binary16 parts of xa*s and xb*s (s a power of two), packed
__device__ __forceinline__ void split2(float xa, float xb, float s, uint32_t &hi, uint32_t &lo)
{
    const _Float16 ha = (_Float16)(xa * s), hb = (_Float16)(xb * s);
    const _Float16 la = (_Float16)fmaf(xa, s, -(float)ha);
    const _Float16 lb = (_Float16)fmaf(xb, s, -(float)hb);
    hi = pack_h2(ha, hb);
    lo = pack_h2(la, lb);
}

// The staging of one activation slice by the 16 lanes of an activation row
// (lane sc_ holds x[16 sc_ .. 16 sc_ + 15] of the super-block, xr): the
// wave's exact-path flags (eb, one bit per even lane), and for stagers the
// binary16 hi/lo parts of quarters 2(sc_ & 1) + h, h = 0, 1, of sub-block
// sc_ / 2 (handed to put(h, hi, lo)), its sum sx (0 when it is computed
// exactly) and the row's 2^-e (inv).  Every lane of the wave must call it
// (cross-lane reductions).  Returns whether the sub-block is computed exactly.
template <typename Put>
__device__ __forceinline__ bool stage_slice(const float4_t (&xr)[4], bool stager, int lane,
                                            uint64_t &eb, float &sx, float &inv, Put &&put)
{
    const int sc_ = lane & 15;
    float m = 0.f, mn = INFINITY, l1 = 0.f, sum = 0.f;
    if (stager) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float a[4] = {fabsf(xr[i].x), fabsf(xr[i].y), fabsf(xr[i].z), fabsf(xr[i].w)};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                m = fmaxf(m, a[c]);
                mn = a[c] > 0.f ? fminf(mn, a[c]) : mn;
                l1 += a[c];
            }
            sum += (xr[i].x + xr[i].y) + (xr[i].z + xr[i].w);
        }
    }
    // the partner lane holds the other half of sub-block sc_ / 2
    float mj = fmaxf(m, dpp_f(m, 0));
    mn = fminf(mn, dpp_f(mn, 0));
    sum += dpp_f(sum, 0);
    // max and sum of |x| over the 16 lanes of this activation row
    m = mj;
    m = fmaxf(m, dpp_f(m, 1));
    m = fmaxf(m, dpp_f(m, 2));
    m = fmaxf(m, dpp_f(m, 3));
    l1 += dpp_f(l1, 0);
    l1 += dpp_f(l1, 1);
    l1 += dpp_f(l1, 2);
    l1 += dpp_f(l1, 3);
    const bool exact = stager && mj > 0.f && (kSplitSpan * mn < m || mj > kDominant * l1);
    eb = __ballot(exact && (sc_ & 1) == 0);
    if (!stager)
        return false;
    // 2^e with the largest |x| in [2^14, 2^15): exponent field 268 - ex,
    // kept in [1, 253] (zero or tiny slices get 2^126)
    const int ex = (int)((__builtin_bit_cast(uint32_t, m) >> 23) & 255u);
    const int fe = min(max(268 - ex, 1), 253);
    const float s = exact ? 0.f : __builtin_bit_cast(float, (uint32_t)fe << 23);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        // quarter 2(sc_ & 1) + h: elements k = 8h .. 8h+7 of this lane's 16
        const float4_t a = xr[2 * h], c = xr[2 * h + 1];
        uint4 hv, lv;
        split2(a.x, a.z, s, hv.x, lv.x); // k0, k2
        split2(a.y, a.w, s, hv.y, lv.y); // k1, k3
        split2(c.x, c.z, s, hv.z, lv.z); // k4, k6
        split2(c.y, c.w, s, hv.w, lv.w); // k5, k7
        put(h, hv, lv);
    }
    sx = exact ? 0.f : sum;
    inv = __builtin_bit_cast(float, (uint32_t)(254 - fe) << 23);
    return exact;
}

// Activations staged once per (product, super-block) for batch B into a
// caller workspace (gq_gemv_q4k_multi_batched_ws), as records that a block
// copies into LDS as they are:
//   bytes [0, 32)            exact-path flags, uint64 [4] (as Smem::exact)
//   bytes [32, 96)           2^-e per activation row, float [16]
//   bytes [96, 608)          sub-block sums, float [8 j][16 rows]
//   bytes [608, 608 + 512 B) binary16 hi parts, 16 bytes [8 j][4 q][B rows]
//   then the lo parts, same layout; padded to whole KiB (the copies move
//   1 KiB per wave instruction).  Rows past B are not written (their
//   outputs are discarded).
constexpr int kRecInv = 32, kRecSx = 96, kRecHi = 608;
constexpr int rec_bytes(int B) { return (kRecHi + 1024 * B + 1023) / 1024 * 1024; }
constexpr int kRecMax = rec_bytes(16);

__device__ __forceinline__ const void *uniform_ptr(const void *p)
{
    const uint64_t v = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const void *)(((uint64_t)hi << 32) | lo);
}

// Packed weights of one 16-row tile for one super-block, as this lane needs
// them: the 16-byte header of its row and the 32 bytes of quant group
// `quarter` (sub-blocks 2*quarter and 2*quarter + 1).
struct WTile {
    uint4 h, qa, qb;
};

// s_waitcnt immediate (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt in
// 6:4, lgkmcnt in 11:8): vmcnt <= vm and lgkmcnt == 0.
constexpr int waitcnt_vm_lgkm0(int vm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4); }

} // namespace

// PRE: the activations come pre-staged (one record per entry and super-block
// in ws, entry e's first record at prefix[e], rbytes each) and are copied into
// LDS by direct-to-LDS loads instead of being staged by every block.
// NS weight register sets: 2 (the weights of s+2 are issued once s is
// computed) or 3 (issued before s is computed, into the set s-1 used, so each
// weight load has two steps to land).
template <bool PAIR, int TW, bool PRE = false, int NS = 2>
__global__ __launch_bounds__(NT, 2) void gemv_q4k_mfma_kernel(const GemvEntry *__restrict__ table,
                                                               GemvEntry inline0, int n,
                                                               long long total, int B,
                                                               const uint8_t *__restrict__ w2,
                                                               const uint8_t *__restrict__ ws,
                                                               const int *__restrict__ prefix,
                                                               int rbytes)
{
    // TW 16-row tiles per wave; a pair's output row holds two weight rows
    // (tile 0 gate, tile 1 up), so a pair block is 64 output rows
    static_assert(!PAIR || TW == 2, "pairs take two tiles per wave");
    static_assert(!PRE || !PAIR, "pre-staged activations: tables of plain products");
    static_assert(2 * kRecMax <= (int)sizeof(Smem), "two records fit the staging area");
    static_assert(NS == 2 || NS == 3, "two or three weight register sets");
    static_assert(NS == 2 || !PRE || 3 * kRecMax <= (int)sizeof(Smem),
                  "three records fit the staging area");
    constexpr int RB = rows_per_block(TW);  // weight rows per block
    constexpr int RBO = PAIR ? RB / 2 : RB; // output rows per block
    __shared__ Smem sm;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, quarter = lane >> 4; // matrix-core lane coordinates

    // staging coordinates: activation row sb, 16 consecutive k from 16*sc_
    const int sb = 4 * wave + (lane >> 4), sc_ = lane & 15;
    const int sj = sc_ >> 1, sq0 = 2 * (sc_ & 1);

    // this workgroup's byte range of the concatenated packed weights
    const long long G = gridDim.x;
    const long long lo_b = total * (long long)blockIdx.x / G;
    const long long hi_b = total * ((long long)blockIdx.x + 1) / G;
    // entries are the same for the whole wave: say so, so that the buffer
    // resources built from them stay in scalar registers
    auto entry = [&](int e) -> GemvEntry {
        GemvEntry r = table ? table[e] : inline0;
        r.w = (const uint8_t *)uniform_ptr(r.w);
        r.x = (const float *)uniform_ptr(r.x);
        r.y = (float *)uniform_ptr(r.y);
        r.M = __builtin_amdgcn_readfirstlane(r.M);
        r.K = __builtin_amdgcn_readfirstlane(r.K);
        r.byte_begin = (long long)uniform_ptr((const void *)r.byte_begin);
        return r;
    };
    // first entry whose bytes reach past lo_b
    int e = 0;
    if (table) {
        int a = 0, z = n - 1;
        while (a < z) { // last entry with byte_begin <= lo_b
            const int mid = (a + z + 1) >> 1;
            if (table[mid].byte_begin <= lo_b)
                a = mid;
            else
                z = mid - 1;
        }
        e = a;
    }
    GemvEntry E = entry(e);
    int recbase = PRE ? __builtin_amdgcn_readfirstlane(prefix[e]) : 0; // first record of entry e
    long long rowb = (long long)(E.K >> 8) * kQ4kBytes; // bytes of one weight row
    long long blkb = rowb * RB;                          // bytes of one block
    // first block of entry e starting at or after lo_b
    int row0 = lo_b > E.byte_begin ? (int)((lo_b - E.byte_begin + blkb - 1) / blkb) * RBO : 0;

    for (;;) {
        while (row0 >= E.M) {
            if (++e >= n)
                return;
            E = entry(e);
            if constexpr (PRE)
                recbase = __builtin_amdgcn_readfirstlane(prefix[e]);
            rowb = (long long)(E.K >> 8) * kQ4kBytes;
            blkb = rowb * RB;
            row0 = 0;
        }
        if (E.byte_begin + (long long)(row0 / RBO) * blkb >= hi_b)
            return;

        // ---- one block: rows [row0, row0 + 128) of entry E, all of K ----
        const int K = E.K, M = E.M, nsb = K >> 8;
        // buffer loads: the matrix (and the activations) as a raw buffer
        // resource in scalar registers, one 32-bit byte offset per lane, the
        // super-block offset as the scalar offset (every matrix on this path
        // has fewer than 2^32 bytes of weights and of activations; reads past
        // the end return zeros)
        const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
            (void *)E.w, (short)0, (int)(uint32_t)((long long)M * rowb), 0x00020000);
        const __amdgpu_buffer_rsrc_t rw2 = PAIR ? __builtin_amdgcn_make_buffer_rsrc(
            (void *)w2, (short)0, (int)(uint32_t)((long long)M * rowb), 0x00020000) : rw;
        const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
            (void *)E.x, (short)0, (int)(uint32_t)((long long)B * K * 4), 0x00020000);
        int rows[TW];
        uint32_t woff[TW];
#pragma unroll
        for (int t = 0; t < TW; ++t) {
            // PAIR: tile 0 is gate rows, tile 1 the same up rows
            rows[t] = PAIR ? row0 + 16 * wave + col : row0 + 16 * TW * wave + 16 * t + col;
            woff[t] = (uint32_t)min(rows[t], M - 1) * (uint32_t)rowb;
        }
        auto load_w = [&](int s, WTile(&wt)[TW]) {
            const int so = s * kQ4kBytes;
#pragma unroll
            for (int t = 0; t < TW; ++t) {
                const __amdgpu_buffer_rsrc_t r = PAIR && t ? rw2 : rw;
                const u32x4 h = __builtin_amdgcn_raw_buffer_load_b128(r, (int)woff[t], so, 0);
                const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(
                    r, (int)(woff[t] + 32 * quarter) + 16, so, 0);
                const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(
                    r, (int)(woff[t] + 32 * quarter) + 32, so, 0);
                wt[t].h = make_uint4(h.x, h.y, h.z, h.w);
                wt[t].qa = make_uint4(a.x, a.y, a.z, a.w);
                wt[t].qb = make_uint4(b.x, b.y, b.z, b.w);
            }
        };
        const bool stager = sb < B;
        const int xoff = (sb * K + 16 * sc_) * 4;
        float4_t xr[4];
        auto load_x = [&](int s) {
            if (stager) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    xr[i] = __builtin_bit_cast(
                        float4_t, __builtin_amdgcn_raw_buffer_load_b128(rx, xoff + 16 * i, s * 1024, 0));
            }
        };
        // binary16 hi/lo parts, sub-block sums and scale of the staged slice
        auto store_x = [&](int buf) {
            uint64_t eb;
            float sx, inv;
            const bool exact = stage_slice(xr, stager, lane, eb, sx, inv,
                                           [&](int h, const uint4 &hv, const uint4 &lv) {
                                               const int q = sq0 + h;
                                               sm.xh[buf][sj][q][sb ^ swz(sj, q)] = hv;
                                               sm.xl[buf][sj][q][sb ^ swz(sj, q)] = lv;
                                           });
            if (lane == 0)
                sm.exact[buf][wave] = eb;
            if (!stager)
                return;
            if (exact) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    *reinterpret_cast<float4_t *>(&sm.xf[buf][sj][sb][16 * (sc_ & 1) + 4 * i]) = xr[i];
            }
            if ((sc_ & 1) == 0)
                sm.sx[buf][sj][sb] = sx;
            if (sc_ == 0)
                sm.inv[buf][sb] = inv;
        };

        // PRE: record s of this entry into LDS buffer buf, 1 KiB per copy,
        // the copies dealt to the waves in turn
        const uint32_t lds_rec = (uint32_t)(size_t)(const __attribute__((address_space(3))) void *)&sm;
        auto issue_rec = [&](int s, int buf) {
            const uint8_t *src = ws + (size_t)(recbase + s) * (size_t)rbytes; // wave-uniform
            const uint32_t dst = lds_rec + (uint32_t)(buf * kRecMax);
            for (int c = wave; c < (rbytes >> 10); c += 4)
                load_lds16(src + 1024 * c, 16u * (uint32_t)lane, dst + 1024u * (uint32_t)c);
        };
        auto recp = [&](int buf) { return reinterpret_cast<const uint8_t *>(&sm) + buf * kRecMax; };
        const int bcol = min(col, B - 1); // rows past B read row B - 1 (outputs discarded)

        float4_t acc[TW], macc[TW];
#pragma unroll
        for (int t = 0; t < TW; ++t) {
            acc[t] = float4_t{0.f, 0.f, 0.f, 0.f};
            macc[t] = float4_t{0.f, 0.f, 0.f, 0.f};
        }

        // one super-block from LDS buffer buf and packed weights wt.  Matrix-
        // core step (p, hh) takes, in quarter q, positions 8p .. 8p+7 of
        // sub-block 2q + hh (the lane's quant group q: low nibbles for hh = 0,
        // high for hh = 1) against activation chunk (2q + hh, p); the k order
        // is permuted alike for both operands, and a lane needs the 6-bit
        // scales of two sub-blocks only
        auto compute = [&](int buf, const WTile(&wt)[TW], int s) {
            // the 6-bit scale of each sub-block is folded into the quant
            // operand: sc*q <= 945 < 1024 is the binary16 subnormal
            // (sc*q)*2^-24 exactly, so one accumulator per tile runs over all
            // eight sub-blocks and d*2^24 is applied once per super-block
            float4_t dacc[TW];
            float mb[TW][2]; // dmin*m_j for j = quarter and 4 + quarter, per tile
            float d24[TW];
            uint32_t scp[TW][2]; // sc of sub-blocks 2q, 2q+1 in both 16-bit halves
            // sub-blocks 2q and 2q + 1: bytes 2(q & 1) and 2(q & 1) + 1 of the
            // packed scale word of sub-blocks 0-3 (q < 2) or 4-7
            const uint32_t bsel = 2u * (uint32_t)(quarter & 1);
#pragma unroll
            for (int t = 0; t < TW; ++t) {
                dacc[t] = float4_t{0.f, 0.f, 0.f, 0.f};
                const uint4 h = wt[t].h;
                const float dmin = half_to_float(h.x >> 16);
                d24[t] = half_to_float(h.x) * 16777216.f;
                const uint32_t sc03 = h.y & 0x3F3F3F3Fu;
                const uint32_t sc47 = (h.w & 0x0F0F0F0Fu) | ((h.y >> 2) & 0x30303030u);
                const uint32_t m03 = h.z & 0x3F3F3F3Fu;
                const uint32_t m47 = ((h.w >> 4) & 0x0F0F0F0Fu) | ((h.z >> 2) & 0x30303030u);
                const uint32_t scw = quarter < 2 ? sc03 : sc47;
                scp[t][0] = __builtin_amdgcn_perm(0u, scw, 0x0C000C00u | (bsel << 16) | bsel);
                scp[t][1] = __builtin_amdgcn_perm(0u, scw, 0x0C000C00u | ((bsel + 1) << 16) | (bsel + 1));
                mb[t][0] = dmin * (float)__builtin_amdgcn_ubfe(m03, 8 * quarter, 8);
                mb[t][1] = dmin * (float)__builtin_amdgcn_ubfe(m47, 8 * quarter, 8);
            }
#pragma unroll
            for (int pp = 0; pp < 4; ++pp) {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int j = 2 * quarter + hh;
                    uint4 xh, xl;
                    if constexpr (PRE) {
                        const uint8_t *r = recp(buf) + kRecHi + ((j * 4 + pp) * B + bcol) * 16;
                        xh = *reinterpret_cast<const uint4 *>(r);
                        xl = *reinterpret_cast<const uint4 *>(r + 512 * B);
                    } else {
                        xh = sm.xh[buf][j][pp][col ^ swz(j, pp)];
                        xl = sm.xl[buf][j][pp][col ^ swz(j, pp)];
                    }
                    const half8_t ah = __builtin_bit_cast(half8_t, xh);
                    const half8_t al = __builtin_bit_cast(half8_t, xl);
#pragma unroll
                    for (int t = 0; t < TW; ++t) {
                        // positions 8pp .. 8pp+7 of the group: low nibbles
                        // (hh = 0) or high nibbles (hh = 1) as 16-bit lanes
                        // (k0,k2), (k1,k3), (k4,k6), (k5,k7), times sc
                        const uint4 &qv = pp < 2 ? wt[t].qa : wt[t].qb;
                        const uint32_t W0 = (pp & 1) ? qv.z : qv.x, W1 = (pp & 1) ? qv.w : qv.y;
                        const uint32_t D0 = hh ? W0 >> 4 : W0;
                        const uint32_t D1 = hh ? W1 >> 4 : W1;
                        const uint32_t mk = 0x000F000Fu;
                        const u16x2 sv = __builtin_bit_cast(u16x2, scp[t][hh]);
                        auto scq = [&](uint32_t v) {
                            return __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, v & mk) * sv);
                        };
                        const uint4 qv2 = make_uint4(scq(D0), scq(D0 >> 8), scq(D1), scq(D1 >> 8));
                        const half8_t bq = __builtin_bit_cast(half8_t, qv2);
                        dacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bq, dacc[t], 0, 0, 0);
                        dacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bq, dacc[t], 0, 0, 0);
                    }
                }
                // bound the live ranges: one position group's operands at a time
                __builtin_amdgcn_sched_barrier(0);
            }
            // sub-blocks computed exactly (rare; the condition is the same for
            // the whole workgroup)
            uint64_t ex4[4];
#pragma unroll
            for (int wv = 0; wv < 4; ++wv) {
                const uint64_t v = PRE ? reinterpret_cast<const uint64_t *>(recp(buf))[wv]
                                       : sm.exact[buf][wv];
                ex4[wv] = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32)) << 32) |
                          __builtin_amdgcn_readfirstlane((uint32_t)v);
            }
            if ((ex4[0] | ex4[1] | ex4[2] | ex4[3]) != 0) {
#pragma unroll 1
                for (int wv = 0; wv < 4; ++wv) {
                    uint64_t bits = ex4[wv];
                    while (bits) {
                        const int bit = __builtin_ctzll(bits);
                        bits &= bits - 1;
                        const int b = 4 * wv + (bit >> 4), j = (bit & 15) >> 1;
                        // the lanes of quarter j >> 1 hold the 32 quants of
                        // sub-block j of their row (bytes 0-31 of the group,
                        // low nibbles for even j, high for odd)
                        const float *xs = PRE ? E.x + (size_t)b * K + 256 * s + 32 * j
                                              : &sm.xf[buf][j][b][0];
#pragma unroll
                        for (int t = 0; t < TW; ++t) {
                            float part = 0.f;
                            if (quarter == (j >> 1)) {
                                const uint4 h = wt[t].h;
                                uint32_t sc, m;
                                q4k_scale_min(h.y, h.z, h.w, j, sc, m);
                                const float dsc = half_to_float(h.x) * (float)sc;
                                const float dmm = half_to_float(h.x >> 16) * (float)m;
                                const uint32_t qw[8] = {wt[t].qa.x, wt[t].qa.y, wt[t].qa.z, wt[t].qa.w,
                                                        wt[t].qb.x, wt[t].qb.y, wt[t].qb.z, wt[t].qb.w};
                                const int sh = 4 * (j & 1);
#pragma unroll
                                for (int i = 0; i < 32; ++i) {
                                    const uint32_t q = (qw[i >> 2] >> (8 * (i & 3) + sh)) & 15u;
                                    part = fmaf(fmaf(dsc, (float)q, -dmm), xs[i], part);
                                }
                            }
                            // from the lane of weight row col in quarter j >> 1
                            part = __shfl(part, col + 16 * (j >> 1), 64);
                            if (quarter == (b >> 2)) {
                                const int i = b & 3;
                                acc[t][0] += i == 0 ? part : 0.f;
                                acc[t][1] += i == 1 ? part : 0.f;
                                acc[t][2] += i == 2 ? part : 0.f;
                                acc[t][3] += i == 3 ? part : 0.f;
                            }
                        }
                    }
                }
            }
            float4_t iv;
            float sx0, sx1;
            if constexpr (PRE) {
                iv = *reinterpret_cast<const float4_t *>(recp(buf) + kRecInv + 16 * quarter);
                const float *sxr = reinterpret_cast<const float *>(recp(buf) + kRecSx);
                sx0 = sxr[16 * quarter + col];
                sx1 = sxr[16 * (4 + quarter) + col];
            } else {
                iv = *reinterpret_cast<const float4_t *>(&sm.inv[buf][4 * quarter]);
                sx0 = sm.sx[buf][quarter][col];
                sx1 = sm.sx[buf][4 + quarter][col];
            }
#pragma unroll
            for (int t = 0; t < TW; ++t) {
                acc[t] = (d24[t] * iv) * dacc[t] + acc[t];
                macc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(sx0, mb[t][0], macc[t], 0, 0, 0);
                macc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(sx1, mb[t][1], macc[t], 0, 0, 0);
            }
        };

        WTile wa[TW], wb[TW];
        if constexpr (PRE && NS == 3) {
            // records in a ring of three; the wait that ends a step retires
            // the copies and the weights of s+1 and leaves the weights of
            // s+2 in flight (the compiler, counting only weight loads, sees
            // the same)
            WTile wc[TW];
            issue_rec(0, 0);
            load_w(0, wa);
            load_w(min(1, nsb - 1), wb);
            __builtin_amdgcn_s_waitcnt(0); // everything, the previous block's stores included
            __builtin_amdgcn_s_barrier();
            auto step3 = [&](int s, int S, const WTile(&cur)[TW], WTile(&far)[TW]) -> bool {
                issue_rec(min(s + 1, nsb - 1), S == 2 ? 0 : S + 1);
                load_w(min(s + 2, nsb - 1), far);
                compute(S, cur, s);
                __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(3 * TW));
                __builtin_amdgcn_s_barrier();
                return s + 1 < nsb;
            };
            for (int s = 0;; s += 3) {
                if (!step3(s, 0, wa, wc))
                    break;
                if (!step3(s + 1, 1, wb, wa))
                    break;
                if (!step3(s + 2, 2, wc, wb))
                    break;
            }
        } else if constexpr (NS == 3) {
            WTile wc[TW];
            load_x(0);
            load_w(0, wa);
            load_w(min(1, nsb - 1), wb);
            store_x(0);
            __syncthreads();
            auto step3 = [&](int s, const WTile(&cur)[TW], WTile(&far)[TW]) -> bool {
                const int buf = s & 1;
                load_x(min(s + 1, nsb - 1));
                load_w(min(s + 2, nsb - 1), far);
                compute(buf, cur, s);
                store_x(buf ^ 1);
                __builtin_amdgcn_s_waitcnt(0xC07F); // lgkmcnt(0): this wave's LDS writes
                __builtin_amdgcn_s_barrier();
                return s + 1 < nsb;
            };
            for (int s = 0;; s += 3) {
                if (!step3(s, wa, wc))
                    break;
                if (!step3(s + 1, wb, wa))
                    break;
                if (!step3(s + 2, wc, wb))
                    break;
            }
        } else if constexpr (PRE) {
            // the copies of record s+1 and the weights of s+2 are issued
            // while s is computed; the wait that ends a step retires the
            // copies and the previous step's weights (loads complete in issue
            // order) and leaves this step's 3 TW weight loads in flight; the
            // compiler, which counts only the weight loads, sees the same
            issue_rec(0, 0);
            load_w(0, wa);
            load_w(min(1, nsb - 1), wb);
            __builtin_amdgcn_s_waitcnt(0); // everything, the previous block's stores included
            __builtin_amdgcn_s_barrier();
            for (int s = 0; s < nsb; s += 2) {
                issue_rec(min(s + 1, nsb - 1), 1);
                compute(0, wa, s);
                load_w(min(s + 2, nsb - 1), wa);
                __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(3 * TW));
                __builtin_amdgcn_s_barrier();
                if (s + 1 >= nsb)
                    break;
                issue_rec(min(s + 2, nsb - 1), 0);
                compute(1, wb, s + 1);
                load_w(min(s + 3, nsb - 1), wb);
                __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(3 * TW));
                __builtin_amdgcn_s_barrier();
            }
        } else {
            load_x(0);
            load_w(0, wa);
            load_w(min(1, nsb - 1), wb);
            store_x(0);
            __syncthreads();
            // two super-blocks per iteration so that the register sets stay
            // fixed; prefetches past the end reload the last super-block
            // (unused)
            for (int s = 0; s < nsb; s += 2) {
                load_x(min(s + 1, nsb - 1));
                compute(0, wa, s);
                load_w(min(s + 2, nsb - 1), wa);
                store_x(1);
                __builtin_amdgcn_s_waitcnt(0xC07F); // lgkmcnt(0): this wave's LDS writes
                __builtin_amdgcn_s_barrier();
                if (s + 1 >= nsb)
                    break;
                load_x(min(s + 2, nsb - 1));
                compute(1, wb, s + 1);
                load_w(min(s + 3, nsb - 1), wb);
                store_x(0);
                __builtin_amdgcn_s_waitcnt(0xC07F);
                __builtin_amdgcn_s_barrier();
            }
        }

        // y[b][row] for b = 4*quarter + i (PAIR: h[b][row] = silu(g) * u)
        if constexpr (PAIR) {
            if (rows[0] < M) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int b = 4 * quarter + i;
                    if (b < B)
                        E.y[(size_t)b * M + rows[0]] =
                            silu(acc[0][i] - macc[0][i]) * (acc[1][i] - macc[1][i]);
                }
            }
        } else {
#pragma unroll
            for (int t = 0; t < TW; ++t) {
                if (rows[t] < M) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int b = 4 * quarter + i;
                        if (b < B)
                            E.y[(size_t)b * M + rows[t]] = acc[t][i] - macc[t][i];
                    }
                }
            }
        }
        row0 += RBO;
    }
}

// prefix[e] = sum over entries e' < e of K/256 (records before entry e),
// prefix[n] = all records; one workgroup.
__global__ __launch_bounds__(1024) void gemv_prefix_kernel(const GemvEntry *__restrict__ table,
                                                          int n, int *__restrict__ prefix)
{
    __shared__ int part[16];
    __shared__ int carry;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0)
        carry = 0;
    __syncthreads();
    for (int base = 0; base < n; base += 1024) {
        const int e = base + tid;
        const int v = e < n ? table[e].K >> 8 : 0;
        int inc = v;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int u = __shfl_up(inc, off, 64);
            if (lane >= off)
                inc += u;
        }
        if (lane == 63)
            part[wave] = inc;
        __syncthreads();
        int before = carry;
        for (int w = 0; w < wave; ++w)
            before += part[w];
        if (e < n)
            prefix[e] = before + inc - v;
        __syncthreads();
        if (tid == 1023)
            carry = before + inc;
        __syncthreads();
    }
    if (tid == 0)
        prefix[n] = carry;
}

// One record of pre-staged activations per workgroup: record r belongs to the
// entry e with prefix[e] <= r < prefix[e + 1], super-block r - prefix[e]; the
// 16 lanes of activation row sb = 4*wave + lane/16 stage it as the blocks of
// the main kernel do.
__global__ __launch_bounds__(NT) void gemv_stage_kernel(const GemvEntry *__restrict__ table, int n,
                                                       const int *__restrict__ prefix, int B,
                                                       uint8_t *__restrict__ recs, int rbytes)
{
    const int r = blockIdx.x;
    int a = 0, z = n - 1;
    while (a < z) { // last entry whose first record is at or before r
        const int mid = (a + z + 1) >> 1;
        if (prefix[mid] <= r)
            a = mid;
        else
            z = mid - 1;
    }
    const GemvEntry E = table[a];
    const int s = r - prefix[a];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int sb = 4 * wave + (lane >> 4), sc_ = lane & 15;
    const int sj = sc_ >> 1, sq0 = 2 * (sc_ & 1);
    const bool stager = sb < B;
    float4_t xr[4];
    if (stager) {
        const float *xp = E.x + (size_t)sb * E.K + 256 * s + 16 * sc_;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            xr[i] = *reinterpret_cast<const float4_t *>(xp + 4 * i);
    }
    uint8_t *rec = recs + (size_t)r * (size_t)rbytes;
    uint64_t eb;
    float sx, inv;
    stage_slice(xr, stager, lane, eb, sx, inv, [&](int h, const uint4 &hv, const uint4 &lv) {
        uint8_t *d = rec + kRecHi + ((sj * 4 + sq0 + h) * B + sb) * 16;
        *reinterpret_cast<uint4 *>(d) = hv;
        *reinterpret_cast<uint4 *>(d + 512 * B) = lv;
    });
    if (lane == 0)
        reinterpret_cast<uint64_t *>(rec)[wave] = eb;
    if (!stager)
        return;
    if ((sc_ & 1) == 0)
        reinterpret_cast<float *>(rec + kRecSx)[16 * sj + sb] = sx;
    if (sc_ == 0)
        reinterpret_cast<float *>(rec + kRecInv)[sb] = inv;
}

long long gemv_mfma_prestaged_bytes(int64_t n, long long records, int B)
{
    return (long long)gemv_prestaged_records_offset(n) + records * (long long)rec_bytes(B);
}

hipError_t launch_gemv_mfma_prestaged(const GemvEntry *table_dev, int n, long long total_bytes,
                                      long long blocks1, long long blocks2, long long blocks3,
                                      long long records, int B, void *ws, hipStream_t s)
{
    int *prefix = static_cast<int *>(ws);
    uint8_t *recs = static_cast<uint8_t *>(ws) + gemv_prestaged_records_offset(n);
    const int rb = rec_bytes(B);
    hipLaunchKernelGGL(gemv_prefix_kernel, dim3(1), dim3(1024), 0, s, table_dev, n, prefix);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    hipLaunchKernelGGL(gemv_stage_kernel, dim3((unsigned)records), dim3(NT), 0, s, table_dev, n,
                       (const int *)prefix, B, recs, rb);
    err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    // 128-row blocks with three weight sets: the records are staged once per
    // product, so larger blocks save nothing, and the third set keeps more
    // weight loads in flight (decode stack at batch 4 1155 -> 1108 us, at
    // batch 16 1375 -> 1313 us, against 192-row blocks with two sets)
    (void)blocks3;
    const int cus = device_cus();
    const GemvEntry none{};
    if (blocks2 < cus) {
        // too few 128-row blocks for one workgroup per CU: 64-row blocks
        const long long grid = blocks1 < 2LL * cus ? blocks1 : 2LL * cus;
        hipLaunchKernelGGL((gemv_q4k_mfma_kernel<false, 1, true, 3>), dim3((unsigned)grid),
                           dim3(NT), 0, s, table_dev, none, n, total_bytes, B,
                           (const uint8_t *)nullptr, (const uint8_t *)recs, (const int *)prefix,
                           rb);
        return hipGetLastError();
    }
    const long long grid = blocks2 < 2LL * cus ? blocks2 : 2LL * cus;
    hipLaunchKernelGGL((gemv_q4k_mfma_kernel<false, 2, true, 3>), dim3((unsigned)grid), dim3(NT),
                       0, s, table_dev, none, n, total_bytes, B, (const uint8_t *)nullptr,
                       (const uint8_t *)recs, (const int *)prefix, rb);
    return hipGetLastError();
}

long long gemv_mfma_blocks(int64_t M, int tiles)
{
    const int rb = rows_per_block(tiles);
    return (M + rb - 1) / rb;
}

hipError_t launch_gemv_mfma(const GemvEntry *table_dev, const GemvEntry &inline0, int n,
                            long long total_bytes, long long blocks1, long long blocks2,
                            long long blocks3, int B, hipStream_t s)
{
    // three tiles per wave (192-row blocks: each block's activation staging
    // serves 1.5 times the weights; decode stack at batch 4 1273 -> 1196 us)
    // when they still give every workgroup of the grid a block, else two
    const int cus = device_cus();
    if (blocks3 >= 2LL * cus) {
        hipLaunchKernelGGL((gemv_q4k_mfma_kernel<false, 3>), dim3((unsigned)(2 * cus)), dim3(NT), 0,
                           s, table_dev, inline0, n, total_bytes, B, (const uint8_t *)nullptr,
                           (const uint8_t *)nullptr, (const int *)nullptr, 0);
    } else if (blocks2 < cus) {
        // too few 128-row blocks for one workgroup per CU (single products up
        // to 32768 rows): 64-row blocks, one 16-row tile per wave, twice the
        // workgroups (measured rotating over 1 GB: 14336 x 4096 at batch 4
        // 35.8 -> 29.2 us, 4096 x 14336 108 -> 86 us, 4096 x 4096 35.5 ->
        // 28.5 us); three weight sets up to batch 8, two above
        const long long grid = blocks1 < 2LL * cus ? blocks1 : 2LL * cus;
        if (B <= 8)
            hipLaunchKernelGGL((gemv_q4k_mfma_kernel<false, 1, false, 3>), dim3((unsigned)grid),
                               dim3(NT), 0, s, table_dev, inline0, n, total_bytes, B,
                               (const uint8_t *)nullptr, (const uint8_t *)nullptr,
                               (const int *)nullptr, 0);
        else
            hipLaunchKernelGGL((gemv_q4k_mfma_kernel<false, 1, false, 2>), dim3((unsigned)grid),
                               dim3(NT), 0, s, table_dev, inline0, n, total_bytes, B,
                               (const uint8_t *)nullptr, (const uint8_t *)nullptr,
                               (const int *)nullptr, 0);
    } else {
        const long long grid = blocks2 < 2LL * cus ? blocks2 : 2LL * cus;
        hipLaunchKernelGGL((gemv_q4k_mfma_kernel<false, 2, false, 3>), dim3((unsigned)grid),
                           dim3(NT), 0, s, table_dev, inline0, n, total_bytes, B,
                           (const uint8_t *)nullptr, (const uint8_t *)nullptr, (const int *)nullptr,
                           0);
    }
    return hipGetLastError();
}

hipError_t launch_gemv_swiglu_mfma(const void *w_gate, const void *w_up, const float *x, float *h,
                                   int64_t M, int64_t K, int B, hipStream_t s)
{
    const GemvEntry e{(const uint8_t *)w_gate, x, h, (int)M, (int)K, 0, 0};
    const long long total = 2LL * M * (K / 256) * kQ4kBytes;
    const long long blocks = (M + 63) / 64;
    const int cus = device_cus();
    const long long grid = blocks < 2LL * cus ? blocks : 2LL * cus;
    hipLaunchKernelGGL((gemv_q4k_mfma_kernel<true, 2, false, 3>), dim3((unsigned)grid), dim3(NT),
                       0, s, nullptr, e, 1, total, B, (const uint8_t *)w_up,
                       (const uint8_t *)nullptr, (const int *)nullptr, 0);
    return hipGetLastError();
}

} // namespace gq
