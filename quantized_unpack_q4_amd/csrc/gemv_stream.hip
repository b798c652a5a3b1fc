// gemv_stream.hip -- batch-1 Q4_K matrix-vector products streamed by a
// persistent grid, for one matrix or for a whole table of independent
// matrices (a decode step) in a single launch.
//
// Decode is memory-bound: every packed weight byte is read once and the
// dequantization is fused into the dot product (page "Building a Rust
// Inference Engine That Matches Llama.cpp", section "Where the wins came
// from").  A launch per matrix costs a fixed ramp-up and drain that, summed
// over a 224-matrix step, is as large as the streaming itself; the pages fight
// the same per-matmul overhead with fewer GPU submissions (page "Frink
// Inference: the Rust alternative to llama.cpp", section "The engine":
// command-buffer waits per token cut from 192 to 20, one submission per group
// of layers).  Here the whole table is one launch: the total weight bytes are
// split into equal contiguous byte ranges, one per workgroup, and a workgroup
// processes every row whose first byte lies inside its range (so every
// workgroup streams the same bytes to within one row).
//
// Lanes per row.  A weight row is covered by 32 lanes (16 super-blocks per
// step) or, when K/256 is a multiple of 8 but not of 16 (K = 14336), by 16
// lanes (8 super-blocks per step), so that no step of a row is half empty.
//
// Arithmetic per lane.  Two lanes share a 256-weight super-block: lane p
// (0 or 1) owns quant groups p and p + 2, i.e. sub-blocks 2p, 2p+1, 2p+4 and
// 2p+5, whose scales come from the same three scale bytes per pair (j, j+4).
// Quants are used as binary16 subnormals (the nibble bits themselves,
// q * 2^-24, or 16q * 2^-24 for high nibbles), so one v_dot2_f32_f16
// multiplies two quants by two activation halves exactly and accumulates in
// binary32.  Per sub-block j the contribution is
// (d*sc_j) * sum(q*x) - (dmin*m_j) * sum(x).  With a one-hot x the result is
// the binary32 weight exactly (d*sc*q exact, one rounding with -dmin*m).
//
// Activations.  Each 32-value sub-block j of x is staged in LDS once per
// matrix as binary16 pairs hi + lo of x * 2^s_j, where 2^s_j brings the
// sub-block's largest |x| into [2^14, 2^15); every value at least 2^-17 of
// that maximum then keeps 22 significant bits (lo stays a normal binary16),
// and every value at least 2^-20 of it a relative error below 2^-19.  The
// sub-block's result is brought to the vector's own scale (its largest |x| in
// [2^14, 2^15)) by an exact power of two, and the row's sum is scaled back
// once at the end, so no intermediate overflows or underflows whatever the
// vector's magnitude.  Two kinds of sub-block skip the split and are computed
// exactly in binary32 instead, each weight dequantized to its binary32 value
// (d*sc*q - dmin*m, one rounding) times the binary32 activation staged in LDS:
// a sub-block whose non-zero |x| span more than 2^20 (the split would lose
// the small ones), and a sub-block holding more than 1/16 of the sum of |x|
// over its super-block (a single dominant activation would otherwise meet a
// near-cancelling d*sc*q - dmin*m through the factored form, whose error
// scales with the two terms rather than with their difference).  Neither
// occurs in practice in standard-normal vectors; both keep spikes, one-hot
// and sparse vectors and wide ranges within the bound.
//
// Pipelining: each wave issues the global loads of its next step before
// computing the current one; the loads are unconditional (out-of-range rows
// and super-blocks read a clamped in-range address and get a zero header), so
// the compiler can wait for exactly the older loads.
#include "gq_device.h"
#include "gq_internal.h"

namespace gq {

namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4 g_u32x4;
typedef __attribute__((address_space(1))) const f32x4 g_f32x4;

__device__ __forceinline__ uint4 gload16(const void *p)
{
    const u32x4 v = *(g_u32x4 *)(p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float4 gloadf4(const float *p)
{
    const f32x4 v = *(g_f32x4 *)(p);
    return make_float4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, a), __builtin_bit_cast(h2_t, b), c,
                                  false);
}

// Sum over each row of 16 lanes (xor 1, xor 2, rotate 4, rotate 8); every lane
// of the row ends with the row's sum.
__device__ __forceinline__ float rowsum16(float v)
{
#define GQ_DPP(x, ctrl)                                                                          \
    __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), ctrl, \
                                                          0xF, 0xF, true))
    v += GQ_DPP(v, 0xB1);  // quad_perm [1,0,3,2]
    v += GQ_DPP(v, 0x4E);  // quad_perm [2,3,0,1]
    v += GQ_DPP(v, 0x124); // row_ror:4
    v += GQ_DPP(v, 0x128); // row_ror:8
#undef GQ_DPP
    return v;
}

__device__ __forceinline__ float lane_value(float v, int lane)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

constexpr int kStreamMaxK = GemvStreamMaxK;
constexpr int kRecs = kStreamMaxK / 4;                      // 16-byte x records
constexpr int kLdsWords = (kRecs + kRecs / 16) * 4 + 2 * (kStreamMaxK / 32);
// binary32 activations (in the vector's scale) of up to kExactSlots sub-blocks
// computed exactly, so that the exact path reads LDS; further ones (vectors
// with a wide range everywhere) read global memory.  kLdsWords + the slots
// stay within 80 KB, two workgroups per CU.
constexpr int kExactSlots = 56;
// a sub-block whose non-zero |x| span more than this is computed exactly
constexpr float kSplitSpan = 1048576.f; // 2^20
// ... and one holding more than this fraction of its super-block's sum of |x|
constexpr float kDominant = 0.0625f;
constexpr int kR = 3;          // row groups per wave step (a group is 2 or 4 rows)
constexpr int kTileRowsMin = 24; // rows per workgroup tile with 32 lanes per row

struct Frag {
    uint4 hd, a0, a1, b0, b1; // header, quant group p (32 B), quant group p+2 (32 B)
    bool ok;
};

__device__ __forceinline__ uint32_t word8(const uint4 &a, const uint4 &b, int i)
{
    return i == 0 ? a.x : i == 1 ? a.y : i == 2 ? a.z : i == 3 ? a.w
         : i == 4 ? b.x : i == 5 ? b.y : i == 6 ? b.z : b.w;
}

} // namespace

// R row groups per wave step, NB weight-load buffers (loads run NB - 1 steps
// ahead of the arithmetic), W waves per workgroup.
// PAIR: one entry whose rows are the pairs (gate row r, up row r) of two
// matrices with the same shape, e.w and w2; the row-group layout puts both
// rows of a pair in one wave, so h[r] = silu(gate_r x) * (up_r x) is formed in
// registers and e.y receives h (M values).  Ranges split at pair granularity.
template <int R, int NB, int W, bool PAIR = false>
__global__ __launch_bounds__(64 * W, 8 / W) void gemv_q4k_stream_kernel(
    const GemvEntry *__restrict__ table, GemvEntry inline0, int n, long long total,
    const uint8_t *__restrict__ w2)
{
    constexpr int kR = R;
    constexpr int kThreads = 64 * W;
    constexpr int kSubPerThread = (kStreamMaxK / 32 + kThreads - 1) / kThreads;
    __shared__ __attribute__((aligned(16))) uint32_t lds[kLdsWords];
    __shared__ __attribute__((aligned(16))) float xex[kExactSlots][32];
    __shared__ int s_nexact;
    uint32_t *xrec = lds;
    float2 *srec = reinterpret_cast<float2 *>(lds + (kRecs + kRecs / 16) * 4);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int p = lane & 1;
    const long long lo = total * (long long)blockIdx.x / gridDim.x;
    const long long hi = total * (long long)(blockIdx.x + 1) / gridDim.x;

    auto entry = [&](int i) -> GemvEntry { return table ? table[i] : inline0; };
    // the last entry whose work begins at or before lo (work_begin increases
    // along the table; entry 0 begins at 0): a kThreads-way search, each
    // thread testing one slot per level, one round trip per level (a single
    // level up to kThreads entries).  Walking the table one dependent load at
    // a time took the workgroups at its end ~57 us on the 224-entry decode
    // stack, and they set the launch's end.
    int di = 0;
    for (int span = n; span > 1;) {
        const int step = (span + kThreads - 1) / kThreads;
        const bool le = tid * step < span && entry(di + tid * step).work_begin <= lo;
        const int cnt = __syncthreads_count(le);
        di += (cnt - 1) * step;
        span = min(step, span - (cnt - 1) * step);
    }
    GemvEntry e = entry(di);

    int nsb = e.K >> 8, r_end = 0, rpg = 2, sps = 16, rsub = 0, sbl = 0;
    long long rowb = (long long)nsb * kQ4kBytes;

    // Activation staging (see the header): records of hi/lo binary16 pairs,
    // and per sub-block j the pair srec[j] = (sum of x over j, factor f_j) in
    // the vector's scale; f_j = 2^(e_j - e) takes sub-block j's products to
    // the vector's scale (times 2^-4 for odd j: high nibbles enter as 16q),
    // 0 for an all-zero sub-block, -1 for one computed exactly.
    __shared__ float s_amax[W];
    int vexp = 0; // the vector's scale is 2^(15 - vexp): max|x| < 2^vexp
    auto stage = [&]() {
        // thread t owns sub-blocks t, t + kThreads, ... (32 activations each,
        // at most 512 sub-blocks): every activation is loaded once, all loads
        // in flight together, and kept in registers for the scale, split and
        // sums.  The 8 sub-blocks of a super-block belong to 8 consecutive
        // lanes of one wave.
        const int nsub = e.K >> 5;
        float4 v[kSubPerThread][8];
        float amax = 0.f;
#pragma unroll
        for (int u = 0; u < kSubPerThread; ++u) {
            const int j = tid + kThreads * u;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                v[u][i] = j < nsub ? gloadf4(e.x + 32 * j + 4 * i) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[u][i].x), fabsf(v[u][i].y)),
                                         fmaxf(fabsf(v[u][i].z), fabsf(v[u][i].w))));
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1)
            amax = fmaxf(amax, __shfl_xor(amax, off, 64));
        if (lane == 0)
            s_amax[wave] = amax;
        if (tid == 0)
            s_nexact = 0;
        __syncthreads();
        amax = s_amax[0];
#pragma unroll
        for (int i = 1; i < W; ++i)
            amax = fmaxf(amax, s_amax[i]);
        vexp = 0;
        if (amax > 0.f)
            (void)frexpf(amax, &vexp); // amax < 2^vexp
        // record i holds x[4i..4i+3]*2^s_j as (hi(x0,x2), hi(x1,x3), lo(x0,x2),
        // lo(x1,x3)); 16 bytes of padding after every 16 records
#pragma unroll
        for (int u = 0; u < kSubPerThread; ++u) {
            const int j = tid + kThreads * u;
            float smax = 0.f, smin = INFINITY, l1 = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float a[4] = {fabsf(v[u][i].x), fabsf(v[u][i].y), fabsf(v[u][i].z),
                                    fabsf(v[u][i].w)};
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    smax = fmaxf(smax, a[c]);
                    smin = a[c] > 0.f ? fminf(smin, a[c]) : smin;
                    l1 += a[c];
                }
            }
            // sum of |x| over the super-block (8 consecutive lanes)
            float sl1 = l1 + __shfl_xor(l1, 1, 64);
            sl1 += __shfl_xor(sl1, 2, 64);
            sl1 += __shfl_xor(sl1, 4, 64);
            if (j >= nsub)
                continue;
            const bool exact = smax > 0.f && (smax > kSplitSpan * smin || smax > kDominant * sl1);
            int ej = 0;
            if (smax > 0.f)
                (void)frexpf(smax, &ej);
            const int sh = 15 - ej;
            const bool split = smax > 0.f && !exact;
            float sum = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float4 w = v[u][i];
                w.x = split ? ldexpf(w.x, sh) : 0.f;
                w.y = split ? ldexpf(w.y, sh) : 0.f;
                w.z = split ? ldexpf(w.z, sh) : 0.f;
                w.w = split ? ldexpf(w.w, sh) : 0.f;
                sum += (w.x + w.y) + (w.z + w.w);
                const h2_t h02 = {(_Float16)w.x, (_Float16)w.z};
                const h2_t h13 = {(_Float16)w.y, (_Float16)w.w};
                const h2_t l02 = {(_Float16)(w.x - (float)h02.x), (_Float16)(w.z - (float)h02.y)};
                const h2_t l13 = {(_Float16)(w.y - (float)h13.x), (_Float16)(w.w - (float)h13.y)};
                const int ri = 8 * j + i;
                *reinterpret_cast<uint4 *>(xrec + 4 * (ri + (ri >> 4))) = make_uint4(
                    __builtin_bit_cast(uint32_t, h02), __builtin_bit_cast(uint32_t, h13),
                    __builtin_bit_cast(uint32_t, l02), __builtin_bit_cast(uint32_t, l13));
            }
            // exact: slot for its binary32 values, factor -(1 + slot)
            int slot = kExactSlots;
            if (exact) {
                slot = min(atomicAdd(&s_nexact, 1), kExactSlots);
                if (slot < kExactSlots) {
                    const int xs = 15 - vexp;
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        *reinterpret_cast<float4 *>(&xex[slot][4 * i]) =
                            make_float4(ldexpf(v[u][i].x, xs), ldexpf(v[u][i].y, xs),
                                        ldexpf(v[u][i].z, xs), ldexpf(v[u][i].w, xs));
                }
            }
            // 2^(e_j - vexp) <= 1, and 2^-4 more for the high-nibble sub-blocks
            const float f = ldexpf(1.f, ej - vexp - 4 * (j & 1));
            srec[j] = split ? make_float2(sum * ldexpf(1.f, ej - vexp), f)
                            : make_float2(0.f, exact ? -1.f - (float)slot : 0.f);
        }
    };

    auto issue = [&](Frag (&f)[kR], int row0, int s) {
        const int sc = s < nsb ? s : nsb - 1;
#pragma unroll
        for (int r = 0; r < kR; ++r) {
            const int row = row0 + rpg * r + rsub;
            const int rc = row < r_end ? row : r_end - 1;
            const uint8_t *base = PAIR && (rc & 1) ? w2 : e.w;
            const size_t vr = PAIR ? (size_t)(rc >> 1) : (size_t)rc;
            const uint8_t *blk = base + vr * rowb + (size_t)sc * kQ4kBytes;
            f[r].hd = gload16(blk);
            f[r].a0 = gload16(blk + 16 + 32 * p);
            f[r].a1 = gload16(blk + 32 + 32 * p);
            f[r].b0 = gload16(blk + 80 + 32 * p);
            f[r].b1 = gload16(blk + 96 + 32 * p);
            f[r].ok = s < nsb && row < r_end;
        }
    };

    // A workgroup owns every row whose first byte lies in [lo, hi): rows of
    // one matrix are split between workgroups at row granularity, so every
    // workgroup streams the same bytes to within one row.
    for (;; ++di) {
        if (di >= n)
            return;
        e = entry(di);
        if (e.work_begin >= hi)
            return;
        nsb = e.K >> 8;
        rowb = (long long)nsb * kQ4kBytes;
        const long long rel_lo = lo - e.work_begin, rel_hi = hi - e.work_begin;
        // rows (pairs of rows) are owned whole: unit of `gr` rows
        const int gr = PAIR ? 2 : 1;
        const long long mrows = (long long)gr * e.M, unit = gr * gemv_row_work(e.K);
        const int r_lo = rel_lo <= 0 ? 0 : (int)min(mrows, gr * ((rel_lo + unit - 1) / unit));
        r_end = (int)min(mrows, gr * ((rel_hi + unit - 1) / unit));
        if (r_lo >= r_end)
            continue;
        // 32 lanes per row (16 super-blocks per step), or 16 lanes per row
        // (8 per step) when that leaves fewer idle lanes in a row's last step
        const int pad32 = ((nsb + 15) & ~15) - nsb, pad16 = ((nsb + 7) & ~7) - nsb;
        const int lsh = pad16 < pad32 ? 4 : 5;
        rpg = 64 >> lsh;
        sps = 1 << (lsh - 1);
        rsub = lane >> lsh;
        sbl = (lane & ((1 << lsh) - 1)) >> 1;
        const int wave_rows = kR * rpg, tile_rows = W * wave_rows;
        const int nchunk = (nsb + sps - 1) / sps;
        const int ntile = (r_end - r_lo + tile_rows - 1) / tile_rows;
        const int step_hi = ntile * nchunk;
        int st = 0;
        Frag A[kR], B[kR], C[kR];
        float acc[kR];
#pragma unroll
        for (int r = 0; r < kR; ++r)
            acc[r] = 0.f;
        // the matrix's first weight loads go out before its activations are
        // staged, so that the two latencies overlap; the barrier before the
        // staging waits for the previous matrix's readers of the LDS records
        auto issue_step = [&](Frag (&f)[kR], int sx) {
            const int t = sx / nchunk, c = sx - t * nchunk;
            issue(f, r_lo + t * tile_rows + wave * wave_rows, c * sps + sbl);
        };
        issue_step(A, 0);
        if (NB == 3)
            issue_step(B, min(1, step_hi - 1));
        __syncthreads();
        stage();
        __syncthreads();

        // cur holds step st; far receives step st + NB - 1 (clamped to the last)
        auto step = [&](Frag (&cur)[kR], Frag (&far)[kR]) -> bool {
            const int t = st / nchunk, c = st - t * nchunk;
            issue_step(far, min(st + NB - 1, step_hi - 1));

            const int s = min(c * sps + sbl, nsb - 1);
            const int r0 = 64 * s + 16 * p; // x record of sub-block 2p, position 0
            const int r4 = r0 + 32;         // x record of sub-block 2p+4
            float P0[kR], P1[kR], P4[kR], P5[kR];
#pragma unroll
            for (int r = 0; r < kR; ++r) {
                P0[r] = 0.f;
                P1[r] = 0.f;
                P4[r] = 0.f;
                P5[r] = 0.f;
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int ia = r0 + i, ib = r0 + 8 + i, ic = r4 + i, id = r4 + 8 + i;
                const uint4 xa = *reinterpret_cast<const uint4 *>(xrec + 4 * (ia + (ia >> 4)));
                const uint4 xb = *reinterpret_cast<const uint4 *>(xrec + 4 * (ib + (ib >> 4)));
                const uint4 xc = *reinterpret_cast<const uint4 *>(xrec + 4 * (ic + (ic >> 4)));
                const uint4 xd = *reinterpret_cast<const uint4 *>(xrec + 4 * (id + (id >> 4)));
#pragma unroll
                for (int r = 0; r < kR; ++r) {
                    const uint32_t D = word8(cur[r].a0, cur[r].a1, i);
                    const uint32_t E = word8(cur[r].b0, cur[r].b1, i);
                    const uint32_t td = D >> 8, te = E >> 8;
                    // quant pairs as binary16 subnormals: low nibbles (q0,q2),(q1,q3)
                    // and high nibbles as 16q
                    const uint32_t dl02 = D & 0x000F000Fu, dl13 = td & 0x000F000Fu;
                    const uint32_t dh02 = D & 0x00F000F0u, dh13 = td & 0x00F000F0u;
                    const uint32_t el02 = E & 0x000F000Fu, el13 = te & 0x000F000Fu;
                    const uint32_t eh02 = E & 0x00F000F0u, eh13 = te & 0x00F000F0u;
                    P0[r] = dot2(dl02, xa.x, P0[r]);
                    P0[r] = dot2(dl02, xa.z, P0[r]);
                    P0[r] = dot2(dl13, xa.y, P0[r]);
                    P0[r] = dot2(dl13, xa.w, P0[r]);
                    P1[r] = dot2(dh02, xb.x, P1[r]);
                    P1[r] = dot2(dh02, xb.z, P1[r]);
                    P1[r] = dot2(dh13, xb.y, P1[r]);
                    P1[r] = dot2(dh13, xb.w, P1[r]);
                    P4[r] = dot2(el02, xc.x, P4[r]);
                    P4[r] = dot2(el02, xc.z, P4[r]);
                    P4[r] = dot2(el13, xc.y, P4[r]);
                    P4[r] = dot2(el13, xc.w, P4[r]);
                    P5[r] = dot2(eh02, xd.x, P5[r]);
                    P5[r] = dot2(eh02, xd.z, P5[r]);
                    P5[r] = dot2(eh13, xd.y, P5[r]);
                    P5[r] = dot2(eh13, xd.w, P5[r]);
                }
            }
            // (sum, factor) of sub-blocks 2p, 2p+1 and 2p+4, 2p+5
            const float4 g01 = *reinterpret_cast<const float4 *>(srec + 8 * s + 2 * p);
            const float4 g45 = *reinterpret_cast<const float4 *>(srec + 8 * s + 2 * p + 4);
            const int o0 = 16 * p, o1 = 16 * p + 8; // bit offsets of scale bytes 2p, 2p+1
            // sub-blocks computed exactly (factor -1); rare, so a divergent branch
            const bool any_exact = fminf(fminf(g01.y, g01.w), fminf(g45.y, g45.w)) < 0.f;
            const int xsh = 15 - vexp;
            const float *xs = e.x + 256 * s;
#pragma unroll
            for (int r = 0; r < kR; ++r) {
                const uint32_t h0 = cur[r].ok ? cur[r].hd.x : 0u;
                const uint32_t h1 = cur[r].hd.y, h2 = cur[r].hd.z, h3 = cur[r].hd.w;
                // sub-blocks j in {2p, 2p+1}: whole 6-bit values in s[j], s[j+4];
                // sub-blocks j+4: low nibbles of s[j+8], top bits of s[j], s[j+4]
                const uint32_t sc0 = __builtin_amdgcn_ubfe(h1, o0, 6);
                const uint32_t m0 = __builtin_amdgcn_ubfe(h2, o0, 6);
                const uint32_t sc1 = __builtin_amdgcn_ubfe(h1, o1, 6);
                const uint32_t m1 = __builtin_amdgcn_ubfe(h2, o1, 6);
                const uint32_t sc4 =
                    __builtin_amdgcn_ubfe(h3, o0, 4) | (__builtin_amdgcn_ubfe(h1, o0 + 6, 2) << 4);
                const uint32_t m4 = __builtin_amdgcn_ubfe(h3, o0 + 4, 4) |
                                    (__builtin_amdgcn_ubfe(h2, o0 + 6, 2) << 4);
                const uint32_t sc5 =
                    __builtin_amdgcn_ubfe(h3, o1, 4) | (__builtin_amdgcn_ubfe(h1, o1 + 6, 2) << 4);
                const uint32_t m5 = __builtin_amdgcn_ubfe(h3, o1 + 4, 4) |
                                    (__builtin_amdgcn_ubfe(h2, o1 + 6, 2) << 4);
                // quants entered as q*2^-24 (low) and q*2^-20 (high): fold 2^24 into d
                const float d = half_to_float(h0);
                const float d24 = d * 16777216.f;
                const float dmin = half_to_float(h0 >> 16);
                float t1 = ((float)sc0 * g01.y) * P0[r];
                t1 = fmaf((float)sc1 * g01.w, P1[r], t1);
                t1 = fmaf((float)sc4 * g45.y, P4[r], t1);
                t1 = fmaf((float)sc5 * g45.w, P5[r], t1);
                float t2 = (float)m0 * g01.x;
                t2 = fmaf((float)m1, g01.z, t2);
                t2 = fmaf((float)m4, g45.x, t2);
                t2 = fmaf((float)m5, g45.z, t2);
                acc[r] = fmaf(-dmin, t2, fmaf(d24, t1, acc[r]));
            }
            if (any_exact) {
                // the sub-blocks marked exact (their split records are zero):
                // each weight as its binary32 value times x in the vector's
                // scale, x loaded once for the kR row groups
#pragma unroll 1
                for (int jj = 0; jj < 4; ++jj) {
                    const float fj = jj == 0 ? g01.y : jj == 1 ? g01.w : jj == 2 ? g45.y : g45.w;
                    if (!(fj < 0.f))
                        continue;
                    const int j = 2 * p + (jj & 1) + 4 * (jj >> 1), shift = 4 * (jj & 1);
                    float dsc[kR], dmm[kR], s0[kR], s1[kR];
#pragma unroll
                    for (int r = 0; r < kR; ++r) {
                        const uint32_t h0 = cur[r].ok ? cur[r].hd.x : 0u;
                        uint32_t sc, m;
                        q4k_scale_min(cur[r].hd.y, cur[r].hd.z, cur[r].hd.w, j, sc, m);
                        dsc[r] = half_to_float(h0) * (float)sc;
                        dmm[r] = half_to_float(h0 >> 16) * (float)m;
                        s0[r] = 0.f;
                        s1[r] = 0.f;
                    }
                    // slot of the binary32 values, or kExactSlots: global memory
                    const int slot = (int)(-fj) - 1;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        float4 xv;
                        if (slot < kExactSlots) {
                            xv = *reinterpret_cast<const float4 *>(&xex[slot][4 * i]);
                        } else {
                            xv = gloadf4(xs + 32 * j + 4 * i);
                            xv = make_float4(ldexpf(xv.x, xsh), ldexpf(xv.y, xsh),
                                             ldexpf(xv.z, xsh), ldexpf(xv.w, xsh));
                        }
                        const float x0 = xv.x, x1 = xv.y, x2 = xv.z, x3 = xv.w;
#pragma unroll
                        for (int r = 0; r < kR; ++r) {
                            const uint32_t D = (jj < 2 ? word8(cur[r].a0, cur[r].a1, i)
                                                       : word8(cur[r].b0, cur[r].b1, i)) >> shift;
                            s0[r] = fmaf(fmaf(dsc[r], (float)(D & 15u), -dmm[r]), x0, s0[r]);
                            s1[r] = fmaf(fmaf(dsc[r], (float)((D >> 8) & 15u), -dmm[r]), x1, s1[r]);
                            s0[r] = fmaf(fmaf(dsc[r], (float)((D >> 16) & 15u), -dmm[r]), x2, s0[r]);
                            s1[r] = fmaf(fmaf(dsc[r], (float)((D >> 24) & 15u), -dmm[r]), x3, s1[r]);
                        }
                    }
#pragma unroll
                    for (int r = 0; r < kR; ++r)
                        acc[r] += s0[r] + s1[r];
                }
            }
            if (c == nchunk - 1) {
                const int row0 = r_lo + t * tile_rows + wave * wave_rows;
                const int xsh_out = 15 - vexp;
#pragma unroll
                for (int r = 0; r < kR; ++r) {
                    // every lane of a 16-lane row ends with that row's sum
                    const float v = ldexpf(rowsum16(acc[r]), -xsh_out);
                    const float q0 = lane_value(v, 0), q1 = lane_value(v, 16);
                    const float q2 = lane_value(v, 32), q3 = lane_value(v, 48);
                    if (PAIR) {
                        // rows come in (gate, up) pairs: rpg 2 holds one
                        // pair per row group, rpg 4 two
                        const int vrow = row0 + rpg * r + 2 * lane;
                        const float g = rpg == 2 ? q0 + q1 : lane == 0 ? q0 : q2;
                        const float u = rpg == 2 ? q2 + q3 : lane == 0 ? q1 : q3;
                        if (lane < rpg / 2 && vrow < r_end)
                            e.y[vrow >> 1] = silu(g) * u;
                    } else if (rpg == 2) {
                        const int row = row0 + 2 * r + lane;
                        if (lane < 2 && row < r_end)
                            e.y[row] = lane == 0 ? q0 + q1 : q2 + q3;
                    } else {
                        const int row = row0 + 4 * r + lane;
                        if (lane < 4 && row < r_end)
                            e.y[row] = lane == 0 ? q0 : lane == 1 ? q1 : lane == 2 ? q2 : q3;
                    }
                    acc[r] = 0.f;
                }
            }
            ++st;
            return st < step_hi;
        };
        if (NB == 2) {
            for (;;) {
                if (!step(A, B))
                    break;
                if (!step(B, A))
                    break;
            }
        } else {
            for (;;) {
                if (!step(A, C))
                    break;
                if (!step(B, A))
                    break;
                if (!step(C, B))
                    break;
            }
        }
    }
}

int device_cus()
{
    // one entry per device, written once with the same value by any thread
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    if (!cus[dev]) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            v <= 0)
            v = 256;
        cus[dev] = v;
    }
    return cus[dev];
}

// Two workgroups per CU, all resident at once: with more (two or more rounds)
// the second round starts staggered behind the first and the last CUs finish
// later (measured on the decode stack: 2 x CUs 741 us, 3 x 751, 4 x 763).
// Launches of under 256 MB of work take one workgroup per CU: each workgroup
// stages the activation vector once, which weighs on short ranges (measured:
// one 14336 x 4096 product 19.9 -> 18.0 us, its gate/up pair 23.6 -> 22.5 us;
// 4096 x 4096 and 4096 x 14336 unchanged).
int gemv_stream_grid(long long total_work, long long tiles)
{
    long long g = total_work < (1LL << 28) ? (long long)device_cus() : 2LL * device_cus();
    if (tiles < g)
        g = tiles;
    return (int)(g > 0 ? g : 1);
}

long long gemv_stream_tiles(int64_t M, int64_t K)
{
    (void)K;
    return (M + kTileRowsMin - 1) / kTileRowsMin;
}

// Launches of one workgroup per CU (under 256 MB) from 16 MB up step two row
// groups per wave instead of three: such a workgroup owns a few dozen rows,
// and the smaller tile leaves less of its last step empty (measured, rotated
// over 1 GB of weights: 14336 x 4096 19.2 -> 18.1 us, 4096 x 14336 27.5 ->
// 23.5 us; 4096 x 4096 and smaller were 4-6% slower with it, and the decode
// stack 1% slower).
static bool gemv_stream_two_groups(long long total_work, int grid)
{
    return grid <= device_cus() && total_work >= (16LL << 20);
}

hipError_t launch_gemv_stream(const GemvEntry *table_dev, const GemvEntry &inline0, int n,
                              long long total_bytes, int grid, hipStream_t s)
{
    if (gemv_stream_two_groups(total_bytes, grid))
        hipLaunchKernelGGL((gemv_q4k_stream_kernel<2, 2, 4>), dim3((unsigned)grid), dim3(256), 0,
                           s, table_dev, inline0, n, total_bytes, nullptr);
    else
        hipLaunchKernelGGL((gemv_q4k_stream_kernel<kR, 2, 4>), dim3((unsigned)grid), dim3(256), 0,
                           s, table_dev, inline0, n, total_bytes, nullptr);
    return hipGetLastError();
}

hipError_t launch_gemv_swiglu(const void *w_gate, const void *w_up, const float *x, float *h,
                              int64_t M, int64_t K, hipStream_t s)
{
    const GemvEntry e{(const uint8_t *)w_gate, x, h, (int)M, (int)K, 0, 0};
    const long long total = 2LL * M * gemv_row_work(K);
    const int grid = gemv_stream_grid(total, gemv_stream_tiles(2 * M, K));
    if (gemv_stream_two_groups(total, grid))
        hipLaunchKernelGGL((gemv_q4k_stream_kernel<2, 2, 4, true>), dim3((unsigned)grid),
                           dim3(256), 0, s, nullptr, e, 1, total, (const uint8_t *)w_up);
    else
        hipLaunchKernelGGL((gemv_q4k_stream_kernel<kR, 2, 4, true>), dim3((unsigned)grid),
                           dim3(256), 0, s, nullptr, e, 1, total, (const uint8_t *)w_up);
    return hipGetLastError();
}

} // namespace gq
