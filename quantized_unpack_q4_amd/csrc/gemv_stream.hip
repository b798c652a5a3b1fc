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
// Activations are scaled by a power of two (max|x| into [2^14, 2^15)), split
// as x = hi + lo with hi, lo binary16 (about 22 significant bits together)
// and staged in LDS once per matrix; the scale is undone exactly.  Quants are
// used as binary16 subnormals (the nibble bits themselves, q * 2^-24, or
// 16q * 2^-24 for high nibbles), so one v_dot2_f32_f16 multiplies two quants
// by two activation halves exactly and accumulates in binary32.  Per
// sub-block j the contribution is (d*sc_j) * sum(q*x) - (dmin*m_j) * sum(x);
// sum(x) per sub-block is staged with x.  With a one-hot x the result is the
// binary32 weight exactly (d*sc*q exact, one rounding with -dmin*m).
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
constexpr int kLdsWords = (kRecs + kRecs / 16) * 4 + kStreamMaxK / 32;
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
    uint32_t *xrec = lds;
    float *ssum = reinterpret_cast<float *>(lds + (kRecs + kRecs / 16) * 4);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int p = lane & 1;
    const long long lo = total * (long long)blockIdx.x / gridDim.x;
    const long long hi = total * (long long)(blockIdx.x + 1) / gridDim.x;

    auto entry = [&](int i) -> GemvEntry { return table ? table[i] : inline0; };
    int di = 0;
    while (di + 1 < n && entry(di + 1).work_begin <= lo)
        ++di;
    GemvEntry e = entry(di);

    int nsb = e.K >> 8, r_end = 0, rpg = 2, sps = 16, rsub = 0, sbl = 0;
    long long rowb = (long long)nsb * kQ4kBytes;

    // Power-of-two scale that brings max|x| into [2^14, 2^15): keeps the
    // binary16 hi/lo split accurate for any finite x of moderate magnitude.
    __shared__ float s_amax[W];
    float inv_scale = 1.f;
    auto stage = [&]() {
        // thread t owns sub-blocks t, t + kThreads, ... (32 activations each,
        // at most 512 sub-blocks): every activation is loaded once, all loads
        // in flight together, and kept in registers for the scale, split and sums
        const int nsub = e.K >> 5;
        float4 v[kSubPerThread][8];
        float amax = 0.f;
#pragma unroll
        for (int u = 0; u < kSubPerThread; ++u) {
            const int j = tid + kThreads * u;
            if (j < nsub) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    v[u][i] = gloadf4(e.x + 32 * j + 4 * i);
                    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[u][i].x), fabsf(v[u][i].y)),
                                             fmaxf(fabsf(v[u][i].z), fabsf(v[u][i].w))));
                }
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1)
            amax = fmaxf(amax, __shfl_xor(amax, off, 64));
        if (lane == 0)
            s_amax[wave] = amax;
        __syncthreads();
        amax = s_amax[0];
#pragma unroll
        for (int i = 1; i < W; ++i)
            amax = fmaxf(amax, s_amax[i]);
        int ex = 0;
        if (amax > 0.f)
            (void)frexpf(amax, &ex); // amax < 2^ex
        const float scale = ldexpf(1.f, 15 - ex);
        inv_scale = ldexpf(1.f, ex - 15);
        // record i holds x[4i..4i+3]*scale as (hi(x0,x2), hi(x1,x3), lo(x0,x2),
        // lo(x1,x3)); 16 bytes of padding after every 16 records.  ssum[j] is
        // the plain binary32 sum of x over sub-block j.
#pragma unroll
        for (int u = 0; u < kSubPerThread; ++u) {
            const int j = tid + kThreads * u;
            if (j < nsub) {
                float sum = 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    float4 w = v[u][i];
                    sum += (w.x + w.y) + (w.z + w.w);
                    w.x *= scale;
                    w.y *= scale;
                    w.z *= scale;
                    w.w *= scale;
                    const h2_t h02 = {(_Float16)w.x, (_Float16)w.z};
                    const h2_t h13 = {(_Float16)w.y, (_Float16)w.w};
                    const h2_t l02 = {(_Float16)(w.x - (float)h02.x), (_Float16)(w.z - (float)h02.y)};
                    const h2_t l13 = {(_Float16)(w.y - (float)h13.x), (_Float16)(w.w - (float)h13.y)};
                    const int ri = 8 * j + i;
                    *reinterpret_cast<uint4 *>(xrec + 4 * (ri + (ri >> 4))) = make_uint4(
                        __builtin_bit_cast(uint32_t, h02), __builtin_bit_cast(uint32_t, h13),
                        __builtin_bit_cast(uint32_t, l02), __builtin_bit_cast(uint32_t, l13));
                }
                ssum[j] = sum;
            }
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
            const float2 s01 = *reinterpret_cast<const float2 *>(ssum + 8 * s + 2 * p);
            const float2 s45 = *reinterpret_cast<const float2 *>(ssum + 8 * s + 2 * p + 4);
            const int o0 = 16 * p, o1 = 16 * p + 8; // bit offsets of scale bytes 2p, 2p+1
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
                const float d24 = half_to_float(h0) * 16777216.f;
                const float dmin = half_to_float(h0 >> 16);
                float t1 = (float)sc0 * P0[r];
                t1 = fmaf((float)sc1 * 0.0625f, P1[r], t1);
                t1 = fmaf((float)sc4, P4[r], t1);
                t1 = fmaf((float)sc5 * 0.0625f, P5[r], t1);
                float t2 = (float)m0 * s01.x;
                t2 = fmaf((float)m1, s01.y, t2);
                t2 = fmaf((float)m4, s45.x, t2);
                t2 = fmaf((float)m5, s45.y, t2);
                acc[r] = fmaf(-dmin, t2, fmaf(d24, t1 * inv_scale, acc[r]));
            }
            if (c == nchunk - 1) {
                const int row0 = r_lo + t * tile_rows + wave * wave_rows;
#pragma unroll
                for (int r = 0; r < kR; ++r) {
                    // every lane of a 16-lane row ends with that row's sum
                    const float v = rowsum16(acc[r]);
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

static int device_cus()
{
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

hipError_t launch_gemv_stream(const GemvEntry *table_dev, const GemvEntry &inline0, int n,
                              long long total_bytes, int grid, hipStream_t s)
{
    hipLaunchKernelGGL((gemv_q4k_stream_kernel<kR, 2, 4>), dim3((unsigned)grid), dim3(256), 0, s,
                       table_dev, inline0, n, total_bytes, nullptr);
    return hipGetLastError();
}

hipError_t launch_gemv_swiglu(const void *w_gate, const void *w_up, const float *x, float *h,
                              int64_t M, int64_t K, hipStream_t s)
{
    const GemvEntry e{(const uint8_t *)w_gate, x, h, (int)M, (int)K, 0, 0};
    const long long total = 2LL * M * gemv_row_work(K);
    const int grid = gemv_stream_grid(total, gemv_stream_tiles(2 * M, K));
    hipLaunchKernelGGL((gemv_q4k_stream_kernel<kR, 2, 4, true>), dim3((unsigned)grid), dim3(256),
                       0, s, nullptr, e, 1, total, (const uint8_t *)w_up);
    return hipGetLastError();
}

} // namespace gq
