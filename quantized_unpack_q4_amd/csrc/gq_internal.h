// gq_internal.h -- launchers behind the C ABI.  Arguments are already
// validated by gq_api.cpp (sizes positive, K a multiple of the block,
// pointers non-null and 16-byte aligned) when these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gq {

hipError_t launch_dequant_q8_0(const void *w, float *out32, uint16_t *out16, int64_t M,
                               int64_t K, hipStream_t s);
hipError_t launch_dequant_q4k(const void *w, float *out32, uint16_t *out16, int64_t M,
                              int64_t K, hipStream_t s);

hipError_t launch_gemv_q8_0(const void *w, const float *x, float *y, int64_t M, int64_t K,
                            int B, hipStream_t s);
hipError_t launch_gemv_q4k(const void *w, const float *x, float *y, int64_t M, int64_t K, int B,
                           hipStream_t s);

// Compute units of the current device (cached per device; 256 if the query fails).
int device_cus();

// Persistent batch-1 Q4_K matrix-vector products over a table of matrices.
constexpr int GemvStreamMaxK = 16384;
// Work of one row of a matrix-vector product in bytes' worth: its weight
// bytes, but at least kGemvRowFloor, the time a row takes whatever its length
// (reduction, epilogue, issue).  The tables split work among workgroups in
// these units, so that a matrix of short rows (a row-parallel shard with
// K = 512 has 288-byte rows) does not leave one workgroup with thousands of
// rows; rows longer than the floor count their bytes alone.  Measured on one
// GPU's 8-way tensor-parallel share of the decode stack (491 MB, o and down
// split along K): 299 -> 142 us at batch 1, the whole stack unchanged.  The
// batch 2-16 kernel splits by bytes (its 128-row blocks amortize the per-row
// cost; the floor made that share 16% slower).
constexpr long long kGemvRowFloor = 1152;
__host__ __device__ inline long long gemv_row_work(long long K)
{
    const long long b = (K / 256) * 144;
    return b > kGemvRowFloor ? b : kGemvRowFloor;
}

struct GemvEntry {
    const uint8_t *w; // Q4_K weights, M rows of K/256 super-blocks
    const float *x;   // [K]
    float *y;         // [M]
    int M, K;
    long long byte_begin; // weight bytes of the entries before this one (batch 2-16 split)
    long long work_begin; // gemv_row_work of the entries before this one (batch-1 split)
};
static_assert(sizeof(GemvEntry) == 48, "table entry layout");
long long gemv_stream_tiles(int64_t M, int64_t K);
int gemv_stream_grid(long long total_work, long long tiles);
// table_dev == nullptr: a single matrix given by inline0 (n must be 1)
hipError_t launch_gemv_stream(const GemvEntry *table_dev, const GemvEntry &inline0, int n,
                              long long total_bytes, int grid, hipStream_t s);

// h[r] = silu(w_gate_r x) * (w_up_r x), batch 1, both M x K Q4_K matrices
// streamed by one launch of the batch-1 kernel (K <= GemvStreamMaxK).
hipError_t launch_gemv_swiglu(const void *w_gate, const void *w_up, const float *x, float *h,
                              int64_t M, int64_t K, hipStream_t s);

// Small-batch (2 <= B <= 16) products on the matrix cores, over a table of
// entries (or the single entry inline0 when table_dev is null); blocks of 64,
// 128 or 192 rows are dealt to workgroups by byte ranges of the packed weights.
long long gemv_mfma_blocks(int64_t M, int tiles); // blocks of 64*tiles rows (tiles 1, 2 or 3)
// The same over a table with the activations staged once per (entry,
// super-block) into a workspace by a pre-pass: [prefix: int32 [n+1]], then at
// gemv_prestaged_records_offset(n) one record of rec_bytes(B) per super-block
// of every entry (records = sum of K/256 over the entries).
inline long long gemv_prestaged_records_offset(int64_t n) { return ((n + 1) * 4 + 255) / 256 * 256; }
long long gemv_mfma_prestaged_bytes(int64_t n, long long records, int B);
hipError_t launch_gemv_mfma_prestaged(const GemvEntry *table_dev, int n, long long total_bytes,
                                      long long blocks1, long long blocks2, long long blocks3,
                                      long long records, int B, void *ws, hipStream_t s);
// h[b][r] = silu(w_gate_r x[b]) * (w_up_r x[b]) for 2 <= B <= 16 on the same
// kernel: blocks of 64 output rows pair 64 gate rows with the same up rows.
hipError_t launch_gemv_swiglu_mfma(const void *w_gate, const void *w_up, const float *x, float *h,
                                   int64_t M, int64_t K, int B, hipStream_t s);
hipError_t launch_gemv_mfma(const GemvEntry *table_dev, const GemvEntry &inline0, int n,
                            long long total_bytes, long long blocks1, long long blocks2,
                            long long blocks3, int B, hipStream_t s);

hipError_t launch_gemm_q4k(const void *w, const uint16_t *x, uint16_t *y, int64_t M, int64_t K,
                           int64_t N, hipStream_t s);
// The same product over Q8_0 weights (K % 64 == 0), on the LDS-tile kernel.
hipError_t launch_gemm_q8_0(const void *w, const uint16_t *x, uint16_t *y, int64_t M, int64_t K,
                            int64_t N, hipStream_t s);
// Large-tile matrix product (prefill): tiles of bm = 256 or 128 weight rows by
// 256 activation rows, Q4_K weights or (q8) Q8_0 weights.  gemm_big_fits: the shape fits the kernel's 32-bit
// activation offsets.  gemm_big_choice: the tile height of the large-tile
// kernel for a shape (256 when there are 256 such tiles or more, else 128
// when there are 192 or more), 0 for the small-tile kernels; the automatic
// dispatch takes it where gemm_kgroups_choice returns 0.
bool gemm_big_fits(int64_t M, int64_t K, int64_t N);
int gemm_big_choice(int64_t M, int64_t K, int64_t N);
hipError_t launch_gemm_big(const void *w, const uint16_t *x, uint16_t *y, int64_t M, int64_t K,
                           int64_t N, int bm, bool q8, hipStream_t s);
// Large-tile product with K split across kg (2 or 4) groups of waves inside
// each workgroup: tiles of 256/kg weight rows x 128 activation rows, one
// workgroup per CU, no workspace; requires (K/256) % kg == 0 and
// gemm_big_fits.  gemm_kgroups_choice: the group count the automatic dispatch
// uses for a shape (0: another family), from an estimate of each family's
// rounds of tiles on the device.
int gemm_kgroups_choice(int64_t M, int64_t K, int64_t N);
hipError_t launch_gemm_kgroups(const void *w, const uint16_t *x, uint16_t *y, int64_t M,
                               int64_t K, int64_t N, int kg, bool q8, hipStream_t s);
// Split-K form of the 256 x 256 large-tile product: `splits` runs of K/splits
// (whole super-blocks) into binary32 partials ws [splits][N][M], then a fixed
// order sum rounded to binary16.  gemm_splitk_choice: the split count that
// needs the fewest rounds of tiles on this device (1 when splitting does not
// help).
int gemm_splitk_choice(int64_t M, int64_t K, int64_t N);
hipError_t launch_gemm_splitk(const void *w, const uint16_t *x, uint16_t *y, int64_t M, int64_t K,
                              int64_t N, int splits, float *ws, hipStream_t s);
// The library's static split-K scratch (no allocation): its size, and its
// device address on the current device (looked up once per device).
constexpr size_t kSplitkScratchBytes = (size_t)64 << 20;
hipError_t splitk_scratch(float **out);

// Mixture-of-experts pieces; ws_off are the region offsets of gq_moe_workspace_offsets.
struct MoeArgs {
    const uint8_t *w_gate, *w_up, *w_down;
    const uint16_t *x;
    const int32_t *ids;
    const float *wts;
    uint16_t *out;
    int64_t T, H, I, E, topk;
    uint8_t *ws;
    size_t off[7];
    int weight_input; // 1: each slot's weight scales the expert's input (h = silu(p g) (p u),
                      // output rows summed unweighted); 0: it scales the expert's output
    int q8_0;         // 1: the three weight stacks are Q8_0 (128-row tile kernel only); 0: Q4_K
};
hipError_t launch_moe(const MoeArgs &a, hipStream_t s);

// Q8_0 products for 2..16 activation rows on the matrix cores (K % 64 == 0).
hipError_t launch_gemv_q8_0_mfma(const void *w, const float *x, float *y, int64_t M, int64_t K,
                                 int B, hipStream_t s);

// A single Q4_K product, 2 <= B <= 16, on the binary32 matrix cores with K
// split over the waves of a workgroup (gemv_q4k_f32.hip).
hipError_t launch_gemv_q4k_f32(const void *w, const float *x, float *y, int64_t M, int64_t K,
                               int B, hipStream_t s);

// Activations as 8-bit blocks of 256 (x [B][K] -> codes [B][K], scales
// [B][K/256], sub-block sums [B][K/32]) and the Q4_K integer-dot product over
// them, 1 <= B <= 16.
hipError_t launch_quantize_q8k(const float *x, int8_t *q, float *d, int32_t *bsum, int64_t B,
                               int64_t K, hipStream_t s);
hipError_t launch_gemv_q4k_q8k(const void *w, const int8_t *q, const float *d,
                               const int32_t *bsum, float *y, int64_t M, int64_t K, int B,
                               hipStream_t s);

// The integer-dot matrix product over 8-bit activation codes (prefill):
// y [N][M] binary32 from Q4_K w, codes q [N][K] and scales d [N][K/256].
hipError_t launch_gemm_q4k_q8k(const void *w, const int8_t *q, const float *d, float *y, int64_t M,
                               int64_t K, int64_t N, hipStream_t s);

// Top-k routing of T tokens over E <= 256 experts (one wave per token).
hipError_t launch_moe_route(const float *logits, int32_t *ids, float *wts, int64_t T, int64_t E,
                            int64_t topk, bool renorm, hipStream_t s);

// Token-tile size used by the grouped products for a given mean tokens per expert.
int moe_token_tile(int64_t assignments, int64_t experts);
// Expert products streamed once per chunk of 64 tokens (few tokens per expert).
bool moe_skinny_applies(int64_t assignments, int64_t experts);
hipError_t launch_moe_skinny(const MoeArgs &a, hipStream_t s);
// Expert products on 256 x 256 tiles (many tokens per expert); token tiles of
// moe_big_token_tile() sorted positions.
bool moe_big_applies(int64_t assignments, int64_t experts, int64_t H, int64_t I);
int moe_big_token_tile();
hipError_t launch_moe_big(const MoeArgs &a, int max_tiles, hipStream_t s);

} // namespace gq
