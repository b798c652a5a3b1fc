/*
 * gq.h -- fused block-dequant matrix products for AMD MI355X (gfx950).
 *
 * The operation (page "Building a Rust Inference Engine That Matches
 * Llama.cpp", section "Where the wins came from"): weights are kept as GGUF
 * quantized blocks (4-bit and 8-bit) and are never expanded into a full
 * precision buffer; each weight is dequantized inside the dot product that
 * consumes it.  Four forms are exported: batch-1 and small-batch
 * matrix-vector products for decode and continuous batching, a matrix
 * product for prefill, and the grouped per-expert form for mixture-of-experts
 * layers (page "Frink Inference: the Rust alternative to llama.cpp", opening
 * paragraph: quantized kernels and expert routing; section "A serving stack
 * with the full sampling surface": continuous batching).
 *
 * Block formats (GGUF; page "Building a Rust Inference Engine That Matches
 * Llama.cpp", sections "What Ferrox actually is" and "Further resources"),
 * little-endian, rows of K weights stored back to back with no padding:
 *
 *   Q8_0  34 bytes per 32 weights: binary16 d, then 32 int8 q; w = d*q.
 *   Q4_K  144 bytes per 256 weights: binary16 d, binary16 dmin, 12 bytes
 *         holding eight 6-bit scales sc[j] and eight 6-bit mins m[j] of the
 *         32-weight sub-blocks j, then 128 bytes of 4-bit quants q (byte 32g+i
 *         holds weight 64g+i in its low nibble and weight 64g+32+i in its high
 *         nibble); w = d*sc[j]*q - dmin*m[j].
 *
 * Each binary32 weight is the exact value rounded once (nearest even); the
 * binary16 weight fed to half-precision matrix cores is that binary32 value
 * rounded to binary16.  Activations of the matrix-vector products stay
 * binary32 (page "Frink Inference: the Rust alternative to llama.cpp",
 * section "Where llama.cpp is still ahead", K-quant item): they are never
 * quantized.
 *
 * Conventions for every entry point:
 *   - All buffer pointers are device pointers on the current HIP device,
 *     allocated and owned by the caller; the library never allocates, frees
 *     or retains them.  Base pointers must be 16-byte aligned.
 *   - Activations and outputs are dense row-major: x[B][K], y[B][M] for the
 *     matrix-vector products; X[N][K], Y[N][M] for the matrix products
 *     (Y = X * W^T).  binary16 buffers are passed as uint16_t bit patterns.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls are
 *     asynchronous: the return value covers argument checks and the launch
 *     only; faults surface at the caller's next synchronisation.
 *   - A call with no work (zero rows, tokens or batch) returns GQ_OK and
 *     launches nothing; its pointers are not checked.  K (H, I) must be
 *     positive.
 *   - On any status other than GQ_OK nothing has been launched and
 *     gq_last_error() (per thread) names the argument and the violated
 *     condition.  Unsupported shapes are refused, never computed on a subset.
 *   - No entry point keeps state between calls apart from the error string;
 *     calls on different streams may run concurrently.
 */
#ifndef GQ_H
#define GQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gq_status {
    GQ_OK = 0,
    GQ_EINVAL = 1,     /* null pointer, negative size, batch out of range, topk outside [1, E] */
    GQ_ESHAPE = 2,     /* K (or H, I) not a multiple of the block size, or a size too large */
    GQ_EALIGN = 3,     /* a base pointer not 16-byte aligned */
    GQ_EWORKSPACE = 4, /* workspace missing or smaller than gq_moe_workspace_bytes() */
    GQ_EHIP = 5        /* the HIP runtime reported an error at launch */
} gq_status;

/* Largest batch accepted by the matrix-vector products. */
#define GQ_GEMV_MAX_BATCH 16

/* Q8_0 matrix-vector product, binary32 activations:
 *   y[b][r] = sum_k w[r][k] * x[b][k]  for r < M, b < B, accumulated in binary32.
 * w: M rows of K/32 Q8_0 blocks (M*K/32*34 bytes).  x: [B][K] float.  y: [B][M] float.
 * Requires K % 32 == 0, 1 <= B <= GQ_GEMV_MAX_BATCH.  With B >= 2 and
 * K % 64 == 0 the block sums d * sum(q*x) run on the binary32 matrix-core
 * products: the quant converted exactly, x as given, products and sums in
 * binary32, d applied once per 32-weight block.  Accuracy: see
 * GQ_GEMV_ACCURACY below (results in the subnormal range: up to one multiple
 * of 2^-149 per block).  An activation row's result does not depend on the
 * other rows; B <= 4 and B >= 5 sum in different orders (two matrix-core
 * products), so a row's bits can differ between the two ranges, and B = 1
 * runs another kernel. */
gq_status gq_gemv_q8_0(const void *w, const float *x, float *y, int64_t M, int64_t K, int64_t B,
                       void *stream);

/* Q4_K matrix-vector product, binary32 activations; same contract as
 * gq_gemv_q8_0 with w holding M rows of K/256 super-blocks (M*K/256*144
 * bytes).  Requires K % 256 == 0, 1 <= B <= GQ_GEMV_MAX_BATCH.  Per 32-weight
 * sub-block the sum is taken in the factored form
 * (d*sc)*sum(q*x) - (dmin*m)*sum(x), with x carried as a binary16 hi + lo
 * pair (products exact, sums binary32): batch 1 on packed dot products with
 * one power-of-two scale per sub-block, batches 3..16 on matrices of more
 * than 32 rows per CU (and, at batch 3..4, of at least 12288 rows) on the
 * matrix cores with one per activation row and
 * super-block (see gq_gemv_q4k_multi_batched).  Every split value keeps a
 * relative error below 2^-19.  A sub-block whose non-zero |x| span more than
 * 2^20 (batch 1; batches 3..16: holding a non-zero |x| below 2^-20 of its
 * super-block's largest), or that holds more than 1/16 of the sum of |x|
 * over its super-block, is computed exactly instead: each weight as its
 * binary32 value times x in binary32.  The other batch 2..16 products
 * (batch 2, batch 3..4 below 12288 rows, up to 32 rows per CU, or matrices
 * beyond the 32-bit offsets of that kernel) dequantize each weight to binary32, fma(q, d*sc, -dmin*m)
 * with one rounding, and take products and sums in binary32 on the matrix
 * cores, K split over the waves of a workgroup (results in the subnormal
 * range: up to K/2 multiples of 2^-149).  K above 16384 at batch 1 runs a
 * kernel that dequantizes every weight to binary32 first.
 *
 * GQ_GEMV_ACCURACY (every binary32-activation product of this header): with
 * S = sum_k |w_k x_k| (w the binary32 weight) and finite inputs,
 * |y - y_exact| <= 1e-5 * S, plus up to a few multiples of 2^-149 when y
 * falls in the binary32 subnormal range, provided no result or partial sum
 * overflows binary32 and the factored sums do not cancel heavily: their
 * rounding follows S_f = sum over split sub-blocks of
 * (|d*sc*q_k| + |dmin*m|) * |x_k|, and the bound is met while S_f stays
 * within a few times S.  Rows of the seeded generator have S_f / S of 1.2 to
 * 1.6; a row can exceed it only when d*sc*q and dmin*m nearly cancel for most
 * of its weights at once.  Single large activations (their sub-block goes to
 * the exact path), wide ranges inside one vector and whole vectors from 1e-40
 * to 1e30 are inside the bound (tested). */
gq_status gq_gemv_q4k(const void *w, const float *x, float *y, int64_t M, int64_t K, int64_t B,
                      void *stream);

/* Batch-1 Q4_K matrix-vector products of a whole table of independent
 * matrices in ONE launch (a decode step of a transformer's linear layers:
 * every weight byte streamed once, no per-matrix launch cost).  The pages cut
 * the same per-matmul overhead by grouping work into fewer GPU submissions
 * (page "Frink Inference: the Rust alternative to llama.cpp", section "The
 * engine").  Use in three steps:
 *   1. bytes = gq_gemv_q4k_multi_table_bytes(n);
 *   2. gq_gemv_q4k_multi_plan(descs, n, table, bytes) checks every descriptor
 *      on the host and writes the work table into host memory `table`;
 *   3. copy those bytes once to a device buffer `table_dev` (16-byte aligned)
 *      and call gq_gemv_q4k_multi(table, table_dev, stream) as often as needed;
 *      each call computes y_i = W_i x_i for every descriptor i.
 * The table holds the descriptors' pointers: it stays valid as long as those
 * buffers do.  table_dev must hold exactly the bytes of `table` (only the host
 * copy is checked).  Each descriptor needs K % 256 == 0, 256 <= K <= 16384,
 * M >= 1 and 16-byte aligned w, x, y; x is [K] and y is [M] (batch 1).
 * Products run concurrently: outputs must not overlap any input. */
typedef struct gq_gemv_desc {
    const void *w; /* Q4_K weights, M rows of K/256 super-blocks */
    const float *x; /* [K] binary32 */
    float *y;       /* [M] binary32 */
    int64_t M, K;
} gq_gemv_desc;

size_t gq_gemv_q4k_multi_table_bytes(int64_t n); /* 0 if n is outside [1, 2^20] */
gq_status gq_gemv_q4k_multi_plan(const gq_gemv_desc *descs, int64_t n, void *table,
                                 size_t table_bytes);
gq_status gq_gemv_q4k_multi(const void *table, const void *table_dev, void *stream);

/* The gate and up products of a feed-forward layer with the SwiGLU epilogue,
 * batch 1, in one launch (the pages credit fused projection kernels, page
 * "Building a Rust Inference Engine That Matches Llama.cpp", section "Where
 * the wins came from"):
 *   h[r] = silu(g_r) * u_r,  g = W_gate x,  u = W_up x,  silu(z) = z / (1 + e^-z)
 * with g and u computed as by gq_gemv_q4k (binary32 activations and sums) and
 * the epilogue in binary32.  w_gate, w_up: M x K Q4_K matrices.  x: [K]
 * binary32.  h: [M] binary32.  Requires K % 256 == 0, 256 <= K <= 16384,
 * 0 <= M <= 2^29 (M = 0 launches nothing), 16-byte aligned pointers; h must
 * not overlap the inputs. */
gq_status gq_gemv_q4k_swiglu(const void *w_gate, const void *w_up, const float *x, float *h,
                             int64_t M, int64_t K, void *stream);

/* gq_gemv_q4k_swiglu at batch B (1 <= B <= 16): x [B][K] binary32, h [B][M]
 * binary32, h[b][r] = silu(g_r(x[b])) * u_r(x[b]).  B = 1 is
 * gq_gemv_q4k_swiglu; for B >= 2 g and u are computed as by
 * gq_gemv_q4k_multi_batched (the matrix cores, the same error bound), one
 * launch streaming both matrices, the epilogue in binary32.  Requires
 * K % 256 == 0, M * (K/256) * 144 < 2^32 and B * K * 4 < 2^31 for B >= 2
 * (GQ_ESHAPE otherwise; B = 1 as gq_gemv_q4k_swiglu), B in [1, 16]
 * (GQ_EINVAL), 16-byte aligned pointers; M = 0 launches nothing; h must not
 * overlap the inputs. */
gq_status gq_gemv_q4k_swiglu_batched(const void *w_gate, const void *w_up, const float *x,
                                     float *h, int64_t M, int64_t K, int64_t B, void *stream);

/* The same planned products at batch B (1 <= B <= 16): descriptor i's x is
 * [B][K] and y is [B][M] (row-major), y_i[b] = W_i x_i[b].  B = 1 is
 * gq_gemv_q4k_multi.  For B >= 2 the products run on the matrix cores (the
 * 4-bit quants times a binary16 hi + lo split of each activation, scaled per
 * activation row and super-block by a power of two; binary32 sums; error
 * bound as for gq_gemv_q4k) and every matrix needs fewer than 2^32 bytes of
 * weights and fewer than 2^31 bytes of activations (GQ_ESHAPE otherwise). */
gq_status gq_gemv_q4k_multi_batched(const void *table, const void *table_dev, int64_t B,
                                    void *stream);

/* gq_gemv_q4k_multi_batched with the activations staged once per product and
 * super-block into a caller workspace by a pre-pass, instead of by every block
 * of 192 weight rows: three launches on the stream (a prefix of the entries'
 * super-blocks, the staging, the products).  Same results, bit for bit, and
 * the same limits; B = 1 is gq_gemv_q4k_multi (ws unused, may be NULL).
 * ws: at least gq_gemv_q4k_multi_batched_ws_bytes(table, B) bytes, 16-byte
 * aligned, contents on entry ignored; it must not be in use by another call
 * while this one runs.  Errors as gq_gemv_q4k_multi_batched, plus
 * GQ_EWORKSPACE (ws NULL or too small) and GQ_EALIGN. */
gq_status gq_gemv_q4k_multi_batched_ws(const void *table, const void *table_dev, int64_t B,
                                       void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes of gq_gemv_q4k_multi_batched_ws (1 for B = 1); 0 if the
 * table or B is invalid. */
size_t gq_gemv_q4k_multi_batched_ws_bytes(const void *table, int64_t B);

/* Q4_K matrix product for prefill, binary16 activations and output:
 *   Y[n][r] = binary16( sum_k X[n][k] * w16[r][k] ),  accumulated in binary32,
 * where w16 is each weight rounded to binary16 as described above.
 * x: [N][K] binary16 bits.  y: [N][M] binary16 bits.  Requires K % 256 == 0. */
gq_status gq_gemm_q4k(const void *w, const uint16_t *x, uint16_t *y, int64_t M, int64_t K,
                      int64_t N, void *stream);

/* The same product over Q8_0 weights (M rows of K/32 blocks):
 *   Y[n][r] = binary16( sum_k X[n][k] * w16[r][k] ),  w16 = binary16(d * q)
 * accumulated in binary32 (d * q is exact; one rounding to binary16).
 * Requires K % 64 == 0 (the small-tile kernel takes two blocks per step;
 * GQ_ESHAPE otherwise), N <= 2^21.  With K % 256 == 0 the large-tile kernel
 * or its K-group form runs it where gq_gemm_q4k would take them. */
gq_status gq_gemm_q8_0(const void *w, const uint16_t *x, uint16_t *y, int64_t M, int64_t K,
                       int64_t N, void *stream);

/* gq_gemm_q8_0 with the kernel family pinned, as gq_gemm_q4k_tiles pins it
 * for Q4_K: tile_rows = 0 automatic, 64 the small-tile kernel (K % 64 == 0),
 * 128 and 256 the large-tile kernel (K % 256 == 0 and N*K*2 < 2^31, else
 * GQ_ESHAPE).  Same result and bound; the summation order differs between
 * families.  GQ_EINVAL for any other tile_rows. */
gq_status gq_gemm_q8_0_tiles(const void *w, const uint16_t *x, uint16_t *y, int64_t M, int64_t K,
                             int64_t N, int64_t tile_rows, void *stream);

/* gq_gemm_q4k with the kernel family pinned instead of chosen from the shape:
 * tile_rows = 0 is the automatic choice of gq_gemm_q4k, 64 the small-tile
 * kernels (64 or 128 weight rows per tile, chosen from the shape), 128 and 256
 * the large-tile kernel with tiles of that many weight rows by 256 activation
 * rows.  Same arguments, result and rounding as gq_gemm_q4k (the summation
 * order inside a tile differs between families, so results agree to binary32
 * rounding, not bit for bit).  Errors: GQ_EINVAL for any other tile_rows;
 * GQ_ESHAPE when N*K*2 >= 2^31 with tile_rows 128 or 256. */
gq_status gq_gemm_q4k_tiles(const void *w, const uint16_t *x, uint16_t *y, int64_t M, int64_t K,
                            int64_t N, int64_t tile_rows, void *stream);

/* gq_gemm_q4k on tiles of 256/groups weight rows by 128 activation rows whose
 * K reduction is split across `groups` groups of waves inside each workgroup
 * (groups = 2 or 4), for products whose large tiles are too few to fill the
 * device (prefill with few tokens and a long K) when no workspace is at hand:
 * group g sums the g-th of `groups` equal runs of K in binary32, the runs'
 * sums are added in run order inside the workgroup (deterministic) and
 * rounded once to binary16.  Same arguments, result and bound as
 * gq_gemm_q4k; the summation order differs, so results agree to binary32
 * rounding, not bit for bit.  Nothing is allocated.  Errors: GQ_EINVAL for
 * other groups; GQ_ESHAPE when groups does not divide K/256 or
 * N*K*2 >= 2^31. */
gq_status gq_gemm_q4k_kgroups(const void *w, const uint16_t *x, uint16_t *y, int64_t M, int64_t K,
                              int64_t N, int64_t groups, void *stream);

/* gq_gemm_q4k with K cut into `splits` equal runs of whole super-blocks, for
 * products whose 256 x 256 tiles are too few to fill the device (prefill with
 * few tokens and a long K): each run's product goes to the caller workspace
 * as binary32 partials ws [splits][N][M], which are then summed in binary32
 * in run order (deterministic) and rounded once to binary16 into y.  Same
 * arguments and bound as gq_gemm_q4k otherwise (binary16 weights, binary32
 * sums); the summation order differs, so results agree to binary32 rounding,
 * not bit for bit.  splits = 0 lets the library choose: the divisor of K/256
 * up to 32 with the least estimated time (rounds of tiles on this device
 * against the traffic of the partials).
 * ws: at least gq_gemm_q4k_splitk_workspace_bytes(M, K, N, splits) bytes,
 * 16-byte aligned; contents on entry are ignored.  Requires M, N >= 1,
 * K % 256 == 0, splits dividing K/256 (else GQ_ESHAPE), 0 <= splits <= 64
 * (else GQ_EINVAL), N*K*2 < 2^31 and M*K*144/256 < 2^32 (else GQ_ESHAPE). */
gq_status gq_gemm_q4k_splitk(const void *w, const uint16_t *x, uint16_t *y, int64_t M, int64_t K,
                             int64_t N, int64_t splits, void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes of gq_gemm_q4k_splitk (splits = 0: for the automatic
 * choice); 0 if the arguments are invalid. */
size_t gq_gemm_q4k_splitk_workspace_bytes(int64_t M, int64_t K, int64_t N, int64_t splits);

/* gq_gemm_q4k_splitk without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the binary32 partials live in a static
 * array inside the library, one per GPU, of
 * gq_gemm_q4k_splitk_static_max_bytes() = 64 MiB, held until the process
 * ends.  The call allocates nothing.  Same arguments, results (bit for bit)
 * and refusals as gq_gemm_q4k_splitk; in addition GQ_EWORKSPACE when
 * splits*N*M*4 bytes exceed the scratch (e.g. 4096 x 14336 x 512 fits with
 * its automatic 8 splits, 4096 tokens do not), and GQ_EHIP when the scratch's
 * device address cannot be looked up.  Every call on one GPU shares that
 * GPU's scratch, which keeps the last call's partials: calls that overlap
 * in time on one GPU (different streams, or host threads) race and must be
 * serialised by the caller. */
gq_status gq_gemm_q4k_splitk_static(const void *w, const uint16_t *x, uint16_t *y, int64_t M,
                                    int64_t K, int64_t N, int64_t splits, void *stream);

/* Size in bytes of gq_gemm_q4k_splitk_static's scratch. */
size_t gq_gemm_q4k_splitk_static_max_bytes(void);

/* Mixture-of-experts feed-forward over Q4_K experts (the grouped form):
 *   for every token t and slot s < topk, with e = topk_ids[t][s]:
 *     g = Wg_e x_t, u = Wu_e x_t            (binary16 matrix cores, binary32 sums)
 *     h = binary16( silu(g) * u )           silu(z) = z / (1 + exp(-z))
 *     d = Wd_e h                            (binary32)
 *   out[t] = binary16( sum_{s = 0..topk-1} topk_w[t][s] * d_s ), summed in slot order.
 * w_gate, w_up: E stacked [I rows][H cols] Q4_K matrices.  w_down: E stacked
 * [H rows][I cols] Q4_K matrices.  x: [T][H] binary16.  topk_ids: [T][topk]
 * int32 in [0, E).  topk_w: [T][topk] float (used as given, no renormalisation).
 * out: [T][H] binary16.  ws: workspace of at least gq_moe_workspace_bytes()
 * bytes (layout: gq_moe_workspace_offsets()); contents on entry are ignored.
 * Requires H % 256 == 0, I % 256 == 0, 1 <= topk <= E <= 256, T*topk <= 2^20.
 * An id outside [0, E) cannot be checked on the host: its slot is skipped
 * (contributes nothing) and counted in the workspace's expert table. */
gq_status gq_moe_gemm_q4k(const void *w_gate, const void *w_up, const void *w_down,
                          const uint16_t *x, const int32_t *topk_ids, const float *topk_w,
                          uint16_t *out, int64_t T, int64_t H, int64_t I, int64_t E,
                          int64_t topk, void *ws, size_t ws_bytes, void *stream);

/* gq_moe_gemm_q4k with each slot's weight applied to the expert's input
 * instead of its output (the Llama 4 form, page "Frink Inference: the Rust
 * alternative to llama.cpp", section "Architecture coverage"):
 *   g = Wg_e (w x), u = Wu_e (w x), h = binary16( silu(g) * u ), d = Wd_e h,
 *   out[t] = binary16( sum over slots of d ),  w = topk_w[t][s].
 * The gate and up products are linear in the input, so they are computed on x
 * and scaled by w in binary32 before the SwiGLU.  Same arguments, workspace
 * and errors as gq_moe_gemm_q4k. */
gq_status gq_moe_gemm_q4k_input_weighted(const void *w_gate, const void *w_up,
                                         const void *w_down, const uint16_t *x,
                                         const int32_t *topk_ids, const float *topk_w,
                                         uint16_t *out, int64_t T, int64_t H, int64_t I,
                                         int64_t E, int64_t topk, void *ws, size_t ws_bytes,
                                         void *stream);

/* The mixture-of-experts layer over Q8_0 expert stacks: the formula of
 * gq_moe_gemm_q4k (and, for the second call, of
 * gq_moe_gemm_q4k_input_weighted) with w_gate, w_up E stacked [I rows][H cols]
 * and w_down E stacked [H rows][I cols] Q8_0 matrices (rows of 34-byte
 * blocks), each weight entering as binary16(d * q).  Q8_0 is the format whose
 * logits the pages report as matching llama.cpp's exactly (page "Frink
 * Inference: the Rust alternative to llama.cpp", the item on K-quant logits
 * drifting).  Same arguments, workspace, shape limits (H % 256 == 0,
 * I % 256 == 0) and errors as gq_moe_gemm_q4k. */
gq_status gq_moe_gemm_q8_0(const void *w_gate, const void *w_up, const void *w_down,
                           const uint16_t *x, const int32_t *topk_ids, const float *topk_w,
                           uint16_t *out, int64_t T, int64_t H, int64_t I, int64_t E,
                           int64_t topk, void *ws, size_t ws_bytes, void *stream);
gq_status gq_moe_gemm_q8_0_input_weighted(const void *w_gate, const void *w_up,
                                          const void *w_down, const uint16_t *x,
                                          const int32_t *topk_ids, const float *topk_w,
                                          uint16_t *out, int64_t T, int64_t H, int64_t I,
                                          int64_t E, int64_t topk, void *ws, size_t ws_bytes,
                                          void *stream);

/* Expert routing on the device (the routing step of the mixture-of-experts
 * layer; the pages' engine routes natively, page "Frink Inference: the Rust
 * alternative to llama.cpp", opening paragraph).  For every token t:
 *   topk_ids[t] = the topk experts with the largest logits[t][e], in
 *                 descending order, equal logits going to the lower expert
 *                 index (softmax is strictly increasing, so these are the
 *                 experts with the largest probabilities; the choice is made
 *                 on the binary32 logits exactly);
 *   topk_w[t][s] = p[topk_ids[t][s]] with p = softmax(logits[t]) in binary32
 *                 (exp(l - max) / sum), or, with renormalize != 0, that
 *                 probability divided by the sum of the topk chosen ones.
 * logits: [T][E] float.  topk_ids: [T][topk] int32.  topk_w: [T][topk] float
 * (the inputs of gq_moe_gemm_q4k).  All device pointers, 16-byte aligned.
 * Requires T >= 0 (T = 0 launches nothing), 1 <= topk <= E <= 256.
 * Non-finite logits are outside the contract. */
gq_status gq_moe_route(const float *logits, int32_t *topk_ids, float *topk_w, int64_t T,
                       int64_t E, int64_t topk, int64_t renormalize, void *stream);

/* Workspace size for gq_moe_gemm_q4k with these sizes (0 if they are invalid). */
size_t gq_moe_workspace_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk);

/* Byte offsets of the workspace regions (each 256-byte aligned), in order:
 *   off[0] expert table     int32 [E+3]    [0..E-1] first sorted position of each
 *                                          expert, [E] valid assignments, [E+1] token
 *                                          tiles, [E+2] assignments dropped because
 *                                          their id is outside [0, E)
 *   off[1] sorted list      int32 [A]      assignment index t*topk+s at each sorted position
 *   off[2] position table   int32 [A]      sorted position of each assignment
 *   off[3] tile list        int32 [2][A+E] (expert, first position) of each token tile
 *   off[4] h                binary16 [A][I] expert activations, sorted order
 *   off[5] d                float [A][H]   expert outputs, sorted order
 *   off[6] total size
 * with A = T*topk.  Returns GQ_EINVAL for invalid sizes. */
gq_status gq_moe_workspace_offsets(int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk,
                                   size_t off[7]);

/* Opt-in integer-dot path (llama.cpp's evaluation of K-quant products, which
 * the pages contrast with keeping activations in binary32: page "Frink
 * Inference: the Rust alternative to llama.cpp", the item on K-quant logits
 * drifting).  Results move from the binary32 product by up to
 * sum_k |w_k| |x_k - d q_k|; the binary32 entry points above remain the
 * default.
 *
 * gq_quantize_q8k: activations as 8-bit blocks of 256 (the pages call the
 * block Q8_K without defining it; read as below).  For every row b < B and
 * block s < K/256 of x [B][K] binary32:
 *   amax = max |x|,  d[b][s] = amax / 127,
 *   q[b][k] = clamp(round_nearest_even(x[b][k] * (127 / amax)), -127, 127),
 *   bsum[b][k/32] = sum of the 32 codes of each sub-block,
 * every step in binary32 (an all-zero block has d = 0, q = 0).
 * q: [B][K] int8; d: [B][K/256] float; bsum: [B][K/32] int32.  Requires
 * K % 256 == 0 and B*K <= 2^34; x, q, d, bsum 16-byte aligned.  Non-finite
 * activations are outside the contract. */
gq_status gq_quantize_q8k(const float *x, int8_t *q, float *d, int32_t *bsum, int64_t B,
                          int64_t K, void *stream);

/* gq_gemv_q4k_q8k: y[b][r] = sum_k w(r, k) * d[b][k/256] * q[b][k] over a Q4_K
 * matrix (M rows of K/256 super-blocks) and activations from
 * gq_quantize_q8k, 1 <= B <= GQ_GEMV_MAX_BATCH.  Per 32-weight sub-block the
 * sums of q4 * q and of q are exact integers (8-bit dot products at batch
 * 1-5, the int8 matrix cores at batch 6-16, where the sub-block scales also
 * apply in int32); the remaining scales are applied in binary32.  Error against
 * the exact value of the same formula: within 1e-5 * sum_k (|d sc q4| +
 * |dmin m|) |d[b] q[b][k]|.  y: [B][M] float.  Requires K % 256 == 0. */
gq_status gq_gemv_q4k_q8k(const void *w, const int8_t *q, const float *d, const int32_t *bsum,
                          float *y, int64_t M, int64_t K, int64_t B, void *stream);

/* gq_gemm_q4k_q8k: the integer-dot matrix product (prefill) over 8-bit
 * activation codes from gq_quantize_q8k (with B = N token rows):
 *   Y[n][r] = sum_k w(r, k) * d[n][k/256] * q[n][k]
 * for a Q4_K matrix (M rows of K/256 super-blocks), q [N][K] int8, d [N][K/256]
 * float, Y [N][M] float (binary32, not rounded to binary16).  The reading of
 * the pages is that of gq_quantize_q8k (page "Frink Inference: the Rust
 * alternative to llama.cpp", section "Where llama.cpp is still ahead",
 * K-quant item: llama.cpp's 8-bit activation blocks, the source of its logit
 * drift; opt-in here, beside the binary16 product gq_gemm_q4k).  Per
 * super-block the sums of q4 * sc * q and of m * q are exact integers (int8
 * matrix cores, the 6-bit scale split into two 3-bit halves folded into the
 * weight bytes); d, dmin and d[n] apply in binary32.  Error against the exact
 * value of the same formula: within 1e-5 * sum_k (|d sc q4| + |dmin m|) *
 * |d[n] q[n][k]|.  Requires K % 256 == 0, N*K <= 2^34; M = 0 or N = 0 does
 * nothing; w, q, d, y 16-byte aligned. */
gq_status gq_gemm_q4k_q8k(const void *w, const int8_t *q, const float *d, float *y, int64_t M,
                          int64_t K, int64_t N, void *stream);

/* Dequantization probes: write every weight of an M x K matrix as binary32
 * (out32, [M][K]) and/or binary16 (out16, [M][K] bits); either may be NULL.
 * Bit-exact with the rounding rule above. */
gq_status gq_dequant_q8_0(const void *w, float *out32, uint16_t *out16, int64_t M, int64_t K,
                          void *stream);
gq_status gq_dequant_q4k(const void *w, float *out32, uint16_t *out16, int64_t M, int64_t K,
                         void *stream);

/* Diagnostics. */
const char *gq_last_error(void);       /* message of this thread's last failed call */
const char *gq_status_str(gq_status s); /* short name of a status */
int gq_version(void);                   /* major*10000 + minor*100 + patch */

#ifdef __cplusplus
}
#endif

#endif /* GQ_H */
