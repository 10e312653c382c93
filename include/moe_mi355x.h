/*
 * moe_mi355x.h -- C ABI of the routed-expert MoE MLP for MI355X (gfx950).
 *
 * The forward of a routed-expert MoE MLP layer, split into the calls below and
 * run on one GPU:
 *
 *   moe_route -> moe_align_sort -> [moe_quantize_fp8 | moe_quantize_mxfp8 (x)]
 *     -> moe_grouped_gemm_swiglu -> moe_grouped_gemm_down -> moe_combine
 *
 * with variants for shared experts (moe_route_shared), the squared-ReLU
 * expert (moe_grouped_gemm_relu2) and GEMM2 with the combine fused
 * (moe_grouped_gemm_down_combine), and the BF16 backward at the end of the
 * file.
 *
 * What is computed follows the pages that describe the method:
 *   - TileScale PR #70 "SM90 FP8 distributed MegaMoE example", Design section:
 *     routing, GEMM1 (gate/up) + SwiGLU with a quantised intermediate, GEMM2,
 *     rows written per (token, top-k slot), reduce over the slots to BF16;
 *     FP8 E4M3 inputs and weights with FP32 per-128 scales.
 *   - FlashInfer PR #5129 (expert-sorted I/O for the cuTile BF16 MoE),
 *     Description: GEMM1 writes into padded expert-sorted rows, GEMM2 reads
 *     them contiguously and scatters back to assignment order, the combine is
 *     unchanged; padded rows feed only dropped output rows.
 *   - FlashInfer PR #6465 (Hopper MXFP4 x FP8 MegaMoE tuning), Benchmark
 *     configuration: E2M1 weights with one shared E8M0 scale per 32 K elements,
 *     E4M3 activations, BF16 input and output.
 *   - Liger-Kernel PR #1463, Summary: empty experts or K slices must not stall
 *     the schedule (empty experts own no tiles here).
 *
 * Conventions common to every call
 *   - All tensors are dense, row-major, the reduction dimension (K) contiguous.
 *     Weights use the [out, in] convention: W1 is [E, 2I, H] with gate rows
 *     [0, I) and up rows [I, 2I) of each expert; W2 is [E, H, I].
 *   - bf16 tensors are passed as uint16_t bit patterns.
 *   - Assignment a = t * k + j is slot j of token t. A = T * k.
 *   - Device pointers: every pointer argument except those documented as host
 *     is a device pointer owned by the caller. The library never allocates or
 *     frees device memory and never synchronises the stream.
 *   - stream: a hipStream_t passed as void* (NULL = the default stream). All
 *     work of a call is enqueued on it; ordering between calls is the caller's.
 *   - Errors: every argument check runs on the host before anything is
 *     enqueued; a rejected call enqueues nothing. A call with T == 0 (or
 *     rows == 0) returns MOE_OK and enqueues nothing. Faults inside kernels
 *     surface at the caller's next synchronisation, not as a return value.
 *   - Calls are reentrant; the library keeps no mutable state beyond a cached
 *     per-device property record (architecture check and CU count).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe_status_t;
#define MOE_OK 0
#define MOE_ERR_INVALID_ARG 1       /* null / misaligned pointer, bad size, k > E, bad block_m */
#define MOE_ERR_UNSUPPORTED_SHAPE 2 /* shape outside what the dtype's kernels support */
#define MOE_ERR_WORKSPACE 3         /* workspace too small */
#define MOE_ERR_DEVICE 4            /* no gfx950 device current, or a launch failed */

/* Numeric path of the grouped GEMMs. */
#define MOE_DTYPE_BF16 0            /* bf16 x, W; fp32 accumulate; bf16 h */
#define MOE_DTYPE_FP8_BLOCK128 1    /* E4M3 x (1x128 fp32 scales), E4M3 W (128x128 fp32 scales); E4M3 h (1x128) */
#define MOE_DTYPE_MXFP4W_MXFP8A 2   /* E4M3 x + E8M0/32, E2M1 W + E8M0/32 along K; E4M3 h + E8M0/32 */

/* Router score function. */
#define MOE_SCORE_SOFTMAX 0         /* softmax over the k selected logits (top-k renormalised) */
#define MOE_SCORE_SIGMOID 1         /* sigmoid(logit) of each selected expert, not renormalised */

/* Limits of this build. */
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 32

/*
 * moe_route -- top-k selection and gate weights per token.
 * TileScale PR #70, Design ("Kernel 1": routing happens before dispatch);
 * the weights are the softmax over the selected logits, which equals a
 * softmax over all experts renormalised over the top k.
 *
 *   logits   [T, E] fp32, device.
 *   topk_ids [T, k] int32, device, out: the k largest logits in descending
 *            order; equal logits -> the lower expert index first.
 *   topk_w   [T, k] fp32, device, out: SOFTMAX: exp(l_j - l_0) / sum_i exp(l_i - l_0);
 *            SIGMOID: 1 / (1 + exp(-l_j)).
 * Requires 1 <= E <= MOE_MAX_EXPERTS, 1 <= k <= min(E, MOE_MAX_TOPK), T >= 0,
 * finite logits. Errors: MOE_ERR_INVALID_ARG, MOE_ERR_DEVICE.
 */
moe_status_t moe_route(const float* logits, int64_t T, int32_t E, int32_t k, int32_t score,
                       int32_t* topk_ids, float* topk_w, void* stream);

/*
 * moe_route_shared -- moe_route plus shared experts: the layer's S = n_shared
 * shared experts, numbered E .. E+S-1 after the E routed ones, are used by
 * every token with weight 1 and no gate (GC-MoE on SM120, Abstract: shared
 * experts folded into the compute; TileScale PR #70, Summary: fused
 * shared-expert execution). They then run through moe_align_sort and the
 * grouped GEMMs as experts E .. E+S-1 in the same task queue, with k + S slots.
 *
 *   logits   [T, E] fp32, device: scores of the routed experts only.
 *   topk_ids [T, k+S] int32, out: slots 0..k-1 as moe_route; slot k+s = E+s.
 *   topk_w   [T, k+S] fp32, out: slots 0..k-1 as moe_route; slots k.. = 1.0f.
 * Requires n_shared >= 0, k + n_shared <= MOE_MAX_TOPK and
 * E + n_shared <= MOE_MAX_EXPERTS, otherwise as moe_route. n_shared = 0 is
 * moe_route. Errors: MOE_ERR_INVALID_ARG, MOE_ERR_DEVICE.
 */
moe_status_t moe_route_shared(const float* logits, int64_t T, int32_t E, int32_t k, int32_t score,
                              int32_t n_shared, int32_t* topk_ids, float* topk_w, void* stream);

/*
 * moe_pick_block_m -- host only. The tile height (rows per tile of the
 * expert-sorted layout) this library's kernels use for a problem, from the
 * mean number of rows per expert (the adaptive token-tile geometry named in
 * the Abstract of "GC-MoE on SM120"). Returns a value in {32, 64, 128, 256}
 * (every tile height the grouped GEMMs take), or -1 for invalid arguments.
 */
int32_t moe_pick_block_m(int32_t dtype, int64_t T, int32_t k, int32_t E, int32_t H, int32_t I);

/*
 * moe_sorted_capacity -- host only. Rows to allocate for the padded sorted
 * layout: ceil((A + min(E, A) * (block_m - 1)) / block_m) * block_m, an upper
 * bound on the padded row count whatever the routing. Returns -1 for invalid
 * arguments.
 */
int64_t moe_sorted_capacity(int64_t T, int32_t k, int32_t E, int32_t block_m);

/*
 * moe_align_sort_workspace_bytes -- host only. Device workspace bytes
 * moe_align_sort needs (0 when T == 0). Returns 0 for invalid arguments.
 */
size_t moe_align_sort_workspace_bytes(int64_t T, int32_t k, int32_t E);

/*
 * moe_align_sort -- expert-sorted, tile-padded permutation of the assignments
 * and the flat tile queue.
 * FlashInfer PR #5129, Description (padded expert-sorted rows); TileScale
 * PR #70, first commit note in the conversation (a flat m-task queue replaces
 * the per-tile expert rescan); Liger-Kernel PR #1463, Summary (empty experts).
 *
 *   topk_ids    [T, k] int32, device, values in [0, E).
 *   counts      [E] int32, out: rows routed to each expert.
 *   offsets     [E + 1] int32, out: exclusive prefix sum of the padded counts
 *               ceil(counts[e] / block_m) * block_m; offsets[E] = padded rows.
 *   sorted_ids  [cap] int32, out, cap = moe_sorted_capacity(T, k, E, block_m):
 *               rows offsets[e] .. offsets[e] + counts[e] - 1 hold the
 *               assignments routed to expert e in increasing a; every other
 *               entry (padding, and the tail past offsets[E]) holds A.
 *   tile_expert [cap / block_m] int32, out: expert of tile i (rows
 *               [i * block_m, (i + 1) * block_m)), -1 for i >= num_tiles.
 *   num_tiles   [1] int32, out (device): offsets[E] / block_m.
 *   ws          device workspace of at least
 *               moe_align_sort_workspace_bytes(T, k, E) bytes (contents
 *               undefined on entry and exit).
 * The result is deterministic (no dependence on atomic ordering). block_m 16
 * gives a valid layout, but the grouped GEMMs take 32, 64, 128 or 256 only
 * (they return MOE_ERR_UNSUPPORTED_SHAPE for 16).
 * Errors: MOE_ERR_INVALID_ARG (block_m not in {16, 32, 64, 128, 256}),
 * MOE_ERR_WORKSPACE, MOE_ERR_DEVICE. Expert ids outside [0, E) are not
 * detected on the device: the caller guarantees them (moe_route does).
 */
moe_status_t moe_align_sort(const int32_t* topk_ids, int64_t T, int32_t k, int32_t E, int32_t block_m,
                            int32_t* counts, int32_t* offsets, int32_t* sorted_ids,
                            int32_t* tile_expert, int32_t* num_tiles,
                            void* ws, size_t ws_bytes, void* stream);

/*
 * moe_align_sort_noalloc -- moe_align_sort for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same kernels and the same outputs, bit for bit,
 * with the workspace taken from a fixed scratch array the library holds in
 * device memory, one per GPU (2 MiB, kept until the process ends). The call
 * allocates nothing.
 *
 * Arguments, outputs and errors as moe_align_sort without ws / ws_bytes.
 * Limit: T * k <= MOE_NOALLOC_MAX_ASSIGNMENTS (with any E <=
 * MOE_MAX_EXPERTS); larger problems return MOE_ERR_WORKSPACE and enqueue
 * nothing. Every call on one GPU shares that GPU's scratch: calls that
 * overlap in time on one GPU (two streams, or two host threads) race and
 * must be serialised by the caller; calls ordered on one stream are safe.
 */
#define MOE_NOALLOC_MAX_ASSIGNMENTS 262144
moe_status_t moe_align_sort_noalloc(const int32_t* topk_ids, int64_t T, int32_t k, int32_t E, int32_t block_m,
                                    int32_t* counts, int32_t* offsets, int32_t* sorted_ids,
                                    int32_t* tile_expert, int32_t* num_tiles, void* stream);

/*
 * moe_quantize_fp8 -- bf16 -> FP8 E4M3 (OCP "E4M3FN", max 448) with one fp32
 * scale per block_rows x 128 block. TileScale PR #70, Design (FP8 E4M3 with
 * FP32 per-128 scales). Per block: amax = max|v|; s = fp32(amax / 448)
 * (correctly rounded), s = 1 when amax = 0; code = E4M3_RN(clamp(fp32(v / s),
 * -448, 448)), ties to even, sign of zero kept.
 *
 *   in    [rows, cols] bf16, device.
 *   q     [rows, cols] uint8 codes, out.
 *   scale [rows / block_rows, cols / 128] fp32, out.
 * block_rows is 1 (activations) or 128 (weights); rows % block_rows == 0 and
 * cols % 128 == 0, else MOE_ERR_UNSUPPORTED_SHAPE.
 */
moe_status_t moe_quantize_fp8(const uint16_t* in, int64_t rows, int64_t cols, int32_t block_rows,
                              uint8_t* q, float* scale, void* stream);

/*
 * moe_quantize_mxfp8 -- bf16 -> MXFP8 along each row: E4M3 codes with one
 * E8M0 scale per 32 consecutive columns (OCP MX v1.0 rule: X = 2^(floor(log2
 * amax) - 8), exponent clamped to [-127, 127]; byte = exponent + 127; an
 * all-zero block gets byte 0; code = E4M3_RN_SAT(v / X)). FlashInfer PR
 * #6465, Benchmark configuration (FP8 activations against K32-scaled MXFP4).
 *
 *   in [rows, cols] bf16; q [rows, cols] uint8; e8m0 [rows, cols / 32] uint8.
 * cols % 32 == 0, else MOE_ERR_UNSUPPORTED_SHAPE.
 */
moe_status_t moe_quantize_mxfp8(const uint16_t* in, int64_t rows, int64_t cols,
                                uint8_t* q, uint8_t* e8m0, void* stream);

/*
 * moe_quantize_mxfp4 -- bf16 -> MXFP4 along each row: E2M1 codes (values
 * 0, 0.5, 1, 1.5, 2, 3, 4, 6), one E8M0 scale per 32 columns (OCP MX v1.0,
 * X = 2^(floor(log2 amax) - 2)); RN ties to even, saturating at 6. FlashInfer
 * PR #6465, Benchmark configuration (E2M1 weights, one scale per 32 along K).
 *
 *   in [rows, cols] bf16; q [rows, cols / 2] uint8, two codes per byte, the
 *   even column in the low nibble; e8m0 [rows, cols / 32] uint8.
 * cols % 32 == 0, else MOE_ERR_UNSUPPORTED_SHAPE.
 */
moe_status_t moe_quantize_mxfp4(const uint16_t* in, int64_t rows, int64_t cols,
                                uint8_t* q, uint8_t* e8m0, void* stream);

/*
 * moe_grouped_gemm_swiglu -- GEMM1 (gate and up projections) of every routed
 * row and the SwiGLU, written into the padded expert-sorted row space.
 * TileScale PR #70, Design ("Kernel 1": L1 GEMM + SwiGLU, quantised
 * intermediate); FlashInfer PR #5129, Description (GEMM1 scatters into the
 * padded sorted rows).
 *
 * For each sorted row r < num_tiles * block_m with a = sorted_ids[r]:
 *   e = tile_expert[r / block_m]; x_row = x[a / k] if a < A else 0;
 *   g_n = x_row . W1[e, n, :], u_n = x_row . W1[e, I + n, :]  (fp32 accumulate)
 *   h[r, n] = silu(g_n) * u_n, stored per dtype:
 *     BF16:           h [cap, I] bf16 (RN); h_scale unused (may be NULL).
 *     FP8_BLOCK128:   h [cap, I] E4M3 codes; h_scale [cap, I / 128] fp32 (the
 *                     moe_quantize_fp8 rule, 1 x 128, applied to the fp32 h).
 *     MXFP4W_MXFP8A:  h [cap, I] E4M3 codes; h_scale [cap, I / 32] E8M0 (the
 *                     moe_quantize_mxfp8 rule applied to the fp32 h).
 *   Pad rows are written too (their h is 0). Rows past num_tiles * block_m are
 *   not touched.
 * Operands per dtype:
 *   BF16:          x [T, H] bf16; W1 [E, 2I, H] bf16; scales unused.
 *   FP8_BLOCK128:  x [T, H] E4M3 + x_scale [T, H / 128] fp32;
 *                  W1 [E*2I, H] E4M3 + w1_scale [E*2I/128, H/128] fp32.
 *   MXFP4W_MXFP8A: x [T, H] E4M3 + x_scale [T, H / 32] E8M0;
 *                  W1 [E*2I, H/2] packed E2M1 + w1_scale [E*2I, H/32] E8M0.
 * sorted_ids / tile_expert / num_tiles come from moe_align_sort with the same
 * T, k, E, block_m; cap = moe_sorted_capacity(T, k, E, block_m).
 * Shapes: BF16 needs H % 8 == 0 and I % 8 == 0; FP8 needs H % 128 == 0 and
 * I % 128 == 0; MX needs H % 128 == 0 and I % 128 == 0
 * (else MOE_ERR_UNSUPPORTED_SHAPE). block_m must be one this dtype's kernels
 * support (moe_pick_block_m returns one), else MOE_ERR_UNSUPPORTED_SHAPE.
 *
 * ws, ws_bytes: optional device workspace (NULL: none) of at least
 * moe_grouped_gemm_workspace_bytes() bytes, 256-byte aligned. Its first 8192
 * bytes are counters: zero them before the first use; every call that
 * completes leaves them zero again (the rest holds partial sums and needs no
 * clearing). With it, the BF16 kernels hand out their tiles from per-XCD
 * queues (workgroups that run faster take more tiles), and balance a short
 * last round of tiles by splitting those tiles' K sum in two halves computed
 * by two workgroups and added in fp32 (a different summation order for those
 * tiles; deterministic for a given problem and device); the FP8 / MX kernels
 * ignore it. Calls that may run at
 * the same time need workspaces of their own. ws_bytes too small ->
 * MOE_ERR_WORKSPACE; misaligned -> MOE_ERR_INVALID_ARG.
 */
moe_status_t moe_grouped_gemm_swiglu(int32_t dtype, const void* x, const void* x_scale,
                                     const void* w1, const void* w1_scale,
                                     const int32_t* sorted_ids, const int32_t* tile_expert,
                                     const int32_t* num_tiles,
                                     int64_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                                     int32_t block_m, int64_t cap,
                                     void* h, void* h_scale, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_grouped_gemm_workspace_bytes -- host only. Bytes of the optional
 * workspace of the grouped GEMM calls on the current device: 8192 bytes of
 * counters (a counter per split slot, the per-XCD queues) and two 256 x 256
 * fp32 partial tiles per slot, one slot per two workgroups of the persistent
 * grid (64 MiB on a 256-CU MI355X). Returns 0
 * when no supported device is current. Not a passage of the pages: the
 * work-balance split is this implementation's.
 */
size_t moe_grouped_gemm_workspace_bytes(void);

/*
 * moe_grouped_gemm_swiglu_h32 -- moe_grouped_gemm_swiglu that also writes
 * the fp32 intermediate before its storage rounding, for callers that check
 * that rounding (bf16 RN, or the FP8 / MXFP8 requantisation) bit for bit.
 *   h32 [cap, I] fp32, out, 16-byte aligned: for every sorted row
 *       r < num_tiles * block_m, h32[r, n] is the value silu(g_n) * u_n that
 *       the kernel rounds (BF16) or quantises (FP8_BLOCK128, MXFP4W_MXFP8A)
 *       into h[r, n] / h_scale (pad rows: 0). Rows past num_tiles * block_m
 *       are not touched.
 * h and h_scale are written exactly as moe_grouped_gemm_swiglu writes them
 * (the same kernels run; only the extra stores are added; with the same ws
 * or none alike). Other arguments and errors as moe_grouped_gemm_swiglu; h32
 * NULL or misaligned -> MOE_ERR_INVALID_ARG.
 */
moe_status_t moe_grouped_gemm_swiglu_h32(int32_t dtype, const void* x, const void* x_scale,
                                         const void* w1, const void* w1_scale,
                                         const int32_t* sorted_ids, const int32_t* tile_expert,
                                         const int32_t* num_tiles,
                                         int64_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                                         int32_t block_m, int64_t cap,
                                         void* h, void* h_scale, float* h32, void* ws, size_t ws_bytes,
                                         void* stream);

/*
 * moe_grouped_gemm_relu2 -- GEMM1 of an ungated expert with the squared-ReLU
 * activation, over the sorted rows. FlashInfer PR #5129, Tests (the sorted
 * path runs SwiGLU and ReLU2) and Measured (the Nemotron shape, ReLU2).
 *
 * As moe_grouped_gemm_swiglu, except that W1 has one projection per output
 * column and the activation is a square of the positive part:
 *   g[r, n] = sum_c x_row[c] * W1[e, n, c]   (fp32 accumulate)
 *   h[r, n] = bf16( max(g, 0)^2 )
 *   BF16 only: x [T, H] bf16; W1 [E, I, H] bf16; h [cap, I] bf16; x_scale,
 *   w1_scale and h_scale are ignored (pass NULL).
 * ws, ws_bytes and errors as for moe_grouped_gemm_swiglu; dtype other than
 * BF16 -> MOE_ERR_UNSUPPORTED_SHAPE.
 */
moe_status_t moe_grouped_gemm_relu2(int32_t dtype, const void* x, const void* x_scale,
                                    const void* w1, const void* w1_scale,
                                    const int32_t* sorted_ids, const int32_t* tile_expert,
                                    const int32_t* num_tiles,
                                    int64_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                                    int32_t block_m, int64_t cap,
                                    void* h, void* h_scale, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_grouped_gemm_down -- GEMM2 (down projection) over the sorted rows; the
 * epilogue writes each real row to assignment order and drops pad rows.
 * FlashInfer PR #5129, Description (GEMM2 loads its A tiles contiguously and
 * scatters to assignment order); TileScale PR #70, Design ("Kernel 2": rows
 * land in a (token, top-k slot) workspace).
 *
 * For each sorted row r < num_tiles * block_m with a = sorted_ids[r] < A:
 *   y[a, c] = bf16( sum_i h_hat[r, i] * W2_hat[e, c, i] ), fp32 accumulate,
 * where h_hat / W2_hat are the dequantised operands:
 *   BF16:          h [cap, I] bf16; W2 [E, H, I] bf16.
 *   FP8_BLOCK128:  h [cap, I] E4M3 + h_scale [cap, I/128] fp32;
 *                  W2 [E*H, I] E4M3 + w2_scale [E*H/128, I/128] fp32.
 *   MXFP4W_MXFP8A: h [cap, I] E4M3 + h_scale [cap, I/32] E8M0;
 *                  W2 [E*H, I/2] packed E2M1 + w2_scale [E*H, I/32] E8M0.
 *   y [A, H] bf16, out: every row a < A is written exactly once.
 * Shape rules, ws and ws_bytes as for moe_grouped_gemm_swiglu (GEMM1 and
 * GEMM2 on one stream may share one workspace).
 */
moe_status_t moe_grouped_gemm_down(int32_t dtype, const void* h, const void* h_scale,
                                   const void* w2, const void* w2_scale,
                                   const int32_t* sorted_ids, const int32_t* tile_expert,
                                   const int32_t* num_tiles,
                                   int64_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                                   int32_t block_m, int64_t cap,
                                   uint16_t* y, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_down_combine_workspace_bytes -- host only. Bytes of the counter
 * workspace moe_grouped_gemm_down_combine needs: T * ceil(H / 128) int32.
 * Returns 0 for invalid arguments.
 */
size_t moe_down_combine_workspace_bytes(int64_t T, int32_t H);

/*
 * moe_grouped_gemm_down_combine -- moe_grouped_gemm_down with the weighted
 * top-k combine fused into its epilogue (TileScale PR #70, Design: "Kernel
 * 2" runs the L2 GEMM, the scatter to (token, slot) rows and the reduce).
 *
 * Writes y exactly as moe_grouped_gemm_down without a workspace (the last
 * round of tiles is never split along K here) and, in the same launch,
 *   out[t, c] = bf16( sum_{j = 0..k-1} topk_w[t, j] * y[t*k + j, c] ),
 * the result moe_combine gives, bit for bit: the workgroup that stores the
 * last of a token's k rows for a block of columns sums that block in fp32 in
 * slot order. The order in which workgroups finish does not change any value.
 *   topk_w [T, k] fp32; out [T, H] bf16 (16-byte aligned);
 *   counters: device workspace of at least
 *     moe_down_combine_workspace_bytes(T, H) bytes, int32-aligned, which
 *     must hold zeros before the call; every call leaves it zero again, so
 *     clear it once when it is allocated. Two calls that overlap in time must
 *     not share a workspace.
 * BF16 only, and y below 2 GiB (T * k * H * 2 bytes: the kernel addresses it
 * with 32-bit offsets); otherwise MOE_ERR_UNSUPPORTED_SHAPE. Other arguments
 * and errors as moe_grouped_gemm_down; a workspace below the size ->
 * MOE_ERR_WORKSPACE.
 */
moe_status_t moe_grouped_gemm_down_combine(int32_t dtype, const void* h, const void* h_scale,
                                           const void* w2, const void* w2_scale,
                                           const int32_t* sorted_ids, const int32_t* tile_expert,
                                           const int32_t* num_tiles,
                                           int64_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                                           int32_t block_m, int64_t cap,
                                           uint16_t* y, const float* topk_w, uint16_t* out,
                                           int32_t* counters, size_t counters_bytes, void* stream);

/*
 * moe_combine -- top-k weighted sum of each token's expert rows.
 * TileScale PR #70, review thread on the reduce tail (sum over the top-k
 * slots into the BF16 output); FlashInfer PR #5129, Description (the combine
 * after the sorted GEMM2 is unchanged).
 *
 *   out[t, c] = bf16( sum_{j = 0..k-1} topk_w[t, j] * y[t*k + j, c] ), summed in
 *   fp32 in slot order, rounded to nearest even.
 *   y [T*k, H] bf16; topk_w [T, k] fp32; out [T, H] bf16.
 * Requires H % 8 == 0 (MOE_ERR_UNSUPPORTED_SHAPE otherwise).
 */
moe_status_t moe_combine(const uint16_t* y, const float* topk_w, int64_t T, int32_t k, int32_t H,
                         uint16_t* out, void* stream);

/* ------------------------------------------------------------------------
 * Backward of the BF16 SwiGLU routed forward (training). Liger-Kernel PR
 * #1463, Summary (SM90 backward) and "MoEBenchmark results" (forward and
 * backward throughput of the BF16 routed-expert MLP): the gradients run over
 * the same padded expert-sorted rows and tile queue as the forward.
 *
 * One training step:
 *   forward:  moe_route -> moe_align_sort -> moe_grouped_gemm_swiglu_save
 *             -> moe_grouped_gemm_down -> moe_combine
 *   backward: moe_backward_combine (dY, dw) -> moe_route_backward (dlogits)
 *             -> moe_grouped_gemm_dh (dGU) -> moe_grouped_gemm_dx (dx rows)
 *             -> moe_combine with unit weights (dx)
 *             -> moe_gather_rows (x in sorted rows)
 *             -> moe_grouped_gemm_wgrad twice (dW2: P = h, Q = dY;
 *                dW1: P = x_sorted, Q = dGU)
 * The GEMM steps need block_m == 256 (else MOE_ERR_UNSUPPORTED_SHAPE);
 * the elementwise steps take any block_m. Shape rules otherwise as for the
 * BF16 forward (H % 8 == 0, I % 8 == 0; one expert's W1 and every sorted-row
 * operand below 2 GiB).
 * ---------------------------------------------------------------------- */

/*
 * moe_grouped_gemm_swiglu_save -- the BF16 moe_grouped_gemm_swiglu that also
 * stores the pre-activations the SwiGLU backward needs.
 *   gu [cap, 2I] bf16, out: gu[r, n] = bf16(g_n), gu[r, I + n] = bf16(u_n) for
 *   every sorted row r < num_tiles * block_m (pad rows: 0).
 * Other arguments, outputs and errors as moe_grouped_gemm_swiglu with
 * dtype = MOE_DTYPE_BF16; gu NULL or not 16-byte aligned -> MOE_ERR_INVALID_ARG.
 */
moe_status_t moe_grouped_gemm_swiglu_save(const void* x, const void* w1,
                                          const int32_t* sorted_ids, const int32_t* tile_expert,
                                          const int32_t* num_tiles,
                                          int64_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                                          int32_t block_m, int64_t cap,
                                          void* h, void* gu, void* stream);

/*
 * moe_backward_combine -- backward of moe_combine, per sorted row.
 *   For each sorted row r < num_tiles * block_m with a = sorted_ids[r]
 *   (t = a / k):
 *     dy[r, c] = bf16( topk_w[a] * dout[t, c] ) if a < A, else 0;
 *     dw[a]    = sum_c dout[t, c] * y[a, c] (fp32, each real a once).
 *   dout [T, H] bf16; topk_w [T, k] fp32; y [T*k, H] bf16 (the forward's
 *   GEMM2 rows); sorted_ids [cap] int32, num_tiles (device int32) from
 *   moe_align_sort with the same block_m; dy [cap, H] bf16 out (rows past
 *   num_tiles * block_m are not written); dw [T, k] fp32 out.
 * Requires H % 8 == 0.
 */
moe_status_t moe_backward_combine(const uint16_t* dout, const float* topk_w, const uint16_t* y,
                                  const int32_t* sorted_ids, const int32_t* num_tiles, int64_t T, int32_t k,
                                  int32_t H, int32_t block_m, int64_t cap, uint16_t* dy, float* dw, void* stream);

/*
 * moe_route_backward -- gradient of the router logits from the gradient of
 * the top-k gate weights (the routed slots only; shared slots have weight 1
 * and no gradient).
 *   For token t and routed expert e = topk_ids[t, j] (j < k):
 *     softmax: dlogits[t, e] = w_j (dw_j - sum_{q<k} w_q dw_q)
 *     sigmoid: dlogits[t, e] = dw_j w_j (1 - w_j)
 *   and dlogits[t, e] = 0 for every expert not selected.
 *   topk_w, dw [T, k + n_shared] fp32; topk_ids [T, k + n_shared] int32;
 *   dlogits [T, E] fp32 out (E routed experts).
 */
moe_status_t moe_route_backward(const float* topk_w, const int32_t* topk_ids, const float* dw, int64_t T,
                                int32_t E, int32_t k, int32_t n_shared, int32_t score, float* dlogits,
                                void* stream);

/*
 * moe_gather_rows -- the tokens in sorted-row order (the token operand of the
 * W1 weight gradient): x_sorted[r, :] = x[sorted_ids[r] / k, :] for real rows,
 * 0 for pad rows, every r < num_tiles * block_m (later rows are not written).
 *   x [T, H] bf16; sorted_ids [cap] int32 and num_tiles (device int32) from
 *   moe_align_sort with the same block_m; x_sorted [cap, H] bf16 out.
 * Requires H % 8 == 0.
 */
moe_status_t moe_gather_rows(const uint16_t* x, const int32_t* sorted_ids, const int32_t* num_tiles, int64_t T,
                             int32_t k, int32_t H, int32_t block_m, int64_t cap, uint16_t* x_sorted, void* stream);

/*
 * moe_grouped_gemm_dh -- gradient through GEMM2 and the SwiGLU, per sorted
 * row r < num_tiles * block_m of expert e = tile_expert[r / block_m]:
 *   dh[r, i]     = sum_c dy[r, c] W2[e, c, i]          (fp32 accumulate)
 *   s = sigmoid(g), with (g, u) = gu[r, i], gu[r, I + i]:
 *   dgu[r, i]     = bf16( dh u s (1 + g (1 - s)) )
 *   dgu[r, I + i] = bf16( dh g s )
 *   dy [cap, H] bf16 (moe_backward_combine); W2 [E, H, I] bf16; gu [cap, 2I]
 *   bf16 (moe_grouped_gemm_swiglu_save); dgu [cap, 2I] bf16 out.
 * block_m must be 256.
 */
moe_status_t moe_grouped_gemm_dh(const void* dy, const void* w2, const void* gu, const int32_t* sorted_ids,
                                 const int32_t* tile_expert, const int32_t* num_tiles, int64_t T, int32_t H,
                                 int32_t I, int32_t E, int32_t k, int32_t block_m, int64_t cap, void* dgu,
                                 void* stream);

/*
 * moe_grouped_gemm_dx -- gradient through GEMM1 to each assignment's row:
 *   for each sorted row r < num_tiles * block_m with a = sorted_ids[r] < A:
 *     dx_rows[a, c] = bf16( sum_n dgu[r, n] W1[e, n, c] ), n over [0, 2I).
 *   dgu [cap, 2I] bf16; W1 [E, 2I, H] bf16; dx_rows [T*k, H] bf16 out
 *   (every row a < A written once). Summing each token's k rows
 *   (moe_combine with topk_w = 1) gives dx.
 * block_m must be 256.
 */
moe_status_t moe_grouped_gemm_dx(const void* dgu, const void* w1, const int32_t* sorted_ids,
                                 const int32_t* tile_expert, const int32_t* num_tiles, int64_t T, int32_t H,
                                 int32_t I, int32_t E, int32_t k, int32_t block_m, int64_t cap, void* dx_rows,
                                 void* stream);

/*
 * moe_grouped_gemm_wgrad -- per-expert weight gradient over the expert's
 * sorted rows r in [offsets[e], offsets[e + 1]):
 *   dw[e, n, m] = sum_r p_rows[r, m] q_rows[r, n]      (fp32 accumulate, fp32 out)
 *   p_rows [cap, M] bf16; q_rows [cap, N] bf16; offsets [E + 1] int32 from
 *   moe_align_sort; dw [E, N, M] fp32 out (experts without rows get 0).
 *   dW2 [E, H, I]: p = h, q = dy, M = I, N = H.
 *   dW1 [E, 2I, H]: p = x_sorted, q = dgu, M = H, N = 2I.
 * Pad rows must be 0 in p or q (they are, for the operands above).
 * Requires M % 8 == 0, N % 8 == 0, block_m == 256, 16-byte aligned pointers.
 */
moe_status_t moe_grouped_gemm_wgrad(const void* p_rows, const void* q_rows, int32_t M, int32_t N,
                                    const int32_t* offsets, int64_t T, int32_t E, int32_t k, int32_t block_m,
                                    int64_t cap, float* dw, void* stream);

/* Human-readable name of a status code (static storage). */
const char* moe_status_string(moe_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
