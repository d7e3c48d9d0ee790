/*
 * moe.h - C ABI of libmoe: the forward pass of a dropless Mixture-of-Experts layer
 * on one AMD Instinct MI355X (gfx950).
 *
 * The layer, as the pages state the problem:
 *   x[T, d] tokens, router W_g[d, E], each token picks k of E experts; expert e is a
 *   SwiGLU MLP with W1[e], W3[e] of shape [d, d_e] and W2[e] of shape [d_e, d];
 *   an optional shared expert (same form, inner size d_e_shared) sees every token.
 *   (TileLang tutorial chapter "MoE, MLA and sparse-attention operators", sections
 *   2.1-2.5; course notes "Dropless and grouped GEMM", sections 1 and 4.)
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is device memory owned by the caller, row-major and
 *     contiguous, 16-byte aligned.  The library never allocates, frees or
 *     synchronises; every kernel is enqueued on `stream` (a hipStream_t; NULL is
 *     the null stream) and the caller synchronises.  Nothing is copied between
 *     host and device: counts and offsets stay in device memory.
 *   - Activations and weights are fp32 (dtype 0) or bf16 (dtype 1); router
 *     logits, routing weights and all accumulation are fp32; integer outputs are
 *     int32.
 *   - Host-side validation runs before anything is enqueued and returns a status;
 *     MOE_EHIP reports a failed kernel launch.  A data error that only the device
 *     can see (an expert id outside [0, E) handed to moe_build_offsets) sets
 *     *err_flag to 1 on the device; the outputs are then unspecified.
 *   - Results are bitwise reproducible run to run: no floating-point atomics, and
 *     every reduction has a fixed order.
 *   - Entry points are reentrant; the library keeps no mutable global state (a
 *     debug build keeps one word per device, see moe_debug_flags).
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe_status;
#define MOE_OK          0
#define MOE_EINVAL      1   /* a shape, pointer, alignment or argument is invalid   */
#define MOE_ENOTSUP     2   /* valid, but not supported by this library (see below) */
#define MOE_EWORKSPACE  3   /* workspace missing or smaller than moe_workspace_bytes */
#define MOE_EHIP        4   /* a HIP launch or runtime call failed                   */

#define MOE_DTYPE_F32   0
#define MOE_DTYPE_BF16  1

#define MOE_OP_GATEUP_SWIGLU 0   /* act = silu(A W1[e]) * (A W3[e]), [rows, d_e] */
#define MOE_OP_DOWN          1   /* y   = A W2[e],                   [rows, d]   */

/*
 * The layer's shape.
 *   T >= 0 tokens (T == 0 is a no-op); d, d_e >= 1 with d % 8 == 0 and d_e % 8 == 0
 *   (bf16) or % 4 == 0 (fp32); 1 <= E <= 1024; 1 <= k <= 1024; T * k < 2^31, and
 *   the block-table bound times block_m < 2^31, for the padded bound of moe_max_blocks
 *   and, unpadded, for the unpadded one too (MOE_EINVAL otherwise).  The
 *   router picks k distinct experts, so routing (moe_route, moe_layer_fwd without
 *   given routes) needs k <= E; rows routed elsewhere may repeat an expert within a
 *   token (k > E is then allowed).
 *   n_groups, topk_groups: 0, 0 for plain top-k; otherwise E % n_groups == 0,
 *   1 <= topk_groups <= n_groups <= 64, and routing needs k <= topk_groups * E /
 *   n_groups (group-limited
 *   routing: experts form n_groups contiguous id ranges, a group scores its largest
 *   logit, only the topk_groups best groups stay eligible; TileLang chapter section
 *   2.2, dropless notes section 4 step 4).
 *   renormalize: 1 divides the k routing weights of a token by their sum.
 *   block_m: every expert's row segment is padded up to a multiple of block_m
 *   (dropless notes section 3); it is also the row granularity of the grouped GEMM.
 *   bf16 needs block_m % 128 == 0 (else MOE_ENOTSUP); fp32 takes any block_m >= 1.
 *   d_e_shared: inner size of the shared expert, 0 = none.
 *   unpadded: 0 = the padded layout above.  1 = unpadded segments (dropless notes
 *   section 11): expert e keeps rows [offsets[e], offsets[e+1]) of the T*k rows with no
 *   padding, the row space is cut into block_m-row tiles, and a tile holding rows of
 *   several experts gets one block-table entry per expert (executed once for each,
 *   restricted to that expert's rows).  Every permuted buffer then has T*k rows.
 */
typedef struct moe_shape {
  int32_t T, d, E, k, d_e;
  int32_t n_groups, topk_groups;
  int32_t renormalize;
  int32_t block_m;
  int32_t d_e_shared;
  int32_t dtype;
  int32_t unpadded;
} moe_shape;

/* Human-readable name of a status code (static storage). */
const char* moe_status_str(moe_status s);

/* Host-only and pure.  Upper bound on the number of block-table entries: padded,
 * sum_e ceil(c_e / block_m) <= floor((T*k + min(E, T*k) * (block_m - 1)) / block_m);
 * unpadded, tiles + (experts with rows) - 1 <= ceil(T*k / block_m) + min(E, T*k) - 1.
 * Returns -1 for an invalid shape. */
int32_t moe_max_blocks(const moe_shape* s);

/* Host-only and pure.  The row count every permuted buffer (x_perm, act, y, row_src)
 * is sized at: padded, moe_max_blocks(s) * block_m - a declared upper bound, since the
 * real padded total is data (dropless notes sections 1 and 4); unpadded, T*k.
 * -1 if invalid. */
int64_t moe_max_rows(const moe_shape* s);

/* Host-only and pure.  Bytes of device workspace that moe_layer_fwd needs; the same
 * amount is enough for moe_route and moe_build_offsets.  0 if the shape is invalid. */
size_t moe_workspace_bytes(const moe_shape* s);

/*
 * Router and selection (TileLang chapter section 2.2; dropless notes section 4
 * steps 2-4).
 *   logits[t, e] = sum_i x[t, i] * w_gate[i, e] + bias[e], accumulated in fp32.
 *   Selection runs on those fp32 logits: within the eligible experts, k rounds of
 *   "largest remaining logit", ties to the lower expert id, so slot j holds the
 *   j-th largest.  topk_w[t, j] = softmax over all E logits at topk_idx[t, j],
 *   divided by the sum of the token's k weights when renormalize is set.
 * In:  x [T, d] (dtype), w_gate [d, E] (dtype), bias [E] fp32 or NULL; x and w_gate
 *      16-byte aligned (MOE_EINVAL otherwise, as for moe_layer_fwd and
 *      moe_layer_fwd_fp8, which take the same w_gate).
 * Out: logits [T, E] fp32 (NULL: not stored), topk_idx [T, k] int32,
 *      topk_w [T, k] fp32.
 * ws:  device workspace of ws_bytes >= moe_workspace_bytes(s).
 */
moe_status moe_route(const moe_shape* s, const void* x, const void* w_gate,
                     const float* bias, float* logits, int32_t* topk_idx,
                     float* topk_w, void* ws, size_t ws_bytes, void* stream);

/*
 * Counts, offsets, padded offsets, block metadata and the permutation, all on the
 * device (TileLang chapter sections 2.2 item 2, 2.3 item 2 and 2.4 (a); dropless
 * notes sections 3, 5 and 7).  With a = t*k + j and c_e the number of assignments
 * with expert e:
 *   counts[e]            = c_e
 *   offsets[e]           = sum_{e' < e} c_e'                  (E+1 entries)
 *   padded_offsets[e]    = sum_{e' < e} ceil(c_e'/block_m)*block_m  (E+1 entries)
 *   num_blocks[0]        = sum_e ceil(c_e / block_m)
 *   block_meta[b]        = {expert, m_start, valid_m} for b < num_blocks, experts in
 *                          ascending order, m_start = padded_offsets[e] + i*block_m,
 *                          valid_m = min(block_m, c_e - i*block_m); entries from
 *                          num_blocks to max_blocks-1 are left untouched
 * With s->unpadded: padded_offsets = offsets; the block table lists, tile by tile
 * (tiles [i*block_m, (i+1)*block_m) of the T*k rows) and inside a tile by expert, one
 * entry per expert with rows in the tile: m_start = its first row there, valid_m its
 * row count there; num_blocks = the number of entries (dropless notes section 11).
 *   pos[a]               = padded_offsets[e] + #{a' < a : topk_idx[a'] = e}
 *                          (a stable sort by expert id)
 *   row_src[r]           = a where pos[a] = r, -1 on every other row r < max_rows
 *   err_flag[0]          = 1 if any id lies outside [0, E) (those assignments are
 *                          skipped and get pos = -1), else 0
 * In:  topk_idx [T*k] int32 (duplicates within a token are allowed).
 * Out: counts [E], offsets [E+1], padded_offsets [E+1], block_meta
 *      [moe_max_blocks(s)][3], num_blocks [1], pos [T*k], row_src [moe_max_rows(s)],
 *      err_flag [1], all int32.
 * ws:  device workspace of ws_bytes >= moe_workspace_bytes(s).
 */
moe_status moe_build_offsets(const moe_shape* s, const int32_t* topk_idx,
                             int32_t* counts, int32_t* offsets,
                             int32_t* padded_offsets, int32_t* block_meta,
                             int32_t* num_blocks, int32_t* pos, int32_t* row_src,
                             int32_t* err_flag, void* ws, size_t ws_bytes,
                             void* stream);

/*
 * moe_build_offsets without a workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same inputs, outputs, results (bit for bit) and errors as moe_build_offsets; its
 * scratch (per-chunk histograms and per-assignment local ranks,
 * moe_build_offsets_scratch_bytes(s) bytes) lives in a device array inside the library,
 * moe_build_offsets_noalloc_capacity() = 8 MiB on each device, held from the first call
 * on that device until the process ends.  The call allocates nothing.
 *   - MOE_ENOTSUP when moe_build_offsets_scratch_bytes(s) exceeds the capacity (about
 *     T*k <= 2,000,000 assignments for E <= 1024); nothing is launched then.
 *   - MOE_EHIP if the array's device address cannot be obtained.
 *   - Every call on one device uses that device's one array: calls that overlap in time
 *     on the same device (another stream, another host thread) race and give undefined
 *     results.  Calls in one stream, one after another, are safe: nothing in the array
 *     needs to start at zero, every entry read is first written by the same call.
 */
moe_status moe_build_offsets_noalloc(const moe_shape* s, const int32_t* topk_idx,
                                     int32_t* counts, int32_t* offsets,
                                     int32_t* padded_offsets, int32_t* block_meta,
                                     int32_t* num_blocks, int32_t* pos, int32_t* row_src,
                                     int32_t* err_flag, void* stream);
/* Host-only and pure: the static scratch's size in bytes, and the scratch bytes a shape
 * needs (0 for an invalid shape). */
size_t moe_build_offsets_noalloc_capacity(void);
size_t moe_build_offsets_scratch_bytes(const moe_shape* s);

/*
 * Permute (in-card dispatch; TileLang chapter section 2.3, dropless notes section 4
 * steps 5-6): x_perm[pos[t*k + j], :] = x[t, :] for every (t, j) with pos >= 0.
 * Pad rows of x_perm are neither written nor read.
 * In:  x [T, d] (dtype), pos [T*k] int32.  Out: x_perm [moe_max_rows(s), d] (dtype).
 */
moe_status moe_permute(const moe_shape* s, const void* x, const int32_t* pos,
                       void* x_perm, void* stream);

/*
 * Grouped GEMM over the contiguous, block_m-aligned expert segments (TileLang
 * chapter section 2.4; dropless notes sections 3, 5 and 7): one launch covers every
 * expert; block b of block_meta computes rows [m_start, m_start + valid_m) against
 * expert `expert`'s weights only.  Rows past valid_m are neither read nor written.
 *   op = MOE_OP_GATEUP_SWIGLU: A = x_perm [rows, d], B0 = W1 [E, d, d_e] (gate),
 *        B1 = W3 [E, d, d_e] (up); C = act [rows, d_e] = silu(A W1[e]) * (A W3[e]),
 *        the dual GEMM sharing one read of A with a fused SiLU-and-multiply epilogue
 *        (TileLang chapter section 2.4 (c)).
 *   op = MOE_OP_DOWN: A = act [rows, d_e], B0 = W2 [E, d_e, d], B1 = NULL;
 *        C = y [rows, d] = A W2[e].
 * block_meta and num_blocks are device pointers (as written by moe_build_offsets);
 * max_blocks (host) bounds num_blocks and sizes the launch, so the host never needs
 * the real block count; 1 <= max_blocks <= moe_max_blocks(s).  A and C hold
 * max_blocks * block_m rows.
 * Dense mode (the shared expert, dropless notes section 1): block_meta and
 * num_blocks both NULL and max_blocks == 0.  A and C then hold s->T rows, every row
 * goes through one expert (B0, B1 point at a single [d, d_e] or [d_e, d] matrix) and
 * s->E, s->k are not used.  This is the launch moe_layer_fwd makes for the shared
 * expert, with d_e = d_e_shared.
 * Errors: MOE_EINVAL for a bad op, NULL or misaligned operands, or a max_blocks
 * outside the range above; nothing is launched then.
 */
moe_status moe_grouped_gemm(const moe_shape* s, int32_t op, const void* A,
                            const void* B0, const void* B1,
                            const int32_t* block_meta, const int32_t* num_blocks,
                            int32_t max_blocks, void* C, void* stream);

/*
 * The grouped GEMM of the routed experts and the shared expert in one call
 * (dropless notes section 1: the shared expert is a dense MLP on every token, next
 * to the routed ones).  The routed half is exactly moe_grouped_gemm with a block
 * table; the shared half is its dense mode over the T unpermuted rows:
 *   op = MOE_OP_GATEUP_SWIGLU: A_shared = x [T, d], B0_shared = Ws1 [d, d_e_shared],
 *        B1_shared = Ws3 [d, d_e_shared]; C_shared = [T, d_e_shared].
 *   op = MOE_OP_DOWN: A_shared = [T, d_e_shared], B0_shared = Ws2 [d_e_shared, d],
 *        B1_shared = NULL; C_shared = [T, d].
 * When d_e_shared == d_e both halves run in one launch, so a small T (decode) does
 * not leave the shared expert's few row blocks alone on the chip; otherwise they
 * run back to back.  Requires s->d_e_shared > 0.  This is the call moe_layer_fwd
 * makes for each op.
 * Errors: MOE_EINVAL for a bad op, d_e_shared == 0, NULL or misaligned operands, or
 * a block table as moe_grouped_gemm rejects it; nothing is launched then.
 */
moe_status moe_grouped_gemm_shared(const moe_shape* s, int32_t op, const void* A,
                                   const void* B0, const void* B1,
                                   const int32_t* block_meta, const int32_t* num_blocks,
                                   int32_t max_blocks, void* C, const void* A_shared,
                                   const void* B0_shared, const void* B1_shared,
                                   void* C_shared, void* stream);

/*
 * Gate/up grouped GEMM with the permute fused into its A-operand loads (direct
 * gather; dropless notes section 4 steps 5-7: the permutation only decides which
 * token row each GEMM row reads).  Identical to permuting x with moe_permute and
 * calling moe_grouped_gemm(_shared) with MOE_OP_GATEUP_SWIGLU, bit for bit, without
 * writing or reading x_perm: row r of the block table's segments reads
 * x[row_src[r] / k, :] for r below its block's valid_m.
 * In:  x [T, d] (bf16), row_src [moe_max_rows(s)] int32 (as written by
 *      moe_build_offsets), w1, w3 [E, d, d_e], the block table as for
 *      moe_grouped_gemm; when d_e_shared > 0 also ws1, ws3 [d, d_e_shared] (the
 *      shared expert over the same x, as moe_grouped_gemm_shared), else NULLs.
 * Out: act [moe_max_rows(s), d_e]; shared_act [T, d_e_shared] when d_e_shared > 0.
 * Errors: MOE_ENOTSUP unless dtype is bf16, d % 32 == 0 and T * d * 2 + 4096 < 2^32
 *      (the byte offsets of gathered rows); MOE_EINVAL as for moe_grouped_gemm.
 *      Nothing is launched then.
 */
moe_status moe_grouped_gemm_gather(const moe_shape* s, const void* x,
                                   const int32_t* row_src, const void* w1,
                                   const void* w3, const int32_t* block_meta,
                                   const int32_t* num_blocks, int32_t max_blocks,
                                   void* act, const void* ws1, const void* ws3,
                                   void* shared_act, void* stream);

/*
 * Combine (TileLang chapter section 2.5; dropless notes section 4 steps 10-11):
 *   out[t, :] = sum_{j = 0..k-1, in this order} topk_w[t, j] * y[pos[t*k + j], :]
 *               (+ shared_out[t, :])
 * accumulated in fp32 and rounded once to dtype; slots with pos < 0 are skipped.
 * In:  y [moe_max_rows(s), d] (dtype), pos [T*k] int32, topk_w [T, k] fp32 or NULL
 *      (unit weights: the sum of each token's k rows, which is the backward of the
 *      permute), shared_out [T, d] (dtype) or NULL.   Out: out [T, d] (dtype).
 */
moe_status moe_combine(const moe_shape* s, const void* y, const int32_t* pos,
                       const float* topk_w, const void* shared_out, void* out,
                       void* stream);

/*
 * The whole layer: route -> build offsets -> permute -> grouped GEMM (gate/up with
 * SiLU*mul, with the shared expert's gate/up on the unpermuted x when there is one)
 * -> grouped GEMM (down, likewise) -> combine.  Where moe_grouped_gemm_gather
 * applies (bf16, d % 32 == 0), the permute is fused into the gate/up loads and
 * x_perm is not written.  The shared expert is a dense SwiGLU MLP on every token,
 * added unweighted (dropless notes section 1).
 * In:  x [T, d]; w_gate [d, E] and bias [E] fp32 (or NULL) when routing;
 *      w1, w3 [E, d, d_e], w2 [E, d_e, d];
 *      ws1, ws3 [d, d_e_shared], ws2 [d_e_shared, d] when d_e_shared > 0 (else NULL);
 *      topk_idx_in [T, k] int32 and topk_w_in [T, k] fp32: when both are non-NULL the
 *      router is skipped and these routes are used as given (rows already routed,
 *      as on one rank of an expert-parallel group); w_gate may then be NULL.
 * Out: out [T, d] (dtype).
 * ws:  device workspace of ws_bytes >= moe_workspace_bytes(s); it holds every
 *      intermediate, laid out by moe_ws_layout.
 */
moe_status moe_layer_fwd(const moe_shape* s, const void* x, const void* w_gate,
                         const float* bias, const void* w1, const void* w3,
                         const void* w2, const void* ws1, const void* ws3,
                         const void* ws2, const int32_t* topk_idx_in,
                         const float* topk_w_in, void* out, void* ws,
                         size_t ws_bytes, void* stream);

/*
 * fp8 expert weights (dropless notes section 12: fp8 weights with a scale per
 * quantisation block).  Format: OCP 8-bit floating point E4M3 ("e4m3fn": bias 7, no
 * infinities, 0x7F / 0xFF are NaN, largest finite value 448), one byte per weight in
 * the bf16 weight's [E, K, N] layout; one fp32 scale per 128 x 128 block,
 * scales[E][ceil(K/128)][ceil(N/128)].  The weight is code value * scale.
 */

/*
 * Quantise bf16 expert matrices w [E, K, N] to fp8: per 128 x 128 block (partial at
 * the edges), scale = amax / 448 in fp32 (1 for an all-zero block), code =
 * clamp(w / scale, -448, 448) in fp32, rounded to the nearest e4m3 value (ties to
 * even).  Requires N % 8 == 0; q 8-byte aligned, w 16-byte aligned.
 * Out: q [E, K, N] uint8, scales [E, ceil(K/128), ceil(N/128)] fp32.
 * Errors: MOE_EINVAL for bad sizes or pointers; nothing is launched then.
 */
moe_status moe_quantize_fp8(int32_t E, int32_t K, int32_t N, const void* w, uint8_t* q,
                            float* scales, void* stream);

/*
 * The inverse map of moe_quantize_fp8's format: w[e][i][j] = bf16(fp32(code) * scale
 * of its 128 x 128 block), the product rounded to nearest even - the same bf16 value
 * that moe_grouped_gemm_fp8 builds in registers for each weight before its MFMA.
 * q [E, K, N] uint8 (8-byte aligned), scales [E, ceil(K/128), ceil(N/128)] fp32,
 * w [E, K, N] bf16 (16-byte aligned, caller-owned).  Requires N % 8 == 0.
 * Errors: MOE_EINVAL for bad sizes or pointers; nothing is launched then.
 */
moe_status moe_dequantize_fp8(int32_t E, int32_t K, int32_t N, const uint8_t* q,
                              const float* scales, void* w, void* stream);

/*
 * The grouped GEMM (as moe_grouped_gemm, one op per call) with fp8 weights:
 * B0 / B1 are (Q0, S0) / (Q1, S1) code and scale arrays of W1 / W3 (gate/up) or W2
 * (down: Q1 = S1 = NULL).  Each 16-deep weight fragment is dequantised to bf16
 * (code * scale, rounded to nearest even) just before the bf16 MFMA; accumulation and
 * the epilogue are fp32, outputs bf16.  The tiling follows the rows per expert
 * (M = T * k over min(E, M) experts): at most 64 on average, 64-row items with wide
 * weight rows (weight streaming); at least 256, the 384-row groups of moe_grouped_gemm's
 * wide kernel (bitwise the same as that kernel on moe_dequantize_fp8's weights); in
 * between, 128-row items.
 * row_src: NULL (A is x_perm) or, for op == MOE_OP_GATEUP_SWIGLU only, the
 * permutation, so that A is x [T, d] and row r reads x[row_src[r] / k] (the permute
 * fused into the loads, as moe_grouped_gemm_gather).
 * A_shared, Q0_shared, S0_shared, Q1_shared, S1_shared, C_shared: all NULL, or the
 * shared expert (needs d_e_shared > 0) as moe_grouped_gemm_shared's second half.
 * ws, ws_bytes: NULL, or device scratch of moe_grouped_gemm_fp8_workspace_bytes(s) bytes
 * (16-byte aligned; MOE_EWORKSPACE if smaller).  With it, the 64-row (weight-streaming)
 * kernel splits the items of its persistent grid's last, partly filled round along the
 * contraction across every work group, then adds each item's pieces in a fixed order
 * in a second small launch, where every block of the table holds at most 64 rows
 * (decode); the results do not depend on timing, only on the device's compute-unit
 * count (which sets the split).  Without it every item runs whole.
 * Requires dtype bf16, block_m == 128, d and d_e (and d_e_shared) multiples of 32,
 * at most 32768 (else MOE_ENOTSUP); the block table as for moe_grouped_gemm.
 */
moe_status moe_grouped_gemm_fp8(const moe_shape* s, int32_t op, const void* A,
                                const uint8_t* Q0, const float* S0, const uint8_t* Q1,
                                const float* S1, const int32_t* block_meta,
                                const int32_t* num_blocks, int32_t max_blocks,
                                const int32_t* row_src, void* C, const void* A_shared,
                                const uint8_t* Q0_shared, const float* S0_shared,
                                const uint8_t* Q1_shared, const float* S1_shared,
                                void* C_shared, void* ws, size_t ws_bytes, void* stream);
/* Host-only and pure: the optional scratch of moe_grouped_gemm_fp8 (two 64-row x 1024
 * fp32 slots for each of up to 256 work groups, behind a 256-byte header: 128 MiB + 256
 * bytes), 0 for an invalid shape. */
size_t moe_grouped_gemm_fp8_workspace_bytes(const moe_shape* s);

/*
 * moe_layer_fwd with fp8 weights: (q1, s1), (q3, s3), (q2, s2) replace w1, w3, w2 and
 * (qs1, ss1), (qs3, ss3), (qs2, ss2) the shared expert's (NULLs when d_e_shared == 0).
 * Same pipeline and requirements as moe_grouped_gemm_fp8.  Where the routed rows
 * M = T * k reach 256 * min(E, M) (experts average at least 256 rows: compute-bound
 * GEMMs) and the workspace has room for them, the layer first dequantises every weight
 * into its workspace (moe_dequantize_fp8) and runs moe_layer_fwd's bf16 kernels on them
 * (the faster way there); otherwise it runs moe_grouped_gemm_fp8's kernels, which
 * dequantise in registers (below 256 rows they also read half the weight bytes).  All
 * paths use the same bf16 weight values; in the 256-row regime both give bitwise the
 * same output.
 * Workspace, 16-byte aligned: moe_fp8_workspace_bytes(s) bytes (moe_workspace_bytes's
 * layout, then the dequantised weights where that path applies, or, where experts
 * average at most 64 rows, moe_grouped_gemm_fp8's optional scratch), or as little as
 * moe_workspace_bytes(s) bytes (no dequantised copy: the in-register path; no scratch:
 * whole items only); MOE_EWORKSPACE below that.
 */
size_t moe_fp8_workspace_bytes(const moe_shape* s);

moe_status moe_layer_fwd_fp8(const moe_shape* s, const void* x, const void* w_gate,
                             const float* bias, const uint8_t* q1, const float* s1,
                             const uint8_t* q3, const float* s3, const uint8_t* q2,
                             const float* s2, const uint8_t* qs1, const float* ss1,
                             const uint8_t* qs3, const float* ss3, const uint8_t* qs2,
                             const float* ss2, const int32_t* topk_idx_in,
                             const float* topk_w_in, void* out, void* ws,
                             size_t ws_bytes, void* stream);

/*
 * Backward pass (dropless notes: the gradients of the grouped GEMMs are grouped GEMMs
 * over the same segments - data gradients through the transposed expert weights,
 * weight gradients reducing over each expert's rows - and the permutation is replayed
 * from the forward's indices).  The gradient of <dout, out> by the chain rule of the
 * forward definition, step by step:
 *   combine  dy[pos[t,j]] = w[t,j] dout[t];  dw[t,j] = <dout[t], y[pos[t,j]]>
 *   down     dact = dy W2[e]^T;  dW2[e] = act_e^T dy_e
 *   SwiGLU   g = A W1[e], u = A W3[e] recomputed;  dg = dact u silu'(g),
 *            du = dact silu(g),  silu'(z) = sigmoid(z) (1 + z (1 - sigmoid(z)))
 *   gate/up  dx_perm = dg W1[e]^T + du W3[e]^T;  dW1[e] | dW3[e] = x_perm_e^T (dg | du)
 *   permute  dx[t] = sum_j dx_perm[pos[t,j]]   (moe_combine with unit weights)
 *   shared   the same three GEMM steps over all tokens with output gradient dout
 *   router   dlogits through the softmax (and renormalisation) with the selection
 *            held fixed;  dW_g = x^T dlogits;  dbias = sum_t dlogits;  dx += dlogits W_g^T
 * All backward entry points need dtype bf16 and d, d_e, d_e_shared multiples of 32
 * (else MOE_ENOTSUP).  Data gradients are bf16 (fp32 accumulation, one rounding);
 * weight gradients, dtopk_w, dlogits, dW_g and dbias are fp32, each element written
 * once (no atomics, fixed summation order).
 */

/*
 * Combine backward.  In: dout [T, d], y [moe_max_rows(s), d] (the forward's down
 * output), pos [T*k], topk_w [T, k].  Out: dy [moe_max_rows(s), d] (rows no slot uses
 * are not written), dtopk_w [T, k] fp32 (0 for slots with pos < 0).  d <= 8192.
 */
moe_status moe_combine_bwd(const moe_shape* s, const void* dout, const void* y,
                           const int32_t* pos, const float* topk_w, void* dy,
                           float* dtopk_w, void* stream);

/*
 * SwiGLU backward fused into the gate/up grouped GEMM: the gate and up products are
 * recomputed from A (x_perm [rows, d], or x [T, d] with row_src as for
 * moe_grouped_gemm_gather) and the forward's weights, and the epilogue writes
 * dgu = [dg | du], [rows, 2 d_e] (dg in columns [0, d_e), du in [d_e, 2 d_e)), from
 * dact [rows, d_e].  The block table as for moe_grouped_gemm.
 * Shared expert: x_shared (= x [T, d]), ws1, ws3, dact_shared [T, d_e_shared] and
 * dgu_shared [T, 2 d_e_shared] all given (needs d_e_shared > 0), or all NULL.
 */
moe_status moe_swiglu_bwd(const moe_shape* s, const void* A, const int32_t* row_src,
                          const void* w1, const void* w3, const void* dact,
                          const int32_t* block_meta, const int32_t* num_blocks,
                          int32_t max_blocks, void* dgu, const void* x_shared,
                          const void* ws1, const void* ws3, const void* dact_shared,
                          void* dgu_shared, void* stream);

/*
 * Data-gradient grouped GEMM (the weights read transposed):
 *   op = MOE_OP_DOWN:         dA = dact [rows, d_e] = dC W2[e]^T, dC = dy [rows, d],
 *                             B0 = W2 [E, d_e, d], B1 = NULL;
 *   op = MOE_OP_GATEUP_SWIGLU: dA = dx_perm [rows, d] = dC [W1[e] | W3[e]]^T,
 *                             dC = dgu [rows, 2 d_e], B0 = W1, B1 = W3 [E, d, d_e].
 * block_meta, num_blocks, max_blocks as for moe_grouped_gemm; block_meta = num_blocks
 * = NULL with max_blocks = 0 is the dense mode (one expert, E = 1, over T rows: the
 * shared expert with s->d_e = d_e_shared).  Only rows the table covers are written.
 * ws: NULL - a kernel reads the weights transposed in place; or device scratch of
 * ws_bytes >= moe_grouped_gemm_dgrad_workspace_bytes(s, op) - the weights are first
 * transposed into it and the forward grouped-GEMM kernels compute the plain product.
 */
size_t moe_grouped_gemm_dgrad_workspace_bytes(const moe_shape* s, int32_t op);
moe_status moe_grouped_gemm_dgrad(const moe_shape* s, int32_t op, const void* dC,
                                  const void* B0, const void* B1, const int32_t* block_meta,
                                  const int32_t* num_blocks, int32_t max_blocks, void* dA,
                                  void* ws, size_t ws_bytes, void* stream);

/*
 * Weight-gradient grouped GEMM, reducing over each expert's rows
 * [padded_offsets[e], padded_offsets[e] + counts[e]) (moe_build_offsets' outputs):
 *   op = MOE_OP_DOWN:          dB0 = dW2 [E, d_e, d] = A_e^T dC_e, A = act [rows, d_e],
 *                              dC = dy [rows, d], dB1 = NULL;
 *   op = MOE_OP_GATEUP_SWIGLU: dB0 = dW1, dB1 = dW3 [E, d, d_e] = A_e^T (dg | du)_e,
 *                              A = x_perm [rows, d], dC = dgu [rows, 2 d_e].
 * counts = padded_offsets = NULL: dense mode over all T rows (E = 1, d_e as in s).
 * fp32 outputs; experts without rows get zeros.
 * ws: NULL - work group b computes output tiles b, b + grid, ... in expert order; or
 * device scratch of ws_bytes >= moe_grouped_gemm_wgrad_workspace_bytes(s), 16-byte
 * aligned - the routed experts' tiles are handed out through a work queue, largest
 * expert first (a one-block kernel ranks the experts by count and clears the queue
 * first), so experts of unequal size do not leave work groups idle at the end.  The
 * results are bitwise the same either way.  Errors: MOE_EWORKSPACE for a short ws.
 */
size_t moe_grouped_gemm_wgrad_workspace_bytes(const moe_shape* s);
moe_status moe_grouped_gemm_wgrad(const moe_shape* s, int32_t op, const void* A,
                                  const void* dC, const int32_t* counts,
                                  const int32_t* padded_offsets, float* dB0, float* dB1,
                                  void* ws, size_t ws_bytes, void* stream);

/*
 * Router backward (TileLang chapter section 2.2's weights w = softmax(logits)[idx],
 * divided by their sum when s->renormalize): the selection is piecewise constant and
 * held fixed.  In: x [T, d], w_gate [d, E] (bf16), logits [T, E] fp32 (the forward's),
 * topk_idx [T, k], dtopk_w [T, k] fp32; dx_in [T, d] or NULL.
 * Out: dlogits [T, E] fp32, dw_gate [d, E] fp32, dbias [E] fp32 (or NULL: skipped),
 *      dx_out [T, d] = dx_in + dlogits w_gate^T (bf16, one rounding).
 * ws:  device scratch of ws_bytes >= moe_router_bwd_workspace_bytes(s) (the token-chunk
 *      partial sums of dw_gate and dbias; may be 0 bytes, ws then NULL).
 */
size_t moe_router_bwd_workspace_bytes(const moe_shape* s);
moe_status moe_router_bwd(const moe_shape* s, const void* x, const void* w_gate,
                          const float* logits, const int32_t* topk_idx, const float* dtopk_w,
                          float* dlogits, float* dw_gate, float* dbias, const void* dx_in,
                          void* dx_out, void* ws, size_t ws_bytes, void* stream);

/*
 * Host-only and pure: bytes of the backward workspace and the offsets of its
 * intermediates (dy, dact, dgu, x_perm, dx_perm [rows, .]; dtopk_w [T, k] and dlogits
 * [T, E] fp32; the shared expert's dact, dgu, dx and the router's dx [T, .]; the
 * router's scratch; where experts average >= 256 rows, the expert weights transposed for
 * the data gradients: W2^T [E][d][d_e], [W1^T; W3^T] [E][2 d_e][d] and the shared
 * expert's likewise).
 */
typedef struct moe_bwd_ws_layout {
  size_t dy, dact, dgu, x_perm, dx_perm, dtopk_w, dlogits, shared_dact, shared_dgu,
         shared_dx, router_dx, router_scratch, wgrad_sched, w2_t, w13_t, ws2_t, ws13_t, total;
} moe_bwd_ws_layout;
size_t moe_bwd_workspace_bytes(const moe_shape* s);
moe_status moe_bwd_workspace_layout(const moe_shape* s, moe_bwd_ws_layout* layout);

/*
 * The layer's backward, after moe_layer_fwd on the same arguments: fwd_ws is that
 * call's workspace (read only: logits, routes, block table, act, y, shared_act).
 * In:  x, w_gate (when the forward routed), w1, w3, w2, ws1, ws3, ws2, topk_idx_in and
 *      topk_w_in exactly as given to moe_layer_fwd; dout [T, d].
 * Out: dx [T, d] (bf16); dw1, dw3 [E, d, d_e], dw2 [E, d_e, d] fp32; dws1, dws3
 *      [d, d_e_shared], dws2 [d_e_shared, d] fp32 when d_e_shared > 0 (else NULL);
 *      dw_gate [d, E] fp32 and dbias [E] fp32 (either may be NULL) when the forward
 *      routed (NULL otherwise); dtopk_w [T, k] fp32 or NULL (the routing weights'
 *      gradient; with given routes it is the only gradient they get).
 * ws:  ws_bytes >= moe_bwd_workspace_bytes(s).
 */
moe_status moe_layer_bwd(const moe_shape* s, const void* x, const void* w_gate,
                         const void* w1, const void* w3, const void* w2, const void* ws1,
                         const void* ws3, const void* ws2, const int32_t* topk_idx_in,
                         const float* topk_w_in, const void* dout, const void* fwd_ws,
                         size_t fwd_ws_bytes, void* dx, float* dw1, float* dw3, float* dw2,
                         float* dws1, float* dws3, float* dws2, float* dw_gate, float* dbias,
                         float* dtopk_w, void* ws, size_t ws_bytes, void* stream);

/*
 * Byte offsets of the intermediates inside the moe_layer_fwd workspace, so that a
 * caller (tests, profilers) can inspect them after a call.  Host-only and pure.
 * Each field is an offset from the workspace base; a field is 0-sized when unused:
 * x_perm where the permute is fused into the gate/up loads (bf16, d % 32 == 0: x's
 * rows are gathered instead, see moe_grouped_gemm_gather), shared_act and shared_out
 * without a shared expert.
 */
typedef struct moe_ws_layout {
  size_t logits, topk_idx, topk_w, counts, offsets, padded_offsets, block_meta,
         num_blocks, pos, row_src, err_flag, x_perm, act, y, shared_act, shared_out,
         scratch, total;
} moe_ws_layout;
moe_status moe_workspace_layout(const moe_shape* s, moe_ws_layout* layout);

/*
 * Debug builds (the library compiled with MOE_DEBUG defined: libmoe_debug.so next to
 * libmoe.so).  The kernels check what they index with before they use it, and skip or
 * clamp what does not fit; a release build does so silently, a debug build also sets
 * a bit of a word kept on each device, so that bad tables and positions handed to an
 * entry point, or produced by an earlier stage, become visible:
 */
#define MOE_DBG_BLOCK_TABLE 0x1u  /* a block-table entry with an expert outside [0, E), a row
                                     count outside [1, block_m] or rows beyond the row
                                     buffers (the entry is skipped) */
#define MOE_DBG_BLOCK_COUNT 0x2u  /* *num_blocks outside [0, max_blocks] (clamped), or a block
                                     table longer than moe_max_blocks while it is built */
#define MOE_DBG_POSITION    0x4u  /* a row position outside [-1, rows) (skipped) */
#define MOE_DBG_GATHER_ROW  0x8u  /* a gathered A row outside the unpermuted rows (clamped) */
#define MOE_DBG_EXPERT_ID   0x10u /* the router wrote an expert id outside [0, E) (NaN
                                     logits; moe_build_offsets then flags it too) */
/*
 * OR of the bits set on the current device since the last clear, into *flags; with
 * clear != 0 the word is reset.  Synchronises the device first, so it reports every
 * kernel enqueued before the call.  Release builds: *flags = 0 and MOE_ENOTSUP.
 * Errors: MOE_EINVAL for flags == NULL, MOE_EHIP if the device cannot be read.
 */
moe_status moe_debug_flags(uint32_t* flags, int32_t clear);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */
