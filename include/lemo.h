/*
 * lemo.h -- C ABI of the contextual-token-sparsity hot path on MI355X (gfx950).
 *
 * Per layer, the method decides which token blocks take part in the layer and
 * moves only those rows:
 *   exact block scores   lemo_block_scores      (pages: Eq. 1, Eq. 2, Figure 6)
 *     batches, causal masking, ragged last block: lemo_block_scores_batched
 *   predicted scores     lemo_predict_scores    (pages: Eq. 3, Figure 8)
 *   per-token predictor  lemo_token_embeddings  (pages: Figure 8; scored by lemo_block_scores)
 *   threshold / compact  lemo_select_mask       (pages: layer threshold, Alg. 1 step 1)
 *   selective load       lemo_gather_pad        (pages: permutation-free movement)
 *   in-place addition    lemo_scatter_residual  (pages: permutation-free movement)
 *     its backward recompute: lemo_residual_recompute
 *   MLP-block scores     lemo_mlp_block_scores, lemo_mlp_block_scores_gated
 *                        (pages: extension of token elimination to the MLP block)
 *   movement fused into the layer's products: lemo_gather_linear, lemo_linear_scatter
 * "The pages" are "Jenga: Enhancing LLM Long-Context Fine-tuning with
 * Contextual Token Sparsity" (USENIX ATC'25; summary page, section 4.2) and
 * the review page of its arXiv version "LeMo" (2501.09767).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - bf16 values are passed as raw 16-bit patterns (lemo_bf16).  Matrices are
 *    row-major; "ld" arguments are row strides in elements.
 *  - Every pointer except the host-side scalars is DEVICE memory owned by the
 *    caller.  The library allocates and frees nothing and keeps no per-call
 *    state; scratch space comes from the caller through `workspace`, sized by
 *    the matching *_workspace() query.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Calls only enqueue work; they never synchronise.  Outputs are valid once
 *    the stream reaches them.  Device-resident results (n_kept, kept_blocks)
 *    flow device-to-device between calls without a host round trip.  A call
 *    enqueues kernel launches only (no allocation, memset or copy), so a
 *    sequence of calls can be captured in a HIP graph and replayed.
 *  - Arguments are validated on the host BEFORE anything is enqueued: a
 *    non-OK status means nothing was launched.  lemo_last_error() gives a
 *    thread-local text for the last non-OK status.  A failing launch returns
 *    LEMO_ERR_DEVICE.
 *  - Device-side conditions never trap: kernels OR bits into the optional
 *    int32 `dev_status` word (the caller clears it): LEMO_DEV_CAP_OVERFLOW,
 *    LEMO_DEV_NONFINITE, LEMO_DEV_BAD_KEPT.
 *  - Pointers to bf16 matrices must be 16-byte aligned and their ld a
 *    multiple of 8 elements (128-bit row access).  Matrices read by the
 *    matrix-core kernels (q, k, x of the per-token predictor and of the
 *    fused products, a, weight) are addressed with 32-bit row offsets:
 *    (rows - 1) * ld must stay below 2^31 - 64 elements, else the call
 *    returns LEMO_ERR_UNSUPPORTED.
 *  - Inputs and outputs of one call must not overlap, except the residual of
 *    lemo_scatter_residual, lemo_residual_recompute and lemo_linear_scatter,
 *    which is updated in place by design.
 *  - Same inputs on the same device give bitwise-identical outputs (no
 *    floating-point atomics anywhere).
 *  - Calls are thread-safe; calls that share output buffers on one stream
 *    are ordered by that stream.
 */
#ifndef LEMO_H
#define LEMO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t lemo_bf16; /* raw bf16 bit pattern */

typedef enum {
  LEMO_OK = 0,
  LEMO_ERR_INVALID_ARG = 1,  /* null pointer, negative or inconsistent size, bad enum */
  LEMO_ERR_UNSUPPORTED = 2,  /* valid but not implemented shape (block, head_dim, rank) */
  LEMO_ERR_ALIGNMENT = 3,    /* pointer not 16-byte aligned or ld not a multiple of 8 */
  LEMO_ERR_WORKSPACE = 4,    /* workspace missing or smaller than the query says */
  LEMO_ERR_DEVICE = 5        /* a HIP call failed; see lemo_last_error() */
} lemo_status;

typedef enum {
  /* Eq. 2 as printed: M[n][m] = max over (i in block n, j in block m, i != j)
   * of (1/H) * sum_h max(0, S^h_ij) -- heads aggregated first, then block max. */
  LEMO_REDUCE_PAPER = 0,
  /* Per-head block max, clamped, then summed over heads:
   * M[n][m] = sum_h max(0, max over (i in n, j in m, i != j) of S^h_ij). */
  LEMO_REDUCE_HEADMAX = 1
} lemo_head_reduce;

typedef enum {
  LEMO_SELECT_THRESHOLD = 0, /* keep block c iff I[c] >= threshold */
  LEMO_SELECT_TOPK = 1,      /* keep the keep_blocks best blocks (ties: lower index) */
  LEMO_SELECT_MEAN = 2       /* threshold = mean of I (Algorithm 1, step 1) */
} lemo_select_mode;

#define LEMO_DEV_CAP_OVERFLOW 1 /* gather: padded row count exceeded cap_rows; writes truncated */
#define LEMO_DEV_NONFINITE 2    /* select: a NaN or infinite score was seen */
#define LEMO_DEV_BAD_KEPT 4     /* gather/scatter: n_kept or a kept block index out of range; skipped */

/* ------------------------------------------------------------------------
 * Exact block scores (Jenga 4.2.1, Eq. 1 and Eq. 2; Figure 6 caption).
 *
 * For heads h < n_heads: S^h_ij = (Q^h_i . K^h_j) / sqrt(head_dim), the raw
 * pre-softmax score (bf16 inputs, fp32 accumulation).  The N x N score matrix
 * is cut into (block x block) tiles B^S_nm; each tile is reduced to one value
 * M[n][m] as chosen by head_reduce (pairs i == j excluded), and the token
 * block score is the column aggregate I[m] = sum over n of M[n][m].
 * S never reaches memory: it lives in registers between the matrix-core
 * product and the reduction.
 *
 *  q, k          bf16 [n_tokens][ld_q|ld_k]; head h occupies columns
 *                h*head_dim .. h*head_dim+head_dim-1.
 *  n_tokens      N > 0, a multiple of block, at most 2^22; with more than
 *                one head at most 2^23 tiles of 128 x 128 per launch
 *                (N <= 370688).
 *  head_dim      64 or 128.   block: 32, 64 or 128.
 *  block_scores  optional fp32 [nb][nb] output M (row n = query block),
 *                nb = n_tokens / block; NULL keeps M in the workspace.
 *  scores        fp32 [nb] output I.
 *  workspace     device scratch of lemo_block_scores_workspace() bytes when
 *                block_scores is NULL; may be NULL / 0 bytes otherwise.
 * Errors: INVALID_ARG (null q/k/scores, N % block, n_heads < 1,
 * ld < n_heads*head_dim, bad head_reduce), UNSUPPORTED (head_dim, block,
 * N > 2^22), ALIGNMENT, WORKSPACE.  Non-finite inputs give unspecified scores.
 * ------------------------------------------------------------------------ */
size_t lemo_block_scores_workspace(int n_tokens, int block); /* bytes needed when block_scores is NULL */
lemo_status lemo_block_scores(const lemo_bf16* q, const lemo_bf16* k, int n_tokens, int n_heads,
                              int head_dim, int ld_q, int ld_k, int block, int head_reduce,
                              float* block_scores, float* scores, void* workspace,
                              size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Exact block scores of a batch of sequences, with a causal variant and a
 * ragged last block (the same Eq. 1 / Eq. 2 / Figure 6 definitions).
 *
 * Sequence b (0 <= b < n_batch) has q + b*batch_stride_q and
 * k + b*batch_stride_k as its [n_tokens][ld] matrices and is scored on its
 * own: no pair crosses sequences.  n_tokens need not be a multiple of block:
 * the last of nb = ceil(n_tokens / block) blocks holds the remaining tokens.
 * With LEMO_SCORES_CAUSAL in flags only pairs j < i take part (decoder
 * attention never pairs a query with a later key): every block above the
 * block diagonal scores 0, diagonal blocks use their strictly lower pairs,
 * and causal launches skip the tiles above the diagonal (about half the
 * work).  Without the flag pairs i == j are excluded as in
 * lemo_block_scores, which this call equals for n_batch = 1 and
 * n_tokens % block == 0.  A block pair with no pair taking part scores 0.
 *
 *  n_batch        1..65535.
 *  batch_stride_* elements between sequences: multiples of 8 and at least
 *                 n_tokens*ld (sequences do not overlap); ignored when
 *                 n_batch == 1.
 *  flags          0 or LEMO_SCORES_CAUSAL.
 *  block_scores   optional fp32 [n_batch][nb][nb] (sequence-major); NULL
 *                 keeps M in the workspace.
 *  scores         fp32 [n_batch][nb].
 *  workspace      lemo_block_scores_batched_workspace() bytes when
 *                 block_scores is NULL.
 * Errors: as lemo_block_scores, plus INVALID_ARG (n_batch < 1, unknown
 * flags, stride smaller than a sequence), UNSUPPORTED (n_batch > 65535, or
 * n_batch times the 128 x 128 tiles of one sequence -- ceil(N/128)^2, or
 * T(ceil(N/128)) = t (t + 1) / 2 with the causal flag -- above 2^23 with
 * more than one head, above 2^31 - 1 with one),
 * ALIGNMENT (stride not a multiple of 8).
 * ------------------------------------------------------------------------ */
#define LEMO_SCORES_CAUSAL 1
size_t lemo_block_scores_batched_workspace(int n_batch, int n_tokens, int block);
lemo_status lemo_block_scores_batched(const lemo_bf16* q, const lemo_bf16* k, int n_batch, int n_tokens,
                                      int n_heads, int head_dim, int ld_q, int ld_k, int64_t batch_stride_q,
                                      int64_t batch_stride_k, int block, int head_reduce, int flags,
                                      float* block_scores, float* scores, void* workspace,
                                      size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Predicted block scores (Jenga 4.2.2, Eq. 3 and Figure 8).
 *
 * Each token block's representative embedding is the mean of its rows,
 *   xbar_m = bf16( (fp32 sum of the block's rows, in row order) / rows );
 * rows = block, or for the last block of a ragged sequence (n_tokens not a
 * multiple of block) the n_tokens mod block remaining rows (an IEEE fp32
 * division; for a whole block it is the exact multiplication by 1/block);
 * the query and key predictors are q_hat = bf16(ReLU(xbar U_q)) V_q and
 * k_hat = bf16(ReLU(xbar U_k)) V_k (fp32 accumulation; q_hat, k_hat fp32);
 * the block-pair score is M_hat[m][n] = max(0, q_hat_m . k_hat_n) and the
 * token block score is the column aggregate I_hat[n] = sum over m of M_hat[m][n].
 *
 *  x             bf16 [n_tokens][ld_x] token embeddings, d_model columns used.
 *  block         power of two, 2..256; nb = ceil(n_tokens / block) <= 65535.
 *  d_model       multiple of 64.   rank: multiple of 32, at most 256.
 *  u_q, u_k      bf16 [d_model][rank] row-major.  v_q, v_k: bf16 [rank][rank].
 *  block_scores  optional fp32 [nb][nb] M_hat (NULL: M_hat is never stored;
 *                the column aggregate is formed on the fly).
 *  scores        fp32 [nb] I_hat.
 *  workspace     lemo_predict_scores_workspace() bytes, 16-byte aligned:
 *                xbar, split-K partial sums of the hidden layer, q_hat, k_hat
 *                (it does not grow with nb^2).
 * Errors: INVALID_ARG, UNSUPPORTED (block, d_model, rank), ALIGNMENT, WORKSPACE.
 * ------------------------------------------------------------------------ */
size_t lemo_predict_scores_workspace(int n_tokens, int d_model, int block, int rank);
lemo_status lemo_predict_scores(const lemo_bf16* x, int n_tokens, int d_model, int ld_x, int block,
                                const lemo_bf16* u_q, const lemo_bf16* v_q, const lemo_bf16* u_k,
                                const lemo_bf16* v_k, int rank, float* block_scores, float* scores,
                                void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * lemo_predict_scores without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments, results and errors as
 * lemo_predict_scores, minus the workspace: the scratch is a fixed 16 MiB
 * array in the library's device code, one per device, held until the process
 * ends.  The call allocates nothing.
 *  Limit: shapes whose lemo_predict_scores_workspace() exceeds 16 MiB (16 *
 *  2^20 bytes) are refused with LEMO_ERR_UNSUPPORTED; e.g. 16384 tokens of
 *  4096 in blocks of 64 with rank 128 need 4.3 MiB, 32768 tokens of 5120 in
 *  blocks of 128 with rank 256 need 5 MiB.
 *  Every call on one device shares that device's array: calls that overlap
 *  on one device (on different streams, or from several threads without
 *  ordering) race and give unspecified results.  No part of the scratch
 *  needs to start at zero.
 * ------------------------------------------------------------------------ */
lemo_status lemo_predict_scores_noalloc(const lemo_bf16* x, int n_tokens, int d_model, int ld_x, int block,
                                        const lemo_bf16* u_q, const lemo_bf16* v_q, const lemo_bf16* u_k,
                                        const lemo_bf16* v_k, int rank, float* block_scores, float* scores,
                                        void* stream);

/* ------------------------------------------------------------------------
 * Per-token predictor embeddings (Jenga 4.2.2, Figure 8, and its complexity
 * analysis, which prices the query and key predictors at one pass per token).
 *
 * For every token row x of X:
 *   q_hat = bf16( bf16(ReLU(x U_q)) V_q ),   k_hat = bf16( bf16(ReLU(x U_k)) V_k ),
 * fp32 accumulation, round to nearest even at both bf16 points.  q_hat and
 * k_hat are the query and key of ONE head of width `rank`: passing them to
 * lemo_block_scores(q_hat, k_hat, n_tokens, 1, rank, ld_out, ld_out, block,
 * ...) gives the per-token predicted block scores (with that call's
 * 1/sqrt(rank) scale; rank 64 or 128 there).
 *
 *  x             bf16 [n_tokens][ld_x], d_model columns used (d_model % 64 == 0).
 *  u_q, u_k      bf16 [d_model][rank]; v_q, v_k bf16 [rank][rank] (rank % 64 == 0, <= 256).
 *  q_hat, k_hat  bf16 [n_tokens][ld_out] outputs, rank columns written.
 *  workspace     lemo_token_embeddings_workspace() bytes.  Rank 128 with
 *                d_model % 256 == 0 runs as one fused launch and needs none
 *                (the function returns 0 and workspace may be NULL); other
 *                shapes hold the transposed weights and the [n_tokens][2 rank]
 *                hidden activations there.
 * Errors: INVALID_ARG, UNSUPPORTED (d_model, rank), ALIGNMENT, WORKSPACE.
 * ------------------------------------------------------------------------ */
size_t lemo_token_embeddings_workspace(int n_tokens, int d_model, int rank);
lemo_status lemo_token_embeddings(const lemo_bf16* x, int n_tokens, int d_model, int ld_x,
                                  const lemo_bf16* u_q, const lemo_bf16* v_q, const lemo_bf16* u_k,
                                  const lemo_bf16* v_k, int rank, lemo_bf16* q_hat, lemo_bf16* k_hat,
                                  int ld_out, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Layer threshold and compaction (Jenga 4.2.1, "Layer-specific Threshold";
 * Algorithm 1 step 1 initialises the threshold to the average block score).
 *
 *  scores        fp32 [n_blocks] token block scores I (device).
 *  n_blocks      1..8192.
 *  mode          lemo_select_mode.  THRESHOLD uses `threshold`; MEAN computes
 *                it as (float64 sum of I in block order) / n_blocks rounded to
 *                fp32; TOPK keeps exactly keep_blocks blocks ordered by score
 *                descending, ties to the lower index, NaN last.
 *  mask          uint8 [n_blocks] out: 1 = keep.
 *  kept_blocks   int32 [n_blocks] out: kept block indices, ascending, in the
 *                first n_kept entries (the rest is left unchanged).
 *  n_kept        int32 device scalar out.
 *  threshold_used optional fp32 device scalar out (TOPK: the last kept score,
 *                +inf when none is kept).
 *  dev_status    optional; LEMO_DEV_NONFINITE is set when a score is NaN/inf.
 * A block is kept iff score >= threshold (NaN never passes).
 * ------------------------------------------------------------------------ */
lemo_status lemo_select_mask(const float* scores, int n_blocks, int mode, float threshold,
                             int keep_blocks, uint8_t* mask, int32_t* kept_blocks, int32_t* n_kept,
                             float* threshold_used, int32_t* dev_status, void* stream);

/* ------------------------------------------------------------------------
 * Selective load (Jenga 4.2.3, Permutation-free Token Movement): the kept
 * tokens are read from their original rows into a dense buffer.
 *
 *  dst[p] = src[kept_blocks[p / block] * block + p % block] for p < R,
 *  R = n_kept * block (bit copy of `width` elements); rows R .. roundup(R,
 *  pad_multiple)-1 are zeroed; rows beyond are not touched.  Rows at or past
 *  cap_rows are never written (LEMO_DEV_CAP_OVERFLOW is set if R rounded up
 *  exceeds cap_rows).  n_kept and kept_blocks are read on the device.
 *  Ragged sequences (n_tokens not a multiple of block): the last block
 *  (index nb - 1) has only n_tokens mod block rows; when it is the last kept
 *  block, as in lemo_select_mask's ascending list, R is that many rows short
 *  of n_kept * block.  A position whose token would lie past n_tokens (the
 *  short block listed before the end) is skipped and flags
 *  LEMO_DEV_BAD_KEPT, like an out-of-range kept index.  The same holds for
 *  lemo_scatter_residual, lemo_residual_recompute and the fused products.
 *  width         multiple of 8; ld_src, ld_dst >= width, multiples of 8.
 *  cap_rows      rows of dst.   pad_multiple >= 1.
 * ------------------------------------------------------------------------ */
lemo_status lemo_gather_pad(const lemo_bf16* src, int n_tokens, int width, int ld_src, int block,
                            const int32_t* kept_blocks, const int32_t* n_kept, lemo_bf16* dst,
                            int ld_dst, int cap_rows, int pad_multiple, int32_t* dev_status,
                            void* stream);

/* ------------------------------------------------------------------------
 * Selective load of several matrices on one kept list in one launch (Jenga
 * 4.2.3, selective load: a layer reads the kept tokens of every matrix it
 * consumes, e.g. the attention input and the MLP activation, from their
 * original rows).  For each source i < n_src the result is exactly that of
 * lemo_gather_pad(srcs[i], n_tokens, widths[i], ld_srcs[i], block, ...,
 * dsts[i], ld_dsts[i], cap_rows, pad_multiple): the same rows, zero padding,
 * untouched rows past the padding, capacity and status behaviour.
 *  n_src          1..4.
 *  srcs, widths, ld_srcs, dsts, ld_dsts   host arrays of n_src entries; the
 *                 matrices they point to are device memory.  Every dsts[i]
 *                 holds at least cap_rows rows; no destination may overlap
 *                 any source or another destination.
 * Errors: INVALID_ARG (NULL, sizes, n_src, ld < width), ALIGNMENT (pointers,
 * ld, width).
 * ------------------------------------------------------------------------ */
lemo_status lemo_gather_pad_multi(int n_src, const lemo_bf16* const* srcs, const int* widths, const int* ld_srcs,
                                  lemo_bf16* const* dsts, const int* ld_dsts, int n_tokens, int block,
                                  const int32_t* kept_blocks, const int32_t* n_kept, int cap_rows, int pad_multiple,
                                  int32_t* dev_status, void* stream);

/* ------------------------------------------------------------------------
 * Token movement fused into the layer's products (Jenga 4.2.3, permutation-
 * free token movement, Figure 18: selective load and in-place addition are
 * carried out inside the computation, not as separate passes).
 *
 * weight is a Linear layer's bf16 matrix stored [d_out][ld_w] (out x in,
 * d_in columns used); the product of a row r is r weight^T with fp32
 * accumulation, rounded to nearest even to bf16.  tok(p) and R = n_kept *
 * block are as for lemo_gather_pad; n_kept and kept_blocks are read on the
 * device.  The results are bit for bit those of lemo_gather_pad followed by
 * the product, and of the product followed by lemo_scatter_residual.
 *
 * lemo_gather_linear: y[p] = bf16(x[tok(p)] weight^T) for p < R; rows R ..
 *   roundup(R, pad_multiple)-1 are zero; rows past that are untouched; rows
 *   past cap_rows are dropped and flag LEMO_DEV_CAP_OVERFLOW.
 *   x [n_tokens][ld_x] (d_in used), y [cap_rows][ld_y] (d_out used).
 * lemo_linear_scatter: residual[tok(p)] = bf16(residual[tok(p)] +
 *   bf16(a[p] weight^T)) for p < R, in place; other rows untouched.  a holds
 *   the kept rows densely, [cap_rows][ld_a] (d_in used); kept rows past
 *   cap_rows are skipped and flag LEMO_DEV_CAP_OVERFLOW.
 * Invalid kept indices are skipped and flag LEMO_DEV_BAD_KEPT; kept_blocks
 * must hold distinct indices (see lemo_scatter_residual).
 * d_in a multiple of 64, d_out a multiple of 8.  One launch holds at most
 * (2^31 - 1) / 512 output tiles of 256 x 256 (rows: cap_rows for the gather,
 * min(cap_rows, n_tokens) for the scatter).  Errors: INVALID_ARG,
 * UNSUPPORTED (d_in, tile count), ALIGNMENT (pointers, ld, d_out).
 * ------------------------------------------------------------------------ */
lemo_status lemo_gather_linear(const lemo_bf16* x, int n_tokens, int d_in, int ld_x, int block,
                               const int32_t* kept_blocks, const int32_t* n_kept, const lemo_bf16* weight,
                               int d_out, int ld_w, lemo_bf16* y, int ld_y, int cap_rows, int pad_multiple,
                               int32_t* dev_status, void* stream);
lemo_status lemo_linear_scatter(const lemo_bf16* a, int d_in, int ld_a, int cap_rows, const lemo_bf16* weight,
                                int d_out, int ld_w, lemo_bf16* residual, int n_tokens, int ld_res, int block,
                                const int32_t* kept_blocks, const int32_t* n_kept, int32_t* dev_status,
                                void* stream);

/* ------------------------------------------------------------------------
 * In-place addition (Jenga 4.2.3): the layer output of every kept token is
 * added to that token's original row of the residual stream; eliminated
 * tokens are left bit-identical.
 *
 *  residual[t] = bf16_rne(fp32(residual[t]) + fp32(y[p])) for p < R,
 *  t = kept_blocks[p / block] * block + p % block, over `width` elements
 *  (R as for lemo_gather_pad: n_kept*block, less the missing rows of a
 *  ragged sequence's short last block).
 *  (fp32 add then round-to-nearest-even: the correctly rounded bf16 sum.)
 *  y             bf16 [>= n_kept*block][ld_y], rows in kept order (as
 *                lemo_gather_pad lays them out).  lemo_scatter_residual
 *                trusts the caller on this: y must hold every kept row.
 *  kept_blocks   distinct block indices (lemo_select_mask's ascending list
 *                is); a block listed twice makes two unsynchronised updates
 *                of the same residual rows, whose result is unspecified.
 *                The same holds for lemo_residual_recompute and
 *                lemo_linear_scatter.
 *
 * lemo_scatter_residual_capped: the same with the number of rows y holds,
 *  y_rows >= 0, as an argument.  Kept rows p >= y_rows (possible when the
 *  layer output was built from a gather that hit its capacity) are left out:
 *  their residual rows stay untouched, y is never read past row y_rows - 1,
 *  and LEMO_DEV_CAP_OVERFLOW is set in dev_status.
 * Invalid kept indices are skipped and flag LEMO_DEV_BAD_KEPT.  width a
 * multiple of 8; ld_res, ld_y >= width, multiples of 8.  Errors: INVALID_ARG
 * (NULL, sizes, negative y_rows, ld < width), ALIGNMENT (pointers, ld, width).
 * ------------------------------------------------------------------------ */
lemo_status lemo_scatter_residual(lemo_bf16* residual, int n_tokens, int width, int ld_res, int block,
                                  const int32_t* kept_blocks, const int32_t* n_kept,
                                  const lemo_bf16* y, int ld_y, int32_t* dev_status, void* stream);
lemo_status lemo_scatter_residual_capped(lemo_bf16* residual, int n_tokens, int width, int ld_res, int block,
                                         const int32_t* kept_blocks, const int32_t* n_kept, const lemo_bf16* y,
                                         int ld_y, int y_rows, int32_t* dev_status, void* stream);

/* ------------------------------------------------------------------------
 * Backward recompute of a layer's input (Jenga 4.2.3, in-place addition:
 * during backpropagation the original input is recovered by subtracting the
 * block's output from the output embeddings), so the forward pass need not
 * keep a copy of the residual stream.
 *
 *  residual[t] = bf16_rne(fp32(residual[t]) - fp32(y[p])) for the same kept
 *  rows p and tokens t as lemo_scatter_residual; eliminated rows, which the
 *  addition never changed, are left bit-identical.  When the forward
 *  addition rounded, the result is not the input bit for bit: each element
 *  is within half a bf16 spacing at the output value plus half a spacing at
 *  the result.  Arguments, errors and dev_status as lemo_scatter_residual;
 *  lemo_residual_recompute_capped takes y_rows as
 *  lemo_scatter_residual_capped does.
 * ------------------------------------------------------------------------ */
lemo_status lemo_residual_recompute(lemo_bf16* residual, int n_tokens, int width, int ld_res, int block,
                                   const int32_t* kept_blocks, const int32_t* n_kept,
                                   const lemo_bf16* y, int ld_y, int32_t* dev_status, void* stream);
lemo_status lemo_residual_recompute_capped(lemo_bf16* residual, int n_tokens, int width, int ld_res, int block,
                                          const int32_t* kept_blocks, const int32_t* n_kept, const lemo_bf16* y,
                                          int ld_y, int y_rows, int32_t* dev_status, void* stream);

/* ------------------------------------------------------------------------
 * Token-block scores from the MLP block (Jenga 4.2.1, "Extend to MLP
 * Block": the intermediate activation rates the tokens -- the ReLU output,
 * or for SiLU-gated MLPs SiLU(gate projection) * up projection).  The pages
 * state no aggregation; as Eq. 2 takes a block maximum and Figure 6 sums
 * along the other axis:
 *   I[m] = sum over channels c of max over tokens i in block m of |A[i][c]|.
 * The last of ceil(n_tokens / block) blocks holds the remaining tokens when
 * n_tokens is not a multiple of block.
 *
 *  act            bf16 [n_tokens][ld_act], width channels used (a ReLU
 *                 output, or any activation: magnitudes are taken).
 *  gate, up       (gated call) bf16 [n_tokens][ld] pre-activation gate and
 *                 up projections; A = SiLU(gate) * up is formed in fp32 in
 *                 registers (SiLU(g) = g / (1 + e^-g)), not rounded and
 *                 never stored.
 *  width          multiple of 8.   block: any positive size.
 *  scores         fp32 [ceil(n_tokens / block)] output I.
 *  workspace      lemo_mlp_block_scores_workspace() bytes (per-chunk partial
 *                 sums), 16-byte aligned.
 * Errors: INVALID_ARG (NULL, sizes, ld < width), ALIGNMENT (pointers, ld,
 * width), WORKSPACE.  Non-finite activations give unspecified scores.
 * ------------------------------------------------------------------------ */
size_t lemo_mlp_block_scores_workspace(int n_tokens, int width, int block);
lemo_status lemo_mlp_block_scores(const lemo_bf16* act, int n_tokens, int width, int ld_act, int block,
                                  float* scores, void* workspace, size_t workspace_bytes, void* stream);
lemo_status lemo_mlp_block_scores_gated(const lemo_bf16* gate, const lemo_bf16* up, int n_tokens, int width,
                                        int ld_gate, int ld_up, int block, float* scores, void* workspace,
                                        size_t workspace_bytes, void* stream);

const char* lemo_status_string(lemo_status s);
const char* lemo_last_error(void); /* thread-local detail of the last non-OK return */
int lemo_version(void);            /* major*10000 + minor*100 + patch */

#ifdef __cplusplus
}
#endif
#endif /* LEMO_H */
