// Host side of the C ABI: argument validation (before anything is enqueued),
// workspace sizing, status strings and the thread-local error text.
#include <climits>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "lemo_internal.h"

namespace {

thread_local std::string g_last_error;

lemo_status fail(lemo_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

lemo_status device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return LEMO_OK;
  return fail(LEMO_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

#define REQUIRE(cond, status, ...) \
  do {                             \
    if (!(cond)) return fail(status, __VA_ARGS__); \
  } while (0)

// Rows of a bf16 matrix: base pointer 16-byte aligned and ld a multiple of 8.
lemo_status check_rows(const void* p, int ld, int width, const char* name) {
  REQUIRE(p != nullptr, LEMO_ERR_INVALID_ARG, "%s is NULL", name);
  REQUIRE(ld >= width, LEMO_ERR_INVALID_ARG, "ld of %s (%d) < width %d", name, ld, width);
  REQUIRE(aligned16(p) && ld % 8 == 0, LEMO_ERR_ALIGNMENT,
          "%s must be 16-byte aligned with ld a multiple of 8 (ld=%d)", name, ld);
  return LEMO_OK;
}

// The matrix-core kernels load rows straight into LDS with a 32-bit per-lane
// byte offset from the matrix base (the column offset goes into the 64-bit
// base), so rows x ld must stay below 2^31 elements.
lemo_status check_offsets(int rows, int ld, const char* name) {
  REQUIRE((long long)(rows > 0 ? rows - 1 : 0) * ld < (1LL << 31) - 64, LEMO_ERR_UNSUPPORTED,
          "%s: %d rows x ld %d is beyond 32-bit row offsets", name, rows, ld);
  return LEMO_OK;
}

}  // namespace

extern "C" {

const char* lemo_status_string(lemo_status s) {
  // A C caller may pass any int here; reading an out-of-range value as the
  // enum type is undefined in C++, so the code is taken from its bytes.
  static_assert(sizeof(lemo_status) == sizeof(int), "lemo_status is an int-sized enum");
  int code;
  memcpy(&code, &s, sizeof code);
  switch (code) {
    case LEMO_OK: return "ok";
    case LEMO_ERR_INVALID_ARG: return "invalid argument";
    case LEMO_ERR_UNSUPPORTED: return "unsupported shape";
    case LEMO_ERR_ALIGNMENT: return "misaligned pointer or leading dimension";
    case LEMO_ERR_WORKSPACE: return "workspace missing or too small";
    case LEMO_ERR_DEVICE: return "device error";
  }
  return "unknown status";
}

const char* lemo_last_error(void) { return g_last_error.c_str(); }

int lemo_version(void) { return 100; }  // 0.1.0

// Exact scores: the block matrix stays within 2^40 entries.  A launch's x
// dimension holds at most 2^31 - 1 work-items, i.e. 2^23 workgroups of 256:
// with more than one head every 128 x 128 tile is a workgroup, so a launch
// takes at most 2^23 tiles (one head: the workgroups walk ranges of tiles).
constexpr int kMaxScoreTokens = 1 << 22;
constexpr long long kMaxWorkgroups = 1LL << 23;
// The fused products launch one workgroup of 512 work-items per 256 x 256
// tile of the output.
constexpr long long kMaxFusedWorkgroups = ((1LL << 31) - 1) / 512;

size_t lemo_block_scores_workspace(int n_tokens, int block) {
  if (n_tokens <= 0 || block <= 0 || n_tokens % block) return 0;
  const size_t nb = (size_t)(n_tokens / block);
  return lemo_align256(nb * nb * sizeof(float));
}

lemo_status lemo_block_scores(const lemo_bf16* q, const lemo_bf16* k, int n_tokens, int n_heads, int head_dim,
                              int ld_q, int ld_k, int block, int head_reduce, float* block_scores, float* scores,
                              void* workspace, size_t workspace_bytes, void* stream) {
  REQUIRE(scores != nullptr, LEMO_ERR_INVALID_ARG, "scores is NULL");
  REQUIRE(n_tokens > 0 && block > 0 && n_heads > 0 && head_dim > 0, LEMO_ERR_INVALID_ARG,
          "sizes must be positive (n_tokens=%d block=%d n_heads=%d head_dim=%d)", n_tokens, block, n_heads,
          head_dim);
  REQUIRE(n_tokens % block == 0, LEMO_ERR_INVALID_ARG, "n_tokens %d is not a multiple of block %d", n_tokens, block);
  REQUIRE(n_tokens <= kMaxScoreTokens, LEMO_ERR_UNSUPPORTED, "n_tokens %d (at most %d)", n_tokens, kMaxScoreTokens);
  REQUIRE(head_reduce == LEMO_REDUCE_PAPER || head_reduce == LEMO_REDUCE_HEADMAX, LEMO_ERR_INVALID_ARG,
          "unknown head_reduce %d", head_reduce);
  REQUIRE((long long)n_heads * head_dim <= (1LL << 30), LEMO_ERR_INVALID_ARG, "n_heads*head_dim too large");
  REQUIRE(head_dim == 64 || head_dim == 128, LEMO_ERR_UNSUPPORTED, "head_dim %d (64 or 128 supported)", head_dim);
  REQUIRE(block == 32 || block == 64 || block == 128, LEMO_ERR_UNSUPPORTED, "block %d (32, 64 or 128 supported)",
          block);
  REQUIRE(head_reduce == LEMO_REDUCE_PAPER || n_heads <= 128, LEMO_ERR_UNSUPPORTED,
          "HEADMAX supports at most 128 heads (got %d)", n_heads);
  const long long ntq = (n_tokens + 127) / 128;
  REQUIRE(n_heads == 1 || ntq * ntq <= kMaxWorkgroups, LEMO_ERR_UNSUPPORTED,
          "%lld tiles in one launch (at most %lld with more than one head)", ntq * ntq, kMaxWorkgroups);
  lemo_status st;
  if ((st = check_rows(q, ld_q, n_heads * head_dim, "q")) != LEMO_OK) return st;
  if ((st = check_rows(k, ld_k, n_heads * head_dim, "k")) != LEMO_OK) return st;
  if ((st = check_offsets(n_tokens, ld_q, "q")) != LEMO_OK) return st;
  if ((st = check_offsets(n_tokens, ld_k, "k")) != LEMO_OK) return st;
  float* m_out = block_scores;
  if (!m_out) {
    const size_t need = lemo_block_scores_workspace(n_tokens, block);
    REQUIRE(workspace != nullptr && workspace_bytes >= need, LEMO_ERR_WORKSPACE,
            "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
    m_out = static_cast<float*>(workspace);
  }
  return device_status(lemo_launch_block_scores(q, k, 1, n_tokens, n_heads, head_dim, ld_q, ld_k, 0, 0, block,
                                                head_reduce, false, m_out, scores, static_cast<hipStream_t>(stream)),
                       "lemo_block_scores launch");
}

size_t lemo_block_scores_batched_workspace(int n_batch, int n_tokens, int block) {
  if (n_batch <= 0 || n_tokens <= 0 || block <= 0) return 0;
  const size_t nb = (size_t)lemo_nblocks(n_tokens, block);
  return lemo_align256((size_t)n_batch * nb * nb * sizeof(float));
}

lemo_status lemo_block_scores_batched(const lemo_bf16* q, const lemo_bf16* k, int n_batch, int n_tokens,
                                      int n_heads, int head_dim, int ld_q, int ld_k, int64_t batch_stride_q,
                                      int64_t batch_stride_k, int block, int head_reduce, int flags,
                                      float* block_scores, float* scores, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  REQUIRE(scores != nullptr, LEMO_ERR_INVALID_ARG, "scores is NULL");
  REQUIRE(n_batch > 0 && n_tokens > 0 && block > 0 && n_heads > 0 && head_dim > 0, LEMO_ERR_INVALID_ARG,
          "sizes must be positive (n_batch=%d n_tokens=%d block=%d n_heads=%d head_dim=%d)", n_batch, n_tokens,
          block, n_heads, head_dim);
  REQUIRE(n_batch <= 65535, LEMO_ERR_UNSUPPORTED, "n_batch %d (at most 65535)", n_batch);
  REQUIRE(n_tokens <= kMaxScoreTokens, LEMO_ERR_UNSUPPORTED, "n_tokens %d (at most %d)", n_tokens, kMaxScoreTokens);
  REQUIRE((flags & ~LEMO_SCORES_CAUSAL) == 0, LEMO_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  REQUIRE(head_reduce == LEMO_REDUCE_PAPER || head_reduce == LEMO_REDUCE_HEADMAX, LEMO_ERR_INVALID_ARG,
          "unknown head_reduce %d", head_reduce);
  REQUIRE((long long)n_heads * head_dim <= (1LL << 30), LEMO_ERR_INVALID_ARG, "n_heads*head_dim too large");
  REQUIRE(head_dim == 64 || head_dim == 128, LEMO_ERR_UNSUPPORTED, "head_dim %d (64 or 128 supported)", head_dim);
  REQUIRE(block == 32 || block == 64 || block == 128, LEMO_ERR_UNSUPPORTED, "block %d (32, 64 or 128 supported)",
          block);
  REQUIRE(head_reduce == LEMO_REDUCE_PAPER || n_heads <= 128, LEMO_ERR_UNSUPPORTED,
          "HEADMAX supports at most 128 heads (got %d)", n_heads);
  const int nb = lemo_nblocks(n_tokens, block);
  const long long ntq = (n_tokens + 127) / 128;
  const long long tiles = (flags & LEMO_SCORES_CAUSAL) ? ntq * (ntq + 1) / 2 : ntq * ntq;
  REQUIRE(n_batch * tiles <= (n_heads == 1 ? 0x7fffffffLL : kMaxWorkgroups), LEMO_ERR_UNSUPPORTED,
          "n_batch * tiles = %lld exceeds one launch (n_batch=%d n_tokens=%d n_heads=%d)", n_batch * tiles, n_batch,
          n_tokens, n_heads);
  lemo_status st;
  if ((st = check_rows(q, ld_q, n_heads * head_dim, "q")) != LEMO_OK) return st;
  if ((st = check_rows(k, ld_k, n_heads * head_dim, "k")) != LEMO_OK) return st;
  if ((st = check_offsets(n_tokens, ld_q, "q")) != LEMO_OK) return st;
  if ((st = check_offsets(n_tokens, ld_k, "k")) != LEMO_OK) return st;
  if (n_batch > 1) {
    // each sequence's rows are 16-byte aligned, and sequences do not overlap
    REQUIRE(batch_stride_q % 8 == 0 && batch_stride_k % 8 == 0, LEMO_ERR_ALIGNMENT,
            "batch strides must be multiples of 8 elements (got %lld, %lld)", (long long)batch_stride_q,
            (long long)batch_stride_k);
    REQUIRE(batch_stride_q >= (int64_t)n_tokens * ld_q && batch_stride_k >= (int64_t)n_tokens * ld_k,
            LEMO_ERR_INVALID_ARG, "batch strides (%lld, %lld) smaller than a sequence (%lld, %lld)",
            (long long)batch_stride_q, (long long)batch_stride_k, (long long)n_tokens * ld_q,
            (long long)n_tokens * ld_k);
  }
  float* m_out = block_scores;
  if (!m_out) {
    const size_t need = lemo_block_scores_batched_workspace(n_batch, n_tokens, block);
    REQUIRE(workspace != nullptr && workspace_bytes >= need, LEMO_ERR_WORKSPACE,
            "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
    m_out = static_cast<float*>(workspace);
  }
  return device_status(lemo_launch_block_scores(q, k, n_batch, n_tokens, n_heads, head_dim, ld_q, ld_k,
                                                n_batch > 1 ? batch_stride_q : 0, n_batch > 1 ? batch_stride_k : 0,
                                                block, head_reduce, (flags & LEMO_SCORES_CAUSAL) != 0, m_out, scores,
                                                static_cast<hipStream_t>(stream)),
                       "lemo_block_scores_batched launch");
}

size_t lemo_predict_scores_workspace(int n_tokens, int d_model, int block, int rank) {
  if (n_tokens <= 0 || block <= 0 || d_model <= 0 || rank <= 0) return 0;
  return lemo_predict_ws_bytes(n_tokens, d_model, block, rank);
}

// Checks shared by lemo_predict_scores and lemo_predict_scores_noalloc.
static lemo_status predict_checks(const lemo_bf16* x, int n_tokens, int d_model, int ld_x, int block,
                                  const lemo_bf16* u_q, const lemo_bf16* v_q, const lemo_bf16* u_k,
                                  const lemo_bf16* v_k, int rank, const float* scores) {
  REQUIRE(scores != nullptr && u_q && v_q && u_k && v_k, LEMO_ERR_INVALID_ARG, "scores or a predictor matrix is NULL");
  REQUIRE(n_tokens > 0 && block > 0 && d_model > 0 && rank > 0, LEMO_ERR_INVALID_ARG,
          "sizes must be positive (n_tokens=%d block=%d d_model=%d rank=%d)", n_tokens, block, d_model, rank);
  REQUIRE(pow2(block) && block >= 2 && block <= 256, LEMO_ERR_UNSUPPORTED, "block %d (power of two, 2..256)", block);
  REQUIRE(d_model % 64 == 0, LEMO_ERR_UNSUPPORTED, "d_model %d (multiple of 64 supported)", d_model);
  REQUIRE(rank % 32 == 0 && rank <= 256, LEMO_ERR_UNSUPPORTED, "rank %d (multiple of 32, at most 256)", rank);
  REQUIRE(lemo_nblocks(n_tokens, block) <= 65535, LEMO_ERR_UNSUPPORTED, "%d blocks (at most 65535)",
          lemo_nblocks(n_tokens, block));
  lemo_status st;
  if ((st = check_rows(x, ld_x, d_model, "x")) != LEMO_OK) return st;
  REQUIRE(aligned16(u_q) && aligned16(v_q) && aligned16(u_k) && aligned16(v_k), LEMO_ERR_ALIGNMENT,
          "predictor matrices must be 16-byte aligned");
  return LEMO_OK;
}

lemo_status lemo_predict_scores(const lemo_bf16* x, int n_tokens, int d_model, int ld_x, int block,
                                const lemo_bf16* u_q, const lemo_bf16* v_q, const lemo_bf16* u_k,
                                const lemo_bf16* v_k, int rank, float* block_scores, float* scores,
                                void* workspace, size_t workspace_bytes, void* stream) {
  lemo_status st = predict_checks(x, n_tokens, d_model, ld_x, block, u_q, v_q, u_k, v_k, rank, scores);
  if (st != LEMO_OK) return st;
  const size_t need = lemo_predict_ws_bytes(n_tokens, d_model, block, rank);
  REQUIRE(workspace != nullptr && workspace_bytes >= need, LEMO_ERR_WORKSPACE,
          "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
  REQUIRE(aligned16(workspace), LEMO_ERR_ALIGNMENT, "workspace must be 16-byte aligned");
  return device_status(lemo_launch_predict(x, n_tokens, d_model, ld_x, block, u_q, v_q, u_k, v_k, rank, block_scores,
                                           scores, workspace, static_cast<hipStream_t>(stream)),
                       "lemo_predict_scores launch");
}

lemo_status lemo_predict_scores_noalloc(const lemo_bf16* x, int n_tokens, int d_model, int ld_x, int block,
                                        const lemo_bf16* u_q, const lemo_bf16* v_q, const lemo_bf16* u_k,
                                        const lemo_bf16* v_k, int rank, float* block_scores, float* scores,
                                        void* stream) {
  lemo_status st = predict_checks(x, n_tokens, d_model, ld_x, block, u_q, v_q, u_k, v_k, rank, scores);
  if (st != LEMO_OK) return st;
  const size_t need = lemo_predict_ws_bytes(n_tokens, d_model, block, rank);
  REQUIRE(need <= lemo_predict_static_capacity(), LEMO_ERR_UNSUPPORTED,
          "this shape needs %zu bytes of scratch; the static scratch holds %zu (use lemo_predict_scores with a "
          "workspace)", need, lemo_predict_static_capacity());
  void* scratch = nullptr;
  if ((st = device_status(lemo_predict_static_scratch(&scratch), "lemo_predict_scores_noalloc scratch lookup")) !=
      LEMO_OK)
    return st;
  return device_status(lemo_launch_predict(x, n_tokens, d_model, ld_x, block, u_q, v_q, u_k, v_k, rank, block_scores,
                                           scores, scratch, static_cast<hipStream_t>(stream)),
                       "lemo_predict_scores_noalloc launch");
}

size_t lemo_token_embeddings_workspace(int n_tokens, int d_model, int rank) {
  if (n_tokens <= 0 || d_model <= 0 || rank <= 0) return 0;
  return lemo_token_ws_bytes(n_tokens, d_model, rank);
}

lemo_status lemo_token_embeddings(const lemo_bf16* x, int n_tokens, int d_model, int ld_x, const lemo_bf16* u_q,
                                  const lemo_bf16* v_q, const lemo_bf16* u_k, const lemo_bf16* v_k, int rank,
                                  lemo_bf16* q_hat, lemo_bf16* k_hat, int ld_out, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  REQUIRE(u_q && v_q && u_k && v_k, LEMO_ERR_INVALID_ARG, "a predictor matrix is NULL");
  REQUIRE(n_tokens > 0 && d_model > 0 && rank > 0, LEMO_ERR_INVALID_ARG,
          "sizes must be positive (n_tokens=%d d_model=%d rank=%d)", n_tokens, d_model, rank);
  REQUIRE(d_model % 64 == 0, LEMO_ERR_UNSUPPORTED, "d_model %d (multiple of 64 supported)", d_model);
  REQUIRE(rank % 64 == 0 && rank <= 256, LEMO_ERR_UNSUPPORTED, "rank %d (multiple of 64, at most 256)", rank);
  lemo_status st;
  if ((st = check_rows(x, ld_x, d_model, "x")) != LEMO_OK) return st;
  if ((st = check_offsets(n_tokens, ld_x, "x")) != LEMO_OK) return st;
  if ((st = check_offsets(n_tokens, 2 * rank, "hidden layer")) != LEMO_OK) return st;
  REQUIRE(lemo_nblocks(n_tokens, 64) * (long long)((2 * rank + 127) / 128) <= kMaxWorkgroups, LEMO_ERR_UNSUPPORTED,
          "n_tokens %d: too many tiles for one launch", n_tokens);
  if ((st = check_rows(q_hat, ld_out, rank, "q_hat")) != LEMO_OK) return st;
  if ((st = check_rows(k_hat, ld_out, rank, "k_hat")) != LEMO_OK) return st;
  REQUIRE(aligned16(u_q) && aligned16(v_q) && aligned16(u_k) && aligned16(v_k), LEMO_ERR_ALIGNMENT,
          "predictor matrices must be 16-byte aligned");
  const size_t need = lemo_token_ws_bytes(n_tokens, d_model, rank);
  if (need > 0) {
    REQUIRE(workspace != nullptr && workspace_bytes >= need, LEMO_ERR_WORKSPACE,
            "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
    REQUIRE(aligned16(workspace), LEMO_ERR_ALIGNMENT, "workspace must be 16-byte aligned");
  }
  return device_status(lemo_launch_token_embed(x, n_tokens, d_model, ld_x, u_q, v_q, u_k, v_k, rank, q_hat, k_hat,
                                               ld_out, workspace, static_cast<hipStream_t>(stream)),
                       "lemo_token_embeddings launch");
}

lemo_status lemo_select_mask(const float* scores, int n_blocks, int mode, float threshold, int keep_blocks,
                             uint8_t* mask, int32_t* kept_blocks, int32_t* n_kept, float* threshold_used,
                             int32_t* dev_status, void* stream) {
  REQUIRE(scores && mask && kept_blocks && n_kept, LEMO_ERR_INVALID_ARG, "scores, mask, kept_blocks or n_kept is NULL");
  REQUIRE(n_blocks > 0, LEMO_ERR_INVALID_ARG, "n_blocks must be positive (got %d)", n_blocks);
  REQUIRE(n_blocks <= 8192, LEMO_ERR_UNSUPPORTED, "n_blocks %d (at most 8192)", n_blocks);
  REQUIRE(mode == LEMO_SELECT_THRESHOLD || mode == LEMO_SELECT_TOPK || mode == LEMO_SELECT_MEAN,
          LEMO_ERR_INVALID_ARG, "unknown select mode %d", mode);
  REQUIRE(mode != LEMO_SELECT_TOPK || (keep_blocks >= 0 && keep_blocks <= n_blocks), LEMO_ERR_INVALID_ARG,
          "keep_blocks %d outside 0..%d", keep_blocks, n_blocks);
  return device_status(lemo_launch_select(scores, n_blocks, mode, threshold, keep_blocks, mask, kept_blocks, n_kept,
                                          threshold_used, dev_status, static_cast<hipStream_t>(stream)),
                       "lemo_select_mask launch");
}

lemo_status lemo_gather_pad(const lemo_bf16* src, int n_tokens, int width, int ld_src, int block,
                            const int32_t* kept_blocks, const int32_t* n_kept, lemo_bf16* dst, int ld_dst,
                            int cap_rows, int pad_multiple, int32_t* dev_status, void* stream) {
  REQUIRE(kept_blocks && n_kept, LEMO_ERR_INVALID_ARG, "kept_blocks or n_kept is NULL");
  REQUIRE(n_tokens > 0 && block > 0 && width > 0 && cap_rows > 0 && pad_multiple > 0, LEMO_ERR_INVALID_ARG,
          "sizes must be positive (n_tokens=%d block=%d width=%d cap_rows=%d pad_multiple=%d)", n_tokens, block,
          width, cap_rows, pad_multiple);
  REQUIRE(width % 8 == 0, LEMO_ERR_ALIGNMENT, "width %d must be a multiple of 8", width);
  lemo_status st;
  if ((st = check_rows(src, ld_src, width, "src")) != LEMO_OK) return st;
  if ((st = check_rows(dst, ld_dst, width, "dst")) != LEMO_OK) return st;
  return device_status(lemo_launch_gather(src, n_tokens, width, ld_src, block, kept_blocks, n_kept, dst, ld_dst,
                                          cap_rows, pad_multiple, dev_status, static_cast<hipStream_t>(stream)),
                       "lemo_gather_pad launch");
}

lemo_status lemo_gather_pad_multi(int n_src, const lemo_bf16* const* srcs, const int* widths, const int* ld_srcs,
                                  lemo_bf16* const* dsts, const int* ld_dsts, int n_tokens, int block,
                                  const int32_t* kept_blocks, const int32_t* n_kept, int cap_rows, int pad_multiple,
                                  int32_t* dev_status, void* stream) {
  REQUIRE(n_src >= 1 && n_src <= 4, LEMO_ERR_INVALID_ARG, "n_src %d (1..4)", n_src);
  REQUIRE(srcs && widths && ld_srcs && dsts && ld_dsts, LEMO_ERR_INVALID_ARG, "an argument array is NULL");
  REQUIRE(kept_blocks && n_kept, LEMO_ERR_INVALID_ARG, "kept_blocks or n_kept is NULL");
  REQUIRE(n_tokens > 0 && block > 0 && cap_rows > 0 && pad_multiple > 0, LEMO_ERR_INVALID_ARG,
          "sizes must be positive (n_tokens=%d block=%d cap_rows=%d pad_multiple=%d)", n_tokens, block, cap_rows,
          pad_multiple);
  for (int i = 0; i < n_src; ++i) {
    REQUIRE(widths[i] > 0, LEMO_ERR_INVALID_ARG, "width of source %d must be positive (got %d)", i, widths[i]);
    REQUIRE(widths[i] % 8 == 0, LEMO_ERR_ALIGNMENT, "width %d of source %d must be a multiple of 8", widths[i], i);
    lemo_status st;
    if ((st = check_rows(srcs[i], ld_srcs[i], widths[i], "src")) != LEMO_OK) return st;
    if ((st = check_rows(dsts[i], ld_dsts[i], widths[i], "dst")) != LEMO_OK) return st;
  }
  return device_status(lemo_launch_gather_multi(n_src, reinterpret_cast<const uint16_t* const*>(srcs), widths,
                                                ld_srcs, reinterpret_cast<uint16_t* const*>(dsts), ld_dsts, n_tokens,
                                                block, kept_blocks, n_kept, cap_rows, pad_multiple, dev_status,
                                                static_cast<hipStream_t>(stream)),
                       "lemo_gather_pad_multi launch");
}

// The scatter and the recompute: y holds y_rows rows (INT_MAX: the caller
// guarantees at least the kept rows).
static lemo_status scatter_common(const char* fn, lemo_bf16* residual, int n_tokens, int width, int ld_res, int block,
                                  const int32_t* kept_blocks, const int32_t* n_kept, const lemo_bf16* y, int ld_y,
                                  int y_rows, int32_t* dev_status, void* stream, bool subtract) {
  REQUIRE(kept_blocks && n_kept, LEMO_ERR_INVALID_ARG, "kept_blocks or n_kept is NULL");
  REQUIRE(n_tokens > 0 && block > 0 && width > 0, LEMO_ERR_INVALID_ARG,
          "sizes must be positive (n_tokens=%d block=%d width=%d)", n_tokens, block, width);
  REQUIRE(y_rows >= 0, LEMO_ERR_INVALID_ARG, "y_rows must not be negative (got %d)", y_rows);
  REQUIRE(width % 8 == 0, LEMO_ERR_ALIGNMENT, "width %d must be a multiple of 8", width);
  lemo_status st;
  if ((st = check_rows(residual, ld_res, width, "residual")) != LEMO_OK) return st;
  if ((st = check_rows(y, ld_y, width, "y")) != LEMO_OK) return st;
  return device_status(lemo_launch_scatter(residual, n_tokens, width, ld_res, block, kept_blocks, n_kept, y, ld_y,
                                           y_rows, dev_status, static_cast<hipStream_t>(stream), subtract),
                       fn);
}

lemo_status lemo_scatter_residual(lemo_bf16* residual, int n_tokens, int width, int ld_res, int block,
                                  const int32_t* kept_blocks, const int32_t* n_kept, const lemo_bf16* y, int ld_y,
                                  int32_t* dev_status, void* stream) {
  return scatter_common("lemo_scatter_residual launch", residual, n_tokens, width, ld_res, block, kept_blocks, n_kept,
                        y, ld_y, INT_MAX, dev_status, stream, false);
}

lemo_status lemo_scatter_residual_capped(lemo_bf16* residual, int n_tokens, int width, int ld_res, int block,
                                         const int32_t* kept_blocks, const int32_t* n_kept, const lemo_bf16* y,
                                         int ld_y, int y_rows, int32_t* dev_status, void* stream) {
  return scatter_common("lemo_scatter_residual_capped launch", residual, n_tokens, width, ld_res, block, kept_blocks,
                        n_kept, y, ld_y, y_rows, dev_status, stream, false);
}

lemo_status lemo_residual_recompute(lemo_bf16* residual, int n_tokens, int width, int ld_res, int block,
                                   const int32_t* kept_blocks, const int32_t* n_kept, const lemo_bf16* y, int ld_y,
                                   int32_t* dev_status, void* stream) {
  return scatter_common("lemo_residual_recompute launch", residual, n_tokens, width, ld_res, block, kept_blocks,
                        n_kept, y, ld_y, INT_MAX, dev_status, stream, true);
}

lemo_status lemo_residual_recompute_capped(lemo_bf16* residual, int n_tokens, int width, int ld_res, int block,
                                          const int32_t* kept_blocks, const int32_t* n_kept, const lemo_bf16* y,
                                          int ld_y, int y_rows, int32_t* dev_status, void* stream) {
  return scatter_common("lemo_residual_recompute_capped launch", residual, n_tokens, width, ld_res, block,
                        kept_blocks, n_kept, y, ld_y, y_rows, dev_status, stream, true);
}

size_t lemo_mlp_block_scores_workspace(int n_tokens, int width, int block) {
  if (n_tokens <= 0 || width <= 0 || block <= 0) return 0;
  const size_t nb = (size_t)lemo_nblocks(n_tokens, block);
  return lemo_align256(nb * lemo_mlp_chunks(width) * sizeof(float));
}

static lemo_status mlp_scores(const char* fn, const lemo_bf16* act, int ld_act, const lemo_bf16* up, int ld_up,
                              int n_tokens, int width, int block, float* scores, void* workspace,
                              size_t workspace_bytes, void* stream) {
  REQUIRE(scores != nullptr, LEMO_ERR_INVALID_ARG, "scores is NULL");
  REQUIRE(n_tokens > 0 && block > 0 && width > 0, LEMO_ERR_INVALID_ARG,
          "sizes must be positive (n_tokens=%d block=%d width=%d)", n_tokens, block, width);
  REQUIRE(width % 8 == 0, LEMO_ERR_ALIGNMENT, "width %d must be a multiple of 8", width);
  REQUIRE(lemo_mlp_chunks(width) <= 65535, LEMO_ERR_UNSUPPORTED, "width %d too large", width);
  REQUIRE(lemo_nblocks(n_tokens, block) <= kMaxWorkgroups, LEMO_ERR_UNSUPPORTED, "%d blocks (at most %lld)",
          lemo_nblocks(n_tokens, block), kMaxWorkgroups);
  lemo_status st;
  if ((st = check_rows(act, ld_act, width, up ? "gate" : "act")) != LEMO_OK) return st;
  if (up && (st = check_rows(up, ld_up, width, "up")) != LEMO_OK) return st;
  const size_t need = lemo_mlp_block_scores_workspace(n_tokens, width, block);
  REQUIRE(workspace != nullptr && workspace_bytes >= need, LEMO_ERR_WORKSPACE,
          "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
  REQUIRE(aligned16(workspace), LEMO_ERR_ALIGNMENT, "workspace must be 16-byte aligned");
  return device_status(lemo_launch_mlp_scores(act, ld_act, up, ld_up, n_tokens, width, block, scores, workspace,
                                              static_cast<hipStream_t>(stream)),
                       fn);
}

lemo_status lemo_mlp_block_scores(const lemo_bf16* act, int n_tokens, int width, int ld_act, int block,
                                  float* scores, void* workspace, size_t workspace_bytes, void* stream) {
  return mlp_scores("lemo_mlp_block_scores launch", act, ld_act, nullptr, 0, n_tokens, width, block, scores,
                    workspace, workspace_bytes, stream);
}

lemo_status lemo_mlp_block_scores_gated(const lemo_bf16* gate, const lemo_bf16* up, int n_tokens, int width,
                                        int ld_gate, int ld_up, int block, float* scores, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  REQUIRE(up != nullptr, LEMO_ERR_INVALID_ARG, "up is NULL");
  return mlp_scores("lemo_mlp_block_scores_gated launch", gate, ld_gate, up, ld_up, n_tokens, width, block, scores,
                    workspace, workspace_bytes, stream);
}

lemo_status lemo_gather_linear(const lemo_bf16* x, int n_tokens, int d_in, int ld_x, int block,
                               const int32_t* kept_blocks, const int32_t* n_kept, const lemo_bf16* weight,
                               int d_out, int ld_w, lemo_bf16* y, int ld_y, int cap_rows, int pad_multiple,
                               int32_t* dev_status, void* stream) {
  REQUIRE(kept_blocks && n_kept, LEMO_ERR_INVALID_ARG, "kept_blocks or n_kept is NULL");
  REQUIRE(n_tokens > 0 && block > 0 && d_in > 0 && d_out > 0 && cap_rows > 0 && pad_multiple > 0,
          LEMO_ERR_INVALID_ARG, "sizes must be positive (n_tokens=%d block=%d d_in=%d d_out=%d cap_rows=%d pad=%d)",
          n_tokens, block, d_in, d_out, cap_rows, pad_multiple);
  REQUIRE(d_in % 64 == 0, LEMO_ERR_UNSUPPORTED, "d_in %d (multiple of 64 supported)", d_in);
  REQUIRE(d_out % 8 == 0, LEMO_ERR_ALIGNMENT, "d_out %d must be a multiple of 8", d_out);
  REQUIRE((long long)lemo_nblocks(cap_rows, 256) * lemo_nblocks(d_out, 256) <= kMaxFusedWorkgroups, LEMO_ERR_UNSUPPORTED,
          "cap_rows %d x d_out %d: more than %lld tiles of 256 x 256 for one launch", cap_rows, d_out,
          kMaxFusedWorkgroups);
  lemo_status st;
  if ((st = check_rows(x, ld_x, d_in, "x")) != LEMO_OK) return st;
  if ((st = check_rows(weight, ld_w, d_in, "weight")) != LEMO_OK) return st;
  if ((st = check_rows(y, ld_y, d_out, "y")) != LEMO_OK) return st;
  if ((st = check_offsets(n_tokens, ld_x, "x")) != LEMO_OK) return st;
  if ((st = check_offsets(d_out, ld_w, "weight")) != LEMO_OK) return st;
  return device_status(lemo_launch_gather_linear(x, n_tokens, d_in, ld_x, block, kept_blocks, n_kept, weight, d_out,
                                                 ld_w, y, ld_y, cap_rows, pad_multiple, dev_status,
                                                 static_cast<hipStream_t>(stream)),
                       "lemo_gather_linear launch");
}

lemo_status lemo_linear_scatter(const lemo_bf16* a, int d_in, int ld_a, int cap_rows, const lemo_bf16* weight,
                                int d_out, int ld_w, lemo_bf16* residual, int n_tokens, int ld_res, int block,
                                const int32_t* kept_blocks, const int32_t* n_kept, int32_t* dev_status,
                                void* stream) {
  REQUIRE(kept_blocks && n_kept, LEMO_ERR_INVALID_ARG, "kept_blocks or n_kept is NULL");
  REQUIRE(n_tokens > 0 && block > 0 && d_in > 0 && d_out > 0 && cap_rows > 0, LEMO_ERR_INVALID_ARG,
          "sizes must be positive (n_tokens=%d block=%d d_in=%d d_out=%d cap_rows=%d)", n_tokens, block, d_in, d_out,
          cap_rows);
  REQUIRE(d_in % 64 == 0, LEMO_ERR_UNSUPPORTED, "d_in %d (multiple of 64 supported)", d_in);
  REQUIRE(d_out % 8 == 0, LEMO_ERR_ALIGNMENT, "d_out %d must be a multiple of 8", d_out);
  // the product covers min(cap_rows, n_tokens) rows (no more rows can be kept)
  const long long prod_rows = cap_rows < n_tokens ? cap_rows : n_tokens;
  REQUIRE((prod_rows + 255) / 256 * lemo_nblocks(d_out, 256) <= kMaxFusedWorkgroups, LEMO_ERR_UNSUPPORTED,
          "%lld rows x d_out %d: more than %lld tiles of 256 x 256 for one launch", prod_rows, d_out,
          kMaxFusedWorkgroups);
  lemo_status st;
  if ((st = check_rows(a, ld_a, d_in, "a")) != LEMO_OK) return st;
  if ((st = check_rows(weight, ld_w, d_in, "weight")) != LEMO_OK) return st;
  if ((st = check_rows(residual, ld_res, d_out, "residual")) != LEMO_OK) return st;
  if ((st = check_offsets(cap_rows, ld_a, "a")) != LEMO_OK) return st;
  if ((st = check_offsets(d_out, ld_w, "weight")) != LEMO_OK) return st;
  return device_status(lemo_launch_linear_scatter(a, d_in, ld_a, cap_rows, weight, d_out, ld_w, residual, n_tokens,
                                                  ld_res, block, kept_blocks, n_kept, dev_status,
                                                  static_cast<hipStream_t>(stream)),
                       "lemo_linear_scatter launch");
}

}  // extern "C"
