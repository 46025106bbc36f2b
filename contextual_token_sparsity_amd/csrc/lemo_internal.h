// Internal declarations shared by the HIP translation units of liblemo.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "lemo.h"

typedef __bf16 lemo_bf16x8 __attribute__((ext_vector_type(8)));
typedef short lemo_i16x8 __attribute__((ext_vector_type(8)));
typedef float lemo_f32x16 __attribute__((ext_vector_type(16)));
typedef float lemo_f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int lemo_u32x4 __attribute__((ext_vector_type(4)));

// Streaming 16-byte accesses for data touched once: the nontemporal hint keeps
// it from displacing other data in L2 and the Infinity Cache (measured ~10-20 %
// faster than plain accesses when the source is not already cached).
__device__ __forceinline__ uint4 lemo_load_stream(const uint16_t* p) {
  const lemo_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const lemo_u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void lemo_store_stream(uint16_t* p, uint4 v) {
  const lemo_u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<lemo_u32x4*>(p));
}

// bf16 pattern -> fp32 value (exact).
__device__ __forceinline__ float lemo_bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 pattern, round to nearest even.  Adding 0x7FFF plus the
// lowest kept bit carries into the kept part exactly when the dropped half
// is above the midpoint, or at it with an odd kept part; a carry out of the
// significand moves to the next binade (and to infinity past the largest
// finite value), as rounding requires.  NaN is kept a quiet NaN.
__device__ __forceinline__ uint32_t lemo_f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Full-wave (64 lanes) maximum.
__device__ __forceinline__ float lemo_wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// Launchers (validated arguments only; return the hipError_t of the launch).
// n_batch sequences, sequence b at q + b*bs_q and k + b*bs_k (elements); M
// and the scores of sequence b at m_out + b*nb*nb and scores + b*nb, where
// nb = ceil(n_tokens / block).
hipError_t lemo_launch_block_scores(const uint16_t* q, const uint16_t* k, int n_batch, int n_tokens, int n_heads,
                                    int head_dim, int ld_q, int ld_k, long long bs_q, long long bs_k, int block,
                                    int head_reduce, bool causal, float* m_out, float* scores, hipStream_t stream);

int lemo_predict_splitk(int nb, int d_model, int rank);
size_t lemo_predict_ws_bytes(int n_tokens, int d_model, int block, int rank);
hipError_t lemo_launch_predict(const uint16_t* x, int n_tokens, int d_model, int ld_x, int block,
                               const uint16_t* u_q, const uint16_t* v_q, const uint16_t* u_k,
                               const uint16_t* v_k, int rank, float* m_out, float* scores,
                               void* workspace, hipStream_t stream);

// lemo_predict_scores_noalloc: capacity of the static scratch array, and its
// device address on the current device (looked up once per device)
size_t lemo_predict_static_capacity();
hipError_t lemo_predict_static_scratch(void** ptr);

size_t lemo_token_ws_bytes(int n_tokens, int d_model, int rank);
hipError_t lemo_launch_token_embed(const uint16_t* x, int n_tokens, int d_model, int ld_x, const uint16_t* u_q,
                                   const uint16_t* v_q, const uint16_t* u_k, const uint16_t* v_k, int rank,
                                   uint16_t* q_hat, uint16_t* k_hat, int ld_out, void* workspace,
                                   hipStream_t stream);

hipError_t lemo_launch_gather_linear(const uint16_t* x, int n_tokens, int d_in, int ld_x, int block,
                                     const int32_t* kept, const int32_t* n_kept, const uint16_t* w, int d_out,
                                     int ld_w, uint16_t* y, int ld_y, int cap_rows, int pad_multiple,
                                     int32_t* dev_status, hipStream_t stream);
hipError_t lemo_launch_linear_scatter(const uint16_t* a, int d_in, int ld_a, int cap_rows, const uint16_t* w,
                                      int d_out, int ld_w, uint16_t* res, int n_tokens, int ld_res, int block,
                                      const int32_t* kept, const int32_t* n_kept, int32_t* dev_status,
                                      hipStream_t stream);

hipError_t lemo_launch_select(const float* scores, int n_blocks, int mode, float threshold,
                              int keep_blocks, uint8_t* mask, int32_t* kept, int32_t* n_kept,
                              float* threshold_used, int32_t* dev_status, hipStream_t stream);

hipError_t lemo_launch_gather(const uint16_t* src, int n_tokens, int width, int ld_src, int block,
                              const int32_t* kept, const int32_t* n_kept, uint16_t* dst, int ld_dst,
                              int cap_rows, int pad_multiple, int32_t* dev_status, hipStream_t stream);
// n_src (1..4) matrices gathered on one kept list in one launch (each with its
// own width, leading dimensions and destination; same cap_rows and padding)
hipError_t lemo_launch_gather_multi(int n_src, const uint16_t* const* srcs, const int* widths, const int* ld_srcs,
                                    uint16_t* const* dsts, const int* ld_dsts, int n_tokens, int block,
                                    const int32_t* kept, const int32_t* n_kept, int cap_rows, int pad_multiple,
                                    int32_t* dev_status, hipStream_t stream);

// subtract: the backward recompute res -= y instead of res += y.  y holds
// y_rows rows (kept rows past them are skipped and flag a capacity overflow).
hipError_t lemo_launch_scatter(uint16_t* res, int n_tokens, int width, int ld_res, int block,
                               const int32_t* kept, const int32_t* n_kept, const uint16_t* y, int ld_y,
                               int y_rows, int32_t* dev_status, hipStream_t stream, bool subtract = false);

// MLP-block scores: act [n_tokens][ld_act]; with `up` non-NULL, act is the
// gate projection and the activation is SiLU(act) * up.  Workspace: fp32
// partials [ceil(n_tokens / block)][lemo_mlp_chunks(width)].
int lemo_mlp_chunks(int width);
hipError_t lemo_launch_mlp_scores(const uint16_t* act, int ld_act, const uint16_t* up, int ld_up, int n_tokens,
                                  int width, int block, float* scores, void* workspace, hipStream_t stream);

hipError_t lemo_launch_colsum(const float* m, int nb, float* out, hipStream_t stream, int n_batch = 1);

static inline size_t lemo_align256(size_t x) { return (x + 255) & ~size_t(255); }

// Blocks of `block` rows covering n rows (n >= 0, block >= 1), formed without
// the int overflow of n + block - 1 for n near INT_MAX.
__host__ __device__ static inline int lemo_nblocks(int n, int block) { return n / block + (n % block != 0); }
