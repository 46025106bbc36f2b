// Layer threshold and mask compaction (Jenga, USENIX ATC'25, section 4.2.1,
// "Layer-specific Threshold"; Algorithm 1, step 1 starts every layer's
// threshold at the average token-block score).
//
// One workgroup of 1024 threads (16 waves) handles up to 8192 blocks:
//   * scores are staged in LDS;
//   * the threshold is the caller's, the mean (float64 sum in block order by
//     one lane, then divided and rounded to fp32), or implied by top-k: the
//     rank of block c is the number of blocks that beat it (higher score, or
//     equal score and lower index; NaN loses to every number);
//   * the ascending kept list is built 1024 blocks at a time: a wave ballot
//     of the keep bits, the lane's prefix from the bits below it (mbcnt), and
//     the waves' counts scanned through LDS.
#include "lemo_internal.h"

namespace {

constexpr int kThreads = 1024;
constexpr int kMaxBlocks = 8192;
constexpr int kPerThread = kMaxBlocks / kThreads;

__device__ __forceinline__ bool beats(float a, int ia, float b, int ib) {
  const bool an = a != a, bn = b != b;
  if (an != bn) return bn;
  if (!an && a != b) return a > b;
  return ia < ib;
}

__global__ __launch_bounds__(kThreads) void k_select(const float* __restrict__ scores, int nb, int mode,
                                                     float threshold, int keep, uint8_t* __restrict__ mask,
                                                     int32_t* __restrict__ kept, int32_t* __restrict__ n_kept,
                                                     float* __restrict__ theta_out, int32_t* __restrict__ status) {
  __shared__ float s[kMaxBlocks];
  __shared__ int wave_cnt[kThreads / 64];
  __shared__ float theta_sh;
  __shared__ int nonfinite;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) {
    nonfinite = 0;
    theta_sh = mode == 1 ? INFINITY : threshold;
  }
  __syncthreads();
  bool bad = false;
  for (int c = tid; c < nb; c += kThreads) {
    const float v = scores[c];
    s[c] = v;
    bad |= !__builtin_isfinite(v);
  }
  if (bad) atomicOr(&nonfinite, 1);
  __syncthreads();

  uint32_t topk_bits = 0;
  if (mode == 2) {
    if (tid == 0) {
      double acc = 0.0;
      for (int c = 0; c < nb; ++c) acc += (double)s[c];
      theta_sh = (float)(acc / (double)nb);
    }
  } else if (mode == 1) {
#pragma unroll 1
    for (int j = 0; j < kPerThread; ++j) {
      const int c = tid + j * kThreads;
      if (c >= nb) break;
      const float v = s[c];
      int rank = 0;
      for (int o = 0; o < nb; ++o) rank += beats(s[o], o, v, c) ? 1 : 0;
      if (rank < keep) topk_bits |= 1u << j;
      if (rank == keep - 1) theta_sh = v;  // exactly one block has this rank
    }
  }
  __syncthreads();
  const float theta = theta_sh;

  int base = 0;
  for (int j = 0; j * kThreads < nb; ++j) {
    const int c = tid + j * kThreads;
    bool k = false;
    if (c < nb) {
      k = (mode == 1) ? ((topk_bits >> j) & 1u) : (s[c] >= theta);
      mask[c] = k ? 1 : 0;
    }
    const unsigned long long bal = __ballot(k);
    const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
    if (lane == 0) wave_cnt[wave] = __popcll(bal);
    __syncthreads();
    int woff = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) {
      const int cw = wave_cnt[w];
      woff += (w < wave) ? cw : 0;
      total += cw;
    }
    if (k) kept[base + woff + below] = c;
    base += total;
    __syncthreads();
  }
  if (tid == 0) {
    *n_kept = base;
    if (theta_out) *theta_out = theta;
    if (status && nonfinite) atomicOr(status, LEMO_DEV_NONFINITE);
  }
}

}  // namespace

hipError_t lemo_launch_select(const float* scores, int n_blocks, int mode, float threshold, int keep_blocks,
                              uint8_t* mask, int32_t* kept, int32_t* n_kept, float* threshold_used,
                              int32_t* dev_status, hipStream_t stream) {
  hipLaunchKernelGGL(k_select, dim3(1), dim3(kThreads), 0, stream, scores, n_blocks, mode, threshold, keep_blocks,
                     mask, kept, n_kept, threshold_used, dev_status);
  return hipGetLastError();
}
