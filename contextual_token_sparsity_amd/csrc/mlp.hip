// Token-block scores from the MLP block's intermediate activations (Jenga,
// USENIX ATC'25, section 4.2.1, "Extend to MLP Block": the output of the ReLU
// layer rates the tokens, or for SiLU-gated MLPs the product of the gate
// projection after SiLU and the up projection).  The score of token block m
// is the sum over channels c of the largest magnitude over the block's tokens,
//   I[m] = sum_c max_{i in m} |A[i][c]|,
// the block max of Eq. 2 taken per channel and aggregated along the channels
// as the column aggregate of Figure 6 is.
//
// HBM-bound: one pass over A (or over the gate and up projections, whose
// SiLU product is formed in registers and never stored).  A workgroup owns
// one token block and a 2048-channel chunk: each thread keeps the running
// maxima of 8 adjacent channels (one 16-byte load per row, 8 rows in flight),
// sums them, and the workgroup reduces its 256 sums in a fixed order into one
// partial per (block, chunk).  A second pass adds each block's partials in
// chunk order.  No atomics: the result is deterministic.
#include "lemo_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kCols = 8;                        // channels per thread (16 bytes of bf16)
constexpr int kChunkCols = kThreads * kCols;    // 2048 channels per workgroup
constexpr int kRowsInFlight = 8;

// SiLU(g) u = g u / (1 + e^-g), with the hardware exponential and reciprocal
// (about 1 ulp each) instead of an IEEE division; for g below about -88 the
// denominator is +inf and its reciprocal 0, so the product is 0.
__device__ __forceinline__ float silu_times(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.f + __expf(-g)) * u;
}

// Fixed-order sum of one value per thread of the workgroup: a butterfly
// inside each wave, then the four wave totals in wave order.
__device__ __forceinline__ float block_sum(float v, float* lds) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = v;
  __syncthreads();
  return ((lds[0] + lds[1]) + lds[2]) + lds[3];
}

// partial[m * n_chunks + chunk] = sum over this chunk's channels of the
// block's channel maxima of |A| (GATED: A = SiLU(gate) * up, in fp32).
template <bool GATED>
__global__ __launch_bounds__(kThreads) void k_mlp_partial(const uint16_t* __restrict__ a, int lda,
                                                          const uint16_t* __restrict__ up, int ldu, int n_tokens,
                                                          int width, int block, float* __restrict__ partial) {
  __shared__ float lds[kThreads / 64];
  const int m = blockIdx.x, chunk = blockIdx.y;
  const int col = chunk * kChunkCols + threadIdx.x * kCols;
  const int r0 = m * block, r1 = min(r0 + block, n_tokens);
  // plain: running max of the magnitude bits (sign cleared), which order like
  // the magnitudes; gated: running max of |SiLU(g) u| in fp32
  uint32_t mbits[kCols] = {};
  float mval[kCols] = {};
  if (col < width) {
    for (int r = r0; r < r1; r += kRowsInFlight) {
      uint4 va[kRowsInFlight], vu[kRowsInFlight];
#pragma unroll
      for (int u = 0; u < kRowsInFlight; ++u) {
        if (r + u < r1) {
          va[u] = lemo_load_stream(a + (size_t)(r + u) * lda + col);
          if (GATED) vu[u] = lemo_load_stream(up + (size_t)(r + u) * ldu + col);
        }
      }
#pragma unroll
      for (int u = 0; u < kRowsInFlight; ++u) {
        if (r + u >= r1) break;
        const uint32_t* pa = &va[u].x;
        const uint32_t* pu = &vu[u].x;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (GATED) {
            const float lo = silu_times(lemo_bf16_to_f32(pa[j] & 0xffffu), lemo_bf16_to_f32(pu[j] & 0xffffu));
            const float hi = silu_times(lemo_bf16_to_f32(pa[j] >> 16), lemo_bf16_to_f32(pu[j] >> 16));
            mval[2 * j] = fmaxf(mval[2 * j], fabsf(lo));
            mval[2 * j + 1] = fmaxf(mval[2 * j + 1], fabsf(hi));
          } else {
            mbits[2 * j] = max(mbits[2 * j], pa[j] & 0x7fffu);
            mbits[2 * j + 1] = max(mbits[2 * j + 1], (pa[j] >> 16) & 0x7fffu);
          }
        }
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kCols; ++j) s += GATED ? mval[j] : lemo_bf16_to_f32(mbits[j]);
  const float total = block_sum(s, lds);
  if (threadIdx.x == 0) partial[(size_t)m * gridDim.y + chunk] = total;
}

// I[m] = partials of block m added in chunk order.
__global__ __launch_bounds__(256) void k_mlp_final(const float* __restrict__ partial, int nb, int n_chunks,
                                                   float* __restrict__ scores) {
  const int m = blockIdx.x * 256 + threadIdx.x;
  if (m >= nb) return;
  float s = 0.f;
  for (int c = 0; c < n_chunks; ++c) s += partial[(size_t)m * n_chunks + c];
  scores[m] = s;
}

}  // namespace

int lemo_mlp_chunks(int width) { return lemo_nblocks(width, kChunkCols); }

hipError_t lemo_launch_mlp_scores(const uint16_t* act, int ld_act, const uint16_t* up, int ld_up, int n_tokens,
                                  int width, int block, float* scores, void* workspace, hipStream_t stream) {
  const int nb = lemo_nblocks(n_tokens, block);
  const int n_chunks = lemo_mlp_chunks(width);
  float* partial = static_cast<float*>(workspace);
  const dim3 grid(nb, n_chunks);
  if (up)
    hipLaunchKernelGGL(k_mlp_partial<true>, grid, dim3(kThreads), 0, stream, act, ld_act, up, ld_up, n_tokens, width,
                       block, partial);
  else
    hipLaunchKernelGGL(k_mlp_partial<false>, grid, dim3(kThreads), 0, stream, act, ld_act, up, ld_up, n_tokens,
                       width, block, partial);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_mlp_final, dim3((nb + 255) / 256), dim3(256), 0, stream, partial, nb, n_chunks, scores);
  return hipGetLastError();
}
