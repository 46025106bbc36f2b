// Exact block-wise token informativeness on the matrix cores (gfx950).
//
// Jenga (USENIX ATC'25), section 4.2.1, Eq. 1 and Eq. 2, Figure 6 caption:
// per head, S^h = Q^h K^h^T / sqrt(head_dim) (raw pre-softmax scores); each
// (block x block) score tile is reduced to one value M[n][m] and the token
// block score is I[m] = sum_n M[n][m].  Pairs i == j are excluded.
//
// Work decomposition: one workgroup owns a 128 x 128 tile of (query rows,
// key rows) and walks all heads.  Per head the Q and K head slices of the
// tile are staged in LDS and four waves each multiply a 64 x 64 sub-tile with
// v_mfma_f32_32x32x16_bf16 (2 x 2 MFMA tiles, fp32 accumulators).  The score
// tile never leaves registers:
//   PAPER   (heads first, then block max): the running sum over heads of
//           max(0, S^h) is kept per element.  Each head's MFMA chain starts
//           from that running sum as its C operand, so after the chain
//           acc = sum + S^h and the update sum = max(acc, sum) costs one VALU
//           op per element and head.
//   HEADMAX (per-head block max): after each head the wave reduces its
//           accumulators to the block maximum of that head; the per-head
//           maxima are clamped at zero and summed after the head loop.
// The i == j pairs sit on the diagonal of diagonal tiles; they are set to 0,
// which leaves both reductions unchanged (PAPER values are >= 0 and HEADMAX
// clamps at 0 after the max).  The scale 1/sqrt(head_dim) (and 1/H for
// PAPER) is applied once to the block value, which is exact up to rounding
// because every step is positively homogeneous.
//
// The column aggregate is a second, deterministic pass (k_colsum).
#include "lemo_internal.h"

namespace {

constexpr int kTile = 128;     // query rows x key rows per workgroup
constexpr int kThreads = 256;  // 4 waves, 2 x 2 arrangement of 64 x 64
constexpr int kMaxHeadsHeadmax = 128;

template <int HD>
struct Cfg {
  static constexpr int kRow = HD + 8;          // LDS row pitch (bf16): +16 B breaks bank aliasing
  static constexpr int kChunks = HD / 8;       // 16-byte chunks per row slice
  static constexpr int kPerThread = kTile * kChunks / kThreads;
};

// Output (row, col) of register `r` of `lane` in a 32x32 MFMA accumulator.
__device__ __forceinline__ int acc_row(int lane, int r) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

template <int HD>
__device__ __forceinline__ void load_head(const uint16_t* __restrict__ base, int ld, int row0, int n_tokens,
                                          int col0, uint4 (&v)[Cfg<HD>::kPerThread]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < Cfg<HD>::kPerThread; ++i) {
    const int c = tid + i * kThreads;
    const int r = c / Cfg<HD>::kChunks;
    const int cc = c % Cfg<HD>::kChunks;
    if (row0 + r < n_tokens)
      v[i] = *reinterpret_cast<const uint4*>(base + (size_t)(row0 + r) * ld + col0 + cc * 8);
    else
      v[i] = make_uint4(0, 0, 0, 0);
  }
}

template <int HD>
__device__ __forceinline__ void store_head(uint16_t* s, const uint4 (&v)[Cfg<HD>::kPerThread]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < Cfg<HD>::kPerThread; ++i) {
    const int c = tid + i * kThreads;
    const int r = c / Cfg<HD>::kChunks;
    const int cc = c % Cfg<HD>::kChunks;
    *reinterpret_cast<uint4*>(s + r * Cfg<HD>::kRow + cc * 8) = v[i];
  }
}

// Maps a linear workgroup id to a (query tile, key tile) pair.  Consecutive
// dispatches go round-robin over the 8 XCDs; this gives each XCD a
// contiguous range of logical tiles, walked in groups of 8 query tiles, so
// that the workgroups resident on one XCD share Q and K rows in its L2.
__device__ __forceinline__ void tile_of(int wg, int ntiles, int& tq, int& tk) {
  const int total = ntiles * ntiles;
  int logical = wg;
  if (total % 8 == 0) logical = (wg % 8) * (total / 8) + wg / 8;
  constexpr int kGroup = 8;
  const int group_span = kGroup * ntiles;
  const int g = logical / group_span;
  const int first = g * kGroup;
  const int rows = min(kGroup, ntiles - first);
  const int in_group = logical % group_span;
  tq = first + in_group % rows;
  tk = in_group / rows;
}

template <int HD, int MODE, int BLK>
__global__ __launch_bounds__(kThreads, 2) void k_block_scores(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, int n_tokens, int n_heads, int ldq,
    int ldk, float out_scale, float* __restrict__ M, int nb, int ntiles) {
  using C = Cfg<HD>;
  __shared__ __attribute__((aligned(16))) uint16_t sQ[kTile * C::kRow];
  __shared__ __attribute__((aligned(16))) uint16_t sK[kTile * C::kRow];
  // Per (wave, MFMA sub-tile) partial block values; HEADMAX keeps one per head.
  constexpr int kParts = (MODE == 0) ? 1 : kMaxHeadsHeadmax;
  __shared__ float part[16][kParts];

  int tq, tk;
  tile_of(blockIdx.x, ntiles, tq, tk);
  const int q0 = tq * kTile, k0 = tk * kTile;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wq = wave >> 1, wk = wave & 1;
  const int l32 = lane & 31, lhi = lane >> 5;
  // A sub-tile holds i == j pairs only if its query and key row ranges coincide.
  const bool diag_wave = (q0 + wq * 64) == (k0 + wk * 64);

  lemo_f32x16 sum[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) sum[a][b][e] = 0.f;

  uint4 vq[C::kPerThread], vk[C::kPerThread];
  load_head<HD>(Q, ldq, q0, n_tokens, 0, vq);
  load_head<HD>(K, ldk, k0, n_tokens, 0, vk);

  for (int h = 0; h < n_heads; ++h) {
    store_head<HD>(sQ, vq);
    store_head<HD>(sK, vk);
    __syncthreads();
    if (h + 1 < n_heads) {  // prefetch the next head while this one multiplies
      load_head<HD>(Q, ldq, q0, n_tokens, (h + 1) * HD, vq);
      load_head<HD>(K, ldk, k0, n_tokens, (h + 1) * HD, vk);
    }
    lemo_f32x16 acc[2][2];
#pragma unroll
    for (int ks = 0; ks < HD / 16; ++ks) {
      lemo_bf16x8 fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        fa[i] = *reinterpret_cast<const lemo_bf16x8*>(sQ + (wq * 64 + i * 32 + l32) * C::kRow + ks * 16 + lhi * 8);
        fb[i] = *reinterpret_cast<const lemo_bf16x8*>(sK + (wk * 64 + i * 32 + l32) * C::kRow + ks * 16 + lhi * 8);
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          if (ks == 0) {
            if (MODE == 0)
              acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a], fb[b], sum[a][b], 0, 0, 0);
            else
              acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a], fb[b], lemo_f32x16{}, 0, 0, 0);
          } else {
            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a], fb[b], acc[a][b], 0, 0, 0);
          }
        }
    }
    __syncthreads();  // LDS is rewritten at the top of the next head

    if (MODE == 0) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int e = 0; e < 16; ++e) sum[a][b][e] = fmaxf(acc[a][b][e], sum[a][b][e]);
    } else {
      if (diag_wave) {
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (acc_row(lane, e) == l32) acc[a][a][e] = 0.f;
      }
      if (BLK >= 64) {
        float m = -INFINITY;
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int e = 0; e < 16; ++e) m = fmaxf(m, acc[a][b][e]);
        m = lemo_wave_max(m);
        if (lane == 0) part[wave * 4][h] = m;
      } else {
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            float m = -INFINITY;
#pragma unroll
            for (int e = 0; e < 16; ++e) m = fmaxf(m, acc[a][b][e]);
            m = lemo_wave_max(m);
            if (lane == 0) part[wave * 4 + a * 2 + b][h] = m;
          }
      }
    }
  }

  if (MODE == 0) {
    if (diag_wave) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (acc_row(lane, e) == l32) sum[a][a][e] = 0.f;
    }
    if (BLK >= 64) {
      float m = 0.f;
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int e = 0; e < 16; ++e) m = fmaxf(m, sum[a][b][e]);
      m = lemo_wave_max(m);
      if (lane == 0) part[wave * 4][0] = m;
    } else {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          float m = 0.f;
#pragma unroll
          for (int e = 0; e < 16; ++e) m = fmaxf(m, sum[a][b][e]);
          m = lemo_wave_max(m);
          if (lane == 0) part[wave * 4 + a * 2 + b][0] = m;
        }
    }
  }
  __syncthreads();

  // Combine the parts that fall in each block of this tile and write M.
  constexpr int kPerDim = kTile / BLK;  // blocks per tile side
  if (tid < kPerDim * kPerDim) {
    const int lq = tid / kPerDim, lk = tid % kPerDim;
    const int bq = q0 / BLK + lq, bk = k0 / BLK + lk;
    if (bq < nb && bk < nb) {
      // parts that cover this block: wave (wq, wk) sub-tile (a, b) covers
      // query rows wq*64 + a*32 and key rows wk*64 + b*32 of the tile
      float val = 0.f;
      if (MODE == 0) {
        for (int p = 0; p < 16; ++p) {
          const int w = p >> 2, a = (p >> 1) & 1, b = p & 1;
          if (BLK >= 64 && (a | b)) continue;
          const int rq = ((w >> 1) * 64 + a * 32) / BLK, rk = ((w & 1) * 64 + b * 32) / BLK;
          if (rq == lq && rk == lk) val = fmaxf(val, part[p][0]);
        }
      } else {
        for (int h = 0; h < n_heads; ++h) {
          float m = -INFINITY;
          for (int p = 0; p < 16; ++p) {
            const int w = p >> 2, a = (p >> 1) & 1, b = p & 1;
            if (BLK >= 64 && (a | b)) continue;
            const int rq = ((w >> 1) * 64 + a * 32) / BLK, rk = ((w & 1) * 64 + b * 32) / BLK;
            if (rq == lq && rk == lk) m = fmaxf(m, part[p][h]);
          }
          val += fmaxf(m, 0.f);
        }
      }
      M[(size_t)bq * nb + bk] = val * out_scale;
    }
  }
}

__global__ void k_colsum(const float* __restrict__ M, int nb, float* __restrict__ out) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= nb) return;
  float s = 0.f;
  for (int r = 0; r < nb; ++r) s += M[(size_t)r * nb + c];
  out[c] = s;
}

template <int HD, int MODE>
hipError_t launch_hd_mode(const uint16_t* q, const uint16_t* k, int n, int h, int ldq, int ldk, int block,
                          float scale, float* m, int nb, hipStream_t st) {
  const int ntiles = (n + kTile - 1) / kTile;
  const dim3 grid(ntiles * ntiles), blk(kThreads);
  switch (block) {
    case 32: hipLaunchKernelGGL((k_block_scores<HD, MODE, 32>), grid, blk, 0, st, q, k, n, h, ldq, ldk, scale, m, nb, ntiles); break;
    case 64: hipLaunchKernelGGL((k_block_scores<HD, MODE, 64>), grid, blk, 0, st, q, k, n, h, ldq, ldk, scale, m, nb, ntiles); break;
    default: hipLaunchKernelGGL((k_block_scores<HD, MODE, 128>), grid, blk, 0, st, q, k, n, h, ldq, ldk, scale, m, nb, ntiles); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t lemo_launch_colsum(const float* m, int nb, float* out, hipStream_t stream) {
  hipLaunchKernelGGL(k_colsum, dim3((nb + 255) / 256), dim3(256), 0, stream, m, nb, out);
  return hipGetLastError();
}

hipError_t lemo_launch_block_scores(const uint16_t* q, const uint16_t* k, int n_tokens, int n_heads,
                                    int head_dim, int ld_q, int ld_k, int block, int head_reduce,
                                    float* m_out, float* scores, hipStream_t stream) {
  const int nb = n_tokens / block;
  const double c = 1.0 / __builtin_sqrt((double)head_dim);
  const float scale = (float)(head_reduce == 0 ? c / n_heads : c);
  hipError_t e;
  if (head_dim == 64)
    e = head_reduce == 0 ? launch_hd_mode<64, 0>(q, k, n_tokens, n_heads, ld_q, ld_k, block, scale, m_out, nb, stream)
                         : launch_hd_mode<64, 1>(q, k, n_tokens, n_heads, ld_q, ld_k, block, scale, m_out, nb, stream);
  else
    e = head_reduce == 0 ? launch_hd_mode<128, 0>(q, k, n_tokens, n_heads, ld_q, ld_k, block, scale, m_out, nb, stream)
                         : launch_hd_mode<128, 1>(q, k, n_tokens, n_heads, ld_q, ld_k, block, scale, m_out, nb, stream);
  if (e != hipSuccess) return e;
  return lemo_launch_colsum(m_out, nb, scores, stream);
}
