// Predicted block scores (Jenga, USENIX ATC'25, section 4.2.2, Eq. 3 and
// Figure 8): a representative embedding per token block goes through a query
// and a key predictor (low-rank matrices with a ReLU between them); the
// product of the two outputs estimates the score of every block pair, which
// is aggregated along the column like the exact scores.
//
// Pipeline (all on the caller's stream, workspace carved by the host):
//   k_pool        xbar[m] = bf16((sum of the block's rows, fp32, in row order) / its row
//                 count: block, or fewer for the last block of a ragged sequence)
//                 -- one pass over X, the only HBM-heavy phase.
//   k_hidden      part[s][m][n] = xbar[m, Ks] . [U_q | U_k][Ks, n]  (bf16 MFMA,
//                 split over s = slices Ks of d_model so that ~1000 waves run)
//   k_project     hid = bf16(max(0, sum_s part[s])) (fixed slice order), then
//                 q_hat = hid_q V_q, k_hat = hid_k V_k in fp32
//   k_pair        M_hat[m][n] = max(0, q_hat[m] . k_hat[n])  (fp32, 16 x 16 tiles)
//   k_colsum      I_hat[n] = sum_m M_hat[m][n]
#include "lemo_internal.h"

namespace {

// ---------------------------------------------------------------- pooling
// One thread owns 8 adjacent columns of one block and walks the block's rows
// in order, so every column sum is formed in the same order as a sequential
// loop.  64 threads cover 512 columns; the grid is (column groups, blocks).
__global__ __launch_bounds__(64) void k_pool(const uint16_t* __restrict__ X, int ld, int d, int block,
                                             int n_tokens, float inv_block, uint16_t* __restrict__ xbar) {
  const int m = blockIdx.y;
  const int c8 = blockIdx.x * 64 + threadIdx.x;
  if (c8 * 8 >= d) return;
  const uint16_t* p = X + (size_t)m * block * ld + c8 * 8;
  // the last block of a ragged sequence holds only the remaining rows
  const int rows = min(block, n_tokens - m * block);
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
#pragma unroll 8
  for (int i = 0; i < rows; ++i) {
    const uint4 v = *reinterpret_cast<const uint4*>(p + (size_t)i * ld);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[2 * j] += lemo_bf16_to_f32(w[j] & 0xffffu);
      acc[2 * j + 1] += lemo_bf16_to_f32(w[j] >> 16);
    }
  }
  // a whole block: times 1/block, exact for its power-of-two size; a short
  // one: an IEEE division by its row count
  if (rows == block) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] *= inv_block;
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = acc[j] / (float)rows;
  }
  uint4 o;
  uint32_t* ow = &o.x;
#pragma unroll
  for (int j = 0; j < 4; ++j) ow[j] = lemo_f32_to_bf16(acc[2 * j]) | (lemo_f32_to_bf16(acc[2 * j + 1]) << 16);
  *reinterpret_cast<uint4*>(xbar + (size_t)m * d + c8 * 8) = o;
}

// ------------------------------------------------------- hidden (split-K)
// Each wave computes one 32 x 32 tile (rows = blocks, cols = predictor
// neurons; cols < rank from U_q, the rest from U_k) over one slice of the
// model dimension with v_mfma_f32_32x32x16_bf16.  The B operand (a column
// of U) is strided in memory: each lane gathers its 8 k-values with 2-byte
// loads, coalesced across the 32 lanes that share a k.
__global__ __launch_bounds__(256) void k_hidden(const uint16_t* __restrict__ xbar, int d, int nb,
                                                const uint16_t* __restrict__ uq, const uint16_t* __restrict__ uk,
                                                int rank, int kslice, int n_mt, float* __restrict__ part) {
  const int lane = threadIdx.x & 63;
  const int tile = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int n_nt = (2 * rank) / 32;
  if (tile >= n_mt * n_nt) return;
  const int mt = tile / n_nt, nt = tile % n_nt;
  const int s = blockIdx.y;
  const int m0 = mt * 32, n0 = nt * 32;
  const uint16_t* U = n0 < rank ? uq : uk;
  const int nn = (n0 % rank) + (lane & 31);
  const int row = m0 + (lane & 31);
  const bool row_ok = row < nb;
  const int kbeg = s * kslice;
  lemo_f32x16 acc = {};
  for (int k = kbeg; k < kbeg + kslice; k += 16) {
    const int kk = k + 8 * (lane >> 5);
    lemo_i16x8 a = {};
    if (row_ok) a = *reinterpret_cast<const lemo_i16x8*>(xbar + (size_t)row * d + kk);
    lemo_i16x8 b;
#pragma unroll
    for (int j = 0; j < 8; ++j) b[j] = (short)U[(size_t)(kk + j) * rank + nn];
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(lemo_bf16x8, a),
                                                  __builtin_bit_cast(lemo_bf16x8, b), acc, 0, 0, 0);
  }
  float* out = part + (size_t)s * nb * (2 * rank);
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int r = m0 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
    if (r < nb) out[(size_t)r * (2 * rank) + n0 + (lane & 31)] = acc[e];
  }
}

// ------------------------------------------------------------- projection
// One workgroup per block row m, 2*rank threads: thread t first forms hidden
// unit t (slices summed in order, ReLU, bf16), then output t of q_hat
// (t < rank) or k_hat (t >= rank) as a sequential fp32 dot over the rank.
__global__ __launch_bounds__(512) void k_project(const float* __restrict__ part, int nslices, int nb, int rank,
                                                 const uint16_t* __restrict__ vq, const uint16_t* __restrict__ vk,
                                                 float* __restrict__ qhat, float* __restrict__ khat) {
  __shared__ float hid[512];
  const int m = blockIdx.x, t = threadIdx.x;
  const int width = 2 * rank;
  float h = 0.f;
#pragma unroll 8
  for (int s = 0; s < nslices; ++s) h += part[((size_t)s * nb + m) * width + t];
  h = fmaxf(h, 0.f);
  hid[t] = lemo_bf16_to_f32(lemo_f32_to_bf16(h));
  __syncthreads();
  const bool is_q = t < rank;
  const int v = is_q ? t : t - rank;
  const uint16_t* V = is_q ? vq : vk;
  const float* hh = hid + (is_q ? 0 : rank);
  // the V column is read 16 rows at a time so its loads overlap; the sum
  // still runs over u in order
  float acc = 0.f;
  for (int u0 = 0; u0 < rank; u0 += 16) {
    float vv[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) vv[j] = lemo_bf16_to_f32(V[(size_t)(u0 + j) * rank + v]);
#pragma unroll
    for (int j = 0; j < 16; ++j) acc = fmaf(hh[u0 + j], vv[j], acc);
  }
  (is_q ? qhat : khat)[(size_t)m * rank + v] = acc;
}

// ------------------------------------------------------------ pair scores
// 16 x 16 tile of M_hat per workgroup, one output per thread; q_hat / k_hat
// rows staged in LDS in 64-wide slices of the rank; the dot runs over v in
// order.
__global__ __launch_bounds__(256) void k_pair(const float* __restrict__ qhat, const float* __restrict__ khat,
                                              int nb, int rank, float* __restrict__ M) {
  __shared__ float sq[16][65];
  __shared__ float sk[16][65];
  const int n0 = blockIdx.x * 16, m0 = blockIdx.y * 16;
  const int t = threadIdx.x, ty = t >> 4, tx = t & 15;
  float acc = 0.f;
  for (int v0 = 0; v0 < rank; v0 += 64) {
    for (int i = t; i < 16 * 64; i += 256) {
      const int r = i >> 6, c = i & 63;
      const bool in = v0 + c < rank;   // rank is a multiple of 32, the slice is 64 wide
      sq[r][c] = (m0 + r < nb && in) ? qhat[(size_t)(m0 + r) * rank + v0 + c] : 0.f;
      sk[r][c] = (n0 + r < nb && in) ? khat[(size_t)(n0 + r) * rank + v0 + c] : 0.f;
    }
    __syncthreads();
#pragma unroll 16
    for (int v = 0; v < 64; ++v) acc = fmaf(sq[ty][v], sk[tx][v], acc);
    __syncthreads();
  }
  if (m0 + ty < nb && n0 + tx < nb) M[(size_t)(m0 + ty) * nb + n0 + tx] = fmaxf(acc, 0.f);
}

struct Layout {
  size_t xbar, part, qhat, khat, m, total;
};

Layout layout(int n_tokens, int d_model, int block, int rank) {
  const int nb = (n_tokens + block - 1) / block;
  const int s = lemo_predict_splitk(nb, d_model, rank);
  Layout L;
  size_t off = 0;
  L.xbar = off; off += lemo_align256((size_t)nb * d_model * 2);
  L.part = off; off += lemo_align256((size_t)s * nb * 2 * rank * 4);
  L.qhat = off; off += lemo_align256((size_t)nb * rank * 4);
  L.khat = off; off += lemo_align256((size_t)nb * rank * 4);
  L.m = off;    off += lemo_align256((size_t)nb * nb * 4);
  L.total = off;
  return L;
}

}  // namespace

// Number of d_model slices for the hidden product: enough 32 x 32 tiles x
// slices to give about 1024 waves, each slice a multiple of 16 columns.
int lemo_predict_splitk(int nb, int d_model, int rank) {
  const int tiles = ((nb + 31) / 32) * ((2 * rank) / 32);
  int s = 1;
  while (s * tiles < 1024 && (d_model % (32 * s)) == 0 && d_model / (2 * s) >= 64) s *= 2;
  return s;
}

size_t lemo_predict_ws_bytes(int n_tokens, int d_model, int block, int rank) {
  return layout(n_tokens, d_model, block, rank).total;
}

hipError_t lemo_launch_predict(const uint16_t* x, int n_tokens, int d_model, int ld_x, int block,
                               const uint16_t* u_q, const uint16_t* v_q, const uint16_t* u_k,
                               const uint16_t* v_k, int rank, float* m_out, float* scores, void* workspace,
                               hipStream_t st) {
  const int nb = (n_tokens + block - 1) / block;
  const Layout L = layout(n_tokens, d_model, block, rank);
  char* ws = static_cast<char*>(workspace);
  uint16_t* xbar = reinterpret_cast<uint16_t*>(ws + L.xbar);
  float* part = reinterpret_cast<float*>(ws + L.part);
  float* qhat = reinterpret_cast<float*>(ws + L.qhat);
  float* khat = reinterpret_cast<float*>(ws + L.khat);
  float* M = m_out ? m_out : reinterpret_cast<float*>(ws + L.m);

  hipLaunchKernelGGL(k_pool, dim3((d_model / 8 + 63) / 64, nb), dim3(64), 0, st, x, ld_x, d_model, block, n_tokens,
                     1.0f / (float)block, xbar);
  const int s = lemo_predict_splitk(nb, d_model, rank);
  const int n_mt = (nb + 31) / 32, n_nt = (2 * rank) / 32;
  hipLaunchKernelGGL(k_hidden, dim3((n_mt * n_nt + 3) / 4, s), dim3(256), 0, st, xbar, d_model, nb, u_q, u_k,
                     rank, d_model / s, n_mt, part);
  hipLaunchKernelGGL(k_project, dim3(nb), dim3(2 * rank), 0, st, part, s, nb, rank, v_q, v_k, qhat, khat);
  hipLaunchKernelGGL(k_pair, dim3((nb + 15) / 16, (nb + 15) / 16), dim3(256), 0, st, qhat, khat, nb, rank, M);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return lemo_launch_colsum(M, nb, scores, st);
}
