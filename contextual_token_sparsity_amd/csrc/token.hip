// Per-token predictor embeddings (Jenga, USENIX ATC'25, section 4.2.2,
// Figure 8 and its complexity analysis: the query and key predictors run once
// per token of the sequence).  For every token row x:
//   q_hat = bf16( bf16(ReLU(x U_q)) V_q ),   k_hat likewise with U_k, V_k,
// with fp32 accumulation and round-to-nearest-even at both bf16 points.  The
// bf16 outputs are the Q and K of one head of width r, which the exact-score
// kernel turns into block scores.
//
// Both products have the form C = A B^T with A and B row-major in the
// reduction index (like Q K^T), once the weights are transposed:
//   hidden  H[N][2r] = bf16(ReLU(X [U_q | U_k]))   A = X,        B = [U_q | U_k]^T  ([2r][d])
//   output  q_hat    = bf16(H[:, :r] V_q)          A = H[:, :r], B = V_q^T           ([r][r])
//           k_hat    = bf16(H[:, r:] V_k)          A = H[:, r:], B = V_k^T
// Both run on the shared k_gemm_nt (gemm_nt.h).
#include "gemm_nt.h"

namespace {

using namespace gemm;

// Up to four dense row-major bf16 matrices to transpose in one launch.
struct TransposeArgs {
  const uint16_t* in[4];
  uint16_t* out[4];
  int rows[4], cols[4];
};

// out[c][r] = in[r][c] for matrix blockIdx.z (rows x cols, dense), one 32 x 32
// tile per workgroup through LDS; workgroups past the matrix's tiles exit.
__global__ __launch_bounds__(256) void k_transpose(TransposeArgs t) {
  __shared__ uint16_t tile[32][33];
  const int z = blockIdx.z;
  const int rows = t.rows[z], cols = t.cols[z];
  const int tcols = (cols + 31) / 32;
  if ((int)blockIdx.x >= tcols * ((rows + 31) / 32)) return;
  const int r0 = (blockIdx.x / tcols) * 32, c0 = (blockIdx.x % tcols) * 32;
  const uint16_t* __restrict__ in = t.in[z];
  uint16_t* __restrict__ out = t.out[z];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = threadIdx.x + k * 256;
    const int r = i >> 5, c = i & 31;
    if (r0 + r < rows && c0 + c < cols) tile[r][c] = in[(size_t)(r0 + r) * cols + c0 + c];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = threadIdx.x + k * 256;
    const int c = i >> 5, r = i & 31;
    if (r0 + r < rows && c0 + c < cols) out[(size_t)(c0 + c) * rows + r0 + r] = tile[r][c];
  }
}

struct Layout {
  size_t ut, vt, hid, total;
};

Layout layout(int n_tokens, int d_model, int rank) {
  Layout L;
  size_t off = 0;
  L.ut = off;  off += lemo_align256((size_t)2 * rank * d_model * 2);     // [U_q | U_k]^T  [2r][d]
  L.vt = off;  off += lemo_align256((size_t)2 * rank * rank * 2);        // V_q^T, V_k^T   [2][r][r]
  L.hid = off; off += lemo_align256((size_t)n_tokens * 2 * rank * 2);    // H              [N][2r]
  L.total = off;
  return L;
}


}  // namespace

size_t lemo_token_ws_bytes(int n_tokens, int d_model, int rank) { return layout(n_tokens, d_model, rank).total; }

hipError_t lemo_launch_token_embed(const uint16_t* x, int n_tokens, int d_model, int ld_x, const uint16_t* u_q,
                                   const uint16_t* v_q, const uint16_t* u_k, const uint16_t* v_k, int rank,
                                   uint16_t* q_hat, uint16_t* k_hat, int ld_out, void* workspace, hipStream_t st) {
  const Layout L = layout(n_tokens, d_model, rank);
  char* ws = static_cast<char*>(workspace);
  uint16_t* ut = reinterpret_cast<uint16_t*>(ws + L.ut);
  uint16_t* vt = reinterpret_cast<uint16_t*>(ws + L.vt);
  uint16_t* hid = reinterpret_cast<uint16_t*>(ws + L.hid);
  const int r2 = 2 * rank;
  // the weights as [U_q | U_k]^T ([2r][d]) and V_q^T, V_k^T ([r][r] each)
  TransposeArgs ta = {{u_q, u_k, v_q, v_k},
                      {ut, ut + (size_t)rank * d_model, vt, vt + (size_t)rank * rank},
                      {d_model, d_model, rank, rank},
                      {rank, rank, rank, rank}};
  const int ttiles = ((max(d_model, rank) + 31) / 32) * ((rank + 31) / 32);
  hipLaunchKernelGGL(k_transpose, dim3(ttiles, 1, 4), dim3(256), 0, st, ta);
  // hidden layer: one product, X against [U_q | U_k]^T
  int tm, tn;
  const RowMap none = {nullptr, nullptr, 1, 0, 1, nullptr};
  const dim3 gh_grid = grid_for(64, 128, n_tokens, r2, 1, tm, tn);
  Args gh = {{x, x}, {ut, ut}, {hid, hid}};
  hipLaunchKernelGGL((k_gemm_nt<kEpiReluBf16, 64, 128, 4>), gh_grid, dim3(kThreads), 0, st, gh, ld_x, d_model, n_tokens, r2,
                     d_model, r2, tm, tn, none);
  // output layer: the query and key products in one launch
  const dim3 go_grid = grid_for(64, 128, n_tokens, rank, 2, tm, tn);
  Args go = {{hid, hid + rank}, {vt, vt + (size_t)rank * rank}, {q_hat, k_hat}};
  hipLaunchKernelGGL((k_gemm_nt<kEpiBf16, 64, 128, 4>), go_grid, dim3(kThreads), 0, st, go, r2, rank, n_tokens, rank, rank,
                     ld_out, tm, tn, none);
  return hipGetLastError();
}
