// Permutation-free token movement fused into the layer's products (Jenga,
// USENIX ATC'25, section 4.2.3 and Figure 18: selective load and in-place
// addition happen inside the computation instead of as separate passes).
//
//   lemo_gather_linear   y[p] = bf16(x[tok(p)] W^T) for the kept rows p < R,
//                        zero rows up to the padding: the kept-row gather is
//                        the A-operand prologue of the product (the direct
//                        global->LDS loads read the token rows in place).
//   lemo_linear_scatter  res[tok(p)] = bf16(res[tok(p)] + bf16(a[p] W^T)):
//                        the in-place addition is the product's epilogue.
// W is stored [out][in] (a Linear layer's layout), which is the B^T operand
// k_gemm_nt (or its ping-pong form, k_gemm_nt_pp, for output widths that are
// a multiple of 256) takes as it is.  Both give bit for bit what the
// stand-alone gather_pad / scatter_residual around the same product give.
#include "gemm_nt.h"

using namespace gemm;

namespace {
// the ping-pong form takes output widths that are a multiple of its 256-wide
// tile (no clamped weight rows) and at least two 64-wide reduction chunks
bool use_pp(int d_in, int d_out) { return d_out % 256 == 0 && d_in >= 128; }
}  // namespace

hipError_t lemo_launch_gather_linear(const uint16_t* x, int n_tokens, int d_in, int ld_x, int block,
                                     const int32_t* kept, const int32_t* n_kept, const uint16_t* w, int d_out,
                                     int ld_w, uint16_t* y, int ld_y, int cap_rows, int pad_multiple,
                                     int32_t* dev_status, hipStream_t st) {
  int tm, tn;
  const dim3 grid = grid_for(256, 256, cap_rows, d_out, 1, tm, tn);
  const Args g = {{x, x}, {w, w}, {y, y}};
  const RowMap rm = {kept, n_kept, block, n_tokens, pad_multiple, dev_status};
  if (use_pp(d_in, d_out))
    hipLaunchKernelGGL((k_gemm_nt_pp<kEpiGather>), grid, dim3(512), 0, st, g, ld_x, ld_w, cap_rows, d_out, d_in, ld_y,
                       tm, tn, rm);
  else
    hipLaunchKernelGGL((k_gemm_nt<kEpiGather, 256, 256, 8>), grid, dim3(512), 0, st, g, ld_x, ld_w, cap_rows, d_out,
                       d_in, ld_y, tm, tn, rm);
  return hipGetLastError();
}

hipError_t lemo_launch_linear_scatter(const uint16_t* a, int d_in, int ld_a, int cap_rows, const uint16_t* w,
                                      int d_out, int ld_w, uint16_t* res, int n_tokens, int ld_res, int block,
                                      const int32_t* kept, const int32_t* n_kept, int32_t* dev_status,
                                      hipStream_t st) {
  int tm, tn;
  const int rows = cap_rows < n_tokens ? cap_rows : n_tokens;
  const dim3 grid = grid_for(256, 256, rows, d_out, 1, tm, tn);
  const Args g = {{a, a}, {w, w}, {res, res}};
  const RowMap rm = {kept, n_kept, block, n_tokens, 1, dev_status};
  if (use_pp(d_in, d_out))
    hipLaunchKernelGGL((k_gemm_nt_pp<kEpiScatterAdd>), grid, dim3(512), 0, st, g, ld_a, ld_w, rows, d_out, d_in, ld_res,
                       tm, tn, rm);
  else
    hipLaunchKernelGGL((k_gemm_nt<kEpiScatterAdd, 256, 256, 8>), grid, dim3(512), 0, st, g, ld_a, ld_w, rows, d_out,
                       d_in, ld_res, tm, tn, rm);
  return hipGetLastError();
}
