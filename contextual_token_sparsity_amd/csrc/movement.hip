// Permutation-free token movement (Jenga, USENIX ATC'25, section 4.2.3):
// "selective load" reads the kept tokens from their original rows, and
// "in-place addition" adds the layer output of each kept token back into its
// original row, so eliminated tokens are never copied, padded or touched.
// In backpropagation the same rows give the layer's input back by
// subtracting the layer output (the recompute variant of the scatter).
//
// Both kernels are HBM-bound row copies: a workgroup of 256 threads moves a
// 4 KiB column stripe (256 x 16 bytes) of a row per step, rows are strided
// over the grid's y dimension, and each thread keeps one or two rows in flight.
// The number of kept rows is read on the device (it comes from the select
// step), so the grid is sized for the worst case and idle slots exit.
#include "lemo_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kUnrollGather = 2;   // rows in flight per thread
constexpr int kUnrollScatter = 1;
constexpr int kRowSlots = 4096;    // the grid's y dimension (row slots)

// a + b (SUB: a - b) on 8 bf16 pairs: fp32 add, round to nearest even.  Two
// bf16 values add or subtract exactly in fp32 unless one is below 2^-16 of
// the other, where the rounded result is the larger one either way, so this
// is the correctly rounded bf16 sum or difference.
template <bool SUB>
__device__ __forceinline__ uint4 add_bf16x8(uint4 a, uint4 b) {
  const uint32_t* pa = &a.x;
  const uint32_t* pb = &b.x;
  uint4 o;
  uint32_t* po = &o.x;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float blo = lemo_bf16_to_f32(pb[j] & 0xffffu), bhi = lemo_bf16_to_f32(pb[j] >> 16);
    const float lo = lemo_bf16_to_f32(pa[j] & 0xffffu) + (SUB ? -blo : blo);
    const float hi = lemo_bf16_to_f32(pa[j] >> 16) + (SUB ? -bhi : bhi);
    po[j] = lemo_f32_to_bf16(lo) | (lemo_f32_to_bf16(hi) << 16);
  }
  return o;
}

// Original token row of dense row p, or -1 when its kept index is invalid or
// the row lies past the sequence (the short last block of a ragged sequence
// listed before the end of the kept list).
__device__ __forceinline__ int token_of(const int32_t* __restrict__ kept, int p, int block, int nb, int n_tokens) {
  const int blk = kept[p / block];
  const int t = blk * block + p % block;
  return (blk >= 0 && blk < nb && t < n_tokens) ? t : -1;
}

// Dense rows of the kept blocks: n_kept whole blocks, less the rows the short
// last block of a ragged sequence lacks when it is the last kept block.
__device__ __forceinline__ int kept_rows(const int32_t* __restrict__ kept, int nk, int block, int nb, int n_tokens) {
  if (nk <= 0) return 0;
  const int last = kept[nk - 1];
  const int short_by = (last >= 0 && last < nb) ? max(0, (last + 1) * block - n_tokens) : 0;
  return nk * block - short_by;
}

// Up to kMaxSources matrices gathered on one kept list in one launch: the
// grid's x dimension is the concatenation of every source's 4 KiB column
// stripes (source i owns stripes first[i] .. first[i+1]-1).
constexpr int kMaxSources = 4;
struct GatherArgs {
  const uint16_t* src[kMaxSources];
  uint16_t* dst[kMaxSources];
  int width[kMaxSources];
  int ld_src[kMaxSources];
  int ld_dst[kMaxSources];
  int first[kMaxSources + 1];
  int n_src;
};

__global__ __launch_bounds__(kThreads) void k_gather(GatherArgs g, int n_tokens, int block,
                                                     const int32_t* __restrict__ kept,
                                                     const int32_t* __restrict__ n_kept_p, int cap_rows,
                                                     int pad_multiple, int32_t* __restrict__ status) {
  const int nb = lemo_nblocks(n_tokens, block);
  const int nk = *n_kept_p;
  const bool bad_count = nk < 0 || nk > nb;
  const int n_rows = bad_count ? 0 : kept_rows(kept, nk, block, nb, n_tokens);
  const long long n_pad = ((long long)n_rows + pad_multiple - 1) / pad_multiple * pad_multiple;
  const int rows = (int)min((long long)cap_rows, n_pad);
  if (status && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
    int flags = 0;
    if (bad_count) flags |= LEMO_DEV_BAD_KEPT;
    if (n_pad > cap_rows) flags |= LEMO_DEV_CAP_OVERFLOW;
    if (flags) atomicOr(status, flags);
  }
  // which source this workgroup's stripe belongs to (uniform)
  int si = 0;
#pragma unroll
  for (int i = 1; i < kMaxSources; ++i)
    if (i < g.n_src && (int)blockIdx.x >= g.first[i]) si = i;
  const uint16_t* __restrict__ src = g.src[si];
  uint16_t* __restrict__ dst = g.dst[si];
  const int width = g.width[si], ld_src = g.ld_src[si], ld_dst = g.ld_dst[si];
  const int ch = ((int)blockIdx.x - g.first[si]) * kThreads + threadIdx.x;
  if (ch * 8 >= width) return;
  const int step = gridDim.y;
  for (int p0 = blockIdx.y; p0 < rows; p0 += step * kUnrollGather) {
    uint4 v[kUnrollGather];
    int tok[kUnrollGather];
#pragma unroll
    for (int u = 0; u < kUnrollGather; ++u) {
      const int p = p0 + u * step;
      v[u] = make_uint4(0, 0, 0, 0);
      tok[u] = -1;
      if (p < n_rows) {
        tok[u] = token_of(kept, p, block, nb, n_tokens);
        if (tok[u] >= 0) v[u] = lemo_load_stream(src + (size_t)tok[u] * ld_src + ch * 8);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnrollGather; ++u) {
      const int p = p0 + u * step;
      if (p >= rows) break;
      if (p < n_rows && tok[u] < 0) {
        if (status) atomicOr(status, LEMO_DEV_BAD_KEPT);
        continue;
      }
      lemo_store_stream(dst + (size_t)p * ld_dst + ch * 8, v[u]);
    }
  }
}

// res[token(p)] = res[token(p)] + y[p] for the kept rows p (SUB: minus).
// y holds y_rows rows: kept rows at or past y_rows are left out (their
// residual rows stay untouched) and flag LEMO_DEV_CAP_OVERFLOW.
template <bool SUB>
__global__ __launch_bounds__(kThreads) void k_scatter(uint16_t* __restrict__ res, int n_tokens, int width, int ld_res,
                                                      int block, const int32_t* __restrict__ kept,
                                                      const int32_t* __restrict__ n_kept_p,
                                                      const uint16_t* __restrict__ y, int ld_y, int y_rows,
                                                      int32_t* __restrict__ status) {
  const int nb = lemo_nblocks(n_tokens, block);
  const int nk = *n_kept_p;
  const bool bad_count = nk < 0 || nk > nb;
  const int all_rows = bad_count ? 0 : kept_rows(kept, nk, block, nb, n_tokens);
  const int n_rows = min(all_rows, y_rows);
  if (status && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
    int flags = 0;
    if (bad_count) flags |= LEMO_DEV_BAD_KEPT;
    if (all_rows > y_rows) flags |= LEMO_DEV_CAP_OVERFLOW;
    if (flags) atomicOr(status, flags);
  }
  const int ch = blockIdx.x * kThreads + threadIdx.x;
  if (ch * 8 >= width) return;
  const int step = gridDim.y;
  for (int p0 = blockIdx.y; p0 < n_rows; p0 += step * kUnrollScatter) {
    uint4 r[kUnrollScatter], a[kUnrollScatter];
    int tok[kUnrollScatter];
#pragma unroll
    for (int u = 0; u < kUnrollScatter; ++u) {
      const int p = p0 + u * step;
      tok[u] = p < n_rows ? token_of(kept, p, block, nb, n_tokens) : -2;
      if (tok[u] >= 0) {
        r[u] = lemo_load_stream(res + (size_t)tok[u] * ld_res + ch * 8);
        a[u] = lemo_load_stream(y + (size_t)p * ld_y + ch * 8);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnrollScatter; ++u) {
      if (tok[u] >= 0) {
        lemo_store_stream(res + (size_t)tok[u] * ld_res + ch * 8, add_bf16x8<SUB>(r[u], a[u]));
      } else if (tok[u] == -1 && status) {
        atomicOr(status, LEMO_DEV_BAD_KEPT);
      }
    }
  }
}

// Workgroups: one per 4 KiB column stripe (x) times 4096 row slots (y,
// fewer when there are fewer rows).  A sweep on the 7B shape (110 of 256
// blocks kept, 7040 rows; sources rotated over three copies so that they
// stream from HBM; back-to-back launches) over 1024..8192 slots and 1, 2 or
// 4 rows in flight per thread: 4096 slots with two rows in flight for the
// gathers (X 70%, the MLP activation 70%, both in one launch 75% of 8 TB/s)
// and one row for the scatter (75%); 8192 slots were 3-9 points slower.  (A
// plain streaming copy peaks at 78% here, a read at 86%, a write at 70%.)
// The slot count does not grow with the capacity: the number of kept rows is
// only known on the device, and a grid sized for every possible row leaves
// most workgroups idle (each still reads n_kept).
dim3 grid_for(int width, int max_rows) {
  const int gx = lemo_nblocks(width / 8, kThreads);
  const int gy = max(1, min(max_rows, kRowSlots));
  return dim3(gx, gy);
}

}  // namespace

hipError_t lemo_launch_gather_multi(int n_src, const uint16_t* const* srcs, const int* widths, const int* ld_srcs,
                                    uint16_t* const* dsts, const int* ld_dsts, int n_tokens, int block,
                                    const int32_t* kept, const int32_t* n_kept, int cap_rows, int pad_multiple,
                                    int32_t* dev_status, hipStream_t stream) {
  GatherArgs g = {};
  g.n_src = n_src;
  int stripes = 0;
  for (int i = 0; i < n_src; ++i) {
    g.src[i] = srcs[i];
    g.dst[i] = dsts[i];
    g.width[i] = widths[i];
    g.ld_src[i] = ld_srcs[i];
    g.ld_dst[i] = ld_dsts[i];
    g.first[i] = stripes;
    stripes += grid_for(widths[i], 1).x;
  }
  g.first[n_src] = stripes;
  const dim3 grid(stripes, grid_for(8, cap_rows).y);
  hipLaunchKernelGGL(k_gather, grid, dim3(kThreads), 0, stream, g, n_tokens, block, kept, n_kept, cap_rows,
                     pad_multiple, dev_status);
  return hipGetLastError();
}

hipError_t lemo_launch_gather(const uint16_t* src, int n_tokens, int width, int ld_src, int block,
                              const int32_t* kept, const int32_t* n_kept, uint16_t* dst, int ld_dst, int cap_rows,
                              int pad_multiple, int32_t* dev_status, hipStream_t stream) {
  return lemo_launch_gather_multi(1, &src, &width, &ld_src, &dst, &ld_dst, n_tokens, block, kept, n_kept, cap_rows,
                                  pad_multiple, dev_status, stream);
}

hipError_t lemo_launch_scatter(uint16_t* res, int n_tokens, int width, int ld_res, int block, const int32_t* kept,
                               const int32_t* n_kept, const uint16_t* y, int ld_y, int y_rows, int32_t* dev_status,
                               hipStream_t stream, bool subtract) {
  const dim3 grid = grid_for(width, min(n_tokens, y_rows));
  if (subtract)
    hipLaunchKernelGGL(k_scatter<true>, grid, dim3(kThreads), 0, stream, res, n_tokens, width, ld_res, block, kept,
                       n_kept, y, ld_y, y_rows, dev_status);
  else
    hipLaunchKernelGGL(k_scatter<false>, grid, dim3(kThreads), 0, stream, res, n_tokens, width, ld_res, block, kept,
                       n_kept, y, ld_y, y_rows, dev_status);
  return hipGetLastError();
}
