// Permutation-free token movement (Jenga, USENIX ATC'25, section 4.2.3):
// "selective load" reads the kept tokens from their original rows, and
// "in-place addition" adds the layer output of each kept token back into its
// original row, so eliminated tokens are never copied, padded or touched.
// In backpropagation the same rows give the layer's input back by
// subtracting the layer output (the recompute variant of the scatter).
//
// Both kernels are HBM-bound row copies: a workgroup of 256 threads moves a
// 4 KiB column stripe (256 x 16 bytes) of a row per step, rows are strided
// over the grid's y dimension, and each thread keeps two rows in flight.
// The number of kept rows is read on the device (it comes from the select
// step), so the grid is sized for the worst case and idle slots exit.
#include "lemo_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kUnrollGather = 2;   // rows in flight per thread
constexpr int kUnrollScatter = 2;

// Streaming 16-byte accesses: every byte is touched once, so the loads and
// stores carry the nontemporal hint and do not displace other data from L2
// and the Infinity Cache (measured ~10-20 % faster than plain accesses when
// the source is not already cached).
typedef unsigned int lemo_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const uint16_t* p) {
  const lemo_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const lemo_u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_stream(uint16_t* p, uint4 v) {
  const lemo_u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<lemo_u32x4*>(p));
}

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

__global__ __launch_bounds__(kThreads) void k_gather(const uint16_t* __restrict__ src, int n_tokens, int width,
                                                     int ld_src, int block, const int32_t* __restrict__ kept,
                                                     const int32_t* __restrict__ n_kept_p, uint16_t* __restrict__ dst,
                                                     int ld_dst, int cap_rows, int pad_multiple,
                                                     int32_t* __restrict__ status) {
  const int nb = (n_tokens + block - 1) / block;
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
  const int ch = blockIdx.x * kThreads + threadIdx.x;
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
        if (tok[u] >= 0) v[u] = load_stream(src + (size_t)tok[u] * ld_src + ch * 8);
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
      store_stream(dst + (size_t)p * ld_dst + ch * 8, v[u]);
    }
  }
}

// res[token(p)] = res[token(p)] + y[p] for the kept rows p (SUB: minus).
template <bool SUB>
__global__ __launch_bounds__(kThreads) void k_scatter(uint16_t* __restrict__ res, int n_tokens, int width, int ld_res,
                                                      int block, const int32_t* __restrict__ kept,
                                                      const int32_t* __restrict__ n_kept_p,
                                                      const uint16_t* __restrict__ y, int ld_y,
                                                      int32_t* __restrict__ status) {
  const int nb = (n_tokens + block - 1) / block;
  const int nk = *n_kept_p;
  const bool bad_count = nk < 0 || nk > nb;
  const int n_rows = bad_count ? 0 : kept_rows(kept, nk, block, nb, n_tokens);
  if (status && bad_count && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0)
    atomicOr(status, LEMO_DEV_BAD_KEPT);
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
        r[u] = load_stream(res + (size_t)tok[u] * ld_res + ch * 8);
        a[u] = load_stream(y + (size_t)p * ld_y + ch * 8);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnrollScatter; ++u) {
      if (tok[u] >= 0) {
        store_stream(res + (size_t)tok[u] * ld_res + ch * 8, add_bf16x8<SUB>(r[u], a[u]));
      } else if (tok[u] == -1 && status) {
        atomicOr(status, LEMO_DEV_BAD_KEPT);
      }
    }
  }
}

// Workgroups: one per 4 KiB column stripe (x) times 8192 row slots (y, fewer
// when there are fewer rows), each thread keeping two rows in flight.
// Measured on the 7B shape with the source streaming from HBM, this beats
// 1024 slots with 8 rows in flight by up to 12% (a plain streaming copy runs
// at about 5.5 TB/s here).  The slot count does not grow with the capacity:
// the number of kept rows is only known on the device, and a grid sized for
// every possible row left most workgroups idle (each still reads n_kept),
// which cost a 4096-wide gather a third of its rate.
dim3 grid_for(int width, int max_rows) {
  const int gx = (width / 8 + kThreads - 1) / kThreads;
  const int gy = max(1, min(max_rows, 8192));
  return dim3(gx, gy);
}

}  // namespace

hipError_t lemo_launch_gather(const uint16_t* src, int n_tokens, int width, int ld_src, int block,
                              const int32_t* kept, const int32_t* n_kept, uint16_t* dst, int ld_dst, int cap_rows,
                              int pad_multiple, int32_t* dev_status, hipStream_t stream) {
  hipLaunchKernelGGL(k_gather, grid_for(width, cap_rows), dim3(kThreads), 0, stream, src, n_tokens, width,
                     ld_src, block, kept, n_kept, dst, ld_dst, cap_rows, pad_multiple, dev_status);
  return hipGetLastError();
}

hipError_t lemo_launch_scatter(uint16_t* res, int n_tokens, int width, int ld_res, int block, const int32_t* kept,
                               const int32_t* n_kept, const uint16_t* y, int ld_y, int32_t* dev_status,
                               hipStream_t stream, bool subtract) {
  if (subtract)
    hipLaunchKernelGGL(k_scatter<true>, grid_for(width, n_tokens), dim3(kThreads), 0, stream, res, n_tokens,
                       width, ld_res, block, kept, n_kept, y, ld_y, dev_status);
  else
    hipLaunchKernelGGL(k_scatter<false>, grid_for(width, n_tokens), dim3(kThreads), 0, stream, res, n_tokens,
                       width, ld_res, block, kept, n_kept, y, ld_y, dev_status);
  return hipGetLastError();
}
