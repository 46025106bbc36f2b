// Layer threshold and mask compaction (Jenga, USENIX ATC'25, section 4.2.1,
// "Layer-specific Threshold"; Algorithm 1, step 1 starts every layer's
// threshold at the average token-block score).
//
// One workgroup of 1024 threads (16 waves) handles up to 8192 blocks:
//   * scores are staged in LDS;
//   * the threshold is the caller's, the mean (float64 sum in block order,
//     then divided and rounded to fp32), or implied by top-k.  The mean's sum
//     is formed by a parallel reduction when every addition is exact (then
//     every order gives the same sum), else by one lane in block order;
//   * top-k: every score becomes an order-preserving 32-bit key (larger key
//     = better score; -0 and +0 share a key as they compare equal; NaN gets
//     the lowest key, below -inf), and the k-th largest key T is found by a
//     radix select in LDS: four rounds of 8 bits, each a histogram of the
//     keys that match the digits chosen so far and a scan of its 256 bins
//     from the top.  The result is the keys above T plus, among the blocks
//     whose key is T, the ones with the lowest indices (ties go to the lower
//     block index), as many as k still needs; the reported threshold is the
//     score of the last of them, the k-th best.  (This replaced ranking
//     every block by counting the blocks that beat it, O(nb^2); counting
//     ranks directly is slower even at 256 blocks.)
//   * the ascending kept list is built 1024 blocks at a time: a wave ballot
//     of the keep bits, the lane's prefix from the bits below it (mbcnt), and
//     the waves' counts scanned through LDS; ties at T are counted the same
//     way in block order.
#include "lemo_internal.h"

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxBlocks = 8192;
constexpr int kPerThread = kMaxBlocks / kThreads;

// Position of the lowest set bit of a finite nonzero double: v is an odd
// multiple of 2^lowest_bit(v).
__device__ __forceinline__ int lowest_bit(double v) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(v);
  const int e = (int)((b >> 52) & 0x7ffu);
  const unsigned long long m = (b & 0xfffffffffffffull) | (e ? (1ull << 52) : 0ull);
  return (e ? e - 1075 : -1074) + __builtin_ctzll(m);
}

// Order-preserving key of a score: a > b as floats iff key(a) > key(b);
// equal floats (including -0 and +0) share a key; every NaN gets 0, below
// the key of -inf (0x007fffff).
__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t b = __float_as_uint(v);
  if ((b & 0x7fffffffu) > 0x7f800000u) return 0u;   // NaN
  if ((b & 0x7fffffffu) == 0u) b = 0u;              // -0 -> +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Sum of `v` over the lanes below this one plus this one (inclusive scan).
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(v, off, 64);
    if (lane >= off) v += y;
  }
  return v;
}

__global__ __launch_bounds__(kThreads) void k_select(const float* __restrict__ scores, int nb, int mode,
                                                     float threshold, int keep, uint8_t* __restrict__ mask,
                                                     int32_t* __restrict__ kept, int32_t* __restrict__ n_kept,
                                                     float* __restrict__ theta_out, int32_t* __restrict__ status) {
  __shared__ float s[kMaxBlocks];
  __shared__ int wave_cnt[kWaves];
  __shared__ int tie_cnt[kWaves];
  __shared__ uint32_t hist[256];
  __shared__ double wsum[kWaves], wmag[kWaves];
  __shared__ int wlsb[kWaves], wfin[kWaves];
  __shared__ int scan_tot[4];
  __shared__ uint32_t sel_key;
  __shared__ int sel_rem;
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

  const bool topk = mode == 1 && keep > 0;
  uint32_t key[kPerThread];
  uint32_t T = 0;       // top-k: the k-th largest key
  int ties_kept = 0;    // top-k: how many blocks with key T are kept
  if (mode == 2) {
    // Each score is a multiple of 2^lowest_bit.  When the magnitudes sum to
    // less than 2^(b + 52), b the smallest such bit over the scores, every
    // partial sum of any subset is a multiple of 2^b of magnitude below
    // 2^(b + 53), so it is a float64 value: every addition is exact, in any
    // order, and the tree sum below equals the sum in block order.  With a
    // non-finite score, or a wider range, one lane sums in block order.
    // Partial sums start at +0, as the sequential one does, so zeros of
    // either sign give the same +0.
    // Up to 1024 blocks wave 0 alone reduces (lane l takes blocks l, l + 64,
    // ...: one butterfly, no barrier); beyond that every wave takes a share
    // and thread 0 adds the 16 wave sums.
    const bool one_wave = nb <= 1024;   // uniform
    double part = 0.0, mag = 0.0;
    int lsb = 0x7fffffff;
    bool fin = true;
    if (!one_wave || wave == 0) {
      const int stride = one_wave ? 64 : kThreads;
      for (int c = tid; c < nb; c += stride) {
        const double v = (double)s[c];
        fin = fin && __builtin_isfinite(v);
        if (v != 0.0 && __builtin_isfinite(v)) lsb = min(lsb, lowest_bit(v));
        part += v;
        mag += fabs(v);
      }
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        part += __shfl_xor(part, off, 64);
        mag += __shfl_xor(mag, off, 64);
        lsb = min(lsb, __shfl_xor(lsb, off, 64));
      }
    }
    const bool wave_fin = __ballot(!fin) == 0ull;
    if (!one_wave) {
      if (lane == 0) {
        wsum[wave] = part;
        wmag[wave] = mag;
        wlsb[wave] = lsb;
        wfin[wave] = wave_fin ? 1 : 0;
      }
      __syncthreads();
    }
    if (tid == 0) {
      double total = part, bound = mag;
      int b = lsb;
      bool all_fin = wave_fin;
      if (!one_wave) {
        total = 0.0;
        bound = 0.0;
        b = 0x7fffffff;
        all_fin = true;
        for (int w = 0; w < kWaves; ++w) {
          total += wsum[w];
          bound += wmag[w];
          b = min(b, wlsb[w]);
          all_fin = all_fin && wfin[w];
        }
      }
      // 2^(b + 52) as a float64 (b >= -149 for float32 inputs, so it is normal)
      const bool exact =
          all_fin && (bound == 0.0 || bound < __longlong_as_double((long long)(b + 52 + 1023) << 52));
      if (!exact) {
        total = 0.0;
        for (int c = 0; c < nb; ++c) total += (double)s[c];
      }
      theta_sh = (float)(total / (double)nb);
    }
  } else if (topk) {
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int c = tid + j * kThreads;
      key[j] = c < nb ? order_key(s[c]) : 0u;
    }
    uint32_t prefix = 0;
    int rem = keep;                 // blocks still to take at or below the digits chosen so far
#pragma unroll 1
    for (int shift = 24; shift >= 0; shift -= 8) {
      const uint32_t hmask = shift == 24 ? 0u : ~((1u << (shift + 8)) - 1u);   // digits already chosen
      if (tid < 256) hist[tid] = 0u;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kPerThread; ++j) {
        const int c = tid + j * kThreads;
        if (c < nb && (key[j] & hmask) == prefix) atomicAdd(&hist[(key[j] >> shift) & 255u], 1u);
      }
      __syncthreads();
      // threads 0..255 take the bins from the top (bin 255 - tid): an
      // inclusive scan gives the count of keys with this digit or a larger one
      int h = 0, incl = 0;
      if (tid < 256) {
        h = (int)hist[255 - tid];
        incl = wave_incl_scan(h, lane);
        if (lane == 63) scan_tot[wave] = incl;
      }
      __syncthreads();
      if (tid < 256) {
        for (int w = 0; w < wave; ++w) incl += scan_tot[w];
        const int excl = incl - h;
        if (excl < rem && rem <= incl) {   // exactly one bin
          sel_key = prefix | ((uint32_t)(255 - tid) << shift);
          sel_rem = rem - excl;
        }
      }
      __syncthreads();
      prefix = sel_key;
      rem = sel_rem;
    }
    T = prefix;
    ties_kept = rem;
  }
  __syncthreads();
  const float theta = theta_sh;

  int base = 0, tie_base = 0;
  for (int j = 0; j * kThreads < nb; ++j) {
    const int c = tid + j * kThreads;
    bool k = false;
    if (mode == 1) {
      // rank of this block among the blocks with key T, in block order
      const bool tie = topk && c < nb && key[j] == T;
      const unsigned long long tb = __ballot(tie);
      const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(tb >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)tb, 0));
      if (lane == 0) tie_cnt[wave] = __popcll(tb);
      __syncthreads();
      int woff = 0, total = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const int cw = tie_cnt[w];
        woff += (w < wave) ? cw : 0;
        total += cw;
      }
      const int rank = tie_base + woff + below;
      k = topk && c < nb && (key[j] > T || (tie && rank < ties_kept));
      if (tie && rank == ties_kept - 1) theta_sh = s[c];   // the k-th best block
      tie_base += total;
    } else if (c < nb) {
      k = s[c] >= theta;
    }
    if (c < nb) mask[c] = k ? 1 : 0;
    const unsigned long long bal = __ballot(k);
    const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
    if (lane == 0) wave_cnt[wave] = __popcll(bal);
    __syncthreads();
    int woff = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
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
    if (theta_out) *theta_out = theta_sh;
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
