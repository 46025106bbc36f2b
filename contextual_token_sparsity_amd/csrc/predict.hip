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
//                 split over slices Ks of d_model so that ~512 workgroups run;
//                 U transposed through LDS)
//   k_project     hid = bf16(max(0, sum_s part[s])) (fixed slice order), then
//                 q_hat = hid_q V_q (stored transposed), k_hat = hid_k V_k in fp32
//   k_pair_colsum I_hat[n] = sum_m max(0, q_hat[m] . k_hat[n]) in a fixed
//                 order; M_hat is written only when the caller asks for it.
#include <mutex>

#include "lemo_internal.h"

namespace {

// ---------------------------------------------------------------- pooling
// One thread owns 8 adjacent columns of one block and walks the block's rows
// in order, so every column sum is formed in the same order as a sequential
// loop.  64 threads cover 512 columns; the grid is (column groups, blocks).
// Plain loads: the gather of the kept rows that follows reads X again, and
// finds part of it in the Infinity Cache.
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
// part[s][m][n] = xbar[m, Ks] . [U_q | U_k][Ks, n] for the 32 x 32 tile
// (rows m = blocks, columns n = predictor neurons; n < rank from U_q, the
// rest from U_k) of a workgroup and its slice Ks of the model dimension.
// The slice is split over the 4 waves (v_mfma_f32_32x32x16_bf16, fp32
// accumulation) and walked in chunks of 64; the waves' sums are added in
// wave order through LDS.  The MFMA B operand needs 8 consecutive k of one
// neuron per lane, but U is stored [d][rank] (neurons contiguous): each
// lane loads two adjacent U rows (16 bytes of 8 neurons each) and writes
// the (k, k+1) pairs of each neuron as one 4-byte word into its wave's LDS
// tile, stored neuron-major, from which the operand is one 16-byte read.
// (Measured: this beats 2-byte gathers of U columns, the 2-byte transposed
// stores, and issuing a whole 128-k round of loads at once.)
constexpr int kHidChunk = 64;                    // k per LDS round
constexpr int kHidLd = kHidChunk + 8;            // LDS row stride (elements): 144 B

__global__ __launch_bounds__(256) void k_hidden(const uint16_t* __restrict__ xbar, int d, int nb,
                                                const uint16_t* __restrict__ uq, const uint16_t* __restrict__ uk,
                                                int rank, int kslice, int n_nt, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint16_t ut[4][32][kHidLd];
  __shared__ float red[3][64][17];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int mt = blockIdx.x / n_nt, nt = blockIdx.x % n_nt;
  const int s = blockIdx.y;
  const int m0 = mt * 32, n0 = nt * 32;
  const uint16_t* U = n0 < rank ? uq : uk;
  const int u0 = n0 % rank;                      // first neuron of the tile within U
  const int row = min(m0 + l32, nb - 1);         // rows past nb read a valid row; dropped below
  const int kw = kslice / 4;                     // this wave's share, a multiple of 16
  const int kbeg = s * kslice + wave * kw;
  const uint16_t* arow = xbar + (size_t)row * d + 8 * hi;
  lemo_f32x16 acc = {};
  for (int c0 = 0; c0 < kw; c0 += kHidChunk) {
    const int cl = min(kHidChunk, kw - c0);      // a multiple of 16
    lemo_bf16x8 a[kHidChunk / 16];
#pragma unroll
    for (int i = 0; i < kHidChunk / 16; ++i)
      if (16 * i < cl) a[i] = *reinterpret_cast<const lemo_bf16x8*>(arow + kbeg + c0 + 16 * i);
    // pair P = i * 64 + lane: U rows r = 2 (P / 4) and r + 1 of the chunk,
    // neurons u0 + 8 (P % 4) .. + 7
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int P = i * 64 + lane, r = 2 * (P >> 2), pc = P & 3;
      if (r < cl) {
        const uint16_t* up = U + (size_t)(kbeg + c0 + r) * rank + u0 + pc * 8;
        const uint4 v0 = *reinterpret_cast<const uint4*>(up);
        const uint4 v1 = *reinterpret_cast<const uint4*>(up + rank);
        const uint32_t w0[4] = {v0.x, v0.y, v0.z, v0.w};
        const uint32_t w1[4] = {v1.x, v1.y, v1.z, v1.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          *reinterpret_cast<uint32_t*>(&ut[wave][pc * 8 + 2 * j][r]) = (w0[j] & 0xffffu) | (w1[j] << 16);
          *reinterpret_cast<uint32_t*>(&ut[wave][pc * 8 + 2 * j + 1][r]) = (w0[j] >> 16) | (w1[j] & 0xffff0000u);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);          // lgkmcnt(0): this wave's LDS writes are done
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < kHidChunk / 16; ++i) {
      if (16 * i < cl) {
        const lemo_bf16x8 b = *reinterpret_cast<const lemo_bf16x8*>(&ut[wave][l32][16 * i + 8 * hi]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b, acc, 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);          // operand reads done before the tile is rewritten
    __builtin_amdgcn_wave_barrier();
  }
  // the four waves' partial tiles, added in wave order
  if (wave > 0) {
#pragma unroll
    for (int e = 0; e < 16; ++e) red[wave - 1][lane][e] = acc[e];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int w = 0; w < 3; ++w)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] += red[w][lane][e];
    float* out = part + (size_t)s * nb * (2 * rank);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = m0 + 8 * (e >> 2) + 4 * hi + (e & 3);
      if (r < nb) out[(size_t)r * (2 * rank) + n0 + l32] = acc[e];
    }
  }
}

// ------------------------------------------------------------- projection
// One block m per workgroup, 2*rank threads: thread t forms hidden unit t
// (the slices' partial sums, all loaded at once, added in slice order;
// ReLU; bf16), then output t of q_hat (t < rank) or k_hat (t >= rank) as a
// sequential fp32 dot over the rank, reading V's column t in rounds of 32
// loads.  q_hat is stored transposed, [rank][nb], so that the pair kernel's
// threads (one per query block) read it with coalesced loads.
constexpr int kProjMaxSlices = 16;

__global__ __launch_bounds__(512) void k_project(const float* __restrict__ part, int nslices, int nb, int rank,
                                                 const uint16_t* __restrict__ vq, const uint16_t* __restrict__ vk,
                                                 float* __restrict__ qhat_t, float* __restrict__ khat) {
  __shared__ float hid[512];
  const int m = blockIdx.x, t = threadIdx.x;
  const int width = 2 * rank;
  float pv[kProjMaxSlices];
#pragma unroll
  for (int s = 0; s < kProjMaxSlices; ++s)
    if (s < nslices) pv[s] = part[((size_t)s * nb + m) * width + t];
  float h = 0.f;
#pragma unroll
  for (int s = 0; s < kProjMaxSlices; ++s)
    if (s < nslices) h += pv[s];
  hid[t] = lemo_bf16_to_f32(lemo_f32_to_bf16(fmaxf(h, 0.f)));
  __syncthreads();
  const bool is_q = t < rank;
  const int v = is_q ? t : t - rank;
  const uint16_t* V = is_q ? vq : vk;
  const float* hh = hid + (is_q ? 0 : rank);
  float acc = 0.f;
  for (int u0 = 0; u0 < rank; u0 += 32) {
    float vv[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) vv[j] = lemo_bf16_to_f32(V[(size_t)(u0 + j) * rank + v]);
#pragma unroll
    for (int j = 0; j < 32; ++j) acc = fmaf(hh[u0 + j], vv[j], acc);
  }
  if (is_q)
    qhat_t[(size_t)v * nb + m] = acc;
  else
    khat[(size_t)m * rank + v] = acc;
}

// ------------------------------------------- pair scores and column sums
// A workgroup owns NC key blocks n; thread t walks the query blocks
// m = t, t + 256, ...: M_hat[m][n] = max(0, q_hat[m] . k_hat[n]) (fp32 dot
// in v order; q_hat read column-wise from its transposed copy in rounds of 32
// values, two rounds in flight: the next round's loads are issued before the
// current round's products), written only when the caller asked for the
// block matrix, and summed per thread in m order; the per-thread sums are
// then added in a fixed order (a butterfly inside each wave, then the four
// waves in order), so I_hat[n] is deterministic.  The k_hat rows are staged
// in LDS while the first two rounds of q_hat loads are in flight.
template <int NC>
__global__ __launch_bounds__(256) void k_pair_colsum(const float* __restrict__ qhat_t, const float* __restrict__ khat,
                                                     int nb, int rank, float* __restrict__ M,
                                                     float* __restrict__ scores) {
  constexpr int kRound = 32;
  __shared__ __attribute__((aligned(16))) float kt[NC][256];
  __shared__ float red[NC][4];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int n0 = blockIdx.x * NC;
  const int nr = rank / kRound;   // rank is a multiple of 32
  float cs[NC] = {};
  for (int m0 = 0; m0 < nb; m0 += 256) {
    const int m = m0 + t;
    const float* qc = qhat_t + min(m, nb - 1);
    float qa[kRound], qb[kRound];
    // round rd of this thread's q_hat column (past the last round: the last
    // round again, not used)
    auto load_round = [&](float (&dst)[kRound], int rd) {
      rd = min(rd, nr - 1);
#pragma unroll
      for (int j = 0; j < kRound; ++j) dst[j] = qc[(size_t)(kRound * rd + j) * nb];
    };
    load_round(qa, 0);
    load_round(qb, 1);
    if (m0 == 0) {   // uniform: every thread takes the first pass
      for (int i = t; i < NC * rank; i += 256) {
        const int n = i / rank, v = i % rank;
        kt[n][v] = n0 + n < nb ? khat[(size_t)(n0 + n) * rank + v] : 0.f;
      }
      __syncthreads();
    }
    float dot[NC] = {};
    auto products = [&](const float (&q)[kRound], int rd) {
#pragma unroll
      for (int j = 0; j < kRound; j += 4) {
#pragma unroll
        for (int n = 0; n < NC; ++n) {
          const float4 k4 = *reinterpret_cast<const float4*>(&kt[n][kRound * rd + j]);
          dot[n] = fmaf(q[j], k4.x, dot[n]);
          dot[n] = fmaf(q[j + 1], k4.y, dot[n]);
          dot[n] = fmaf(q[j + 2], k4.z, dot[n]);
          dot[n] = fmaf(q[j + 3], k4.w, dot[n]);
        }
      }
    };
    for (int rd = 0; rd < nr; rd += 2) {
      products(qa, rd);
      if (rd + 1 >= nr) break;
      load_round(qa, rd + 2);
      products(qb, rd + 1);
      load_round(qb, rd + 3);
    }
    if (m < nb) {
#pragma unroll
      for (int n = 0; n < NC; ++n) {
        const float val = fmaxf(dot[n], 0.f);
        cs[n] += val;
        if (M && n0 + n < nb) M[(size_t)m * nb + n0 + n] = val;
      }
    }
  }
#pragma unroll
  for (int n = 0; n < NC; ++n) {
    float v = cs[n];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) v += __shfl_xor(v, off, 64);
    if (lane == 0) red[n][wave] = v;
  }
  __syncthreads();
  if (t < NC && n0 + t < nb) scores[n0 + t] = ((red[t][0] + red[t][1]) + red[t][2]) + red[t][3];
}

struct Layout {
  size_t xbar, part, qhat, khat, total;   // qhat: transposed, [rank][nb]
};

Layout layout(int n_tokens, int d_model, int block, int rank) {
  const int nb = lemo_nblocks(n_tokens, block);
  const int s = lemo_predict_splitk(nb, d_model, rank);
  Layout L;
  size_t off = 0;
  L.xbar = off; off += lemo_align256((size_t)nb * d_model * 2);
  L.part = off; off += lemo_align256((size_t)s * nb * 2 * rank * 4);
  L.qhat = off; off += lemo_align256((size_t)nb * rank * 4);
  L.khat = off; off += lemo_align256((size_t)nb * rank * 4);
  L.total = off;
  return L;
}

// Scratch of lemo_predict_scores_noalloc: a fixed device array instead of a
// caller workspace, for callers that cannot allocate.  Each device that loads
// the library holds its own copy for the life of the process.  Host code
// never uses the array's name as an address: the device address is fetched
// once per device with hipGetSymbolAddress (with that device current) and
// kept in g_static_ptr.
constexpr size_t kStaticScratchBytes = size_t(16) << 20;
constexpr int kMaxDevices = 64;
static __device__ __attribute__((aligned(256))) uint8_t scratch[kStaticScratchBytes];

std::mutex g_static_mu;
void* g_static_ptr[kMaxDevices] = {};

}  // namespace

size_t lemo_predict_static_capacity() { return kStaticScratchBytes; }

// Device address of the current device's scratch array (looked up on the
// first call for that device).
hipError_t lemo_predict_static_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_static_mu);
  if (!g_static_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_static_ptr[dev] = p;
  }
  *ptr = g_static_ptr[dev];
  return hipSuccess;
}

// Number of d_model slices for the hidden product: each workgroup takes one
// slice of d_model (split over its 4 waves in multiples of 16).  Enough
// slices to give about 512 workgroups, at most 16 (the projection adds
// them), each at least 256 columns wide (64 per wave) and dividing d_model
// into multiples of 64 columns.
int lemo_predict_splitk(int nb, int d_model, int rank) {
  const int tiles = ((nb + 31) / 32) * ((2 * rank) / 32);
  const int want = (512 + tiles - 1) / tiles;
  int best = 1;
  for (int s = 2; s <= 16 && s <= want; ++s)
    if ((d_model / 64) % s == 0 && d_model / s >= 256) best = s;
  return best;
}

size_t lemo_predict_ws_bytes(int n_tokens, int d_model, int block, int rank) {
  return layout(n_tokens, d_model, block, rank).total;
}

hipError_t lemo_launch_predict(const uint16_t* x, int n_tokens, int d_model, int ld_x, int block,
                               const uint16_t* u_q, const uint16_t* v_q, const uint16_t* u_k,
                               const uint16_t* v_k, int rank, float* m_out, float* scores, void* workspace,
                               hipStream_t st) {
  const int nb = lemo_nblocks(n_tokens, block);
  const Layout L = layout(n_tokens, d_model, block, rank);
  char* ws = static_cast<char*>(workspace);
  uint16_t* xbar = reinterpret_cast<uint16_t*>(ws + L.xbar);
  float* part = reinterpret_cast<float*>(ws + L.part);
  float* qhat = reinterpret_cast<float*>(ws + L.qhat);
  float* khat = reinterpret_cast<float*>(ws + L.khat);

  hipLaunchKernelGGL(k_pool, dim3((d_model / 8 + 63) / 64, nb), dim3(64), 0, st, x, ld_x, d_model, block, n_tokens,
                     1.0f / (float)block, xbar);
  const int s = lemo_predict_splitk(nb, d_model, rank);
  const int n_mt = (nb + 31) / 32, n_nt = (2 * rank) / 32;
  hipLaunchKernelGGL(k_hidden, dim3(n_mt * n_nt, s), dim3(256), 0, st, xbar, d_model, nb, u_q, u_k, rank,
                     d_model / s, n_nt, part);
  hipLaunchKernelGGL(k_project, dim3(nb), dim3(2 * rank), 0, st, part, s, nb, rank, v_q, v_k, qhat, khat);
  // one key block per workgroup while that still gives few workgroups
  if (nb <= 1024)
    hipLaunchKernelGGL(k_pair_colsum<1>, dim3(nb), dim3(256), 0, st, qhat, khat, nb, rank, m_out, scores);
  else
    hipLaunchKernelGGL(k_pair_colsum<2>, dim3((nb + 1) / 2), dim3(256), 0, st, qhat, khat, nb, rank, m_out, scores);
  return hipGetLastError();
}
