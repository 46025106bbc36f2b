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
// k_gemm_nt computes one 128 x 128 tile of C per workgroup of 4 waves (64 x 64
// per wave as 2 x 2 v_mfma_f32_32x32x16_bf16 tiles), streaming the reduction
// in 64-wide chunks through a 2-stage LDS ring filled by direct global->LDS
// loads, with 16-byte pieces XOR-swizzled per row so the operand reads are
// free of bank conflicts.
#include "lemo_internal.h"

namespace {

constexpr int kT = 128;                         // tile rows (A) and columns (B)
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kChunk = 64;                      // reduction elements per stage
constexpr int kRowBytes = kChunk * 2;           // 128 B
constexpr int kRegion = kT * kRowBytes;         // 16 KiB (A or B part of a stage)
constexpr int kStageBytes = 2 * kRegion;        // 32 KiB
constexpr int kDma = kRegion / (kThreads * 16); // 4 loads of 16 B per thread per region

__shared__ __attribute__((aligned(1024))) uint8_t g_tile[2 * kStageBytes];

// Piece swizzle of LDS row r (distinct for 8 consecutive rows and for the 8
// even/odd rows among 16 consecutive rows).
__device__ __forceinline__ int swz(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }

__device__ __forceinline__ int acc_row(int lane, int e) { return 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3); }

// 16-byte direct global->LDS load per lane: lane l reads base + voff and writes lds + 16 l.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff), "s"(base) : "memory");
}

enum { kEpiReluBf16 = 0, kEpiBf16 = 1 };

// C[m][n] = sum_k A[m][k] B[n][k] for m < M, n < Nn; K a multiple of 64.
// Rows of A (B) past M (Nn) read a valid row and their results are dropped.
template <int EPI>
__global__ __launch_bounds__(kThreads, 2) void k_gemm_nt(const uint16_t* __restrict__ A, int lda,
                                                         const uint16_t* __restrict__ B, int ldb, int M, int Nn,
                                                         int K, uint16_t* __restrict__ C, int ldc) {
  const int m0 = blockIdx.x * kT, n0 = blockIdx.y * kT;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wq = wave >> 1, wk = wave & 1;
  const int l32 = lane & 31, hi = lane >> 5;
  const uint32_t lds0 = (uint32_t)(uintptr_t)g_tile;

  // instruction i of wave w fills LDS row (i*4 + w)*8 + lane/8 of a region,
  // physical piece lane%8, which holds logical piece (lane%8) ^ swz(row)
  uint32_t voffA[kDma], voffB[kDma];
#pragma unroll
  for (int i = 0; i < kDma; ++i) {
    const int r = (i * kWaves + wave) * 8 + (lane >> 3);
    const int piece = (lane & 7) ^ swz(r);
    voffA[i] = (uint32_t)(((size_t)min(m0 + r, M - 1) * lda + piece * 8) * 2);
    voffB[i] = (uint32_t)(((size_t)min(n0 + r, Nn - 1) * ldb + piece * 8) * 2);
  }
  auto issue = [&](int c, int stage) {
    const uint32_t base = lds0 + (uint32_t)(stage * kStageBytes);
#pragma unroll
    for (int i = 0; i < kDma; ++i) {
      dma16(A + c * kChunk, voffA[i], base + (uint32_t)((i * kWaves + wave) * 1024));
      dma16(B + c * kChunk, voffB[i], base + kRegion + (uint32_t)((i * kWaves + wave) * 1024));
    }
  };

  // per-lane LDS read offsets for the 4 k-steps of a chunk (operand rows all
  // have r & 15 == l32 & 15, so one swizzle serves them)
  uint32_t offA[4], offB[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int piece = (2 * s + hi) ^ swz(l32);
    offA[s] = (uint32_t)((wq * 64 + l32) * kRowBytes + piece * 16);
    offB[s] = (uint32_t)(kRegion + (wk * 64 + l32) * kRowBytes + piece * 16);
  }

  lemo_f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;
  lemo_bf16x8 fa[2][2], fb[2][2];
  auto read_frags = [&](int buf, const uint8_t* st, int s) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      fa[buf][i] = *reinterpret_cast<const lemo_bf16x8*>(st + offA[s] + i * 32 * kRowBytes);
      fb[buf][i] = *reinterpret_cast<const lemo_bf16x8*>(st + offB[s] + i * 32 * kRowBytes);
    }
  };

  const int nchunks = K / kChunk;
  issue(0, 0);
  for (int c = 0; c < nchunks; ++c) {
    // this wave's loads of chunk c have landed; after the barrier every
    // wave's have, and every wave is done with the other stage
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    if (c + 1 < nchunks) issue(c + 1, (c + 1) & 1);
    const uint8_t* st = g_tile + (c & 1) * kStageBytes;
    read_frags(0, st, 0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int cur = s & 1;
      if (s + 1 < 4) read_frags(cur ^ 1, st, s + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][a], fb[cur][b], acc[a][b], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // epilogue: bf16 (after ReLU for the hidden layer), bounds-checked
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int col = n0 + wk * 64 + b * 32 + l32;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wq * 64 + a * 32 + acc_row(lane, e);
        float v = acc[a][b][e];
        if (EPI == kEpiReluBf16) v = fmaxf(v, 0.f);
        if (row < M && col < Nn) C[(size_t)row * ldc + col] = (uint16_t)lemo_f32_to_bf16(v);
      }
    }
}

// out[c][r] = in[r][c] for a rows x cols bf16 matrix (64 x 64 tiles through LDS).
__global__ __launch_bounds__(256) void k_transpose(const uint16_t* __restrict__ in, int rows, int cols, int ld_in,
                                                   uint16_t* __restrict__ out, int ld_out) {
  __shared__ uint16_t t[64][65];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int r = i >> 6, c = i & 63;
    if (r0 + r < rows && c0 + c < cols) t[r][c] = in[(size_t)(r0 + r) * ld_in + c0 + c];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int c = i >> 6, r = i & 63;
    if (r0 + r < rows && c0 + c < cols) out[(size_t)(c0 + c) * ld_out + r0 + r] = t[r][c];
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

void launch_transpose(const uint16_t* in, int rows, int cols, int ld_in, uint16_t* out, int ld_out,
                      hipStream_t st) {
  hipLaunchKernelGGL(k_transpose, dim3((cols + 63) / 64, (rows + 63) / 64), dim3(256), 0, st, in, rows, cols, ld_in,
                     out, ld_out);
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
  launch_transpose(u_q, d_model, rank, rank, ut, d_model, st);
  launch_transpose(u_k, d_model, rank, rank, ut + (size_t)rank * d_model, d_model, st);
  launch_transpose(v_q, rank, rank, rank, vt, rank, st);
  launch_transpose(v_k, rank, rank, rank, vt + (size_t)rank * rank, rank, st);
  const int tm = (n_tokens + kT - 1) / kT;
  hipLaunchKernelGGL(k_gemm_nt<kEpiReluBf16>, dim3(tm, (r2 + kT - 1) / kT), dim3(kThreads), 0, st, x, ld_x, ut,
                     d_model, n_tokens, r2, d_model, hid, r2);
  hipLaunchKernelGGL(k_gemm_nt<kEpiBf16>, dim3(tm, (rank + kT - 1) / kT), dim3(kThreads), 0, st, hid, r2, vt, rank,
                     n_tokens, rank, rank, q_hat, ld_out);
  hipLaunchKernelGGL(k_gemm_nt<kEpiBf16>, dim3(tm, (rank + kT - 1) / kT), dim3(kThreads), 0, st, hid + rank, r2,
                     vt + (size_t)rank * rank, rank, n_tokens, rank, rank, k_hat, ld_out);
  return hipGetLastError();
}
