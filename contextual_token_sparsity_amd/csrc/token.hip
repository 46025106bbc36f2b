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
// k_gemm_nt computes one 64 x 128 tile of C per workgroup of 4 waves (32 x 64
// per wave as 1 x 2 v_mfma_f32_32x32x16_bf16 tiles; small tiles so that the
// 16384 x 256 hidden product still spreads over 512 workgroups), streaming the reduction
// in 64-wide chunks through a 3-stage LDS ring filled by direct global->LDS
// loads (two chunks in flight: each chunk is only 8 MFMAs per wave, so the
// loads of X, which come from HBM, need the extra lead), with 16-byte pieces
// XOR-swizzled per row so the operand reads are free of bank conflicts.
#include "lemo_internal.h"

namespace {

constexpr int kTM = 64;                        // tile rows (A)
constexpr int kTN = 128;                        // tile columns (B rows)
constexpr int kWaves = 4;                       // 2 x 2 waves of 32 x 64
constexpr int kThreads = kWaves * 64;
constexpr int kChunk = 64;                      // reduction elements per stage
constexpr int kRowBytes = kChunk * 2;           // 128 B
constexpr int kRegionA = kTM * kRowBytes;       // 8 KiB
constexpr int kRegionB = kTN * kRowBytes;       // 16 KiB
constexpr int kStageBytes = kRegionA + kRegionB;
constexpr int kDmaA = kRegionA / (kThreads * 16);   // 2 loads of 16 B per thread
constexpr int kDmaB = kRegionB / (kThreads * 16);   // 4

constexpr int kStages = 3;                      // 72 KiB: two workgroups per CU
constexpr int kDmaPerChunk = kDmaA + kDmaB;

__shared__ __attribute__((aligned(1024))) uint8_t g_tile[kStages * kStageBytes];

// Piece swizzle of LDS row r (distinct for 8 consecutive rows and for the 8
// even/odd rows among 16 consecutive rows).
__device__ __forceinline__ int swz(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }

__device__ __forceinline__ int acc_row(int lane, int e) { return 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3); }

// 16-byte direct global->LDS load per lane: lane l reads base + voff and writes lds + 16 l.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff), "s"(base) : "memory");
}

enum { kEpiReluBf16 = 0, kEpiBf16 = 1 };

// Operands of up to two independent products launched together (blockIdx.z).
struct GemmArgs {
  const uint16_t* a[2];
  const uint16_t* b[2];
  uint16_t* c[2];
};

// C[m][n] = sum_k A[m][k] B[n][k] for m < M, n < Nn; K a multiple of 64.
// Rows of A (B) past M (Nn) read a valid row and their results are dropped.
// Workgroup ids go round-robin over the 8 XCDs; the tn_count column tiles of
// one row block are given to ids on the same XCD, back to back, so that the
// second read of those rows of A hits that XCD's L2.
template <int EPI>
__global__ __launch_bounds__(kThreads, 2) void k_gemm_nt(GemmArgs g, int lda, int ldb, int M, int Nn, int K, int ldc,
                                                         int tm_count, int tn_count) {
  const uint16_t* __restrict__ A = g.a[blockIdx.z];
  const uint16_t* __restrict__ B = g.b[blockIdx.z];
  uint16_t* __restrict__ C = g.c[blockIdx.z];
  int tm, tn;
  {
    const int w = blockIdx.x;
    if (tm_count % 8 == 0) {
      const int j = w / 8;
      tn = j % tn_count;
      tm = (j / tn_count) * 8 + w % 8;
    } else {
      tm = w / tn_count;
      tn = w % tn_count;
    }
  }
  const int m0 = tm * kTM, n0 = tn * kTN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wq = wave >> 1, wk = wave & 1;
  const int l32 = lane & 31, hi = lane >> 5;
  const uint32_t lds0 = (uint32_t)(uintptr_t)g_tile;

  // instruction i of wave w fills LDS row (i*4 + w)*8 + lane/8 of a region,
  // physical piece lane%8, which holds logical piece (lane%8) ^ swz(row)
  uint32_t voffA[kDmaA], voffB[kDmaB];
#pragma unroll
  for (int i = 0; i < kDmaB; ++i) {
    const int r = (i * kWaves + wave) * 8 + (lane >> 3);
    const int piece = (lane & 7) ^ swz(r);
    if (i < kDmaA) voffA[i] = (uint32_t)(((size_t)min(m0 + r, M - 1) * lda + piece * 8) * 2);
    voffB[i] = (uint32_t)(((size_t)min(n0 + r, Nn - 1) * ldb + piece * 8) * 2);
  }
  auto issue = [&](int c, int stage) {
    const uint32_t base = lds0 + (uint32_t)(stage * kStageBytes);
#pragma unroll
    for (int i = 0; i < kDmaB; ++i) {
      if (i < kDmaA) dma16(A + c * kChunk, voffA[i], base + (uint32_t)((i * kWaves + wave) * 1024));
      dma16(B + c * kChunk, voffB[i], base + kRegionA + (uint32_t)((i * kWaves + wave) * 1024));
    }
  };

  // per-lane LDS read offsets for the 4 k-steps of a chunk (operand rows all
  // have r & 15 == l32 & 15, so one swizzle serves them)
  uint32_t offA[4], offB[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int piece = (2 * s + hi) ^ swz(l32);
    offA[s] = (uint32_t)((wq * 32 + l32) * kRowBytes + piece * 16);
    offB[s] = (uint32_t)(kRegionA + (wk * 64 + l32) * kRowBytes + piece * 16);
  }

  lemo_f32x16 acc[1][2];
#pragma unroll
  for (int a = 0; a < 1; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;
  lemo_bf16x8 fa[2][1], fb[2][2];
  auto read_frags = [&](int buf, const uint8_t* st, int s) {
    fa[buf][0] = *reinterpret_cast<const lemo_bf16x8*>(st + offA[s]);
#pragma unroll
    for (int i = 0; i < 2; ++i) fb[buf][i] = *reinterpret_cast<const lemo_bf16x8*>(st + offB[s] + i * 32 * kRowBytes);
  };

  const int nchunks = K / kChunk;
  issue(0, 0);
  if (nchunks > 1) issue(1, 1);
  for (int c = 0; c < nchunks; ++c) {
    // this wave's loads of chunk c have landed (only chunk c+1's may still be
    // in flight); after the barrier every wave's have, and every wave is done
    // with chunk c-1's stage, which is refilled with chunk c+2
    if (c + 1 < nchunks)
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(kDmaPerChunk) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    if (c + 2 < nchunks) issue(c + 2, (c + 2) % kStages);
    const uint8_t* st = g_tile + (c % kStages) * kStageBytes;
    read_frags(0, st, 0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int cur = s & 1;
      if (s + 1 < 4) read_frags(cur ^ 1, st, s + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int b = 0; b < 2; ++b)
        acc[0][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][0], fb[cur][b], acc[0][b], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // epilogue: bf16 (after ReLU for the hidden layer), bounds-checked
#pragma unroll
  for (int a = 0; a < 1; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int col = n0 + wk * 64 + b * 32 + l32;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wq * 32 + a * 32 + acc_row(lane, e);
        float v = acc[a][b][e];
        if (EPI == kEpiReluBf16) v = fmaxf(v, 0.f);
        if (row < M && col < Nn) C[(size_t)row * ldc + col] = (uint16_t)lemo_f32_to_bf16(v);
      }
    }
}

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
  const int tm = (n_tokens + kTM - 1) / kTM;
  // hidden layer: one product, X against [U_q | U_k]^T
  const int tn_h = (r2 + kTN - 1) / kTN;
  GemmArgs gh = {{x, x}, {ut, ut}, {hid, hid}};
  hipLaunchKernelGGL(k_gemm_nt<kEpiReluBf16>, dim3(tm * tn_h, 1, 1), dim3(kThreads), 0, st, gh, ld_x, d_model,
                     n_tokens, r2, d_model, r2, tm, tn_h);
  // output layer: the query and key products in one launch
  const int tn_o = (rank + kTN - 1) / kTN;
  GemmArgs go = {{hid, hid + rank}, {vt, vt + (size_t)rank * rank}, {q_hat, k_hat}};
  hipLaunchKernelGGL(k_gemm_nt<kEpiBf16>, dim3(tm * tn_o, 1, 2), dim3(kThreads), 0, st, go, r2, rank, n_tokens,
                     rank, rank, ld_out, tm, tn_o);
  return hipGetLastError();
}
