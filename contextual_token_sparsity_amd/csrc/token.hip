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
// Rank 128 with d_model a multiple of 256 (the usual shape) runs as one fused
// launch, k_token_fused; other shapes run the transposes and both products
// on the shared k_gemm_nt (gemm_nt.h), with the hidden layer in the workspace.
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

// ------------------------------------------------------ fused rank-128 path
// One workgroup computes 128 token rows of ONE predictor (query or key): the
// hidden tile H = bf16(ReLU(X U)) [128][128] and then out = bf16(H V), so the
// hidden layer never leaves the chip and the weights are never transposed in
// memory.  The hidden product is the heavy part (2 * 128 * 128 * d_model
// flops against 128 * d_model * 2 bytes of X): X streams through a 4-stage LDS
// ring in 64-wide chunks by direct global->LDS loads, and each 64-row chunk of
// U ([d_model][128], hidden units contiguous) goes through registers and is
// written transposed (hidden-unit-major, pairs of reduction elements per
// 4-byte word), the layout the matrix-core B operand reads.
//   8 waves = 2 groups x (2 x 2 waves of 64 x 64).  Group g takes k-steps 2g
//   and 2g + 1 of every chunk; the two groups' fp32 sums are added once, at the
//   end, through LDS (group 0's value plus group 1's, always in that order).
//   Loads run 3 chunks (X) and 4 chunks (U) ahead of the chunk in use.
// The query and key workgroups of one row tile are given ids on the same XCD,
// dispatched together, so the second read of those X rows hits L2.
namespace fused {

constexpr int kR = 128;                        // hidden units of each predictor
constexpr int kTM = 128;                       // token rows per workgroup
constexpr int kThr = 512;                      // 8 waves
constexpr int kRegion = 128 * kRowBytes;       // 128 LDS rows of 64 bf16
constexpr int kStageBytes = 2 * kRegion;       // X rows, then U^T rows
constexpr int kStages = 4;
constexpr int kLds = kStages * kStageBytes;    // 128 KiB
constexpr int kLdo = kR + 8;                   // output staging row stride (elements)

// Piece swizzle of a 128-B LDS row: distinct over 8 consecutive rows (operand
// reads), over the even and over the odd rows of 16 consecutive rows, and over
// 8 rows spaced 8 apart (the transposing writes).
__device__ __forceinline__ int fsw(int r) { return (r ^ (r >> 3)) & 7; }

// One lane's share of a 64-row chunk of a [rows][128] weight: rows 2kp and
// 2kp + 1 (kp = 0..31 within the chunk), columns 8ng .. 8ng + 7.
struct WItem {
  uint4 r0, r1;
};

__device__ __forceinline__ void w_load(WItem& it, const uint16_t* __restrict__ w, int row0, int ng) {
  it.r0 = *reinterpret_cast<const uint4*>(w + (size_t)row0 * kR + ng * 8);
  it.r1 = *reinterpret_cast<const uint4*>(w + (size_t)(row0 + 1) * kR + ng * 8);
}

// Writes the item transposed into a region: LDS row n = column of the weight,
// 4-byte word kp = (row 2kp, row 2kp + 1) of that column.
__device__ __forceinline__ void w_store(uint8_t* region, const WItem& it, int kp, int ng) {
  const uint32_t a[4] = {it.r0.x, it.r0.y, it.r0.z, it.r0.w};
  const uint32_t b[4] = {it.r1.x, it.r1.y, it.r1.z, it.r1.w};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int n = 8 * ng + j;
    const uint32_t word = (j & 1) ? ((a[j >> 1] >> 16) | (b[j >> 1] & 0xffff0000u))
                                  : ((a[j >> 1] & 0xffffu) | (b[j >> 1] << 16));
    *reinterpret_cast<uint32_t*>(region + n * kRowBytes + (((kp >> 2) ^ fsw(n)) << 4) + (kp & 3) * 4) = word;
  }
}

}  // namespace fused

// Grid: 2 * n_tiles workgroups (n_tiles = ceil(n_tokens / 128)); d_model a
// multiple of 256.  Rows past the sequence read its last row and are not
// written.
__global__ __launch_bounds__(fused::kThr, 1) void k_token_fused(
    const uint16_t* __restrict__ x, int ld_x, int n_tokens, int d_model, const uint16_t* __restrict__ u_q,
    const uint16_t* __restrict__ v_q, const uint16_t* __restrict__ u_k, const uint16_t* __restrict__ v_k,
    uint16_t* __restrict__ q_hat, uint16_t* __restrict__ k_hat, int ld_out, int n_tiles) {
  using namespace fused;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLds];
  int t, h;
  {
    const int id = blockIdx.x;
    if (n_tiles % 8 == 0) {
      const int j = id >> 3;
      h = j & 1;
      t = (j >> 1) * 8 + (id & 7);
    } else {
      t = id >> 1;
      h = id & 1;
    }
  }
  const uint16_t* __restrict__ U = h ? u_k : u_q;
  const uint16_t* __restrict__ V = h ? v_k : v_q;
  uint16_t* __restrict__ out = h ? k_hat : q_hat;
  const int m0 = t * kTM;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = wave >> 2, wq = (wave >> 1) & 1, wn = wave & 1;
  const int l32 = lane & 31, hi = lane >> 5;
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds;

  // X: instruction i of this wave fills LDS row (8i + wave) * 8 + lane / 8 of
  // the stage's X region, physical piece lane % 8 (logical piece
  // (lane % 8) ^ fsw(row))
  uint32_t voff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = (i * 8 + wave) * 8 + (lane >> 3);
    const int row = min(m0 + r, n_tokens - 1);
    voff[i] = (uint32_t)(((size_t)row * ld_x + (((lane & 7) ^ fsw(r)) * 8)) * 2);
  }
  const int nch = d_model / kChunk;
  auto issue_x = [&](int c, int stage) {
    const uint32_t base = lds0 + (uint32_t)(stage * kStageBytes);
    const uint16_t* src = x + (size_t)min(c, nch - 1) * kChunk;   // past the end: the last chunk again, unused
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16(src, voff[i], base + (uint32_t)((i * 8 + wave) * 1024));
  };
  // U: this lane's (kp, ng) within every chunk; the 8 lanes of one kp read
  // 128 consecutive bytes of a row
  const int kp = 4 * wave + ((lane >> 3) & 3), ng = (lane & 7) + 8 * hi;
  auto load_u = [&](fused::WItem& it, int c) { w_load(it, U, min(c, nch - 1) * kChunk + 2 * kp, ng); };

  // operand read offsets: group g, k-step s reads piece 4g + 2s + hi of rows
  // wq*64 + 32a + l32 (X) and wn*64 + 32b + l32 (U^T)
  uint32_t offA[2][2], offB[2][2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const int P = 4 * g + 2 * s + hi;
      const int ra = wq * 64 + a * 32 + l32, rb = wn * 64 + a * 32 + l32;
      offA[s][a] = (uint32_t)(ra * kRowBytes + ((P ^ fsw(ra)) << 4));
      offB[s][a] = (uint32_t)(kRegion + rb * kRowBytes + ((P ^ fsw(rb)) << 4));
    }

  lemo_f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;

  // issue order per chunk: U loads (2), then X loads (2).  Loads past the end
  // re-read the last chunk into stages nobody reads again, so that every wait
  // below sees the same count of younger loads.
  fused::WItem w0, w1, w2, w3;
  load_u(w0, 0);
  issue_x(0, 0);
  load_u(w1, 1);
  issue_x(1, 1);
  load_u(w2, 2);
  issue_x(2, 2);
  load_u(w3, 3);
  w_store(lds + kRegion, w0, kp, ng);

  // chunk c: its U item was stored at the end of chunk c-1; `next` holds
  // chunk c+1's, `slot` (chunk c's, already stored) receives chunk c+4's
  auto step = [&](int c, fused::WItem& next, fused::WItem& slot) {
    // at least 8 loads (U(c+2), X(c+1), U(c+3), X(c+2)) were issued after X(c):
    // X(c) has landed; after the barrier every wave's X(c) and U(c) writes are
    // visible, and chunk c-1's stage (refilled with chunk c+3) is free
    asm volatile("s_waitcnt vmcnt(8)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    load_u(slot, c + 4);
    issue_x(c + 3, (c + 3) & 3);
    const uint8_t* st = lds + (c & 3) * kStageBytes;
    lemo_bf16x8 fa[2][2], fb[2][2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        fa[s][a] = *reinterpret_cast<const lemo_bf16x8*>(st + offA[s][a]);
        fb[s][a] = *reinterpret_cast<const lemo_bf16x8*>(st + offB[s][a]);
      }
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[s][a], fb[s][b], acc[a][b], 0, 0, 0);
    // the eight operand reads first, then the eight products
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    // chunk c+1's U^T into its stage (last read for chunk c-3).  Kept after
    // the products: hoisted, its use of the loaded registers would make the
    // compiler wait for younger loads too
    __builtin_amdgcn_sched_barrier(0);
    w_store(lds + ((c + 1) & 3) * kStageBytes + kRegion, next, kp, ng);
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int c = 0; c < nch; c += 4) {
    step(c, w1, w0);
    step(c + 1, w2, w1);
    step(c + 2, w3, w2);
    step(c + 3, w0, w3);
  }

  // ---- epilogue.  LDS: [0, 64K) the sums the groups exchange; [64K, 96K) H
  // as the A operand (two 64-unit regions); [96K, 128K) V^T as the B operand.
  asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  fused::WItem v0, v1;
  w_load(v0, V, 2 * kp, ng);
  w_load(v1, V, kChunk + 2 * kp, ng);
  uint8_t* hreg = lds + 65536;
  uint8_t* vreg = hreg + 2 * kRegion;
  // group g finalises row tile a = g of its 64 x 64 and hands the other tile
  // to the other group, 4 values per 16-byte write
  lemo_f32x4* xch = reinterpret_cast<lemo_f32x4*>(lds);
  const int wi = wave & 3;
  auto hand_over = [&](const lemo_f32x16 (&tile)[2]) {
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const lemo_f32x4 v = {tile[b][4 * q], tile[b][4 * q + 1], tile[b][4 * q + 2], tile[b][4 * q + 3]};
        xch[(((g * 4 + wi) * 2 + b) * 4 + q) * 64 + lane] = v;
      }
  };
  if (g == 0)
    hand_over(acc[1]);
  else
    hand_over(acc[0]);
  w_store(vreg, v0, kp, ng);
  w_store(vreg + kRegion, v1, kp, ng);
  __syncthreads();
  // H[m][j] = bf16(max(0, group 0 + group 1)), tokens m = wq*64 + 32g +
  // acc_row(lane, e), hidden unit j = wn*64 + 32b + l32
  auto finalise = [&](const lemo_f32x16 (&tile)[2]) {
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const lemo_f32x4 o = xch[((((1 - g) * 4 + wi) * 2 + b) * 4 + q) * 64 + lane];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int e = 4 * q + u;
          const float mine = tile[b][e];
          const float v = fmaxf(g == 0 ? mine + o[u] : o[u] + mine, 0.f);
          const int m = wq * 64 + g * 32 + acc_row(lane, e);
          const int j = b * 32 + l32;
          *reinterpret_cast<uint16_t*>(hreg + wn * kRegion + m * kRowBytes + (((j >> 3) ^ fsw(m)) << 4) +
                                       (j & 7) * 2) = (uint16_t)lemo_f32_to_bf16(v);
        }
      }
  };
  if (g == 0)
    finalise(acc[0]);
  else
    finalise(acc[1]);
  __syncthreads();
  // out[m][n] = sum_j H[m][j] V[j][n]: wave owns rows (wave/2)*32 .. +32 and
  // columns (wave%2)*64 .. +64
  lemo_f32x16 o[2];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[b][e] = 0.f;
  const int orow = (wave >> 1) * 32 + l32;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const int rg = ks >> 2, P = 2 * (ks & 3) + hi;
    const lemo_bf16x8 fa = *reinterpret_cast<const lemo_bf16x8*>(hreg + rg * kRegion + orow * kRowBytes +
                                                                 ((P ^ fsw(orow)) << 4));
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int nrow = (wave & 1) * 64 + b * 32 + l32;
      const lemo_bf16x8 fb = *reinterpret_cast<const lemo_bf16x8*>(vreg + rg * kRegion + nrow * kRowBytes +
                                                                   ((P ^ fsw(nrow)) << 4));
      o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb, o[b], 0, 0, 0);
    }
  }
  __syncthreads();
  uint16_t* stile = reinterpret_cast<uint16_t*>(lds);
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e)
      stile[((wave >> 1) * 32 + acc_row(lane, e)) * kLdo + (wave & 1) * 64 + b * 32 + l32] =
          (uint16_t)lemo_f32_to_bf16(o[b][e]);
  __syncthreads();
  for (int idx = tid; idx < kTM * (kR / 8); idx += kThr) {
    const int r = idx >> 4, c8 = idx & 15;
    if (m0 + r >= n_tokens) continue;
    *reinterpret_cast<uint4*>(out + (size_t)(m0 + r) * ld_out + c8 * 8) =
        *reinterpret_cast<const uint4*>(stile + r * kLdo + c8 * 8);
  }
}

bool fused_shape(int d_model, int rank) { return rank == fused::kR && d_model % 256 == 0; }

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

size_t lemo_token_ws_bytes(int n_tokens, int d_model, int rank) {
  return fused_shape(d_model, rank) ? 0 : layout(n_tokens, d_model, rank).total;
}

hipError_t lemo_launch_token_embed(const uint16_t* x, int n_tokens, int d_model, int ld_x, const uint16_t* u_q,
                                   const uint16_t* v_q, const uint16_t* u_k, const uint16_t* v_k, int rank,
                                   uint16_t* q_hat, uint16_t* k_hat, int ld_out, void* workspace, hipStream_t st) {
  if (fused_shape(d_model, rank)) {
    const int n_tiles = (n_tokens + fused::kTM - 1) / fused::kTM;
    hipLaunchKernelGGL(k_token_fused, dim3(2 * n_tiles), dim3(fused::kThr), 0, st, x, ld_x, n_tokens, d_model, u_q,
                       v_q, u_k, v_k, q_hat, k_hat, ld_out, n_tiles);
    return hipGetLastError();
  }
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
