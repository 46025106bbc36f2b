// C = A B^T on the matrix cores (gfx950), with A and B row-major in the
// reduction index (like Q K^T; a Linear layer's weight [out][in] is such a B).
// Device code shared by the per-token predictor and the fused movement
// products; each translation unit gets its own copy (internal linkage).
//
// One TM x TN tile of C per workgroup of WAVES waves in a 2 x (WAVES/2)
// grid of v_mfma_f32_32x32x16_bf16 tiles:
//   64 x 128, 4 waves of 32 x 64: a narrow B (more workgroups: the
//     predictor's 16384 x 256 hidden layer still spreads over 512), 3-stage
//     ring (two chunks in flight), two workgroups per CU;
//   256 x 256, 8 waves of 128 x 64: a d x d weight.  Against 128 x 128 tiles
//     this halves the refill bytes and cuts the operand reads per MFMA by a
//     quarter; on this power-limited part less data movement per flop means
//     a higher clock.  2-stage ring (128 KiB), one workgroup (two waves per
//     SIMD) per CU.  Output widths that are a multiple of 256 run the
//     ping-pong form of this tile (k_gemm_nt_pp below).
// The reduction streams in 64-wide chunks through an LDS ring filled by
// direct global->LDS loads, with the 16-byte pieces of each 128-B LDS row
// XOR-swizzled so that the operand reads are free of bank conflicts.  The
// epilogue stages the bf16 tile in LDS (the ring, or a larger buffer when the
// tile does not fit in it).  Workgroup ids go round-robin
// over the 8 XCDs; when there are few column tiles (a narrow B, e.g. the
// predictor's hidden layer), the column tiles of one row block are given to
// ids on the same XCD, back to back, so the second read of those rows of A
// hits L2; with many column tiles (a d x d weight) the plain row-major order
// keeps each XCD on a quarter of B instead.
//
// Epilogues (EPI):
//   kEpiReluBf16   C[m][n] = bf16(max(0, acc))                       (dense rows)
//   kEpiBf16       C[m][n] = bf16(acc)                               (dense rows)
//   kEpiGather     A row m is token row tok(m) of the kept blocks (selective
//                  load in the operand prologue); C[m][n] = bf16(acc) for
//                  m < R, 0 for R <= m < roundup(R, pad), within cap rows
//   kEpiScatterAdd A rows dense; the product is added in place to residual
//                  row tok(m): res = bf16(f32(res) + f32(bf16(acc))), m < R
// with tok(m) = kept[m / block] * block + m % block and R = n_kept * block
// read on the device (less the rows the short last block of a ragged
// sequence lacks, when it is the last kept block).  Rows whose kept index is
// out of range, or whose token lies past the sequence, are skipped and
// flagged, as the stand-alone gather and scatter do.
#pragma once

#include <type_traits>

#include "lemo_internal.h"

namespace {

namespace gemm {

constexpr int kThreads = 256;                       // 4-wave workgroups (64 x 128 tiles)
constexpr int kChunk = 64;                          // reduction elements per stage
constexpr int kRowBytes = kChunk * 2;               // 128 B

// TM x TN tile per workgroup of WAVES waves in a 2 x (WAVES/2) grid, each
// wave TM/2 x TN/(WAVES/2) as v_mfma_f32_32x32x16_bf16 tiles
template <int TM, int TN, int WAVES>
struct Tile {
  static constexpr int kWaves = WAVES;
  static constexpr int kThr = WAVES * 64;
  static constexpr int kWN = WAVES / 2;                        // waves along the columns
  static constexpr int kRegionA = TM * kRowBytes;
  static constexpr int kRegionB = TN * kRowBytes;
  static constexpr int kStageBytes = kRegionA + kRegionB;
  static constexpr int kDmaA = kRegionA / (kThr * 16);        // loads of 16 B per thread and chunk
  static constexpr int kDmaB = kRegionB / (kThr * 16);
  static constexpr int kStages = TM == 64 ? 3 : 2;
  static constexpr int kDmaPerChunk = kDmaA + kDmaB;
  static constexpr int kWRows = TM / 2, kWCols = TN / kWN;     // per wave
  static constexpr int kMT = kWRows / 32, kNT = kWCols / 32;   // MFMA tiles per wave
  static constexpr int kOcc = TM * TN >= 256 * 256 ? 1 : 2;    // workgroups per CU
  static constexpr int kLdt = TN + 8;                          // epilogue staging row stride (elements)
  static constexpr int kRing = kStages * kStageBytes;
  static constexpr int kLdsBytes = kRing > TM * kLdt * 2 ? kRing : TM * kLdt * 2;
};

enum { kEpiReluBf16 = 0, kEpiBf16 = 1, kEpiGather = 2, kEpiScatterAdd = 3 };

// Piece swizzle of LDS row r (distinct for 8 consecutive rows and for the 8
// even/odd rows among 16 consecutive rows).
__device__ __forceinline__ int swz(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }

__device__ __forceinline__ int acc_row(int lane, int e) { return 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3); }

// 16-byte direct global->LDS load per lane: lane l reads base + voff and writes lds + 16 l.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff), "s"(base) : "memory");
}

// Operands of up to two independent products launched together (blockIdx.z).
struct Args {
  const uint16_t* a[2];
  const uint16_t* b[2];
  uint16_t* c[2];
};

// Kept-block row map of the gather / scatter epilogues.
struct RowMap {
  const int32_t* kept;
  const int32_t* n_kept;
  int block;
  int n_tokens;
  int pad_multiple;
  int32_t* status;
};

// C[m][n] = sum_k A[m][k] B[n][k] for m < M (the row capacity of C for the
// gather epilogue), n < Nn; K a multiple of 64, Nn and ldc multiples of 8.  Rows of A (B) past the rows
// in use read a valid row, and their results are dropped.
template <int EPI, int TM, int TN, int WAVES>
__global__ __launch_bounds__(WAVES * 64, (Tile<TM, TN, WAVES>::kOcc)) void k_gemm_nt(
    Args g, int lda, int ldb, int M, int Nn, int K, int ldc, int tm_count, int tn_count, RowMap rm) {
  using T = Tile<TM, TN, WAVES>;
  constexpr int kRegionA = T::kRegionA, kStageBytes = T::kStageBytes, kDmaA = T::kDmaA, kStages = T::kStages;
  constexpr int kDmaB = T::kDmaB, kDmaPerChunk = T::kDmaPerChunk, kMT = T::kMT, kNT = T::kNT;
  constexpr int kWaves = T::kWaves, kThr = T::kThr, kWN = T::kWN;
  constexpr int kWM = T::kWRows, kWC = T::kWCols;    // rows and columns per wave
  constexpr int kTN = TN;
  __shared__ __attribute__((aligned(1024))) uint8_t g_tile[T::kLdsBytes];
  constexpr bool kMapped = EPI == kEpiGather || EPI == kEpiScatterAdd;
  const uint16_t* __restrict__ A = g.a[blockIdx.z];
  const uint16_t* __restrict__ B = g.b[blockIdx.z];
  uint16_t* __restrict__ C = g.c[blockIdx.z];
  int tm, tn;
  {
    const int w = blockIdx.x;
    if (tm_count % 8 == 0 && tn_count <= 4) {
      const int j = w / 8;
      tn = j % tn_count;
      tm = (j / tn_count) * 8 + w % 8;
    } else {
      tm = w / tn_count;
      tn = w % tn_count;
    }
  }
  const int m0 = tm * TM, n0 = tn * kTN;

  // rows in use: all M, or the kept rows (plus zero padding for the gather)
  int R = M, rows_used = M, nb = 0;
  if (kMapped) {
    nb = (rm.n_tokens + rm.block - 1) / rm.block;
    const int nk = *rm.n_kept;
    const bool bad = nk < 0 || nk > nb;
    R = bad ? 0 : nk * rm.block;
    if (!bad && nk > 0) {
      // the short last block of a ragged sequence, when it is the last kept
      // block, has fewer rows
      const int last = rm.kept[nk - 1];
      if (last >= 0 && last < nb) R -= max(0, (last + 1) * rm.block - rm.n_tokens);
    }
    if (EPI == kEpiGather) {
      const long long pad = ((long long)R + rm.pad_multiple - 1) / rm.pad_multiple * rm.pad_multiple;
      rows_used = (int)min((long long)M, pad);
      if (rm.status && blockIdx.x == 0 && blockIdx.z == 0 && threadIdx.x == 0) {
        int f = 0;
        if (bad) f |= LEMO_DEV_BAD_KEPT;
        if (pad > M) f |= LEMO_DEV_CAP_OVERFLOW;
        if (f) atomicOr(rm.status, f);
      }
      R = min(R, M);
    } else {
      if (rm.status && bad && blockIdx.x == 0 && blockIdx.z == 0 && threadIdx.x == 0)
        atomicOr(rm.status, LEMO_DEV_BAD_KEPT);
      if (R > M) {
        if (rm.status && blockIdx.x == 0 && blockIdx.z == 0 && threadIdx.x == 0)
          atomicOr(rm.status, LEMO_DEV_CAP_OVERFLOW);
        R = M;
      }
      rows_used = R;
    }
  }
  if (m0 >= rows_used) return;   // the whole workgroup: before any barrier

  // token row of kept row m, or -1 (index out of range, or a row past the
  // sequence: the short last block listed before the end)
  auto tok_of = [&](int m) {
    const int blk = rm.kept[m / rm.block];
    const int t = blk * rm.block + m % rm.block;
    return (blk >= 0 && blk < nb && t < rm.n_tokens) ? t : -1;
  };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wq = wave / kWN, wk = wave % kWN;
  const int l32 = lane & 31, hi = lane >> 5;
  const uint32_t lds0 = (uint32_t)(uintptr_t)g_tile;

  // instruction i of wave w fills LDS row (i*4 + w)*8 + lane/8 of a region,
  // physical piece lane%8, which holds logical piece (lane%8) ^ swz(row)
  uint32_t voffA[kDmaA], voffB[kDmaB];
#pragma unroll
  for (int i = 0; i < kDmaA; ++i) {
    const int r = (i * kWaves + wave) * 8 + (lane >> 3);
    const int piece = (lane & 7) ^ swz(r);
    int arow;
    if (EPI == kEpiGather) {
      const int t = m0 + r < R ? tok_of(m0 + r) : -1;
      arow = t >= 0 ? t : 0;
    } else {
      arow = min(m0 + r, rows_used - 1);
    }
    voffA[i] = (uint32_t)(((size_t)arow * lda + piece * 8) * 2);
  }
#pragma unroll
  for (int i = 0; i < kDmaB; ++i) {
    const int r = (i * kWaves + wave) * 8 + (lane >> 3);
    const int piece = (lane & 7) ^ swz(r);
    voffB[i] = (uint32_t)(((size_t)min(n0 + r, Nn - 1) * ldb + piece * 8) * 2);
  }
  auto issue = [&](int c, int stage) {
    const uint32_t base = lds0 + (uint32_t)(stage * kStageBytes);
#pragma unroll
    for (int i = 0; i < kDmaA; ++i) dma16(A + c * kChunk, voffA[i], base + (uint32_t)((i * kWaves + wave) * 1024));
#pragma unroll
    for (int i = 0; i < kDmaB; ++i)
      dma16(B + c * kChunk, voffB[i], base + kRegionA + (uint32_t)((i * kWaves + wave) * 1024));
  };

  // per-lane LDS read offsets for the 4 k-steps of a chunk (operand rows all
  // have r & 15 == l32 & 15, so one swizzle serves them)
  uint32_t offA[4], offB[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int piece = (2 * s + hi) ^ swz(l32);
    offA[s] = (uint32_t)((wq * kWM + l32) * kRowBytes + piece * 16);
    offB[s] = (uint32_t)(kRegionA + (wk * kWC + l32) * kRowBytes + piece * 16);
  }

  lemo_f32x16 acc[kMT][kNT];
#pragma unroll
  for (int a = 0; a < kMT; ++a)
#pragma unroll
    for (int b = 0; b < kNT; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;
  lemo_bf16x8 fa[2][kMT], fb[2][kNT];
  auto read_frags = [&](int buf, const uint8_t* st, int s) {
#pragma unroll
    for (int a = 0; a < kMT; ++a)
      fa[buf][a] = *reinterpret_cast<const lemo_bf16x8*>(st + offA[s] + a * 32 * kRowBytes);
#pragma unroll
    for (int i = 0; i < kNT; ++i)
      fb[buf][i] = *reinterpret_cast<const lemo_bf16x8*>(st + offB[s] + i * 32 * kRowBytes);
  };

  const int nchunks = K / kChunk;
  static_assert(kStages == 2 || kStages == 3, "ring depth");
  issue(0, 0);
  if (kStages == 3 && nchunks > 1) issue(1, 1);
  for (int c = 0; c < nchunks; ++c) {
    if constexpr (kStages == 3) {
      // this wave's loads of chunk c have landed (only chunk c+1's may still
      // be in flight); after the barrier every wave's have, and every wave is
      // done with chunk c-1's stage, which is refilled with chunk c+2
      if (c + 1 < nchunks)
        asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(kDmaPerChunk) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      if (c + 2 < nchunks) issue(c + 2, (c + 2) % kStages);
    } else {
      // chunk c has landed everywhere after the barrier, and every wave is
      // done with the other stage, which is refilled with chunk c+1
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      if (c + 1 < nchunks) issue(c + 1, (c + 1) % kStages);
    }
    const uint8_t* st = g_tile + (c % kStages) * kStageBytes;
    read_frags(0, st, 0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int cur = s & 1;
      if (s + 1 < 4) read_frags(cur ^ 1, st, s + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int a = 0; a < kMT; ++a)
#pragma unroll
        for (int b = 0; b < kNT; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][a], fb[cur][b], acc[a][b], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // epilogue: the bf16 tile is staged in LDS (the ring is free once every
  // wave is past the last chunk), then written with 16-byte row accesses
  constexpr int kLdt = T::kLdt;                      // LDS row stride (elements)
  asm volatile("s_barrier" ::: "memory");
  uint16_t* stile = reinterpret_cast<uint16_t*>(g_tile);
#pragma unroll
  for (int a = 0; a < kMT; ++a)
#pragma unroll
    for (int b = 0; b < kNT; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float v = acc[a][b][e];
        if (EPI == kEpiReluBf16) v = fmaxf(v, 0.f);
        stile[(wq * kWM + a * 32 + acc_row(lane, e)) * kLdt + wk * kWC + b * 32 + l32] = (uint16_t)lemo_f32_to_bf16(v);
      }
  __syncthreads();
  constexpr int kPieces = kTN / 8;                   // 16-byte pieces per tile row
  for (int idx = tid; idx < TM * kPieces; idx += kThr) {
    const int r = idx / kPieces, c8 = idx % kPieces;
    const int row = m0 + r, col = n0 + c8 * 8;
    if (row >= rows_used || col >= Nn) continue;
    const uint4 y = *reinterpret_cast<const uint4*>(stile + r * kLdt + c8 * 8);
    if (EPI == kEpiBf16 || EPI == kEpiReluBf16) {
      *reinterpret_cast<uint4*>(C + (size_t)row * ldc + col) = y;
    } else if (EPI == kEpiGather) {
      uint4 out = y;
      if (row >= R) {
        out = make_uint4(0, 0, 0, 0);               // zero padding
      } else if (tok_of(row) < 0) {
        if (rm.status) atomicOr(rm.status, LEMO_DEV_BAD_KEPT);
        continue;                                   // invalid kept block: row left as it is
      }
      *reinterpret_cast<uint4*>(C + (size_t)row * ldc + col) = out;
    } else {
      const int t = tok_of(row);
      if (t < 0) {
        if (rm.status) atomicOr(rm.status, LEMO_DEV_BAD_KEPT);
        continue;
      }
      uint16_t* p = C + (size_t)t * ldc + col;
      const uint4 res = *reinterpret_cast<const uint4*>(p);
      const uint32_t* rw = &res.x;
      const uint32_t* yw = &y.x;
      uint4 o;
      uint32_t* ow = &o.x;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float lo = lemo_bf16_to_f32(rw[j] & 0xffffu) + lemo_bf16_to_f32(yw[j] & 0xffffu);
        const float hi2 = lemo_bf16_to_f32(rw[j] >> 16) + lemo_bf16_to_f32(yw[j] >> 16);
        ow[j] = lemo_f32_to_bf16(lo) | (lemo_f32_to_bf16(hi2) << 16);
      }
      *reinterpret_cast<uint4*>(p) = o;
    }
  }
}

// ---------------------------------------------------------------------------
// Eight-wave ping-pong form of the 256 x 256 tile (d x d weights whose output
// width is a multiple of 256).  The waves form two groups of four (waves w
// and w + 4 share a SIMD): group g owns rows 128 g .. 128 g + 127 of the tile
// as four 128 x 64 wave tiles.  Between barriers the groups take turns: one
// runs the 32 MFMAs of a 64-wide chunk from operands already in registers
// while the other reads its next chunk's operands from LDS.  Phase 2c: group
// 0 multiplies chunk c, group 1 reads it; phase 2c+1: group 1 multiplies
// chunk c, group 0 reads chunk c+1.  The multiplying group issues refills
// between its MFMAs (one after every second MFMA): group 0 its own A rows of
// chunk c+2 (free since it read chunk c), group 1 the B rows and its A rows
// of chunk c+2 (free once it has read chunk c).  A 2-stage ring of 64 KiB
// stages; past the last chunk the loads repeat the last chunk's columns into
// the stage that chunk number maps to, so every wait counts the same loads.
namespace pp {
constexpr int kTM = 256, kTN = 256, kThr = 512;
constexpr int kRegionA = kTM * kRowBytes;                 // 32 KiB
constexpr int kStageBytes = kRegionA + kTN * kRowBytes;   // 64 KiB
constexpr int kDmaA = (kRegionA / 2) / (256 * 16);        // 4 loads per lane: a group's A rows
constexpr int kDmaB = (kTN * kRowBytes) / (256 * 16);     // 8: the B rows (group 1)
constexpr int kLdt = kTN + 8;
constexpr int kLdsBytes = 2 * kStageBytes > kTM * kLdt * 2 ? 2 * kStageBytes : kTM * kLdt * 2;
}  // namespace pp

template <int EPI>
__global__ __launch_bounds__(pp::kThr, 1) void k_gemm_nt_pp(Args g, int lda, int ldb, int M, int Nn, int K, int ldc,
                                                           int tm_count, int tn_count, RowMap rm) {
  constexpr int kMT = 4, kNT = 2;              // 128 x 64 per wave
  __shared__ __attribute__((aligned(1024))) uint8_t g_tile[pp::kLdsBytes];
  constexpr bool kMapped = EPI == kEpiGather || EPI == kEpiScatterAdd;
  const uint16_t* __restrict__ A = g.a[blockIdx.z];
  const uint16_t* __restrict__ B = g.b[blockIdx.z];
  uint16_t* __restrict__ C = g.c[blockIdx.z];
  const int tm = blockIdx.x / tn_count, tn = blockIdx.x % tn_count;
  const int m0 = tm * pp::kTM, n0 = tn * pp::kTN;

  int R = M, rows_used = M, nb = 0;
  if (kMapped) {
    nb = (rm.n_tokens + rm.block - 1) / rm.block;
    const int nk = *rm.n_kept;
    const bool bad = nk < 0 || nk > nb;
    R = bad ? 0 : nk * rm.block;
    if (!bad && nk > 0) {
      const int last = rm.kept[nk - 1];
      if (last >= 0 && last < nb) R -= max(0, (last + 1) * rm.block - rm.n_tokens);
    }
    if (EPI == kEpiGather) {
      const long long pad = ((long long)R + rm.pad_multiple - 1) / rm.pad_multiple * rm.pad_multiple;
      rows_used = (int)min((long long)M, pad);
      if (rm.status && blockIdx.x == 0 && blockIdx.z == 0 && threadIdx.x == 0) {
        int f = 0;
        if (bad) f |= LEMO_DEV_BAD_KEPT;
        if (pad > M) f |= LEMO_DEV_CAP_OVERFLOW;
        if (f) atomicOr(rm.status, f);
      }
      R = min(R, M);
    } else {
      if (rm.status && bad && blockIdx.x == 0 && blockIdx.z == 0 && threadIdx.x == 0)
        atomicOr(rm.status, LEMO_DEV_BAD_KEPT);
      if (R > M) {
        if (rm.status && blockIdx.x == 0 && blockIdx.z == 0 && threadIdx.x == 0)
          atomicOr(rm.status, LEMO_DEV_CAP_OVERFLOW);
        R = M;
      }
      rows_used = R;
    }
  }
  if (m0 >= rows_used) return;   // the whole workgroup: before any barrier

  auto tok_of = [&](int m) {
    const int blk = rm.kept[m / rm.block];
    const int t = blk * rm.block + m % rm.block;
    return (blk >= 0 && blk < nb && t < rm.n_tokens) ? t : -1;
  };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, wl = wave & 3;    // group, wave in the group (= column quarter)
  const int l32 = lane & 31, hi = lane >> 5;
  const uint32_t lds0 = (uint32_t)(uintptr_t)g_tile;
  const int nch = K / kChunk;                  // >= 2 (launcher)

  // loads: instruction i of wave wl of a group fills LDS row (i*4 + wl)*8 +
  // lane/8 of a 128-row (A) or 256-row (B) region, physical piece lane%8;
  // those rows all have the same r & 15, so one piece offset serves them
  const int drow = wl * 8 + (lane >> 3);
  const uint32_t dpiece = (uint32_t)((((lane & 7) ^ swz(drow)) * 8) * 2);
  uint32_t voffA[pp::kDmaA];
#pragma unroll
  for (int i = 0; i < pp::kDmaA; ++i) {
    const int r = grp * 128 + i * 32 + drow;
    int arow;
    if (EPI == kEpiGather) {
      const int t = m0 + r < R ? tok_of(m0 + r) : -1;
      arow = t >= 0 ? t : 0;
    } else {
      arow = min(m0 + r, rows_used - 1);
    }
    voffA[i] = (uint32_t)((size_t)arow * lda * 2) + dpiece;
  }
  // B rows n0 + 32 i + drow: Nn is a multiple of 256, so row 32 i is the
  // scalar part of the address
  const uint32_t voffB = (uint32_t)((size_t)(n0 + drow) * ldb * 2) + dpiece;
  auto dmaA = [&](int c, int i) {
    const int cc = min(c, nch - 1);
    const uint32_t base = lds0 + (uint32_t)((c & 1) * pp::kStageBytes) + (uint32_t)(grp * 128 * kRowBytes);
    dma16(A + cc * kChunk, voffA[i], base + (uint32_t)((i * 4 + wl) * 1024));
  };
  auto dmaB = [&](int c, int i) {
    const int cc = min(c, nch - 1);
    const uint32_t base = lds0 + (uint32_t)((c & 1) * pp::kStageBytes) + (uint32_t)pp::kRegionA;
    dma16(B + (size_t)i * 32 * ldb + cc * kChunk, voffB, base + (uint32_t)((i * 4 + wl) * 1024));
  };

  uint32_t offA[4], offB[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int piece = (2 * s + hi) ^ swz(l32);
    offA[s] = (uint32_t)((grp * 128 + l32) * kRowBytes + piece * 16);
    offB[s] = (uint32_t)(pp::kRegionA + (wl * 64 + l32) * kRowBytes + piece * 16);
  }
  lemo_bf16x8 fa[4][kMT], fb[4][kNT];
  auto read_chunk = [&](int c) {
    uint32_t so = (uint32_t)((c & 1) * pp::kStageBytes);
    asm volatile("" : "+s"(so));
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint8_t* pa = g_tile + offA[s] + so;
      const uint8_t* pb = g_tile + offB[s] + so;
#pragma unroll
      for (int a = 0; a < kMT; ++a) fa[s][a] = *reinterpret_cast<const lemo_bf16x8*>(pa + a * 32 * kRowBytes);
#pragma unroll
      for (int b = 0; b < kNT; ++b) fb[s][b] = *reinterpret_cast<const lemo_bf16x8*>(pb + b * 32 * kRowBytes);
    }
  };

  lemo_f32x16 acc[kMT][kNT];
#pragma unroll
  for (int a = 0; a < kMT; ++a)
#pragma unroll
    for (int b = 0; b < kNT; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;
  auto pin_acc = [&]() {
#pragma unroll
    for (int a = 0; a < kMT; ++a)
#pragma unroll
      for (int b = 0; b < kNT; ++b) asm volatile("" : "+v"(acc[a][b]));
  };
  // the 32 MFMAs of the chunk in fa/fb; group 0 issues its 4 A loads of
  // chunk dc, group 1 its 8 B loads then its 4 A loads, one after every
  // second MFMA
  auto compute = [&](auto G_, int dc) {
    constexpr int G = decltype(G_)::value;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int a = 0; a < kMT; ++a) asm volatile("" : "+v"(fa[s][a]));
#pragma unroll
      for (int b = 0; b < kNT; ++b) asm volatile("" : "+v"(fb[s][b]));
    }
    pin_acc();
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int a = 0; a < kMT; ++a)
#pragma unroll
        for (int b = 0; b < kNT; ++b) {
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[s][a], fb[s][b], acc[a][b], 0, 0, 0);
          const int m = (s * kMT + a) * kNT + b;
          constexpr int kLoads = G == 0 ? pp::kDmaA : pp::kDmaB + pp::kDmaA;
          if ((m & 1) && m / 2 < kLoads) {
            __builtin_amdgcn_sched_barrier(0);
            const int j = m / 2;
            if (G == 0)
              dmaA(dc, j);
            else if (j < pp::kDmaB)
              dmaB(dc, j);
            else
              dmaA(dc, j - pp::kDmaB);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
    __builtin_amdgcn_s_setprio(0);
    pin_acc();
  };

  // prologue: chunks 0 and 1 in flight (each group its own share), chunk 0's
  // rows of this wave landed
  if (grp == 0) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int i = 0; i < pp::kDmaA; ++i) dmaA(c, i);
    asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  } else {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int i = 0; i < pp::kDmaB; ++i) dmaB(c, i);
#pragma unroll
      for (int i = 0; i < pp::kDmaA; ++i) dmaA(c, i);
    }
    asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
  }
  asm volatile("s_barrier" ::: "memory");

  auto run = [&](auto G_) {
    constexpr int G = decltype(G_)::value;
    if (G == 0) read_chunk(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    for (int c = 0; c < nch; ++c) {
      // phase 2c
      if (G == 0)
        compute(G_, c + 2);
      else
        read_chunk(c);
      __builtin_amdgcn_sched_barrier(0);
      // chunk c+1's A rows of group 0 and its B rows have landed: group 0
      // keeps its loads of chunk c+2 in flight (4), group 1 its A rows of
      // chunk c+1 (4, issued after the B rows)
      asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      // phase 2c+1
      if (G == 1) {
        compute(G_, c + 2);
        // group 1's A rows of chunk c+1 have landed; its 12 loads of chunk
        // c+2 stay in flight
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
      } else if (c + 1 < nch) {
        read_chunk(c + 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the repeated loads past the last chunk
  };
  if (grp == 0)
    run(std::integral_constant<int, 0>{});
  else
    run(std::integral_constant<int, 1>{});

  // epilogue: as k_gemm_nt's (wave tile rows 128 grp, columns 64 wl)
  asm volatile("s_barrier" ::: "memory");
  uint16_t* stile = reinterpret_cast<uint16_t*>(g_tile);
#pragma unroll
  for (int a = 0; a < kMT; ++a)
#pragma unroll
    for (int b = 0; b < kNT; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float v = acc[a][b][e];
        if (EPI == kEpiReluBf16) v = fmaxf(v, 0.f);
        stile[(grp * 128 + a * 32 + acc_row(lane, e)) * pp::kLdt + wl * 64 + b * 32 + l32] =
            (uint16_t)lemo_f32_to_bf16(v);
      }
  __syncthreads();
  constexpr int kPieces = pp::kTN / 8;
  for (int idx = tid; idx < pp::kTM * kPieces; idx += pp::kThr) {
    const int r = idx / kPieces, c8 = idx % kPieces;
    const int row = m0 + r, col = n0 + c8 * 8;
    if (row >= rows_used || col >= Nn) continue;
    const uint4 y = *reinterpret_cast<const uint4*>(stile + r * pp::kLdt + c8 * 8);
    if (EPI == kEpiBf16 || EPI == kEpiReluBf16) {
      *reinterpret_cast<uint4*>(C + (size_t)row * ldc + col) = y;
    } else if (EPI == kEpiGather) {
      uint4 out = y;
      if (row >= R) {
        out = make_uint4(0, 0, 0, 0);
      } else if (tok_of(row) < 0) {
        if (rm.status) atomicOr(rm.status, LEMO_DEV_BAD_KEPT);
        continue;
      }
      *reinterpret_cast<uint4*>(C + (size_t)row * ldc + col) = out;
    } else {
      const int t = tok_of(row);
      if (t < 0) {
        if (rm.status) atomicOr(rm.status, LEMO_DEV_BAD_KEPT);
        continue;
      }
      uint16_t* p = C + (size_t)t * ldc + col;
      const uint4 res = *reinterpret_cast<const uint4*>(p);
      const uint32_t* rw = &res.x;
      const uint32_t* yw = &y.x;
      uint4 o;
      uint32_t* ow = &o.x;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float lo = lemo_bf16_to_f32(rw[j] & 0xffffu) + lemo_bf16_to_f32(yw[j] & 0xffffu);
        const float hi2 = lemo_bf16_to_f32(rw[j] >> 16) + lemo_bf16_to_f32(yw[j] >> 16);
        ow[j] = lemo_f32_to_bf16(lo) | (lemo_f32_to_bf16(hi2) << 16);
      }
      *reinterpret_cast<uint4*>(p) = o;
    }
  }
}

// Grid of k_gemm_nt<., TM, TN, WAVES>: row tiles x column tiles, products in z.
inline dim3 grid_for(int tile_rows, int tile_cols, int rows, int cols, int products, int& tm_count, int& tn_count) {
  tm_count = lemo_nblocks(rows, tile_rows);
  tn_count = lemo_nblocks(cols, tile_cols);
  return dim3(tm_count * tn_count, 1, products);
}

}  // namespace gemm

}  // namespace
