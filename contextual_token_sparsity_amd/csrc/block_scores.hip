// Exact block-wise token informativeness on the matrix cores (gfx950).
//
// Jenga (USENIX ATC'25), section 4.2.1, Eq. 1 and Eq. 2, Figure 6 caption:
// per head, S^h = Q^h K^h^T / sqrt(head_dim) (raw pre-softmax scores); each
// (block x block) score tile is reduced to one value M[n][m] and the token
// block score is I[m] = sum_n M[n][m].  Pairs i == j are excluded.
//
// Work decomposition
//   A workgroup of 4 waves owns a 128 x 128 tile of (query rows, key rows)
//   and walks every head; two workgroups share each CU.  Each wave multiplies
//   a 64 x 64 sub-tile with v_mfma_f32_32x32x16_bf16 (2 x 2 MFMA tiles, fp32
//   accumulators in VGPRs).  The head dimension is streamed in 64-wide chunks
//   through a 2-stage LDS ring (64 KiB per workgroup) filled by direct
//   global->LDS loads (global_load_lds_dwordx4): chunk c+1 loads while chunk c
//   multiplies, one barrier per chunk.  The two workgroups on a CU have
//   independent barriers, so one's barrier/restart bubbles are filled by the
//   other's MFMAs.  LDS rows are 128 B; the 16-B pieces of row r are stored
//   XOR-swizzled (piece p at p ^ swz(r)) so that the MFMA operand reads (32
//   rows, one piece each) hit distinct banks.  Operand reads run one k-step
//   ahead of the MFMAs.
//
// The score tile never leaves registers:
//   PAPER   (heads first, then block max): each head's MFMA chain starts
//           from 0 and the head is folded in as sum += max(0, S^h).  For a
//           non-negative float the bit pattern orders like a signed integer
//           while a negative float is a negative integer, so the clamp is one
//           v_max_i32 against 0.  At head_dim 64 (one chunk per head, so the
//           fold weighs twice as much per MFMA) the chain starts from the
//           running sum instead: it ends at sum + S^h, and the fold
//           max(sum + S^h, sum) is one v_max_i32 per element.  The two
//           register sets swap roles from head to head, and a head's fold is
//           deferred to the next head's first k-step, one sub-tile ahead of
//           each first MFMA, so that it runs under the MFMAs: 11 % faster
//           there; at head_dim 128 within +-1 % (box-dependent), so that path
//           keeps the chain from 0.
//   HEADMAX (per-head block max): the head's accumulators are reduced with
//           v_max_i32 starting from 0, which yields max(0, block max) (the
//           clamp is free for the same reason), then across lanes; the clamped
//           per-head maxima are summed over heads in head order.
// Pairs that take no part are set to 0, which changes neither reduction
// (PAPER values are >= 0, HEADMAX clamps at 0), and a block pair with none
// left scores 0: the i == j pairs on the diagonal of diagonal sub-tiles; in
// the causal variant (decoder attention pairs no query with a later key)
// every j >= i; and, when N is not a multiple of the block size, the rows
// past the sequence end that fill the last tile (loaded as copies of row
// N-1).  Only waves whose 64 x 64 square holds such a pair test them.  The
// scale 1/sqrt(head_dim) (and 1/H for PAPER) is applied once to the block
// value; every step is positively homogeneous so this is exact up to
// rounding.
//
// Launches without a ragged last block, with an even head count and enough
// tiles to fill the chip (causal ones with N a multiple of 256) run
// k_block_scores_pp instead: one
// eight-wave workgroup per CU on a 256 x 128 tile, whose two groups of four
// waves take turns between matrix phases and memory phases (its comment
// below gives the schedule).
//
// Causal launches cover only the tiles on or below the tile diagonal; each
// tile below it also writes the zeros of its mirror tile above.  A batch of
// independent sequences is the grid's y dimension.  The column aggregate is a
// second, deterministic pass (k_colsum).
#include <type_traits>

#include "lemo_internal.h"

namespace {

constexpr int kTQ = 128;        // query rows per workgroup
constexpr int kTK = 128;        // key rows per workgroup
constexpr int kWaves = 4;       // 2 (query) x 2 (key) waves of 64 x 64
constexpr int kThreads = kWaves * 64;
constexpr int kChunk = 64;      // head-dim elements per pipeline stage
constexpr int kRowBytes = kChunk * 2;              // 128 B: eight 16-B pieces
constexpr int kStageQ = kTQ * kRowBytes;           // 16 KiB
constexpr int kStageK = kTK * kRowBytes;           // 16 KiB
constexpr int kStageBytes = kStageQ + kStageK;     // 32 KiB
constexpr int kStages = 2;                         // 64 KiB per workgroup: two workgroups per CU
constexpr int kDmaQ = kStageQ / (kThreads * 16);   // 4 loads of 16 B per thread
constexpr int kDmaK = kStageK / (kThreads * 16);   // 4
constexpr int kDmaPerChunk = kDmaQ + kDmaK;
constexpr int kMaxHeadsHeadmax = 128;

static_assert(kDmaQ * kThreads * 16 == kStageQ && kDmaK * kThreads * 16 == kStageK, "stage split");

__shared__ __attribute__((aligned(1024))) uint8_t g_stage[kStages * kStageBytes];

// Piece swizzle of LDS row r: distinct for 8 consecutive rows and for the 8
// even (odd) rows among 16 consecutive rows, so a wave's 32-row operand read
// is conflict-free whether the LDS serves 8 or 16 pieces per cycle.
__device__ __forceinline__ int swz(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }

// Output row of register e of `lane` in a 32x32 MFMA accumulator (column = lane % 32).
__device__ __forceinline__ int acc_row(int lane, int e) { return 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3); }

// One 16-byte direct global->LDS load per lane: lane l reads base + voff and
// writes lds_base + 16 l.  (No register result; completion is tracked with
// vmcnt by the caller.)
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_base), "v"(voff), "s"(base) : "memory");
}

__device__ __forceinline__ int imax(int a, int b) { return a > b ? a : b; }

// Maximum over the wave's 64 lanes, as a wave-uniform value, without LDS
// round trips: DPP swaps inside each row of 16 lanes (quad pairs, quad
// halves, half-row mirror, row mirror) leave every lane of a row with the
// row's maximum; the four row maxima are then read out as scalars.  (A
// butterfly of __shfl_xor goes through LDS: six round trips per reduction;
// the DPP form made HEADMAX, which reduces every head, 9% faster.)
__device__ __forceinline__ int wave_imax(int v) {
  v = imax(v, __builtin_amdgcn_update_dpp(v, v, 0xB1, 0xF, 0xF, false));    // quad_perm [1,0,3,2]
  v = imax(v, __builtin_amdgcn_update_dpp(v, v, 0x4E, 0xF, 0xF, false));    // quad_perm [2,3,0,1]
  v = imax(v, __builtin_amdgcn_update_dpp(v, v, 0x141, 0xF, 0xF, false));   // row_half_mirror
  v = imax(v, __builtin_amdgcn_update_dpp(v, v, 0x140, 0xF, 0xF, false));   // row_mirror
  return imax(imax(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
              imax(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

// Workgroup wg runs on XCD wg % 8 as its (wg / 8)-th workgroup there.  Give
// XCD x the x-th of 8 contiguous ranges of the logical order (the first
// total % 8 ranges one longer), so each XCD's L2 serves neighbouring tiles.
__device__ __forceinline__ int xcd_logical(int wg, int total) {
  const int x = wg % 8, base = total / 8, rem = total % 8;
  return x * base + min(x, rem) + wg / 8;
}

// Maps a logical tile index to a (query tile, key tile) pair.  Dispatch goes
// round-robin over the 8 XCDs; each XCD gets a contiguous range of logical
// tiles (xcd_logical), walked in groups of 8 query tiles so that the 64 workgroups
// resident on one XCD (2 per CU) cover an 8 x 8 patch of tiles and share Q
// and K rows in that XCD's L2.  (Groups of 2, 4 or 16 rows, or a serpentine
// walk, time within 1-2 % of this at N = 16384.)
__device__ __forceinline__ void tile_of(int logical, int ntq, int ntk, int& tq, int& tk) {
  constexpr int kGroup = 8;
  const int span = kGroup * ntk;
  const int g = logical / span;
  const int first = g * kGroup;
  const int rows = min(kGroup, ntq - first);
  const int in_group = logical - g * span;
  tq = first + in_group % rows;
  tk = in_group / rows;
}

// Causal launches: the tiles (tq, tk) with tk <= tq, ntq * (ntq + 1) / 2 of
// them, in groups of 8 query tiles as in tile_of.  The
// groups before group g hold the T(8g) tiles of query tiles < 8g, where
// T(x) = x (x + 1) / 2; inside a group the key tiles left of the group's
// first query tile are full columns of `rows` tiles, then the group's own
// triangle follows row by row.
__device__ __forceinline__ int tri(int x) { return x * (x + 1) / 2; }

// the r with T(r) <= t < T(r + 1)
__device__ __forceinline__ int tri_row(int t) {
  int r = (int)((__builtin_sqrtf(8.f * (float)t + 1.f) - 1.f) * 0.5f);
  while (tri(r + 1) <= t) ++r;
  while (r > 0 && tri(r) > t) --r;
  return r;
}

__device__ __forceinline__ void tri_tile_of(int logical, int ntq, int& tq, int& tk) {
  constexpr int kGroup = 8;
  const int first = (tri_row(logical) / kGroup) * kGroup;
  const int rows = min(kGroup, ntq - first);
  const int in_group = logical - tri(first);
  if (in_group < rows * first) {
    tq = first + in_group % rows;
    tk = in_group / rows;
  } else {
    const int t = in_group - rows * first;
    const int i = tri_row(t);
    tq = first + i;
    tk = first + t - tri(i);
  }
}

// Which pairs a launch must exclude.  kMaskDiag: only i == j, all a launch
// needs when N is a multiple of the block size (rows past N in the last tile
// then form whole blocks that are never written); kMaskRagged: also rows past
// N inside the last block; kMaskCausal: every j >= i and rows past N.
enum { kMaskDiag = 0, kMaskRagged = 1, kMaskCausal = 2 };

template <int HD, int MODE, int BLK, int MASK>
__global__ __launch_bounds__(kThreads, 2) void k_block_scores(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, int n_tokens, int n_heads, int ldq,
    int ldk, long long bsq, long long bsk, float out_scale, float* __restrict__ M, int nb, int ntq, int ntk) {
  constexpr bool CAUSAL = MASK == kMaskCausal;
  constexpr int kCPH = HD / kChunk;                      // chunks per head
  // PAPER at head_dim 64 starts each head's MFMA chain from the running sum,
  // so the fold is one max per element; the fold of a head is deferred to the
  // next head's first k-step and interleaved one sub-tile at a time with its
  // first MFMAs.  At head_dim 128 this measured within +-1 % of the chain
  // from 0 (box-dependent), which stays there.
  constexpr bool kSumChain = MODE == 0 && HD == 64;
  constexpr int kParts = (MODE == 1 && BLK == 128) ? kMaxHeadsHeadmax : 1;
  __shared__ float part[kWaves][kParts];                 // HEADMAX, 128-row blocks: per-head wave maxima
  __shared__ float fin[kWaves * 4];                      // final per-(wave, sub-tile) values

  // the grid is (tiles per sequence) x (sequences); the batch's tiles form
  // one logical order, sequence by sequence, split into XCD ranges
  const int T = gridDim.x;
  const int logical = xcd_logical(blockIdx.y * T + blockIdx.x, T * gridDim.y);
  const int seq = logical / T;
  int tq, tk;
  if (CAUSAL)
    tri_tile_of(logical - seq * T, ntq, tq, tk);
  else
    tile_of(logical - seq * T, ntq, ntk, tq, tk);
  Q += (size_t)seq * bsq;
  K += (size_t)seq * bsk;
  M += (size_t)seq * nb * nb;
  const int q0 = tq * kTQ, k0 = tk * kTK;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wq = wave >> 1, wk = wave & 1;
  const int l32 = lane & 31, hi = lane >> 5;
  // does this wave's 64 x 64 square hold a pair that takes no part?
  const int qlo = q0 + wq * 64, klo = k0 + wk * 64;
  const bool mask_wave = MASK == kMaskDiag
                             ? klo == qlo
                             : (CAUSAL ? klo >= qlo : klo == qlo) || qlo + 64 > n_tokens || klo + 64 > n_tokens;
  const uint32_t lds0 = (uint32_t)(uintptr_t)g_stage;

  // ---- per-lane DMA byte offsets: instruction i of this wave fills LDS
  // pieces P = (i*kWaves + wave)*64 + lane of the Q (i < kDmaQ) or K region, i.e.
  // row P/8 and physical piece P%8, which holds logical piece (P%8) ^ swz(row).
  uint32_t voff[kDmaPerChunk];
#pragma unroll
  for (int i = 0; i < kDmaPerChunk; ++i) {
    const bool is_q = i < kDmaQ;
    const int ii = is_q ? i : i - kDmaQ;
    const int r = (ii * kWaves + wave) * 8 + (lane >> 3);
    const int piece = (lane & 7) ^ swz(r);
    const int grow = min((is_q ? q0 : k0) + r, n_tokens - 1);   // rows past N: any valid row
    voff[i] = (uint32_t)(((size_t)grow * (is_q ? ldq : ldk) + piece * 8) * 2);
  }
  // loads of chunk c (head h, part kc) into stage `stage`
  auto issue = [&](int h, int kc, int stage) {
    const int col = h * HD + kc * kChunk;
    const uint16_t* qb = Q + col;
    const uint16_t* kb = K + col;
    const uint32_t base = lds0 + (uint32_t)(stage * kStageBytes);
#pragma unroll
    for (int i = 0; i < kDmaPerChunk; ++i) {
      const bool is_q = i < kDmaQ;
      const int ii = is_q ? i : i - kDmaQ;
      dma16(is_q ? (const void*)qb : (const void*)kb, voff[i],
            base + (is_q ? 0u : (uint32_t)kStageQ) + (uint32_t)((ii * kWaves + wave) * 1024));
    }
  };

  // ---- per-lane LDS read offsets (bytes from g_stage, stage 0) for the four
  // k-steps of a chunk; every operand row this lane reads has r & 15 == l32 & 15.
  uint32_t offA[4], offB[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int piece = (2 * s + hi) ^ swz(l32);
    offA[s] = (uint32_t)((wq * 64 + l32) * kRowBytes + piece * 16);
    offB[s] = (uint32_t)(kStageQ + (wk * 64 + l32) * kRowBytes + piece * 16);
  }

  // Zeroes the entries of sub-tile (a, b) whose pair takes no part: i == j
  // (j >= i when causal), or a query or key row past the sequence end.
  // Element e of this lane pairs query row qb + r_e (r_e = acc_row(lane, e)
  // - 4 hi, a constant per e) with key row kr.  The empty asm makes both
  // bases opaque, so the compares are redone at each call rather than hoisted
  // out of the head loop as 64 live lane masks.
  auto mask_tile = [&](lemo_f32x16& v, int a, int b) {
    int qb = qlo + a * 32 + 4 * hi;
    int kr = klo + b * 32 + l32;
    asm volatile("" : "+v"(qb), "+v"(kr));
    const int dq = kr - qb;                                  // i == j at r_e == dq
    const int lim = kr >= n_tokens ? 0 : n_tokens - qb;      // rows r_e >= lim are out
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = 8 * (e >> 2) + (e & 3);
      const bool out = (CAUSAL ? r <= dq : r == dq) || r >= lim;
      if (out) v[e] = 0.f;
    }
  };

  // the exclusions of sub-tile (a, b) of a masked wave; with kMaskDiag only
  // the diagonal of the diagonal sub-tiles (a plain compare: the general
  // form costs HEADMAX about 4 % even in the waves that skip it)
  auto exclude = [&](lemo_f32x16& v, int a, int b) {
    if (MASK == kMaskDiag) {
      if (a == b) {
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (acc_row(lane, e) == l32) v[e] = 0.f;
      }
    } else {
      mask_tile(v, a, b);
    }
  };

  lemo_f32x16 sum[2][2];          // PAPER: running sum over heads of max(0, S^h)
  lemo_f32x16 acc[2][2][2];       // [head parity][sub-tile]: S^h of the current and previous head
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) sum[a][b][e] = 0.f;
  if (kSumChain) {   // the first head's deferred fold then reads zeros
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[0][a][b][e] = 0.f;
  }
  float total[2][2] = {{0.f, 0.f}, {0.f, 0.f}};  // HEADMAX, blocks <= 64 rows: sum over heads
  int hm_lane = 0;                                // HEADMAX, blocks >= 64: this lane's running block max

  // HEADMAX: folds sub-tile t = (a, b) of a finished head (accumulators
  // acc[P]) into the cross-head state (the clamped block maxima summed over
  // heads).  Runs interleaved with the next head's MFMAs.
  auto finalize = [&](auto P_, int t, int h) {
    constexpr int P = decltype(P_)::value;
    const int a = t >> 1, b = t & 1;
    int m = BLK >= 64 ? hm_lane : 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) m = imax(m, __float_as_int(acc[P][a][b][e]));
    if (BLK >= 64) {
      hm_lane = m;
      if (t == 3) {  // all four sub-tiles lie in one block: reduce across lanes
        m = wave_imax(m);
        hm_lane = 0;
        if (BLK == 128) {
          if (lane == 0) part[wave][h] = __int_as_float(m);
        } else {
          total[0][0] += __int_as_float(m);
        }
      }
    } else {
      total[a][b] += __int_as_float(wave_imax(m));
    }
  };

  const int nchunks = n_heads * kCPH;
  lemo_bf16x8 fa[2][2], fb[2][2];   // operand fragments, [k-step buffer][sub-tile]
  auto read_frags = [&](int buf, const uint8_t* st, int s) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      fa[buf][i] = *reinterpret_cast<const lemo_bf16x8*>(st + offA[s] + i * 32 * kRowBytes);
      fb[buf][i] = *reinterpret_cast<const lemo_bf16x8*>(st + offB[s] + i * 32 * kRowBytes);
    }
  };

  issue(0, 0, 0);

  // One head h into acc[P].  Each chunk step: this wave's loads of chunk c
  // have landed (nothing newer is in flight), then a workgroup barrier, after
  // which chunk c is complete in LDS and every wave has consumed chunk c-1
  // (its operands are in registers), so the other stage is refilled with
  // chunk c+1 while chunk c is multiplied.  The barrier is a plain s_barrier:
  // no LDS fence is needed, since no wave reads LDS that another wave wrote.
  // Two workgroups share each CU; their barriers are independent, so one
  // workgroup's barrier and restart bubbles are filled by the other's MFMAs.
  // During the head's first chunk the previous head (acc[1-P]) is folded in
  // (HEADMAX), one sub-tile per k-step, under the MFMAs.
  auto do_head = [&](auto P_, int h) {
    constexpr int P = decltype(P_)::value;
#pragma unroll
    for (int kc = 0; kc < kCPH; ++kc) {
      const int c = h * kCPH + kc;
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      if (c + 1 < nchunks) issue((c + 1) / kCPH, (c + 1) % kCPH, (c + 1) % kStages);
      const uint8_t* st = g_stage + (c % kStages) * kStageBytes;
      read_frags(0, st, 0);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int cur = s & 1;
        // operand reads run one k-step ahead of the MFMAs; the scheduling
        // fences keep the compiler from folding the two buffers into one
        if (s + 1 < 4) read_frags(cur ^ 1, st, s + 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            if (kSumChain) {
              // PAPER: even heads run their chain in acc[0] from the running
              // sum in sum[], odd heads in sum[] from acc[0].  At a head's
              // first k-step, sub-tile by sub-tile: the previous head's fold
              // (its chain c0 := max(c0, d), d holding the sum before that
              // head), then the first MFMA, written out with its own
              // destination because the compiler would otherwise copy the
              // source into it first; the s_nop covers the wait after the
              // fold's VALU writes of that source.
              lemo_f32x16& d = P == 0 ? acc[0][a][b] : sum[a][b];
              lemo_f32x16& c0 = P == 0 ? sum[a][b] : acc[0][a][b];
              if (kc == 0 && s == 0) {
                // the previous head's fold of this sub-tile: c0 (its chain)
                // = max(c0, d) (d still holds the sum before that head)
#pragma unroll
                for (int e = 0; e < 16; ++e) c0[e] = __int_as_float(imax(__float_as_int(c0[e]), __float_as_int(d[e])));
                asm volatile("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %3"
                             : "=&v"(d) : "v"(fa[cur][a]), "v"(fb[cur][b]), "v"(c0));
                __builtin_amdgcn_sched_barrier(0);   // the next sub-tile's fold runs under this MFMA
              } else
                d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][a], fb[cur][b], d, 0, 0, 0);
            } else if (kc == 0 && s == 0) {  // first k-step of a head: the chain starts from 0
              acc[P][a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][a], fb[cur][b], lemo_f32x16{}, 0, 0, 0);
            } else {
              acc[P][a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][a], fb[cur][b], acc[P][a][b], 0, 0, 0);
            }
          }
        if (MODE == 1 && kc == 0 && h > 0) finalize(std::integral_constant<int, 1 - P>{}, s, h - 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (MODE == 0 && !kSumChain) {
      // sum += max(0, S^h): a negative float is a negative integer, so the
      // clamp is one v_max_i32 against 0
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            sum[a][b][e] += __int_as_float(imax(__float_as_int(acc[P][a][b][e]), 0));
    }
    // HEADMAX: excluded pairs leave the head's tile before it is folded in
    // (one pass, only in waves that hold such pairs, outside the
    // interleaved fold so the common path keeps its schedule)
    if (MODE == 1 && mask_wave) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) exclude(acc[P][a][b], a, b);
    }
  };

  if (kSumChain) {
    int h = 0;
    for (; h + 1 < n_heads; h += 2) {
      do_head(std::integral_constant<int, 0>{}, h);
      do_head(std::integral_constant<int, 1>{}, h + 1);
    }
    if (h < n_heads) {   // an odd head count: the last head's chain is in acc[0]
      do_head(std::integral_constant<int, 0>{}, h);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            sum[a][b][e] = __int_as_float(imax(__float_as_int(acc[0][a][b][e]), __float_as_int(sum[a][b][e])));
    } else {             // an even head count: the last head's chain is in sum
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            sum[a][b][e] = __int_as_float(imax(__float_as_int(sum[a][b][e]), __float_as_int(acc[0][a][b][e])));
    }
  } else if (MODE == 0) {
    for (int h = 0; h < n_heads; ++h) do_head(std::integral_constant<int, 0>{}, h);
  } else {
    int h = 0;
    for (; h + 1 < n_heads; h += 2) {
      do_head(std::integral_constant<int, 0>{}, h);
      do_head(std::integral_constant<int, 1>{}, h + 1);
    }
    if (h < n_heads) {
      do_head(std::integral_constant<int, 0>{}, h);
#pragma unroll
      for (int t = 0; t < 4; ++t) finalize(std::integral_constant<int, 0>{}, t, h);
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) finalize(std::integral_constant<int, 1>{}, t, h - 1);
    }
  }

  // ---- per-(wave, sub-tile) block values -> fin[]
  if (MODE == 0) {
    if (mask_wave) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) exclude(sum[a][b], a, b);
    }
    if (BLK >= 64) {
      int m = 0;
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int e = 0; e < 16; ++e) m = imax(m, __float_as_int(sum[a][b][e]));
      m = wave_imax(m);
      if (lane == 0) fin[wave * 4] = __int_as_float(m);
    } else {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          int m = 0;
#pragma unroll
          for (int e = 0; e < 16; ++e) m = imax(m, __float_as_int(sum[a][b][e]));
          m = wave_imax(m);
          if (lane == 0) fin[wave * 4 + a * 2 + b] = __int_as_float(m);
        }
    }
  } else if (BLK == 64) {
    if (lane == 0) fin[wave * 4] = total[0][0];
  } else if (BLK == 32) {
    if (lane == 0) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) fin[wave * 4 + a * 2 + b] = total[a][b];
    }
  }
  __syncthreads();

  // ---- combine the parts of each block of this tile and write M
  constexpr int kBQ = kTQ / BLK, kBK = kTK / BLK;   // blocks per tile side
  if (tid < kBQ * kBK) {
    const int lq = tid / kBK, lk = tid % kBK;
    const int bq = q0 / BLK + lq, bk = k0 / BLK + lk;
    if (bq < nb && bk < nb) {
      float val = 0.f;
      if (MODE == 1 && BLK == 128) {
        // waves (wq, wk) with wq / 2 == lq cover this block; heads summed in order
        for (int h = 0; h < n_heads; ++h) {
          float m = 0.f;
          for (int w = 0; w < kWaves; ++w)
            if ((w >> 1) * 64 / BLK == lq) m = fmaxf(m, part[w][h]);
          val += m;
        }
      } else {
        // sub-tile (a, b) of wave (wq, wk) covers query rows wq*64 + a*32 and
        // key rows wk*64 + b*32 of the tile; PAPER takes the max of the parts,
        // HEADMAX (blocks <= 64 rows) has exactly one part per block
        for (int p = 0; p < kWaves * 4; ++p) {
          const int w = p >> 2, a = (p >> 1) & 1, b = p & 1;
          if (BLK >= 64 && (a | b)) continue;
          const int rq = ((w >> 1) * 64 + a * 32) / BLK, rk = ((w & 1) * 64 + b * 32) / BLK;
          if (rq == lq && rk == lk) val = fmaxf(val, fin[p]);
        }
      }
      M[(size_t)bq * nb + bk] = val * out_scale;
      // causal: the mirror tile (tk, tq) above the diagonal is not launched;
      // its blocks have no pair with j < i
      if (CAUSAL && tq != tk) M[(size_t)bk * nb + bq] = 0.f;
    }
  }
}

// ---------------------------------------------------------------------------
// Eight-wave form of the same reduction (the launcher's choice for launches
// without a ragged last block, with an even head count and enough tiles to
// fill the chip; causal ones also need N to be a multiple of 256, and then
// cover the tiles on or below the diagonal, with the exclusions and mirror
// zeros of k_block_scores).  One workgroup per CU owns a 256 x 128 tile (query rows x key
// rows): 25 % fewer refill bytes per MFMA than two 128 x 128 workgroups.
// Its waves form two groups of four, one wave of each group per SIMD, each
// group a 2 x 2 grid of 64 x 64 wave tiles (group g: query rows 128 g ..
// 128 g + 127).  The groups take turns between barriers: while one group
// runs a whole 64-wide chunk of MFMAs from operands already in registers,
// the other reads its next chunk's operands from LDS and folds its last head,
// so every phase keeps the matrix cores of all four SIMDs busy with one
// wave's MFMAs while the other wave's LDS reads and VALU work run beside
// them.  The refills (direct global->LDS loads into a 3-stage ring of 48 KiB
// stages) are issued by the multiplying group, one after every second MFMA.
//
// Phases: 2c (group 0 multiplies chunk c, group 1 reads it) and 2c+1
// (group 1 multiplies chunk c, group 0 reads chunk c+1).  Chunk c+1 must be
// in LDS at the barrier that ends phase 2c; each wave then has the loads of
// chunks c+1 and c+2 in flight (group 1 issues its part of chunk c+3 in
// phase 2c+1, group 0 its part of chunk c+2 in phase 2c), so the wait is
// always "6 loads may remain".  Past the last chunk the loads repeat the last
// chunk's columns into the stage that chunk number maps to, which is no
// longer read, so the count holds to the end.  The stage of chunk c is free
// once both groups have read it (phases 2c-1 and 2c).
//
// PAPER folds each head with one VALU op per element: head h runs its MFMA
// chain in register set h % 2 starting from the other set, which holds the
// running sum R, so the chain ends at R + S^h and the fold is
// set[h % 2] = max(set[h % 2], set[1 - h % 2]) = R + max(0, S^h).  The first
// MFMA of a head is written out in assembly with its own destination (the
// compiler would otherwise copy the source set into it first).  HEADMAX
// chains start from 0 and fold as in k_block_scores.
namespace pp {
constexpr int kTQ = 256, kTK = 128, kWaves = 8, kThreads = 512;
constexpr int kStageQ = kTQ * kRowBytes;                 // 32 KiB
constexpr int kStageK = kTK * kRowBytes;                 // 16 KiB
constexpr int kStageBytes = kStageQ + kStageK;           // 48 KiB
constexpr int kStages = 3;                               // 144 KiB
constexpr int kDmaQ = kStageQ / (kThreads * 16);         // 4 loads of 16 B per lane
constexpr int kDmaK = kStageK / (kThreads * 16);         // 2
constexpr int kDma = kDmaQ + kDmaK;
static_assert(kDmaQ * kThreads * 16 == kStageQ && kDmaK * kThreads * 16 == kStageK, "stage split");
static_assert(kDma == 6, "the barrier waits count 6 loads per chunk and wave");

// as tile_of, with 32 resident workgroups per XCD (one per CU): groups of 4
// query tiles, so that the resident workgroups cover 4 x 8 tiles
__device__ __forceinline__ void tile_of(int logical, int ntq, int ntk, int& tq, int& tk) {
  constexpr int kGroup = 4;
  const int span = kGroup * ntk;
  const int g = logical / span;
  const int first = g * kGroup;
  const int rows = min(kGroup, ntq - first);
  const int in_group = logical - g * span;
  tq = first + in_group % rows;
  tk = in_group / rows;
}

// Causal launches (N a multiple of 256, so 2 ntq key tiles): the tiles
// (tq, tk) with tk <= 2 tq + 1, i.e. those holding a pair j < i, ntq (ntq + 1)
// of them.  Groups of 4 query tiles as above; the tiles of the query tiles
// before group g number 4g (4g + 1) (query tile t has 2t + 2), and inside a
// group the key tiles up to 2 first + 1 are full columns of the group's rows,
// then each pair of columns loses the group's top row.
__device__ __forceinline__ void tri_tile_of(int logical, int ntq, int& tq, int& tk) {
  int g = (int)((__builtin_sqrtf(1.f + 16.f * (float)logical) - 1.f) * 0.125f);   // 16 g^2 + 4 g <= logical
  while (g > 0 && 4 * g * (4 * g + 1) > logical) --g;
  while (4 * (g + 1) < ntq && 4 * (g + 1) * (4 * (g + 1) + 1) <= logical) ++g;
  const int first = 4 * g;
  const int rows = min(4, ntq - first);
  int idx = logical - first * (first + 1);
  const int full = rows * (2 * first + 2);
  if (idx < full) {
    tk = idx / rows;
    tq = first + idx % rows;
    return;
  }
  idx -= full;
  int j = 0;   // columns 2 first + 2 + 2j and + 1 hold rows first + 1 + j .. first + rows - 1
  while (idx >= 2 * (rows - 1 - j)) {
    idx -= 2 * (rows - 1 - j);
    ++j;
  }
  const int n = rows - 1 - j;
  tk = 2 * first + 2 + 2 * j + idx / n;
  tq = first + 1 + j + idx % n;
}
}  // namespace pp

template <int HD, int MODE, int BLK, bool CAUSAL>
__global__ __launch_bounds__(pp::kThreads, 1) void k_block_scores_pp(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, int n_tokens, int n_heads, int ldq, int ldk,
    long long bsq, long long bsk, float out_scale, float* __restrict__ M, int nb, int ntq, int ntk) {
  constexpr int kCPH = HD / kChunk;
  constexpr int kParts = (MODE == 1 && BLK == 128) ? kMaxHeadsHeadmax : 1;
  __shared__ __attribute__((aligned(1024))) uint8_t ring[pp::kStages * pp::kStageBytes];
  __shared__ float part[pp::kWaves][kParts];   // HEADMAX, 128-row blocks: per-head wave maxima
  __shared__ float fin[pp::kWaves * 4];        // final per-(wave, sub-tile) values

  const int T = gridDim.x;
  const int logical = xcd_logical(blockIdx.y * T + blockIdx.x, T * gridDim.y);
  const int seq = logical / T;
  int tq, tk;
  if (CAUSAL)
    pp::tri_tile_of(logical - seq * T, ntq, tq, tk);
  else
    pp::tile_of(logical - seq * T, ntq, ntk, tq, tk);
  Q += (size_t)seq * bsq;
  K += (size_t)seq * bsk;
  M += (size_t)seq * nb * nb;
  const int q0 = tq * pp::kTQ, k0 = tk * pp::kTK;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;   // waves w and w + 4 share a SIMD
  const int wq = (wave >> 1) & 1, wk = wave & 1;
  const int l32 = lane & 31, hi = lane >> 5;
  const int qlo = q0 + grp * 128 + wq * 64, klo = k0 + wk * 64;
  // does this wave's 64 x 64 square hold a pair that takes no part: i == j
  // (a diagonal block), or j >= i when causal
  const bool mask_wave = CAUSAL ? klo >= qlo : klo == qlo;
  const uint32_t lds0 = (uint32_t)(uintptr_t)ring;
  const int C = n_heads * kCPH;        // chunks; n_heads is even (launcher)

  // ---- loads: instruction i of this wave fills LDS row 64 ii + drow of the
  // Q (i < kDmaQ) or K region, physical piece lane % 8 (logical piece
  // (lane % 8) ^ swz(row); the rows of one lane differ by 64, so one piece
  // offset serves all of them)
  const int drow = wave * 8 + (lane >> 3);
  const uint32_t dpiece = (uint32_t)((((lane & 7) ^ swz(drow)) * 8) * 2);
  uint32_t voff[pp::kDma];
#pragma unroll
  for (int i = 0; i < pp::kDma; ++i) {
    const bool is_q = i < pp::kDmaQ;
    const int ii = is_q ? i : i - pp::kDmaQ;
    const int grow = min((is_q ? q0 : k0) + 64 * ii + drow, n_tokens - 1);   // rows past N: any valid row
    voff[i] = (uint32_t)((size_t)grow * (is_q ? ldq : ldk) * 2) + dpiece;
  }
  // load i of chunk dc into the stage dc maps to; past the last chunk the
  // last chunk's columns again
  auto dma = [&](int dc, int i) {
    const int cc = min(dc, C - 1);
    const int col = (cc / kCPH) * HD + (cc % kCPH) * kChunk;
    const bool is_q = i < pp::kDmaQ;
    const int ii = is_q ? i : i - pp::kDmaQ;
    const uint32_t base = lds0 + (uint32_t)((dc % pp::kStages) * pp::kStageBytes);
    dma16(is_q ? (const void*)(Q + col) : (const void*)(K + col), voff[i],
          base + (is_q ? 0u : (uint32_t)pp::kStageQ) + (uint32_t)((ii * pp::kWaves + wave) * 1024));
  };

  // ---- operand reads of one chunk: all four k-steps into registers
  uint32_t offA[4], offB[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int piece = (2 * s + hi) ^ swz(l32);
    offA[s] = (uint32_t)((grp * 128 + wq * 64 + l32) * kRowBytes + piece * 16);
    offB[s] = (uint32_t)(pp::kStageQ + (wk * 64 + l32) * kRowBytes + piece * 16);
  }
  lemo_bf16x8 fa[4][2], fb[4][2];   // [k-step][sub-tile row / column]
  auto read_chunk = [&](int c) {
    // the stage offset is opaque to the compiler, which would otherwise keep
    // the read addresses of all three stages in registers
    uint32_t so = (uint32_t)((c % pp::kStages) * pp::kStageBytes);
    asm volatile("" : "+s"(so));
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint8_t* pa = ring + offA[s] + so;
      const uint8_t* pb = ring + offB[s] + so;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        fa[s][i] = *reinterpret_cast<const lemo_bf16x8*>(pa + i * 32 * kRowBytes);
        fb[s][i] = *reinterpret_cast<const lemo_bf16x8*>(pb + i * 32 * kRowBytes);
      }
    }
  };

  // PAPER: the two register sets of the running sum (see above); HEADMAX:
  // acc holds the head's chain
  lemo_f32x16 acc[2][2], sum[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        sum[a][b][e] = 0.f;
        acc[a][b][e] = 0.f;
      }
  float total[2][2] = {{0.f, 0.f}, {0.f, 0.f}};   // HEADMAX, blocks <= 64 rows: sum over heads

  // Empty volatile asm pins a value to a point of the instruction stream.
  // Volatile asm keeps its order with the barriers, so a phase's arithmetic
  // (which the barriers alone would not hold in place: the compiler moved a
  // fold into the neighbouring matrix phase) stays between its barriers.
  auto pin_acc = [&]() {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) asm volatile("" : "+v"(acc[a][b]));
  };
  auto pin_sum = [&]() {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) asm volatile("" : "+v"(sum[a][b]));
  };

  // A matrix phase: the 16 MFMAs of the chunk in fa/fb (FIRST: the head's
  // first chunk) for a head of parity P, with this wave's loads of chunk dc
  // (none if dc < 0) issued one after every second MFMA, where they wait for
  // the vector memory path under queued MFMAs.  The raised wave priority
  // lets these MFMAs issue ahead of the other wave's reads and VALU work.
  auto compute = [&](auto FIRST_, auto P_, int dc) {
    constexpr bool FIRST = decltype(FIRST_)::value;
    constexpr int P = decltype(P_)::value;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < 2; ++i) asm volatile("" : "+v"(fa[s][i]), "+v"(fb[s][i]));
    pin_acc();
    if (MODE == 0) pin_sum();
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          if (MODE == 0) {
            lemo_f32x16& d = P == 0 ? acc[a][b] : sum[a][b];
            lemo_f32x16& c0 = P == 0 ? sum[a][b] : acc[a][b];
            if (FIRST && s == 0)   // the s_nop covers the wait after the fold's VALU writes of c0
              asm volatile("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %3"
                           : "=&v"(d)
                           : "v"(fa[s][a]), "v"(fb[s][b]), "v"(c0));
            else
              d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[s][a], fb[s][b], d, 0, 0, 0);
          } else {
            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                fa[s][a], fb[s][b], (FIRST && s == 0) ? lemo_f32x16{} : acc[a][b], 0, 0, 0);
          }
          const int m = s * 4 + a * 2 + b;
          if ((m & 1) && m / 2 < pp::kDma) {
            __builtin_amdgcn_sched_barrier(0);
            if (dc >= 0) dma(dc, m / 2);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
    __builtin_amdgcn_s_setprio(0);
    pin_acc();
    if (MODE == 0) pin_sum();
  };

  // zeroes the pairs of sub-tile (a, b) that take no part: i == j on the
  // diagonal sub-tiles, or (causal) every j >= i.  Element e of this lane
  // pairs query row qb + r_e with key row kr; the empty asm keeps the compares
  // from being hoisted out of the head loop as live lane masks.
  auto exclude = [&](lemo_f32x16& v, int a, int b) {
    if (!CAUSAL) {
      if (a == b) {
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (acc_row(lane, e) == l32) v[e] = 0.f;
      }
    } else {
      int qb = qlo + a * 32 + 4 * hi;
      int kr = klo + b * 32 + l32;
      asm volatile("" : "+v"(qb), "+v"(kr));
      const int dq = kr - qb;   // j >= i at r_e <= dq
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (8 * (e >> 2) + (e & 3) <= dq) v[e] = 0.f;
    }
  };
  // folds head h, which ran with parity P
  auto fold = [&](auto P_, int h) {
    constexpr int P = decltype(P_)::value;
    pin_acc();
    if (MODE == 0) {
      pin_sum();
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          lemo_f32x16& d = P == 0 ? acc[a][b] : sum[a][b];
          const lemo_f32x16& o = P == 0 ? sum[a][b] : acc[a][b];
#pragma unroll
          for (int e = 0; e < 16; ++e) d[e] = __int_as_float(imax(__float_as_int(d[e]), __float_as_int(o[e])));
        }
      pin_sum();
      pin_acc();
    } else {
      if (mask_wave) {
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < 2; ++b) exclude(acc[a][b], a, b);
      }
      if (BLK >= 64) {
        int m = 0;
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int e = 0; e < 16; ++e) m = imax(m, __float_as_int(acc[a][b][e]));
        m = wave_imax(m);
        if (BLK == 128) {
          if (lane == 0 && h >= 0) part[wave][h] = __int_as_float(m);
        } else {
          total[0][0] += __int_as_float(m);
        }
      } else {
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            int m = 0;
#pragma unroll
            for (int e = 0; e < 16; ++e) m = imax(m, __float_as_int(acc[a][b][e]));
            total[a][b] += __int_as_float(wave_imax(m));
          }
      }
    }
  };

  // ---- prologue: chunks 0-2 in flight, chunk 0 landed
#pragma unroll
  for (int c = 0; c < 3; ++c)
#pragma unroll
    for (int i = 0; i < pp::kDma; ++i) dma(c, i);
  asm volatile("s_waitcnt vmcnt(12)\n\ts_barrier" ::: "memory");

  // Each group runs its own copy of the loop (the same barriers, the same
  // number of times), so no value is merged between the groups' paths.
  auto run = [&](auto G_) {
    constexpr int G = decltype(G_)::value;
    auto chunk = [&](int h, auto KC_, auto P_) {
      constexpr int kc = decltype(KC_)::value;
      constexpr int P = decltype(P_)::value;
      const int c = h * kCPH + kc;
      // phase 2c: group 0 multiplies chunk c, with its loads of chunk c + 2
      // (chunks 0-2 came with the prologue); group 1 reads chunk c, then
      // folds its previous head while the reads are in flight (both sets
      // start at zero, so the fold before the first head changes nothing)
      if (G == 0) {
        compute(std::integral_constant<bool, kc == 0>{}, P_, c >= 1 ? c + 2 : -1);
      } else {
        read_chunk(c);
        if (kc == 0) {
          __builtin_amdgcn_sched_barrier(0);
          fold(std::integral_constant<int, 1 - P>{}, h - 1);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_waitcnt vmcnt(6) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      // phase 2c+1: group 1 multiplies chunk c, with its loads of chunk
      // c + 3; group 0 reads chunk c+1 and folds head h after its last chunk
      if (G == 1) {
        compute(std::integral_constant<bool, kc == 0>{}, P_, c + 3);
      } else {
        if (c + 1 < C) read_chunk(c + 1);
        if (kc == kCPH - 1) {
          __builtin_amdgcn_sched_barrier(0);
          fold(P_, h);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    };
    auto head = [&](int h, auto P_) {
      chunk(h, std::integral_constant<int, 0>{}, P_);
      if (kCPH == 2) chunk(h, std::integral_constant<int, kCPH - 1>{}, P_);
    };
    if (G == 0) read_chunk(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    for (int h = 0; h < n_heads; h += 2) {
      head(h, std::integral_constant<int, 0>{});
      head(h + 1, std::integral_constant<int, 1>{});
    }
    if (G == 1) fold(std::integral_constant<int, 1>{}, n_heads - 1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the repeated loads past the last chunk
  };
  if (grp == 0)
    run(std::integral_constant<int, 0>{});
  else
    run(std::integral_constant<int, 1>{});

  // ---- per-(wave, sub-tile) block values -> fin[]; PAPER: an even head
  // count leaves the sum in the odd heads' set, sum[]
  if (MODE == 0) {
    if (mask_wave) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) exclude(sum[a][b], a, b);
    }
    if (BLK >= 64) {
      int m = 0;
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int e = 0; e < 16; ++e) m = imax(m, __float_as_int(sum[a][b][e]));
      m = wave_imax(m);
      if (lane == 0) fin[wave * 4] = __int_as_float(m);
    } else {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          int m = 0;
#pragma unroll
          for (int e = 0; e < 16; ++e) m = imax(m, __float_as_int(sum[a][b][e]));
          m = wave_imax(m);
          if (lane == 0) fin[wave * 4 + a * 2 + b] = __int_as_float(m);
        }
    }
  } else if (BLK == 64) {
    if (lane == 0) fin[wave * 4] = total[0][0];
  } else if (BLK == 32) {
    if (lane == 0) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) fin[wave * 4 + a * 2 + b] = total[a][b];
    }
  }
  __syncthreads();

  // ---- combine the parts of each block of this tile and write M
  constexpr int kBQ = pp::kTQ / BLK, kBK = pp::kTK / BLK;
  if (tid < kBQ * kBK) {
    const int lq = tid / kBK, lk = tid % kBK;
    const int bq = q0 / BLK + lq, bk = k0 / BLK + lk;
    if (bq < nb && bk < nb) {
      float val = 0.f;
      if (MODE == 1 && BLK == 128) {
        // the four waves of group lq cover this block; heads summed in order
        for (int h = 0; h < n_heads; ++h) {
          float m = 0.f;
          for (int w = 4 * lq; w < 4 * lq + 4; ++w) m = fmaxf(m, part[w][h]);
          val += m;
        }
      } else {
        // sub-tile (a, b) of wave (g, wq, wk) covers query rows
        // 128 g + 64 wq + 32 a and key rows 64 wk + 32 b of the tile
        for (int p = 0; p < pp::kWaves * 4; ++p) {
          const int w = p >> 2, a = (p >> 1) & 1, b = p & 1;
          if (BLK >= 64 && (a | b)) continue;
          const int rq = ((w >> 2) * 128 + ((w >> 1) & 1) * 64 + a * 32) / BLK;
          const int rk = ((w & 1) * 64 + b * 32) / BLK;
          if (rq == lq && rk == lk) val = fmaxf(val, fin[p]);
        }
      }
      M[(size_t)bq * nb + bk] = val * out_scale;
      // causal: the mirror block above the diagonal has no pair with j < i
      if (CAUSAL && bq > bk) M[(size_t)bk * nb + bq] = 0.f;
    }
  }
}

// One head (the per-token predictor's q_hat, k_hat of width r; full launches
// of one sequence with blocks of 32 or 64 and N a multiple of 1024 run
// k_scores_one_head_pp below): PAPER and
// HEADMAX coincide, M = max(0, block max of S), and a tile has only
// HD / 64 chunks, so a workgroup walks `per_wg` consecutive logical tiles
// with the loads of the next tile's first chunk in flight during the current
// tile's last chunk (one pipeline over (tile, chunk)).  Same 128 x 128 tile,
// waves, LDS ring, swizzle and exclusions as k_block_scores; the score tile
// is reduced straight from the accumulators.  With blocks of 32 or 64 rows
// each wave holds whole blocks and writes them itself, so there is no barrier
// between tiles beyond the ring's.
template <int HD, int BLK, int MASK>
__global__ __launch_bounds__(kThreads, 2) void k_scores_one_head(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, int n_tokens, int ldq, int ldk, long long bsq,
    long long bsk, float out_scale, float* __restrict__ M, int nb, int ntq, int ntk, int tiles_per_seq, int total,
    int per_wg) {
  constexpr bool CAUSAL = MASK == kMaskCausal;
  constexpr int kCPH = HD / kChunk;
  __shared__ float fin[kWaves];                          // 128-row blocks: per-wave maxima
  const int rank = xcd_logical(blockIdx.x, gridDim.x);
  const int t_begin = rank * per_wg, t_end = min(total, t_begin + per_wg);
  if (t_begin >= t_end) return;                          // uniform: the whole workgroup leaves

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wq = wave >> 1, wk = wave & 1;
  const int l32 = lane & 31, hi = lane >> 5;
  const uint32_t lds0 = (uint32_t)(uintptr_t)g_stage;

  // DMA: instruction i (Q: i < 4, K: i >= 4) of this wave fills row
  // 32 ii + r0 of the tile's Q or K region; every such row has the same
  // r & 15, so one swizzled piece offset serves all of them.
  const int r0 = wave * 8 + (lane >> 3);
  const uint32_t pc = (uint32_t)((((lane & 7) ^ swz(r0)) * 8) * 2);
  struct Tile { int q0, k0; size_t qoff, koff, moff; bool mirror; };
  auto tile = [&](int t) {
    const int seq = t / tiles_per_seq;
    int tq, tk;
    if (CAUSAL)
      tri_tile_of(t - seq * tiles_per_seq, ntq, tq, tk);
    else
      tile_of(t - seq * tiles_per_seq, ntq, ntk, tq, tk);
    return Tile{tq * kTQ, tk * kTK, (size_t)seq * bsq, (size_t)seq * bsk, (size_t)seq * nb * nb, CAUSAL && tq != tk};
  };
  auto issue = [&](const Tile& tl, int kc, int stage) {
    const uint16_t* qb = Q + tl.qoff + kc * kChunk;
    const uint16_t* kb = K + tl.koff + kc * kChunk;
    const uint32_t base = lds0 + (uint32_t)(stage * kStageBytes);
#pragma unroll
    for (int i = 0; i < kDmaPerChunk; ++i) {
      const bool is_q = i < kDmaQ;
      const int ii = is_q ? i : i - kDmaQ;
      const int grow = min((is_q ? tl.q0 : tl.k0) + 32 * ii + r0, n_tokens - 1);   // rows past N: any valid row
      const uint32_t voff = (uint32_t)((size_t)grow * (is_q ? ldq : ldk) * 2) + pc;
      dma16(is_q ? (const void*)qb : (const void*)kb, voff,
            base + (is_q ? 0u : (uint32_t)kStageQ) + (uint32_t)((ii * kWaves + wave) * 1024));
    }
  };
  uint32_t offA[4], offB[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int piece = (2 * s + hi) ^ swz(l32);
    offA[s] = (uint32_t)((wq * 64 + l32) * kRowBytes + piece * 16);
    offB[s] = (uint32_t)(kStageQ + (wk * 64 + l32) * kRowBytes + piece * 16);
  }
  lemo_bf16x8 fa[2][2], fb[2][2];
  auto read_frags = [&](int buf, const uint8_t* st, int s) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      fa[buf][i] = *reinterpret_cast<const lemo_bf16x8*>(st + offA[s] + i * 32 * kRowBytes);
      fb[buf][i] = *reinterpret_cast<const lemo_bf16x8*>(st + offB[s] + i * 32 * kRowBytes);
    }
  };

  Tile cur = tile(t_begin);
  issue(cur, 0, 0);
  int c = 0;                                             // chunks consumed so far: stage parity
  for (int t = t_begin; t < t_end; ++t) {
    Tile next = cur;
    if (t + 1 < t_end) next = tile(t + 1);
    lemo_f32x16 acc[2][2];
#pragma unroll
    for (int kc = 0; kc < kCPH; ++kc, ++c) {
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      if (kc + 1 < kCPH)
        issue(cur, kc + 1, (c + 1) % kStages);
      else if (t + 1 < t_end)
        issue(next, 0, (c + 1) % kStages);
      const uint8_t* st = g_stage + (c % kStages) * kStageBytes;
      read_frags(0, st, 0);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int b0 = s & 1;
        if (s + 1 < 4) read_frags(b0 ^ 1, st, s + 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < 2; ++b)
            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[b0][a], fb[b0][b],
                                                                (kc == 0 && s == 0) ? lemo_f32x16{} : acc[a][b], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // exclusions (only in waves whose square holds such a pair), then the
    // block maxima of max(0, S): an integer max from 0 on the float bits
    const int qlo = cur.q0 + wq * 64, klo = cur.k0 + wk * 64;
    const bool mask_wave = MASK == kMaskDiag
                               ? klo == qlo
                               : (CAUSAL ? klo >= qlo : klo == qlo) || qlo + 64 > n_tokens || klo + 64 > n_tokens;
    if (mask_wave) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          int qb = qlo + a * 32 + 4 * hi;
          int kr = klo + b * 32 + l32;
          asm volatile("" : "+v"(qb), "+v"(kr));
          const int dq = kr - qb;
          const int lim = kr >= n_tokens ? 0 : n_tokens - qb;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int r = 8 * (e >> 2) + (e & 3);
            const bool out = MASK == kMaskDiag ? (a == b && r == dq)
                                               : ((CAUSAL ? r <= dq : r == dq) || r >= lim);
            if (out) acc[a][b][e] = 0.f;
          }
        }
    }
    float* Mt = M + cur.moff;
    if (BLK == 32) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          int m = 0;
#pragma unroll
          for (int e = 0; e < 16; ++e) m = imax(m, __float_as_int(acc[a][b][e]));
          m = wave_imax(m);
          const int bq = (qlo + 32 * a) / 32, bk = (klo + 32 * b) / 32;
          if (lane == 0 && bq < nb && bk < nb) {
            Mt[(size_t)bq * nb + bk] = __int_as_float(m) * out_scale;
            if (cur.mirror) Mt[(size_t)bk * nb + bq] = 0.f;
          }
        }
    } else {
      int m = 0;
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int e = 0; e < 16; ++e) m = imax(m, __float_as_int(acc[a][b][e]));
      m = wave_imax(m);
      if (BLK == 64) {
        const int bq = qlo / 64, bk = klo / 64;
        if (lane == 0 && bq < nb && bk < nb) {
          Mt[(size_t)bq * nb + bk] = __int_as_float(m) * out_scale;
          if (cur.mirror) Mt[(size_t)bk * nb + bq] = 0.f;
        }
      } else {
        // 128-row blocks: the four waves' maxima meet in LDS
        if (lane == 0) fin[wave] = __int_as_float(m);
        __syncthreads();
        const int bq = cur.q0 / 128, bk = cur.k0 / 128;
        if (tid == 0 && bq < nb && bk < nb) {
          Mt[(size_t)bq * nb + bk] = fmaxf(fmaxf(fin[0], fin[1]), fmaxf(fin[2], fin[3])) * out_scale;
          if (cur.mirror) Mt[(size_t)bk * nb + bq] = 0.f;
        }
      }
    }
    cur = next;
  }
}

// Eight-wave form of the one-head scores (full launches of one sequence,
// blocks of 32 or 64 rows, N a multiple of 1024, at least 512 tiles): one
// workgroup per CU walks tiles rank,
// rank + G, rank + 2G, ... of the 256 x 128 tile order of k_block_scores_pp
// (G workgroups, XCD ranges as in a plain launch of G), with the same two
// wave groups, phases, ring and loads; the load stream runs on across tile
// boundaries.  A tile is kCPH chunks; when a group has multiplied a tile's
// last chunk, its next memory phase reduces the tile to block maxima (the
// exclusions first, on diagonal squares) and writes them: with blocks of 64
// rows or fewer each wave holds whole blocks.  Each wave keeps two cursors
// over its tiles, one for the loads and one for the output, stepped without
// division: in the tile order (groups of 4 query tiles, 4 ntk tiles each),
// adding G to a tile's index moves it G positions within its group, with a
// carry into the next group.
template <int HD, int BLK>
__global__ __launch_bounds__(pp::kThreads, 1) void k_scores_one_head_pp(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, int n_tokens, int ldq, int ldk, float out_scale,
    float* __restrict__ M, int nb, int ntk, int total) {
  constexpr int kCPH = HD / kChunk;
  static_assert(BLK == 32 || BLK == 64, "blocks within one wave's square");
  __shared__ __attribute__((aligned(1024))) uint8_t ring[pp::kStages * pp::kStageBytes];
  const int G = gridDim.x;
  const int rank = xcd_logical(blockIdx.x, G);
  const int U = (total - rank + G - 1) / G;   // this workgroup's tiles (>= 1: G <= total)
  const int C = U * kCPH;                     // its chunks
  const int span = 4 * ntk;                   // tiles per group of 4 query tiles

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int wq = (wave >> 1) & 1, wk = wave & 1;
  const int l32 = lane & 31, hi = lane >> 5;
  const uint32_t lds0 = (uint32_t)(uintptr_t)ring;

  // a cursor over this workgroup's tiles: group index and position in group
  struct Cursor {
    int unit, g, pos;
  };
  auto cursor_at0 = [&]() { return Cursor{0, rank / span, rank % span}; };
  auto advance = [&](Cursor& cu) {
    if (cu.unit + 1 >= U) return;   // stays on the last tile (the repeated loads)
    ++cu.unit;
    cu.pos += G;
    while (cu.pos >= span) {
      cu.pos -= span;
      ++cu.g;
    }
  };
  auto q0_of = [&](const Cursor& cu) { return (4 * cu.g + (cu.pos & 3)) * pp::kTQ; };
  auto k0_of = [&](const Cursor& cu) { return (cu.pos >> 2) * pp::kTK; };

  const int drow = wave * 8 + (lane >> 3);
  const uint32_t dpiece = (uint32_t)((((lane & 7) ^ swz(drow)) * 8) * 2);
  Cursor dcur = cursor_at0();   // the tile of the next chunk this wave loads
  int dkc = 0;                  // and its chunk within the tile
  // this wave's 6 loads of its next chunk (in order), into the stage chunk dc maps to
  int dnext = 0;                // the chunk number of the next load batch
  auto dma_one = [&](int i) {
    const bool is_q = i < pp::kDmaQ;
    const int ii = is_q ? i : i - pp::kDmaQ;
    const int row = (is_q ? q0_of(dcur) : k0_of(dcur)) + 64 * ii + drow;
    const uint32_t voff = (uint32_t)((size_t)row * (is_q ? ldq : ldk) * 2) + dpiece;
    const uint32_t base = lds0 + (uint32_t)((dnext % pp::kStages) * pp::kStageBytes);
    dma16(is_q ? (const void*)(Q + dkc * kChunk) : (const void*)(K + dkc * kChunk), voff,
          base + (is_q ? 0u : (uint32_t)pp::kStageQ) + (uint32_t)((ii * pp::kWaves + wave) * 1024));
  };
  auto dma_done = [&]() {   // after the 6 loads of a chunk: step the load cursor
    ++dnext;
    if (dnext < C) {
      if (++dkc == kCPH) {
        dkc = 0;
        advance(dcur);
      }
    }
  };

  uint32_t offA[4], offB[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int piece = (2 * s + hi) ^ swz(l32);
    offA[s] = (uint32_t)((grp * 128 + wq * 64 + l32) * kRowBytes + piece * 16);
    offB[s] = (uint32_t)(pp::kStageQ + (wk * 64 + l32) * kRowBytes + piece * 16);
  }
  lemo_bf16x8 fa[4][2], fb[4][2];
  auto read_chunk = [&](int c) {
    uint32_t so = (uint32_t)((c % pp::kStages) * pp::kStageBytes);
    asm volatile("" : "+s"(so));
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint8_t* pa = ring + offA[s] + so;
      const uint8_t* pb = ring + offB[s] + so;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        fa[s][i] = *reinterpret_cast<const lemo_bf16x8*>(pa + i * 32 * kRowBytes);
        fb[s][i] = *reinterpret_cast<const lemo_bf16x8*>(pb + i * 32 * kRowBytes);
      }
    }
  };

  lemo_f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;
  auto pin_acc = [&]() {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) asm volatile("" : "+v"(acc[a][b]));
  };
  // a matrix phase over the chunk in fa/fb, with this wave's loads of its next
  // chunk between the MFMAs when `loads`
  auto compute = [&](auto FIRST_, bool loads) {
    constexpr bool FIRST = decltype(FIRST_)::value;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < 2; ++i) asm volatile("" : "+v"(fa[s][i]), "+v"(fb[s][i]));
    if (!FIRST) pin_acc();
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              fa[s][a], fb[s][b], (FIRST && s == 0) ? lemo_f32x16{} : acc[a][b], 0, 0, 0);
          const int m = s * 4 + a * 2 + b;
          if ((m & 1) && m / 2 < pp::kDma) {
            __builtin_amdgcn_sched_barrier(0);
            if (loads) dma_one(m / 2);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
    __builtin_amdgcn_s_setprio(0);
    pin_acc();
    if (loads) dma_done();
  };

  // the block maxima of the tile at the output cursor, then the cursor steps
  Cursor ocur = cursor_at0();
  auto output = [&]() {
    pin_acc();
    const int qlo = q0_of(ocur) + grp * 128 + wq * 64, klo = k0_of(ocur) + wk * 64;
    if (klo == qlo) {   // the i == j pairs of the diagonal sub-tiles
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (acc_row(lane, e) == l32) acc[a][a][e] = 0.f;
    }
    if (BLK == 32) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          int m = 0;
#pragma unroll
          for (int e = 0; e < 16; ++e) m = imax(m, __float_as_int(acc[a][b][e]));
          m = wave_imax(m);
          if (lane == 0) M[(size_t)((qlo + 32 * a) / 32) * nb + (klo + 32 * b) / 32] = __int_as_float(m) * out_scale;
        }
    } else {
      int m = 0;
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int e = 0; e < 16; ++e) m = imax(m, __float_as_int(acc[a][b][e]));
      m = wave_imax(m);
      if (lane == 0) M[(size_t)(qlo / 64) * nb + klo / 64] = __int_as_float(m) * out_scale;
    }
    advance(ocur);
  };

  // prologue: chunks 0-2 in flight (C >= 3 is not required: past the last
  // chunk the loads repeat it), chunk 0 landed
#pragma unroll
  for (int c = 0; c < 3; ++c) {
#pragma unroll
    for (int i = 0; i < pp::kDma; ++i) dma_one(i);
    dma_done();
  }
  asm volatile("s_waitcnt vmcnt(12)\n\ts_barrier" ::: "memory");

  auto run = [&](auto G_) {
    constexpr int G2 = decltype(G_)::value;
    auto chunk = [&](int c, auto KC_) {
      constexpr int kc = decltype(KC_)::value;
      // phase 2c: group 0 multiplies chunk c (with its loads of chunk c + 2
      // from c = 1 on); group 1 reads chunk c, then outputs its last tile
      if (G2 == 0) {
        compute(std::integral_constant<bool, kc == 0>{}, c >= 1);
      } else {
        read_chunk(c);
        if (kc == 0 && c > 0) {
          __builtin_amdgcn_sched_barrier(0);
          output();
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_waitcnt vmcnt(6) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      // phase 2c+1: group 1 multiplies chunk c (with its loads of chunk
      // c + 3); group 0 reads chunk c+1, then outputs the tile chunk c ends
      if (G2 == 1) {
        compute(std::integral_constant<bool, kc == 0>{}, true);
      } else {
        if (c + 1 < C) read_chunk(c + 1);
        if (kc == kCPH - 1) {
          __builtin_amdgcn_sched_barrier(0);
          output();
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    };
    if (G2 == 0) read_chunk(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    for (int c = 0; c < C; c += kCPH) {
      chunk(c, std::integral_constant<int, 0>{});
      if (kCPH == 2) chunk(c + 1, std::integral_constant<int, kCPH - 1>{});
    }
    if (G2 == 1) output();
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };
  if (grp == 0)
    run(std::integral_constant<int, 0>{});
  else
    run(std::integral_constant<int, 1>{});
}

// Column sums I[c] = sum_r M[r][c].  A workgroup owns 16 columns; its 256
// threads split the rows into 16 interleaved slices (thread (slice, column)
// adds rows slice, slice+16, ... in order), then one thread per column adds
// the 16 slice sums in slice order.  Fixed order, so the result is
// deterministic.
__global__ __launch_bounds__(256) void k_colsum(const float* __restrict__ M, int nb, float* __restrict__ out) {
  __shared__ float partial[16][17];
  M += (size_t)blockIdx.y * nb * nb;   // sequence blockIdx.y of a batch
  out += (size_t)blockIdx.y * nb;
  const int col = blockIdx.x * 16 + (threadIdx.x & 15);
  const int slice = threadIdx.x >> 4;
  float s = 0.f;
  if (col < nb) {
#pragma unroll 4
    for (int r = slice; r < nb; r += 16) s += M[(size_t)r * nb + col];
  }
  partial[slice][threadIdx.x & 15] = s;
  __syncthreads();
  if (threadIdx.x < 16 && blockIdx.x * 16 + threadIdx.x < nb) {
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) t += partial[i][threadIdx.x];
    out[blockIdx.x * 16 + threadIdx.x] = t;
  }
}

template <int HD, int MODE, int MASK>
hipError_t launch_variant(const uint16_t* q, const uint16_t* k, int n_batch, int n, int h, int ldq, int ldk,
                          long long bsq, long long bsk, int block, float scale, float* m, int nb, hipStream_t st) {
  const int ntq = (n + kTQ - 1) / kTQ, ntk = (n + kTK - 1) / kTK;
  const dim3 grid(MASK == kMaskCausal ? ntq * (ntq + 1) / 2 : ntq * ntk, n_batch), blk(kThreads);
  switch (block) {
    case 32:
      hipLaunchKernelGGL((k_block_scores<HD, MODE, 32, MASK>), grid, blk, 0, st, q, k, n, h, ldq, ldk, bsq, bsk,
                         scale, m, nb, ntq, ntk);
      break;
    case 64:
      hipLaunchKernelGGL((k_block_scores<HD, MODE, 64, MASK>), grid, blk, 0, st, q, k, n, h, ldq, ldk, bsq, bsk,
                         scale, m, nb, ntq, ntk);
      break;
    default:
      hipLaunchKernelGGL((k_block_scores<HD, MODE, 128, MASK>), grid, blk, 0, st, q, k, n, h, ldq, ldk, bsq, bsk,
                         scale, m, nb, ntq, ntk);
      break;
  }
  return hipGetLastError();
}

template <int HD, int MASK>
hipError_t launch_one_head(const uint16_t* q, const uint16_t* k, int n_batch, int n, int ldq, int ldk, long long bsq,
                           long long bsk, int block, float scale, float* m, int nb, hipStream_t st) {
  const int ntq = (n + kTQ - 1) / kTQ, ntk = (n + kTK - 1) / kTK;
  const int per_seq = MASK == kMaskCausal ? ntq * (ntq + 1) / 2 : ntq * ntk;
  const int total = per_seq * n_batch;
  // about 16 chunks per workgroup, but at least 1024 workgroups (4 per CU)
  // while the tiles allow
  const int want = (16 + HD / kChunk - 1) / (HD / kChunk);
  // and at most 2^23 workgroups (a launch's x dimension holds 2^31 - 1 work-items)
  const int per_wg = max(max(1, min(want, total / 1024)), (int)((total + (1LL << 23) - 1) >> 23));
  const dim3 grid((total + per_wg - 1) / per_wg), blk(kThreads);
  switch (block) {
    case 32:
      hipLaunchKernelGGL((k_scores_one_head<HD, 32, MASK>), grid, blk, 0, st, q, k, n, ldq, ldk, bsq, bsk, scale, m, nb,
                         ntq, ntk, per_seq, total, per_wg);
      break;
    case 64:
      hipLaunchKernelGGL((k_scores_one_head<HD, 64, MASK>), grid, blk, 0, st, q, k, n, ldq, ldk, bsq, bsk, scale, m, nb,
                         ntq, ntk, per_seq, total, per_wg);
      break;
    default:
      hipLaunchKernelGGL((k_scores_one_head<HD, 128, MASK>), grid, blk, 0, st, q, k, n, ldq, ldk, bsq, bsk, scale, m,
                         nb, ntq, ntk, per_seq, total, per_wg);
      break;
  }
  return hipGetLastError();
}

template <int HD>
hipError_t launch_one_head_mask(const uint16_t* q, const uint16_t* k, int n_batch, int n, int ldq, int ldk,
                                long long bsq, long long bsk, int block, bool causal, float scale, float* m, int nb,
                                hipStream_t st) {
  // the eight-wave form: one sequence, no mask, blocks of 32 or 64 rows, N a
  // multiple of 1024 (groups of 4 whole query tiles), at least 512 tiles
  const long long tiles = (long long)(n / pp::kTQ) * (n / pp::kTK);
  if (!causal && n_batch == 1 && n % 1024 == 0 && (block == 32 || block == 64) && tiles >= 512 &&
      tiles <= 0x7fffffffLL) {
    const int ntk = n / pp::kTK, grid = 256;
    if (block == 32)
      hipLaunchKernelGGL((k_scores_one_head_pp<HD, 32>), dim3(grid), dim3(pp::kThreads), 0, st, q, k, n, ldq, ldk,
                         scale, m, nb, ntk, (int)tiles);
    else
      hipLaunchKernelGGL((k_scores_one_head_pp<HD, 64>), dim3(grid), dim3(pp::kThreads), 0, st, q, k, n, ldq, ldk,
                         scale, m, nb, ntk, (int)tiles);
    return hipGetLastError();
  }
  if (causal) return launch_one_head<HD, kMaskCausal>(q, k, n_batch, n, ldq, ldk, bsq, bsk, block, scale, m, nb, st);
  if (n % block) return launch_one_head<HD, kMaskRagged>(q, k, n_batch, n, ldq, ldk, bsq, bsk, block, scale, m, nb, st);
  return launch_one_head<HD, kMaskDiag>(q, k, n_batch, n, ldq, ldk, bsq, bsk, block, scale, m, nb, st);
}

template <int HD, int MODE, bool CAUSAL>
hipError_t launch_pp(const uint16_t* q, const uint16_t* k, int n_batch, int n, int h, int ldq, int ldk, long long bsq,
                     long long bsk, int block, float scale, float* m, int nb, hipStream_t st) {
  const int ntq = (n + pp::kTQ - 1) / pp::kTQ, ntk = (n + pp::kTK - 1) / pp::kTK;
  const dim3 grid(CAUSAL ? ntq * (ntq + 1) : ntq * ntk, n_batch), blk(pp::kThreads);
  switch (block) {
    case 32:
      hipLaunchKernelGGL((k_block_scores_pp<HD, MODE, 32, CAUSAL>), grid, blk, 0, st, q, k, n, h, ldq, ldk, bsq, bsk,
                         scale, m, nb, ntq, ntk);
      break;
    case 64:
      hipLaunchKernelGGL((k_block_scores_pp<HD, MODE, 64, CAUSAL>), grid, blk, 0, st, q, k, n, h, ldq, ldk, bsq, bsk,
                         scale, m, nb, ntq, ntk);
      break;
    default:
      hipLaunchKernelGGL((k_block_scores_pp<HD, MODE, 128, CAUSAL>), grid, blk, 0, st, q, k, n, h, ldq, ldk, bsq, bsk,
                         scale, m, nb, ntq, ntk);
      break;
  }
  return hipGetLastError();
}

// The eight-wave kernel takes launches without a ragged last block, with an
// even head count, at least 16 chunks per tile (below that its per-tile
// start weighs more than it saves) and at least 512 of its tiles (two per
// CU; smaller launches leave CUs idle with one workgroup per CU); causal
// launches also need N to be a multiple of its 256-row tile.
bool use_pp(int n_batch, int n, int h, int hd, bool causal) {
  const long long ntq = (n + pp::kTQ - 1) / pp::kTQ, ntk = (n + pp::kTK - 1) / pp::kTK;
  const long long tiles = causal ? ntq * (ntq + 1) : ntq * ntk;
  return h % 2 == 0 && (long long)h * (hd / kChunk) >= 16 && tiles * n_batch >= 512 &&
         tiles * pp::kThreads <= 0x7fffffffLL && (!causal || n % pp::kTQ == 0);
}

template <int HD, int MODE>
hipError_t launch_hd_mode(const uint16_t* q, const uint16_t* k, int n_batch, int n, int h, int ldq, int ldk,
                          long long bsq, long long bsk, int block, bool causal, float scale, float* m, int nb,
                          hipStream_t st) {
  if (causal) {
    if (use_pp(n_batch, n, h, HD, true))
      return launch_pp<HD, MODE, true>(q, k, n_batch, n, h, ldq, ldk, bsq, bsk, block, scale, m, nb, st);
    return launch_variant<HD, MODE, kMaskCausal>(q, k, n_batch, n, h, ldq, ldk, bsq, bsk, block, scale, m, nb, st);
  }
  if (n % block)
    return launch_variant<HD, MODE, kMaskRagged>(q, k, n_batch, n, h, ldq, ldk, bsq, bsk, block, scale, m, nb, st);
  if (use_pp(n_batch, n, h, HD, false))
    return launch_pp<HD, MODE, false>(q, k, n_batch, n, h, ldq, ldk, bsq, bsk, block, scale, m, nb, st);
  return launch_variant<HD, MODE, kMaskDiag>(q, k, n_batch, n, h, ldq, ldk, bsq, bsk, block, scale, m, nb, st);
}

}  // namespace

hipError_t lemo_launch_colsum(const float* m, int nb, float* out, hipStream_t stream, int n_batch) {
  hipLaunchKernelGGL(k_colsum, dim3((nb + 15) / 16, n_batch), dim3(256), 0, stream, m, nb, out);
  return hipGetLastError();
}

hipError_t lemo_launch_block_scores(const uint16_t* q, const uint16_t* k, int n_batch, int n_tokens, int n_heads,
                                    int head_dim, int ld_q, int ld_k, long long bs_q, long long bs_k, int block,
                                    int head_reduce, bool causal, float* m_out, float* scores, hipStream_t stream) {
  const int nb = (n_tokens + block - 1) / block;
  const double c = 1.0 / __builtin_sqrt((double)head_dim);
  const float scale = (float)(head_reduce == 0 ? c / n_heads : c);
  hipError_t e;
  if (n_heads == 1)   // both head reductions give max(0, block max of S)
    e = head_dim == 64 ? launch_one_head_mask<64>(q, k, n_batch, n_tokens, ld_q, ld_k, bs_q, bs_k, block, causal,
                                                  scale, m_out, nb, stream)
                       : launch_one_head_mask<128>(q, k, n_batch, n_tokens, ld_q, ld_k, bs_q, bs_k, block, causal,
                                                   scale, m_out, nb, stream);
  else if (head_dim == 64)
    e = head_reduce == 0 ? launch_hd_mode<64, 0>(q, k, n_batch, n_tokens, n_heads, ld_q, ld_k, bs_q, bs_k, block,
                                                 causal, scale, m_out, nb, stream)
                         : launch_hd_mode<64, 1>(q, k, n_batch, n_tokens, n_heads, ld_q, ld_k, bs_q, bs_k, block,
                                                 causal, scale, m_out, nb, stream);
  else
    e = head_reduce == 0 ? launch_hd_mode<128, 0>(q, k, n_batch, n_tokens, n_heads, ld_q, ld_k, bs_q, bs_k, block,
                                                  causal, scale, m_out, nb, stream)
                         : launch_hd_mode<128, 1>(q, k, n_batch, n_tokens, n_heads, ld_q, ld_k, bs_q, bs_k, block,
                                                  causal, scale, m_out, nb, stream);
  if (e != hipSuccess) return e;
  return lemo_launch_colsum(m_out, nb, scores, stream, n_batch);
}
