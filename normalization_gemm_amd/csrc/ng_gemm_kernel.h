// bf16 MFMA GEMM with fused row-norm epilogues for gfx950.
//
// One kernel template serves four epilogues:
//   EPI_NONE      C = A @ B                               (unfused baseline GEMM)
//   EPI_LAZY      C = (A @ B) * rstd(A)                   (Lazy Pre-Norm)
//   EPI_LAZY_BIAS C = (A @ B') * rstd(A) + bias            (Lazy Pre-Norm with the
//                 affine folded into the weights: B' = diag(gamma) B, bias = beta^T B)
//   EPI_ROW_RMS / EPI_ROW_LN
//                 C = norm(A @ B), whole row in one workgroup (N <= BN)
//   EPI_ROW_RMS_RES / EPI_ROW_LN_RES
//                 C = norm(A @ B + R), S_out = A @ B + R (optional): a
//                 residual connection followed by a post-norm
//   EPI_PRE_LN    C = rstd(A) * (A @ B' - mean(A) * colsum) + bias: LayerNorm
//                 of A's rows before the product, carried through it (B' =
//                 diag(gamma) B, colsum = 1^T B', bias = beta^T B; row
//                 statistics from a pre-pass)
//   EPI_LAZY_BWD  input gradient of Lazy Pre-Norm, the norm's backward in the
//                 epilogue of dA_hat = dC @ B^T: C = rstd * acc - c * X with
//                 c = rstd^3 * sum_n(acc * X) / N per row (X the forward A,
//                 rstd saved by the forward pass)
//   cross-workgroup: C = norm(A @ B [+ R]) for rows split over workgroups;
//                 per-row fp32 partials merged through a workspace
//                 (persistent grid, gemm_xwg_kernel below)
//
// Lazy Pre-Norm ("Free normalization fusion", section "Lazy Pre-Norm"): a
// per-row scale commutes with the product, so the sum of squares of each row
// of A accumulates from the A fragments already read for the MFMAs and the
// scale rstd is applied to the fp32 accumulators after the k-loop.
//
// Epilogue norms ("Free normalization fusion", section "Multi-CTA Norm
// Fusion"): a row norm is a per-row reduction followed by an elementwise
// apply, and only the reduction needs the whole row.  Each workgroup reduces
// its slice of the row from its fp32 accumulators; when several workgroups
// share a row they exchange one (mean, M2) pair (or one sum of squares) per
// row and each applies the norm to its own slice.  Norm formulas: "RMSNorm
// fusion on Ascend", sections 1.1 (LayerNorm) and 1.2 (RMSNorm).
//
// Data layout in LDS per pipeline stage (k-tile depth BK = 64, or 32):
//   A tile  [BM][BK] bf16, rows of 2*BK bytes; 16-byte chunk c of row m is
//           stored at chunk c ^ (m & 7) for BK = 64, c ^ ((m >> 1) & 3) for
//           BK = 32 (conflict-free 16-byte fragment reads of 16 rows).
//   B tile  KN: blocked [BK/4][BN/16][4][16] bf16 (128-byte blocks of 4 k-rows
//           x 16 columns), read with the transposing LDS read: each 16-lane
//           group reads one whole block.
//           NK: [BN][BK] bf16, same layout as A.
// MFMA: v_mfma_f32_16x16x32_bf16 with B as the first operand and A as the
// second, so each lane's accumulators hold four consecutive columns of one
// output row: acc[i][j][r] = C[m0 + 16i + (lane & 15)][n0 + 16j + 4(lane >> 4) + r].
#pragma once

#include "ng_device.h"

namespace ng {


enum Epi {
  EPI_NONE = 0,
  EPI_LAZY = 1,
  EPI_ROW_RMS = 2,
  EPI_ROW_LN = 3,
  EPI_LAZY_BIAS = 4,
  EPI_ROW_RMS_RES = 5,
  EPI_ROW_LN_RES = 6,
  EPI_PRE_LN = 7,
  EPI_LAZY_BWD = 8
};
constexpr bool epi_lazy(int e) { return e == EPI_LAZY || e == EPI_LAZY_BIAS; }
constexpr bool epi_row(int e) {
  return e == EPI_ROW_RMS || e == EPI_ROW_LN || e == EPI_ROW_RMS_RES || e == EPI_ROW_LN_RES;
}
constexpr bool epi_ln(int e) { return e == EPI_ROW_LN || e == EPI_ROW_LN_RES; }
constexpr bool epi_res(int e) { return e == EPI_ROW_RMS_RES || e == EPI_ROW_LN_RES; }
enum NormKind { NORM_RMS = 0, NORM_LAYER = 1 };

// Workspace layout of the cross-workgroup row norm (byte offsets).  A round
// of the persistent grid covers R row blocks, one per "slot"; the entries of
// a round go to its slots and the next round reuses them (safe: a workgroup
// writes its next round's entries only after it has read every final of
// this round's row block, which the other workgroups of the block publish
// only after reading all of its partials).
//   [0]        int error word (0 = ok, 1 = a wait timed out)
//   [4]        uint tag base: round `it` of a call tags its entries base +
//              1 + it; the last workgroup of a call to finish stores base +
//              rounds back
//   [8]        uint number of workgroups of the running call that finished
//   [256]      partial[slots][BM][tiles_n], 16 bytes per (row, column
//              tile): {mean_t, tag, M2_t, tag} (LayerNorm) or
//              {0, tag, sum x^2, tag} (RMSNorm)
//   [fin_off]  final[slots][BM], 16 bytes per row: {mean, tag, rstd, tag}
// Each 8-byte half of an entry carries the tag of the round that wrote it,
// and 8-byte accesses are single transactions, so a reader that finds its own
// round's tag in both halves holds the whole entry.  Entries of earlier
// rounds and calls never match, so nothing needs resetting between rounds or
// calls.  The host sizes the workspace for min(tiles_m, kXwgMaxResident /
// tiles_n) slots, at least as many as any launch uses.
constexpr int kXwgMaxResident = 1024;
struct XwgLayout {
  static constexpr size_t kErr = 0;
  static constexpr size_t kTag = 4;
  static constexpr size_t kDone = 8;
  static constexpr size_t kPart = 256;
  static __host__ __device__ size_t fin_off(int slots, int parts, int bm) {
    return kPart + (size_t)slots * bm * parts * 16u;
  }
  static __host__ __device__ size_t bytes(int slots, int parts, int bm) {
    return fin_off(slots, parts, bm) + (size_t)slots * bm * 16u;
  }
};

struct GemmParams {
  const uint16_t* A;
  const uint16_t* B;
  uint16_t* C;
  const uint16_t* gamma;
  const uint16_t* beta;
  const float* bias;  // EPI_LAZY_BIAS: fp32 [N]
  const uint16_t* R;  // residual epilogues: bf16 [M][N] added before the norm
  uint16_t* S_out;    // residual epilogues: optional bf16 [M][N] output A @ B + R
  const float* colsum;    // EPI_PRE_LN: fp32 [N] column sums of the folded weights
  const float* row_mean;  // EPI_PRE_LN: fp32 [M] mean of each row of A
  const float* row_rstd;  // EPI_PRE_LN: fp32 [M] rstd of each row of A; EPI_LAZY_BWD: saved rstd
  const uint16_t* Xin;    // EPI_LAZY_BWD: the forward input A, bf16 [M][N]
  uint16_t* scaled_out;   // EPI_LAZY_BWD, optional: bf16 [M][K] rstd * (this product's A)
  float* mean_out;
  float* rstd_out;
  char* ws;
  int M, N, K;
  float eps;
  int norm_kind;
  int tiles_m, tiles_n;
  int iters;       // persistent grid: tile rounds
  int spin_limit;  // persistent grid: bounded wait (iterations of ~1 us)
  // Order in which the grid walks its tiles: tile t is taken as
  // (order_a * t + order_c) mod total, a bijection since order_a is coprime
  // to total.  (1, 0) is the natural order; other values exist to check that
  // results do not depend on which workgroup reaches a tile first.
  int order_a, order_c;
};

// Tile index t of a walk over `total` tiles in the launch's tile order.
__device__ __forceinline__ int ordered_tile(const GemmParams& p, int t, int total) {
  if (p.order_a == 1 && p.order_c == 0) return t;
  return (int)(((uint64_t)(uint32_t)p.order_a * (uint64_t)(uint32_t)t + (uint32_t)p.order_c) %
               (uint64_t)(uint32_t)total);
}

// KN: B stored [K, N] (else [N, K]).  AKM: A stored [K, M] (the reduction
// index is A's storage row: the weight-gradient products), read like B[K, N].
// RS: one operand is scaled per reduction index by row_rstd and rounded to
// bf16 before the MFMAs (the normalized A of Lazy Pre-Norm rebuilt from A
// and its saved rstd): 1 = the A k-tile, 2 = the B k-tile, in LDS one k-tile
// ahead of its use (32-deep k-tiles in 4 stages; both operands stored with
// the reduction index as their row).
// BK: k-tile depth (64, or 32 for deeper pipelines within the LDS budget).
// ANT: A is fetched with nontemporal loads (tiles whose workgroup is the only
// reader of its rows of A: one column tile per row block).
template <int BM_, int BN_, int WM_, int WN_, bool KN_, int STAGES_ = 2, bool AKM_ = false,
          int RS_ = 0, int BK_ = 64, bool ANT_ = false>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, STAGES = STAGES_;
  static constexpr bool ANT = ANT_;
  static constexpr bool KN = KN_;
  static constexpr bool AKM = AKM_;
  static constexpr int RS = RS_;
  static constexpr int BK = BK_;
  static constexpr int KK = BK / 32;   // k32 sub-steps per k-tile
  static constexpr int CPR = BK / 8;   // 16-byte chunks per row of A (and B[N,K])
  static constexpr int RB = BK * 2;    // bytes per row of A (and B[N,K])
  static constexpr int NT = 64 * WM * WN;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / 16, FN = WTN / 16;
  static constexpr int A_BYTES = BM * BK * 2;
  static constexpr int B_BYTES = BN * BK * 2;
  // RS: the k-tile's scales, in a 1 KB slot after B
  static constexpr int R_BYTES = RS ? 1024 : 0;
  static constexpr int STAGE = A_BYTES + B_BYTES + R_BYTES;
  static constexpr int A_PER = BM * BK / 8 / NT;  // 16-byte chunks per thread
  static constexpr int B_PER = BN * BK / 8 / NT;
  static constexpr int RED_BYTES = WN * BM * 4;   // cross-wave row partials
  static constexpr int FIN_BYTES = BM * 16;       // per-row (mean, rstd, tile mean)
  static constexpr int RED_OFF = STAGES * STAGE;      // LDS byte offsets
  static constexpr int FIN_OFF = RED_OFF + RED_BYTES;
  // Output staging: 2 KB per wave (16 rows x 128 bytes).  In a region of its
  // own when it fits (the next tile's transfers may then be in flight while
  // the tile is stored), else on top of stage 0, which is free after the k-loop.
  static constexpr int STG_BYTES = (NT / 64) * 2048;
  static constexpr bool STG_OWN = FIN_OFF + FIN_BYTES + STG_BYTES <= 160 * 1024;
  static constexpr int STG_OFF = STG_OWN ? FIN_OFF + FIN_BYTES : 0;
  static constexpr int LDS = STG_OWN ? STG_OFF + STG_BYTES : FIN_OFF + FIN_BYTES;
  // 16-byte output stores per thread per tile
  static constexpr int C_STORES = FM * (FN / 4) * 2;
  static_assert(STG_OWN || STG_BYTES <= STAGE, "output staging");
  static_assert(FN % 4 == 0, "64-column output groups");
  static_assert(STAGES >= 2 && STAGES <= 4, "pipeline depth");
  static_assert(BK == 64 || BK == 32, "k-tile depth");
  static_assert(RS == 0 || (BK == 32 && STAGES == 4), "scaled operands: 32-deep k-tiles in 4 stages");
  static_assert(BM % (16 * WM) == 0 && BN % (16 * WN) == 0, "wave tile");
  static_assert((BM * BK / 8) % NT == 0 && (BN * BK / 8) % NT == 0, "loader split");
  static_assert((BN & (BN - 1)) == 0 && BN >= 16, "BN power of two");
  static_assert(!AKM || ((BM & (BM - 1)) == 0 && BM >= 16), "BM power of two");
  static_assert(RS >= 0 && RS <= 2, "scale side");
  static_assert(RS == 0 || (RS == 1 ? AKM : KN), "scaled operand: a blocked [K, X] tile");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

// Byte offset of element (k, n) of the B (KN) tile in its blocked layout:
// 128-byte blocks of 4 k-rows x 16 columns, block rows of BN/16 blocks.  The
// column-block index is XORed with bit 3 of k so that the blocks that the
// four 16-lane groups of one transposing read touch (k/8 = g) alternate
// between the two 128-byte halves of the 64-bank LDS (measured: 1.5x faster
// than the plain blocked layout).
template <int BN>
__host__ __device__ constexpr uint32_t b_blk_off(int k, int n) {
  return (uint32_t)((((k >> 2) * (BN / 16) + ((n >> 4) ^ ((k >> 3) & 1))) << 7) +
                    ((k & 3) << 5) + ((n & 15) << 1));
}

// Chunk swizzle of the A (and B[N,K]) rows: position of chunk c of row r is
// c ^ a_swz(r).  For 64-byte rows (BK = 32) the XOR takes bits 1-2 of the
// row: measured on gfx950 (SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE on the
// 256x256 tile) 2 % conflict cycles, against 25 % with bits 2-3.
template <class T>
__host__ __device__ constexpr int a_swz(int r) {
  return T::CPR == 8 ? (r & 7) : ((r >> 1) & 3);
}

// Global -> LDS staging.  Each wave moves 1 KB per buffer_load ... lds
// instruction (16 bytes per lane, landing at consecutive LDS addresses); the
// swizzle is applied on the global side by choosing which 16-byte chunk each
// lane fetches.  Chunks outside the matrices read as zero: rows past the end
// fall outside the buffer resource, and chunks past K (A, B[N,K]) or past N
// (B[K,N]) get an out-of-range offset.
template <class T>
struct DmaPlan {
  static constexpr int A_INS = T::A_BYTES / 1024 / (T::NT / 64);  // instructions per wave
  static constexpr int B_INS = T::B_BYTES / 1024 / (T::NT / 64);
  // RS: one more transfer, the k-tile's scales, issued by wave 0 only (the
  // other waves read them after the barrier that follows every wave's wait
  // for the k-tile); INS counts wave 0's transfers.
  static constexpr int R_INS = T::RS ? 1 : 0;
  static constexpr int INS = A_INS + B_INS + R_INS;
  static_assert(A_INS * 1024 * (T::NT / 64) == T::A_BYTES, "A tile split");
  static_assert(B_INS * 1024 * (T::NT / 64) == T::B_BYTES, "B tile split");
  static_assert(INS < 32, "vmcnt budget");
  int wave;
  uint32_t a_voff;          // A (and B[N,K]): lane part of the offset, row 0 of the wave
  uint32_t a_kc;            // k offset (elements) of this lane's chunk within the k-tile
  uint32_t b_voff[B_INS];   // B[K,N]: lane part per instruction (N tail folded in)
  uint32_t a_km[T::AKM ? A_INS : 1];  // A[K,M]: lane part per instruction (M tail folded in)
  uint32_t r_voff;          // RS: this lane's 16 bytes of the scales (lanes 0 .. BK/4-1)
  uint32_t a_row_bytes;     // K * 2
  // Bytes of the tile's rows from the start of their k-tile 0 (A, and B
  // stored [N, K]: at most 256 rows of 2K bytes, at most 2^31 under the
  // K limit); B stored [K, N]: bytes of a whole k-tile and of the last one
  // from its first column, each at most 0x7FFFFFF0.  A k-tile's buffer size
  // follows from these with 32-bit scalar arithmetic.
  uint32_t a_tile_bytes, b_tile_bytes, b_kt_bytes, b_last_bytes;

  // Blocked-layout slot (16 bytes) -> (k row, column) of a [K, X] tile of
  // width W (B[K,N], or A[K,M]).
  template <int W>
  static __device__ __forceinline__ void blk_slot(int slot, int& kr, int& xc) {
    const int blk = slot >> 3, in = slot & 7;
    kr = 4 * (blk / (W / 16)) + (in >> 1);
    xc = 16 * ((blk % (W / 16)) ^ ((kr >> 3) & 1)) + 8 * (in & 1);
  }

  __device__ __forceinline__ void init(const GemmParams& p, int m_base, int n_base, int lane,
                                       int wave_) {
    wave = wave_;
    a_row_bytes = (uint32_t)p.K * 2u;
    // one transfer moves 64/CPR whole rows; lane: row lane / CPR, position
    // lane % CPR, which holds chunk position ^ swizzle(row)
    const int row_in = lane / T::CPR, pos = lane % T::CPR;
    const uint32_t c = (uint32_t)(pos ^ a_swz<T>(row_in));
    a_kc = 8u * c;
    a_voff = (uint32_t)row_in * a_row_bytes + 16u * c;
    r_voff = lane < T::BK / 4 ? 16u * (uint32_t)lane : kOOB;
    if constexpr (!T::AKM) a_tile_bytes = (uint32_t)min(p.M - m_base, T::BM) * a_row_bytes;
    if constexpr (T::KN && !T::AKM) {
      const int nk = (p.K + T::BK - 1) / T::BK;
      const int last_rows = p.K - (nk - 1) * T::BK;
      const uint64_t full = ((uint64_t)T::BK * p.N - n_base) * 2u;
      const uint64_t last = ((uint64_t)last_rows * p.N - n_base) * 2u;
      b_kt_bytes = full > 0x7FFFFFF0ull ? 0x7FFFFFF0u : (uint32_t)full;
      b_last_bytes = last > 0x7FFFFFF0ull ? 0x7FFFFFF0u : (uint32_t)last;
    } else if constexpr (!T::KN) {
      b_tile_bytes = (uint32_t)min(p.N - n_base, T::BN) * a_row_bytes;
    }
    if constexpr (T::AKM) {
#pragma unroll
      for (int j = 0; j < A_INS; ++j) {
        int kr, mc;
        blk_slot<T::BM>((wave * A_INS + j) * 64 + lane, kr, mc);
        const bool ok = m_base + mc < p.M;
        a_km[j] = ok ? (uint32_t)kr * (uint32_t)p.M * 2u + 2u * (uint32_t)mc : kOOB;
      }
    }
    if constexpr (T::KN) {
      // LDS slot (16 bytes) -> (k, n) of the blocked layout -> global offset
#pragma unroll
      for (int j = 0; j < B_INS; ++j) {
        int kr, nc;
        blk_slot<T::BN>((wave * B_INS + j) * 64 + lane, kr, nc);  // 16-byte slot in the B stage
        const bool ok = n_base + nc < p.N;
        b_voff[j] = ok ? (uint32_t)kr * (uint32_t)p.N * 2u + 2u * (uint32_t)nc : kOOB;
      }
    }
  }

  // Transfer j of k-tile kt of A into the A region at LDS byte address `st`.
  __device__ __forceinline__ void issue_a(const GemmParams& p, int m_base, int kt, uint32_t st,
                                          int j) const {
    const int k0 = kt * T::BK;
    if constexpr (T::AKM) {
      const uint64_t off = (uint64_t)k0 * p.M + m_base;
      const __amdgpu_buffer_rsrc_t rs =
          make_rsrc(p.A + off, ((uint64_t)p.K * p.M - off) * 2u);
      dma16(rs, st + (uint32_t)(wave * A_INS + j) * 1024u, a_km[j], 0u);
      return;
    }
    const uint64_t off = (uint64_t)m_base * p.K + k0;
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc_n(p.A + off, umin32(uniform(a_tile_bytes) - 2u * (uint32_t)k0, 0x7FFFFFF0u));
    const uint32_t v = (k0 + (int)a_kc < p.K) ? a_voff : kOOB;
    const uint32_t row0 = (uint32_t)((wave * A_INS + j) * (64 / T::CPR));
    dma16<T::ANT>(rs, st + (uint32_t)(wave * A_INS + j) * 1024u, v, row0 * a_row_bytes);
  }
  // Transfer j of k-tile kt of B into the B region at LDS byte address `st`.
  __device__ __forceinline__ void issue_b(const GemmParams& p, int n_base, int kt, uint32_t st,
                                          int j) const {
    const int k0 = kt * T::BK;
    if constexpr (T::KN) {
      const uint64_t off = (uint64_t)k0 * p.N + n_base;
      // (the weight-gradient tiles, short of scalar registers, size it the
      // long way from the kernel arguments)
      const __amdgpu_buffer_rsrc_t rs =
          T::AKM ? make_rsrc(p.B + off, ((uint64_t)p.K * p.N - off) * 2u)
                 : make_rsrc_n(p.B + off,
                               uniform(k0 + T::BK <= p.K ? b_kt_bytes : b_last_bytes));
      dma16(rs, st + (uint32_t)(wave * B_INS + j) * 1024u, b_voff[j], 0u);
    } else {
      const uint64_t off = (uint64_t)n_base * p.K + k0;
      const __amdgpu_buffer_rsrc_t rs =
          make_rsrc_n(p.B + off, umin32(uniform(b_tile_bytes) - 2u * (uint32_t)k0, 0x7FFFFFF0u));
      const uint32_t v = (k0 + (int)a_kc < p.K) ? a_voff : kOOB;
      const uint32_t row0 = (uint32_t)((wave * B_INS + j) * (64 / T::CPR));
      dma16(rs, st + (uint32_t)(wave * B_INS + j) * 1024u, v, row0 * a_row_bytes);
    }
  }
  // RS: the k-tile's BK scales (16 bytes per lane; the other lanes write
  // zeros into the rest of the 1 KB slot).
  __device__ __forceinline__ void issue_r(const GemmParams& p, int kt, uint32_t st) const {
    const int k0 = kt * T::BK;
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(p.row_rstd + k0, k0 < p.K ? (uint64_t)(p.K - k0) * 4u : 0u);
    dma16(rs, st, r_voff, 0u);
  }
  // Transfer number d (0 .. INS-1) of k-tile kt into the stage at `st` (A
  // region first, then B, then, from wave 0, the scales).
  __device__ __forceinline__ void issue(const GemmParams& p, int m_base, int n_base, int kt,
                                        uint32_t st, int d) const {
    if (d < A_INS) issue_a(p, m_base, kt, st, d);
    else if (d < A_INS + B_INS) issue_b(p, n_base, kt, st + T::A_BYTES, d - A_INS);
    else if (wave == 0) issue_r(p, kt, st + T::A_BYTES + T::B_BYTES);
  }
};

template <class T>
struct Frags {
  u32x4 a[T::FM];
  u32x4 b[T::FN];
};

// LDS reads of one k32 sub-step's fragments, split into items so that they
// can be spread between MFMAs: items 0..FM-1 read A fragments; the rest read
// B fragments (two transposing 8-byte reads each for B[K,N], one 16-byte read
// for B[N,K]).  Per lane only a base address per sub-step is computed; the
// fragment index enters as a compile-time offset.
//
// With a_xor = 1 the A fragment slots are permuted (slot i holds fragment
// i ^ 1), so that two waves sharing rows hold different fragments in the
// same slots; the Lazy Pre-Norm squares use this to split their work.
template <class T>
struct FragReader {
  static constexpr int A_ITEMS = T::AKM ? 2 * T::FM : T::FM;
  static constexpr int B_ITEMS = T::KN ? 2 * T::FN : T::FN;
  static constexpr int ITEMS = A_ITEMS + B_ITEMS;
  static constexpr uint32_t FSTRIDE = 16u * T::RB;  // bytes per 16-row fragment of A / B[N,K]
  uint32_t a_base[T::KK];  // per kk: A slot 0 of this lane (even slots), from the A region
  uint32_t a_odd[T::KK];   // per kk: base for odd slots
  uint32_t b_base[T::KK];  // per kk: B fragment 0 (half 0) of this lane, from the B region
  uint32_t b_odd[T::KK];   // KN: base for odd fragments (the XOR in b_blk_off)

  __device__ __forceinline__ void init(int wm, int wn, int lane, int a_xor = 0) {
    const int l16 = lane & 15, g = lane >> 4;
#pragma unroll
    for (int kk = 0; kk < T::KK; ++kk) {
      const int row = wm * T::WTM + l16;
      // (row = l16 modulo 16, which is all the swizzle looks at)
      const uint32_t a0 = (uint32_t)(row * T::RB + (((kk * 4 + g) ^ a_swz<T>(l16)) << 4));
      // slot i reads fragment i ^ a_xor: +FSTRIDE for even slots, -FSTRIDE for
      // odd ones (odd slots are >= 1, so the sum never wraps below zero)
      a_base[kk] = a0 + FSTRIDE * (uint32_t)a_xor;
      a_odd[kk] = a0 - FSTRIDE * (uint32_t)a_xor;
      if constexpr (T::AKM) {
        // as B[K,N] below, with rows of A in place of columns of B
        const int k = kk * 32 + 8 * g + (l16 >> 2);
        const int m = wm * T::WTM + 4 * (l16 & 3);
        const uint32_t p = (uint32_t)((k >> 3) & 1);
        const uint32_t b0 = b_blk_off<T::BM>(k, m) + 256u;
        a_base[kk] = b0;
        a_odd[kk] = b0 - 256u * p;
      }
      if constexpr (T::KN) {
        // k = kk*32 + 8g + (l16 >> 2) (+4 for the second half), n = wn*WTN +
        // 16j + 4*(l16 & 3).  Fragment j sits at block (j ^ p), p = g & 1,
        // i.e. at +128 j from b_base (even j) or b_odd (odd j).
        const int k = kk * 32 + 8 * g + (l16 >> 2);
        const int n = wn * T::WTN + 4 * (l16 & 3);
        const uint32_t p = (uint32_t)((k >> 3) & 1);
        const uint32_t b0 = b_blk_off<T::BN>(k, n) + 256u;  // fragment 0 (+256: see b_odd)
        b_base[kk] = b0;                       // even j: block j ^ p = j + p (p already in b0)
        b_odd[kk] = b0 - 256u * p;             // odd j: block j ^ p = j - p
        // (both carry +256 so that b_odd stays non-negative; read() takes it off)
      } else {
        const int brow = wn * T::WTN + l16;
        b_base[kk] = (uint32_t)(brow * T::RB + (((kk * 4 + g) ^ a_swz<T>(l16)) << 4));
      }
    }
  }
  // a_st / b_st: LDS byte offsets of the A and B regions holding this k-tile.
  __device__ __forceinline__ void read(Frags<T>& f, int item, lds_char* lds, uint32_t a_st,
                                       uint32_t b_st, int kk) const {
    if constexpr (T::AKM) {
      if (item < A_ITEMS) {
        const int i = item >> 1, h = item & 1;
        const uint32_t o = (uint32_t)i * 128u + (uint32_t)h * (uint32_t)(T::BM / 16) * 128u;
        const u32x2 v = lds_read_tr16(lds, a_st - 256u + ((i & 1) ? a_odd[kk] : a_base[kk]) + o);
        if (h == 0) { f.a[i][0] = v[0]; f.a[i][1] = v[1]; }
        else { f.a[i][2] = v[0]; f.a[i][3] = v[1]; }
        return;
      }
    } else {
      if (item < T::FM) {
        f.a[item] = lds_read16(lds, a_st + ((item & 1) ? a_odd[kk] : a_base[kk]) +
                                        (uint32_t)item * FSTRIDE);
        return;
      }
    }
    const int bi = item - A_ITEMS;
    if constexpr (T::KN) {
      const int j = bi >> 1, h = bi & 1;
      // +16 columns per fragment = next block; +4 k-rows per half = next block row
      const uint32_t o = (uint32_t)j * 128u + (uint32_t)h * (uint32_t)(T::BN / 16) * 128u;
      const u32x2 v = lds_read_tr16(lds, b_st - 256u + ((j & 1) ? b_odd[kk] : b_base[kk]) + o);
      if (h == 0) { f.b[j][0] = v[0]; f.b[j][1] = v[1]; }
      else { f.b[j][2] = v[0]; f.b[j][3] = v[1]; }
    } else {
      f.b[bi] = lds_read16(lds, b_st + b_base[kk] + (uint32_t)bi * FSTRIDE);
    }
  }
};

__device__ __forceinline__ uint32_t scale_pair(uint32_t w, float r_lo, float r_hi) {
  return pack_bf16x2(bf16_lo(w) * r_lo, bf16_hi(w) * r_hi);
}

// Regrouped Lazy Pre-Norm weight gradient.  dB = A_hat^T dC with A_hat =
// rstd * A equals A^T (rstd * dC): the scale can sit on the upstream
// gradient instead, so that the weight gradient becomes a plain product.  The
// input-gradient kernel, whose own A operand is dC ([M, K] here), writes
// rstd * dC, rounded to bf16, for the rows of each row block, split by rows
// over the row block's `parts` workgroups (rows past M are skipped).  It
// runs in the epilogue, after the k-loop's transfers have all landed, so its
// loads and stores are the compiler's to count.
template <class T>
__device__ __forceinline__ void write_scaled_rows(const GemmParams& p, int m_base, int part,
                                                  int parts, int tid) {
  const int rows = min(T::BM, p.M - m_base);
  const int rpp = (rows + parts - 1) / parts;
  const int r0 = part * rpp, r1 = min(rows, r0 + rpp);
  const int cpr = p.K / 8;  // 16-byte chunks per row
  constexpr int RB = 4;     // rows in flight per lane
  for (int c = tid; c < cpr; c += T::NT) {
    for (int r = r0; r < r1; r += RB) {
      u32x4 v[RB];
      float sc[RB];
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        if (r + b < r1) {
          const size_t off = (size_t)(m_base + r + b) * (size_t)p.K + 8u * (size_t)c;
          v[b] = *(const u32x4*)(p.A + off);
          sc[b] = p.row_rstd[m_base + r + b];
        }
      }
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        if (r + b < r1) {
          const size_t off = (size_t)(m_base + r + b) * (size_t)p.K + 8u * (size_t)c;
          u32x4 w = v[b];
#pragma unroll
          for (int q = 0; q < 4; ++q) w[q] = scale_pair(w[q], sc[b], sc[b]);
          *(u32x4*)(p.scaled_out + off) = w;
        }
      }
    }
  }
}

// RS: the scaled operand's k-tile is scaled in LDS, once per workgroup (a
// fragment is held by several waves: WN of them for A, WM for B), each wave
// the 16-byte chunks that its own transfers wrote.  In the blocked [K, X]
// layout a chunk holds 8 elements of one k row, which share one scale.
template <class T>
constexpr bool scale_b_side() { return T::RS == 2; }
template <class T>
constexpr bool scale_ahead() { return T::RS != 0; }

template <class T>
struct ChunkScaler {
  static constexpr bool BS = scale_b_side<T>();
  static constexpr int INS = BS ? DmaPlan<T>::B_INS : DmaPlan<T>::A_INS;
  static constexpr int W = BS ? T::BN : T::BM;
  static constexpr uint32_t REGION = BS ? (uint32_t)T::A_BYTES : 0u;
  static constexpr uint32_t RSLOT = (uint32_t)(T::A_BYTES + T::B_BYTES);
  // A wave's transfer j moves slots (wave*INS + j)*64 + lane, i.e. 16-byte
  // block (wave*INS + j)*8 + lane/8 of the blocked layout (W/16 blocks per
  // row of 4 k rows).  When a block row holds a whole number of waves'
  // blocks, all INS chunks of a lane sit in one block row, at k row
  // 4*kb + (lane % 8)/2 with kb = (wave*INS*8) / (W/16): a wave needs the
  // four scales of k rows 4*kb .. 4*kb+3, one per lane.
  static_assert(T::RS == 0 || (W / 16) % (INS * 8) == 0, "a wave's chunks share their k rows");
  static __device__ __forceinline__ int kb(int wave) { return (wave * INS * 8) / (W / 16); }
  u32x4 v;
  float r;
  uint32_t o;  // LDS byte offset of chunk 0
  // chunk 0's bytes and the lane's scale, from the stage at `st`
  __device__ __forceinline__ void load_first(lds_char* lds, uint32_t st, int wave, int lane) {
    r = *(lds_float*)(lds + st + RSLOT + 16u * (uint32_t)kb(wave) + (uint32_t)((lane & 6) << 1));
    o = st + REGION + (uint32_t)(wave * INS) * 1024u + (uint32_t)lane * 16u;
    v = lds_read16(lds, o);
  }
  // chunk j (> 0): 1 KB after chunk j-1
  __device__ __forceinline__ void load(lds_char* lds, int j) {
    v = lds_read16(lds, o + (uint32_t)j * 1024u);
  }
  // dword w (0 .. 3) of the loaded chunk: its bf16 pair times the scale
  __device__ __forceinline__ void scale(int w) { v[w] = scale_pair(v[w], r, r); }
  __device__ __forceinline__ void store(lds_char* lds, int j) const {
    lds_write16(lds, o + (uint32_t)j * 1024u, v);
  }
};

template <class T>
__device__ __forceinline__ void scale_own_chunks(lds_char* lds, uint32_t st, int wave, int lane) {
  static_assert(scale_ahead<T>(), "scaled operand");
  int ln = lane;
  asm volatile("" : "+v"(ln));
  ChunkScaler<T> sc;
#pragma unroll
  for (int j = 0; j < ChunkScaler<T>::INS; ++j) {
    if (j == 0) sc.load_first(lds, st, wave, ln);
    else sc.load(lds, j);
#pragma unroll
    for (int w = 0; w < 4; ++w) sc.scale(w);
    sc.store(lds, j);
  }
}

// The sub-step that computes k-tile kt scales the chunks of k-tile
// kt+2 that this wave's own transfers wrote (they have landed: the wait
// before the sub-step covers kt+2), one chunk at a time: read at slot
// SC_GAP*j, scaled one dword per slot from SC_GAP*j + SC_LAT on, written back
// at the slot after; the barrier before the next sub-step publishes them,
// and the sub-step after that reads them as fragments.  No wave touches
// k-tile kt+2's stage in between: the reads of the sub-step are of kt+1, its
// transfers refill kt's.
template <class T>
constexpr int sc_lat() { return 6; }
template <class T>
constexpr int sc_gap() { return sc_lat<T>() + 5; }

// Lazy Pre-Norm sum of squares on the matrix cores.  For an A fragment F
// (16 rows x 32 k of the sub-step), one MFMA of F with itself gives the 16x16
// Gram block F F^T, whose diagonal holds each row's sum of squares over those
// 32 k: bf16 products are exact in fp32 and accumulate in fp32 across the
// k-loop, as in the GEMM itself.  Diagonal element r lands in lane
// 16*(r >> 2) + r, register r & 3 (the MFMA output layout).  With two waves
// per row set (lazy_split) each wave takes only its even slots, which hold
// different fragments in the two waves (FragReader's a_xor): FM/2 extra MFMAs
// on FM*FN, and the halves are swapped after the k-loop.  (Measured on
// gfx950: 1.2 % over the plain GEMM, against 3 % for squaring with VALU FMAs
// placed between the MFMAs and more for v_dot2_f32_bf16.)
template <class T>
constexpr bool lazy_split() { return T::WN == 2 && T::FM % 2 == 0; }
template <class T>
constexpr int lazy_slots() { return lazy_split<T>() ? T::FM / 2 : T::FM; }

// Without the split (one wave per row set, the narrow-row tile) the Gram
// MFMAs would add FM per FM*FN products, and the squares are taken on the
// VALU instead: the lane's 8 elements of the fragment, one fmaf each, spread
// over the products' slots, into register 0 of the slot's accumulator (the
// lane's own row and k-group; the later lane-group sum adds the row's four
// k-groups).  (Measured on 256x128x64: 4.9 against 5.2 us; on the 256x256
// tile with the split, the Gram MFMAs are faster: 922-925 against
// 937-942 us on 32768x4096x4096.)
template <class T>
constexpr bool lazy_valu() { return !lazy_split<T>(); }

// Gram accumulator g belongs to slot (lazy_split ? 2g : g); each is updated
// once per sub-step, after the last product MFMA that shares its fragment
// (on the VALU path: one element every STEP/8 slots).
template <class T>
__device__ __forceinline__ void lazy_gram(int q, const Frags<T>& cur,
                                          f32x4 (&gram)[lazy_slots<T>()]) {
  constexpr int STEP = (T::FM * T::FN) / lazy_slots<T>();
  static_assert((T::FM * T::FN) % lazy_slots<T>() == 0, "Gram MFMA spacing");
  if constexpr (lazy_valu<T>()) {
    static_assert(STEP % 8 == 0, "VALU squares: 8 elements per fragment");
    if (q % (STEP / 8) == STEP / 8 - 1) {
      const int g = q / STEP;
      const int e = (q % STEP) / (STEP / 8);  // element 0..7 of the lane's 8
      const uint32_t w = cur.a[g][e >> 1];
      const float x = (e & 1) ? bf16_hi(w) : bf16_lo(w);
      gram[g][0] = fmaf(x, x, gram[g][0]);
    }
  } else if (q % STEP == STEP - 1) {
    const int g = q / STEP;
    const int k = lazy_split<T>() ? 2 * g : g;
    gram[g] = mfma_16x16x32(cur.a[k], cur.a[k], gram[g]);
  }
}

// One k32 sub-step: FM*FN MFMAs on `cur`, with the LDS reads of the next
// sub-step's fragments (into `nxt`) and, when dma_on, the LDS transfers of a
// later k-tile spread evenly between them.  (On the last sub-step the reads
// fetch stale but in-bounds LDS data that is never used: one code path keeps
// the accumulators in place.)  For Lazy Pre-Norm the Gram MFMAs of the A
// fragments join the sequence.
// DM: 0 = issue the transfers when dma_on, 1 = always, 2 = never (the last
// two make the choice at compile time, without a branch per transfer).
// SC (scaled operands): 0 = no scaling ahead, 1 = scale the stage at sc_st,
// 2 = do so when sc_on.
template <class T, bool LAZY, int DM = 0, int SC = 0>
__device__ __forceinline__ void substep(f32x4 (&acc)[T::FM][T::FN],
                                        f32x4 (&gram)[lazy_slots<T>()],
                                        const Frags<T>& cur, Frags<T>& nxt, lds_char* lds,
                                        const FragReader<T>& rd, uint32_t rd_st, int rd_kk,
                                        const DmaPlan<T>& dma,
                                        bool dma_on, const GemmParams& p, int m_base,
                                        int n_base, int dma_kt, uint32_t dma_st,
                                        uint32_t sc_st = 0, bool sc_on = false, int lane = 0) {
  constexpr int NM = T::FM * T::FN;
  constexpr int NR = FragReader<T>::ITEMS;
  constexpr int ND = DmaPlan<T>::INS;
  ChunkScaler<T> sc;
  constexpr int SCJ = ChunkScaler<T>::INS;
  static_assert(!scale_ahead<T>() || sc_gap<T>() * SCJ <= NM, "scale-ahead slots");
#pragma unroll
  for (int q = 0; q < NM; ++q) {
    const int i = q / T::FN, j = q % T::FN;
    acc[i][j] = mfma_16x16x32(cur.b[j], cur.a[i], acc[i][j]);
    if constexpr (scale_ahead<T>() && SC != 0) {
      if (SC == 1 || sc_on) {
        constexpr int G = sc_gap<T>(), L = sc_lat<T>();
        const int j = q / G, u = q % G;
        if (j < SCJ) {
          if (u == 0) {
            if (j == 0) sc.load_first(lds, sc_st, dma.wave, lane);
            else sc.load(lds, j);
          }
          if (u >= L && u < L + 4) sc.scale(u - L);
          if (u == L + 4) sc.store(lds, j);
        }
      }
    }
    if constexpr (LAZY) lazy_gram<T>(q, cur, gram);
#pragma unroll
    for (int r = (q * NR) / NM; r < ((q + 1) * NR) / NM; ++r)
      rd.read(nxt, r, lds, rd_st, rd_st + T::A_BYTES, rd_kk);
#pragma unroll
    for (int d = (q * ND) / NM; d < ((q + 1) * ND) / NM; ++d)
      if (DM == 1 || (DM == 0 && dma_on)) dma.issue(p, m_base, n_base, dma_kt, dma_st, d);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Full k-loop for the tile at (m_base, n_base).  STAGES LDS stages used as a
// ring; fragments double-buffered in registers.  Per k-tile kt (stage s):
//   sub-step 0: MFMAs on (kt, k 0..31) while reading (kt, k 32..63);
//   wait for k-tile kt+1's transfers, barrier;
//   sub-step 1: MFMAs on (kt, k 32..63) while reading (kt+1, k 0..31) and
//               issuing k-tile kt+STAGES's transfers into stage s (no wave
//               reads stage s any more after the barrier).
// LDS transfers of the first STAGES k-tiles of the tile at (m_base, n_base):
// k-tiles 0, 1, ..., or with `rev` (the tile's k-loop walks downwards) the
// last ones, nk-1, nk-2, ....
template <class T>
__device__ __forceinline__ void issue_prologue(const GemmParams& p, uint32_t lds0, int m_base,
                                               int n_base, int tid, bool rev = false) {
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  DmaPlan<T> dma;
  dma.init(p, m_base, n_base, lane, wave);
  constexpr int ND = DmaPlan<T>::INS;
  const int nk = (p.K + T::BK - 1) / T::BK;
#pragma unroll
  for (int st = 0; st < T::STAGES; ++st) {
    if (st < nk) {
#pragma unroll
      for (int d = 0; d < ND; ++d)
        dma.issue(p, m_base, n_base, rev ? nk - 1 - st : st, lds0 + st * T::STAGE, d);
    }
  }
}

// Wait until a k-tile has landed in LDS, given that `after` later k-tiles
// (ND transfers each, 0 .. STAGES-1 of them) and X other vector-memory
// operations were issued after it.  Vector-memory operations of a wave
// complete in issue order, so at most after*ND + X may remain outstanding;
// X must not exceed the true count (more operations only make the wait
// stricter).
template <int ND, int STAGES, int X = 0>
__device__ __forceinline__ void wait_ktile(int after) {
  if (STAGES > 3 && after >= 3) wait_vmcnt<(STAGES > 3 ? 3 * ND + X : 0)>();
  else if (STAGES > 2 && after == 2) wait_vmcnt<(STAGES > 2 ? 2 * ND + X : 0)>();
  else if (after == 1) wait_vmcnt<ND + X>();
  else wait_vmcnt<X>();
}

// prologue_issued: the first STAGES k-tiles were issued by the caller (or by
// the previous tile's k-loop, see below).
// stores_after: the caller then issued at least T::C_STORES further
// vector-memory operations (the previous tile's output) before this call.
// LAZY: ss[i] receives this lane's share of slot i's row sums of squares
// (summed over the 4 lane groups they give the row's total over this wave's
// A fragments; zero for slots the wave did not take).
// Cross-tile prefetch (32-deep k-tiles only, nk >= STAGES): with nx_m >= 0
// the sub-steps whose refill would lie past the end of this tile's k-loop
// issue the first STAGES k-tiles of the next tile (m_base nx_m, n_base nx_n)
// instead, into the stages this tile vacates, so that they land during this
// tile's last k-tiles rather than behind its epilogue.  k-tile j of a tile
// sits in stage (j + srot) % STAGES; the next tile's srot is (srot + nk) %
// STAGES.  Every sub-step then issues STAGES - 2 k-tiles' worth of
// transfers after the one awaited, tile after tile.  (A tile's epilogue
// polls and loads wait for every earlier transfer, so transfers issued after
// the k-loop would hold them up.)
// REV: the k-tiles are walked downwards (k-tile nk-1 first); nx_rev: the
// next tile's walk, for its prefetched first k-tiles.  The sum over k then
// runs in the other order, which changes the fp32 rounding, not the result.
template <class T, bool LAZY, bool REV = false>
__device__ __forceinline__ void mainloop(const GemmParams& p, f32x4 (&acc)[T::FM][T::FN],
                                         float (&ss)[T::FM], lds_char* lds, uint32_t lds0,
                                         int m_base, int n_base, int tid,
                                         bool prologue_issued = false, bool stores_after = false,
                                         int srot = 0, int nx_m = -1, int nx_n = 0,
                                         bool nx_rev = false) {
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / T::WN, wn = wave % T::WN;
  f32x4 gram[lazy_slots<T>()];
#pragma unroll
  for (int g = 0; g < lazy_slots<T>(); ++g) gram[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < T::FM; ++i) {
    ss[i] = 0.f;
#pragma unroll
    for (int j = 0; j < T::FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  DmaPlan<T> dma;
  dma.init(p, m_base, n_base, lane, wave);
  FragReader<T> rd;
  rd.init(wm, wn, lane, (LAZY && lazy_split<T>()) ? wn : 0);
  constexpr int ND = DmaPlan<T>::INS;
  constexpr int NR = FragReader<T>::ITEMS;
  const int nk = (p.K + T::BK - 1) / T::BK;
  const bool xt = !scale_ahead<T>() && nx_m >= 0 && nk >= T::STAGES;
  // global k-tile of the walk's k-th k-tile
  auto kmap = [&](int k) { return REV ? nk - 1 - k : k; };
  // LDS byte offset of the stage that holds k-tile k
  auto stg = [&](int k) { return (uint32_t)((k + srot) % T::STAGES) * T::STAGE; };
  // Wait until a k-tile has landed with `after` later k-tiles (and, with
  // st_after, the caller's output stores) still allowed in flight.  With a
  // scaled operand only wave 0 issues the scale transfers.
  auto waitk = [&](int after, bool st_after) {
    constexpr int NDW = ND - DmaPlan<T>::R_INS;  // transfers per k-tile of waves 1..
    if (DmaPlan<T>::R_INS && wave == 0) {
      if (st_after) wait_ktile<ND, T::STAGES, T::C_STORES>(after);
      else wait_ktile<ND, T::STAGES>(after);
    } else {
      if (st_after) wait_ktile<NDW, T::STAGES, T::C_STORES>(after);
      else wait_ktile<NDW, T::STAGES>(after);
    }
  };

  if (!prologue_issued) issue_prologue<T>(p, lds0, m_base, n_base, tid, REV);
  if constexpr (scale_ahead<T>()) {
    // k-tiles 0 and 1 are scaled here, the later ones one k-tile ahead
    const int after = nk >= 2 ? min(nk, T::STAGES) - 2 : 0;
    waitk(after, stores_after);
    // (wave 0's scale transfers have landed for every wave after a barrier)
    __syncthreads();
    scale_own_chunks<T>(lds, stg(0), wave, lane);
    if (nk >= 2) scale_own_chunks<T>(lds, stg(1), wave, lane);
  } else {
    waitk(min(nk, T::STAGES) - 1, stores_after);
  }
  __syncthreads();
  Frags<T> f0, f1;
#pragma unroll
  for (int r = 0; r < NR; ++r) rd.read(f0, r, lds, stg(0), stg(0) + T::A_BYTES, 0);

  int cur_s = srot % T::STAGES;  // (KK = 2 loop) stage of k-tile kt
  int kt = 0;
  // k-tile kt+1 must have landed; k-tiles kt+2 .. kt+STAGES-1 may still fly
  // (and, while kt+1 is a prologue k-tile, the caller's stores after them)
  auto wait_next = [&](int kt) {
    if constexpr (scale_ahead<T>()) {
      // k-tile kt+1 was awaited (and scaled) one sub-step earlier; kt+2 is
      // scaled during this one
      if (kt + 2 < nk) {
        const int after = min(nk - 1, kt + T::STAGES - 1) - (kt + 2);
        waitk(after, stores_after && kt + 2 < T::STAGES);
      }
      return;
    }
    if (kt + 1 < nk) {
      const int after = xt ? T::STAGES - 2 : min(nk - 1, kt + T::STAGES - 1) - (kt + 1);
      waitk(after, stores_after && kt + 1 < T::STAGES);
    }
  };
  if constexpr (T::KK == 1) {
    // One k32 sub-step per k-tile.  Before k-tile kt is computed (its
    // fragments are in registers), k-tile kt+1 must have landed; the sub-step
    // reads kt+1's fragments and refills kt's stage, whose reads all completed
    // before the barrier, with k-tile kt+STAGES.  Two k-tiles per trip keep
    // the two fragment sets in fixed registers.
    // steady state, peeled: both k-tiles of a trip refill a stage
    for (; kt + 1 + T::STAGES < nk; kt += 2) {
      const uint32_t s0 = stg(kt);
      const uint32_t s1 = stg(kt + 1);
      const uint32_t s2 = stg(kt + 2);
      wait_next(kt);
      __syncthreads();
      substep<T, LAZY, 1, 1>(acc, gram, f0, f1, lds, rd, s1, 0, dma, true, p, m_base, n_base,
                             kmap(kt + T::STAGES), lds0 + s0, s2, true, lane);
      wait_next(kt + 1);
      __syncthreads();
      substep<T, LAZY, 1, 1>(acc, gram, f1, f0, lds, rd, s2, 0, dma, true, p, m_base, n_base,
                             kmap(kt + 1 + T::STAGES), lds0 + s1, stg(kt + 3), true, lane);
    }
    // the last sub-steps: refills of this tile while there are k-tiles left,
    // then (cross-tile prefetch) the next tile's first k-tiles
    bool switched = false;
    auto refill = [&](int u, bool& on, int& mb, int& nb, int& uk) {
      on = u < nk;
      mb = m_base;
      nb = n_base;
      uk = kmap(u);
      if (!on && xt) {
        if (!switched) {
          dma.init(p, nx_m, nx_n, lane, wave);
          switched = true;
        }
        on = true;
        mb = nx_m;
        nb = nx_n;
        uk = nx_rev ? 2 * nk - 1 - u : u - nk;
      }
    };
    for (; kt < nk; kt += 2) {
      bool on;
      int mb, nb, uk;
      wait_next(kt);
      __syncthreads();
      refill(kt + T::STAGES, on, mb, nb, uk);
      if constexpr (scale_ahead<T>())
        substep<T, LAZY, 0, 2>(acc, gram, f0, f1, lds, rd, stg(kt + 1), 0, dma, on, p, mb, nb,
                               uk, lds0 + stg(kt), stg(kt + 2), kt + 2 < nk, lane);
      else
        substep<T, LAZY>(acc, gram, f0, f1, lds, rd, stg(kt + 1), 0, dma, on, p, mb, nb, uk,
                         lds0 + stg(kt));
      if (kt + 1 >= nk) break;
      wait_next(kt + 1);
      __syncthreads();
      refill(kt + 1 + T::STAGES, on, mb, nb, uk);
      if constexpr (scale_ahead<T>())
        substep<T, LAZY, 0, 2>(acc, gram, f1, f0, lds, rd, stg(kt + 2), 0, dma, on, p, mb, nb,
                               uk, lds0 + stg(kt + 1), stg(kt + 3), kt + 3 < nk, lane);
      else
        substep<T, LAZY>(acc, gram, f1, f0, lds, rd, stg(kt + 2), 0, dma, on, p, mb, nb, uk,
                         lds0 + stg(kt + 1));
    }
  } else {
    if constexpr (!LAZY) {
      // steady state, peeled: every k-tile refills its stage, with no branch per
      // transfer (for Lazy Pre-Norm the second copy of the loop body costs
      // registers that it does not have to spare)
      for (; kt + T::STAGES < nk; ++kt) {
        const int nxt_s = cur_s + 1 == T::STAGES ? 0 : cur_s + 1;
        const uint32_t cur = (uint32_t)cur_s * T::STAGE;
        const uint32_t nxt = (uint32_t)nxt_s * T::STAGE;
        substep<T, LAZY, 2>(acc, gram, f0, f1, lds, rd, cur, 1, dma, false, p, m_base, n_base, 0, 0);
        wait_next(kt);
        __syncthreads();
        substep<T, LAZY, 1>(acc, gram, f1, f0, lds, rd, nxt, 0, dma, true, p, m_base, n_base,
                            kmap(kt + T::STAGES), lds0 + cur);
        cur_s = nxt_s;
      }
    }
    bool switched = false;
    for (; kt < nk; ++kt) {
      const int nxt_s = cur_s + 1 == T::STAGES ? 0 : cur_s + 1;
      const uint32_t cur = (uint32_t)cur_s * T::STAGE;
      const uint32_t nxt = (uint32_t)nxt_s * T::STAGE;
      substep<T, LAZY, 2>(acc, gram, f0, f1, lds, rd, cur, 1, dma, false, p, m_base, n_base, 0, 0);
      wait_next(kt);
      __syncthreads();
      // stage cur is free now: refill it with k-tile kt+STAGES, or (cross-tile
      // prefetch) with the next tile's first k-tiles
      int u = kt + T::STAGES, mb = m_base, nb = n_base;
      bool on = u < nk;
      if (on) {
        u = kmap(u);
      } else if (xt) {
        if (!switched) {
          dma.init(p, nx_m, nx_n, lane, wave);
          switched = true;
        }
        on = true;
        mb = nx_m;
        nb = nx_n;
        u = nx_rev ? 2 * nk - 1 - u : u - nk;
      }
      substep<T, LAZY>(acc, gram, f1, f0, lds, rd, nxt, 0, dma, on, p, mb, nb, u, lds0 + cur);
      cur_s = nxt_s;
    }
  }
  // every wave is done with the stages before they are reused
  __syncthreads();
  if constexpr (LAZY) {
    // the Gram diagonal: row l16 of a slot in lane group l16 >> 2, register
    // l16 & 3; the other lane groups contribute zero to the later lane-group
    // sum (VALU path: every lane holds its k-group's partial in register 0)
    const int l16 = lane & 15, g = lane >> 4;
    const int r = l16 & 3;
#pragma unroll
    for (int gi = 0; gi < lazy_slots<T>(); ++gi) {
      const f32x4 d = gram[gi];
      const float v = r == 0 ? d[0] : r == 1 ? d[1] : r == 2 ? d[2] : d[3];
      ss[lazy_split<T>() ? 2 * gi : gi] = lazy_valu<T>() ? d[0] : (g == (l16 >> 2) ? v : 0.f);
    }
  }
}

// Sum over the 4 lane groups sharing (lane & 15): a row's partial over this
// wave's columns (or, for the lazy sum of squares, over this wave's k-groups).
// v_permlane16_swap / v_permlane32_swap hand every lane both members of its
// xor-16 (then xor-32) pair, lower lane first, so all four lanes add the same
// operands in the same order: (x0 + x16) + (x32 + x48).
__device__ __forceinline__ float reduce_lane_groups(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto p16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float s16 = __uint_as_float(p16[0]) + __uint_as_float(p16[1]);
  const uint32_t w = __float_as_uint(s16);
  const auto p32 = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return __uint_as_float(p32[0]) + __uint_as_float(p32[1]);
}

template <class T>
__device__ __forceinline__ void combine_waves(float (&out)[T::FM], lds_char* lds, int wm, int wn,
                                              int lane);

// Per-row sums of this workgroup's accumulators over its valid columns,
// combined across the WN waves that share rows through LDS (fixed order).
// mode 0: sum x;  mode 1: sum (x - center[i])^2;  mode 2: sum x^2.
// Result: out[i] for row wm*WTM + 16i + (lane & 15), same in all lanes of the group.
template <class T>
__device__ __forceinline__ void wave_row_sums(const f32x4 (&acc)[T::FM][T::FN],
                                              const bool (&colv)[T::FN], int mode,
                                              const float (&center)[T::FM], float (&out)[T::FM]);

template <class T>
__device__ __forceinline__ void tile_row_sums(const f32x4 (&acc)[T::FM][T::FN],
                                              const bool (&colv)[T::FN], int mode,
                                              const float (&center)[T::FM], float (&out)[T::FM],
                                              lds_char* lds, int wm, int wn, int lane) {
  wave_row_sums<T>(acc, colv, mode, center, out);
  combine_waves<T>(out, lds, wm, wn, lane);
}

// The same sums over this wave's columns only (no exchange between waves).
template <class T>
__device__ __forceinline__ void wave_row_sums(const f32x4 (&acc)[T::FM][T::FN],
                                              const bool (&colv)[T::FN], int mode,
                                              const float (&center)[T::FM], float (&out)[T::FM]) {
#pragma unroll
  for (int i = 0; i < T::FM; ++i) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < T::FN; ++j) {
      if (!colv[j]) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float x = acc[i][j][r];
        if (mode == 0) s += x;
        else if (mode == 1) { float d = x - center[i]; s = fmaf(d, d, s); }
        else s = fmaf(x, x, s);
      }
    }
    out[i] = reduce_lane_groups(s);
  }
}

// Sum of per-wave row partials over the WN waves that share rows, through
// LDS in a fixed order (no-op for WN = 1).  Two barriers when WN > 1.
template <class T>
__device__ __forceinline__ void combine_waves(float (&out)[T::FM], lds_char* lds, int wm, int wn,
                                              int lane) {
  const uint32_t red = T::RED_OFF;
  if constexpr (T::WN > 1) {
    if (lane < 16) {
#pragma unroll
      for (int i = 0; i < T::FM; ++i)
        *(lds_float*)(lds + red + (wn * T::BM + wm * T::WTM + 16 * i + lane) * 4) = out[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
      float s = 0.f;
      for (int w = 0; w < T::WN; ++w)
        s += *(lds_float*)(lds + red + (w * T::BM + wm * T::WTM + 16 * i + (lane & 15)) * 4);
      out[i] = s;
    }
    __syncthreads();
  }
}

// Byte offset of 16-byte chunk c (0..7) of row r (0..15) in a wave's 2 KB
// output staging block.  XORing the chunk with (r >> 1) & 7 lets both the
// 8-byte fragment writes (16 rows per 32 lanes) and the 16-byte row reads
// touch every LDS bank once per pass.
__device__ __forceinline__ uint32_t stg_chunk(int r, int c) {
  return (uint32_t)(r * 128 + ((c ^ ((r >> 1) & 7)) << 4));
}

// A bf16 [M][N] matrix's tile, staged in the pipeline stages between a
// tile's k-loop and the next tile's first transfers (the residual R, or the
// forward input of the Lazy backward).  Each wave moves its WTM x WTN slice:
// 256-byte rows (WTN = 128 columns), one 1 KB transfer per 4 rows, 16-byte
// chunk c of row r at chunk position c ^ (r & 15) so that a fragment read
// (16 rows, one chunk each) touches every bank once.  Each wave reads back
// only the rows it moved, so its own transfer count is the only wait.  Rows
// past M and columns past N read as zero.  The slices start after the output
// staging when the staging lies on the stages.
template <class T>
constexpr uint32_t tile_lds_base() {
  return T::STG_OWN ? 0u : (uint32_t)T::STG_BYTES;
}

template <class T>
__device__ __forceinline__ uint32_t tile_lds_region(int wave) {
  return tile_lds_base<T>() +
         (uint32_t)__builtin_amdgcn_readfirstlane(wave) * (uint32_t)T::WTM * 256u;
}

template <class T>
__device__ __forceinline__ void load_tile_lds(const GemmParams& p, const uint16_t* src,
                                              uint32_t lds0, int m_base, int n_base, int wave,
                                              int wn, int lane) {
  static_assert(T::WTN == 128, "staged rows of 16 chunks");
  static_assert(tile_lds_base<T>() + (T::NT / 64) * T::WTM * 256 <= T::STAGES * T::STAGE,
                "staged slices fit the stages");
  static_assert(T::WTM % 4 == 0, "4 rows per transfer");
  // wave-uniform copies (the transfer's LDS address and buffer are scalar)
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int m_w = __builtin_amdgcn_readfirstlane(m_base + (wv / T::WN) * T::WTM);
  const int n_w = n_base + wn * T::WTN;
  const uint32_t region = tile_lds_region<T>(wv);
  const uint64_t total = (uint64_t)p.M * (uint64_t)p.N;
  const int rq = lane >> 4, c = (lane & 15);
#pragma unroll
  for (int q = 0; q < T::WTM / 4; ++q) {
    // rows m_w + 4q .. +3 from a base at row m_w + 4q (offsets below 2^28)
    const uint64_t base = (uint64_t)(m_w + 4 * q) * (uint64_t)p.N;
    const uint64_t left = total > base ? (total - base) * 2u : 0u;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(src + base, left);
    const int r = 4 * q + rq;
    const int n = n_w + 8 * (c ^ (r & 15));
    const uint32_t voff = n < p.N ? ((uint32_t)rq * (uint32_t)p.N + (uint32_t)n) * 2u : kOOB;
    dma16(rs, lds0 + region + (uint32_t)q * 1024u, voff, 0);
  }
  wait_vmcnt<0>();
}

// The 4 bf16 of the staged tile at this lane's accumulator acc[i][j].
template <class T>
__device__ __forceinline__ u32x2 tile_lds_frag(lds_char* lds, uint32_t region, int i, int j,
                                               int lane) {
  const int l16 = lane & 15, g = lane >> 4;
  const int pos = (2 * j + (g >> 1)) ^ l16;
  return *(lds_u32x2*)(lds + region + (uint32_t)(16 * i + l16) * 256u + (uint32_t)pos * 16u +
                       8u * (uint32_t)(g & 1));
}

// Per-row sums of acc * X over this wave's columns, X the staged tile (zero
// past N).
template <class T>
__device__ __forceinline__ void wave_dot_sums(const f32x4 (&acc)[T::FM][T::FN], lds_char* lds,
                                              int wave, int lane, float (&out)[T::FM]) {
  const uint32_t region = tile_lds_region<T>(wave);
#pragma unroll
  for (int i = 0; i < T::FM; ++i) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < T::FN; ++j) {
      const u32x2 x = tile_lds_frag<T>(lds, region, i, j, lane);
      s = fmaf(acc[i][j][0], bf16_lo(x[0]), s);
      s = fmaf(acc[i][j][1], bf16_hi(x[0]), s);
      s = fmaf(acc[i][j][2], bf16_lo(x[1]), s);
      s = fmaf(acc[i][j][3], bf16_hi(x[1]), s);
    }
    out[i] = reduce_lane_groups(s);
  }
}

// The same sums over the workgroup's columns, combined across the waves
// sharing rows.
template <class T>
__device__ __forceinline__ void tile_dot_sums(const f32x4 (&acc)[T::FM][T::FN], lds_char* lds,
                                              int wave, int wm, int wn, int lane,
                                              float (&out)[T::FM]) {
  wave_dot_sums<T>(acc, lds, wave, lane, out);
  combine_waves<T>(out, lds, wm, wn, lane);
}

// Per-column gamma/beta of a wave's columns, as loaded bf16 pairs: g[j] and
// b[j] hold the 4 columns 16j + 4(lane >> 4) .. +3 of the wave's slice
// (1 and 0 where absent).  Loaded ahead of the row statistics so that their
// latency overlaps them.
template <class T>
struct Affine {
  u32x2 g[T::FN], b[T::FN];
};

template <class T>
__device__ __forceinline__ void load_affine(const GemmParams& p, int n_base, int wn, int lane,
                                            Affine<T>& aff) {
  const int g = lane >> 4;
#pragma unroll
  for (int j = 0; j < T::FN; ++j) {
    aff.g[j] = u32x2{0x3f803f80u, 0x3f803f80u};  // bf16 1.0 pairs
    aff.b[j] = u32x2{0u, 0u};
    const int n = n_base + wn * T::WTN + 16 * j + 4 * g;
    if (n < p.N) {
      if (p.gamma) aff.g[j] = *(const u32x2*)(p.gamma + n);
      if (p.beta) aff.b[j] = *(const u32x2*)(p.beta + n);
    }
  }
}

// Per-column fp32 bias of a wave's columns: v[j] holds the 4 columns
// 16j + 4(lane >> 4) .. +3 of the wave's slice (0 past N).
template <class T>
struct Bias {
  f32x4 v[T::FN];
};

template <class T>
__device__ __forceinline__ void load_bias(const GemmParams& p, int n_base, int wn, int lane,
                                          Bias<T>& bias) {
  const int g = lane >> 4;
#pragma unroll
  for (int j = 0; j < T::FN; ++j) {
    const int n = n_base + wn * T::WTN + 16 * j + 4 * g;
    bias.v[j] = n < p.N ? *(const f32x4*)(p.bias + n) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// Scale/shift the accumulators by per-row (mean, rstd) and (AFFINE) the
// per-column gamma/beta, or (BIAS) add a per-column fp32 bias after the row
// scale, or (PRELN) apply rstd * x - mean * rstd * colsum + bias with the
// per-column fp32 colsum/bias loaded per 64-column group, or (BWD) apply
// rstd * x - mean * X with X the staged tile (mean holds the row's c), round
// to bf16 and store the tile.  Each 16-row x
// 64-column piece goes through the wave's LDS staging block so that every
// global store writes whole 128-byte row segments (16 bytes per lane) instead
// of 8-byte pieces of 16 rows.  Exactly T::C_STORES buffer stores per thread
// are issued; rows past M and columns past N fall outside the buffer range
// and are dropped.  Slot i of acc holds fragment i ^ a_xor.
template <class T, bool AFFINE, bool BIAS = false, bool PRELN = false, bool BWD = false>
__device__ __forceinline__ void apply_store(const GemmParams& p, const f32x4 (&acc)[T::FM][T::FN],
                                            const float (&mean)[T::FM], const float (&rstd)[T::FM],
                                            bool use_mean, const Affine<T>& aff,
                                            const Bias<T>& bias, lds_char* lds, int m_base,
                                            int n_base, int wave, int wm, int wn, int lane,
                                            int a_xor = 0) {
  const int l16 = lane & 15, g = lane >> 4;
  const uint32_t stg = (uint32_t)T::STG_OFF + (uint32_t)wave * 2048u;
  // fragment writes: lane (l16, g) of fragment jj holds 4 columns = 8 bytes
  // at byte 32*jj + 8*g of row l16
  const uint32_t w0 = stg + stg_chunk(l16, g >> 1) + 8u * (uint32_t)(g & 1);
  const uint32_t w1 = stg + stg_chunk(l16, 2 + (g >> 1)) + 8u * (uint32_t)(g & 1);
  const uint32_t w2 = stg + stg_chunk(l16, 4 + (g >> 1)) + 8u * (uint32_t)(g & 1);
  const uint32_t w3 = stg + stg_chunk(l16, 6 + (g >> 1)) + 8u * (uint32_t)(g & 1);
  // row reads: lane reads chunk (lane & 7) of rows (lane >> 3) and (lane >> 3) + 8
  const int rr = lane >> 3, rc = lane & 7;
  const uint32_t r0 = stg + stg_chunk(rr, rc), r1 = stg + stg_chunk(rr + 8, rc);
  const uint32_t row_bytes = (uint32_t)p.N * 2u;
  const uint32_t xreg = BWD ? tile_lds_region<T>(wave) : 0u;
#pragma unroll
  for (int q = 0; q < T::FN / 4; ++q) {
    const u32x2* gw = &aff.g[4 * q];
    const u32x2* bw = &aff.b[4 * q];
    const int n_st = n_base + wn * T::WTN + 64 * q + 8 * rc;
    const uint32_t voff_c = n_st < p.N ? 2u * (uint32_t)n_st : kOOB;
    f32x4 pc[PRELN ? 4 : 1], pb[PRELN ? 4 : 1];
    if constexpr (PRELN) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int n = n_base + wn * T::WTN + 64 * q + 16 * jj + 4 * g;
        const bool in = n < p.N;
        pc[jj] = in ? *(const f32x4*)(p.colsum + n) : f32x4{0.f, 0.f, 0.f, 0.f};
        pb[jj] = (in && p.bias) ? *(const f32x4*)(p.bias + n) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
      const float sh = use_mean ? -mean[i] * rstd[i] : 0.f;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const f32x4 x = acc[i][4 * q + jj];
        float y[4];
        if constexpr (AFFINE) {
          y[0] = fmaf(fmaf(x[0], rstd[i], sh), bf16_lo(gw[jj][0]), bf16_lo(bw[jj][0]));
          y[1] = fmaf(fmaf(x[1], rstd[i], sh), bf16_hi(gw[jj][0]), bf16_hi(bw[jj][0]));
          y[2] = fmaf(fmaf(x[2], rstd[i], sh), bf16_lo(gw[jj][1]), bf16_lo(bw[jj][1]));
          y[3] = fmaf(fmaf(x[3], rstd[i], sh), bf16_hi(gw[jj][1]), bf16_hi(bw[jj][1]));
        } else if constexpr (BIAS) {
#pragma unroll
          for (int r = 0; r < 4; ++r) y[r] = fmaf(x[r], rstd[i], bias.v[4 * q + jj][r]);
        } else if constexpr (PRELN) {
#pragma unroll
          for (int r = 0; r < 4; ++r) y[r] = fmaf(x[r], rstd[i], fmaf(sh, pc[jj][r], pb[jj][r]));
        } else if constexpr (BWD) {
          const u32x2 xv = tile_lds_frag<T>(lds, xreg, i, 4 * q + jj, lane);
          y[0] = fmaf(x[0], rstd[i], -mean[i] * bf16_lo(xv[0]));
          y[1] = fmaf(x[1], rstd[i], -mean[i] * bf16_hi(xv[0]));
          y[2] = fmaf(x[2], rstd[i], -mean[i] * bf16_lo(xv[1]));
          y[3] = fmaf(x[3], rstd[i], -mean[i] * bf16_hi(xv[1]));
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) y[r] = fmaf(x[r], rstd[i], sh);
        }
        const uint32_t w = jj == 0 ? w0 : jj == 1 ? w1 : jj == 2 ? w2 : w3;
        *(lds_u32x2*)(lds + w) = u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
      }
      const u32x4 v0 = lds_read16(lds, r0);
      const u32x4 v1 = lds_read16(lds, r1);
      // rows m0 .. m0+15 of the output from a base at row m0 (32-bit offsets
      // stay below 2^31 for any N <= 2^24)
      const int m0 = m_base + wm * T::WTM + 16 * (i ^ a_xor);
      const uint64_t base = (uint64_t)m0 * (uint64_t)p.N;
      const uint64_t total = (uint64_t)p.M * (uint64_t)p.N;
      const uint64_t left = total > base ? (total - base) * 2u : 0u;
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.C + base, left);
      const uint32_t o0 = voff_c == kOOB ? kOOB : voff_c + (uint32_t)rr * row_bytes;
      const uint32_t o1 = voff_c == kOOB ? kOOB : voff_c + (uint32_t)(rr + 8) * row_bytes;
      __builtin_amdgcn_raw_buffer_store_b128(v0, rs, o0, 0, kStoreNT);
      __builtin_amdgcn_raw_buffer_store_b128(v1, rs, o1, 0, kStoreNT);
    }
  }
}

// Row statistics of this tile's slice of each row, from the fp32
// accumulators: LayerNorm (s1, s2) = (tile mean, tile M2 = sum (x - mean)^2),
// two passes over registers; RMSNorm (0, sum x^2).
template <class T, bool LN>
__device__ __forceinline__ void tile_stats(const GemmParams& p, const f32x4 (&acc)[T::FM][T::FN],
                                           lds_char* lds, int n_base, int wm, int wn, int lane,
                                           float (&s1)[T::FM], float (&s2)[T::FM]) {
  const int g = lane >> 4;
  bool colv[T::FN];
#pragma unroll
  for (int j = 0; j < T::FN; ++j) colv[j] = (n_base + wn * T::WTN + 16 * j + 4 * g) < p.N;
  const int n_tile = min(T::BN, p.N - n_base);
  float zero[T::FM];
#pragma unroll
  for (int i = 0; i < T::FM; ++i) zero[i] = 0.f;
  if constexpr (LN) {
    tile_row_sums<T>(acc, colv, 0, zero, s1, lds, wm, wn, lane);
    const float inv = 1.0f / (float)n_tile;
#pragma unroll
    for (int i = 0; i < T::FM; ++i) s1[i] *= inv;
    tile_row_sums<T>(acc, colv, 1, s1, s2, lds, wm, wn, lane);
  } else {
    tile_row_sums<T>(acc, colv, 2, zero, s2, lds, wm, wn, lane);
#pragma unroll
    for (int i = 0; i < T::FM; ++i) s1[i] = 0.f;
  }
}

// Per-row scale of the Lazy Pre-Norm epilogue from the k-loop's sums of
// squares: rstd = 1 / sqrt(sum_k a^2 / K + eps).  Slot i of the wave holds
// fragment i ^ a_xor.  With lazy_split the two waves of a row set each
// summed half of the fragments; they swap their halves through LDS.  The
// workgroup holding column tile 0 also writes rstd_out.
template <class T>
__device__ __forceinline__ void lazy_rstd(const GemmParams& p, const float (&ss)[T::FM],
                                          float (&rstd)[T::FM], lds_char* lds, int m_base,
                                          int tn, int wm, int wn, int lane, int a_xor) {
  const float inv_k = 1.0f / (float)p.K;
  const int l16 = lane & 15, g = lane >> 4;
  float s[T::FM];
#pragma unroll
  for (int i = 0; i < T::FM; ++i) s[i] = reduce_lane_groups(ss[i]);
  if constexpr (lazy_split<T>()) {
    const uint32_t red = T::RED_OFF;
    if (g == 0) {
#pragma unroll
      for (int i = 0; i < T::FM; i += 2)
        *(lds_float*)(lds + red + (wm * T::WTM + 16 * (i ^ a_xor) + l16) * 4) = s[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
      s[i] = *(lds_float*)(lds + red + (wm * T::WTM + 16 * (i ^ a_xor) + l16) * 4);
  }
#pragma unroll
  for (int i = 0; i < T::FM; ++i) {
    rstd[i] = 1.0f / __builtin_sqrtf(fmaf(s[i], inv_k, p.eps));
    const int m = m_base + wm * T::WTM + 16 * (i ^ a_xor) + l16;
    if (p.rstd_out && tn == 0 && wn == 0 && g == 0 && m < p.M) p.rstd_out[m] = rstd[i];
  }
}

// Residual connection of the post-norm epilogues: acc += R over the wave's
// WTM x WTN slice (R staged through the pipeline stages, load_tile_lds),
// then (when S_out is given) S_out = bf16(acc).  Ends with a barrier, after
// which the stages may be reused.  A workgroup reads R only inside its own
// tile and before it writes C or S_out there, so R may be the very buffer
// that C or S_out is.
template <class T>
__device__ __forceinline__ void add_residual(const GemmParams& p, f32x4 (&acc)[T::FM][T::FN],
                                             lds_char* lds, uint32_t lds0, int m_base, int n_base,
                                             int wave, int wm, int wn, int lane) {
  load_tile_lds<T>(p, p.R, lds0, m_base, n_base, wave, wn, lane);
  const uint32_t region = tile_lds_region<T>(wave);
#pragma unroll
  for (int i = 0; i < T::FM; ++i) {
#pragma unroll
    for (int j = 0; j < T::FN; ++j) {
      const u32x2 v = tile_lds_frag<T>(lds, region, i, j, lane);
      acc[i][j][0] += bf16_lo(v[0]);
      acc[i][j][1] += bf16_hi(v[0]);
      acc[i][j][2] += bf16_lo(v[1]);
      acc[i][j][3] += bf16_hi(v[1]);
    }
  }
  __syncthreads();
  if (p.S_out) {
    GemmParams ph = p;
    ph.C = p.S_out;
    float zero[T::FM], one[T::FM];
#pragma unroll
    for (int i = 0; i < T::FM; ++i) { zero[i] = 0.f; one[i] = 1.f; }
    Affine<T> no_aff;
    Bias<T> no_bias;
    apply_store<T, false>(ph, acc, zero, one, false, no_aff, no_bias, lds, m_base, n_base, wave,
                          wm, wn, lane);
  }
}

// Per-row (mean, rstd) that the epilogue applies to a finished tile:
// EPI_NONE (0, 1); EPI_LAZY* (0, rstd of the row of A); EPI_PRE_LN the
// pre-pass statistics of the row of A; EPI_ROW_* the row's statistics over
// the tile (which holds whole rows).  Also writes the
// statistic outputs.  ax: slot permutation of the accumulators (lazy_split).
template <class T, int EPI>
__device__ __forceinline__ void tile_scale(const GemmParams& p, const f32x4 (&acc)[T::FM][T::FN],
                                           const float (&ss)[T::FM], lds_char* lds, int m_base,
                                           int n_base, int tn, int wm, int wn, int lane, int ax,
                                           float (&mean)[T::FM], float (&rstd)[T::FM]) {
#pragma unroll
  for (int i = 0; i < T::FM; ++i) { mean[i] = 0.f; rstd[i] = 1.f; }
  if constexpr (epi_lazy(EPI)) {
    lazy_rstd<T>(p, ss, rstd, lds, m_base, tn, wm, wn, lane, ax);
  } else if constexpr (EPI == EPI_LAZY_BWD) {
    // c = rstd^3 * sum(acc * X) / N, carried in mean[]
    const int l16 = lane & 15;
    float s[T::FM];
    tile_dot_sums<T>(acc, lds, wm * T::WN + wn, wm, wn, lane, s);
    const float inv_n = 1.0f / (float)p.N;
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
      const int m = m_base + wm * T::WTM + 16 * i + l16;
      const float r = m < p.M ? p.row_rstd[m] : 0.f;
      rstd[i] = r;
      mean[i] = r * r * r * s[i] * inv_n;
    }
  } else if constexpr (EPI == EPI_PRE_LN) {
    const int l16 = lane & 15;
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
      const int m = m_base + wm * T::WTM + 16 * i + l16;
      if (m < p.M) {
        mean[i] = p.row_mean[m];
        rstd[i] = p.row_rstd[m];
      }
    }
  } else if constexpr (epi_row(EPI)) {
    const int l16 = lane & 15, g = lane >> 4;
    float s1[T::FM], s2[T::FM];
    tile_stats<T, epi_ln(EPI)>(p, acc, lds, n_base, wm, wn, lane, s1, s2);
    const float inv_n = 1.0f / (float)p.N;
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
      mean[i] = s1[i];
      rstd[i] = 1.0f / __builtin_sqrtf(fmaf(s2[i], inv_n, p.eps));
    }
    if (p.mean_out || p.rstd_out) {
      if (tn == 0 && wn == 0 && g == 0) {
#pragma unroll
        for (int i = 0; i < T::FM; ++i) {
          const int m = m_base + wm * T::WTM + 16 * i + l16;
          if (m < p.M) {
            if (p.mean_out) p.mean_out[m] = mean[i];
            if (p.rstd_out) p.rstd_out[m] = rstd[i];
          }
        }
      }
    }
  }
}

template <class T, int EPI>
__device__ __forceinline__ void tile_store(const GemmParams& p, const f32x4 (&acc)[T::FM][T::FN],
                                           const float (&mean)[T::FM], const float (&rstd)[T::FM],
                                           const Affine<T>& aff, const Bias<T>& bias, lds_char* lds,
                                           int m_base, int n_base, int wave, int wm, int wn,
                                           int lane, int ax) {
  apply_store<T, epi_row(EPI), EPI == EPI_LAZY_BIAS, EPI == EPI_PRE_LN, EPI == EPI_LAZY_BWD>(
      p, acc, mean, rstd, epi_ln(EPI) || EPI == EPI_PRE_LN, aff, bias, lds, m_base, n_base, wave,
      wm, wn, lane, ax);
}

// Per-column data the epilogue needs, loaded before the row statistics so
// that its latency overlaps them.
template <class T, int EPI>
__device__ __forceinline__ void load_columns(const GemmParams& p, int n_base, int wn, int lane,
                                             Affine<T>& aff, Bias<T>& bias) {
  if constexpr (epi_row(EPI)) load_affine<T>(p, n_base, wn, lane, aff);
  if constexpr (EPI == EPI_LAZY_BIAS) load_bias<T>(p, n_base, wn, lane, bias);
}

template <class T, int EPI>
__device__ __forceinline__ void process_tile(const GemmParams& p, lds_char* lds, int tm, int tn) {
  int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / T::WN, wn = wave % T::WN;
  const int m_base = tm * T::BM, n_base = tn * T::BN;
  const int ax = (epi_lazy(EPI) && lazy_split<T>()) ? wn : 0;
  f32x4 acc[T::FM][T::FN];
  float ss[T::FM];
  mainloop<T, epi_lazy(EPI)>(p, acc, ss, lds, lds_addr_of(lds), m_base, n_base, tid);
  if constexpr (epi_res(EPI))
    add_residual<T>(p, acc, lds, lds_addr_of(lds), m_base, n_base, wave, wm, wn, lane);
  if constexpr (EPI == EPI_LAZY_BWD)
    load_tile_lds<T>(p, p.Xin, lds_addr_of(lds), m_base, n_base, wave, wn, lane);
  Affine<T> aff;
  Bias<T> bias;
  load_columns<T, EPI>(p, n_base, wn, lane, aff, bias);
  float mean[T::FM], rstd[T::FM];
  tile_scale<T, EPI>(p, acc, ss, lds, m_base, n_base, tn, wm, wn, lane, ax, mean, rstd);
  tile_store<T, EPI>(p, acc, mean, rstd, aff, bias, lds, m_base, n_base, wave, wm, wn, lane, ax);
  if constexpr (EPI == EPI_LAZY_BWD)
    if (p.scaled_out) write_scaled_rows<T>(p, m_base, tn, p.tiles_n, tid);
}

// Tile order shared by the grids: tiles grouped 4 tile-rows high, column-major
// inside a group, and every XCD (workgroup id mod 8) handed a contiguous run
// of that order so the workgroups resident on one XCD share A and B panels in
// its L2.
__device__ __forceinline__ void grouped_tile(int t, int tiles_m, int tiles_n, int gh, int& tm,
                                             int& tn) {
  const int group = t / (gh * tiles_n);
  const int first = group * gh;
  const int h = min(gh, tiles_m - first);
  const int in_g = t - group * gh * tiles_n;
  tm = first + in_g % h;
  tn = in_g / h;
}

__device__ __forceinline__ int xcd_contiguous(int b, int total) {
  const int per = total / 8, rem = total % 8;
  const int x = b % 8, local = b / 8;
  return x * per + min(x, rem) + local;
}

// One workgroup per output tile (shapes with few tiles, and tiles whose
// output staging shares LDS with the pipeline stages).
template <class T, int EPI>
__global__ void __launch_bounds__(T::NT) gemm_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) char smem[T::LDS];
  lds_char* lds = lds_base(smem);
  const int total = p.tiles_m * p.tiles_n;
  const int t = ordered_tile(p, xcd_contiguous(blockIdx.x, total), total);
  int tm, tn;
  grouped_tile(t, p.tiles_m, p.tiles_n, 4, tm, tn);
  process_tile<T, EPI>(p, lds, tm, tn);
}

// Lazy Pre-Norm's walk of the persistent grid.  Every column tile of a row
// block needs the same row scales, so each workgroup takes "strips" of
// kLazyStrip consecutive column tiles of one row block and computes the sums
// of squares (the Gram MFMAs) only on a strip's first tile; the strip's later
// tiles reuse its rstd, computed from the same rows of A in the same order,
// so the result does not depend on which tile computed it.  Strips are
// numbered over the (row block, column group) grid in groups 8 row blocks
// high, column-major inside a group, and workgroup w walks strips w, w + G,
// ...: the 32 workgroups of an XCD then hold 8 row blocks x 4 column groups,
// which reads as many A and B panels per round (12) as the 4 x 8 blocks of
// the other walks.
constexpr int kLazyStrip = 4;

// The walk's tile number idx (strip idx / kLazyStrip, position idx %
// kLazyStrip) of the workgroup whose first strip is `first`, advanced past
// the positions of short strips (the last column group of a row) that fall
// outside the matrix.  Returns false past the end of the walk.
__device__ __forceinline__ bool lazy_strip_tile(const GemmParams& p, int first, int G, int& idx,
                                                int& tm, int& tn) {
  const int n_cg = (p.tiles_n + kLazyStrip - 1) / kLazyStrip;
  const int strips = p.tiles_m * n_cg;
  while (true) {
    const int s = first + (idx / kLazyStrip) * G;
    if (s >= strips) return false;
    int cg;
    grouped_tile(ordered_tile(p, s, strips), p.tiles_m, n_cg, 8, tm, cg);
    tn = cg * kLazyStrip + idx % kLazyStrip;
    if (tn < p.tiles_n) return true;
    idx = (idx / kLazyStrip + 1) * kLazyStrip;  // rest of a short strip
  }
}

// Persistent grid for Lazy Pre-Norm (EPI_LAZY, EPI_LAZY_BIAS) on the strip
// walk above: a tile whose row block is the previous tile's runs the plain
// k-loop and reuses the previous rstd (kept per accumulator fragment).
template <class T, int EPI>
__device__ __forceinline__ void lazy_persistent(const GemmParams& p, lds_char* lds) {
  const uint32_t lds0 = lds_addr_of(lds);
  const int G = gridDim.x;
  const int first = (G % 8 == 0) ? xcd_contiguous(blockIdx.x, G) : (int)blockIdx.x;
  int idx = 0, tm = 0, tn = 0;
  bool have = lazy_strip_tile(p, first, G, idx, tm, tn);
  if (have) {
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    issue_prologue<T>(p, lds0, tm * T::BM, tn * T::BN, tid);
  }
  int tm_prev = -1;
  float rs_frag[T::FM];  // rstd of this lane's row in accumulator fragment f
  bool first_tile = true;
  while (have) {
    // opaque thread id: keeps lane-dependent addresses from being hoisted
    // out of the tile loop (where they would be spilled)
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / T::WN, wn = wave % T::WN;
    const int m_base = tm * T::BM, n_base = tn * T::BN;
    const bool reuse = tm == tm_prev;
    f32x4 acc[T::FM][T::FN];
    float ss[T::FM];
    float mean[T::FM], rstd[T::FM];
    int ax;
    if (reuse) {
      mainloop<T, false>(p, acc, ss, lds, lds0, m_base, n_base, tid, true, !first_tile);
      ax = 0;
      const int l16 = lane & 15, g = lane >> 4;
#pragma unroll
      for (int i = 0; i < T::FM; ++i) {
        mean[i] = 0.f;
        rstd[i] = rs_frag[i];
        const int m = m_base + wm * T::WTM + 16 * i + l16;
        if (p.rstd_out && tn == 0 && wn == 0 && g == 0 && m < p.M) p.rstd_out[m] = rstd[i];
      }
    } else {
      mainloop<T, true>(p, acc, ss, lds, lds0, m_base, n_base, tid, true, !first_tile);
      ax = lazy_split<T>() ? wn : 0;
      tile_scale<T, EPI>(p, acc, ss, lds, m_base, n_base, tn, wm, wn, lane, ax, mean, rstd);
#pragma unroll
      for (int i = 0; i < T::FM; ++i) rs_frag[i ^ ax] = rstd[i];
      tm_prev = tm;
    }
    Affine<T> aff;
    Bias<T> bias;
    load_columns<T, EPI>(p, n_base, wn, lane, aff, bias);
    int idx2 = idx + 1, tm2 = 0, tn2 = 0;
    const bool have2 = lazy_strip_tile(p, first, G, idx2, tm2, tn2);
    if (have2) issue_prologue<T>(p, lds0, tm2 * T::BM, tn2 * T::BN, tid);
    tile_store<T, EPI>(p, acc, mean, rstd, aff, bias, lds, m_base, n_base, wave, wm, wn, lane, ax);
    idx = idx2;
    tm = tm2;
    tn = tn2;
    have = have2;
    first_tile = false;
  }
}

// Persistent grid: gridDim.x workgroups (at most one round of resident
// workgroups) walk the tile order with stride gridDim.x.  After a tile's
// k-loop a workgroup computes the tile's row scales, issues the LDS transfers
// that start its next tile, then scales and stores the finished tile, so the
// next tile's first k-tiles stream in behind the epilogue.  All epilogues
// whose tile holds what it needs (EPI_NONE, EPI_LAZY*, EPI_ROW_*, EPI_PRE_LN).
// KW (plain GEMM): the tiles of every second pass over the tile order
// (gridDim.x tiles) walk the k-tiles downwards, as in the cross-workgroup
// grid.  The direction follows the tile's place in the natural order, so a
// permuted order (a diagnostic) gives the same sums.
template <class T, int EPI, bool KW = false>
__global__ void __launch_bounds__(T::NT) gemm_persistent_kernel(GemmParams p) {
  static_assert(!KW || EPI == EPI_NONE, "alternating k-walk: plain GEMM only");
  static_assert(T::STG_OWN, "persistent tiles need their own output staging");
  __shared__ __attribute__((aligned(16))) char smem[T::LDS];
  lds_char* lds = lds_base(smem);
  if constexpr (epi_lazy(EPI)) {
    lazy_persistent<T, EPI>(p, lds);
    return;
  }
  const uint32_t lds0 = lds_addr_of(lds);
  const int G = gridDim.x;
  const int total = p.tiles_m * p.tiles_n;
  const int first = (G % 8 == 0) ? xcd_contiguous(blockIdx.x, G) : (int)blockIdx.x;
  if (first < total) {
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    int tm, tn;
    const int j = ordered_tile(p, first, total);
    grouped_tile(j, p.tiles_m, p.tiles_n, 4, tm, tn);
    issue_prologue<T>(p, lds0, tm * T::BM, tn * T::BN, tid, KW && ((j / G) & 1));
  }
  // cross-tile prefetch (both k-loop shapes): not for the epilogues that
  // stage data through the stages (the pre-norm epilogue's per-row loads
  // wait for the prefetched transfers, which are older, but the next k-loop
  // then starts on landed k-tiles)
  constexpr bool kCross = (EPI == EPI_NONE || EPI == EPI_PRE_LN) && !scale_ahead<T>();
  const int nk = (p.K + T::BK - 1) / T::BK;
  int srot = 0;
  for (int t = first; t < total; t += G) {
    // opaque thread id: keeps lane-dependent addresses from being hoisted
    // out of the tile loop (where they would be spilled)
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / T::WN, wn = wave % T::WN;
    int tm, tn;
    const int j = ordered_tile(p, t, total);
    grouped_tile(j, p.tiles_m, p.tiles_n, 4, tm, tn);
    const int m_base = tm * T::BM, n_base = tn * T::BN;
    const int ax = (epi_lazy(EPI) && lazy_split<T>()) ? wn : 0;
    const bool has_next = t + G < total;
    int tm2 = 0, tn2 = 0, j2 = 0;
    if (has_next) {
      j2 = ordered_tile(p, t + G, total);
      grouped_tile(j2, p.tiles_m, p.tiles_n, 4, tm2, tn2);
    }
    const bool xt = kCross && has_next && nk >= T::STAGES;
    f32x4 acc[T::FM][T::FN];
    float ss[T::FM];
    const bool rev = KW && ((j / G) & 1), nx_rev = KW && has_next && ((j2 / G) & 1);
    if (rev)
      mainloop<T, false, KW>(p, acc, ss, lds, lds0, m_base, n_base, tid, true, t != first, srot,
                             xt ? tm2 * T::BM : -1, tn2 * T::BN, nx_rev);
    else
      mainloop<T, epi_lazy(EPI)>(p, acc, ss, lds, lds0, m_base, n_base, tid, true, t != first,
                                 srot, xt ? tm2 * T::BM : -1, tn2 * T::BN, nx_rev);
    if constexpr (epi_res(EPI))
      add_residual<T>(p, acc, lds, lds0, m_base, n_base, wave, wm, wn, lane);
    Affine<T> aff;
    Bias<T> bias;
    load_columns<T, EPI>(p, n_base, wn, lane, aff, bias);
    float mean[T::FM], rstd[T::FM];
    tile_scale<T, EPI>(p, acc, ss, lds, m_base, n_base, tn, wm, wn, lane, ax, mean, rstd);
    if (has_next && !xt) issue_prologue<T>(p, lds0, tm2 * T::BM, tn2 * T::BN, tid, nx_rev);
    tile_store<T, EPI>(p, acc, mean, rstd, aff, bias, lds, m_base, n_base, wave, wm, wn, lane,
                       ax);
    srot = xt ? (srot + nk) % T::STAGES : 0;
  }
}

// ---------------------------------------------------------------------------
// Cross-workgroup row norm (rows wider than one tile).
//
// Persistent grid of R * tiles_n workgroups, no more than the device holds
// at once.  Round `it` covers the complete row blocks it*R .. it*R+R-1, one
// column tile per workgroup.  For its tile a workgroup
//   1. runs the k-loop;
//   2. reduces its slice of every row from the fp32 accumulators and
//      publishes one (mean_t, M2_t) pair -- or (0, sum x^2) -- per row;
//   3. issues the LDS transfers that start its next tile;
//   4. merges, for its own share of the row block's rows (BM / tiles_n of
//      them), the partials of all column tiles (Chan's update for mean/M2, in
//      a fixed order) and publishes each row's (mean, rstd);
//   5. reads (mean, rstd) of all BM rows, normalizes the accumulators still
//      held in registers and stores the tile once.
// Steps 4 and 5 poll until the entries carry the call's tag.  Every wait
// points at workgroups of the same round.  The grid fits the device, so once
// other work on the device drains all of its workgroups are resident and
// every wait ends; the polls are bounded (about a second) and a wait that
// gives up raises the error word, so a call that overlaps another such grid
// on the same device reports an error instead of hanging.  Entries are
// written and read with agent-scope (sc1) accesses, which bypass the per-XCD
// L2.

// sc1 buffer views of a slot's partials and final statistics (R slots,
// parts partials per row).
template <class T>
__device__ __forceinline__ int xwg_parts(const GemmParams& p) { return p.tiles_n; }
template <class T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t xwg_part_rsrc(const GemmParams& p, int slot) {
  const size_t blk = (size_t)T::BM * xwg_parts<T>(p) * 16u;
  return make_rsrc(p.ws + XwgLayout::kPart + (size_t)slot * blk, blk);
}
template <class T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t xwg_fin_rsrc(const GemmParams& p, int slot,
                                                              int slots) {
  const size_t blk = (size_t)T::BM * 16u;
  return make_rsrc(p.ws + XwgLayout::fin_off(slots, xwg_parts<T>(p), T::BM) + (size_t)slot * blk,
                   blk);
}

// 16-byte sc1 load of a tagged entry, repeated until both halves carry `tag`.
// If the bounded wait gives up, the error word is raised and the entry reads
// as NaN, so that every statistic and output element that depends on it is
// NaN: an output of a failed exchange can never look plausible.
__device__ __forceinline__ u32x4 xwg_poll(const GemmParams& p, __amdgpu_buffer_rsrc_t rs,
                                          uint32_t off, uint32_t tag) {
  u32x4 v;
  int spins = 0;
  while (true) {
    v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 16);
    if (v[1] == tag && v[3] == tag) break;
    if (++spins > p.spin_limit) {
      store_agent((int*)(p.ws + XwgLayout::kErr), 1);
      v = u32x4{0x7FC00000u, tag, 0x7FC00000u, tag};
      break;
    }
    __builtin_amdgcn_s_sleep(1);
    asm volatile("" ::: "memory");  // reload on every pass
  }
  return v;
}

// Chan's combination of two (count, mean, M2) summaries, first one first.
__device__ __forceinline__ void chan_combine(float& n_a, float& mu_a, float& m2_a, float n_b,
                                             float mu_b, float m2_b) {
  const float nn = n_a + n_b;
  const float w = nn > 0.f ? n_b / nn : 0.f;
  const float d = mu_b - mu_a;
  mu_a = fmaf(d, w, mu_a);
  m2_a = m2_a + m2_b + d * d * (n_a * w);
  n_a = nn;
}

// Step 2: the workgroup's slice of every row (its BN columns), reduced over
// the tile: LayerNorm (mean_t, M2_t), RMSNorm (0, sum x^2); BWD (0, sum
// acc * X), X the staged forward input.
template <class T, bool LN, bool BWD = false>
__device__ __forceinline__ void xwg_publish(const GemmParams& p, const f32x4 (&acc)[T::FM][T::FN],
                                            lds_char* lds, int slot, int tn, int tid,
                                            uint32_t tag) {
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / T::WN, wn = wave % T::WN;
  const int l16 = lane & 15, g = lane >> 4;
  float s1[T::FM], s2[T::FM];
  if constexpr (BWD) {
    tile_dot_sums<T>(acc, lds, wave, wm, wn, lane, s2);
#pragma unroll
    for (int i = 0; i < T::FM; ++i) s1[i] = 0.f;
  } else {
    tile_stats<T, LN>(p, acc, lds, tn * T::BN, wm, wn, lane, s1, s2);
  }
  const int parts = xwg_parts<T>(p);
  const __amdgpu_buffer_rsrc_t prs = xwg_part_rsrc<T>(p, slot);
  if (wn == 0 && g == 0) {
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
      const int r = wm * T::WTM + 16 * i + l16;
      const u32x4 v = {__float_as_uint(s1[i]), tag, __float_as_uint(s2[i]), tag};
      __builtin_amdgcn_raw_buffer_store_b128(v, prs, (uint32_t)(r * parts + tn) * 16u, 0, 16);
    }
  }
}

// Step 4.  Rows r0 .. r1-1 of the row block belong to this workgroup.  A row
// is merged by `cpl` lanes (a power of two, at most 64, at least tiles_n
// when tiles_n <= 64): lane li takes column tiles li, li+cpl, ... in order,
// then the lanes combine pairwise, lower lanes first.  BWD: the row's plain
// sum is published as is (in the rstd slot).
template <class T, bool LN, bool BWD = false>
__device__ __forceinline__ void xwg_merge_rows(const GemmParams& p, int slot, int slots, int tm,
                                               int tn, int tid, uint32_t tag) {
  constexpr int NW = T::NT / 64;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tiles_n = p.tiles_n;
  const int parts = xwg_parts<T>(p);
  const int rpw = (T::BM + tiles_n - 1) / tiles_n;
  const int r0 = tn * rpw, r1 = min(T::BM, r0 + rpw);
  int cpl = 1;
  while (cpl < parts && cpl < 64) cpl <<= 1;
  const int rows_per_pass = 64 / cpl;
  const int sub = lane / cpl, li = lane % cpl;
  const __amdgpu_buffer_rsrc_t prs = xwg_part_rsrc<T>(p, slot);
  const __amdgpu_buffer_rsrc_t frs = xwg_fin_rsrc<T>(p, slot, slots);
  const float inv_n = 1.0f / (float)p.N;
  for (int rb = r0 + wave * rows_per_pass; rb < r1; rb += NW * rows_per_pass) {
    const int row = rb + sub;
    const bool active = row < r1;
    float n = 0.f, mu = 0.f, m2 = 0.f;
    if (active) {
      for (int t = li; t < parts; t += cpl) {
        const u32x4 v = xwg_poll(p, prs, (uint32_t)(row * parts + t) * 16u, tag);
        if constexpr (LN) {
          chan_combine(n, mu, m2, (float)min(T::BN, p.N - t * T::BN), __uint_as_float(v[0]),
                       __uint_as_float(v[2]));
        } else {
          m2 += __uint_as_float(v[2]);
        }
      }
    }
    for (int o = 1; o < cpl; o <<= 1) {
      const float n_o = xor_shfl(n, o), mu_o = xor_shfl(mu, o), m2_o = xor_shfl(m2, o);
      if constexpr (LN) {
        if (li & o) {  // this lane holds the upper half: combine (partner, self)
          float na = n_o, ma = mu_o, qa = m2_o;
          chan_combine(na, ma, qa, n, mu, m2);
          n = na; mu = ma; m2 = qa;
        } else {
          chan_combine(n, mu, m2, n_o, mu_o, m2_o);
        }
      } else {
        m2 = (li & o) ? m2_o + m2 : m2 + m2_o;
      }
    }
    if (active && li == 0) {
      const float r = BWD ? m2 : 1.0f / __builtin_sqrtf(fmaf(m2, inv_n, p.eps));
      const float mean = LN ? mu : 0.f;
      const u32x4 v = {__float_as_uint(mean), tag, __float_as_uint(r), tag};
      __builtin_amdgcn_raw_buffer_store_b128(v, frs, (uint32_t)row * 16u, 0, 16);
      const int m = tm * T::BM + row;
      if (!BWD && m < p.M) {
        if (p.mean_out) p.mean_out[m] = mean;
        if (p.rstd_out) p.rstd_out[m] = r;
      }
    }
  }
}

// KW: the k-loops of odd rounds walk the k-tiles downwards, so that a round
// starts on the k-tiles of B (and A) that the last one read most recently --
// those still in the Infinity Cache when one round's operands exceed it.
template <class T, bool LN, bool RES = false, bool BWD = false, bool KW = false>
__global__ void __launch_bounds__(T::NT) gemm_xwg_kernel(GemmParams p) {
  static_assert(!KW || (!RES && !BWD), "alternating k-walk: plain norm epilogues only");
  static_assert(T::STG_OWN, "persistent tiles need their own output staging");
  __shared__ __attribute__((aligned(16))) char smem[T::LDS];
  lds_char* lds = lds_base(smem);
  const uint32_t lds0 = lds_addr_of(lds);
  const int G = gridDim.x;
  const int R = G / p.tiles_n;
  const int j = ordered_tile(p, (G % 8 == 0) ? xcd_contiguous(blockIdx.x, G) : (int)blockIdx.x, G);
  const int gh = (R % 4 == 0) ? 4 : ((R % 2 == 0) ? 2 : 1);
  int rb_in, tn;
  grouped_tile(j, R, p.tiles_n, gh, rb_in, tn);
  // tag base of this call; round `it` tags its entries base + 1 + it
  const uint32_t base =
      __builtin_amdgcn_readfirstlane((uint32_t)load_agent((const int*)(p.ws + XwgLayout::kTag)));
  if (rb_in < p.tiles_m) {
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    issue_prologue<T>(p, lds0, rb_in * T::BM, tn * T::BN, tid);
  }
  // cross-tile prefetch of the next round's first k-tiles inside the k-loop:
  // not with the residual or the backward, which stage data through the
  // stages after the k-loop, nor on the two-stage 64-deep tiles, where the
  // exchange's polls, waiting behind the prefetched transfers, start later
  // (measured ~1 % slower on 8192x16384x8192 with B stored [N, K])
  constexpr bool kCross = T::KK == 1 && !RES && !BWD && !scale_ahead<T>();
  const int nk = (p.K + T::BK - 1) / T::BK;
  int srot = 0;
  for (int it = 0; it < p.iters; ++it) {
    const int tm = it * R + rb_in;
    if (tm >= p.tiles_m) break;
    // opaque thread id: keeps lane-dependent addresses from being hoisted
    // out of the tile loop (where they would be spilled)
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / T::WN, wn = wave % T::WN;
    const int l16 = lane & 15;
    const int m_base = tm * T::BM, n_base = tn * T::BN;
    const uint32_t tag = base + 1u + (uint32_t)it;
    f32x4 acc[T::FM][T::FN];
    float ss[T::FM];
    // (BWD: the previous tile's output stores precede this tile's first
    // transfers, so they are not counted after them)
    const bool xt = kCross && tm + R < p.tiles_m && nk >= T::STAGES;
    const bool rev = KW && (it & 1), nx_rev = KW && !(it & 1);
    if (rev)
      mainloop<T, false, KW>(p, acc, ss, lds, lds0, m_base, n_base, tid, true, it > 0, srot,
                             xt ? (tm + R) * T::BM : -1, n_base, nx_rev);
    else
      mainloop<T, false>(p, acc, ss, lds, lds0, m_base, n_base, tid, true, !BWD && it > 0, srot,
                         xt ? (tm + R) * T::BM : -1, n_base, nx_rev);
    if constexpr (RES) add_residual<T>(p, acc, lds, lds0, m_base, n_base, wave, wm, wn, lane);
    if constexpr (BWD) load_tile_lds<T>(p, p.Xin, lds0, m_base, n_base, wave, wn, lane);
    xwg_publish<T, LN, BWD>(p, acc, lds, rb_in, tn, tid, tag);
    Affine<T> aff;
    if constexpr (!BWD) {
      load_affine<T>(p, n_base, wn, lane, aff);
      if (tm + R < p.tiles_m && !xt)
        issue_prologue<T>(p, lds0, (tm + R) * T::BM, n_base, tid, nx_rev);
    }
    xwg_merge_rows<T, LN, BWD>(p, rb_in, R, tm, tn, tid, tag);
    // (regrouped weight gradient: this workgroup's rows of rstd * dC, while
    // the other workgroups of the row block merge)
    if constexpr (BWD)
      if (p.scaled_out) write_scaled_rows<T>(p, m_base, tn, p.tiles_n, tid);
    // step 5: (mean, rstd) of this wave's rows; BWD: (c, rstd) from the row's
    // sum of acc * X and the saved rstd
    const __amdgpu_buffer_rsrc_t frs = xwg_fin_rsrc<T>(p, rb_in, R);
    float mean[T::FM], rstd[T::FM];
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
      const u32x4 v = xwg_poll(p, frs, (uint32_t)(wm * T::WTM + 16 * i + l16) * 16u, tag);
      if constexpr (BWD) {
        const int m = m_base + wm * T::WTM + 16 * i + l16;
        const float r = m < p.M ? p.row_rstd[m] : 0.f;
        rstd[i] = r;
        mean[i] = r * r * r * __uint_as_float(v[2]) * (1.0f / (float)p.N);
      } else {
        mean[i] = __uint_as_float(v[0]);
        rstd[i] = __uint_as_float(v[2]);
      }
    }
    Bias<T> no_bias;
    apply_store<T, !BWD, false, false, BWD>(p, acc, mean, rstd, LN, aff, no_bias, lds, m_base,
                                            n_base, wave, wm, wn, lane);
    if constexpr (BWD) {
      // every wave has read its staged X: the stages may take the next tile
      if (tm + R < p.tiles_m) {
        __syncthreads();
        issue_prologue<T>(p, lds0, (tm + R) * T::BM, n_base, tid);
      }
    }
    srot = xt ? (srot + nk) % T::STAGES : 0;
  }
  // the last workgroup to finish advances the call counter (every workgroup
  // read it at its start)
  if (threadIdx.x == 0) {
    int* done = (int*)(p.ws + XwgLayout::kDone);
    if (add_agent(done, 1) == G - 1) {
      store_agent((int*)(p.ws + XwgLayout::kTag), (int)(base + (uint32_t)p.iters));
      store_agent(done, 0);
    }
  }
}

}  // namespace ng
