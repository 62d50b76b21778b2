// bf16 MFMA GEMM with fused row-norm epilogues for gfx950.
//
// One kernel template serves four epilogues:
//   EPI_NONE      C = A @ B                               (unfused baseline GEMM)
//   EPI_LAZY      C = (A @ B) * rstd(A)                   (Lazy Pre-Norm)
//   EPI_ROW_LOCAL C = norm(A @ B), whole row in one workgroup (N <= BN)
//   EPI_ROW_XWG   C = norm(A @ B), row split over workgroups; per-row fp32
//                 partials merged through a workspace (persistent grid)
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
// Data layout in LDS per pipeline stage (BK = 64):
//   A tile  [BM][64] bf16, 128-byte rows; 16-byte chunk c of row m is stored
//           at chunk c ^ (m & 7) (conflict-free 16-byte fragment reads).
//   B tile  KN: [64][BN] bf16 rows (N contiguous), read with the transposing
//           LDS read; 32-byte pair p of row k stored at p ^ h(k).
//           NK: [BN][64] bf16, same layout as A.
// MFMA: v_mfma_f32_16x16x32_bf16 with B as the first operand and A as the
// second, so each lane's accumulators hold four consecutive columns of one
// output row: acc[i][j][r] = C[m0 + 16i + (lane & 15)][n0 + 16j + 4(lane >> 4) + r].
#pragma once

#include "ng_device.h"

namespace ng {

constexpr int BK = 64;

enum Epi { EPI_NONE = 0, EPI_LAZY = 1, EPI_ROW_LOCAL = 2, EPI_ROW_XWG = 3 };
enum NormKind { NORM_RMS = 0, NORM_LAYER = 1 };

// Workspace layout for EPI_ROW_XWG (byte offsets).
//   [0]            int error word (0 = ok, 1 = a wait timed out)
//   [256 + 4 rb]   int arrive[row_blocks]
//   [..]           int depart[row_blocks]
//   [part_off]     float2 partial[row_blocks][tiles_n][BM]
struct XwgLayout {
  static constexpr size_t kErr = 0;
  static constexpr size_t kCnt = 256;
  static __host__ __device__ size_t part_off(int row_blocks) {
    size_t end = kCnt + 8u * (size_t)row_blocks;
    return (end + 255) & ~(size_t)255;
  }
  static __host__ __device__ size_t bytes(int row_blocks, int tiles_n, int bm) {
    return part_off(row_blocks) + (size_t)row_blocks * tiles_n * bm * 8u;
  }
};

struct GemmParams {
  const uint16_t* A;
  const uint16_t* B;
  uint16_t* C;
  const uint16_t* gamma;
  const uint16_t* beta;
  float* mean_out;
  float* rstd_out;
  char* ws;
  int M, N, K;
  float eps;
  int norm_kind;
  int tiles_m, tiles_n;
  int iters;       // persistent grid: tile rounds
  int spin_limit;  // persistent grid: bounded wait (iterations of ~1 us)
};

template <int BM_, int BN_, int WM_, int WN_, bool KN_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr bool KN = KN_;
  static constexpr int NT = 64 * WM * WN;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / 16, FN = WTN / 16;
  static constexpr int A_BYTES = BM * BK * 2;
  static constexpr int B_BYTES = BN * BK * 2;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int A_PER = BM * BK / 8 / NT;  // 16-byte chunks per thread
  static constexpr int B_PER = BN * BK / 8 / NT;
  static constexpr int RED_BYTES = WN * BM * 4;   // cross-wave row partials
  static constexpr int FIN_BYTES = BM * 8;        // per-row (mean, rstd)
  static constexpr int LDS = 2 * STAGE + RED_BYTES + FIN_BYTES;
  static_assert(BM % (16 * WM) == 0 && BN % (16 * WN) == 0, "wave tile");
  static_assert((BM * BK / 8) % NT == 0 && (BN * BK / 8) % NT == 0, "loader split");
  static_assert((BN & (BN - 1)) == 0 && BN >= 16, "BN power of two");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

// Swizzle of the B (KN) tile: the 16 rows a transposing read touches at once
// (k = 8g + i, g, i in 0..3) land on distinct 32-byte bank groups.
template <int BN>
__device__ __forceinline__ uint32_t b_row_swz(int k) {
  return (uint32_t)(((k & 3) | (((k >> 3) & 3) << 2)) & (BN / 16 - 1));
}

template <class T>
struct Stage {
  u32x4 a[T::A_PER];
  u32x4 b[T::B_PER];
};

// Global -> registers for k-tile starting at k0.  Chunks outside the matrix
// (row >= rows valid, k >= K, n >= N) read as zero.
template <class T>
__device__ __forceinline__ void load_tile(Stage<T>& st, const uint16_t* __restrict__ Ablk,
                                          const uint16_t* __restrict__ Bblk, int m_valid,
                                          int n_valid, int K, int N, int k0, int tid) {
#pragma unroll
  for (int i = 0; i < T::A_PER; ++i) {
    int q = tid + i * T::NT;
    int row = q >> 3, c = q & 7;
    int k = k0 + 8 * c;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row < m_valid && k < K) v = *(const u32x4*)(Ablk + (size_t)row * K + k);
    st.a[i] = v;
  }
  if constexpr (T::KN) {
    constexpr int CPR = T::BN / 8;
#pragma unroll
    for (int i = 0; i < T::B_PER; ++i) {
      int q = tid + i * T::NT;
      int kr = q / CPR, c = q % CPR;
      int k = k0 + kr;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (k < K && 8 * c < n_valid) v = *(const u32x4*)(Bblk + (size_t)k * N + 8 * c);
      st.b[i] = v;
    }
  } else {
#pragma unroll
    for (int i = 0; i < T::B_PER; ++i) {
      int q = tid + i * T::NT;
      int row = q >> 3, c = q & 7;
      int k = k0 + 8 * c;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row < n_valid && k < K) v = *(const u32x4*)(Bblk + (size_t)row * K + k);
      st.b[i] = v;
    }
  }
}

template <class T>
__device__ __forceinline__ void store_tile(const Stage<T>& st, lds_char* lds, uint32_t stage_off,
                                           int tid) {
#pragma unroll
  for (int i = 0; i < T::A_PER; ++i) {
    int q = tid + i * T::NT;
    int row = q >> 3, c = q & 7;
    lds_write16(lds, stage_off + row * 128 + ((c ^ (row & 7)) << 4), st.a[i]);
  }
  if constexpr (T::KN) {
    constexpr int CPR = T::BN / 8;
#pragma unroll
    for (int i = 0; i < T::B_PER; ++i) {
      int q = tid + i * T::NT;
      int kr = q / CPR, c = q % CPR;
      uint32_t pc = (uint32_t)c ^ (b_row_swz<T::BN>(kr) << 1);
      lds_write16(lds, stage_off + T::A_BYTES + kr * (T::BN * 2) + (pc << 4), st.b[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < T::B_PER; ++i) {
      int q = tid + i * T::NT;
      int row = q >> 3, c = q & 7;
      lds_write16(lds, stage_off + T::A_BYTES + row * 128 + ((c ^ (row & 7)) << 4), st.b[i]);
    }
  }
}

// MFMAs for one BK=64 stage: two k32 sub-steps.
template <class T, bool LAZY>
__device__ __forceinline__ void compute_stage(f32x4 (&acc)[T::FM][T::FN], float (&ss)[T::FM],
                                              lds_char* lds, uint32_t stage_off, int wm, int wn,
                                              int lane) {
  const int l16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    u32x4 af[T::FM], bfr[T::FN];
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
      int row = wm * T::WTM + 16 * i + l16;
      int c = kk * 4 + g;
      af[i] = lds_read16(lds, stage_off + row * 128 + ((c ^ (row & 7)) << 4));
    }
#pragma unroll
    for (int j = 0; j < T::FN; ++j) {
      if constexpr (T::KN) {
        int ncol = wn * T::WTN + 16 * j + 4 * (l16 & 3);
        uint32_t c = (uint32_t)(ncol >> 3);
        uint32_t half = (uint32_t)(l16 & 1) << 3;
        int kr0 = kk * 32 + 8 * g + (l16 >> 2);
        int kr1 = kr0 + 4;
        uint32_t o0 = stage_off + T::A_BYTES + kr0 * (T::BN * 2) +
                      ((c ^ (b_row_swz<T::BN>(kr0) << 1)) << 4) + half;
        uint32_t o1 = stage_off + T::A_BYTES + kr1 * (T::BN * 2) +
                      ((c ^ (b_row_swz<T::BN>(kr1) << 1)) << 4) + half;
        u32x2 lo = lds_read_tr16(lds, o0);
        u32x2 hi = lds_read_tr16(lds, o1);
        bfr[j] = u32x4{lo[0], lo[1], hi[0], hi[1]};
      } else {
        int row = wn * T::WTN + 16 * j + l16;
        int c = kk * 4 + g;
        bfr[j] = lds_read16(lds, stage_off + T::A_BYTES + row * 128 + ((c ^ (row & 7)) << 4));
      }
    }
    if constexpr (LAZY) {
#pragma unroll
      for (int i = 0; i < T::FM; ++i) ss[i] = sumsq_bf16x8(af[i], ss[i]);
    }
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
      for (int j = 0; j < T::FN; ++j) acc[i][j] = mfma_16x16x32(bfr[j], af[i], acc[i][j]);
  }
}

// Full k-loop for the tile at (m_base, n_base): two LDS stages, the next
// k-tile's global loads in flight during the current stage's MFMAs.
template <class T, bool LAZY>
__device__ __forceinline__ void mainloop(const GemmParams& p, f32x4 (&acc)[T::FM][T::FN],
                                         float (&ss)[T::FM], lds_char* lds, int m_base,
                                         int n_base) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / T::WN, wn = wave % T::WN;
#pragma unroll
  for (int i = 0; i < T::FM; ++i) {
    ss[i] = 0.f;
#pragma unroll
    for (int j = 0; j < T::FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int m_valid = min(T::BM, p.M - m_base);
  const int n_valid = min(T::BN, p.N - n_base);
  const uint16_t* Ablk = p.A + (size_t)m_base * p.K;
  const uint16_t* Bblk = T::KN ? p.B + n_base : p.B + (size_t)n_base * p.K;
  const int nk = (p.K + BK - 1) / BK;

  Stage<T> st;
  load_tile<T>(st, Ablk, Bblk, m_valid, n_valid, p.K, p.N, 0, tid);
  store_tile<T>(st, lds, 0, tid);
  if (nk > 1) load_tile<T>(st, Ablk, Bblk, m_valid, n_valid, p.K, p.N, BK, tid);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const uint32_t cur = (uint32_t)(kt & 1) * T::STAGE;
    const uint32_t nxt = (uint32_t)((kt + 1) & 1) * T::STAGE;
    compute_stage<T, LAZY>(acc, ss, lds, cur, wm, wn, lane);
    if (kt + 1 < nk) {
      store_tile<T>(st, lds, nxt, tid);
      if (kt + 2 < nk) load_tile<T>(st, Ablk, Bblk, m_valid, n_valid, p.K, p.N, (kt + 2) * BK, tid);
    }
    __syncthreads();
  }
}

// Sum over the 4 lane groups sharing (lane & 15): a row's partial over this
// wave's columns (or, for the lazy sum of squares, over this wave's k-groups).
__device__ __forceinline__ float reduce_lane_groups(float v) {
  v += xor_shfl(v, 16);
  v += xor_shfl(v, 32);
  return v;
}

// Per-row sums of this workgroup's accumulators over its valid columns,
// combined across the WN waves that share rows through LDS (fixed order).
// mode 0: sum x;  mode 1: sum (x - center[i])^2;  mode 2: sum x^2.
// Result: out[i] for row wm*WTM + 16i + (lane & 15), same in all lanes of the group.
template <class T>
__device__ __forceinline__ void tile_row_sums(const f32x4 (&acc)[T::FM][T::FN],
                                              const bool (&colv)[T::FN], int mode,
                                              const float (&center)[T::FM], float (&out)[T::FM],
                                              lds_char* lds, int wm, int wn, int lane) {
  const uint32_t red = 2 * T::STAGE;
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

// Scale/shift the accumulators by per-row (mean, rstd) and the per-column
// affine, round to bf16 and store the valid part of the tile.
template <class T>
__device__ __forceinline__ void apply_store(const GemmParams& p, f32x4 (&acc)[T::FM][T::FN],
                                            const float (&mean)[T::FM], const float (&rstd)[T::FM],
                                            bool use_mean, int m_base, int n_base, int wm, int wn,
                                            int lane) {
  const int l16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int j = 0; j < T::FN; ++j) {
    const int n = n_base + wn * T::WTN + 16 * j + 4 * g;
    if (n >= p.N) continue;
    float gm[4] = {1.f, 1.f, 1.f, 1.f}, bt[4] = {0.f, 0.f, 0.f, 0.f};
    if (p.gamma) {
      u32x2 w = *(const u32x2*)(p.gamma + n);
      gm[0] = bf16_lo(w[0]); gm[1] = bf16_hi(w[0]); gm[2] = bf16_lo(w[1]); gm[3] = bf16_hi(w[1]);
    }
    if (p.beta) {
      u32x2 w = *(const u32x2*)(p.beta + n);
      bt[0] = bf16_lo(w[0]); bt[1] = bf16_hi(w[0]); bt[2] = bf16_lo(w[1]); bt[3] = bf16_hi(w[1]);
    }
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
      const int m = m_base + wm * T::WTM + 16 * i + l16;
      if (m >= p.M) continue;
      const float sh = use_mean ? -mean[i] * rstd[i] : 0.f;
      float y[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) y[r] = fmaf(fmaf(acc[i][j][r], rstd[i], sh), gm[r], bt[r]);
      u32x2 o = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
      *(u32x2*)(p.C + (size_t)m * p.N + n) = o;
    }
  }
}

template <class T, int EPI>
__device__ __forceinline__ void process_tile(const GemmParams& p, lds_char* lds, int tm, int tn) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / T::WN, wn = wave % T::WN;
  const int l16 = lane & 15, g = lane >> 4;
  const int m_base = tm * T::BM, n_base = tn * T::BN;

  f32x4 acc[T::FM][T::FN];
  float ss[T::FM];
  mainloop<T, EPI == EPI_LAZY>(p, acc, ss, lds, m_base, n_base);

  float mean[T::FM], rstd[T::FM];
  if constexpr (EPI == EPI_NONE) {
#pragma unroll
    for (int i = 0; i < T::FM; ++i) { mean[i] = 0.f; rstd[i] = 1.f; }
    GemmParams q = p;
    q.gamma = nullptr;
    q.beta = nullptr;
    apply_store<T>(q, acc, mean, rstd, false, m_base, n_base, wm, wn, lane);
  } else if constexpr (EPI == EPI_LAZY) {
    const float inv_k = 1.0f / (float)p.K;
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
      float s = reduce_lane_groups(ss[i]);
      rstd[i] = 1.0f / __builtin_sqrtf(fmaf(s, inv_k, p.eps));
      mean[i] = 0.f;
      const int m = m_base + wm * T::WTM + 16 * i + l16;
      if (p.rstd_out && tn == 0 && wn == 0 && g == 0 && m < p.M) p.rstd_out[m] = rstd[i];
    }
    GemmParams q = p;
    q.gamma = nullptr;
    q.beta = nullptr;
    apply_store<T>(q, acc, mean, rstd, false, m_base, n_base, wm, wn, lane);
  } else {
    // Row statistics of this tile's slice of each row.
    bool colv[T::FN];
    int n_tile = 0;  // valid columns in this tile
#pragma unroll
    for (int j = 0; j < T::FN; ++j) colv[j] = (n_base + wn * T::WTN + 16 * j + 4 * g) < p.N;
    n_tile = min(T::BN, p.N - n_base);
    const bool ln = p.norm_kind == NORM_LAYER;
    float zero[T::FM], s1[T::FM], s2[T::FM];
#pragma unroll
    for (int i = 0; i < T::FM; ++i) zero[i] = 0.f;
    if (ln) {
      tile_row_sums<T>(acc, colv, 0, zero, s1, lds, wm, wn, lane);
#pragma unroll
      for (int i = 0; i < T::FM; ++i) s1[i] = s1[i] / (float)n_tile;  // tile mean
      tile_row_sums<T>(acc, colv, 1, s1, s2, lds, wm, wn, lane);      // tile M2
    } else {
      tile_row_sums<T>(acc, colv, 2, zero, s2, lds, wm, wn, lane);    // tile sum x^2
#pragma unroll
      for (int i = 0; i < T::FM; ++i) s1[i] = 0.f;
    }
    if constexpr (EPI == EPI_ROW_LOCAL) {
      const float inv_n = 1.0f / (float)p.N;
#pragma unroll
      for (int i = 0; i < T::FM; ++i) {
        mean[i] = s1[i];
        rstd[i] = 1.0f / __builtin_sqrtf(fmaf(s2[i], inv_n, p.eps));
      }
    } else {
      // Cross-workgroup merge of per-row partials (persistent grid, all
      // workgroups of a row block co-resident).
      const uint32_t fin = 2 * T::STAGE + T::RED_BYTES;
      const int row_blocks = p.tiles_m;
      int* err = (int*)(p.ws + XwgLayout::kErr);
      int* arrive = (int*)(p.ws + XwgLayout::kCnt);
      int* depart = arrive + row_blocks;
      float* part = (float*)(p.ws + XwgLayout::part_off(row_blocks));
      float* mypart = part + ((size_t)tm * p.tiles_n + tn) * T::BM * 2;
      if (wn == 0 && g == 0) {
#pragma unroll
        for (int i = 0; i < T::FM; ++i) {
          const int r = wm * T::WTM + 16 * i + l16;
          store_agent(mypart + 2 * r, s1[i]);
          store_agent(mypart + 2 * r + 1, s2[i]);
        }
      }
      wait_all_mem();
      __syncthreads();
      if (tid == 0) {
        add_agent(arrive + tm, 1);
        int spins = 0;
        while (load_agent(arrive + tm) < p.tiles_n) {
          __builtin_amdgcn_s_sleep(4);
          if (++spins > p.spin_limit) {
            store_agent(err, 1);
            break;
          }
        }
      }
      __syncthreads();
      // Merge the tiles_n partials of each row in fixed tile order (all
      // workgroups of the row block compute identical statistics).
      for (int row = tid; row < T::BM; row += T::NT) {
        const float* rowpart = part + (size_t)tm * p.tiles_n * T::BM * 2 + 2 * row;
        float mu = 0.f, m2 = 0.f, cnt = 0.f;
        for (int t = 0; t < p.tiles_n; ++t) {
          const float a = load_agent(rowpart + (size_t)t * T::BM * 2);
          const float b = load_agent(rowpart + (size_t)t * T::BM * 2 + 1);
          const float nt = (float)min(T::BN, p.N - t * T::BN);
          if (ln) {
            const float nn = cnt + nt;
            const float d = a - mu;
            mu = fmaf(d, nt / nn, mu);
            m2 = m2 + b + d * d * (cnt * nt / nn);
            cnt = nn;
          } else {
            m2 += b;
          }
        }
        const float r = 1.0f / __builtin_sqrtf(fmaf(m2, 1.0f / (float)p.N, p.eps));
        *(lds_f32x2*)(lds + fin + row * 8) = f32x2{mu, r};
      }
      wait_all_mem();
      __syncthreads();
      if (tid == 0) {
        // Last workgroup to leave resets the row block's counters for the
        // next call (all have passed the wait by then).
        if (add_agent(depart + tm, 1) == p.tiles_n - 1) {
          store_agent(arrive + tm, 0);
          store_agent(depart + tm, 0);
        }
      }
#pragma unroll
      for (int i = 0; i < T::FM; ++i) {
        f32x2 st = *(lds_f32x2*)(lds + fin + (wm * T::WTM + 16 * i + l16) * 8);
        mean[i] = st[0];
        rstd[i] = st[1];
      }
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
    apply_store<T>(p, acc, mean, rstd, ln, m_base, n_base, wm, wn, lane);
  }
}

// Tile order shared by both grids: tiles grouped 4 tile-rows high, column-major
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

template <class T, int EPI>
__global__ void __launch_bounds__(T::NT) gemm_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) char smem[T::LDS];
  lds_char* lds = lds_base(smem);
  const int total = p.tiles_m * p.tiles_n;
  const int t = xcd_contiguous(blockIdx.x, total);
  int tm, tn;
  grouped_tile(t, p.tiles_m, p.tiles_n, 4, tm, tn);
  process_tile<T, EPI>(p, lds, tm, tn);
}

// Persistent grid for EPI_ROW_XWG: gridDim.x = R * tiles_n workgroups, all
// co-resident (cooperative launch).  Round `it` covers the complete row blocks
// it*R .. it*R+R-1, so every workgroup a tile waits for is working on the
// same round.
template <class T>
__global__ void __launch_bounds__(T::NT) gemm_xwg_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) char smem[T::LDS];
  lds_char* lds = lds_base(smem);
  const int G = gridDim.x;
  const int R = G / p.tiles_n;
  const int j = (G % 8 == 0) ? xcd_contiguous(blockIdx.x, G) : (int)blockIdx.x;
  const int gh = (R % 4 == 0) ? 4 : ((R % 2 == 0) ? 2 : 1);
  int rb_in, tn;
  grouped_tile(j, R, p.tiles_n, gh, rb_in, tn);
  for (int it = 0; it < p.iters; ++it) {
    const int tm = it * R + rb_in;
    if (tm >= p.tiles_m) break;
    process_tile<T, EPI_ROW_XWG>(p, lds, tm, tn);
  }
}

}  // namespace ng
