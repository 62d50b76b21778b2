// Folding a pre-norm affine into the next product's weights, for Lazy
// Pre-Norm with gamma/beta:
//   (rmsnorm(A) * gamma + beta) @ B = rstd(A) * (A @ B') + bias,
//   B' = diag(gamma) B   (row k of B, as [K, N], scaled by gamma[k]),
//   bias = beta^T B      (fp32, one value per output column).
// ("Free normalization fusion", section "Lazy Pre-Norm": the per-column affine
// is what keeps the plain row-scale identity from applying; "RMSNorm fusion on
// Ascend", section 6.4: at inference gamma is fixed and can be merged into the
// following matmul's weights ahead of time.)  Both are one-off weight
// transforms.  The pre-LayerNorm product also needs colsum = 1^T B' (the same
// column sum with every beta[k] = 1, taken over the folded weights): the row
// mean of A passes through the product as mean * colsum.
#pragma once

#include "ng_device.h"

namespace ng {

struct FoldParams {
  const uint16_t* B;
  const uint16_t* gamma;  // [K] or NULL (1)
  const uint16_t* beta;   // [K] or NULL (0)
  uint16_t* B_folded;     // same layout as B; may be B itself
  float* bias;            // [N] or NULL (not computed)
  int64_t K, N;
  int nk;                 // 1: B stored [N, K]
  int ones;               // fold_bias_kernel: every beta[k] = 1 (column sums)
};

// B' = diag(gamma) B, 8 elements (16 bytes) per thread and step, rounded to
// bf16 (nearest even).  K and N are multiples of 8, so the 8 elements of a
// chunk share one k ([K, N]) or hold 8 consecutive k ([N, K]).
__global__ void __launch_bounds__(256) fold_gamma_kernel(FoldParams p) {
  const int64_t chunks = p.K * p.N / 8;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < chunks; c += stride) {
    const u32x4 v = ((const u32x4*)p.B)[c];
    const int64_t e = c * 8;
    float g[8];
    if (!p.gamma) {
#pragma unroll
      for (int i = 0; i < 8; ++i) g[i] = 1.f;
    } else if (p.nk) {
      const u32x4 gw = *(const u32x4*)(p.gamma + e % p.K);
#pragma unroll
      for (int w = 0; w < 4; ++w) { g[2 * w] = bf16_lo(gw[w]); g[2 * w + 1] = bf16_hi(gw[w]); }
    } else {
      const uint16_t gk = p.gamma[e / p.N];
      const float gf = __uint_as_float((uint32_t)gk << 16);
#pragma unroll
      for (int i = 0; i < 8; ++i) g[i] = gf;
    }
    u32x4 o;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      o[w] = pack_bf16x2(bf16_lo(v[w]) * g[2 * w], bf16_hi(v[w]) * g[2 * w + 1]);
    ((u32x4*)p.B_folded)[c] = o;
  }
}

// bias[n] = sum_k beta[k] * B[k][n] in fp32 (bf16 products are exact in
// fp32); with `ones`, the column sums sum_k B[k][n].  [K, N]: 64 columns per workgroup, thread (slice s, column c) sums
// k = s, s+4, ... (coalesced across c); the four slices are added in order.
// [N, K]: one column per wave, lane l sums k = l, l+64, ... (contiguous), then
// the lanes combine pairwise in a fixed order.
__global__ void __launch_bounds__(256) fold_bias_kernel(FoldParams p) {
  __shared__ float part[4][64];
  const int t = threadIdx.x;
  if (!p.nk) {
    const int c = t & 63, s = t >> 6;
    const int64_t n = (int64_t)blockIdx.x * 64 + c;
    float acc = 0.f;
    if (n < p.N && (p.beta || p.ones)) {
      for (int64_t k = s; k < p.K; k += 4) {
        const float b = __uint_as_float((uint32_t)p.B[k * p.N + n] << 16);
        const float be = p.ones ? 1.f : __uint_as_float((uint32_t)p.beta[k] << 16);
        acc = fmaf(be, b, acc);
      }
    }
    part[s][c] = acc;
    __syncthreads();
    if (s == 0 && n < p.N) p.bias[n] = (part[0][c] + part[1][c]) + (part[2][c] + part[3][c]);
  } else {
    const int lane = t & 63, w = t >> 6;
    const int64_t n = (int64_t)blockIdx.x * 4 + w;
    float acc = 0.f;
    if (n < p.N && (p.beta || p.ones)) {
      for (int64_t k = lane; k < p.K; k += 64) {
        const float b = __uint_as_float((uint32_t)p.B[n * p.K + k] << 16);
        const float be = p.ones ? 1.f : __uint_as_float((uint32_t)p.beta[k] << 16);
        acc = fmaf(be, b, acc);
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float other = __shfl_xor(acc, o, 64);
      acc = (lane & o) ? other + acc : acc + other;
    }
    if (lane == 0 && n < p.N) p.bias[n] = acc;
  }
}

}  // namespace ng
