// Standalone row norm (RMSNorm / LayerNorm) over a bf16 matrix -- the norm
// half of the unfused baseline.  Memory-bound: each element is read once
// (16-byte loads, kept in registers) and written once.
//
// Formulas: "RMSNorm fusion on Ascend", sections 1.1 and 1.2 (mean and biased
// variance, or mean of squares, over the row; eps inside the square root;
// gamma/beta per column).  LayerNorm takes its variance in a second pass over
// the registers, around the row mean.
//
// Residual form (RES): the row is S = X + R, a residual connection followed by
// the norm ("Free normalization fusion", section "FlashNormAttention").  S is
// rounded to bf16 as it is formed (the residual stream's storage type),
// optionally stored to S_out, and normalized.
#pragma once

#include "ng_device.h"

namespace ng {

struct NormParams {
  const uint16_t* X;
  const uint16_t* gamma;
  const uint16_t* beta;
  const uint16_t* R;  // RES: bf16 [rows][cols]
  uint16_t* S_out;    // RES: optional bf16 [rows][cols] output X + R
  uint16_t* Y;
  float* mean_out;
  float* rstd_out;
  int rows, cols;
  int kind;  // 0 RMS, 1 LayerNorm
  float eps;
};

// Row reduction over LPR consecutive lanes (LPR <= 64: within a wave; larger:
// wave partials combined through LDS in fixed order).
template <int LPR>
__device__ __forceinline__ float row_reduce(float v, float* red, int tid) {
  constexpr int WL = LPR < 64 ? LPR : 64;
#pragma unroll
  for (int m = WL / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  if constexpr (LPR > 64) {
    constexpr int WPR = LPR / 64;  // waves per row
    const int wave = tid >> 6;
    if ((tid & 63) == 0) red[wave] = v;
    __syncthreads();
    const int first = (wave / WPR) * WPR;
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < WPR; ++w) s += red[first + w];
    __syncthreads();
    v = s;
  }
  return v;
}

// LPR lanes per row, CPL 16-byte chunks per lane; 256 threads per block.
template <int LPR, int CPL, bool RES = false>
__global__ void __launch_bounds__(256) norm_kernel(NormParams p) {
  constexpr int RPB = 256 / LPR;  // rows per block
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const int r_in = tid / LPR, lr = tid % LPR;
  const long row = (long)blockIdx.x * RPB + r_in;
  const bool rv = row < p.rows;
  const int nch = p.cols >> 3;
  const u32x4* xr = (const u32x4*)(p.X + row * (long)p.cols);
  u32x4 v[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int idx = lr + c * LPR;
    v[c] = u32x4{0u, 0u, 0u, 0u};
    if (rv && idx < nch) v[c] = xr[idx];
  }
  if constexpr (RES) {
    const u32x4* rr = (const u32x4*)(p.R + row * (long)p.cols);
    u32x4* sr = (u32x4*)(p.S_out + row * (long)p.cols);
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int idx = lr + c * LPR;
      if (!rv || idx >= nch) continue;
      const u32x4 r = rr[idx];
#pragma unroll
      for (int w = 0; w < 4; ++w)
        v[c][w] = pack_bf16x2(bf16_lo(v[c][w]) + bf16_lo(r[w]), bf16_hi(v[c][w]) + bf16_hi(r[w]));
      if (p.S_out) sr[idx] = v[c];
    }
  }
  const bool ln = p.kind == 1;
  // pass 1: sum x (LayerNorm) or sum x^2 (RMSNorm)
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < CPL; ++c)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float a = bf16_lo(v[c][w]), b = bf16_hi(v[c][w]);
      if (ln) s += a + b;
      else s = fmaf(a, a, fmaf(b, b, s));
    }
  s = row_reduce<LPR>(s, red, tid);
  const float inv_n = 1.0f / (float)p.cols;
  float mean = 0.f, var;
  if (ln) {
    mean = s * inv_n;
    float s2 = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      if (lr + c * LPR >= nch) continue;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float a = bf16_lo(v[c][w]) - mean, b = bf16_hi(v[c][w]) - mean;
        s2 = fmaf(a, a, fmaf(b, b, s2));
      }
    }
    var = row_reduce<LPR>(s2, red, tid) * inv_n;
  } else {
    var = s * inv_n;
  }
  const float rstd = 1.0f / __builtin_sqrtf(var + p.eps);
  const float sh = -mean * rstd;
  if (!rv) return;
  if (lr == 0) {
    if (p.mean_out) p.mean_out[row] = mean;
    if (p.rstd_out) p.rstd_out[row] = rstd;
  }
  if (!p.Y) return;  // statistics only (the pre-pass of the pre-LayerNorm product)
  u32x4* yr = (u32x4*)(p.Y + row * (long)p.cols);
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int idx = lr + c * LPR;
    if (idx >= nch) continue;
    float g[8], bt[8];
    if (p.gamma) {
      const u32x4 gw = ((const u32x4*)p.gamma)[idx];
#pragma unroll
      for (int w = 0; w < 4; ++w) { g[2 * w] = bf16_lo(gw[w]); g[2 * w + 1] = bf16_hi(gw[w]); }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) g[e] = 1.f;
    }
    if (p.beta) {
      const u32x4 bw = ((const u32x4*)p.beta)[idx];
#pragma unroll
      for (int w = 0; w < 4; ++w) { bt[2 * w] = bf16_lo(bw[w]); bt[2 * w + 1] = bf16_hi(bw[w]); }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) bt[e] = 0.f;
    }
    u32x4 o;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float a = fmaf(fmaf(bf16_lo(v[c][w]), rstd, sh), g[2 * w], bt[2 * w]);
      const float b = fmaf(fmaf(bf16_hi(v[c][w]), rstd, sh), g[2 * w + 1], bt[2 * w + 1]);
      o[w] = pack_bf16x2(a, b);
    }
    yr[idx] = o;
  }
}

// Standalone RMSNorm backward (no affine), the norm half of the unfused
// baseline of the Lazy backward: for a row x with saved rstd and upstream
// gradient dy,  dx = rstd * dy - rstd^3 * (sum_k dy_k x_k) / cols * x  (the
// chain rule of y = x * rstd, rstd = (mean(x^2) + eps)^(-1/2)).  Both rows
// stay in registers; LPR lanes per row, CPL 16-byte chunks per lane.
struct NormBwdParams {
  const uint16_t* dY;
  const uint16_t* X;
  const float* rstd;
  uint16_t* dX;
  int rows, cols;
};

template <int LPR, int CPL>
__global__ void __launch_bounds__(256) norm_bwd_kernel(NormBwdParams p) {
  constexpr int RPB = 256 / LPR;
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const int r_in = tid / LPR, lr = tid % LPR;
  const long row = (long)blockIdx.x * RPB + r_in;
  const bool rv = row < p.rows;
  const int nch = p.cols >> 3;
  const u32x4* dyr = (const u32x4*)(p.dY + row * (long)p.cols);
  const u32x4* xr = (const u32x4*)(p.X + row * (long)p.cols);
  u32x4 dy[CPL], x[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int idx = lr + c * LPR;
    dy[c] = u32x4{0u, 0u, 0u, 0u};
    x[c] = u32x4{0u, 0u, 0u, 0u};
    if (rv && idx < nch) {
      dy[c] = dyr[idx];
      x[c] = xr[idx];
    }
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < CPL; ++c)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      s = fmaf(bf16_lo(dy[c][w]), bf16_lo(x[c][w]), s);
      s = fmaf(bf16_hi(dy[c][w]), bf16_hi(x[c][w]), s);
    }
  s = row_reduce<LPR>(s, red, tid);
  if (!rv) return;
  const float r = p.rstd[row];
  const float cx = r * r * r * s / (float)p.cols;
  u32x4* dxr = (u32x4*)(p.dX + row * (long)p.cols);
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int idx = lr + c * LPR;
    if (idx >= nch) continue;
    u32x4 o;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float a = fmaf(bf16_lo(dy[c][w]), r, -cx * bf16_lo(x[c][w]));
      const float b = fmaf(bf16_hi(dy[c][w]), r, -cx * bf16_hi(x[c][w]));
      o[w] = pack_bf16x2(a, b);
    }
    dxr[idx] = o;
  }
}

// Zero-fill (workspace reset) without hipMemsetAsync, so it may be captured
// in a HIP graph.
__global__ void __launch_bounds__(256) fill_zero_kernel(u32x4* p, size_t n16, uint32_t* tail,
                                                        size_t ntail) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t k = i; k < n16; k += stride) p[k] = u32x4{0u, 0u, 0u, 0u};
  if (i < ntail) tail[i] = 0u;
}

}  // namespace ng
