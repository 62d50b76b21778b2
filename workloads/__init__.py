"""Seeded synthetic inputs for the norm-fused GEMM path.

This module is shared by the CPU oracle, the tests and the benchmark.  It
holds no arithmetic of the method itself: it only draws random numbers and
rounds them to bfloat16 storage.

Input recipe (the same for every workload):

* ``numpy.random.default_rng(seed)`` (PCG64), values drawn in float32 in a
  fixed order: A's standard normals ``[M, K]``, then the per-row scales of A
  (when the workload has them), then the per-row shifts of A (when it has
  them), then B's standard normals ``[K, N]`` times
  ``sqrt(1/K)``, then gamma, then beta, then (residual forms) the residual
  R's standard normals ``[M, N]`` (unit variance, the scale of ``A @ B``),
  then (backward forms) the upstream gradient dC's standard normals
  ``[M, N]``.
* ``N(mu, v)`` in a workload description is read with ``v`` as the variance,
  so ``B ~ N(0, 1/K)`` keeps ``A @ B`` at unit variance per element and
  ``gamma ~ N(1, 0.1)`` has standard deviation ``sqrt(0.1)``.
* A per-row scale "log-uniform[0.1, 10]" is ``10 ** U(-1, 1)`` multiplied
  into the float32 row before rounding; a per-row shift is ``U(-2, 2)``
  added after the scale (rows whose mean is far from zero relative to their
  spread, the case a LayerNorm's mean term exists for).
* Every array is rounded from float32 to bfloat16 with round-to-nearest-even
  and returned as raw ``uint16`` bit patterns; the caller decodes them.

The five named workloads are the shapes the pages' method is exercised on:
two small-N cases (the ads-model regime where naive epilogue fusion applies,
N = 64/128) and three LLM-scale hidden sizes.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

# Operation identifiers (match the C-ABI's op codes for workspace sizing).
OP_LAZY = "rmsnorm_gemm_lazy"
OP_GEMM_RMSNORM = "gemm_rmsnorm"
OP_GEMM_LAYERNORM = "gemm_layernorm"
OP_LAZY_AFFINE = "rmsnorm_gemm_lazy_affine"
OP_GEMM_ADD_RMSNORM = "gemm_add_rmsnorm"
OP_GEMM_ADD_LAYERNORM = "gemm_add_layernorm"
OP_PRENORM_LN = "layernorm_gemm_prenorm"
OP_LAZY_BWD = "rmsnorm_gemm_lazy_backward_input"
OP_LAZY_BWD_W = "rmsnorm_gemm_lazy_backward_weight"
OP_LAZY_BWD_RG = "rmsnorm_gemm_lazy_backward"


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    op: str
    M: int
    N: int
    K: int
    eps: float
    row_scale: bool = False
    row_shift: bool = False
    gamma: bool = False
    beta: bool = False
    residual: bool = False
    upstream: bool = False
    description: str = ""

    @property
    def flops(self) -> int:
        # both gradients of the regrouped backward: two products
        return (4 if self.op == OP_LAZY_BWD_RG else 2) * self.M * self.N * self.K


WORKLOADS = [
    Workload("lazy_rms_256x128x64", OP_LAZY, 256, 64, 128, 1e-6, row_scale=True,
             description="Lazy Pre-Norm RMSNorm (no affine) A 256x128 (row scale "
                         "log-uniform[0.1,10]) @ B 128x64"),
    Workload("gemm_ln_65536x512x128", OP_GEMM_LAYERNORM, 65536, 128, 512, 1e-5,
             description="GEMM + LayerNorm epilogue (no affine) over the full row, "
                         "A 65536x512 @ B 512x128"),
    Workload("lazy_rms_32768x4096x4096", OP_LAZY, 32768, 4096, 4096, 1e-6, row_scale=True,
             description="Lazy Pre-Norm RMSNorm (no affine), LLM shape, A 32768x4096 @ "
                         "B 4096x4096"),
    Workload("gemm_rms_16384x4096x8192", OP_GEMM_RMSNORM, 16384, 8192, 4096, 1e-6, gamma=True,
             description="GEMM + RMSNorm epilogue with gamma over N=8192, A 16384x4096 @ "
                         "B 4096x8192"),
    Workload("gemm_ln_8192x8192x16384", OP_GEMM_LAYERNORM, 8192, 16384, 8192, 1e-5,
             gamma=True, beta=True,
             description="GEMM + LayerNorm epilogue with gamma and beta, large N, "
                         "A 8192x8192 @ B 8192x16384"),
]
# Further forms beyond the five named workloads, on the same shapes: Lazy
# Pre-Norm with a per-column affine (gamma, beta of length K) folded into the
# weights, and the post-norm epilogues with a residual added to the product
# first (one narrow-row and one wide-row case).
NEXT_WORKLOADS = [
    Workload("lazy_rms_affine_32768x4096x4096", OP_LAZY_AFFINE, 32768, 4096, 4096, 1e-6,
             row_scale=True, gamma=True, beta=True,
             description="Lazy Pre-Norm RMSNorm with gamma and beta (length K) folded into B, "
                         "A 32768x4096 @ B 4096x4096"),
    Workload("prenorm_ln_32768x4096x4096", OP_PRENORM_LN, 32768, 4096, 4096, 1e-5,
             row_scale=True, row_shift=True, gamma=True, beta=True,
             description="pre-LayerNorm with gamma and beta (length K) fused with the product, "
                         "A 32768x4096 (row scale and shift) @ B 4096x4096"),
    Workload("lazy_rms_bwd_32768x4096x4096", OP_LAZY_BWD, 32768, 4096, 4096, 1e-6,
             row_scale=True, upstream=True,
             description="Lazy Pre-Norm input gradient: dC 32768x4096 @ B^T, the RMSNorm "
                         "backward over rows of A (32768x4096) in the epilogue"),
    Workload("lazy_rms_bwd_weight_32768x4096x4096", OP_LAZY_BWD_W, 32768, 4096, 4096, 1e-6,
             row_scale=True, upstream=True,
             description="Lazy Pre-Norm weight gradient: A_hat^T @ dC over 32768 rows, A_hat "
                         "rebuilt from A (32768x4096) and rstd"),
    Workload("lazy_rms_bwd_regrouped_32768x4096x4096", OP_LAZY_BWD_RG, 32768, 4096, 4096, 1e-6,
             row_scale=True, upstream=True,
             description="Lazy Pre-Norm backward, both gradients, the weight gradient "
                         "regrouped: the input gradient over rows of A (32768x4096) also "
                         "writes rstd * dC, then dB = A^T @ (rstd * dC)"),
    Workload("gemm_add_ln_65536x512x128", OP_GEMM_ADD_LAYERNORM, 65536, 128, 512, 1e-5,
             residual=True,
             description="GEMM + residual add + LayerNorm epilogue (no affine), "
                         "A 65536x512 @ B 512x128 + R 65536x128"),
    Workload("gemm_add_rms_16384x4096x8192", OP_GEMM_ADD_RMSNORM, 16384, 8192, 4096, 1e-6,
             gamma=True, residual=True,
             description="GEMM + residual add + RMSNorm epilogue with gamma over N=8192, "
                         "A 16384x4096 @ B 4096x8192 + R 16384x8192"),
]
WORKLOAD_BY_NAME = {w.name: w for w in WORKLOADS + NEXT_WORKLOADS}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return raw bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Decode raw bfloat16 bits to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Inputs:
    A: np.ndarray                   # uint16 bits [M, K]
    B: np.ndarray                   # uint16 bits [K, N] (logical layout)
    gamma: Optional[np.ndarray]     # uint16 bits [N] or None
    beta: Optional[np.ndarray]      # uint16 bits [N] or None
    R: Optional[np.ndarray] = None  # uint16 bits [M, N] or None (residual forms)
    dC: Optional[np.ndarray] = None  # uint16 bits [M, N] or None (backward forms)


def make_inputs(M: int, N: int, K: int, *, seed: int = 0, row_scale: bool = False,
                gamma: bool = False, beta: bool = False,
                gamma_len: Optional[int] = None, residual: bool = False,
                row_shift: bool = False, upstream: bool = False) -> Inputs:
    """Draw one seeded input set in the fixed order documented above.

    ``gamma_len`` overrides the length of gamma/beta (default N).
    """
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((M, K), dtype=np.float32)
    if row_scale:
        s = (10.0 ** rng.uniform(-1.0, 1.0, size=M)).astype(np.float32)
        a *= s[:, None]
    if row_shift:
        a += rng.uniform(-2.0, 2.0, size=M).astype(np.float32)[:, None]
    A = f32_to_bf16_bits(a)
    del a
    b = rng.standard_normal((K, N), dtype=np.float32)
    b *= np.float32(math.sqrt(1.0 / K))
    B = f32_to_bf16_bits(b)
    del b
    L = N if gamma_len is None else gamma_len
    g = bt = None
    if gamma:
        g = f32_to_bf16_bits(1.0 + math.sqrt(0.1) * rng.standard_normal(L, dtype=np.float32))
    if beta:
        bt = f32_to_bf16_bits(math.sqrt(0.1) * rng.standard_normal(L, dtype=np.float32))
    R = None
    if residual:
        R = f32_to_bf16_bits(rng.standard_normal((M, N), dtype=np.float32))
    dC = None
    if upstream:
        dC = f32_to_bf16_bits(rng.standard_normal((M, N), dtype=np.float32))
    return Inputs(A, B, g, bt, R, dC)


def workload_inputs(w: Workload, seed: int = 0) -> Inputs:
    # a pre-norm's affine acts on rows of A (length K)
    gl = w.K if w.op in (OP_LAZY_AFFINE, OP_PRENORM_LN) else None
    return make_inputs(w.M, w.N, w.K, seed=seed, row_scale=w.row_scale,
                       gamma=w.gamma, beta=w.beta, gamma_len=gl, residual=w.residual,
                       row_shift=w.row_shift, upstream=w.upstream)
