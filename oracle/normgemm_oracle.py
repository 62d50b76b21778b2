"""Plain float64 definitions of the norm-fused GEMM operations.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.

Sources (cited by page title and section):

* "Free normalization fusion" (aixai.ru blog, Russian), section "Lazy
  Pre-Norm": the fused product is C = rmsnorm(A) @ B with rmsnorm(A) equal to
  A times the per-row inverse root-mean-square, and the row scale commutes
  with the matrix product.
* Same page, section "Multi-CTA Norm Fusion": any normalization splits into a
  per-row reduction (rstd, or mean and variance) followed by an elementwise
  apply; this is the form of the GEMM-epilogue norms.
* "RMSNorm fusion on Ascend" (gsyq.cn, Chinese), section 1.1 (LayerNorm: mean,
  biased variance over the H elements of a row, (x - mean)/sqrt(var + eps),
  then gamma * x_norm + beta) and section 1.2 (RMSNorm: x / sqrt(mean(x^2) +
  eps) * gamma).  The extracted text lost the "+" before eps; eps is read as
  added inside the square root, which the page's own code sample confirms.

H, the length a row is normalized over, is K for the Lazy Pre-Norm form (a
row of A) and N for the GEMM-epilogue forms (a row of A @ B).
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact decode of raw bfloat16 bit patterns (uint16) to float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bfloat16, nearest with ties to even.

    Rounds directly from float64 (no intermediate float32 rounding), so the
    result is the bfloat16 value nearest to ``x``.  Used only to express the
    precision of a bfloat16 output in the tests.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                       # x = m * 2**e, 0.5 <= |m| < 1
    # bfloat16 keeps 8 significant bits: scale the mantissa to [128, 256).
    q = np.rint(m * 256.0)                   # numpy rint rounds ties to even
    y = np.ldexp(q / 256.0, e).astype(np.float32)
    return (y.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _f64(x) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_to_f64(x)
    return np.asarray(x, dtype=np.float64)


def gemm(A, B) -> np.ndarray:
    """X = A @ B in float64.  A is [M, K], B is [K, N] (logical layout)."""
    A = _f64(A)
    B = _f64(B)
    return A @ B


def rms_norm_rows(X, eps: float, gamma=None) -> Tuple[np.ndarray, np.ndarray]:
    """RMSNorm of each row of X (section 1.2 of the Ascend page).

    ms = (1/H) * sum_i x_i^2,  rstd = 1/sqrt(ms + eps),  y = x * rstd * gamma.
    Returns (Y, rstd).  gamma is per column; None means 1.
    """
    X = _f64(X)
    H = X.shape[1]
    ms = np.sum(X * X, axis=1) / H
    rstd = 1.0 / np.sqrt(ms + eps)
    Y = X * rstd[:, None]
    if gamma is not None:
        Y = Y * _f64(gamma)[None, :]
    return Y, rstd


def layer_norm_rows(X, eps: float, gamma=None, beta=None
                    ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """LayerNorm of each row of X (section 1.1 of the Ascend page).

    mean = (1/H) sum_i x_i,  var = (1/H) sum_i (x_i - mean)^2 (biased, two
    passes),  rstd = 1/sqrt(var + eps),  y = (x - mean) * rstd * gamma + beta.
    Returns (Y, mean, rstd).  gamma/beta are per column; None means 1 / 0.
    """
    X = _f64(X)
    H = X.shape[1]
    mean = np.sum(X, axis=1) / H
    D = X - mean[:, None]
    var = np.sum(D * D, axis=1) / H
    rstd = 1.0 / np.sqrt(var + eps)
    Y = D * rstd[:, None]
    if gamma is not None:
        Y = Y * _f64(gamma)[None, :]
    if beta is not None:
        Y = Y + _f64(beta)[None, :]
    return Y, mean, rstd


def rmsnorm_gemm_lazy(A, B, eps: float) -> Tuple[np.ndarray, np.ndarray]:
    """C = rmsnorm(A) @ B for RMSNorm without affine ("Lazy Pre-Norm" section).

    The definition is computed as written: each row of A is normalized over
    its K elements first (unrounded float64), then multiplied by B.  The fused
    kernel's reordering (A @ B) * rstd is equal in exact arithmetic; it is not
    used here.  Returns (C, rstd) with rstd per row of A.
    """
    A_hat, rstd = rms_norm_rows(A, eps)
    return A_hat @ _f64(B), rstd


def rmsnorm_gemm_lazy_affine(A, B, eps: float, gamma=None, beta=None
                             ) -> Tuple[np.ndarray, np.ndarray]:
    """C = (rmsnorm(A) * gamma + beta) @ B: pre-RMSNorm with per-column affine
    (gamma, beta of length K), then the product.

    The "Lazy Pre-Norm" section states that the row-scale trick does not hold
    with an elementwise affine, which scales columns of A; "RMSNorm fusion on
    Ascend", section 6.4, notes that for inference gamma is fixed and can be
    merged into the following matmul's weights ahead of time.  The oracle
    computes the definition as written: normalize each row of A over its K
    elements, apply gamma and beta per column, then multiply by B (no
    folding).  Returns (C, rstd) with rstd per row of A.
    """
    Y, rstd = rms_norm_rows(A, eps, gamma)
    if beta is not None:
        Y = Y + _f64(beta)[None, :]
    return Y @ _f64(B), rstd


def lazy_fold_affine(B, gamma=None, beta=None) -> Tuple[np.ndarray, np.ndarray]:
    """The weight fold of the Lazy Pre-Norm affine form, in float64:
    B_folded = diag(gamma) B (row k of B scaled by gamma[k]) and
    bias = beta^T B (one value per output column).  With these,
    (rmsnorm(A) * gamma + beta) @ B = rstd(A) * (A @ B_folded) + bias
    ("RMSNorm fusion on Ascend", section 6.4: gamma merged into the weights).
    """
    Bf = _f64(B)
    K, N = Bf.shape
    g = np.ones(K) if gamma is None else _f64(gamma)
    b = np.zeros(K) if beta is None else _f64(beta)
    return g[:, None] * Bf, b @ Bf


def layernorm_gemm_prenorm(A, B, eps: float, gamma=None, beta=None
                           ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """C = LayerNorm(A) @ B: a pre-LayerNorm over each row of A (length K),
    with per-column gamma/beta of length K, then the product.

    The "Lazy Pre-Norm" section states that its row-scale identity does not
    cover LayerNorm; "RMSNorm fusion on Ascend", section 2.2, fuses a norm
    with the following matmul in two stages: row statistics first, then the
    normalized tiles enter the product.  The oracle computes the definition
    as written: normalize each row of A (section 1.1), apply gamma and beta,
    then multiply by B.  Returns (C, mean, rstd) per row of A.
    """
    Y, mean, rstd = layer_norm_rows(A, eps, gamma, beta)
    return Y @ _f64(B), mean, rstd


def layernorm_gemm_fold(B, gamma=None, beta=None
                        ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """The weight fold of the pre-LayerNorm product, in float64:
    B_folded = diag(gamma) B, colsum = 1^T B_folded (column sums of the folded
    weights) and bias = beta^T B.  Each row of LayerNorm(A) is
    (a - mean) * rstd * gamma + beta, and the product is linear, so
    LayerNorm(A) @ B = rstd * (A @ B_folded - mean * colsum) + bias, with
    mean and rstd per row of A and colsum, bias per output column.
    """
    Bf, bias = lazy_fold_affine(B, gamma, beta)
    return Bf, Bf.sum(axis=0), bias


def rmsnorm_gemm_lazy_backward(A, B, dC, eps: float
                               ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradients of C = rmsnorm(A) @ B (RMSNorm without affine, the Lazy
    Pre-Norm product) for an upstream gradient dC.

    "Free normalization fusion", section "Lazy Pre-Norm": the normalized A is
    never stored, so the backward pass has to rebuild it from A and the saved
    per-row rstd; the "fusion regrouping" remark (the norm's backward fused
    into the epilogue of a different matmul) places the norm backward after
    dA_hat = dC @ B^T.  The formulas are the chain rule of the forward
    definition, written out:
        A_hat = rstd * A                 (rstd per row of A, over its K entries)
        dA_hat = dC @ B^T
        dB = A_hat^T @ dC
        dA = rstd * (dA_hat - A_hat * mean_k(dA_hat * A_hat))
    (the last from rstd = (mean(a^2) + eps)^(-1/2): d rstd / d a_k =
    -rstd^3 a_k / K).  Returns (dA, dB, rstd).
    """
    A_hat, rstd = rms_norm_rows(A, eps)
    G = _f64(dC)
    dA_hat = G @ _f64(B).T
    dB = lazy_backward_weight(A, dC, eps)
    K = A_hat.shape[1]
    dot = (dA_hat * A_hat).sum(axis=1, keepdims=True) / K
    dA = rstd[:, None] * (dA_hat - A_hat * dot)
    return dA, dB, rstd


def lazy_backward_weight(A, dC, eps: float, rows=None) -> np.ndarray:
    """dB = A_hat^T @ dC, the weight gradient of C = rmsnorm(A) @ B, with
    A_hat = rmsnorm(A) (no affine).  `rows` selects rows of dB (columns of A)
    so that a few rows of a large dB can be formed alone."""
    A_hat, _ = rms_norm_rows(A, eps)
    if rows is not None:
        A_hat = A_hat[:, rows]
    return A_hat.T @ _f64(dC)


def gemm_rmsnorm(A, B, eps: float, gamma=None) -> Tuple[np.ndarray, np.ndarray]:
    """Y = RMSNorm(A @ B) over each full output row (H = N), optional gamma.

    The epilogue form of the "Multi-CTA Norm Fusion" section: reduce each
    whole row of the product, then apply.  Returns (Y, rstd).
    """
    return rms_norm_rows(gemm(A, B), eps, gamma)


def gemm_layernorm(A, B, eps: float, gamma=None, beta=None
                   ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Y = LayerNorm(A @ B) over each full output row (H = N), optional affine.

    Returns (Y, mean, rstd).
    """
    return layer_norm_rows(gemm(A, B), eps, gamma, beta)


def gemm_add_rmsnorm(A, B, R, eps: float, gamma=None
                     ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Y = RMSNorm(A @ B + R) over each full row (H = N), optional gamma:
    a residual connection followed by a post-norm, the residual added before
    the row statistics ("Free normalization fusion", section
    "FlashNormAttention": residual connection, then post-RMSNorm, with the
    residual added into the matrix-core accumulator).  Returns (Y, rstd, S)
    with S = A @ B + R, the sum the norm is taken over.
    """
    S = gemm(A, B) + _f64(R)
    Y, rstd = rms_norm_rows(S, eps, gamma)
    return Y, rstd, S


def gemm_add_layernorm(A, B, R, eps: float, gamma=None, beta=None
                       ) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """Y = LayerNorm(A @ B + R) over each full row (H = N), optional affine.
    Returns (Y, mean, rstd, S) with S = A @ B + R.
    """
    S = gemm(A, B) + _f64(R)
    Y, mean, rstd = layer_norm_rows(S, eps, gamma, beta)
    return Y, mean, rstd, S


def norm(X, kind: str, eps: float, gamma=None, beta=None):
    """Standalone row norm of X: kind 'rms' or 'layer'.

    For RMSNorm a beta, when given, is added after gamma as in the LayerNorm
    affine ("RMSNorm fusion on Ascend", section 1.1: gamma * x_norm + beta); it
    is the unfused form of a pre-norm with a full elementwise affine, the case
    the "Lazy Pre-Norm" section names as outside the row-scale identity.
    Returns (Y, mean_or_None, rstd).
    """
    if kind == "rms":
        Y, rstd = rms_norm_rows(X, eps, gamma)
        if beta is not None:
            Y = Y + _f64(beta)[None, :]
        return Y, None, rstd
    if kind == "layer":
        return layer_norm_rows(X, eps, gamma, beta)
    raise ValueError(f"unknown norm kind {kind!r}")


def rel_err(got, ref) -> float:
    """max |got - ref| / (1 + |ref|) over all elements (0.0 for empty)."""
    got = _f64(got)
    ref = _f64(ref)
    if ref.size == 0:
        return 0.0
    return float(np.max(np.abs(got - ref) / (1.0 + np.abs(ref))))
