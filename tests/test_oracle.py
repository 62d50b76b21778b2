"""Pins for the CPU oracle, independent of the oracle's own code.

Every test here checks the oracle against something the pages or plain
mathematics fix: exact brute force on tiny inputs, the hand-worked examples
in tests/golden/, closed forms, invariants, special cases that reduce to a
textbook routine, and the pages' stated limitations of Lazy Pre-Norm.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def _bf16_inputs(M, N, K, seed, **kw):
    x = workloads.make_inputs(M, N, K, seed=seed, **kw)
    return x


# ---------------------------------------------------------------- bf16 codec
def test_bf16_decode_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x4049, 0x7F7F], dtype=np.uint16)
    want = [1.0, -2.0, 1.0078125, 0.0, -0.0, 3.140625, 3.3895313892515355e38]
    got = oracle.bf16_to_f64(bits)
    assert list(got) == want


def test_bf16_encode_ties_to_even():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to the even mantissa (1.0).
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: ties to 1 + 2^-6.
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20, -2.5])
    got = oracle.bf16_to_f64(oracle.f64_to_bf16_bits(x))
    assert list(got) == [1.0, 1.0 + 2.0 ** -6, 1.0 + 2.0 ** -7, -2.5]


# ------------------------------------------------------ GEMM by brute force
@pytest.mark.parametrize("M,K,N", [(4, 4, 4), (3, 5, 7), (6, 2, 1)])
def test_gemm_matches_exact_rational_triple_loop(M, K, N):
    x = _bf16_inputs(M, N, K, seed=11, row_scale=True)
    A = [[Fraction(float(v)) for v in row] for row in oracle.bf16_to_f64(x.A)]
    B = [[Fraction(float(v)) for v in row] for row in oracle.bf16_to_f64(x.B)]
    exact = [[sum(A[i][k] * B[k][j] for k in range(K)) for j in range(N)] for i in range(M)]
    got = oracle.gemm(x.A, x.B)
    assert got.shape == (M, N)
    for i in range(M):
        for j in range(N):
            e = float(exact[i][j])
            assert abs(got[i, j] - e) <= 1e-15 * (1.0 + abs(e))


# ------------------------------------------------------ hand-worked fixtures
def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_hand_worked_examples(case):
    A = np.array(case["A"], dtype=np.float64)
    B = np.array(case["B"], dtype=np.float64)
    eps = case["eps"]
    gamma = np.array(case["gamma"], dtype=np.float64) if "gamma" in case else None
    beta = np.array(case["beta"], dtype=np.float64) if "beta" in case else None
    if case["op"] == "rmsnorm_gemm_lazy":
        C, rstd = oracle.rmsnorm_gemm_lazy(A, B, eps)
        mean = None
    elif case["op"] == "rmsnorm_gemm_lazy_affine":
        C, rstd = oracle.rmsnorm_gemm_lazy_affine(A, B, eps, gamma, beta)
        mean = None
    elif case["op"] == "gemm_rmsnorm":
        C, rstd = oracle.gemm_rmsnorm(A, B, eps, gamma)
        mean = None
    elif case["op"] == "layernorm_gemm_prenorm":
        C, mean, rstd = oracle.layernorm_gemm_prenorm(A, B, eps, gamma, beta)
    elif case["op"] == "gemm_add_layernorm":
        R = np.array(case["R"], dtype=np.float64)
        C, mean, rstd, S = oracle.gemm_add_layernorm(A, B, R, eps, gamma, beta)
        np.testing.assert_allclose(S, [[float(v) for v in row] for row in case["S"]], rtol=0)
    else:
        C, mean, rstd = oracle.gemm_layernorm(A, B, eps, gamma, beta)
    want = np.array([[float(v) for v in row] for row in case["C"]])
    np.testing.assert_allclose(C, want, rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(rstd, [float(r[0]) for r in case["rstd"]], rtol=1e-15)
    if "mean" in case:
        np.testing.assert_allclose(mean, [float(r[0]) for r in case["mean"]], rtol=1e-15)


# ------------------------------------------------------------ closed forms
@pytest.mark.parametrize("c,eps,H", [(3.0, 0.0, 5), (-0.25, 1e-6, 8), (7.5, 0.7, 3), (1e-3, 1e-6, 16)])
def test_rms_of_constant_row(c, eps, H):
    # mean of squares of a constant row is c^2, so y = c / sqrt(c^2 + eps)
    X = np.full((2, H), c)
    Y, rstd = oracle.rms_norm_rows(X, eps)
    np.testing.assert_allclose(Y, c / math.sqrt(c * c + eps), rtol=1e-14)
    np.testing.assert_allclose(rstd, 1.0 / math.sqrt(c * c + eps), rtol=1e-14)


@pytest.mark.parametrize("a,b,eps", [(1.0, 3.0, 0.0), (5.0, -1.0, 0.5), (0.1, 0.1000001, 1e-5)])
def test_layernorm_of_two_element_row(a, b, eps):
    # mean (a+b)/2, deviations +-d with d = (a-b)/2, variance d^2
    d = (a - b) / 2.0
    Y, mean, rstd = oracle.layer_norm_rows(np.array([[a, b]]), eps)
    s = math.sqrt(d * d + eps)
    np.testing.assert_allclose(Y[0], [d / s, -d / s], rtol=1e-9, atol=1e-15)
    np.testing.assert_allclose(mean, [(a + b) / 2.0], rtol=1e-15)


def test_rms_zero_row_lazy():
    # zero row: rstd = 1/sqrt(eps) and the output row is zero (degenerate case)
    A = np.zeros((2, 8))
    A[1] = 1.0
    B = np.arange(24, dtype=np.float64).reshape(8, 3)
    C, rstd = oracle.rmsnorm_gemm_lazy(A, B, 1e-6)
    assert rstd[0] == pytest.approx(1e3, rel=1e-12)
    assert np.all(C[0] == 0.0)


def test_layernorm_constant_row_gives_beta():
    X = np.full((3, 6), 2.5)
    beta = np.linspace(-1, 1, 6)
    gamma = np.linspace(0.5, 2, 6)
    Y, mean, rstd = oracle.layer_norm_rows(X, 1e-5, gamma, beta)
    np.testing.assert_allclose(Y, np.broadcast_to(beta, Y.shape), atol=1e-15)
    np.testing.assert_allclose(mean, 2.5)


# --------------------------------------------------------------- invariants
def test_layernorm_rows_zero_mean_unit_variance():
    # With eps = 0 every output row has mean 0 and biased variance exactly 1;
    # H = 5 makes a 1/(H-1) variance visible (it would give 4/5).
    rng = np.random.default_rng(3)
    X = rng.standard_normal((40, 5)) * rng.uniform(0.1, 10, size=(40, 1)) + rng.standard_normal((40, 1))
    Y, _, _ = oracle.layer_norm_rows(X, 0.0)
    np.testing.assert_allclose(Y.mean(axis=1), 0.0, atol=1e-14)
    np.testing.assert_allclose((Y * Y).mean(axis=1), 1.0, rtol=1e-13)


def test_layernorm_variance_with_eps():
    # With eps > 0 the output row variance is var/(var + eps) < 1; for rows of
    # the form c + [-d, +d, -d, +d] the variance is d^2.
    d = np.array([0.1, 0.5, 2.0])
    X = 3.0 + d[:, None] * np.array([-1.0, 1.0, -1.0, 1.0])[None, :]
    eps = 0.05
    Y, _, _ = oracle.layer_norm_rows(X, eps)
    np.testing.assert_allclose((Y * Y).mean(axis=1), d * d / (d * d + eps), rtol=1e-12)


def test_gemm_rmsnorm_rows_unit_rms_eps0():
    x = _bf16_inputs(17, 24, 16, seed=5)
    Y, _ = oracle.gemm_rmsnorm(x.A, x.B, 0.0)
    np.testing.assert_allclose((Y * Y).mean(axis=1), 1.0, rtol=1e-13)


@pytest.mark.parametrize("eps", [1e-6, 0.5])
def test_rms_row_scale_invariance(eps):
    # rmsnorm_eps(s * x) = rmsnorm_{eps/s^2}(x) exactly, for any per-row s > 0.
    rng = np.random.default_rng(7)
    A = rng.standard_normal((12, 32))
    B = rng.standard_normal((32, 9))
    s = 10.0 ** rng.uniform(-1, 1, size=12)
    C1, r1 = oracle.rmsnorm_gemm_lazy(A * s[:, None], B, eps)
    # eps/s^2 differs per row: evaluate row by row
    for i in range(12):
        C2, r2 = oracle.rmsnorm_gemm_lazy(A[i:i + 1], B, eps / s[i] ** 2)
        np.testing.assert_allclose(C1[i], C2[0], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(r1[i] * s[i], r2[0], rtol=1e-12)


def test_lazy_identity_row_scale_commutes_with_matmul():
    # (A * rstd) @ B == (A @ B) * rstd  (section "Lazy Pre-Norm")
    x = _bf16_inputs(33, 20, 48, seed=9, row_scale=True)
    C, rstd = oracle.rmsnorm_gemm_lazy(x.A, x.B, 1e-6)
    late = oracle.gemm(x.A, x.B) * rstd[:, None]
    np.testing.assert_allclose(C, late, rtol=1e-12, atol=1e-13)


def test_affine_is_columnwise():
    x = _bf16_inputs(9, 13, 16, seed=4, gamma=True, beta=True)
    g = oracle.bf16_to_f64(x.gamma)
    b = oracle.bf16_to_f64(x.beta)
    Y0, m0, r0 = oracle.gemm_layernorm(x.A, x.B, 1e-5)
    Y1, m1, r1 = oracle.gemm_layernorm(x.A, x.B, 1e-5, x.gamma, x.beta)
    np.testing.assert_allclose(Y1, Y0 * g[None, :] + b[None, :], rtol=1e-14, atol=1e-15)
    np.testing.assert_array_equal(m0, m1)
    np.testing.assert_array_equal(r0, r1)
    Z0, _ = oracle.gemm_rmsnorm(x.A, x.B, 1e-6)
    Z1, _ = oracle.gemm_rmsnorm(x.A, x.B, 1e-6, x.gamma)
    np.testing.assert_allclose(Z1, Z0 * g[None, :], rtol=1e-14, atol=1e-15)


# --------------------------------------------- reductions to textbook cases
def test_lazy_with_identity_B_is_plain_rmsnorm():
    x = _bf16_inputs(10, 16, 16, seed=2, row_scale=True)
    C, rstd = oracle.rmsnorm_gemm_lazy(x.A, np.eye(16), 1e-6)
    Y, _, r2 = oracle.norm(x.A, "rms", 1e-6)
    np.testing.assert_allclose(C, Y, rtol=1e-15, atol=1e-15)
    np.testing.assert_array_equal(rstd, r2)


def test_epilogue_norms_with_identity_A_normalize_rows_of_B():
    x = _bf16_inputs(12, 40, 12, seed=6)
    Y, r = oracle.gemm_rmsnorm(np.eye(12), x.B, 1e-6)
    Y2, _, r2 = oracle.norm(x.B, "rms", 1e-6)
    np.testing.assert_allclose(Y, Y2, rtol=1e-15, atol=1e-15)
    Z, m, rz = oracle.gemm_layernorm(np.eye(12), x.B, 1e-5)
    Z2, m2, rz2 = oracle.norm(x.B, "layer", 1e-5)
    np.testing.assert_allclose(Z, Z2, rtol=1e-15, atol=1e-15)


# ------------------------------------- the pages' limitations of Lazy Pre-Norm
def test_lazy_is_not_prenorm_with_columnwise_gamma():
    # A per-column gamma on K does not commute with the product: the Lazy form
    # (A @ B) * rstd differs from rmsnorm_gamma(A) @ B by far more than the
    # GPU tolerance.
    x = _bf16_inputs(64, 32, 64, seed=8, row_scale=True, gamma=True, gamma_len=64)
    C_lazy, _ = oracle.rmsnorm_gemm_lazy(x.A, x.B, 1e-6)
    Yg, _, _ = oracle.norm(x.A, "rms", 1e-6, gamma=x.gamma)
    C_affine = oracle.gemm(Yg, x.B)
    assert oracle.rel_err(C_lazy, C_affine) > 0.05


def test_lazy_affine_without_affine_is_lazy():
    # gamma = 1, beta = 0 given explicitly: the affine path reduces to the
    # plain Lazy Pre-Norm product
    rng = np.random.default_rng(31)
    A = rng.standard_normal((5, 7)) * 3.0
    B = rng.standard_normal((7, 4))
    C1, r1 = oracle.rmsnorm_gemm_lazy_affine(A, B, 1e-6, np.ones(7), np.zeros(7))
    C0, r0 = oracle.rmsnorm_gemm_lazy(A, B, 1e-6)
    np.testing.assert_allclose(C1, C0, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(r1, r0, rtol=1e-15)


def test_lazy_affine_folds_into_weights():
    # (rmsnorm(A) * gamma + beta) @ B == rstd * (A @ (diag(gamma) B)) + beta @ B:
    # gamma scales the K rows of B, beta becomes a per-column bias (the
    # folding the weight-merge passage describes); shapes with K != N so that
    # a gamma applied along the wrong axis could not pass
    rng = np.random.default_rng(32)
    for (M, K, N) in [(3, 5, 7), (6, 4, 2)]:
        A = rng.standard_normal((M, K)) * rng.uniform(0.1, 10.0, size=(M, 1))
        B = rng.standard_normal((K, N))
        g = rng.uniform(0.5, 2.0, size=K)
        b = rng.standard_normal(K)
        C, rstd = oracle.rmsnorm_gemm_lazy_affine(A, B, 1e-5, g, b)
        ms = np.mean(A * A, axis=1)
        r = 1.0 / np.sqrt(ms + 1e-5)
        folded = r[:, None] * (A @ (g[:, None] * B)) + (b @ B)[None, :]
        np.testing.assert_allclose(C, folded, rtol=1e-12, atol=1e-12)
        # the oracle's fold helper gives the same B_folded and bias
        Bf, bias = oracle.lazy_fold_affine(B, g, b)
        np.testing.assert_allclose(r[:, None] * (A @ Bf) + bias[None, :], C, rtol=1e-12,
                                   atol=1e-12)
        np.testing.assert_allclose(rstd, r, rtol=1e-14)
        wrong = r[:, None] * (A @ B) * np.resize(g, N)[None, :] + (b @ B)[None, :]
        assert np.max(np.abs(C - wrong)) > 1e-2


def test_lazy_affine_is_affine_rmsnorm_then_matmul():
    # the Lazy-affine definition agrees with the standalone RMSNorm (gamma,
    # beta) followed by the product, and the RMSNorm beta is a plain column shift
    rng = np.random.default_rng(33)
    A = rng.standard_normal((4, 6)) * 2.0
    B = rng.standard_normal((6, 3))
    g = rng.uniform(0.5, 2.0, size=6)
    b = rng.standard_normal(6)
    Y, _, r = oracle.norm(A, "rms", 1e-6, g, b)
    Y0, _, _ = oracle.norm(A, "rms", 1e-6, g)
    np.testing.assert_allclose(Y - Y0, np.broadcast_to(b, Y.shape), rtol=0, atol=1e-14)
    C, rstd = oracle.rmsnorm_gemm_lazy_affine(A, B, 1e-6, g, b)
    np.testing.assert_allclose(C, Y @ B, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(rstd, r, rtol=1e-15)


def test_residual_norms_reduce_to_plain_forms():
    # R = 0: the residual forms are the plain epilogue norms; A = 0: they are
    # the standalone norm of R
    rng = np.random.default_rng(34)
    A = rng.standard_normal((5, 6))
    B = rng.standard_normal((6, 9))
    R = rng.standard_normal((5, 9)) * 2.0
    g = rng.uniform(0.5, 2.0, size=9)
    b = rng.standard_normal(9)
    Z = np.zeros((5, 9))
    Y, r, S = oracle.gemm_add_rmsnorm(A, B, Z, 1e-6, g)
    Y0, r0 = oracle.gemm_rmsnorm(A, B, 1e-6, g)
    np.testing.assert_allclose(Y, Y0, rtol=1e-14, atol=1e-14)
    Y, m, r, S = oracle.gemm_add_layernorm(A, B, Z, 1e-5, g, b)
    Y0, m0, r0 = oracle.gemm_layernorm(A, B, 1e-5, g, b)
    np.testing.assert_allclose(Y, Y0, rtol=1e-14, atol=1e-14)
    Y, r, S = oracle.gemm_add_rmsnorm(np.zeros((5, 6)), B, R, 1e-6, g)
    Yn, _, rn = oracle.norm(R, "rms", 1e-6, g)
    np.testing.assert_allclose(Y, Yn, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(S, R, rtol=0, atol=0)
    Y, m, r, S = oracle.gemm_add_layernorm(np.zeros((5, 6)), B, R, 1e-5, g, b)
    Yn, mn, rn = oracle.norm(R, "layer", 1e-5, g, b)
    np.testing.assert_allclose(Y, Yn, rtol=1e-14, atol=1e-14)


def test_residual_is_added_before_the_statistics():
    # adding R after normalizing gives a different result (the residual
    # shifts the row statistics)
    rng = np.random.default_rng(35)
    A = rng.standard_normal((4, 8))
    B = rng.standard_normal((8, 16))
    R = rng.standard_normal((4, 16)) * 3.0 + 1.0
    Y, _, _, _ = oracle.gemm_add_layernorm(A, B, R, 1e-5)
    Y_after, _, _ = oracle.gemm_layernorm(A, B, 1e-5)
    assert np.max(np.abs(Y - (Y_after + R))) > 1e-1
    # LayerNorm output rows of the sum are zero-mean, unit-variance
    np.testing.assert_allclose(Y.mean(axis=1), 0.0, atol=1e-12)
    np.testing.assert_allclose(Y.var(axis=1), 1.0, rtol=1e-4)


def test_prenorm_layernorm_invariances():
    # LayerNorm removes a per-row shift and (eps = 0) a positive per-row
    # scale of A, so the product does not see them
    rng = np.random.default_rng(41)
    A = rng.standard_normal((6, 16))
    B = rng.standard_normal((16, 5))
    g = rng.uniform(0.5, 2.0, size=16)
    b = rng.standard_normal(16)
    C, mean, rstd = oracle.layernorm_gemm_prenorm(A, B, 0.0, g, b)
    shift = rng.uniform(-50, 50, size=(6, 1))
    C2, mean2, rstd2 = oracle.layernorm_gemm_prenorm(A + shift, B, 0.0, g, b)
    np.testing.assert_allclose(C2, C, rtol=1e-9, atol=1e-9)
    np.testing.assert_allclose(mean2, mean + shift[:, 0], rtol=1e-12)
    scale = rng.uniform(0.1, 10, size=(6, 1))
    C3, _, rstd3 = oracle.layernorm_gemm_prenorm(A * scale, B, 0.0, g, b)
    np.testing.assert_allclose(C3, C, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(rstd3, rstd / scale[:, 0], rtol=1e-12)
    # beta enters after the norm, as the row vector beta^T B on every row
    C0, _, _ = oracle.layernorm_gemm_prenorm(A, B, 0.0, g, None)
    np.testing.assert_allclose(C - C0, np.broadcast_to(b @ B, C.shape), rtol=1e-12, atol=1e-12)


def test_prenorm_layernorm_of_zero_mean_rows_is_rmsnorm():
    # rows with mean exactly 0: LayerNorm equals RMSNorm (the RMSNorm oracle
    # is pinned on its own)
    rng = np.random.default_rng(42)
    X = rng.standard_normal((5, 12))
    X = X - X.mean(axis=1, keepdims=True)
    B = rng.standard_normal((12, 7))
    g = rng.uniform(0.5, 2.0, size=12)
    C, mean, rstd = oracle.layernorm_gemm_prenorm(X, B, 1e-5, g)
    Yr, rr = oracle.rms_norm_rows(X, 1e-5, g)
    np.testing.assert_allclose(C, Yr @ B, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(rstd, rr, rtol=1e-12)
    np.testing.assert_allclose(mean, 0.0, atol=1e-15)


def test_prenorm_layernorm_fold_identity():
    # rstd * (A @ B_folded - mean * colsum) + bias reproduces the definition;
    # leaving out the mean term, or taking colsum of B instead of B_folded,
    # does not
    rng = np.random.default_rng(43)
    A = rng.standard_normal((4, 24)) + 3.0
    B = rng.standard_normal((24, 6))
    g = rng.uniform(0.5, 2.0, size=24)
    b = rng.standard_normal(24)
    C, mean, rstd = oracle.layernorm_gemm_prenorm(A, B, 1e-5, g, b)
    Bf, colsum, bias = oracle.layernorm_gemm_fold(B, g, b)
    np.testing.assert_allclose(Bf, g[:, None] * B, rtol=0)
    np.testing.assert_allclose(bias, b @ B, rtol=1e-14)
    got = rstd[:, None] * (A @ Bf - mean[:, None] * colsum[None, :]) + bias[None, :]
    np.testing.assert_allclose(got, C, rtol=1e-10, atol=1e-10)
    wrong = rstd[:, None] * (A @ Bf) + bias[None, :]
    assert np.max(np.abs(wrong - C)) > 1e-1
    wrong = rstd[:, None] * (A @ Bf - mean[:, None] * B.sum(axis=0)[None, :]) + bias[None, :]
    assert np.max(np.abs(wrong - C)) > 1e-1


def _lazy_loss(A, B, G, eps):
    C, _ = oracle.rmsnorm_gemm_lazy(A, B, eps)
    return float((C * G).sum())


@pytest.mark.parametrize("eps", [1e-6, 0.3])
def test_lazy_backward_matches_finite_differences(eps):
    # central differences of the forward oracle's scalar loss sum(C * G),
    # for every entry of dA and dB (truncation error O(h^2) ~ 1e-10 at
    # h = 1e-5; the loss is linear in B, so dB's differences are exact up
    # to rounding)
    rng = np.random.default_rng(51)
    M, K, N = 3, 5, 4
    A = rng.standard_normal((M, K)) * np.array([[0.5], [2.0], [1.0]])
    B = rng.standard_normal((K, N))
    G = rng.standard_normal((M, N))
    dA, dB, rstd = oracle.rmsnorm_gemm_lazy_backward(A, B, G, eps)
    h = 1e-5
    for m in range(M):
        for k in range(K):
            E = np.zeros_like(A)
            E[m, k] = h
            fd = (_lazy_loss(A + E, B, G, eps) - _lazy_loss(A - E, B, G, eps)) / (2 * h)
            assert abs(dA[m, k] - fd) <= 1e-7 * (1 + abs(fd)), (m, k, dA[m, k], fd)
    for k in range(K):
        for n in range(N):
            E = np.zeros_like(B)
            E[k, n] = h
            fd = (_lazy_loss(A, B + E, G, eps) - _lazy_loss(A, B - E, G, eps)) / (2 * h)
            assert abs(dB[k, n] - fd) <= 1e-7 * (1 + abs(fd)), (k, n)
    np.testing.assert_allclose(rstd, oracle.rms_norm_rows(A, eps)[1], rtol=1e-15)


def test_lazy_backward_input_gradient_is_orthogonal_to_rows():
    # with eps = 0 the forward output does not change when a row of A is
    # scaled, so the input gradient has no component along the row itself
    rng = np.random.default_rng(52)
    A = rng.standard_normal((6, 32)) * rng.uniform(0.1, 10, size=(6, 1))
    B = rng.standard_normal((32, 9))
    G = rng.standard_normal((6, 9))
    dA, dB, _ = oracle.rmsnorm_gemm_lazy_backward(A, B, G, 0.0)
    np.testing.assert_allclose((dA * A).sum(axis=1), 0.0, atol=1e-12)
    # and the weight gradient is the normalized A transposed times G
    A_hat, _ = oracle.rms_norm_rows(A, 0.0)
    np.testing.assert_allclose(dB, A_hat.T @ G, rtol=1e-13)


def test_lazy_backward_weight_rows_are_rows_of_the_full_gradient():
    rng = np.random.default_rng(53)
    A = rng.standard_normal((40, 12))
    G = rng.standard_normal((40, 7))
    full = oracle.lazy_backward_weight(A, G, 1e-6)
    rows = np.array([0, 5, 11])
    np.testing.assert_array_equal(oracle.lazy_backward_weight(A, G, 1e-6, rows), full[rows])
    _, dB, _ = oracle.rmsnorm_gemm_lazy_backward(A, rng.standard_normal((12, 7)), G, 1e-6)
    np.testing.assert_array_equal(dB, full)


def test_lazy_is_not_layernorm_prenorm():
    # LayerNorm subtracts the row mean, which breaks the commutation.
    rng = np.random.default_rng(12)
    A = rng.standard_normal((64, 64)) + 2.0     # rows with a clear mean
    B = rng.standard_normal((64, 16)) / 8.0
    C_lazy, _ = oracle.rmsnorm_gemm_lazy(A, B, 1e-6)
    Yl, _, _ = oracle.norm(A, "layer", 1e-6)
    assert oracle.rel_err(C_lazy, oracle.gemm(Yl, B)) > 0.05


# -------------------- reduce-then-apply decomposition (section "Multi-CTA")
@pytest.mark.parametrize("slices", [[128], [64, 64], [50, 30, 48], [1] * 8 + [120]])
def test_sliced_row_statistics_merge_to_full_row(slices):
    # Each slice of a row reduces on its own (count, mean, M2); merging the
    # slices pairwise reproduces the full-row mean and variance the oracle
    # uses.  This is the only exchange the cross-workgroup epilogue needs.
    rng = np.random.default_rng(21)
    X = rng.standard_normal((6, sum(slices))) * 3.0 + 1.5
    _, mean, rstd = oracle.layer_norm_rows(X, 0.0)
    _, rstd_rms = oracle.rms_norm_rows(X, 0.0)
    n_acc = 0
    mean_acc = np.zeros(6)
    m2_acc = np.zeros(6)
    sq_acc = np.zeros(6)
    start = 0
    for w in slices:
        part = X[:, start:start + w]
        start += w
        mt = part.sum(axis=1) / w
        m2t = ((part - mt[:, None]) ** 2).sum(axis=1)
        sq_acc += (part * part).sum(axis=1)
        n_new = n_acc + w
        delta = mt - mean_acc
        mean_acc = mean_acc + delta * (w / n_new)
        m2_acc = m2_acc + m2t + delta * delta * (n_acc * w / n_new)
        n_acc = n_new
    np.testing.assert_allclose(mean_acc, mean, rtol=1e-13)
    np.testing.assert_allclose(1.0 / np.sqrt(m2_acc / n_acc), rstd, rtol=1e-12)
    np.testing.assert_allclose(1.0 / np.sqrt(sq_acc / n_acc), rstd_rms, rtol=1e-13)


def test_rel_err_definition():
    assert oracle.rel_err(np.array([1.0, 2.0]), np.array([1.0, 2.0])) == 0.0
    assert oracle.rel_err(np.array([1.5]), np.array([1.0])) == pytest.approx(0.25)
    assert oracle.rel_err(np.zeros((0, 3)), np.zeros((0, 3))) == 0.0


# ------------------------------------------------------- input generator
def test_workload_inputs_are_seeded_and_shaped():
    w = workloads.WORKLOADS[0]
    x1 = workloads.workload_inputs(w)
    x2 = workloads.workload_inputs(w)
    assert x1.A.shape == (256, 128) and x1.B.shape == (128, 64)
    assert x1.A.dtype == np.uint16 and x1.gamma is None
    np.testing.assert_array_equal(x1.A, x2.A)
    np.testing.assert_array_equal(x1.B, x2.B)
    # row scales 10**U(-1,1): row RMS within [0.1, 10] up to sampling noise
    rms = np.sqrt((oracle.bf16_to_f64(x1.A) ** 2).mean(axis=1))
    assert rms.min() > 0.05 and rms.max() < 15
    # B ~ N(0, 1/K): per-element variance 1/128
    assert abs(oracle.bf16_to_f64(x1.B).var() * 128 - 1.0) < 0.1


def test_workload_table_matches_descriptions():
    names = [w.name for w in workloads.WORKLOADS]
    assert len(names) == 5 and len(set(names)) == 5
    w = workloads.WORKLOAD_BY_NAME["gemm_ln_8192x8192x16384"]
    assert (w.M, w.N, w.K, w.gamma, w.beta, w.eps) == (8192, 16384, 8192, True, True, 1e-5)
    x = workloads.make_inputs(8, 16, 8, seed=0, gamma=True, beta=True)
    g = oracle.bf16_to_f64(x.gamma)
    assert x.gamma.shape == (16,) and x.beta.shape == (16,) and abs(g.mean() - 1.0) < 0.5
