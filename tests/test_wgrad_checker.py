"""The weight-gradient bar used by the GPU tests, exercised on the CPU.

dB = A_hat^T dC sums M products of the bf16-rounded normalized A; the bar
(tests/gpu_util.py, wgrad_excess) adds a statistical allowance for those
roundings to the plain 1e-2 * (1 + |ref|).  It must accept a gradient formed
exactly as the kernel forms it (A_hat rounded to bf16, then the products) and
reject a systematic error of 2 %.
"""
import numpy as np

import oracle
import workloads
from gpu_util import wgrad_excess

M, N, K = 32768, 64, 64


def _case():
    x = workloads.make_inputs(M, N, K, seed=5, row_scale=True, upstream=True)
    A_hat, _ = oracle.rms_norm_rows(x.A, 1e-6)
    dC = oracle.bf16_to_f64(x.dC)
    ref = oracle.lazy_backward_weight(x.A, x.dC, 1e-6)
    return A_hat, dC, ref


def test_accepts_the_gradient_of_bf16_rounded_a_hat():
    A_hat, dC, ref = _case()
    A_r = oracle.bf16_to_f64(oracle.f64_to_bf16_bits(A_hat))   # the stored-A_hat rounding
    got = oracle.bf16_to_f64(oracle.f64_to_bf16_bits(A_r.T @ dC))  # bf16 output
    assert np.all(wgrad_excess(got, ref, A_hat, dC) <= 0)


def test_rejects_a_two_percent_error():
    A_hat, dC, ref = _case()
    got = oracle.bf16_to_f64(oracle.f64_to_bf16_bits(1.02 * ref))
    excess = wgrad_excess(got, ref, A_hat, dC)
    assert np.any(excess > 0)
    # and on a good share of the elements, not just the largest one
    assert np.mean(excess > 0) > 0.05


def test_rejects_one_k_tile_left_unscaled():
    # a plausible kernel slip: one 64-row slice of the reduction multiplied by
    # A instead of A_hat
    x = workloads.make_inputs(M, N, K, seed=6, row_scale=True, upstream=True)
    A_hat, _ = oracle.rms_norm_rows(x.A, 1e-6)
    dC = oracle.bf16_to_f64(x.dC)
    ref = A_hat.T @ dC
    bad = A_hat.copy()
    bad[:64] = oracle.bf16_to_f64(x.A)[:64]
    got = oracle.bf16_to_f64(oracle.f64_to_bf16_bits(bad.T @ dC))
    assert np.any(wgrad_excess(got, ref, A_hat, dC) > 0)
