"""Helpers for the GPU tests: move bf16 bit arrays to and from the device."""
import numpy as np

TOL = 1e-2  # max |gpu - oracle| / (1 + |oracle|) for bf16 outputs with fp32 accumulation


def up(bits, dev="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def down(t):
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def b_for_layout(Bbits, layout):
    """Logical [K, N] bits -> the array passed for that layout."""
    return Bbits if layout == "kn" else np.ascontiguousarray(Bbits.T)


def log(msg):
    print(msg, flush=True)


def wgrad_excess(got, ref, A_hat, dC):
    """How far a weight gradient dB = A_hat^T dC (rows of dB = columns of
    A_hat) exceeds its bar, per element (<= 0 everywhere means it passes).

    The kernel multiplies A_hat rounded to bf16 (nearest even, the rounding a
    stored A_hat has) -- or, regrouped, A times rstd * dC rounded to bf16 --
    so each product a_m * g_m carries an independent relative error of at
    most 2^-9, roughly uniform: the sum over the M rows
    errs by about 2^-9 / sqrt(3) * sqrt(sum_m (a_m g_m)^2) (one standard
    deviation).  The bar is the plain 1e-2 * (1 + |ref|) plus 8 * 2^-9 times
    that root sum of squares (about 14 standard deviations, so a correct
    kernel never reaches it, while a systematic error of 2 % does wherever
    |ref| is above ~1.6 standard deviations of dB).  Arguments are float64:
    got, ref [K', N]; A_hat [M, K']; dC [M, N].
    """
    rss = np.sqrt((A_hat * A_hat).T @ (dC * dC))
    return np.abs(got - ref) - TOL * (1.0 + np.abs(ref)) - 8.0 * 2.0 ** -9 * rss
