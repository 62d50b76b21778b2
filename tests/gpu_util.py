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


def sample_rows(M, n, seed=0):
    rng = np.random.default_rng(seed)
    rows = set([0, M - 1, M // 2])
    rows.update(int(r) for r in rng.integers(0, M, size=n))
    return np.array(sorted(rows))


def log(msg):
    print(msg, flush=True)
