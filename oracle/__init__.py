"""CPU oracle for the norm-fused GEMM path -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The product path (the HIP library and its
Python binding) never calls it and shares no code with it.

Everything here is plain NumPy in float64 on the exact bfloat16 input values
(bfloat16 is a subset of float64, so inputs carry no rounding).  Each routine
computes the plain definition of its operation, with no blocking, fusion or
reordering; the only library primitive used is NumPy's matrix product.
"""
from .normgemm_oracle import (  # noqa: F401
    bf16_to_f64,
    f64_to_bf16_bits,
    gemm,
    rms_norm_rows,
    layer_norm_rows,
    rmsnorm_gemm_lazy,
    rmsnorm_gemm_lazy_affine,
    lazy_fold_affine,
    gemm_rmsnorm,
    gemm_layernorm,
    gemm_add_rmsnorm,
    layernorm_gemm_prenorm,
    layernorm_gemm_fold,
    rmsnorm_gemm_lazy_backward,
    lazy_backward_weight,
    gemm_add_layernorm,
    norm,
    rel_err,
)
