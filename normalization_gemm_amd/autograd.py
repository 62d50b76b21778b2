"""Lazy Pre-Norm as a differentiable torch op (RMSNorm without affine, then a
product), for training loops: the forward pass is ng_rmsnorm_gemm_lazy and
keeps the per-row rstd; the backward pass calls the library's gradients
("Free normalization fusion", aixai.ru, section "Lazy Pre-Norm": the
normalized input is never stored and backward rebuilds it from the input and
the saved rstd):

  both gradients   ng_rmsnorm_gemm_lazy_backward (dA fused with dC @ B^T,
                   dB = A^T @ (rstd * dC) as a plain product; needs M x N
                   bf16 of scratch, allocated here)
  input only       ng_rmsnorm_gemm_lazy_backward_input
  weight only      ng_rmsnorm_gemm_lazy_backward_weight (A_hat rebuilt
                   inside the product)

Every step runs in the library's kernels; this module only reshapes and
routes tensors.  Inputs are bf16 CUDA tensors; gradients come back in bf16.
"""
import torch

from . import (rmsnorm_gemm_lazy, rmsnorm_gemm_lazy_backward, rmsnorm_gemm_lazy_backward_input,
               rmsnorm_gemm_lazy_backward_weight)


class _LazyRMSNormGemm(torch.autograd.Function):
    @staticmethod
    def forward(ctx, A, B, eps, b_layout):
        rstd = torch.empty(A.shape[0], dtype=torch.float32, device=A.device)
        C = rmsnorm_gemm_lazy(A, B, eps=eps, b_layout=b_layout, rstd_out=rstd)
        ctx.save_for_backward(A, B, rstd)
        ctx.b_layout = b_layout
        return C

    @staticmethod
    def backward(ctx, dC):
        A, B, rstd = ctx.saved_tensors
        dC = dC.to(torch.bfloat16).contiguous()
        want_a, want_b = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        dA = dB = None
        if want_a and want_b:
            dA, dB = rmsnorm_gemm_lazy_backward(dC, B, A, rstd, b_layout=ctx.b_layout)
        elif want_a:
            dA = rmsnorm_gemm_lazy_backward_input(dC, B, A, rstd, b_layout=ctx.b_layout)
        elif want_b:
            dB = rmsnorm_gemm_lazy_backward_weight(A, dC, rstd, b_layout=ctx.b_layout)
        return dA, dB, None, None


def _apply(x, B, eps, b_layout, n_out):
    if x.dim() < 1:
        raise ValueError("x must have at least one dimension")
    lead = x.shape[:-1]
    A = x.reshape(-1, x.shape[-1]).contiguous()
    C = _LazyRMSNormGemm.apply(A, B.contiguous(), float(eps), b_layout)
    return C.reshape(*lead, n_out)


def lazy_rmsnorm_linear(x, weight, eps: float = 1e-6):
    """rmsnorm(x) @ weight^T over the last dimension of x ([..., K]), with
    weight [N, K] as a torch.nn.Linear stores it; returns [..., N]."""
    return _apply(x, weight, eps, "nk", weight.shape[0])


def lazy_rmsnorm_matmul(x, B, eps: float = 1e-6):
    """rmsnorm(x) @ B over the last dimension of x ([..., K]), with B [K, N];
    returns [..., N]."""
    return _apply(x, B, eps, "kn", B.shape[1])
