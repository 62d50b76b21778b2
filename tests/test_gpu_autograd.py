"""Lazy Pre-Norm through torch autograd (normalization_gemm_amd.autograd):
the forward output and the gradients that autograd routes to the library's
backward calls, against the float64 oracle on the same seeded inputs.  Bars
as in the parity tests: outputs and input gradients within
1e-2 * (1 + |oracle|); weight gradients with the statistical allowance for
the bf16 roundings of the normalized input (gpu_util.wgrad_excess)."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import TOL, b_for_layout, down, log, up, wgrad_excess

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

from normalization_gemm_amd.autograd import lazy_rmsnorm_linear, lazy_rmsnorm_matmul  # noqa: E402


def _check(name, got_bits, ref):
    err = oracle.rel_err(got_bits, ref)
    log("%s: max rel err %.3e" % (name, err))
    assert np.all(np.isfinite(oracle.bf16_to_f64(got_bits))), name
    assert err <= TOL, (name, err)


def _check_wgrad(name, got_bits, ref, x):
    A_hat, _ = oracle.rms_norm_rows(x.A, 1e-6)
    got = oracle.bf16_to_f64(got_bits)
    excess = wgrad_excess(got, ref, A_hat, oracle.bf16_to_f64(x.dC))
    log("%s: worst excess over the bar %.3e" % (name, excess.max()))
    assert np.all(np.isfinite(got)), name
    assert np.all(excess <= 0), (name, excess.max())


def _run(x, shape, layout, grad_x, grad_w):
    K = x.A.shape[1]
    N = x.B.shape[1]
    xt = up(x.A).reshape(*shape, K).requires_grad_(grad_x)
    w = up(b_for_layout(x.B, layout)).requires_grad_(grad_w)
    f = lazy_rmsnorm_linear if layout == "nk" else lazy_rmsnorm_matmul
    y = f(xt, w, eps=1e-6)
    assert tuple(y.shape) == tuple(shape) + (N,)
    y.backward(up(x.dC).reshape(*shape, N))
    torch.cuda.synchronize()
    return y, xt.grad, w.grad


@pytest.mark.parametrize("layout", ["kn", "nk"])
@pytest.mark.parametrize("grads", ["both", "input", "weight"])
def test_lazy_rmsnorm_autograd(layout, grads):
    # x [2, 150, 264] -> 300 rows; N = 520: several tiles and ragged tails
    shape, K, N = (2, 150), 264, 520
    M = shape[0] * shape[1]
    x = workloads.make_inputs(M, N, K, seed=97, row_scale=True, upstream=True)
    gx, gw = grads in ("both", "input"), grads in ("both", "weight")
    log("autograd lazy %s, gradients: %s" % (layout, grads))
    y, dx, dw = _run(x, shape, layout, gx, gw)
    C_ref, _ = oracle.rmsnorm_gemm_lazy(x.A, x.B, 1e-6)
    _check("forward", down(y.reshape(M, N)), C_ref)
    assert (dx is not None) == gx and (dw is not None) == gw
    if gx:
        dA_ref, _, _ = oracle.rmsnorm_gemm_lazy_backward(x.A, x.B, x.dC, 1e-6)
        assert tuple(dx.shape) == shape + (K,)
        _check("input gradient", down(dx.reshape(M, K)), dA_ref)
    if gw:
        dB_ref = oracle.lazy_backward_weight(x.A, x.dC, 1e-6)
        got = down(dw) if layout == "kn" else np.ascontiguousarray(down(dw).T)
        _check_wgrad("weight gradient", got, dB_ref, x)


def test_lazy_rmsnorm_autograd_in_a_chain():
    # the op between two torch ops: the upstream gradient arrives as a
    # non-contiguous view and the input gradient flows on to a leaf
    M, K, N = 96, 128, 192
    x = workloads.make_inputs(M, N, K, seed=98, row_scale=True, upstream=True)
    leaf = up(x.A).float().requires_grad_(True)
    w = up(b_for_layout(x.B, "nk")).requires_grad_(True)
    y = lazy_rmsnorm_linear(leaf.to(torch.bfloat16), w, eps=1e-6)
    # y^T then a product with dC^T: d/dy of sum(y^T * dC^T) is dC, handed
    # back as the transpose of a transposed tensor
    (y.t() * up(x.dC).t()).float().sum().backward()
    torch.cuda.synchronize()
    dA_ref, _, _ = oracle.rmsnorm_gemm_lazy_backward(x.A, x.B, x.dC, 1e-6)
    _check("chained input gradient", down(leaf.grad.to(torch.bfloat16)), dA_ref)
    dB_ref = oracle.lazy_backward_weight(x.A, x.dC, 1e-6)
    _check_wgrad("chained weight gradient", np.ascontiguousarray(down(w.grad).T), dB_ref, x)
