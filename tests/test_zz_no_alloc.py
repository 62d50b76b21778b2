"""ng_gemm_layernorm_noalloc through the C ABI: the same outputs as
ng_gemm_layernorm with a caller workspace, call after call through the one
static scratch array (the second call smaller than the first, then the first
shape again), on the cross-workgroup and the row-local strategy."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import TOL, down, log, up

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import normalization_gemm_amd as ng  # noqa: E402
from normalization_gemm_amd import _lib  # noqa: E402


def _run_both(M, N, K, seed):
    x = workloads.make_inputs(M, N, K, seed=seed, gamma=True, beta=True)
    A, B, g, b = up(x.A), up(x.B), up(x.gamma), up(x.beta)
    st = torch.cuda.current_stream().cuda_stream
    # reference: the workspace variant, its own zeroed workspace
    ws = ng.Workspace(max(256, ng.ng_workspace_bytes(ng.NG_OP_GEMM_LAYERNORM, M, N, K)))
    C_ws = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    mean_ws = torch.empty(M, dtype=torch.float32, device="cuda")
    rstd_ws = torch.empty(M, dtype=torch.float32, device="cuda")
    assert _lib.ng_gemm_layernorm(A.data_ptr(), B.data_ptr(), g.data_ptr(), b.data_ptr(),
                                  C_ws.data_ptr(), M, N, K, 0, 1e-5, mean_ws.data_ptr(),
                                  rstd_ws.data_ptr(), ws.ptr(), ws.nbytes, st) == 0
    # the no-allocation variant
    C = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    mean = torch.full((M,), 7.0, dtype=torch.float32, device="cuda")
    rstd = torch.full((M,), 7.0, dtype=torch.float32, device="cuda")
    status = _lib.ng_gemm_layernorm_noalloc(A.data_ptr(), B.data_ptr(), g.data_ptr(),
                                            b.data_ptr(), C.data_ptr(), M, N, K, 0, 1e-5,
                                            mean.data_ptr(), rstd.data_ptr(), st)
    assert status == 0, _lib.ng_last_error()
    torch.cuda.synchronize()
    assert ws.status() == 0
    ref, _, _ = oracle.gemm_layernorm(x.A, x.B, 1e-5, x.gamma, x.beta)
    err = oracle.rel_err(down(C), ref)
    log("noalloc M=%d N=%d K=%d: max rel err %.3e" % (M, N, K, err))
    assert np.all(np.isfinite(oracle.bf16_to_f64(down(C))))
    assert err <= TOL
    assert torch.equal(C.view(torch.int16), C_ws.view(torch.int16))
    assert torch.equal(mean, mean_ws) and torch.equal(rstd, rstd_ws)


def test_noalloc_matches_the_workspace_variant_call_after_call():
    # cross-workgroup rows: 16 column tiles, several rounds; then a smaller
    # shape (fewer row blocks and column tiles); then the first shape again
    _run_both(5000, 4096, 264, seed=71)
    _run_both(700, 1000, 136, seed=72)
    _run_both(5000, 4096, 264, seed=73)


def test_noalloc_row_local_rows():
    # rows of one workgroup tile need no scratch
    _run_both(1000, 128, 200, seed=74)
    _run_both(300, 256, 64, seed=75)


def test_noalloc_takes_many_rows():
    # the scratch holds one round of row blocks, whatever M is: 20000 rows of
    # 16384 columns (more than fit a per-row-block layout of 16 MiB)
    _run_both(20000, 16384, 64, seed=76)
