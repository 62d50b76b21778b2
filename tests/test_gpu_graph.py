"""HIP graph capture and replay of the library's calls.

The cross-workgroup kernels tag every exchanged entry with a call counter
that the last workgroup of a call advances on the device, so a captured call
replays with fresh tags and needs no reset between replays; the workspace
reset is a fill kernel, not a memset.  Each graph here is replayed several
times with eager work (a clear of the output, an eager call through the same
workspace, a synchronization) between the replays, and every replay is
checked against the oracle.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import TOL, b_for_layout, down, log, up, wgrad_excess

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import normalization_gemm_amd as ng  # noqa: E402


def _check(name, got_bits, ref):
    err = oracle.rel_err(got_bits, ref)
    log("%s: max rel err %.3e" % (name, err))
    assert np.all(np.isfinite(oracle.bf16_to_f64(got_bits))), name
    assert err <= TOL, (name, err)


def _capture(fn):
    """Run fn once eagerly on a side stream (first-call setup stays outside
    the graph), then capture it."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_graph_replays_cross_workgroup_layernorm():
    M, N, K = 1000, 4096, 256
    x = workloads.make_inputs(M, N, K, seed=61, gamma=True, beta=True)
    A, B, g, b = up(x.A), up(x.B), up(x.gamma), up(x.beta)
    ws = ng.Workspace(ng.ng_workspace_bytes(ng.NG_OP_GEMM_LAYERNORM, M, N, K))
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ref, _, _ = oracle.gemm_layernorm(x.A, x.B, 1e-5, x.gamma, x.beta)
    graph = _capture(lambda: ng.gemm_layernorm(A, B, g, b, eps=1e-5, out=C, workspace=ws))
    for rep in range(4):
        C.zero_()
        graph.replay()
        torch.cuda.synchronize()
        _check("graph replay %d" % rep, down(C), ref)
        D = ng.gemm_layernorm(A, B, g, b, eps=1e-5, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(D.view(torch.int16), C.view(torch.int16))
    assert ws.status() == 0


def test_graph_replays_a_chain_of_forms():
    # one graph: workspace reset, a residual wide-row norm, the Lazy forward
    # and its input gradient (wide rows, sharing the workspace in order)
    M, N, K = 600, 1024, 520
    x = workloads.make_inputs(M, N, K, seed=62, row_scale=True, gamma=True, residual=True,
                              upstream=True)
    A, B, g, R, G = up(x.A), up(x.B), up(x.gamma), up(x.R), up(x.dC)
    nb = max(ng.ng_workspace_bytes(ng.NG_OP_GEMM_ADD_RMSNORM, M, N, K),
             ng.ng_workspace_bytes(ng.NG_OP_RMSNORM_GEMM_LAZY_BWD_INPUT, M, N, K))
    ws = ng.Workspace(nb)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    dA = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    rstd = torch.empty(M, dtype=torch.float32, device="cuda")

    def chain():
        assert ng.ng_workspace_reset(ws.ptr(), ws.nbytes,
                                     torch.cuda.current_stream().cuda_stream) == 0
        ng.gemm_add_rmsnorm(A, B, R, g, eps=1e-6, out=Y, workspace=ws)
        ng.rmsnorm_gemm_lazy(A, B, eps=1e-6, out=C, rstd_out=rstd)
        ng.rmsnorm_gemm_lazy_backward_input(G, B, A, rstd, out=dA, workspace=ws)

    ref_y = oracle.gemm_add_rmsnorm(x.A, x.B, x.R, 1e-6, x.gamma)[0]
    ref_c = oracle.rmsnorm_gemm_lazy(x.A, x.B, 1e-6)[0]
    ref_da = oracle.rmsnorm_gemm_lazy_backward(x.A, x.B, x.dC, 1e-6)[0]
    graph = _capture(chain)
    for rep in range(3):
        for t in (Y, C, dA):
            t.zero_()
        graph.replay()
        torch.cuda.synchronize()
        _check("chain replay %d: residual rmsnorm" % rep, down(Y), ref_y)
        _check("chain replay %d: lazy" % rep, down(C), ref_c)
        _check("chain replay %d: lazy input gradient" % rep, down(dA), ref_da)
    assert ws.status() == 0


def test_graph_replays_the_backward():
    # one graph: the Lazy forward (saving rstd), both gradients regrouped
    # (wide rows: the input gradient also writes rstd * dC, then the plain
    # product), and the weight gradient rebuilt on chip
    M, N, K = 700, 264, 520
    x = workloads.make_inputs(M, N, K, seed=63, row_scale=True, upstream=True)
    A, B, G = up(x.A), up(x.B), up(x.dC)
    ws = ng.Workspace(ng.ng_workspace_bytes(ng.NG_OP_RMSNORM_GEMM_LAZY_BWD_INPUT, M, N, K))
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    dA = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    dB = torch.empty((K, N), dtype=torch.bfloat16, device="cuda")
    dB2 = torch.empty((K, N), dtype=torch.bfloat16, device="cuda")
    sc = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    rstd = torch.empty(M, dtype=torch.float32, device="cuda")

    def chain():
        ng.rmsnorm_gemm_lazy(A, B, eps=1e-6, out=C, rstd_out=rstd)
        ng.rmsnorm_gemm_lazy_backward(G, B, A, rstd, out_dA=dA, out_dB=dB, scratch=sc,
                                      workspace=ws)
        ng.rmsnorm_gemm_lazy_backward_weight(A, G, rstd, out=dB2)

    ref_da = oracle.rmsnorm_gemm_lazy_backward(x.A, x.B, x.dC, 1e-6)[0]
    ref_db = oracle.lazy_backward_weight(x.A, x.dC, 1e-6)
    A_hat, _ = oracle.rms_norm_rows(x.A, 1e-6)
    G64 = oracle.bf16_to_f64(x.dC)
    graph = _capture(chain)
    for rep in range(3):
        for t in (dA, dB, dB2):
            t.zero_()
        graph.replay()
        torch.cuda.synchronize()
        _check("backward replay %d: dA" % rep, down(dA), ref_da)
        for name, t in (("regrouped dB", dB), ("rebuilt dB", dB2)):
            excess = wgrad_excess(oracle.bf16_to_f64(down(t)), ref_db, A_hat, G64)
            log("backward replay %d: %s worst excess %.3e" % (rep, name, excess.max()))
            assert np.all(excess <= 0), (rep, name)
    assert ws.status() == 0


def test_bounded_wait_reports_timeout_with_nan_output_and_recovers():
    # A wait bound of zero polls makes every cross-workgroup wait that does
    # not find its entry at once give up: the kernel still runs to its end,
    # the workspace's error word reports it, every output element and
    # statistic that depends on a failed wait is NaN (and every other one is
    # correct), and after a reset the next call is correct again.  (Forced
    # from the host; no wave is left waiting.)
    M, N, K = 2048, 8192, 2048
    x = workloads.make_inputs(M, N, K, seed=63, gamma=True)
    A, B, g = up(x.A), up(x.B), up(x.gamma)
    ws = ng.Workspace(ng.ng_workspace_bytes(ng.NG_OP_GEMM_RMSNORM, M, N, K))
    rstd = torch.empty(M, dtype=torch.float32, device="cuda")
    with ng.debug_option(ng.NG_DEBUG_WAIT_SPINS, 0):
        C = ng.gemm_rmsnorm(A, B, g, eps=1e-6, workspace=ws, rstd_out=rstd)
        torch.cuda.synchronize()
    status = ws.status()
    log("status after zero-poll waits: %s" % ng.ng_status_string(status))
    assert status == ng._lib.NG_ERR_TIMEOUT
    ref, rref = oracle.gemm_rmsnorm(x.A, x.B, 1e-6, x.gamma)
    got = oracle.bf16_to_f64(down(C))
    bad = np.isnan(got)
    log("elements left NaN by failed waits: %d of %d" % (bad.sum(), bad.size))
    assert bad.any()
    assert np.all(np.isfinite(got[~bad]))
    assert np.max(np.abs(got[~bad] - ref[~bad]) / (1.0 + np.abs(ref[~bad]))) <= TOL
    r = rstd.cpu().numpy().astype(np.float64)
    ok = ~np.isnan(r)
    assert np.all(np.abs(r[ok] - rref[ok]) / rref[ok] <= 1e-3)
    # the workspace works again after a reset
    assert ng.ng_workspace_reset(ws.ptr(), ws.nbytes, torch.cuda.current_stream().cuda_stream) == 0
    C = ng.gemm_rmsnorm(A, B, g, eps=1e-6, workspace=ws)
    torch.cuda.synchronize()
    assert ws.status() == 0
    _check("after reset", down(C), ref)
