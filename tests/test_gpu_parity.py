"""Parity of the HIP path against the CPU oracle, through the C ABI.

Every fused op is compared element by element with the float64 oracle on the
same seeded bf16 inputs: small shapes that span several tiles with ragged
tails, and every named workload at full size (every output element and every
statistic output).  Bar: |gpu - oracle| <= 1e-2 * (1 + |oracle|) everywhere;
fp32 statistic outputs within 1e-3 relative.
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


def _check_wgrad(name, got_bits, ref, A_bits, dC_bits, eps, rows=None):
    # dB sums M products of the bf16-rounded normalized A: on top of the
    # plain bar, a statistical allowance for those roundings (wgrad_excess)
    A_hat, _ = oracle.rms_norm_rows(A_bits, eps)
    if rows is not None:
        A_hat = A_hat[:, rows]
    got = oracle.bf16_to_f64(got_bits)
    excess = wgrad_excess(got, ref, A_hat, oracle.bf16_to_f64(dC_bits))
    log("%s: max rel err %.3e, worst excess over the bar %.3e" % (
        name, oracle.rel_err(got_bits, ref), excess.max()))
    assert np.all(np.isfinite(got)), name
    assert np.all(excess <= 0), (name, excess.max())


def _check_stat(name, got, ref):
    got = got.cpu().numpy().astype(np.float64)
    rel = np.max(np.abs(got - ref) / np.abs(ref))
    log("%s: stat max rel err %.3e" % (name, rel))
    assert rel <= 1e-3, (name, rel)


SMALL_LAZY = [(256, 64, 128), (300, 136, 200), (1, 8, 8), (77, 128, 72), (513, 520, 264),
              (130, 256, 64)]


@pytest.mark.parametrize("layout", ["kn", "nk"])
@pytest.mark.parametrize("M,N,K", SMALL_LAZY)
def test_lazy_small(M, N, K, layout):
    log("lazy M=%d N=%d K=%d %s" % (M, N, K, layout))
    x = workloads.make_inputs(M, N, K, seed=M + N + K, row_scale=True)
    rstd = torch.empty(M, dtype=torch.float32, device="cuda")
    C = ng.rmsnorm_gemm_lazy(up(x.A), up(b_for_layout(x.B, layout)), eps=1e-6, b_layout=layout,
                             rstd_out=rstd)
    torch.cuda.synchronize()
    ref, rref = oracle.rmsnorm_gemm_lazy(x.A, x.B, 1e-6)
    _check("lazy", down(C), ref)
    _check_stat("lazy rstd", rstd, rref)


SMALL_EPI = [(300, 128, 96), (64, 64, 64), (1000, 256, 136), (129, 200, 520), (517, 1000, 200),
             (260, 264, 64), (33, 2048, 128), (700, 512, 256)]


@pytest.mark.parametrize("affine", [False, True])
@pytest.mark.parametrize("layout", ["kn", "nk"])
@pytest.mark.parametrize("M,N,K", SMALL_EPI)
def test_gemm_layernorm_small(M, N, K, layout, affine):
    log("gemm_layernorm M=%d N=%d K=%d %s affine=%s" % (M, N, K, layout, affine))
    x = workloads.make_inputs(M, N, K, seed=3 * M + N + K, gamma=affine, beta=affine)
    mean = torch.empty(M, dtype=torch.float32, device="cuda")
    rstd = torch.empty(M, dtype=torch.float32, device="cuda")
    g = up(x.gamma) if affine else None
    b = up(x.beta) if affine else None
    C = ng.gemm_layernorm(up(x.A), up(b_for_layout(x.B, layout)), g, b, eps=1e-5,
                          b_layout=layout, mean_out=mean, rstd_out=rstd)
    torch.cuda.synchronize()
    ref, mref, rref = oracle.gemm_layernorm(x.A, x.B, 1e-5, x.gamma, x.beta)
    _check("gemm_layernorm", down(C), ref)
    _check_stat("rstd", rstd, rref)
    got_mean = mean.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(got_mean - mref) / (1.0 + np.abs(mref))) <= 1e-3


@pytest.mark.parametrize("affine", [False, True])
@pytest.mark.parametrize("layout", ["kn", "nk"])
@pytest.mark.parametrize("M,N,K", SMALL_EPI)
def test_gemm_rmsnorm_small(M, N, K, layout, affine):
    log("gemm_rmsnorm M=%d N=%d K=%d %s affine=%s" % (M, N, K, layout, affine))
    x = workloads.make_inputs(M, N, K, seed=5 * M + N + K, gamma=affine)
    rstd = torch.empty(M, dtype=torch.float32, device="cuda")
    g = up(x.gamma) if affine else None
    C = ng.gemm_rmsnorm(up(x.A), up(b_for_layout(x.B, layout)), g, eps=1e-6, b_layout=layout,
                        rstd_out=rstd)
    torch.cuda.synchronize()
    ref, rref = oracle.gemm_rmsnorm(x.A, x.B, 1e-6, x.gamma)
    _check("gemm_rmsnorm", down(C), ref)
    _check_stat("rstd", rstd, rref)


@pytest.mark.parametrize("layout", ["kn", "nk"])
@pytest.mark.parametrize("M,N,K", [(256, 64, 128), (300, 136, 200), (513, 520, 264), (64, 128, 8)])
def test_gemm_small(M, N, K, layout):
    x = workloads.make_inputs(M, N, K, seed=7 + M)
    C = ng.gemm(up(x.A), up(b_for_layout(x.B, layout)), b_layout=layout)
    torch.cuda.synchronize()
    _check("gemm %dx%dx%d" % (M, N, K), down(C), oracle.gemm(x.A, x.B))


@pytest.mark.parametrize("kind", ["rms", "layer"])
@pytest.mark.parametrize("rows,cols", [(1, 8), (37, 128), (300, 136), (65, 1000), (17, 4096),
                                       (9, 8200), (3, 16384), (2, 65536)])
def test_norm_small(rows, cols, kind):
    x = workloads.make_inputs(1, cols, 8, seed=rows + cols, gamma=True, beta=True)
    rng = np.random.default_rng(rows * cols)
    Xbits = workloads.f32_to_bf16_bits(
        (rng.standard_normal((rows, cols)) * 2.0 + 0.5).astype(np.float32))
    beta = up(x.beta) if kind == "layer" else None
    mean = torch.empty(rows, dtype=torch.float32, device="cuda") if kind == "layer" else None
    rstd = torch.empty(rows, dtype=torch.float32, device="cuda")
    Y = ng.norm(up(Xbits), kind, up(x.gamma), beta, eps=1e-5, mean_out=mean, rstd_out=rstd)
    torch.cuda.synchronize()
    ref, mref, rref = oracle.norm(Xbits, kind, 1e-5, x.gamma, x.beta if kind == "layer" else None)
    _check("norm %s %dx%d" % (kind, rows, cols), down(Y), ref)
    _check_stat("norm rstd", rstd, rref)


# -------------------------------------------- Lazy Pre-Norm with folded affine
@pytest.mark.parametrize("layout", ["kn", "nk"])
@pytest.mark.parametrize("M,N,K", [(256, 64, 128), (300, 136, 200), (77, 128, 72),
                                   (513, 520, 264), (1, 8, 8)])
def test_lazy_affine_small(M, N, K, layout):
    log("lazy affine M=%d N=%d K=%d %s" % (M, N, K, layout))
    x = workloads.make_inputs(M, N, K, seed=M + 2 * N + K, row_scale=True, gamma=True,
                              beta=True, gamma_len=K)
    B = up(b_for_layout(x.B, layout))
    Bf, bias = ng.lazy_fold_affine(B, up(x.gamma), up(x.beta), b_layout=layout)
    rstd = torch.empty(M, dtype=torch.float32, device="cuda")
    C = ng.rmsnorm_gemm_lazy_affine(up(x.A), Bf, bias, eps=1e-6, b_layout=layout,
                                    rstd_out=rstd)
    torch.cuda.synchronize()
    # the fold: diag(gamma) B rounded once to bf16 (bit-exact), bias in fp32
    Bf_ref, bias_ref = oracle.lazy_fold_affine(x.B, x.gamma, x.beta)
    want = oracle.f64_to_bf16_bits(Bf_ref)
    got = down(Bf)
    if layout == "nk":
        got = got.T
    assert np.array_equal(got, want)
    Bd = np.abs(oracle.bf16_to_f64(x.B))
    bound = K * 6e-8 * (np.abs(oracle.bf16_to_f64(x.beta)) @ Bd) + 1e-30
    assert np.all(np.abs(bias.cpu().numpy().astype(np.float64) - bias_ref) <= bound)
    ref, rref = oracle.rmsnorm_gemm_lazy_affine(x.A, x.B, 1e-6, x.gamma, x.beta)
    _check("lazy affine", down(C), ref)
    _check_stat("lazy affine rstd", rstd, rref)


def test_lazy_affine_without_bias_is_lazy_on_folded_weights():
    M, N, K = 600, 512, 256
    x = workloads.make_inputs(M, N, K, seed=5, row_scale=True, gamma=True, gamma_len=K)
    Bf, _ = ng.lazy_fold_affine(up(x.B), up(x.gamma), None)
    C1 = ng.rmsnorm_gemm_lazy_affine(up(x.A), Bf, None, eps=1e-6)
    C0 = ng.rmsnorm_gemm_lazy(up(x.A), Bf, eps=1e-6)
    torch.cuda.synchronize()
    assert torch.equal(C1.view(torch.int16), C0.view(torch.int16))
    ref, _ = oracle.rmsnorm_gemm_lazy_affine(x.A, x.B, 1e-6, x.gamma)
    _check("lazy affine gamma only", down(C1), ref)


@pytest.mark.parametrize("rows,cols", [(37, 128), (65, 1000), (9, 8200)])
def test_norm_rms_with_beta(rows, cols):
    x = workloads.make_inputs(1, cols, 8, seed=rows + 3 * cols, gamma=True, beta=True)
    rng = np.random.default_rng(rows * cols + 1)
    Xbits = workloads.f32_to_bf16_bits(
        (rng.standard_normal((rows, cols)) * 2.0 + 0.5).astype(np.float32))
    Y = ng.norm(up(Xbits), "rms", up(x.gamma), up(x.beta), eps=1e-6)
    torch.cuda.synchronize()
    ref, _, _ = oracle.norm(Xbits, "rms", 1e-6, x.gamma, x.beta)
    _check("norm rms beta %dx%d" % (rows, cols), down(Y), ref)


# ------------------------------------------- persistent grids, several rounds
# The 256x256-tile kernels run as persistent grids of one workgroup per
# resident slot: these shapes give some workgroups two tiles (more tiles than
# slots), ragged M, N and K tails, and, for the cross-workgroup norm, several
# rounds of row blocks, more than 64 column tiles per row (several partials
# per merging lane) and the widest row the grid holds (one row per merging
# workgroup).

@pytest.mark.parametrize("layout", ["kn", "nk"])
def test_persistent_gemm_and_lazy_multi_tile_ragged(layout):
    M, N, K = 256 * 18 + 37, 256 * 16 + 72, 200
    log("persistent gemm/lazy M=%d N=%d K=%d %s" % (M, N, K, layout))
    x = workloads.make_inputs(M, N, K, seed=11, row_scale=True)
    A, B = up(x.A), up(b_for_layout(x.B, layout))
    C = ng.gemm(A, B, b_layout=layout)
    rstd = torch.empty(M, dtype=torch.float32, device="cuda")
    L = ng.rmsnorm_gemm_lazy(A, B, eps=1e-6, b_layout=layout, rstd_out=rstd)
    torch.cuda.synchronize()
    _check("persistent gemm", down(C), oracle.gemm(x.A, x.B))
    ref, rref = oracle.rmsnorm_gemm_lazy(x.A, x.B, 1e-6)
    _check("persistent lazy", down(L), ref)
    _check_stat("persistent lazy rstd", rstd, rref)


@pytest.mark.parametrize("kind,layout", [("layer", "kn"), ("rms", "nk")])
def test_cross_workgroup_several_rounds_ragged(kind, layout):
    # 10 column tiles -> 25 row blocks per round; 31 row blocks -> 2 rounds
    M, N, K = 256 * 30 + 100, 256 * 9 + 24, 136
    log("xwg rounds %s M=%d N=%d K=%d %s" % (kind, M, N, K, layout))
    x = workloads.make_inputs(M, N, K, seed=21, gamma=True, beta=kind == "layer")
    A, B = up(x.A), up(b_for_layout(x.B, layout))
    rstd = torch.empty(M, dtype=torch.float32, device="cuda")
    if kind == "layer":
        mean = torch.empty(M, dtype=torch.float32, device="cuda")
        C = ng.gemm_layernorm(A, B, up(x.gamma), up(x.beta), eps=1e-5, b_layout=layout,
                              mean_out=mean, rstd_out=rstd)
        torch.cuda.synchronize()
        ref, mref, rref = oracle.gemm_layernorm(x.A, x.B, 1e-5, x.gamma, x.beta)
        got_mean = mean.cpu().numpy().astype(np.float64)
        assert np.max(np.abs(got_mean - mref) / (1.0 + np.abs(mref))) <= 1e-3
    else:
        C = ng.gemm_rmsnorm(A, B, up(x.gamma), eps=1e-6, b_layout=layout, rstd_out=rstd)
        torch.cuda.synchronize()
        ref, rref = oracle.gemm_rmsnorm(x.A, x.B, 1e-6, x.gamma)
    _check("xwg rounds %s" % kind, down(C), ref)
    _check_stat("xwg rounds rstd", rstd, rref)


@pytest.mark.parametrize("kind", ["layer", "rms"])
@pytest.mark.parametrize("M,N", [(300, 256 * 65 + 8), (100, 65536)])
def test_cross_workgroup_many_column_tiles(M, N, kind):
    K = 64
    log("xwg wide %s M=%d N=%d K=%d" % (kind, M, N, K))
    x = workloads.make_inputs(M, N, K, seed=N % 1000 + M, gamma=True, beta=kind == "layer")
    A, B = up(x.A), up(x.B)
    rstd = torch.empty(M, dtype=torch.float32, device="cuda")
    if kind == "layer":
        C = ng.gemm_layernorm(A, B, up(x.gamma), up(x.beta), eps=1e-5, rstd_out=rstd)
        torch.cuda.synchronize()
        ref, _, rref = oracle.gemm_layernorm(x.A, x.B, 1e-5, x.gamma, x.beta)
    else:
        C = ng.gemm_rmsnorm(A, B, up(x.gamma), eps=1e-6, rstd_out=rstd)
        torch.cuda.synchronize()
        ref, rref = oracle.gemm_rmsnorm(x.A, x.B, 1e-6, x.gamma)
    _check("xwg wide %s %dx%d" % (kind, M, N), down(C), ref)
    _check_stat("xwg wide rstd", rstd, rref)


# -------------------------------------- residual add before the post-norm
def _residual_call(kind, x, layout, eps, s_out=None, out=None, R=None, stats=True):
    """Run gemm_add_{layer,rms}norm on the inputs; return (C, mean, rstd)."""
    M = x.A.shape[0]
    A, B = up(x.A), up(b_for_layout(x.B, layout))
    R = up(x.R) if R is None else R
    g = up(x.gamma) if x.gamma is not None else None
    rstd = torch.empty(M, dtype=torch.float32, device="cuda") if stats else None
    mean = None
    if kind == "layer":
        b = up(x.beta) if x.beta is not None else None
        mean = torch.empty(M, dtype=torch.float32, device="cuda") if stats else None
        C = ng.gemm_add_layernorm(A, B, R, g, b, eps=eps, b_layout=layout, out=out, s_out=s_out,
                                  mean_out=mean, rstd_out=rstd)
    else:
        C = ng.gemm_add_rmsnorm(A, B, R, g, eps=eps, b_layout=layout, out=out, s_out=s_out,
                                rstd_out=rstd)
    return C, mean, rstd


def _residual_ref(kind, x, eps, rows=None):
    A = x.A if rows is None else x.A[rows]
    R = x.R if rows is None else x.R[rows]
    if kind == "layer":
        Y, mean, rstd, S = oracle.gemm_add_layernorm(A, x.B, R, eps, x.gamma, x.beta)
    else:
        Y, rstd, S = oracle.gemm_add_rmsnorm(A, x.B, R, eps, x.gamma)
        mean = None
    return Y, mean, rstd, S


# row-local (N <= 128, N <= 256) and cross-workgroup shapes, ragged in M, N, K
SMALL_RES = [(300, 128, 96), (64, 64, 64), (1000, 256, 136), (129, 200, 520), (517, 1000, 200),
             (33, 2048, 128), (260, 264, 64)]


@pytest.mark.parametrize("kind", ["layer", "rms"])
@pytest.mark.parametrize("layout", ["kn", "nk"])
@pytest.mark.parametrize("M,N,K", SMALL_RES)
def test_gemm_add_norm_small(M, N, K, layout, kind):
    log("gemm_add_%snorm M=%d N=%d K=%d %s" % (kind, M, N, K, layout))
    affine = (M + N) % 2 == 0
    x = workloads.make_inputs(M, N, K, seed=5 * M + N + K, gamma=affine,
                              beta=affine and kind == "layer", residual=True)
    S_dev = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    eps = 1e-5 if kind == "layer" else 1e-6
    C, mean, rstd = _residual_call(kind, x, layout, eps, s_out=S_dev)
    torch.cuda.synchronize()
    Y, mref, rref, S = _residual_ref(kind, x, eps)
    _check("gemm_add_%snorm" % kind, down(C), Y)
    _check("gemm_add s_out", down(S_dev), S)
    _check_stat("gemm_add rstd", rstd, rref)
    if mean is not None:
        got_mean = mean.cpu().numpy().astype(np.float64)
        assert np.max(np.abs(got_mean - mref) / (1.0 + np.abs(mref))) <= 1e-3


@pytest.mark.parametrize("kind", ["layer", "rms"])
@pytest.mark.parametrize("N", [128, 256, 1000])
def test_gemm_add_norm_in_place(N, kind):
    # R may be the buffer of the sum output or of the normalized output
    M, K = 300, 72
    x = workloads.make_inputs(M, N, K, seed=N + 7, gamma=True, beta=True, residual=True)
    eps = 1e-5
    Y, _, _, S = _residual_ref(kind, x, eps)
    R1 = up(x.R)
    C1, _, _ = _residual_call(kind, x, "kn", eps, s_out=R1, R=R1, stats=False)
    R2 = up(x.R)
    C2, _, _ = _residual_call(kind, x, "kn", eps, out=R2, R=R2, stats=False)
    torch.cuda.synchronize()
    _check("in place: s_out is R", down(R1), S)
    _check("in place: s_out is R (C)", down(C1), Y)
    _check("in place: out is R", down(R2), Y)
    assert C2.data_ptr() == R2.data_ptr()


def test_gemm_add_norm_cross_workgroup_rounds_ragged():
    # 10 column tiles -> 25 row blocks per round; 31 row blocks -> 2 rounds
    M, N, K = 256 * 30 + 100, 256 * 9 + 24, 136
    for kind, layout in (("layer", "nk"), ("rms", "kn")):
        log("xwg residual rounds %s M=%d N=%d K=%d %s" % (kind, M, N, K, layout))
        x = workloads.make_inputs(M, N, K, seed=23, gamma=True, beta=kind == "layer",
                                  residual=True)
        eps = 1e-5 if kind == "layer" else 1e-6
        C, _, rstd = _residual_call(kind, x, layout, eps)
        torch.cuda.synchronize()
        Y, _, rref, _ = _residual_ref(kind, x, eps)
        _check("xwg residual rounds %s" % kind, down(C), Y)
        _check_stat("xwg residual rstd", rstd, rref)


def test_gemm_add_norm_cross_workgroup_deep_k():
    # k-loops of 8 or more 32-deep k-tiles stream R into the stages under
    # their last k-tiles (B[K,N]); 10 column tiles, 2 rounds, ragged M, N, K
    M, N, K = 256 * 30 + 100, 256 * 9 + 24, 520
    for kind, layout in (("layer", "kn"), ("rms", "kn"), ("rms", "nk")):
        log("xwg residual deep k %s M=%d N=%d K=%d %s" % (kind, M, N, K, layout))
        x = workloads.make_inputs(M, N, K, seed=29, gamma=True, beta=kind == "layer",
                                  residual=True)
        eps = 1e-5 if kind == "layer" else 1e-6
        S_dev = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        C, mean, rstd = _residual_call(kind, x, layout, eps, s_out=S_dev)
        torch.cuda.synchronize()
        Y, mref, rref, S = _residual_ref(kind, x, eps)
        _check("xwg residual deep k %s" % kind, down(C), Y)
        _check("xwg residual deep k s_out", down(S_dev), S)
        _check_stat("xwg residual deep k rstd", rstd, rref)
        if mean is not None:
            got_mean = mean.cpu().numpy().astype(np.float64)
            assert np.max(np.abs(got_mean - mref) / (1.0 + np.abs(mref))) <= 1e-3


def test_gemm_add_norm_zero_residual_matches_plain():
    # R = 0: the residual forms give exactly the plain epilogue's result
    for N in (128, 1000):
        x = workloads.make_inputs(200, N, 64, seed=N, gamma=True, beta=True)
        A, B, g, b = up(x.A), up(x.B), up(x.gamma), up(x.beta)
        Z = torch.zeros((200, N), dtype=torch.bfloat16, device="cuda")
        C0 = ng.gemm_layernorm(A, B, g, b, eps=1e-5)
        C1 = ng.gemm_add_layernorm(A, B, Z, g, b, eps=1e-5)
        R0 = ng.gemm_rmsnorm(A, B, g, eps=1e-6)
        R1 = ng.gemm_add_rmsnorm(A, B, Z, g, eps=1e-6)
        torch.cuda.synchronize()
        assert torch.equal(C0.view(torch.int16), C1.view(torch.int16)), N
        assert torch.equal(R0.view(torch.int16), R1.view(torch.int16)), N


@pytest.mark.parametrize("kind", ["rms", "layer"])
@pytest.mark.parametrize("rows,cols", [(1, 8), (37, 128), (300, 136), (65, 1000), (9, 8200)])
def test_add_norm_small(rows, cols, kind):
    log("add_norm %s rows=%d cols=%d" % (kind, rows, cols))
    x = workloads.make_inputs(rows, cols, 8, seed=rows * 3 + cols, gamma=True, beta=True,
                              residual=True)
    X = workloads.f32_to_bf16_bits(np.random.default_rng(rows).standard_normal(
        (rows, cols), dtype=np.float32))
    Sd = torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda")
    rstd = torch.empty(rows, dtype=torch.float32, device="cuda")
    eps = 1e-5
    Yd = ng.add_norm(up(X), up(x.R), kind, up(x.gamma), up(x.beta), eps=eps, s_out=Sd,
                     rstd_out=rstd)
    torch.cuda.synchronize()
    S = oracle.bf16_to_f64(X) + oracle.bf16_to_f64(x.R)
    Y, _, rref = oracle.norm(S, kind, eps, x.gamma, x.beta)
    _check("add_norm %s" % kind, down(Yd), Y)
    _check("add_norm s_out", down(Sd), S)
    _check_stat("add_norm rstd", rstd, rref)


# ------------------------------------------ pre-LayerNorm through the product
def _prenorm_case(x, layout, eps, affine=True):
    """Fold on the GPU, then the two-stage product; returns (C, mean, rstd,
    B_folded, colsum, bias) as device tensors."""
    K = x.A.shape[1]
    g = up(x.gamma) if affine and x.gamma is not None else None
    b = up(x.beta) if affine and x.beta is not None else None
    Bf, colsum, bias = ng.layernorm_gemm_fold(up(b_for_layout(x.B, layout)), g, b,
                                              b_layout=layout)
    mean = torch.empty(x.A.shape[0], dtype=torch.float32, device="cuda")
    rstd = torch.empty(x.A.shape[0], dtype=torch.float32, device="cuda")
    C = ng.layernorm_gemm_prenorm(up(x.A), Bf, colsum, bias, eps=eps, b_layout=layout,
                                  mean_out=mean, rstd_out=rstd)
    assert K == x.A.shape[1]
    return C, mean, rstd, Bf, colsum, bias


def _check_fold(x, layout, Bf, colsum, bias, affine=True):
    g = x.gamma if affine else None
    bt = x.beta if affine else None
    Bf_ref, _, bias_ref = oracle.layernorm_gemm_fold(x.B, g, bt)
    # B_folded: gamma * B rounded to bf16 (nearest even), bit for bit
    Bf_bits = oracle.f64_to_bf16_bits(Bf_ref)
    assert np.array_equal(down(Bf), b_for_layout(Bf_bits, layout))
    # colsum over the rounded folded weights; fp32 sums of exact products
    Bfr = oracle.bf16_to_f64(Bf_bits)
    bound = Bfr.shape[0] * 6e-8 * np.abs(Bfr).sum(axis=0) + 1e-30
    got = colsum.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - Bfr.sum(axis=0)) <= bound)
    got = bias.cpu().numpy().astype(np.float64)
    if bt is None:
        assert np.all(got == 0.0)
    else:
        bb = np.abs(oracle.bf16_to_f64(bt)) @ np.abs(oracle.bf16_to_f64(x.B))
        assert np.all(np.abs(got - bias_ref) <= x.B.shape[0] * 6e-8 * bb + 1e-30)


def _check_prenorm_stats(mean, rstd, mref, rref):
    got_mean = mean.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(got_mean - mref) / (1.0 + np.abs(mref))) <= 1e-3
    _check_stat("prenorm rstd", rstd, rref)


@pytest.mark.parametrize("layout", ["kn", "nk"])
@pytest.mark.parametrize("M,N,K", [(256, 64, 128), (300, 136, 200), (77, 128, 72),
                                   (513, 520, 264), (130, 256, 64), (1, 8, 8)])
def test_prenorm_layernorm_small(M, N, K, layout):
    log("prenorm layernorm M=%d N=%d K=%d %s" % (M, N, K, layout))
    x = workloads.make_inputs(M, N, K, seed=7 * M + N + K, row_scale=True, row_shift=True,
                              gamma=True, beta=True, gamma_len=K)
    C, mean, rstd, Bf, colsum, bias = _prenorm_case(x, layout, 1e-5)
    torch.cuda.synchronize()
    _check_fold(x, layout, Bf, colsum, bias)
    ref, mref, rref = oracle.layernorm_gemm_prenorm(x.A, x.B, 1e-5, x.gamma, x.beta)
    _check("prenorm layernorm", down(C), ref)
    _check_prenorm_stats(mean, rstd, mref, rref)


def test_prenorm_layernorm_without_affine_and_large_mean():
    # no gamma/beta: B_folded = B, colsum = column sums of B, bias = 0; rows
    # whose mean is 30 standard deviations from zero exercise the mean term
    M, N, K = 300, 520, 136
    x = workloads.make_inputs(M, N, K, seed=77, gamma=True, beta=True, gamma_len=K)
    a = oracle.bf16_to_f64(x.A) + 30.0
    x.A = oracle.f64_to_bf16_bits(a)
    C, mean, rstd, Bf, colsum, bias = _prenorm_case(x, "kn", 1e-5, affine=False)
    torch.cuda.synchronize()
    _check_fold(x, "kn", Bf, colsum, bias, affine=False)
    ref, mref, rref = oracle.layernorm_gemm_prenorm(x.A, x.B, 1e-5)
    _check("prenorm no affine, mean 30", down(C), ref)
    _check_prenorm_stats(mean, rstd, mref, rref)


def test_prenorm_layernorm_persistent_multi_tile_ragged():
    M, N, K = 256 * 9 + 37, 256 * 5 + 72, 200
    x = workloads.make_inputs(M, N, K, seed=12, row_scale=True, row_shift=True, gamma=True,
                              beta=True, gamma_len=K)
    C, mean, rstd, _, _, _ = _prenorm_case(x, "nk", 1e-5)
    torch.cuda.synchronize()
    ref, mref, rref = oracle.layernorm_gemm_prenorm(x.A, x.B, 1e-5, x.gamma, x.beta)
    _check("prenorm persistent", down(C), ref)
    _check_prenorm_stats(mean, rstd, mref, rref)


# ------------------------------------------------- Lazy Pre-Norm backward
def _lazy_bwd(x, layout, eps, workspace=None):
    """Forward (saves rstd), then the fused input gradient; returns (dA, rstd)."""
    M = x.A.shape[0]
    A, B = up(x.A), up(b_for_layout(x.B, layout))
    rstd = torch.empty(M, dtype=torch.float32, device="cuda")
    ng.rmsnorm_gemm_lazy(A, B, eps=eps, b_layout=layout, rstd_out=rstd)
    dA = ng.rmsnorm_gemm_lazy_backward_input(up(x.dC), B, A, rstd, b_layout=layout,
                                             workspace=workspace)
    return dA, rstd


# forward (M, N, K): rows of A of length K <= 128, <= 256 and wider (cross-workgroup)
@pytest.mark.parametrize("layout", ["kn", "nk"])
@pytest.mark.parametrize("M,N,K", [(256, 64, 128), (300, 136, 200), (77, 72, 128), (513, 264, 520),
                                   (130, 64, 256), (1, 8, 8), (260, 96, 1000)])
def test_lazy_backward_input_small(M, N, K, layout):
    log("lazy backward M=%d N=%d K=%d %s" % (M, N, K, layout))
    x = workloads.make_inputs(M, N, K, seed=11 * M + N + K, row_scale=True, upstream=True)
    dA, rstd = _lazy_bwd(x, layout, 1e-6)
    torch.cuda.synchronize()
    ref, _, rref = oracle.rmsnorm_gemm_lazy_backward(x.A, x.B, x.dC, 1e-6)
    _check("lazy backward dA", down(dA), ref)
    _check_stat("lazy backward rstd (forward)", rstd, rref)


def test_lazy_backward_input_cross_workgroup_deep_product():
    # the product dC @ B^T runs over N = 520 (17 k-tiles): with B stored [N, K]
    # the forward input streams into the stages under the last k-tiles
    M, N, K = 256 * 30 + 100, 520, 256 * 9 + 24
    for layout in ("nk", "kn"):
        log("lazy backward xwg deep product M=%d N=%d K=%d %s" % (M, N, K, layout))
        x = workloads.make_inputs(M, N, K, seed=37, row_scale=True, upstream=True)
        dA, _ = _lazy_bwd(x, layout, 1e-6)
        torch.cuda.synchronize()
        ref = oracle.rmsnorm_gemm_lazy_backward(x.A, x.B, x.dC, 1e-6)[0]
        _check("lazy backward xwg deep product", down(dA), ref)


def test_lazy_backward_input_cross_workgroup_rounds_ragged():
    # 10 column tiles of dA -> 25 row blocks per round; 31 row blocks -> 2 rounds
    M, N, K = 256 * 30 + 100, 136, 256 * 9 + 24
    for layout in ("kn", "nk"):
        log("lazy backward xwg rounds M=%d N=%d K=%d %s" % (M, N, K, layout))
        x = workloads.make_inputs(M, N, K, seed=31, row_scale=True, upstream=True)
        dA, _ = _lazy_bwd(x, layout, 1e-6)
        torch.cuda.synchronize()
        ref = oracle.rmsnorm_gemm_lazy_backward(x.A, x.B, x.dC, 1e-6)[0]
        _check("lazy backward xwg rounds", down(dA), ref)


def _check_scaled(name, got_bits, dC_bits, rstd_ref):
    # rstd * dC rounded once to bf16: within one bf16 rounding (2^-8
    # relative, nearest even) of the fp64 product, plus the fp32 rstd's error
    ref = rstd_ref[:, None] * oracle.bf16_to_f64(dC_bits)
    got = oracle.bf16_to_f64(got_bits)
    err = np.abs(got - ref) - (2.0 ** -8 + 1e-5) * np.abs(ref)
    log("%s: worst excess over one rounding %.3e" % (name, err.max()))
    assert np.all(err <= 0), (name, err.max())


# the regrouped backward: forward (M, N, K) over the input gradient's three
# strategies (rows of length K <= 128, <= 256, wider: one and several rounds)
@pytest.mark.parametrize("layout", ["kn", "nk"])
@pytest.mark.parametrize("M,N,K", [(300, 136, 128), (77, 72, 200), (513, 264, 520), (1, 8, 8),
                                   (260, 96, 1000), (256 * 30 + 100, 136, 256 * 9 + 24)])
def test_lazy_backward_regrouped(M, N, K, layout):
    log("lazy backward regrouped M=%d N=%d K=%d %s" % (M, N, K, layout))
    x = workloads.make_inputs(M, N, K, seed=7 * M + N + K, row_scale=True, upstream=True)
    A, B = up(x.A), up(b_for_layout(x.B, layout))
    rstd = torch.empty(M, dtype=torch.float32, device="cuda")
    ng.rmsnorm_gemm_lazy(A, B, eps=1e-6, b_layout=layout, rstd_out=rstd)
    scratch = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    dA, dB = ng.rmsnorm_gemm_lazy_backward(up(x.dC), B, A, rstd, b_layout=layout,
                                           scratch=scratch)
    torch.cuda.synchronize()
    dA_ref, _, rref = oracle.rmsnorm_gemm_lazy_backward(x.A, x.B, x.dC, 1e-6)
    _check("regrouped dA", down(dA), dA_ref)
    _check_scaled("regrouped rstd * dC", down(scratch), x.dC, rref)
    ref = oracle.lazy_backward_weight(x.A, x.dC, 1e-6)
    got = down(dB) if layout == "kn" else np.ascontiguousarray(down(dB).T)
    _check_wgrad("regrouped dB %s" % layout, got, ref, x.A, x.dC, 1e-6)


def test_lazy_backward_regrouped_empty_rows():
    dC = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    A = torch.zeros((0, 128), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((128, 64), dtype=torch.bfloat16, device="cuda")
    rstd = torch.zeros(0, dtype=torch.float32, device="cuda")
    dB = torch.full((128, 64), 3.0, dtype=torch.bfloat16, device="cuda")
    dA, dB = ng.rmsnorm_gemm_lazy_backward(dC, B, A, rstd, out_dB=dB,
                                           scratch=torch.empty(0, dtype=torch.bfloat16,
                                                               device="cuda"))
    torch.cuda.synchronize()
    assert tuple(dA.shape) == (0, 128)
    assert int(torch.count_nonzero(dB)) == 0


def test_calls_on_a_side_stream_match_the_current_stream():
    # every output and temporary the helpers allocate themselves (the
    # regrouped backward's scratch, the pre-norm statistics, the per-stream
    # workspace of the wide-row epilogue) for calls launched on another
    # stream than the current one; the kernels are deterministic, so the
    # results equal the same calls on the current stream bit for bit
    M, N, K = 700, 1040, 264
    x = workloads.make_inputs(M, N, K, seed=83, row_scale=True, row_shift=True, gamma=True,
                              beta=True, gamma_len=K, upstream=True)
    A, B, dC = up(x.A), up(x.B), up(x.dC)
    g, b = up(x.gamma), up(x.beta)
    xn = workloads.make_inputs(M, N, K, seed=84, gamma=True, beta=True)
    An, Bn, gn, bn = up(xn.A), up(xn.B), up(xn.gamma), up(xn.beta)

    def run(stream):
        rstd = torch.empty(M, dtype=torch.float32, device="cuda")
        out = [ng.rmsnorm_gemm_lazy(A, B, eps=1e-6, rstd_out=rstd, stream=stream)]
        out += list(ng.rmsnorm_gemm_lazy_backward(dC, B, A, rstd, stream=stream))
        Bf, colsum, bias = ng.layernorm_gemm_fold(B, g, b, stream=stream)
        out.append(ng.layernorm_gemm_prenorm(A, Bf, colsum, bias, eps=1e-5, stream=stream))
        out.append(ng.gemm_layernorm(An, Bn, gn, bn, eps=1e-5, stream=stream))
        return out

    ref = run(None)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    got = run(side)
    side.synchronize()
    torch.cuda.synchronize()
    names = ["lazy", "regrouped dA", "regrouped dB", "prenorm", "wide-row layernorm"]
    for name, r, o in zip(names, ref, got):
        assert torch.equal(r.view(torch.int16), o.view(torch.int16)), name
    c_ref, _, _ = oracle.gemm_layernorm(xn.A, xn.B, 1e-5, xn.gamma, xn.beta)
    _check("wide-row layernorm on a side stream", down(got[4]), c_ref)


# forward (M, N, K): M (the reduction here) ragged and short; N, K over tiles
@pytest.mark.parametrize("layout", ["kn", "nk"])
@pytest.mark.parametrize("M,N,K", [(300, 136, 200), (77, 264, 520), (1000, 64, 128), (1, 8, 8),
                                   (513, 520, 264)])
def test_lazy_backward_weight_small(M, N, K, layout):
    log("lazy backward weight M=%d N=%d K=%d %s" % (M, N, K, layout))
    x = workloads.make_inputs(M, N, K, seed=13 * M + N + K, row_scale=True, upstream=True)
    A = up(x.A)
    rstd = torch.empty(M, dtype=torch.float32, device="cuda")
    ng.rmsnorm_gemm_lazy(A, up(b_for_layout(x.B, layout)), eps=1e-6, b_layout=layout,
                         rstd_out=rstd)
    dB = ng.rmsnorm_gemm_lazy_backward_weight(A, up(x.dC), rstd, b_layout=layout)
    torch.cuda.synchronize()
    ref = oracle.lazy_backward_weight(x.A, x.dC, 1e-6)
    got = down(dB) if layout == "kn" else np.ascontiguousarray(down(dB).T)
    _check_wgrad("lazy backward dB %s" % layout, got, ref, x.A, x.dC, 1e-6)


# the scaled operand's pipeline (32-deep k-tiles, 4 stages, scaling one
# k-tile ahead) with 2, 4, 5, 6 and 7 k-tiles over the forward rows: the
# prologue and tail paths around the steady loop
@pytest.mark.parametrize("layout", ["kn", "nk"])
@pytest.mark.parametrize("M", [40, 128, 150, 170, 200])
def test_lazy_backward_weight_short_reductions(M, layout):
    N, K = 264, 136
    log("lazy backward weight short M=%d %s" % (M, layout))
    x = workloads.make_inputs(M, N, K, seed=5 * M + 3, row_scale=True, upstream=True)
    A = up(x.A)
    rstd = torch.empty(M, dtype=torch.float32, device="cuda")
    ng.rmsnorm_gemm_lazy(A, up(b_for_layout(x.B, layout)), eps=1e-6, b_layout=layout,
                         rstd_out=rstd)
    dB = ng.rmsnorm_gemm_lazy_backward_weight(A, up(x.dC), rstd, b_layout=layout)
    torch.cuda.synchronize()
    ref = oracle.lazy_backward_weight(x.A, x.dC, 1e-6)
    got = down(dB) if layout == "kn" else np.ascontiguousarray(down(dB).T)
    _check_wgrad("lazy backward dB short %s" % layout, got, ref, x.A, x.dC, 1e-6)


def test_weight_gradient_products_many_tiles():
    # 17 x 17 = 289 output tiles on a 256-workgroup grid: some workgroups take
    # a second tile, whose first k-tiles are issued before the first tile's
    # output is stored (the scaled pipeline's waits count those stores)
    M, N, K = 100, 4352, 4352
    x = workloads.make_inputs(M, N, K, seed=41, row_scale=True, upstream=True)
    A, G = up(x.A), up(x.dC)
    rstd = torch.empty(M, dtype=torch.float32, device="cuda")
    ng.rmsnorm_gemm_lazy(A, up(x.B), eps=1e-6, rstd_out=rstd)
    ref = oracle.lazy_backward_weight(x.A, x.dC, 1e-6)
    for layout in ("kn", "nk"):
        log("weight gradient many tiles %s" % layout)
        dB = ng.rmsnorm_gemm_lazy_backward_weight(A, G, rstd, b_layout=layout)
        torch.cuda.synchronize()
        got = down(dB) if layout == "kn" else np.ascontiguousarray(down(dB).T)
        _check_wgrad("weight gradient many tiles %s" % layout, got, ref, x.A, x.dC, 1e-6)
    # the plain transposed product on the same tiles: A^T @ dC
    C = ng.gemm_at(A, G)
    torch.cuda.synchronize()
    _check("gemm_at many tiles", down(C),
           oracle.gemm(np.ascontiguousarray(x.A.T), x.dC))


def test_lazy_backward_weight_empty_rows_give_zero():
    dC = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    A = torch.zeros((0, 128), dtype=torch.bfloat16, device="cuda")
    rstd = torch.zeros(0, dtype=torch.float32, device="cuda")
    dB = torch.full((128, 64), 3.0, dtype=torch.bfloat16, device="cuda")
    ng.rmsnorm_gemm_lazy_backward_weight(A, dC, rstd, out=dB)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(dB)) == 0


@pytest.mark.parametrize("M,N,K", [(256, 64, 128), (264, 520, 77), (8, 8, 1), (1000, 136, 300)])
def test_gemm_at_small(M, N, K):
    # C = A^T @ B with A stored [K, M], B stored [K, N]
    rng = np.random.default_rng(M + N + K)
    At = workloads.f32_to_bf16_bits(rng.standard_normal((K, M), dtype=np.float32))
    Bk = workloads.f32_to_bf16_bits(rng.standard_normal((K, N), dtype=np.float32)
                                    / np.float32(np.sqrt(K)))
    C = ng.gemm_at(up(At), up(Bk))
    torch.cuda.synchronize()
    _check("gemm_at %dx%dx%d" % (M, N, K), down(C), oracle.gemm(np.ascontiguousarray(At.T), Bk))


@pytest.mark.parametrize("rows,cols", [(1, 8), (37, 128), (300, 136), (65, 1000), (9, 8200)])
def test_rmsnorm_backward_small(rows, cols):
    # the standalone norm backward is the oracle's input gradient with B = I
    x = workloads.make_inputs(rows, cols, cols, seed=rows + 5 * cols, row_scale=True,
                              upstream=True)
    eye = np.eye(cols)
    ref, _, rref = oracle.rmsnorm_gemm_lazy_backward(x.A, eye, x.dC, 1e-6)
    rstd = torch.as_tensor(rref.astype(np.float32), device="cuda")
    dX = ng.rmsnorm_backward(up(x.dC), up(x.A), rstd)
    torch.cuda.synchronize()
    _check("rmsnorm backward %dx%d" % (rows, cols), down(dX), ref)


# ------------------------------------------ strategy consistency on one shape
def _ulp_distance(a_bits, b_bits):
    """Distance in bf16 units in the last place (sign-magnitude bit patterns
    mapped onto one ordered integer line)."""
    def ordered(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, -(x & 0x7FFF), x & 0x7FFF)
    return np.abs(ordered(a_bits) - ordered(b_bits))


@pytest.mark.parametrize("N", [128, 256])
@pytest.mark.parametrize("form", ["layer", "rms", "residual_rms", "lazy_backward"])
def test_row_local_and_cross_workgroup_paths_agree(N, form):
    # The same shape through the workgroup-local reduction and, with the
    # row-local maximum set to 0, through the cross-workgroup exchange: both
    # meet the oracle bar and differ by at most 2 bf16 ulp.
    M, K = 700, 200
    if form == "lazy_backward":
        # the backward normalizes rows of length K (here N plays that role)
        x = workloads.make_inputs(M, 136, N, seed=N + 71, row_scale=True, upstream=True)
        A, B = up(x.A), up(x.B)
        rstd = torch.empty(M, dtype=torch.float32, device="cuda")
        ng.rmsnorm_gemm_lazy(A, B, eps=1e-6, rstd_out=rstd)
        run = lambda: ng.rmsnorm_gemm_lazy_backward_input(up(x.dC), B, A, rstd)
        ref = oracle.rmsnorm_gemm_lazy_backward(x.A, x.B, x.dC, 1e-6)[0]
    else:
        x = workloads.make_inputs(M, N, K, seed=N + 72, gamma=True, beta=True, residual=True)
        A, B, g, b, R = up(x.A), up(x.B), up(x.gamma), up(x.beta), up(x.R)
        if form == "layer":
            run = lambda: ng.gemm_layernorm(A, B, g, b, eps=1e-5)
            ref = oracle.gemm_layernorm(x.A, x.B, 1e-5, x.gamma, x.beta)[0]
        elif form == "rms":
            run = lambda: ng.gemm_rmsnorm(A, B, g, eps=1e-6)
            ref = oracle.gemm_rmsnorm(x.A, x.B, 1e-6, x.gamma)[0]
        else:
            run = lambda: ng.gemm_add_rmsnorm(A, B, R, g, eps=1e-6)
            ref = oracle.gemm_add_rmsnorm(x.A, x.B, x.R, 1e-6, x.gamma)[0]
    local = run()
    torch.cuda.synchronize()
    with ng.debug_option(ng.NG_DEBUG_ROW_LOCAL_MAX, 0):
        cross = run()
        torch.cuda.synchronize()
    _check("%s N=%d row-local" % (form, N), down(local), ref)
    _check("%s N=%d cross-workgroup" % (form, N), down(cross), ref)
    d = _ulp_distance(down(local), down(cross))
    log("%s N=%d: max ulp distance between the paths %d" % (form, N, d.max()))
    assert d.max() <= 2


# ------------------------------------------------ tile order (stress case)
# The grids take their output tiles in a reversed or shuffled order (a
# diagnostic option): which workgroup reaches which tile first changes, in
# particular which workgroups of a row block publish, merge and wait first on
# the cross-workgroup path.  Every output must match the oracle and be
# bit-identical to the natural order's (per-tile arithmetic and the merge
# order of the partials do not depend on the tile order).

def _order_cases():
    # (label, run(x) -> device tensors, oracle(x) -> reference of the first)
    return {
        # cross-workgroup LayerNorm: 16 column tiles -> 16 row blocks per
        # round, 40 row blocks -> 3 rounds, ragged M and N
        "xwg_layernorm": ((10000, 4000, 264), dict(gamma=True, beta=True),
                          lambda x, A, B: [ng.gemm_layernorm(A, B, up(x.gamma), up(x.beta),
                                                             eps=1e-5)],
                          lambda x: oracle.gemm_layernorm(x.A, x.B, 1e-5, x.gamma, x.beta)[0]),
        "xwg_residual_rmsnorm": ((8000, 2056, 136), dict(gamma=True, residual=True),
                                 lambda x, A, B: [ng.gemm_add_rmsnorm(A, B, up(x.R), up(x.gamma),
                                                                      eps=1e-6)],
                                 lambda x: oracle.gemm_add_rmsnorm(x.A, x.B, x.R, 1e-6,
                                                                   x.gamma)[0]),
        # the same with R streamed in under the last of 17 k-tiles
        "xwg_residual_layernorm_deep_k": ((6000, 2056, 520),
                                          dict(gamma=True, beta=True, residual=True),
                                          lambda x, A, B: [ng.gemm_add_layernorm(
                                              A, B, up(x.R), up(x.gamma), up(x.beta),
                                              eps=1e-5)],
                                          lambda x: oracle.gemm_add_layernorm(
                                              x.A, x.B, x.R, 1e-5, x.gamma, x.beta)[0]),
        # persistent 256x256 grid with more tiles than slots (two rounds)
        "persistent_lazy": ((5000, 4000, 264), dict(row_scale=True),
                            lambda x, A, B: [ng.rmsnorm_gemm_lazy(A, B, eps=1e-6)],
                            lambda x: oracle.rmsnorm_gemm_lazy(x.A, x.B, 1e-6)[0]),
        "persistent_gemm": ((5000, 4000, 264), dict(),
                            lambda x, A, B: [ng.gemm(A, B)],
                            lambda x: oracle.gemm(x.A, x.B)),
        # one workgroup per tile (row-local norm)
        "rowlocal_layernorm": ((5000, 200, 264), dict(gamma=True, beta=True),
                               lambda x, A, B: [ng.gemm_layernorm(A, B, up(x.gamma), up(x.beta),
                                                                  eps=1e-5)],
                               lambda x: oracle.gemm_layernorm(x.A, x.B, 1e-5, x.gamma,
                                                               x.beta)[0]),
    }


@pytest.mark.parametrize("order", ["reversed", "shuffled"])
@pytest.mark.parametrize("case", sorted(_order_cases()))
def test_tile_order_does_not_change_results(case, order):
    (M, N, K), kw, run, ref_fn = _order_cases()[case]
    mode = {"reversed": ng.NG_TILE_ORDER_REVERSED, "shuffled": ng.NG_TILE_ORDER_SHUFFLED}[order]
    log("tile order %s: %s M=%d N=%d K=%d" % (order, case, M, N, K))
    x = workloads.make_inputs(M, N, K, seed=M + N + K + 7, **kw)
    A, B = up(x.A), up(x.B)
    natural = run(x, A, B)
    torch.cuda.synchronize()
    with ng.debug_option(ng.NG_DEBUG_TILE_ORDER, mode):
        permuted = run(x, A, B)
        torch.cuda.synchronize()
    _check("%s %s order" % (case, order), down(permuted[0]), ref_fn(x))
    for a, b in zip(natural, permuted):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), case


@pytest.mark.parametrize("kind,layout,K", [("layer", "kn", 200), ("rms", "nk", 200),
                                           ("layer", "nk", 72), ("rms", "kn", 520)])
def test_alternating_k_walk(kind, layout, K):
    # 10 column tiles -> 25 row blocks per round; 61 row blocks -> 3 rounds,
    # the middle one walking K downwards (ragged last k-tile first), with the
    # next round's first k-tiles prefetched in both directions (K = 72 on the
    # 64-deep tiles: fewer k-tiles than the prefetch needs)
    M, N = 256 * 60 + 100, 256 * 9 + 24
    log("alternating k-walk %s M=%d N=%d K=%d %s" % (kind, M, N, K, layout))
    x = workloads.make_inputs(M, N, K, seed=K + 5, gamma=True, beta=kind == "layer")
    A, B = up(x.A), up(b_for_layout(x.B, layout))
    rstd = torch.empty(M, dtype=torch.float32, device="cuda")

    def run():
        if kind == "layer":
            return ng.gemm_layernorm(A, B, up(x.gamma), up(x.beta), eps=1e-5, b_layout=layout,
                                     rstd_out=rstd)
        return ng.gemm_rmsnorm(A, B, up(x.gamma), eps=1e-6, b_layout=layout, rstd_out=rstd)

    with ng.debug_option(ng.NG_DEBUG_K_WALK, ng.NG_K_WALK_ALTERNATE):
        C1 = run()
        C2 = run()
        # the plain product's persistent grid: 610 tiles, 3 passes of 256
        P = ng.gemm(A, B, b_layout=layout)
        # each tile keeps its walk when the grids take the tiles in another
        # order: the same sums, bit for bit
        with ng.debug_option(ng.NG_DEBUG_TILE_ORDER, ng.NG_TILE_ORDER_SHUFFLED):
            C3 = run()
            P3 = ng.gemm(A, B, b_layout=layout)
        torch.cuda.synchronize()
    assert torch.equal(C1.view(torch.int16), C3.view(torch.int16))
    assert torch.equal(P.view(torch.int16), P3.view(torch.int16))
    if kind == "layer":
        ref, _, rref = oracle.gemm_layernorm(x.A, x.B, 1e-5, x.gamma, x.beta)
    else:
        ref, rref = oracle.gemm_rmsnorm(x.A, x.B, 1e-6, x.gamma)
    _check("alternating k-walk %s %s K=%d" % (kind, layout, K), down(C1), ref)
    _check_stat("alternating k-walk rstd", rstd, rref)
    assert torch.equal(C1.view(torch.int16), C2.view(torch.int16))
    _check("alternating k-walk gemm %s K=%d" % (layout, K), down(P), oracle.gemm(x.A, x.B))


# ------------------------------------------------------------ edge cases
def test_longest_rows_of_length_k():
    # K = 2^22, the longest row the products read: a full 256-row tile spans
    # 255 * 2K + 64 bytes from its first row, just inside the 2 GiB buffer
    # range; a second, 4-row tile and two column tiles (the last ragged)
    M, N, K = 260, 264, 1 << 22
    log("longest rows M=%d N=%d K=%d" % (M, N, K))
    x = workloads.make_inputs(M, N, K, seed=3)
    ref = oracle.gemm(x.A, x.B)
    ref_lazy, rref = oracle.rmsnorm_gemm_lazy(x.A, x.B, 1e-6)
    A = up(x.A)
    for layout in ("kn", "nk"):
        B = up(b_for_layout(x.B, layout))
        C = ng.gemm(A, B, b_layout=layout)
        rstd = torch.empty(M, dtype=torch.float32, device="cuda")
        L = ng.rmsnorm_gemm_lazy(A, B, eps=1e-6, b_layout=layout, rstd_out=rstd)
        torch.cuda.synchronize()
        _check("gemm K=2^22 %s" % layout, down(C), ref)
        _check("lazy K=2^22 %s" % layout, down(L), ref_lazy)
        _check_stat("lazy K=2^22 rstd %s" % layout, rstd, rref)
        del B, C, L
    del A
    torch.cuda.empty_cache()


def test_empty_M_is_a_no_op():
    # M == 0: the calls return NG_OK without touching any buffer (A and C may
    # be NULL), and the helpers return empty outputs
    A = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    B = torch.ones((64, 512), dtype=torch.bfloat16, device="cuda")
    C = ng.gemm_layernorm(A, B, eps=1e-5)
    C2 = ng.rmsnorm_gemm_lazy(A, B)
    torch.cuda.synchronize()
    assert C.shape == (0, 512) and C2.shape == (0, 512)
    st = torch.cuda.current_stream().cuda_stream
    Bp = B.data_ptr()
    assert ng.ng_gemm(None, Bp, None, 0, 512, 64, 0, st) == 0
    assert ng.ng_rmsnorm_gemm_lazy(None, Bp, None, 0, 512, 64, 0, 1e-6, None, st) == 0
    assert ng.ng_gemm_layernorm(None, Bp, None, None, None, 0, 512, 64, 0, 1e-5, None, None,
                                None, 0, st) == 0
    assert ng.ng_norm(None, None, None, None, 0, 512, 0, 1e-6, None, None, st) == 0
    torch.cuda.synchronize()
    assert torch.equal(B, torch.ones_like(B))


def test_lazy_zero_rows_and_eps_zero():
    # zero row: rstd = 1/sqrt(eps), output row 0; eps = 0 on a nonzero row
    x = workloads.make_inputs(64, 64, 64, seed=1)
    A = x.A.copy()
    A[5] = 0
    rstd = torch.empty(64, dtype=torch.float32, device="cuda")
    C = ng.rmsnorm_gemm_lazy(up(A), up(x.B), eps=1e-6, rstd_out=rstd)
    torch.cuda.synchronize()
    ref, rref = oracle.rmsnorm_gemm_lazy(A, x.B, 1e-6)
    _check("lazy zero row", down(C), ref)
    assert abs(float(rstd[5]) - 1e3) <= 1e-3 * 1e3
    A[5] = x.A[5]
    C = ng.rmsnorm_gemm_lazy(up(A), up(x.B), eps=0.0)
    torch.cuda.synchronize()
    ref, _ = oracle.rmsnorm_gemm_lazy(A, x.B, 0.0)
    _check("lazy eps=0", down(C), ref)


@pytest.mark.parametrize("N", [128, 1024])
def test_layernorm_constant_rows_give_beta(N):
    # A with a single nonzero column and B with a constant row -> every output
    # row is constant, so LayerNorm returns beta exactly (degenerate case).
    M, K = 96, 64
    A = np.zeros((M, K), dtype=np.float32)
    A[:, 0] = np.linspace(-3, 3, M)
    B = np.zeros((K, N), dtype=np.float32)
    B[0, :] = 1.0
    x = workloads.make_inputs(1, N, 8, seed=2, gamma=True, beta=True)
    Ab, Bb = workloads.f32_to_bf16_bits(A), workloads.f32_to_bf16_bits(B)
    C = ng.gemm_layernorm(up(Ab), up(Bb), up(x.gamma), up(x.beta), eps=1e-5)
    torch.cuda.synchronize()
    ref, _, _ = oracle.gemm_layernorm(Ab, Bb, 1e-5, x.gamma, x.beta)
    _check("constant rows", down(C), ref)
    dev = np.abs(oracle.bf16_to_f64(down(C)) - oracle.bf16_to_f64(x.beta)[None, :])
    assert dev.max() <= 1e-2


def test_cross_workgroup_path_is_deterministic_and_leaves_workspace_ready():
    M, N, K = 1000, 4096, 256
    x = workloads.make_inputs(M, N, K, seed=99, gamma=True, beta=True)
    ws = ng.Workspace(ng.ng_workspace_bytes(ng.NG_OP_GEMM_LAYERNORM, M, N, K))
    args = (up(x.A), up(x.B), up(x.gamma), up(x.beta))
    C1 = ng.gemm_layernorm(*args, eps=1e-5, workspace=ws)
    C2 = ng.gemm_layernorm(*args, eps=1e-5, workspace=ws)
    # a different shape through the same workspace
    y = workloads.make_inputs(300, 2048, 64, seed=98, gamma=True)
    C3 = ng.gemm_rmsnorm(up(y.A), up(y.B), up(y.gamma), eps=1e-6, workspace=ws)
    assert ws.status() == 0
    torch.cuda.synchronize()
    assert torch.equal(C1.view(torch.int16), C2.view(torch.int16))
    # header: error word 0, call counter advanced once per call, no workgroup
    # of a running call left over
    header = ws.buf[0:12].view(torch.int32).cpu().numpy()
    assert header[0] == 0 and header[1] == 3 and header[2] == 0
    ref, _ = oracle.gemm_rmsnorm(y.A, y.B, 1e-6, y.gamma)
    _check("xwg second shape", down(C3), ref)


# --------------------------------------------- full-size named workloads
# Every element of every output, and every statistic output, of each named
# workload at full size is compared with the oracle.  The oracle runs in
# chunks of rows (rows are independent in every op), with B decoded once.
CHUNK_ROWS = 2048


def _full_compare(name, C, M, ref_rows, stats=None, allowance=None):
    """C: device output [M, ...]; ref_rows(r0, r1) -> (Y rows, {stat: rows});
    stats: {stat: device float32 [M]} to compare (1e-3 relative; the mean
    relative to 1 + |mean|); allowance(r0, r1) -> an absolute error per
    element added to the bar (only for an unfused baseline that stores an
    intermediate in bf16)."""
    got_all = down(C)
    got_stats = {k: v.cpu().numpy().astype(np.float64) for k, v in (stats or {}).items()}
    worst, worst_stat = 0.0, 0.0
    for r0 in range(0, M, CHUNK_ROWS):
        r1 = min(M, r0 + CHUNK_ROWS)
        ref, ref_stats = ref_rows(r0, r1)
        got = oracle.bf16_to_f64(got_all[r0:r1])
        assert np.all(np.isfinite(got)), (name, r0)
        err = np.abs(got - ref)
        if allowance is not None:
            err = np.maximum(err - allowance(r0, r1), 0.0)
        worst = max(worst, float(np.max(err / (1.0 + np.abs(ref)))))
        for k, g in got_stats.items():
            r = ref_stats[k]
            den = (1.0 + np.abs(r)) if k == "mean" else np.abs(r)
            worst_stat = max(worst_stat, float(np.max(np.abs(g[r0:r1] - r) / den)))
    log("%s: every element, max rel err %.3e; statistics %s max rel err %.3e" % (
        name, worst, sorted(got_stats), worst_stat))
    assert worst <= TOL, (name, worst)
    assert worst_stat <= 1e-3, (name, worst_stat)


def _f32(M):
    return torch.empty(M, dtype=torch.float32, device="cuda")


def _workload_case(w, layout="kn"):
    log("workload %s %s (full output)" % (w.name, layout))
    x = workloads.workload_inputs(w)
    B64 = oracle.bf16_to_f64(x.B)
    A, B = up(x.A), up(b_for_layout(x.B, layout))
    g = up(x.gamma) if x.gamma is not None else None
    b = up(x.beta) if x.beta is not None else None
    M = w.M
    if w.op == workloads.OP_LAZY:
        rstd = _f32(M)
        C = ng.rmsnorm_gemm_lazy(A, B, eps=w.eps, b_layout=layout, rstd_out=rstd)
        stats = {"rstd": rstd}

        def ref_rows(r0, r1):
            Y, r = oracle.rmsnorm_gemm_lazy(x.A[r0:r1], B64, w.eps)
            return Y, {"rstd": r}
    elif w.op == workloads.OP_LAZY_AFFINE:
        rstd = _f32(M)
        Bf, bias = ng.lazy_fold_affine(B, g, b, b_layout=layout)
        C = ng.rmsnorm_gemm_lazy_affine(A, Bf, bias, eps=w.eps, b_layout=layout, rstd_out=rstd)
        stats = {"rstd": rstd}

        def ref_rows(r0, r1):
            Y, r = oracle.rmsnorm_gemm_lazy_affine(x.A[r0:r1], B64, w.eps, x.gamma, x.beta)
            return Y, {"rstd": r}
    elif w.op == workloads.OP_LAZY_BWD:
        C, rstd = _lazy_bwd(x, layout, w.eps)
        stats = {"rstd": rstd}

        def ref_rows(r0, r1):
            dA, _, r = oracle.rmsnorm_gemm_lazy_backward(x.A[r0:r1], B64, x.dC[r0:r1], w.eps)
            return dA, {"rstd": r}
    elif w.op == workloads.OP_LAZY_BWD_W:
        rstd = _f32(M)
        ng.rmsnorm_gemm_lazy(A, B, eps=w.eps, b_layout=layout, rstd_out=rstd)
        C = ng.rmsnorm_gemm_lazy_backward_weight(A, up(x.dC), rstd, b_layout=layout)
        if layout == "nk":
            C = C.t().contiguous()
        torch.cuda.synchronize()
        ref = oracle.lazy_backward_weight(x.A, x.dC, w.eps)
        _check_wgrad(w.name + " (every element)", down(C), ref, x.A, x.dC, w.eps)
        return
    elif w.op == workloads.OP_LAZY_BWD_RG:
        rstd = _f32(M)
        ng.rmsnorm_gemm_lazy(A, B, eps=w.eps, b_layout=layout, rstd_out=rstd)
        scratch = torch.empty((M, w.N), dtype=torch.bfloat16, device="cuda")
        C, dB = ng.rmsnorm_gemm_lazy_backward(up(x.dC), B, A, rstd, b_layout=layout,
                                              scratch=scratch)
        if layout == "nk":
            dB = dB.t().contiguous()
        torch.cuda.synchronize()
        ref = oracle.lazy_backward_weight(x.A, x.dC, w.eps)
        _check_wgrad(w.name + " dB (every element)", down(dB), ref, x.A, x.dC, w.eps)
        del ref
        _check_scaled(w.name + " rstd * dC (every element)", down(scratch), x.dC,
                      oracle.rms_norm_rows(x.A, w.eps)[1])
        stats = {"rstd": rstd}

        def ref_rows(r0, r1):
            dA, _, r = oracle.rmsnorm_gemm_lazy_backward(x.A[r0:r1], B64, x.dC[r0:r1], w.eps)
            return dA, {"rstd": r}
    elif w.op == workloads.OP_PRENORM_LN:
        C, mean, rstd = _prenorm_case(x, layout, w.eps)[:3]
        stats = {"mean": mean, "rstd": rstd}

        def ref_rows(r0, r1):
            Y, mu, r = oracle.layernorm_gemm_prenorm(x.A[r0:r1], B64, w.eps, x.gamma, x.beta)
            return Y, {"mean": mu, "rstd": r}
    elif w.op in (workloads.OP_GEMM_ADD_RMSNORM, workloads.OP_GEMM_ADD_LAYERNORM):
        kind = "layer" if w.op == workloads.OP_GEMM_ADD_LAYERNORM else "rms"
        C, mean, rstd = _residual_call(kind, x, layout, w.eps)
        stats = {"rstd": rstd} if mean is None else {"mean": mean, "rstd": rstd}

        def ref_rows(r0, r1):
            A_r, R_r = x.A[r0:r1], x.R[r0:r1]
            if kind == "layer":
                Y, mu, r, _ = oracle.gemm_add_layernorm(A_r, B64, R_r, w.eps, x.gamma, x.beta)
                return Y, {"mean": mu, "rstd": r}
            Y, r, _ = oracle.gemm_add_rmsnorm(A_r, B64, R_r, w.eps, x.gamma)
            return Y, {"rstd": r}
    elif w.op == workloads.OP_GEMM_RMSNORM:
        rstd = _f32(M)
        C = ng.gemm_rmsnorm(A, B, g, eps=w.eps, b_layout=layout, rstd_out=rstd)
        stats = {"rstd": rstd}

        def ref_rows(r0, r1):
            Y, r = oracle.gemm_rmsnorm(x.A[r0:r1], B64, w.eps, x.gamma)
            return Y, {"rstd": r}
    else:
        mean, rstd = _f32(M), _f32(M)
        C = ng.gemm_layernorm(A, B, g, b, eps=w.eps, b_layout=layout, mean_out=mean,
                              rstd_out=rstd)
        stats = {"mean": mean, "rstd": rstd}

        def ref_rows(r0, r1):
            Y, mu, r = oracle.gemm_layernorm(x.A[r0:r1], B64, w.eps, x.gamma, x.beta)
            return Y, {"mean": mu, "rstd": r}
    torch.cuda.synchronize()
    _full_compare("%s %s" % (w.name, layout), C, M, ref_rows, stats)


@pytest.mark.parametrize("name", [w.name for w in workloads.WORKLOADS])
def test_named_workload_full_size(name):
    _workload_case(workloads.WORKLOAD_BY_NAME[name])


@pytest.mark.parametrize("name", [w.name for w in workloads.NEXT_WORKLOADS])
def test_next_workload_full_size(name):
    _workload_case(workloads.WORKLOAD_BY_NAME[name])


def test_named_workload_nk_layout_large():
    _workload_case(workloads.WORKLOAD_BY_NAME["gemm_rms_16384x4096x8192"], layout="nk")


# B stored [N, K] (a Linear weight) at full size on the other large forms: the
# 2-stage 64-deep tiles forward, and the backward's products in the other
# layout (the input gradient then reads B as [K, N] on 32-deep tiles, whose
# regrouped copy runs in the epilogue)
@pytest.mark.parametrize("name", ["lazy_rms_32768x4096x4096", "gemm_ln_8192x8192x16384",
                                  "lazy_rms_bwd_32768x4096x4096",
                                  "lazy_rms_bwd_regrouped_32768x4096x4096"])
def test_workload_nk_layout_full_size(name):
    _workload_case(workloads.WORKLOAD_BY_NAME[name], layout="nk")


# The unfused pairs the hidden-latency metric is measured against, at full
# size, every element.
def test_unfused_pairs_full_size_epilogue_forms():
    w = workloads.WORKLOAD_BY_NAME["gemm_ln_65536x512x128"]
    x = workloads.workload_inputs(w)
    B64 = oracle.bf16_to_f64(x.B)
    Y = ng.norm(ng.gemm(up(x.A), up(x.B)), "layer", eps=w.eps)
    torch.cuda.synchronize()
    _full_compare("unfused gemm->layernorm", Y, w.M,
                  lambda r0, r1: (oracle.gemm_layernorm(x.A[r0:r1], B64, w.eps)[0], {}))
    for name in ("gemm_rms_16384x4096x8192", "gemm_ln_8192x8192x16384"):
        w = workloads.WORKLOAD_BY_NAME[name]
        x = workloads.workload_inputs(w)
        B64 = oracle.bf16_to_f64(x.B)
        kind = "layer" if w.op == workloads.OP_GEMM_LAYERNORM else "rms"
        b = up(x.beta) if x.beta is not None else None
        Y = ng.norm(ng.gemm(up(x.A), up(x.B)), kind, up(x.gamma), b, eps=w.eps)
        torch.cuda.synchronize()
        if kind == "layer":
            ref = lambda r0, r1: (oracle.gemm_layernorm(x.A[r0:r1], B64, w.eps, x.gamma,
                                                        x.beta)[0], {})
        else:
            ref = lambda r0, r1: (oracle.gemm_rmsnorm(x.A[r0:r1], B64, w.eps, x.gamma)[0], {})
        _full_compare("unfused gemm->%snorm %s" % (kind, name), Y, w.M, ref)
        del Y


def test_unfused_pair_lazy_full_size():
    w = workloads.WORKLOAD_BY_NAME["lazy_rms_32768x4096x4096"]
    x = workloads.workload_inputs(w)
    B64 = oracle.bf16_to_f64(x.B)
    C = ng.gemm(ng.norm(up(x.A), "rms", eps=w.eps), up(x.B))
    torch.cuda.synchronize()
    _full_compare("unfused rmsnorm->gemm", C, w.M,
                  lambda r0, r1: (oracle.rmsnorm_gemm_lazy(x.A[r0:r1], B64, w.eps)[0], {}))


def test_residual_unfused_pair_full_size():
    # ng_gemm, then ng_add_norm.  This baseline stores X = A @ B in bf16 and
    # forms S = X + R in bf16: where X and R nearly cancel, X's rounding is
    # large next to S and the norm scales it up, so its bar adds the two
    # storage roundings (half an ulp of X and of S, <= 2^-9 relative each)
    # carried through the row scale and gamma.  (The fused form adds R to the
    # fp32 accumulators and meets the plain bar.)
    w = workloads.WORKLOAD_BY_NAME["gemm_add_rms_16384x4096x8192"]
    x = workloads.workload_inputs(w)
    B64 = oracle.bf16_to_f64(x.B)
    gamma = np.abs(oracle.bf16_to_f64(x.gamma))
    Y = ng.add_norm(ng.gemm(up(x.A), up(x.B)), up(x.R), "rms", up(x.gamma), eps=w.eps)
    torch.cuda.synchronize()

    def allowance(r0, r1):
        X = oracle.gemm(x.A[r0:r1], B64)
        _, rstd, S = oracle.gemm_add_rmsnorm(x.A[r0:r1], B64, x.R[r0:r1], w.eps)
        return 2.0 ** -9 * (np.abs(X) + np.abs(S)) * rstd[:, None] * gamma[None, :]

    _full_compare("unfused gemm->add_norm", Y, w.M,
                  lambda r0, r1: (oracle.gemm_add_rmsnorm(x.A[r0:r1], B64, x.R[r0:r1], w.eps,
                                                          x.gamma)[0], {}),
                  allowance=allowance)


def test_prenorm_unfused_pair_full_size():
    # ng_norm, then ng_gemm
    w = workloads.WORKLOAD_BY_NAME["prenorm_ln_32768x4096x4096"]
    x = workloads.workload_inputs(w)
    B64 = oracle.bf16_to_f64(x.B)
    C = ng.gemm(ng.norm(up(x.A), "layer", up(x.gamma), up(x.beta), eps=w.eps), up(x.B))
    torch.cuda.synchronize()
    _full_compare("unfused layernorm->gemm", C, w.M,
                  lambda r0, r1: (oracle.layernorm_gemm_prenorm(x.A[r0:r1], B64, w.eps, x.gamma,
                                                                x.beta)[0], {}))


def test_lazy_backward_unfused_pair_full_size():
    # ng_gemm (dC @ B^T), then ng_rmsnorm_backward
    w = workloads.WORKLOAD_BY_NAME["lazy_rms_bwd_32768x4096x4096"]
    x = workloads.workload_inputs(w)
    B64 = oracle.bf16_to_f64(x.B)
    A, B = up(x.A), up(x.B)
    rstd = _f32(w.M)
    ng.rmsnorm_gemm_lazy(A, B, eps=w.eps, rstd_out=rstd)
    dA = ng.rmsnorm_backward(ng.gemm(up(x.dC), B, b_layout="nk"), A, rstd)
    torch.cuda.synchronize()
    _full_compare("unfused gemm->rmsnorm backward", dA, w.M,
                  lambda r0, r1: (oracle.rmsnorm_gemm_lazy_backward(
                      x.A[r0:r1], B64, x.dC[r0:r1], w.eps)[0], {}))


def test_lazy_backward_weight_unfused_pair_full_size():
    # ng_norm (A_hat stored), then ng_gemm_at (A_hat^T @ dC)
    w = workloads.WORKLOAD_BY_NAME["lazy_rms_bwd_weight_32768x4096x4096"]
    x = workloads.workload_inputs(w)
    dB = ng.gemm_at(ng.norm(up(x.A), "rms", eps=w.eps), up(x.dC))
    torch.cuda.synchronize()
    ref = oracle.lazy_backward_weight(x.A, x.dC, w.eps)
    _check_wgrad("unfused rmsnorm->gemm_at (every element)", down(dB), ref, x.A, x.dC, w.eps)
