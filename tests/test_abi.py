"""C-ABI checks that need no GPU: the library loads, exports every entry point
the header declares, and rejects bad arguments before making any HIP call."""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "normgemm.h")

from normalization_gemm_amd import _lib  # noqa: E402

lib_missing = not os.path.exists(_lib.LIB_PATH)
pytestmark = pytest.mark.skipif(lib_missing, reason="libnormgemm.so not built")

# Fake but well-aligned device addresses: validation never dereferences them.
P = 0x7F0000000000
P2 = P + 0x100000
P3 = P + 0x200000
BAD = P + 2  # not 16-byte aligned


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ng_\w+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    names = header_functions()
    for n in ("ng_rmsnorm_gemm_lazy", "ng_gemm_layernorm", "ng_gemm_rmsnorm", "ng_gemm",
              "ng_norm", "ng_workspace_bytes", "ng_lazy_fold_affine",
              "ng_rmsnorm_gemm_lazy_affine", "ng_gemm_add_rmsnorm", "ng_gemm_add_layernorm",
              "ng_add_norm", "ng_layernorm_gemm_fold", "ng_layernorm_gemm_prenorm",
              "ng_rmsnorm_gemm_lazy_backward_input", "ng_rmsnorm_backward",
              "ng_rmsnorm_gemm_lazy_backward_weight", "ng_gemm_at",
              "ng_rmsnorm_gemm_lazy_backward"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for name in header_functions():
        assert hasattr(lib, name), name
    assert sorted(_lib.exported_names()) == header_functions()


def test_binding_constants_match_the_header():
    # every enumerator the header defines has the same value in the binding
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    consts = dict(re.findall(r"\b(NG_[A-Z0-9_]+)\s*=\s*(-?\d+)", text))
    assert len(consts) > 20
    for name, value in consts.items():
        assert getattr(_lib, name) == int(value), name


def test_binding_signatures_match_the_header():
    # argument counts of every prototype in the header against the ctypes
    # table (a mismatch would pass arguments in the wrong slots)
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    protos = dict(re.findall(r"\b(ng_\w+)\s*\(([^)]*)\)\s*;", text))
    assert set(protos) == set(_lib.exported_names())
    for name, args in protos.items():
        n = 0 if args.strip() in ("", "void") else len(args.split(","))
        assert len(_lib._SIGNATURES[name][1]) == n, name


def test_status_strings():
    assert _lib.ng_status_string(0) == "NG_OK"
    assert _lib.ng_status_string(1) == "NG_ERR_INVALID_ARG"
    assert _lib.ng_status_string(5) == "NG_ERR_TIMEOUT"
    assert _lib.ng_status_string(99) == "NG_ERR_UNKNOWN"


def lazy(A=P, B=P2, C=P3, M=64, N=64, K=64, lay=0, eps=1e-6, rstd=None):
    return _lib.ng_rmsnorm_gemm_lazy(A, B, C, M, N, K, lay, eps, rstd, None)


@pytest.mark.parametrize("kw,code", [
    (dict(A=None), 1), (dict(B=None), 1), (dict(C=None), 1),
    (dict(A=BAD), 1), (dict(C=BAD), 1),
    (dict(M=-1), 1), (dict(N=0), 1), (dict(K=0), 1), (dict(K=-8), 1),
    (dict(N=1 << 25), 1),
    (dict(lay=2), 1), (dict(lay=-1), 1),
    (dict(eps=-1.0), 1), (dict(eps=math.nan), 1), (dict(eps=math.inf), 1),
    (dict(N=60), 2), (dict(K=100), 2),
    (dict(rstd=P + 2), 1),
])
def test_lazy_argument_checks(kw, code):
    assert lazy(**kw) == code
    assert _lib.ng_last_error() != ""


def test_empty_M_is_a_noop():
    assert lazy(M=0) == 0
    assert lazy(M=0, A=None, C=None) == 0
    assert lazy(M=0, B=None) == 1
    assert _lib.ng_norm(None, None, None, None, 0, 64, 1, 1e-6, None, None, None) == 0
    assert _lib.ng_gemm(P, P2, P3, 0, 64, 64, 0, None) == 0
    assert _lib.ng_norm(P, None, None, P2, 0, 64, 0, 1e-6, None, None, None) == 0
    assert _lib.ng_gemm_layernorm(P, P2, None, None, P3, 0, 4096, 64, 0, 1e-5, None, None,
                                  None, 0, None) == 0


def test_gemm_norm_workspace_checks():
    need = _lib.ng_workspace_bytes(_lib.NG_OP_GEMM_LAYERNORM, 1000, 4096, 512)
    assert need > 0
    # no workspace for wide rows
    assert _lib.ng_gemm_layernorm(P, P2, None, None, P3, 1000, 4096, 512, 0, 1e-5, None, None,
                                  None, 0, None) == 3
    # too small
    assert _lib.ng_gemm_rmsnorm(P, P2, None, P3, 1000, 4096, 512, 0, 1e-6, None, P,
                                need - 8, None) == 3
    # misaligned workspace
    assert _lib.ng_gemm_rmsnorm(P, P2, None, P3, 1000, 4096, 512, 0, 1e-6, None, P + 16,
                                need, None) == 3
    # narrow rows need none
    assert _lib.ng_workspace_bytes(_lib.NG_OP_GEMM_LAYERNORM, 1000, 256, 512) == 0
    assert _lib.ng_workspace_bytes(_lib.NG_OP_RMSNORM_GEMM_LAZY, 1000, 4096, 512) == 0
    assert _lib.ng_workspace_bytes(_lib.NG_OP_GEMM, 1000, 4096, 512) == 0


def _ws_formula(M, N):
    # 256-byte header; then per slot (a row block of one round: at most
    # 1024 co-resident workgroups, and no more than the matrix has) one
    # 16-byte tagged partial per (row, column tile) and one 16-byte tagged
    # (mean, rstd) per row
    rb, tn = -(-M // 256), -(-N // 256)
    slots = max(1, min(rb, 1024 // tn))
    return 256 + slots * 256 * tn * 16 + slots * 256 * 16


def test_workspace_size_formula():
    for M, N in [(16384, 8192), (8192, 16384), (1000, 4100), (300, 2048), (1 << 24, 512),
                 (1 << 20, 65536)]:
        assert _lib.ng_workspace_bytes(_lib.NG_OP_GEMM_RMSNORM, M, N, 4096) == _ws_formula(M, N)
    # it stops growing with M once a round's row blocks are covered
    assert (_lib.ng_workspace_bytes(_lib.NG_OP_GEMM_LAYERNORM, 1 << 24, 16384, 64) ==
            _lib.ng_workspace_bytes(_lib.NG_OP_GEMM_LAYERNORM, 4096, 16384, 64))


def test_no_allocation_scratch_holds_every_shape():
    # the static scratch of ng_gemm_layernorm_noalloc (16 MiB) holds the
    # exchange of every accepted shape (rows up to 2^24, rows of up to 65536
    # columns)
    worst = max(_lib.ng_workspace_bytes(_lib.NG_OP_GEMM_LAYERNORM, 1 << 24, 8 * n, 64)
                for n in range(33, 8193))
    assert worst <= 16 << 20, worst


def test_gemm_norm_argument_checks():
    ok_ws = _lib.ng_workspace_bytes(_lib.NG_OP_GEMM_LAYERNORM, 64, 4096, 64)
    # gamma/beta misaligned
    assert _lib.ng_gemm_layernorm(P, P2, P + 8, None, P3, 64, 128, 64, 0, 1e-5, None, None,
                                  None, 0, None) == 1
    assert _lib.ng_gemm_layernorm(P, P2, None, P + 8, P3, 64, 128, 64, 0, 1e-5, None, None,
                                  None, 0, None) == 1
    assert _lib.ng_gemm_layernorm(P, P2, None, None, P3, 64, 128, 64, 0, -1.0, None, None,
                                  None, 0, None) == 1
    assert _lib.ng_gemm_layernorm(P, P2, None, None, P3, 64, 4096, 64, 5, 1e-5, None, None,
                                  P, ok_ws, None) == 1
    assert _lib.ng_gemm_rmsnorm(P, P2, None, P3, 64, 100, 64, 0, 1e-6, None, None, 0, None) == 2


def test_norm_argument_checks():
    f = _lib.ng_norm
    assert f(None, None, None, P2, 4, 64, 0, 1e-6, None, None, None) == 1
    assert f(P, None, None, BAD, 4, 64, 0, 1e-6, None, None, None) == 1
    assert f(P, None, None, P2, 4, 64, 7, 1e-6, None, None, None) == 1
    assert f(P, None, None, P2, 4, 64, 0, 1e-6, P3, None, None) == 1   # mean_out with RMS
    assert f(P, None, None, P2, 4, 64, 0, 1e-6, P3, None, None) == 1   # mean_out with RMS
    assert f(P, None, None, P2, 4, 60, 1, 1e-6, None, None, None) == 2
    assert f(P, None, None, P2, 4, 65536 + 8, 1, 1e-6, None, None, None) == 2
    assert f(P, None, None, P2, 4, 0, 1, 1e-6, None, None, None) == 1


def test_lazy_affine_argument_checks():
    fold = _lib.ng_lazy_fold_affine
    # NULL or misaligned B / B_folded, bad sizes or layout -> invalid argument
    assert fold(None, None, None, P2, None, 64, 64, 0, None) == 1
    assert fold(P, None, None, None, None, 64, 64, 0, None) == 1
    assert fold(BAD, None, None, P2, None, 64, 64, 0, None) == 1
    assert fold(P, None, None, P2, None, 0, 64, 0, None) == 1
    assert fold(P, None, None, P2, None, 64, 64, 7, None) == 1
    assert fold(P, BAD, None, P2, None, 64, 64, 0, None) == 1
    assert fold(P, None, BAD, P2, None, 64, 64, 0, None) == 1
    assert fold(P, None, None, P2, P3 + 2, 64, 64, 0, None) == 1
    # K or N not a multiple of 8 -> unsupported
    assert fold(P, None, None, P2, None, 60, 64, 0, None) == 2
    lazy = _lib.ng_rmsnorm_gemm_lazy_affine
    assert lazy(P, P2, P3 + 4, P3, 64, 64, 64, 0, 1e-6, None, None) == 1   # bias misaligned
    assert lazy(P, None, None, P3, 64, 64, 64, 0, 1e-6, None, None) == 1   # B NULL
    assert lazy(P, P2, None, P3, 64, 64, 64, 0, -1.0, None, None) == 1     # eps < 0
    assert lazy(P, P2, None, P3, 64, 100, 64, 0, 1e-6, None, None) == 2    # N % 8
    assert lazy(None, P2, None, None, 0, 64, 64, 0, 1e-6, None, None) == 0  # M = 0: no-op


P4 = P + 0x300000
P5 = P + 0x400000
P6 = P + 0x500000


def test_residual_argument_checks():
    rms, ln = _lib.ng_gemm_add_rmsnorm, _lib.ng_gemm_add_layernorm
    ws = _lib.ng_workspace_bytes(_lib.NG_OP_GEMM_ADD_LAYERNORM, 64, 4096, 64)
    assert ws == _lib.ng_workspace_bytes(_lib.NG_OP_GEMM_LAYERNORM, 64, 4096, 64) > 0
    assert _lib.ng_workspace_bytes(_lib.NG_OP_GEMM_ADD_RMSNORM, 64, 4096, 64) == ws
    assert _lib.ng_workspace_bytes(_lib.NG_OP_GEMM_ADD_RMSNORM, 64, 256, 64) == 0
    # R required, 16-byte aligned; S_out optional, aligned, not C
    assert rms(P, P2, None, None, P3, None, 64, 128, 64, 0, 1e-6, None, None, 0, None) == 1
    assert rms(P, P2, BAD, None, P3, None, 64, 128, 64, 0, 1e-6, None, None, 0, None) == 1
    assert rms(P, P2, P4, None, P3, BAD, 64, 128, 64, 0, 1e-6, None, None, 0, None) == 1
    assert rms(P, P2, P4, None, P3, P3, 64, 128, 64, 0, 1e-6, None, None, 0, None) == 1
    assert ln(P, P2, P4, None, None, P3, P3, 64, 128, 64, 0, 1e-5, None, None, None, 0,
              None) == 1
    # gamma/beta misaligned, bad eps, N % 8
    assert ln(P, P2, P4, P + 8, None, P3, None, 64, 128, 64, 0, 1e-5, None, None, None, 0,
              None) == 1
    assert ln(P, P2, P4, None, P + 8, P3, None, 64, 128, 64, 0, 1e-5, None, None, None, 0,
              None) == 1
    assert rms(P, P2, P4, None, P3, None, 64, 128, 64, 0, -1.0, None, None, 0, None) == 1
    assert rms(P, P2, P4, None, P3, None, 64, 100, 64, 0, 1e-6, None, None, 0, None) == 2
    # wide rows need the workspace
    assert ln(P, P2, P4, None, None, P3, None, 64, 4096, 64, 0, 1e-5, None, None, None, 0,
              None) == 3
    assert rms(P, P2, P4, None, P3, P5, 64, 4096, 64, 0, 1e-6, None, P, ws - 16, None) == 3
    # M = 0: a no-op, even with R NULL
    assert rms(None, P2, None, None, None, None, 0, 4096, 64, 0, 1e-6, None, None, 0, None) == 0
    assert ln(None, P2, None, None, None, None, None, 0, 128, 64, 0, 1e-5, None, None, None, 0,
              None) == 0


def test_add_norm_argument_checks():
    f = _lib.ng_add_norm
    assert f(P, None, None, None, P2, None, 4, 64, 0, 1e-6, None, None, None) == 1   # R NULL
    assert f(P, BAD, None, None, P2, None, 4, 64, 0, 1e-6, None, None, None) == 1    # R misaligned
    assert f(P, P3, None, None, P2, BAD, 4, 64, 0, 1e-6, None, None, None) == 1      # S_out misaligned
    assert f(P, P3, None, None, P2, P2, 4, 64, 0, 1e-6, None, None, None) == 1       # S_out == Y
    assert f(P, P3, None, None, P2, None, 4, 64, 0, 1e-6, P4, None, None) == 1       # RMS mean_out
    assert f(P, P3, None, None, P2, None, 4, 60, 1, 1e-6, None, None, None) == 2
    assert f(None, None, None, None, None, None, 0, 64, 1, 1e-6, None, None, None) == 0


def test_prenorm_layernorm_argument_checks():
    fold = _lib.ng_layernorm_gemm_fold
    assert fold(P, None, None, P2, None, P3, 64, 64, 0, None) == 1          # colsum NULL
    assert fold(P, None, None, P2, P4 + 4, P3, 64, 64, 0, None) == 1        # colsum misaligned
    assert fold(P, None, P5, P2, P4, None, 64, 64, 0, None) == 1            # beta without bias
    assert fold(P, None, None, P2, P4, P3 + 8, 64, 64, 0, None) == 1        # bias misaligned
    assert fold(P, None, None, P2, P4, None, 60, 64, 0, None) == 2          # K % 8
    f = _lib.ng_layernorm_gemm_prenorm
    assert f(P, P2, None, None, P3, 64, 64, 64, 0, 1e-5, P4, P5, None) == 1    # colsum NULL
    assert f(P, P2, P4 + 4, None, P3, 64, 64, 64, 0, 1e-5, P4, P5, None) == 1  # colsum misaligned
    assert f(P, P2, P4, P4 + 8, P3, 64, 64, 64, 0, 1e-5, P4, P5, None) == 1   # bias misaligned
    assert f(P, P2, P4, None, P3, 64, 64, 64, 0, 1e-5, None, P5, None) == 1   # mean NULL
    assert f(P, P2, P4, None, P3, 64, 64, 64, 0, 1e-5, P4, P5 + 2, None) == 1  # rstd misaligned
    assert f(P, P2, P4, None, P3, 64, 64, 64, 0, -1.0, P4, P5, None) == 1     # eps < 0
    assert f(P, P2, P4, None, P3, 64, 64, 65544, 0, 1e-5, P4, P5, None) == 2  # K > 65536
    assert f(P, P2, P4, None, P3, 64, 100, 64, 0, 1e-5, P4, P5, None) == 2    # N % 8
    assert f(None, P2, P4, None, None, 0, 64, 64, 0, 1e-5, None, None, None) == 0  # M = 0


def test_lazy_backward_argument_checks():
    f = _lib.ng_rmsnorm_gemm_lazy_backward_input
    op = _lib.NG_OP_RMSNORM_GEMM_LAZY_BWD_INPUT
    # rows of the forward A (length K) decide the strategy and the workspace
    assert _lib.ng_workspace_bytes(op, 64, 128, 256) == 0
    ws = _lib.ng_workspace_bytes(op, 64, 128, 4096)
    assert ws == _lib.ng_workspace_bytes(_lib.NG_OP_GEMM_RMSNORM, 64, 4096, 128) > 0
    assert f(P, P2, None, P4, P3, 64, 128, 64, 0, None, 0, None) == 1     # A NULL
    assert f(P, P2, P5, None, P3, 64, 128, 64, 0, None, 0, None) == 1     # rstd NULL
    assert f(P, P2, BAD, P4, P3, 64, 128, 64, 0, None, 0, None) == 1      # A misaligned
    assert f(P, P2, P5, P4 + 2, P3, 64, 128, 64, 0, None, 0, None) == 1   # rstd misaligned
    assert f(P, P2, P5, P4, P3, 64, 128, 64, 3, None, 0, None) == 1       # layout
    assert f(P, P2, P5, P4, P3, 64, 128, 60, 0, None, 0, None) == 2       # K % 8
    assert f(P, P2, P5, P4, P3, 64, 128, 4096, 0, None, 0, None) == 3     # workspace
    assert f(P, P2, P5, P4, P3, 64, 128, 4096, 1, P, ws - 16, None) == 3
    assert f(None, P2, None, None, None, 0, 128, 64, 0, None, 0, None) == 0  # M = 0
    w = _lib.ng_rmsnorm_gemm_lazy_backward_weight
    assert w(None, P2, P3, P4, 64, 128, 64, 0, None) == 1        # A NULL
    assert w(P, P2, P3, None, 64, 128, 64, 0, None) == 1         # dB NULL
    assert w(P, BAD, P3, P4, 64, 128, 64, 0, None) == 1          # dC misaligned
    assert w(P, P2, P3 + 2, P4, 64, 128, 64, 0, None) == 1       # rstd misaligned
    assert w(P, P2, P3, P4, 64, 128, 64, 2, None) == 1           # layout
    assert w(P, P2, P3, P4, 64, 100, 64, 0, None) == 2           # N % 8
    b = _lib.ng_rmsnorm_gemm_lazy_backward
    SC = 1 << 44  # scratch of 64 * 128 * 2 bytes, away from the other arguments
    assert b(P, P2, P5, P4, P3, None, SC, 64, 128, 64, 0, None, 0, None) == 1   # dB NULL
    assert b(P, P2, P5, P4, P3, P6, None, 64, 128, 64, 0, None, 0, None) == 1   # scratch NULL
    assert b(P, P2, P5, P4, P3, P6, SC + 8, 64, 128, 64, 0, None, 0, None) == 1  # misaligned
    # the scratch overlapping the input gradient, or starting inside dC
    assert b(P, P2, P5, P4, P3, P6, P3 - 1024, 64, 128, 64, 0, None, 0, None) == 1
    assert "overlap" in _lib.ng_last_error()
    assert b(P, P2, P5, P4, P3, P6, P + 4096, 64, 128, 64, 0, None, 0, None) == 1
    # ... or the workspace (K = 4096 needs one)
    wsb = _lib.ng_workspace_bytes(_lib.NG_OP_RMSNORM_GEMM_LAZY_BWD_INPUT, 64, 128, 4096)
    WS = 1 << 45
    assert b(P, P2, P5, P4, P3, P6, WS + 256, 64, 128, 4096, 0, WS, wsb, None) == 1
    assert "overlap" in _lib.ng_last_error()
    # then the input gradient's checks
    assert b(P, P2, None, P4, P3, P6, SC, 64, 128, 64, 0, None, 0, None) == 1   # A NULL
    assert b(P, P2, P5, P4, P3, P6, SC, 64, 128, 60, 0, None, 0, None) == 2     # K % 8
    assert b(P, P2, P5, P4, P3, P6, SC, 64, 128, 4096, 0, None, 0, None) == 3   # workspace
    at = _lib.ng_gemm_at
    assert at(None, P2, P3, 64, 64, 8, None) == 1
    assert at(P, P2, P3, 60, 64, 8, None) == 2                   # M % 8
    assert at(P, P2, P3, 64, 64, 0, None) == 1                   # K = 0
    g = _lib.ng_rmsnorm_backward
    assert g(None, P2, P3, P4, 4, 64, None) == 1
    assert g(P, BAD, P3, P4, 4, 64, None) == 1
    assert g(P, P2, P3 + 2, P4, 4, 64, None) == 1
    assert g(P, P2, P3, P4, 4, 60, None) == 2
    assert g(None, None, None, None, 0, 64, None) == 0


def test_workspace_helpers_argument_checks():
    assert _lib.ng_workspace_reset(None, 256, None) == 1
    assert _lib.ng_workspace_reset(P + 16, 256, None) == 1
    assert _lib.ng_workspace_status(None, None) == 1


def test_package_has_no_cpu_fallback():
    import normalization_gemm_amd as ng
    import torch
    A = torch.zeros((8, 8), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ng.rmsnorm_gemm_lazy(A, A)
    with pytest.raises(ValueError):
        ng.norm(A, "rms")


K_MAX = 1 << 22  # longest row of A [M, K] or B [N, K] a tile reads (header)


@pytest.mark.parametrize("lay", [0, 1])
def test_k_limit_at_the_boundary(lay):
    # 255 * 2K + 128 must stay below the 2 GiB buffer range of a 256-row tile
    assert 255 * 2 * K_MAX + 128 <= 0x7FFFFFF0
    M, N = 64, 64
    # just inside: validation passes (M = 0 stops before any launch)
    assert lazy(M=0, N=N, K=K_MAX, lay=lay) == 0
    assert _lib.ng_gemm(P, P2, P3, 0, N, K_MAX, lay, None) == 0
    # just outside: unsupported, for every entry point that reads rows of length K
    assert lazy(M=0, N=N, K=K_MAX + 8, lay=lay) == 2
    assert "2^22" in _lib.ng_last_error()
    assert lazy(M=M, N=N, K=K_MAX + 8, lay=lay) == 2
    assert _lib.ng_gemm(P, P2, P3, M, N, K_MAX + 8, lay, None) == 2
    assert _lib.ng_rmsnorm_gemm_lazy_affine(P, P2, None, P3, M, N, K_MAX + 8, lay, 1e-6, None,
                                            None) == 2
    assert _lib.ng_gemm_rmsnorm(P, P2, None, P3, M, N, K_MAX + 8, lay, 1e-6, None, None, 0,
                                None) == 2
    assert _lib.ng_gemm_layernorm(P, P2, None, None, P3, M, 4096, K_MAX + 8, lay, 1e-5, None,
                                  None, P, 1 << 20, None) == 2
    assert _lib.ng_gemm_add_rmsnorm(P, P2, P4, None, P3, None, M, N, K_MAX + 8, lay, 1e-6, None,
                                    None, 0, None) == 2
    # the input gradient's product reads rows of dC, of length N (forward)
    assert _lib.ng_rmsnorm_gemm_lazy_backward_input(P, P2, P5, P4, P3, M, K_MAX + 8, 64, lay,
                                                    None, 0, None) == 2


def test_weight_gradient_products_take_long_reductions():
    # A stored [K, M] (the reduction over storage rows): K up to 2^24 passes
    # validation (K reaches no row offset); checked without a launch (M, N
    # fail on alignment instead when they are set wrong)
    assert _lib.ng_gemm_at(P, P2, P3, 64, 64, (1 << 24) + 1, None) == 1   # K > 2^24
    assert _lib.ng_gemm_at(P, P2, P3, 60, 64, 1 << 24, None) == 2         # M % 8, K ok
    assert _lib.ng_rmsnorm_gemm_lazy_backward_weight(P, P2, P3, P4, 1 << 24, 100, 64, 0,
                                                     None) == 2           # N % 8, M ok


def test_debug_options():
    f = _lib.ng_set_debug_option
    assert f(_lib.NG_DEBUG_WAIT_SPINS, -2) == 1
    assert f(_lib.NG_DEBUG_WAIT_SPINS, (1 << 30) + 1) == 1
    assert f(_lib.NG_DEBUG_ROW_LOCAL_MAX, 257) == 1
    assert f(_lib.NG_DEBUG_TILE_ORDER, 3) == 1
    assert f(_lib.NG_DEBUG_K_WALK, 3) == 1
    assert f(_lib.NG_DEBUG_K_WALK, -1) == 1
    assert f(99, 0) == 1
    # the row-local maximum moves the workspace boundary, and is restored
    assert _lib.ng_workspace_bytes(_lib.NG_OP_GEMM_LAYERNORM, 1000, 256, 64) == 0
    assert f(_lib.NG_DEBUG_ROW_LOCAL_MAX, 0) == 0
    try:
        assert _lib.ng_workspace_bytes(_lib.NG_OP_GEMM_LAYERNORM, 1000, 256, 64) > 0
    finally:
        assert f(_lib.NG_DEBUG_ROW_LOCAL_MAX, -1) == 0
    assert _lib.ng_workspace_bytes(_lib.NG_OP_GEMM_LAYERNORM, 1000, 256, 64) == 0
    for v in (1, 2, 0):
        assert f(_lib.NG_DEBUG_TILE_ORDER, v) == 0
    for v in (_lib.NG_K_WALK_UPWARD, _lib.NG_K_WALK_ALTERNATE, _lib.NG_K_WALK_AUTO):
        assert f(_lib.NG_DEBUG_K_WALK, v) == 0
    assert f(_lib.NG_DEBUG_WAIT_SPINS, 0) == 0
    assert f(_lib.NG_DEBUG_WAIT_SPINS, -1) == 0


def test_autograd_op_has_no_cpu_fallback():
    # the differentiable op routes to the library only: CPU tensors are
    # refused before any call, never computed another way
    torch = pytest.importorskip("torch")
    from normalization_gemm_amd.autograd import lazy_rmsnorm_linear, lazy_rmsnorm_matmul
    x = torch.zeros((4, 16), dtype=torch.bfloat16, requires_grad=True)
    with pytest.raises(ValueError, match="GPU"):
        lazy_rmsnorm_linear(x, torch.zeros((8, 16), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="GPU"):
        lazy_rmsnorm_matmul(x, torch.zeros((16, 8), dtype=torch.bfloat16))
