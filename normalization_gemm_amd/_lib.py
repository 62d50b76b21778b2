"""ctypes view of libnormgemm.so: the C ABI declared in include/normgemm.h.

Functions here take raw integers for device pointers and streams and return
the C status code, with the same names as the C entry points.  Loading fails
loudly if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libnormgemm.so")

NG_OK = 0
NG_ERR_INVALID_ARG = 1
NG_ERR_UNSUPPORTED = 2
NG_ERR_WORKSPACE = 3
NG_ERR_HIP = 4
NG_ERR_TIMEOUT = 5

NG_NORM_RMS = 0
NG_NORM_LAYER = 1
NG_B_KN = 0
NG_B_NK = 1

NG_OP_RMSNORM_GEMM_LAZY = 0
NG_OP_GEMM_RMSNORM = 1
NG_OP_GEMM_LAYERNORM = 2
NG_OP_GEMM = 3
NG_OP_NORM = 4
NG_OP_GEMM_ADD_RMSNORM = 5
NG_OP_GEMM_ADD_LAYERNORM = 6
NG_OP_RMSNORM_GEMM_LAZY_BWD_INPUT = 7

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int
_F = ctypes.c_float
_SZ = ctypes.c_size_t

_SIGNATURES = {
    "ng_rmsnorm_gemm_lazy": (_I, [_P, _P, _P, _I64, _I64, _I64, _I, _F, _P, _P]),
    "ng_gemm_rmsnorm": (_I, [_P, _P, _P, _P, _I64, _I64, _I64, _I, _F, _P, _P, _SZ, _P]),
    "ng_gemm_layernorm": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _F, _P, _P, _P, _SZ, _P]),
    "ng_gemm_add_rmsnorm": (_I, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _F, _P, _P, _SZ,
                                 _P]),
    "ng_gemm_add_layernorm": (_I, [_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _F, _P, _P,
                                   _P, _SZ, _P]),
    "ng_layernorm_gemm_fold": (_I, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I, _P]),
    "ng_layernorm_gemm_prenorm": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _F, _P, _P, _P]),
    "ng_rmsnorm_gemm_lazy_backward_input": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _P,
                                                 _SZ, _P]),
    "ng_rmsnorm_backward": (_I, [_P, _P, _P, _P, _I64, _I64, _P]),
    "ng_rmsnorm_gemm_lazy_backward_weight": (_I, [_P, _P, _P, _P, _I64, _I64, _I64, _I, _P]),
    "ng_gemm_at": (_I, [_P, _P, _P, _I64, _I64, _I64, _P]),
    "ng_lazy_fold_affine": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I, _P]),
    "ng_rmsnorm_gemm_lazy_affine": (_I, [_P, _P, _P, _P, _I64, _I64, _I64, _I, _F, _P, _P]),
    "ng_gemm": (_I, [_P, _P, _P, _I64, _I64, _I64, _I, _P]),
    "ng_norm": (_I, [_P, _P, _P, _P, _I64, _I64, _I, _F, _P, _P, _P]),
    "ng_add_norm": (_I, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I, _F, _P, _P, _P]),
    "ng_workspace_bytes": (_SZ, [_I, _I64, _I64, _I64]),
    "ng_workspace_reset": (_I, [_P, _SZ, _P]),
    "ng_workspace_status": (_I, [_P, _P]),
    "ng_status_string": (ctypes.c_char_p, [_I]),
    "ng_last_error": (ctypes.c_char_p, []),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load the built library (once).  Raises ImportError if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                "libnormgemm.so is not built at %s; run `python -m normalization_gemm_amd.build`"
                % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def exported_names():
    return list(_SIGNATURES)


def _call(name, *args):
    return getattr(load(), name)(*args)


def ng_rmsnorm_gemm_lazy(A, B, C, M, N, K, b_layout, eps, rstd_out, stream):
    return _call("ng_rmsnorm_gemm_lazy", A, B, C, M, N, K, b_layout, eps, rstd_out, stream)


def ng_lazy_fold_affine(B, gamma, beta, B_folded, bias, K, N, b_layout, stream):
    return _call("ng_lazy_fold_affine", B, gamma, beta, B_folded, bias, K, N, b_layout, stream)


def ng_rmsnorm_gemm_lazy_affine(A, B_folded, bias, C, M, N, K, b_layout, eps, rstd_out, stream):
    return _call("ng_rmsnorm_gemm_lazy_affine", A, B_folded, bias, C, M, N, K, b_layout, eps,
                 rstd_out, stream)


def ng_gemm_rmsnorm(A, B, gamma, C, M, N, K, b_layout, eps, rstd_out, workspace,
                    workspace_bytes, stream):
    return _call("ng_gemm_rmsnorm", A, B, gamma, C, M, N, K, b_layout, eps, rstd_out,
                 workspace, workspace_bytes, stream)


def ng_gemm_layernorm(A, B, gamma, beta, C, M, N, K, b_layout, eps, mean_out, rstd_out,
                      workspace, workspace_bytes, stream):
    return _call("ng_gemm_layernorm", A, B, gamma, beta, C, M, N, K, b_layout, eps, mean_out,
                 rstd_out, workspace, workspace_bytes, stream)


def ng_gemm_add_rmsnorm(A, B, R, gamma, C, S_out, M, N, K, b_layout, eps, rstd_out, workspace,
                        workspace_bytes, stream):
    return _call("ng_gemm_add_rmsnorm", A, B, R, gamma, C, S_out, M, N, K, b_layout, eps,
                 rstd_out, workspace, workspace_bytes, stream)


def ng_gemm_add_layernorm(A, B, R, gamma, beta, C, S_out, M, N, K, b_layout, eps, mean_out,
                          rstd_out, workspace, workspace_bytes, stream):
    return _call("ng_gemm_add_layernorm", A, B, R, gamma, beta, C, S_out, M, N, K, b_layout, eps,
                 mean_out, rstd_out, workspace, workspace_bytes, stream)


def ng_layernorm_gemm_fold(B, gamma, beta, B_folded, colsum, bias, K, N, b_layout, stream):
    return _call("ng_layernorm_gemm_fold", B, gamma, beta, B_folded, colsum, bias, K, N, b_layout,
                 stream)


def ng_layernorm_gemm_prenorm(A, B_folded, colsum, bias, C, M, N, K, b_layout, eps, mean, rstd,
                              stream):
    return _call("ng_layernorm_gemm_prenorm", A, B_folded, colsum, bias, C, M, N, K, b_layout, eps,
                 mean, rstd, stream)


def ng_rmsnorm_gemm_lazy_backward_input(dC, B, A, rstd, dA, M, N, K, b_layout, workspace,
                                         workspace_bytes, stream):
    return _call("ng_rmsnorm_gemm_lazy_backward_input", dC, B, A, rstd, dA, M, N, K, b_layout,
                 workspace, workspace_bytes, stream)


def ng_rmsnorm_gemm_lazy_backward_weight(A, dC, rstd, dB, M, N, K, b_layout, stream):
    return _call("ng_rmsnorm_gemm_lazy_backward_weight", A, dC, rstd, dB, M, N, K, b_layout,
                 stream)


def ng_gemm_at(A, B, C, M, N, K, stream):
    return _call("ng_gemm_at", A, B, C, M, N, K, stream)


def ng_rmsnorm_backward(dY, X, rstd, dX, rows, cols, stream):
    return _call("ng_rmsnorm_backward", dY, X, rstd, dX, rows, cols, stream)


def ng_gemm(A, B, C, M, N, K, b_layout, stream):
    return _call("ng_gemm", A, B, C, M, N, K, b_layout, stream)


def ng_norm(X, gamma, beta, Y, rows, cols, kind, eps, mean_out, rstd_out, stream):
    return _call("ng_norm", X, gamma, beta, Y, rows, cols, kind, eps, mean_out, rstd_out, stream)


def ng_add_norm(X, R, gamma, beta, Y, S_out, rows, cols, kind, eps, mean_out, rstd_out, stream):
    return _call("ng_add_norm", X, R, gamma, beta, Y, S_out, rows, cols, kind, eps, mean_out,
                 rstd_out, stream)


def ng_workspace_bytes(op, M, N, K):
    return _call("ng_workspace_bytes", op, M, N, K)


def ng_workspace_reset(workspace, workspace_bytes, stream):
    return _call("ng_workspace_reset", workspace, workspace_bytes, stream)


def ng_workspace_status(workspace, stream):
    return _call("ng_workspace_status", workspace, stream)


def ng_status_string(status):
    return _call("ng_status_string", status).decode()


def ng_last_error():
    return _call("ng_last_error").decode()
