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

NG_DEBUG_WAIT_SPINS = 0
NG_DEBUG_ROW_LOCAL_MAX = 1
NG_DEBUG_TILE_ORDER = 2
NG_TILE_ORDER_NATURAL = 0
NG_TILE_ORDER_REVERSED = 1
NG_TILE_ORDER_SHUFFLED = 2
NG_DEBUG_K_WALK = 3
NG_K_WALK_AUTO = 0
NG_K_WALK_UPWARD = 1
NG_K_WALK_ALTERNATE = 2

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
    "ng_rmsnorm_gemm_lazy_backward": (_I, [_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _P,
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
    "ng_set_debug_option": (_I, [_I, _I64]),
    "ng_gemm_layernorm_noalloc": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _F, _P, _P, _P]),
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


def _delegate(name):
    def fn(*args):
        return getattr(load(), name)(*args)
    fn.__name__ = fn.__qualname__ = name
    fn.__doc__ = "C entry point %s (include/normgemm.h); returns what it returns." % name
    return fn


# One Python function per C entry point, same name and argument order.
for _name in _SIGNATURES:
    globals()[_name] = _delegate(_name)
del _name


def ng_status_string(status):
    return _call("ng_status_string", status).decode()


def ng_last_error():
    return _call("ng_last_error").decode()
