"""normalization_gemm_amd: norm-fused bf16 GEMM on MI355X (gfx950).

Thin Python layer over libnormgemm (include/normgemm.h).  PyTorch provides
device memory and streams only: every step runs in the library's HIP kernels.
There is no CPU or PyTorch fallback; a missing library or a CPU tensor is an
error.

Raw C-ABI calls (integer pointers, status codes) live in ``_lib`` under the C
names (``ng_rmsnorm_gemm_lazy``, ...).  The tensor helpers below allocate the
outputs with torch, launch on the current stream and raise NormGemmError on a
non-zero status.
"""
from __future__ import annotations

from typing import Optional

from . import _lib
from ._lib import (  # noqa: F401
    NG_B_KN, NG_B_NK, NG_NORM_LAYER, NG_NORM_RMS, NG_OK,
    NG_OP_GEMM, NG_OP_GEMM_ADD_LAYERNORM, NG_OP_GEMM_ADD_RMSNORM, NG_OP_GEMM_LAYERNORM,
    NG_OP_GEMM_RMSNORM, NG_OP_NORM, NG_OP_RMSNORM_GEMM_LAZY, NG_OP_RMSNORM_GEMM_LAZY_BWD_INPUT,
    ng_gemm, ng_gemm_add_layernorm, ng_gemm_add_rmsnorm, ng_gemm_layernorm, ng_gemm_rmsnorm,
    ng_add_norm, ng_last_error, ng_layernorm_gemm_fold, ng_layernorm_gemm_prenorm,
    ng_lazy_fold_affine, ng_norm, ng_rmsnorm_backward, ng_rmsnorm_gemm_lazy_backward,
    ng_rmsnorm_gemm_lazy_backward_input,
    ng_rmsnorm_gemm_lazy_backward_weight, ng_gemm_at,
    ng_rmsnorm_gemm_lazy, ng_rmsnorm_gemm_lazy_affine, ng_status_string, ng_workspace_bytes,
    ng_workspace_reset, ng_workspace_status, ng_set_debug_option,
    NG_DEBUG_ROW_LOCAL_MAX, NG_DEBUG_TILE_ORDER, NG_DEBUG_WAIT_SPINS, NG_TILE_ORDER_NATURAL,
    NG_TILE_ORDER_REVERSED, NG_TILE_ORDER_SHUFFLED, NG_DEBUG_K_WALK, NG_K_WALK_AUTO,
    NG_K_WALK_UPWARD, NG_K_WALK_ALTERNATE,
)

__all__ = [
    "NormGemmError", "rmsnorm_gemm_lazy", "lazy_fold_affine", "rmsnorm_gemm_lazy_affine",
    "gemm_rmsnorm", "gemm_layernorm", "gemm_add_rmsnorm", "gemm_add_layernorm", "gemm", "norm",
    "add_norm", "layernorm_gemm_fold", "layernorm_gemm_prenorm",
    "rmsnorm_gemm_lazy_backward_input", "rmsnorm_gemm_lazy_backward_weight",
    "rmsnorm_gemm_lazy_backward", "rmsnorm_backward",
    "gemm_at",
    "Workspace", "library_path", "debug_option",
]


class NormGemmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (%s)" % (where, ng_status_string(status), ng_last_error()))


class debug_option:
    """Context manager: set a diagnostic option of the library (see
    ng_set_debug_option) for the duration of a block, then restore `reset`
    (the option's default)."""

    _DEFAULT = {NG_DEBUG_WAIT_SPINS: -1, NG_DEBUG_ROW_LOCAL_MAX: -1,
                NG_DEBUG_TILE_ORDER: NG_TILE_ORDER_NATURAL, NG_DEBUG_K_WALK: NG_K_WALK_AUTO}

    def __init__(self, option: int, value: int):
        self.option, self.value = option, value

    def __enter__(self):
        _check(ng_set_debug_option(self.option, self.value), "ng_set_debug_option")
        return self

    def __exit__(self, *exc):
        _check(ng_set_debug_option(self.option, self._DEFAULT[self.option]), "ng_set_debug_option")
        return False


def library_path() -> str:
    _lib.load()
    return _lib.LIB_PATH


def _torch():
    import torch
    return torch


def _check(status: int, where: str):
    if status != NG_OK:
        raise NormGemmError(status, where)


def _dev_bf16(t, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be on the GPU (got %s)" % (name, t.device))
    if t.dtype != torch.bfloat16:
        raise TypeError("%s must be bfloat16 (got %s)" % (name, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _empty(shape, dtype, device, stream):
    """A new tensor for a call launched on `stream`.  torch's allocator ties a
    block to the stream current at allocation; when the call runs on another
    stream the block is recorded on that one too, so that it is not handed
    out again (after the caller drops a temporary or an output) before the
    launch stream has passed the call."""
    torch = _torch()
    t = torch.empty(shape, dtype=dtype, device=device)
    if stream is not None:
        dev = torch.device(device)
        handle = _stream(stream)
        if handle != torch.cuda.current_stream(dev).cuda_stream:
            t.record_stream(torch.cuda.ExternalStream(handle, device=dev))
    return t


def _layout(b_layout):
    if b_layout in ("kn", NG_B_KN):
        return NG_B_KN
    if b_layout in ("nk", NG_B_NK):
        return NG_B_NK
    raise ValueError("b_layout must be 'kn' or 'nk'")


def _shapes(A, B, lay):
    if A.dim() != 2 or B.dim() != 2:
        raise ValueError("A and B must be 2-D")
    M, K = A.shape
    if lay == NG_B_KN:
        K2, N = B.shape
    else:
        N, K2 = B.shape
    if K2 != K:
        raise ValueError("inner dimensions differ: A %s, B %s" % (tuple(A.shape), tuple(B.shape)))
    return M, N, K


class Workspace:
    """Device scratch for the cross-workgroup epilogue.  It is zero-filled on
    `stream` (default: the current stream) by the library's fill kernel, so
    the fill is ordered before any call on that stream; the kernels leave it
    ready for the next call.  One workspace must not serve two calls that can
    run at the same time (e.g. on two streams without an ordering between
    them)."""

    def __init__(self, nbytes: int, device=None, stream=None):
        torch = _torch()
        dev = torch.device(device if device is not None else "cuda")
        self.nbytes = max(256, (int(nbytes) + 255) // 256 * 256)
        self.buf = torch.empty(self.nbytes, dtype=torch.uint8, device=dev)
        handle = _stream(stream)
        if stream is not None and handle != torch.cuda.current_stream(dev).cuda_stream:
            # used on another stream than the one that allocated it: the
            # allocator must not hand the block out again before that stream
            # has passed every call made on it
            self.buf.record_stream(torch.cuda.ExternalStream(handle, device=dev))
        _check(ng_workspace_reset(self.ptr(), self.nbytes, handle), "ng_workspace_reset")

    def ptr(self):
        return self.buf.data_ptr()

    def status(self, stream=None) -> int:
        return ng_workspace_status(self.ptr(), _stream(stream))


# Workspaces the tensor helpers create, one per (device, stream): calls on one
# stream run in order, so they can share one; calls on different streams get
# different workspaces.
_ws_cache = {}


def _workspace(op, M, N, K, device, workspace, stream):
    need = ng_workspace_bytes(op, M, N, K)
    if need == 0:
        return None, 0
    if workspace is not None:
        return workspace.ptr(), workspace.nbytes
    handle = _stream(stream)
    key = (str(device), handle)
    ws = _ws_cache.get(key)
    if ws is None or ws.nbytes < need:
        # (a replaced workspace's block is held back by the allocator until
        # the stream has passed the calls that used it: record_stream above,
        # or the stream that allocated it)
        ws = Workspace(need, device, stream=handle)
        _ws_cache[key] = ws
    return ws.ptr(), ws.nbytes


def rmsnorm_gemm_lazy(A, B, *, eps: float = 1e-6, b_layout="kn", out=None, rstd_out=None,
                      stream=None):
    """C = rmsnorm(A) @ B (RMSNorm without affine) as (A @ B) * rstd(A)."""
    torch = _torch()
    _dev_bf16(A, "A"); _dev_bf16(B, "B")
    lay = _layout(b_layout)
    M, N, K = _shapes(A, B, lay)
    C = out if out is not None else _empty((M, N), torch.bfloat16, A.device, stream)
    _dev_bf16(C, "out")
    _check(ng_rmsnorm_gemm_lazy(_ptr(A), _ptr(B), _ptr(C), M, N, K, lay, float(eps),
                                _ptr(rstd_out), _stream(stream)), "ng_rmsnorm_gemm_lazy")
    return C


def lazy_fold_affine(B, gamma=None, beta=None, *, b_layout="kn", out=None, bias_out=None,
                     stream=None):
    """Fold a pre-norm affine into the weights: returns (B_folded, bias) with
    B_folded = diag(gamma) B (bf16, B's layout) and bias = beta^T B (fp32 [N])."""
    torch = _torch()
    _dev_bf16(B, "B")
    lay = _layout(b_layout)
    if B.dim() != 2:
        raise ValueError("B must be 2-D")
    K, N = B.shape if lay == NG_B_KN else (B.shape[1], B.shape[0])
    if gamma is not None:
        _dev_bf16(gamma, "gamma")
    if beta is not None:
        _dev_bf16(beta, "beta")
    Bf = out if out is not None else _empty(B.shape, B.dtype, B.device, stream)
    _dev_bf16(Bf, "out")
    bias = bias_out if bias_out is not None else _empty(N, torch.float32, B.device, stream)
    _check(ng_lazy_fold_affine(_ptr(B), _ptr(gamma), _ptr(beta), _ptr(Bf), _ptr(bias), K, N, lay,
                               _stream(stream)), "ng_lazy_fold_affine")
    return Bf, bias


def rmsnorm_gemm_lazy_affine(A, B_folded, bias=None, *, eps: float = 1e-6, b_layout="kn",
                             out=None, rstd_out=None, stream=None):
    """C = (rmsnorm(A) * gamma + beta) @ B from the folded weights of
    lazy_fold_affine: rstd(A) * (A @ B_folded) + bias."""
    torch = _torch()
    _dev_bf16(A, "A"); _dev_bf16(B_folded, "B_folded")
    lay = _layout(b_layout)
    M, N, K = _shapes(A, B_folded, lay)
    if bias is not None and (bias.dtype != torch.float32 or bias.device.type != "cuda"
                             or not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous float32 GPU tensor")
    C = out if out is not None else _empty((M, N), torch.bfloat16, A.device, stream)
    _dev_bf16(C, "out")
    _check(ng_rmsnorm_gemm_lazy_affine(_ptr(A), _ptr(B_folded), _ptr(bias), _ptr(C), M, N, K, lay,
                                       float(eps), _ptr(rstd_out), _stream(stream)),
           "ng_rmsnorm_gemm_lazy_affine")
    return C


def layernorm_gemm_fold(B, gamma=None, beta=None, *, b_layout="kn", out=None, stream=None):
    """One-off weight fold of the pre-LayerNorm product: returns (B_folded,
    colsum, bias) with B_folded = diag(gamma) B (bf16, B's layout), colsum the
    fp32 column sums of B_folded and bias = beta^T B (fp32 [N])."""
    torch = _torch()
    _dev_bf16(B, "B")
    lay = _layout(b_layout)
    if B.dim() != 2:
        raise ValueError("B must be 2-D")
    K, N = B.shape if lay == NG_B_KN else (B.shape[1], B.shape[0])
    if gamma is not None:
        _dev_bf16(gamma, "gamma")
    if beta is not None:
        _dev_bf16(beta, "beta")
    Bf = out if out is not None else _empty(B.shape, B.dtype, B.device, stream)
    _dev_bf16(Bf, "out")
    colsum = _empty(N, torch.float32, B.device, stream)
    bias = _empty(N, torch.float32, B.device, stream)
    _check(ng_layernorm_gemm_fold(_ptr(B), _ptr(gamma), _ptr(beta), _ptr(Bf), _ptr(colsum),
                                  _ptr(bias), K, N, lay, _stream(stream)), "ng_layernorm_gemm_fold")
    return Bf, colsum, bias


def layernorm_gemm_prenorm(A, B_folded, colsum, bias=None, *, eps: float = 1e-5, b_layout="kn",
                           out=None, mean_out=None, rstd_out=None, stream=None):
    """C = (LayerNorm(A) * gamma + beta) @ B from the folded weights of
    layernorm_gemm_fold: a row-statistics pre-pass, then
    rstd * (A @ B_folded - mean * colsum) + bias."""
    torch = _torch()
    _dev_bf16(A, "A"); _dev_bf16(B_folded, "B_folded")
    lay = _layout(b_layout)
    M, N, K = _shapes(A, B_folded, lay)
    for t, name in ((colsum, "colsum"), (bias, "bias")):
        if t is not None and (t.dtype != torch.float32 or t.device.type != "cuda"
                              or not t.is_contiguous() or t.numel() != N):
            raise ValueError("%s must be a contiguous float32 GPU tensor of %d values" % (name, N))
    if colsum is None:
        raise ValueError("colsum is required")
    mean = mean_out if mean_out is not None else _empty(M, torch.float32, A.device, stream)
    rstd = rstd_out if rstd_out is not None else _empty(M, torch.float32, A.device, stream)
    C = out if out is not None else _empty((M, N), torch.bfloat16, A.device, stream)
    _dev_bf16(C, "out")
    _check(ng_layernorm_gemm_prenorm(_ptr(A), _ptr(B_folded), _ptr(colsum), _ptr(bias), _ptr(C),
                                     M, N, K, lay, float(eps), _ptr(mean), _ptr(rstd),
                                     _stream(stream)), "ng_layernorm_gemm_prenorm")
    return C


def _f32_vec(t, n, name):
    torch = _torch()
    if (t.dtype != torch.float32 or t.device.type != "cuda" or not t.is_contiguous()
            or t.numel() != n):
        raise ValueError("%s must be a contiguous float32 GPU tensor of %d values" % (name, n))


def rmsnorm_gemm_lazy_backward_input(dC, B, A, rstd, *, b_layout="kn", out=None,
                                     workspace: Optional[Workspace] = None, stream=None):
    """dA for C = rmsnorm(A) @ B (no affine) given dC: the norm's backward
    fused into the epilogue of dC @ B^T, from A and the forward's rstd."""
    torch = _torch()
    _dev_bf16(dC, "dC"); _dev_bf16(B, "B"); _dev_bf16(A, "A")
    lay = _layout(b_layout)
    M, N, K = _shapes(A, B, lay)
    if tuple(dC.shape) != (M, N):
        raise ValueError("dC must be [%d, %d] (got %s)" % (M, N, tuple(dC.shape)))
    _f32_vec(rstd, M, "rstd")
    dA = out if out is not None else _empty((M, K), torch.bfloat16, A.device, stream)
    _dev_bf16(dA, "out")
    ws, wsb = _workspace(NG_OP_RMSNORM_GEMM_LAZY_BWD_INPUT, M, N, K, A.device, workspace, stream)
    _check(ng_rmsnorm_gemm_lazy_backward_input(_ptr(dC), _ptr(B), _ptr(A), _ptr(rstd), _ptr(dA),
                                               M, N, K, lay, ws, wsb, _stream(stream)),
           "ng_rmsnorm_gemm_lazy_backward_input")
    return dA


def rmsnorm_gemm_lazy_backward_weight(A, dC, rstd, *, b_layout="kn", out=None, stream=None):
    """dB for C = rmsnorm(A) @ B (no affine) given dC: A_hat^T @ dC with the
    normalized A rebuilt from A and the forward's rstd; dB in B's layout."""
    torch = _torch()
    _dev_bf16(A, "A"); _dev_bf16(dC, "dC")
    lay = _layout(b_layout)
    if A.dim() != 2 or dC.dim() != 2 or A.shape[0] != dC.shape[0]:
        raise ValueError("A [M, K] and dC [M, N] must share M")
    M, K = A.shape
    N = dC.shape[1]
    _f32_vec(rstd, M, "rstd")
    shape = (K, N) if lay == NG_B_KN else (N, K)
    dB = out if out is not None else _empty(shape, torch.bfloat16, A.device, stream)
    _dev_bf16(dB, "out")
    if tuple(dB.shape) != shape:
        raise ValueError("out must be %s" % (shape,))
    _check(ng_rmsnorm_gemm_lazy_backward_weight(_ptr(A), _ptr(dC), _ptr(rstd), _ptr(dB), M, N, K,
                                                lay, _stream(stream)),
           "ng_rmsnorm_gemm_lazy_backward_weight")
    return dB


def rmsnorm_gemm_lazy_backward(dC, B, A, rstd, *, b_layout="kn", out_dA=None, out_dB=None,
                               scratch=None, workspace: Optional[Workspace] = None, stream=None):
    """(dA, dB) for C = rmsnorm(A) @ B (no affine) given dC, the weight
    gradient regrouped: the input-gradient kernel also writes rstd * dC into
    `scratch` (bf16 [M, N]) and dB = A^T @ scratch is a plain product; dB in
    B's layout."""
    torch = _torch()
    _dev_bf16(dC, "dC"); _dev_bf16(B, "B"); _dev_bf16(A, "A")
    lay = _layout(b_layout)
    M, N, K = _shapes(A, B, lay)
    if tuple(dC.shape) != (M, N):
        raise ValueError("dC must be [%d, %d] (got %s)" % (M, N, tuple(dC.shape)))
    _f32_vec(rstd, M, "rstd")
    dA = out_dA if out_dA is not None else _empty((M, K), torch.bfloat16, A.device, stream)
    _dev_bf16(dA, "out_dA")
    shape = (K, N) if lay == NG_B_KN else (N, K)
    dB = out_dB if out_dB is not None else _empty(shape, torch.bfloat16, A.device, stream)
    _dev_bf16(dB, "out_dB")
    if tuple(dB.shape) != shape:
        raise ValueError("out_dB must be %s" % (shape,))
    sc = scratch if scratch is not None else _empty((M, N), torch.bfloat16, A.device, stream)
    _dev_bf16(sc, "scratch")
    if sc.numel() != M * N:
        raise ValueError("scratch must hold %d bf16 values" % (M * N))
    ws, wsb = _workspace(NG_OP_RMSNORM_GEMM_LAZY_BWD_INPUT, M, N, K, A.device, workspace, stream)
    _check(ng_rmsnorm_gemm_lazy_backward(_ptr(dC), _ptr(B), _ptr(A), _ptr(rstd), _ptr(dA),
                                         _ptr(dB), _ptr(sc), M, N, K, lay, ws, wsb,
                                         _stream(stream)),
           "ng_rmsnorm_gemm_lazy_backward")
    return dA, dB


def gemm_at(A, B, *, out=None, stream=None):
    """C = A^T @ B with A stored [K, M] and B stored [K, N]."""
    torch = _torch()
    _dev_bf16(A, "A"); _dev_bf16(B, "B")
    if A.dim() != 2 or B.dim() != 2 or A.shape[0] != B.shape[0]:
        raise ValueError("A [K, M] and B [K, N] must share K")
    K, M = A.shape
    N = B.shape[1]
    C = out if out is not None else _empty((M, N), torch.bfloat16, A.device, stream)
    _dev_bf16(C, "out")
    _check(ng_gemm_at(_ptr(A), _ptr(B), _ptr(C), M, N, K, _stream(stream)), "ng_gemm_at")
    return C


def rmsnorm_backward(dY, X, rstd, *, out=None, stream=None):
    """Standalone RMSNorm backward (no affine): dX from dY, X and the saved rstd."""
    torch = _torch()
    _dev_bf16(dY, "dY"); _dev_bf16(X, "X")
    if X.dim() != 2 or tuple(dY.shape) != tuple(X.shape):
        raise ValueError("dY and X must be 2-D of one shape")
    rows, cols = X.shape
    _f32_vec(rstd, rows, "rstd")
    dX = out if out is not None else _empty(X.shape, X.dtype, X.device, stream)
    _dev_bf16(dX, "out")
    _check(ng_rmsnorm_backward(_ptr(dY), _ptr(X), _ptr(rstd), _ptr(dX), rows, cols,
                               _stream(stream)), "ng_rmsnorm_backward")
    return dX


def gemm_rmsnorm(A, B, gamma=None, *, eps: float = 1e-6, b_layout="kn", out=None,
                 rstd_out=None, workspace: Optional[Workspace] = None, stream=None):
    """C = RMSNorm(A @ B) over each output row, optional per-column gamma."""
    torch = _torch()
    _dev_bf16(A, "A"); _dev_bf16(B, "B")
    if gamma is not None:
        _dev_bf16(gamma, "gamma")
    lay = _layout(b_layout)
    M, N, K = _shapes(A, B, lay)
    C = out if out is not None else _empty((M, N), torch.bfloat16, A.device, stream)
    _dev_bf16(C, "out")
    ws, wsb = _workspace(NG_OP_GEMM_RMSNORM, M, N, K, A.device, workspace, stream)
    _check(ng_gemm_rmsnorm(_ptr(A), _ptr(B), _ptr(gamma), _ptr(C), M, N, K, lay, float(eps),
                           _ptr(rstd_out), ws, wsb, _stream(stream)), "ng_gemm_rmsnorm")
    return C


def gemm_layernorm(A, B, gamma=None, beta=None, *, eps: float = 1e-5, b_layout="kn", out=None,
                   mean_out=None, rstd_out=None, workspace: Optional[Workspace] = None,
                   stream=None):
    """C = LayerNorm(A @ B) over each output row, optional per-column gamma/beta."""
    torch = _torch()
    _dev_bf16(A, "A"); _dev_bf16(B, "B")
    if gamma is not None:
        _dev_bf16(gamma, "gamma")
    if beta is not None:
        _dev_bf16(beta, "beta")
    lay = _layout(b_layout)
    M, N, K = _shapes(A, B, lay)
    C = out if out is not None else _empty((M, N), torch.bfloat16, A.device, stream)
    _dev_bf16(C, "out")
    ws, wsb = _workspace(NG_OP_GEMM_LAYERNORM, M, N, K, A.device, workspace, stream)
    _check(ng_gemm_layernorm(_ptr(A), _ptr(B), _ptr(gamma), _ptr(beta), _ptr(C), M, N, K, lay,
                             float(eps), _ptr(mean_out), _ptr(rstd_out), ws, wsb,
                             _stream(stream)), "ng_gemm_layernorm")
    return C


def _residual(R, S_out, M, N):
    _dev_bf16(R, "R")
    if tuple(R.shape) != (M, N):
        raise ValueError("R must be [%d, %d] (got %s)" % (M, N, tuple(R.shape)))
    if S_out is not None:
        _dev_bf16(S_out, "s_out")
        if tuple(S_out.shape) != (M, N):
            raise ValueError("s_out must be [%d, %d]" % (M, N))


def gemm_add_rmsnorm(A, B, R, gamma=None, *, eps: float = 1e-6, b_layout="kn", out=None,
                     s_out=None, rstd_out=None, workspace: Optional[Workspace] = None,
                     stream=None):
    """C = RMSNorm(A @ B + R) over each output row, optional per-column gamma;
    s_out, when given, receives A @ B + R in bf16 (R may be out or s_out for
    an in-place update)."""
    torch = _torch()
    _dev_bf16(A, "A"); _dev_bf16(B, "B")
    if gamma is not None:
        _dev_bf16(gamma, "gamma")
    lay = _layout(b_layout)
    M, N, K = _shapes(A, B, lay)
    _residual(R, s_out, M, N)
    C = out if out is not None else _empty((M, N), torch.bfloat16, A.device, stream)
    _dev_bf16(C, "out")
    ws, wsb = _workspace(NG_OP_GEMM_ADD_RMSNORM, M, N, K, A.device, workspace, stream)
    _check(ng_gemm_add_rmsnorm(_ptr(A), _ptr(B), _ptr(R), _ptr(gamma), _ptr(C), _ptr(s_out), M, N,
                               K, lay, float(eps), _ptr(rstd_out), ws, wsb, _stream(stream)),
           "ng_gemm_add_rmsnorm")
    return C


def gemm_add_layernorm(A, B, R, gamma=None, beta=None, *, eps: float = 1e-5, b_layout="kn",
                       out=None, s_out=None, mean_out=None, rstd_out=None,
                       workspace: Optional[Workspace] = None, stream=None):
    """C = LayerNorm(A @ B + R) over each output row, optional per-column
    gamma/beta; s_out as for gemm_add_rmsnorm."""
    torch = _torch()
    _dev_bf16(A, "A"); _dev_bf16(B, "B")
    if gamma is not None:
        _dev_bf16(gamma, "gamma")
    if beta is not None:
        _dev_bf16(beta, "beta")
    lay = _layout(b_layout)
    M, N, K = _shapes(A, B, lay)
    _residual(R, s_out, M, N)
    C = out if out is not None else _empty((M, N), torch.bfloat16, A.device, stream)
    _dev_bf16(C, "out")
    ws, wsb = _workspace(NG_OP_GEMM_ADD_LAYERNORM, M, N, K, A.device, workspace, stream)
    _check(ng_gemm_add_layernorm(_ptr(A), _ptr(B), _ptr(R), _ptr(gamma), _ptr(beta), _ptr(C),
                                 _ptr(s_out), M, N, K, lay, float(eps), _ptr(mean_out),
                                 _ptr(rstd_out), ws, wsb, _stream(stream)),
           "ng_gemm_add_layernorm")
    return C


def gemm(A, B, *, b_layout="kn", out=None, stream=None):
    """C = A @ B (bf16 out, fp32 accumulation): the unfused baseline GEMM."""
    torch = _torch()
    _dev_bf16(A, "A"); _dev_bf16(B, "B")
    lay = _layout(b_layout)
    M, N, K = _shapes(A, B, lay)
    C = out if out is not None else _empty((M, N), torch.bfloat16, A.device, stream)
    _dev_bf16(C, "out")
    _check(ng_gemm(_ptr(A), _ptr(B), _ptr(C), M, N, K, lay, _stream(stream)), "ng_gemm")
    return C


def norm(X, kind: str, gamma=None, beta=None, *, eps: float = 1e-5, out=None, mean_out=None,
         rstd_out=None, stream=None):
    """Standalone row norm ('rms' or 'layer'): the unfused baseline norm."""
    torch = _torch()
    _dev_bf16(X, "X")
    if X.dim() != 2:
        raise ValueError("X must be 2-D")
    k = {"rms": NG_NORM_RMS, "layer": NG_NORM_LAYER}[kind]
    if gamma is not None:
        _dev_bf16(gamma, "gamma")
    if beta is not None:
        _dev_bf16(beta, "beta")
    Y = out if out is not None else _empty(X.shape, X.dtype, X.device, stream)
    _dev_bf16(Y, "out")
    rows, cols = X.shape
    _check(ng_norm(_ptr(X), _ptr(gamma), _ptr(beta), _ptr(Y), rows, cols, k, float(eps),
                   _ptr(mean_out), _ptr(rstd_out), _stream(stream)), "ng_norm")
    return Y


def add_norm(X, R, kind: str, gamma=None, beta=None, *, eps: float = 1e-5, out=None, s_out=None,
             mean_out=None, rstd_out=None, stream=None):
    """Standalone residual add + row norm: Y = norm(X + R) with X + R rounded
    to bf16 (s_out, when given, receives it): the unfused baseline's norm."""
    torch = _torch()
    _dev_bf16(X, "X")
    if X.dim() != 2:
        raise ValueError("X must be 2-D")
    rows, cols = X.shape
    _residual(R, s_out, rows, cols)
    k = {"rms": NG_NORM_RMS, "layer": NG_NORM_LAYER}[kind]
    if gamma is not None:
        _dev_bf16(gamma, "gamma")
    if beta is not None:
        _dev_bf16(beta, "beta")
    Y = out if out is not None else _empty(X.shape, X.dtype, X.device, stream)
    _dev_bf16(Y, "out")
    _check(ng_add_norm(_ptr(X), _ptr(R), _ptr(gamma), _ptr(beta), _ptr(Y), _ptr(s_out), rows, cols,
                       k, float(eps), _ptr(mean_out), _ptr(rstd_out), _stream(stream)),
           "ng_add_norm")
    return Y
