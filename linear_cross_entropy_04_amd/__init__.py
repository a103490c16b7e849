"""Chunked fused linear cross-entropy for AMD MI355X (gfx950).

Python binding of ``libflce.so`` (declared in ``include/flce.h``): argument
marshalling only.  Every step of the computation runs in the library's HIP
kernels; there is no Python or CPU fallback, and a missing library raises.

The operation is the one the Liger Kernel pages call as
``loss_fn(weight, input, target)`` (project overview page, "Método de API de
Baixo Nível"): the LM-head projection fused with cross-entropy over tokens
whose target is not ``ignore_index`` -- their mean, their sum, or the
per-token losses with an upstream gradient per token.  On the same kernels:
cross-entropy on given logits (``cross_entropy``) and the fused-linear
post-training losses the pages list (``orpo_loss``, ``preference_loss`` for
ORPO / SimPO / CPO / DPO, ``kto_loss``, and their module forms).
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "FLCE_F32", "FLCE_BF16", "FLCEError", "flce_workspace_bytes", "flce_plan", "flce_fwd_bwd",
    "flce_fwd_bwd_noalloc", "flce_noalloc_scratch_bytes",
    "flce_fwd", "flce_fwd_bwd_ex", "flce_fwd_ex", "REDUCTIONS", "flce_scale_inplace", "flce_status_string", "flce_last_error", "lib_path",
    "flce_profile_enable", "flce_profile_read", "flce_profile_select",
    "workspace", "loss", "FusedLinearCrossEntropyLoss",
    "flce_ce_workspace_bytes", "flce_ce_fwd_bwd", "flce_ce_fwd", "cross_entropy",
    "flce_orpo_workspace_bytes", "flce_orpo_fwd_bwd", "flce_orpo_fwd", "orpo_loss",
    "FusedLinearORPOLoss", "PAIR_KINDS", "flce_pair_workspace_bytes", "flce_pair_fwd_bwd",
    "flce_pair_fwd", "preference_loss", "sequence_logps", "FusedLinearSimPOLoss",
    "FusedLinearCPOLoss", "FusedLinearDPOLoss", "flce_kto_workspace_bytes", "flce_kto_fwd_bwd",
    "flce_kto_fwd", "flce_kto_reference_point", "kto_loss", "kto_reference_point",
    "FusedLinearKTOLoss",
]

FLCE_F32 = 0
FLCE_BF16 = 1
FLCE_OK, FLCE_EINVAL, FLCE_ELABEL, FLCE_EWORKSPACE, FLCE_EHIP, FLCE_EUNSUPPORTED = range(6)
REDUCTIONS = {"mean": 0, "sum": 1, "none": 2}        # flce_reduction

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libflce.so")
_lib = None

_p, _i64, _i32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t


class FLCEError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = f"{where}: {flce_status_string(status)} (status {status})"
        if status == FLCE_EHIP:
            msg += f": {flce_last_error()}"
        super().__init__(msg)
        self.status = status


def lib_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built; run `python -m "
                          "linear_cross_entropy_04_amd.build_lib` (or __graft_entry__.build())")
    l = ctypes.CDLL(_LIB_PATH)
    l.flce_workspace_bytes.argtypes = [_i64, _i64, _i64, _i32, _i64]
    l.flce_workspace_bytes.restype = _sz
    l.flce_plan.argtypes = [_i64, _i64, _i64, _i32, ctypes.POINTER(_i64), _sz,
                            ctypes.POINTER(_sz)]
    l.flce_plan.restype = _i32
    l.flce_fwd_bwd.argtypes = [_p, _p, _p, _i64, _i64, _i64, _i32, _i64, _i64,
                               ctypes.POINTER(ctypes.c_float), _p, _p, _p, _p, _p, _sz, _p]
    l.flce_fwd_bwd.restype = _i32
    l.flce_fwd.argtypes = [_p, _p, _p, _i64, _i64, _i64, _i32, _i64, _i64,
                           ctypes.POINTER(ctypes.c_float), _p, _p, _p, _sz, _p]
    l.flce_fwd.restype = _i32
    l.flce_fwd_bwd_ex.argtypes = [_p, _p, _p, _i64, _i64, _i64, _i32, _i64, _i64, _i32, _p, _i32,
                                  ctypes.POINTER(ctypes.c_float), _p, _p, _p, _p, _p, _p, _sz,
                                  _p]
    l.flce_fwd_bwd_ex.restype = _i32
    l.flce_fwd_ex.argtypes = [_p, _p, _p, _i64, _i64, _i64, _i32, _i64, _i64, _i32,
                              ctypes.POINTER(ctypes.c_float), _p, _p, _p, _p, _sz, _p]
    l.flce_fwd_ex.restype = _i32
    l.flce_ce_workspace_bytes.argtypes = [_i64]
    l.flce_ce_workspace_bytes.restype = _sz
    l.flce_ce_fwd_bwd.argtypes = [_p, _p, _i64, _i64, _i32, _i64, _i32, _p,
                                  ctypes.POINTER(ctypes.c_float), _p, _p, _p, _p, _sz, _p]
    l.flce_ce_fwd_bwd.restype = _i32
    l.flce_ce_fwd.argtypes = [_p, _p, _i64, _i64, _i32, _i64, _i32,
                              ctypes.POINTER(ctypes.c_float), _p, _p, _p, _p, _sz, _p]
    l.flce_ce_fwd.restype = _i32
    l.flce_orpo_workspace_bytes.argtypes = [_i64, _i64, _i64, _i64, _i32, _i64]
    l.flce_orpo_workspace_bytes.restype = _sz
    l.flce_orpo_fwd_bwd.argtypes = [_p, _p, _p, _i64, _i64, _i64, _i64, _i32, _i64,
                                    ctypes.c_float, _i64, ctypes.POINTER(ctypes.c_float),
                                    ctypes.POINTER(ctypes.c_float), _p, _p, _p, _p, _p, _p, _sz,
                                    _p]
    l.flce_orpo_fwd_bwd.restype = _i32
    l.flce_orpo_fwd.argtypes = [_p, _p, _p, _i64, _i64, _i64, _i64, _i32, _i64, ctypes.c_float,
                                _i64, ctypes.POINTER(ctypes.c_float),
                                ctypes.POINTER(ctypes.c_float), _p, _p, _p, _p, _sz, _p]
    l.flce_orpo_fwd.restype = _i32
    l.flce_pair_workspace_bytes.argtypes = [_i64, _i64, _i64, _i64, _i32, _i64]
    l.flce_pair_workspace_bytes.restype = _sz
    _f = ctypes.c_float
    l.flce_pair_fwd_bwd.argtypes = [_i32, _p, _p, _p, _i64, _i64, _i64, _i64, _i32, _i64, _f, _f,
                                    _f, _p, _p, _i64, ctypes.POINTER(_f), ctypes.POINTER(_f), _p,
                                    _p, _p, _p, _p, _p, _sz, _p]
    l.flce_pair_fwd_bwd.restype = _i32
    l.flce_pair_fwd.argtypes = [_i32, _p, _p, _p, _i64, _i64, _i64, _i64, _i32, _i64, _f, _f, _f,
                                _p, _p, _i64, ctypes.POINTER(_f), ctypes.POINTER(_f), _p, _p, _p,
                                _p, _sz, _p]
    l.flce_pair_fwd.restype = _i32
    l.flce_kto_workspace_bytes.argtypes = [_i64, _i64, _i64, _i64, _i32, _i64]
    l.flce_kto_workspace_bytes.restype = _sz
    l.flce_kto_fwd_bwd.argtypes = [_p, _p, _p, _i64, _i64, _i64, _i64, _i32, _i64, _p, _p, _f, _f,
                                   _f, _f, _i64, ctypes.POINTER(_f), _p, _p, _p, _p, _p, _sz, _p]
    l.flce_kto_fwd_bwd.restype = _i32
    l.flce_kto_fwd.argtypes = [_p, _p, _p, _i64, _i64, _i64, _i64, _i32, _i64, _p, _p, _f, _f, _f,
                               _f, _i64, ctypes.POINTER(_f), _p, _p, _p, _sz, _p]
    l.flce_kto_fwd.restype = _i32
    l.flce_noalloc_scratch_bytes.argtypes = []
    l.flce_noalloc_scratch_bytes.restype = _sz
    l.flce_fwd_bwd_noalloc.argtypes = [_p, _p, _p, _i64, _i64, _i64, _i32, _i64, _i64,
                                       ctypes.POINTER(_f), _p, _p, _p, _p, _p]
    l.flce_fwd_bwd_noalloc.restype = _i32
    l.flce_kto_reference_point.argtypes = [_p, _p, _p, _i64, _i64, _i64, _i64, _i32, _i64, _p,
                                           _i64, ctypes.POINTER(_f), _p, _p, _p, _sz, _p]
    l.flce_kto_reference_point.restype = _i32
    l.flce_scale_inplace.argtypes = [_p, _i64, _i32, _p, _p]
    l.flce_scale_inplace.restype = _i32
    l.flce_status_string.argtypes = [_i32]
    l.flce_status_string.restype = ctypes.c_char_p
    l.flce_last_error.argtypes = []
    l.flce_last_error.restype = ctypes.c_char_p
    l.flce_profile_enable.argtypes = [_i32]
    l.flce_profile_enable.restype = _i32
    l.flce_profile_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_i64), _i32]
    l.flce_profile_read.restype = _i32
    l.flce_profile_select.argtypes = [ctypes.c_uint32]
    l.flce_profile_select.restype = _i32
    l.flce_kernel_name.argtypes = [_i32]
    l.flce_kernel_name.restype = ctypes.c_char_p
    _lib = l
    return l


def flce_status_string(status: int) -> str:
    return _load().flce_status_string(int(status)).decode()


def flce_last_error() -> str:
    return _load().flce_last_error().decode()


KERNEL_CLASSES = 12


def flce_profile_enable(enable: bool = True) -> None:
    """Turn per-kernel event timing on or off (process-wide)."""
    _load().flce_profile_enable(1 if enable else 0)


def flce_profile_select(classes=None) -> None:
    """Time only these kernel classes (names as flce_profile_read reports
    them, or FLCE_K_* ids) while timing is on; None: every class."""
    if classes is None:
        mask = 0xFFFFFFFF
    else:
        l = _load()
        names = {l.flce_kernel_name(k).decode(): k for k in range(KERNEL_CLASSES)}
        mask = 0
        for c in classes:
            k = names[c] if isinstance(c, str) else int(c)
            if not 0 <= k < KERNEL_CLASSES:
                raise ValueError(f"kernel class {c!r}")
            mask |= 1 << k
    _load().flce_profile_select(mask)


def flce_profile_read() -> dict:
    """{kernel class name: (summed ms, launches)} since the last read; clears."""
    ms = (ctypes.c_double * KERNEL_CLASSES)()
    n = (_i64 * KERNEL_CLASSES)()
    st = _load().flce_profile_read(ms, n, KERNEL_CLASSES)
    if st != FLCE_OK:
        raise FLCEError(st, "flce_profile_read")
    return {_load().flce_kernel_name(k).decode(): (float(ms[k]), int(n[k]))
            for k in range(KERNEL_CLASSES)}


def flce_workspace_bytes(N: int, H: int, V: int, dtype: int, chunk_tokens: int = 0) -> int:
    return int(_load().flce_workspace_bytes(N, H, V, dtype, chunk_tokens))


def flce_plan(N: int, H: int, V: int, dtype: int, scratch_budget_bytes: int = 0,
              chunk_tokens: int = 0) -> tuple[int, int, int]:
    """Returns (status, chunk_tokens, peak_scratch_bytes)."""
    c = _i64(chunk_tokens)
    peak = _sz(0)
    st = _load().flce_plan(N, H, V, dtype, ctypes.byref(c), scratch_budget_bytes, ctypes.byref(peak))
    return int(st), int(c.value), int(peak.value)


# ------------------------------------------------------------------ marshalling

def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return FLCE_BF16
    if t.dtype == torch.float32:
        return FLCE_F32
    raise ValueError(f"unsupported dtype {t.dtype}; expected bfloat16 or float32")


def _dev(t, name, dtype=None, shape=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a HIP device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def workspace(N: int, H: int, V: int, dtype: int, chunk_tokens: int = 0, device=None) -> torch.Tensor:
    """A device workspace of the size flce_workspace_bytes reports."""
    nbytes = flce_workspace_bytes(N, H, V, dtype, chunk_tokens)
    if nbytes == 0:
        raise FLCEError(FLCE_EINVAL, "flce_workspace_bytes")
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def flce_fwd_bwd(X: torch.Tensor, W: torch.Tensor, labels: torch.Tensor, ignore_index: int,
                 chunk_tokens: int, dX: torch.Tensor, dW: torch.Tensor, workspace: torch.Tensor,
                 stream=None, row_loss: torch.Tensor | None = None,
                 row_lse: torch.Tensor | None = None) -> float:
    """Call libflce's flce_fwd_bwd on device tensors; returns the loss."""
    N, H = X.shape
    V = W.shape[0]
    dt = _dtype_code(X)
    _dev(X, "X")
    _dev(W, "W", X.dtype, (V, H))
    _dev(labels, "labels", torch.int64, (N,))
    _dev(dX, "dX", X.dtype, (N, H))
    _dev(dW, "dW", torch.float32, (V, H))
    _dev(workspace, "workspace")
    _dev(row_loss, "row_loss", torch.float32, (N,))
    _dev(row_lse, "row_lse", torch.float32, (N,))
    loss = ctypes.c_float(0.0)
    st = _load().flce_fwd_bwd(_ptr(X), _ptr(W), _ptr(labels), N, H, V, dt, ignore_index,
                              chunk_tokens, ctypes.byref(loss), _ptr(dX), _ptr(dW),
                              _ptr(row_loss), _ptr(row_lse), _ptr(workspace),
                              workspace.numel(), _stream(stream, X.device))
    if st != FLCE_OK:
        raise FLCEError(st, "flce_fwd_bwd")
    return float(loss.value)


def flce_noalloc_scratch_bytes() -> int:
    return int(_load().flce_noalloc_scratch_bytes())


def flce_fwd_bwd_noalloc(X: torch.Tensor, W: torch.Tensor, labels: torch.Tensor,
                         ignore_index: int, chunk_tokens: int, dX: torch.Tensor, dW: torch.Tensor,
                         stream=None, row_loss: torch.Tensor | None = None,
                         row_lse: torch.Tensor | None = None) -> float:
    """Call libflce's flce_fwd_bwd_noalloc (no workspace argument: the library's
    own device scratch array); returns the loss."""
    N, H = X.shape
    V = W.shape[0]
    dt = _dtype_code(X)
    _dev(X, "X")
    _dev(W, "W", X.dtype, (V, H))
    _dev(labels, "labels", torch.int64, (N,))
    _dev(dX, "dX", X.dtype, (N, H))
    _dev(dW, "dW", torch.float32, (V, H))
    _dev(row_loss, "row_loss", torch.float32, (N,))
    _dev(row_lse, "row_lse", torch.float32, (N,))
    loss = ctypes.c_float(0.0)
    st = _load().flce_fwd_bwd_noalloc(_ptr(X), _ptr(W), _ptr(labels), N, H, V, dt, ignore_index,
                                      chunk_tokens, ctypes.byref(loss), _ptr(dX), _ptr(dW),
                                      _ptr(row_loss), _ptr(row_lse), _stream(stream, X.device))
    if st != FLCE_OK:
        raise FLCEError(st, "flce_fwd_bwd_noalloc")
    return float(loss.value)


def flce_fwd(X: torch.Tensor, W: torch.Tensor, labels: torch.Tensor, ignore_index: int,
             chunk_tokens: int, workspace: torch.Tensor, stream=None,
             row_loss: torch.Tensor | None = None, row_lse: torch.Tensor | None = None) -> float:
    """Call libflce's flce_fwd on device tensors; returns the loss."""
    N, H = X.shape
    V = W.shape[0]
    dt = _dtype_code(X)
    _dev(X, "X")
    _dev(W, "W", X.dtype, (V, H))
    _dev(labels, "labels", torch.int64, (N,))
    _dev(workspace, "workspace")
    _dev(row_loss, "row_loss", torch.float32, (N,))
    _dev(row_lse, "row_lse", torch.float32, (N,))
    loss = ctypes.c_float(0.0)
    st = _load().flce_fwd(_ptr(X), _ptr(W), _ptr(labels), N, H, V, dt, ignore_index,
                          chunk_tokens, ctypes.byref(loss), _ptr(row_loss), _ptr(row_lse),
                          _ptr(workspace), workspace.numel(), _stream(stream, X.device))
    if st != FLCE_OK:
        raise FLCEError(st, "flce_fwd")
    return float(loss.value)


def _reduction_code(reduction: str) -> int:
    if reduction not in REDUCTIONS:
        raise ValueError(f"reduction must be one of {tuple(REDUCTIONS)}, got {reduction!r}")
    return REDUCTIONS[reduction]


def flce_fwd_bwd_ex(X: torch.Tensor, W: torch.Tensor, labels: torch.Tensor, ignore_index: int,
                    chunk_tokens: int, dX: torch.Tensor, dW: torch.Tensor,
                    workspace: torch.Tensor, reduction: str = "mean",
                    grad_rows: torch.Tensor | None = None, accumulate_dw: bool = False,
                    row_loss: torch.Tensor | None = None, row_lse: torch.Tensor | None = None,
                    logprob: torch.Tensor | None = None, stream=None) -> float:
    """Call libflce's flce_fwd_bwd_ex on device tensors; returns the loss."""
    N, H = X.shape
    V = W.shape[0]
    dt = _dtype_code(X)
    _dev(X, "X")
    _dev(W, "W", X.dtype, (V, H))
    _dev(labels, "labels", torch.int64, (N,))
    _dev(dX, "dX", X.dtype, (N, H))
    _dev(dW, "dW", torch.float32, (V, H))
    _dev(workspace, "workspace")
    for t, name in ((grad_rows, "grad_rows"), (row_loss, "row_loss"), (row_lse, "row_lse"),
                    (logprob, "logprob")):
        _dev(t, name, torch.float32, (N,))
    loss = ctypes.c_float(0.0)
    st = _load().flce_fwd_bwd_ex(_ptr(X), _ptr(W), _ptr(labels), N, H, V, dt, ignore_index,
                                 chunk_tokens, _reduction_code(reduction), _ptr(grad_rows),
                                 1 if accumulate_dw else 0, ctypes.byref(loss), _ptr(dX),
                                 _ptr(dW), _ptr(row_loss), _ptr(row_lse), _ptr(logprob),
                                 _ptr(workspace), workspace.numel(), _stream(stream, X.device))
    if st != FLCE_OK:
        raise FLCEError(st, "flce_fwd_bwd_ex")
    return float(loss.value)


def flce_fwd_ex(X: torch.Tensor, W: torch.Tensor, labels: torch.Tensor, ignore_index: int,
                chunk_tokens: int, workspace: torch.Tensor, reduction: str = "mean",
                row_loss: torch.Tensor | None = None, row_lse: torch.Tensor | None = None,
                logprob: torch.Tensor | None = None, stream=None) -> float:
    """Call libflce's flce_fwd_ex on device tensors; returns the loss."""
    N, H = X.shape
    V = W.shape[0]
    dt = _dtype_code(X)
    _dev(X, "X")
    _dev(W, "W", X.dtype, (V, H))
    _dev(labels, "labels", torch.int64, (N,))
    _dev(workspace, "workspace")
    for t, name in ((row_loss, "row_loss"), (row_lse, "row_lse"), (logprob, "logprob")):
        _dev(t, name, torch.float32, (N,))
    loss = ctypes.c_float(0.0)
    st = _load().flce_fwd_ex(_ptr(X), _ptr(W), _ptr(labels), N, H, V, dt, ignore_index,
                             chunk_tokens, _reduction_code(reduction), ctypes.byref(loss),
                             _ptr(row_loss), _ptr(row_lse), _ptr(logprob), _ptr(workspace),
                             workspace.numel(), _stream(stream, X.device))
    if st != FLCE_OK:
        raise FLCEError(st, "flce_fwd_ex")
    return float(loss.value)


def flce_ce_workspace_bytes(N: int) -> int:
    return int(_load().flce_ce_workspace_bytes(N))


def _ce_args(logits, labels, workspace, grad_rows, row_loss, row_lse, logprob):
    N, V = logits.shape
    _dev(logits, "logits")
    _dev(labels, "labels", torch.int64, (N,))
    _dev(workspace, "workspace")
    for t, name in ((grad_rows, "grad_rows"), (row_loss, "row_loss"), (row_lse, "row_lse"),
                    (logprob, "logprob")):
        _dev(t, name, torch.float32, (N,))
    return N, V, _dtype_code(logits)


def flce_ce_fwd_bwd(logits: torch.Tensor, labels: torch.Tensor, ignore_index: int,
                    workspace: torch.Tensor, reduction: str = "mean",
                    grad_rows: torch.Tensor | None = None, row_loss: torch.Tensor | None = None,
                    row_lse: torch.Tensor | None = None, logprob: torch.Tensor | None = None,
                    stream=None) -> float:
    """Call libflce's flce_ce_fwd_bwd: returns the loss; logits is overwritten
    with dL/dlogits."""
    N, V, dt = _ce_args(logits, labels, workspace, grad_rows, row_loss, row_lse, logprob)
    loss = ctypes.c_float(0.0)
    st = _load().flce_ce_fwd_bwd(_ptr(logits), _ptr(labels), N, V, dt, ignore_index,
                                 _reduction_code(reduction), _ptr(grad_rows), ctypes.byref(loss),
                                 _ptr(row_loss), _ptr(row_lse), _ptr(logprob), _ptr(workspace),
                                 workspace.numel(), _stream(stream, logits.device))
    if st != FLCE_OK:
        raise FLCEError(st, "flce_ce_fwd_bwd")
    return float(loss.value)


def flce_ce_fwd(logits: torch.Tensor, labels: torch.Tensor, ignore_index: int,
                workspace: torch.Tensor, reduction: str = "mean",
                row_loss: torch.Tensor | None = None, row_lse: torch.Tensor | None = None,
                logprob: torch.Tensor | None = None, stream=None) -> float:
    """Call libflce's flce_ce_fwd (logits read only); returns the loss."""
    N, V, dt = _ce_args(logits, labels, workspace, None, row_loss, row_lse, logprob)
    loss = ctypes.c_float(0.0)
    st = _load().flce_ce_fwd(_ptr(logits), _ptr(labels), N, V, dt, ignore_index,
                             _reduction_code(reduction), ctypes.byref(loss), _ptr(row_loss),
                             _ptr(row_lse), _ptr(logprob), _ptr(workspace), workspace.numel(),
                             _stream(stream, logits.device))
    if st != FLCE_OK:
        raise FLCEError(st, "flce_ce_fwd")
    return float(loss.value)


def flce_orpo_workspace_bytes(n_pairs: int, T: int, H: int, V: int, dtype: int,
                              chunk_pairs: int = 0) -> int:
    return int(_load().flce_orpo_workspace_bytes(n_pairs, T, H, V, dtype, chunk_pairs))


def _orpo_args(X, W, labels, n_pairs, workspace, chosen_logp, rejected_logp, log_odds_ratio):
    N, H = X.shape
    V = W.shape[0]
    if n_pairs <= 0 or N % (2 * n_pairs) != 0:
        raise ValueError(f"X has {N} rows: not 2 * n_pairs = {2 * n_pairs} equal sequences")
    _dev(X, "X")
    _dev(W, "W", X.dtype, (V, H))
    _dev(labels, "labels", torch.int64, (N,))
    _dev(workspace, "workspace")
    for t, name in ((chosen_logp, "chosen_logp"), (rejected_logp, "rejected_logp"),
                    (log_odds_ratio, "log_odds_ratio")):
        _dev(t, name, torch.float32, (n_pairs,))
    return N // (2 * n_pairs), H, V, _dtype_code(X)


def flce_orpo_fwd_bwd(X: torch.Tensor, W: torch.Tensor, labels: torch.Tensor, n_pairs: int,
                      ignore_index: int, beta: float, chunk_pairs: int, dX: torch.Tensor,
                      dW: torch.Tensor, workspace: torch.Tensor,
                      chosen_logp: torch.Tensor | None = None,
                      rejected_logp: torch.Tensor | None = None,
                      log_odds_ratio: torch.Tensor | None = None,
                      stream=None) -> tuple[float, float]:
    """Call libflce's flce_orpo_fwd_bwd: X holds 2 n_pairs sequences (chosen
    first) as rows; returns (loss, nll)."""
    T, H, V, dt = _orpo_args(X, W, labels, n_pairs, workspace, chosen_logp, rejected_logp,
                             log_odds_ratio)
    _dev(dX, "dX", X.dtype, tuple(X.shape))
    _dev(dW, "dW", torch.float32, (V, H))
    loss, nll = ctypes.c_float(0.0), ctypes.c_float(0.0)
    st = _load().flce_orpo_fwd_bwd(_ptr(X), _ptr(W), _ptr(labels), n_pairs, T, H, V, dt,
                                   ignore_index, float(beta), chunk_pairs, ctypes.byref(loss),
                                   ctypes.byref(nll), _ptr(dX), _ptr(dW), _ptr(chosen_logp),
                                   _ptr(rejected_logp), _ptr(log_odds_ratio), _ptr(workspace),
                                   workspace.numel(), _stream(stream, X.device))
    if st != FLCE_OK:
        raise FLCEError(st, "flce_orpo_fwd_bwd")
    return float(loss.value), float(nll.value)


def flce_orpo_fwd(X: torch.Tensor, W: torch.Tensor, labels: torch.Tensor, n_pairs: int,
                  ignore_index: int, beta: float, chunk_pairs: int, workspace: torch.Tensor,
                  chosen_logp: torch.Tensor | None = None,
                  rejected_logp: torch.Tensor | None = None,
                  log_odds_ratio: torch.Tensor | None = None,
                  stream=None) -> tuple[float, float]:
    """Call libflce's flce_orpo_fwd; returns (loss, nll)."""
    T, H, V, dt = _orpo_args(X, W, labels, n_pairs, workspace, chosen_logp, rejected_logp,
                             log_odds_ratio)
    loss, nll = ctypes.c_float(0.0), ctypes.c_float(0.0)
    st = _load().flce_orpo_fwd(_ptr(X), _ptr(W), _ptr(labels), n_pairs, T, H, V, dt,
                               ignore_index, float(beta), chunk_pairs, ctypes.byref(loss),
                               ctypes.byref(nll), _ptr(chosen_logp), _ptr(rejected_logp),
                               _ptr(log_odds_ratio), _ptr(workspace), workspace.numel(),
                               _stream(stream, X.device))
    if st != FLCE_OK:
        raise FLCEError(st, "flce_orpo_fwd")
    return float(loss.value), float(nll.value)


PAIR_KINDS = {"orpo": 0, "simpo": 1, "cpo": 2, "dpo": 3}          # flce_pair_loss


def _pair_kind(kind: str) -> int:
    if kind not in PAIR_KINDS:
        raise ValueError(f"kind must be one of {tuple(PAIR_KINDS)}, got {kind!r}")
    return PAIR_KINDS[kind]


def flce_pair_workspace_bytes(n_pairs: int, T: int, H: int, V: int, dtype: int,
                              chunk_pairs: int = 0) -> int:
    return int(_load().flce_pair_workspace_bytes(n_pairs, T, H, V, dtype, chunk_pairs))


def flce_pair_fwd_bwd(kind: str, X: torch.Tensor, W: torch.Tensor, labels: torch.Tensor,
                      n_pairs: int, ignore_index: int, beta: float, gamma: float, alpha: float,
                      chunk_pairs: int, dX: torch.Tensor, dW: torch.Tensor,
                      workspace: torch.Tensor, ref_chosen_logp: torch.Tensor | None = None,
                      ref_rejected_logp: torch.Tensor | None = None,
                      chosen_logp: torch.Tensor | None = None,
                      rejected_logp: torch.Tensor | None = None,
                      pair_logit: torch.Tensor | None = None, stream=None) -> tuple[float, float]:
    """Call libflce's flce_pair_fwd_bwd; returns (loss, nll)."""
    T, H, V, dt = _orpo_args(X, W, labels, n_pairs, workspace, chosen_logp, rejected_logp,
                             pair_logit)
    _dev(dX, "dX", X.dtype, tuple(X.shape))
    _dev(dW, "dW", torch.float32, (V, H))
    _dev(ref_chosen_logp, "ref_chosen_logp", torch.float32, (n_pairs,))
    _dev(ref_rejected_logp, "ref_rejected_logp", torch.float32, (n_pairs,))
    loss, nll = ctypes.c_float(0.0), ctypes.c_float(0.0)
    st = _load().flce_pair_fwd_bwd(_pair_kind(kind), _ptr(X), _ptr(W), _ptr(labels), n_pairs, T,
                                   H, V, dt, ignore_index, float(beta), float(gamma),
                                   float(alpha), _ptr(ref_chosen_logp), _ptr(ref_rejected_logp),
                                   chunk_pairs, ctypes.byref(loss), ctypes.byref(nll), _ptr(dX),
                                   _ptr(dW), _ptr(chosen_logp), _ptr(rejected_logp),
                                   _ptr(pair_logit), _ptr(workspace), workspace.numel(),
                                   _stream(stream, X.device))
    if st != FLCE_OK:
        raise FLCEError(st, "flce_pair_fwd_bwd")
    return float(loss.value), float(nll.value)


def flce_pair_fwd(kind: str, X: torch.Tensor, W: torch.Tensor, labels: torch.Tensor,
                  n_pairs: int, ignore_index: int, beta: float, gamma: float, alpha: float,
                  chunk_pairs: int, workspace: torch.Tensor,
                  ref_chosen_logp: torch.Tensor | None = None,
                  ref_rejected_logp: torch.Tensor | None = None,
                  chosen_logp: torch.Tensor | None = None,
                  rejected_logp: torch.Tensor | None = None,
                  pair_logit: torch.Tensor | None = None, stream=None) -> tuple[float, float]:
    """Call libflce's flce_pair_fwd; returns (loss, nll)."""
    T, H, V, dt = _orpo_args(X, W, labels, n_pairs, workspace, chosen_logp, rejected_logp,
                             pair_logit)
    _dev(ref_chosen_logp, "ref_chosen_logp", torch.float32, (n_pairs,))
    _dev(ref_rejected_logp, "ref_rejected_logp", torch.float32, (n_pairs,))
    loss, nll = ctypes.c_float(0.0), ctypes.c_float(0.0)
    st = _load().flce_pair_fwd(_pair_kind(kind), _ptr(X), _ptr(W), _ptr(labels), n_pairs, T, H, V,
                               dt, ignore_index, float(beta), float(gamma), float(alpha),
                               _ptr(ref_chosen_logp), _ptr(ref_rejected_logp), chunk_pairs,
                               ctypes.byref(loss), ctypes.byref(nll), _ptr(chosen_logp),
                               _ptr(rejected_logp), _ptr(pair_logit), _ptr(workspace),
                               workspace.numel(), _stream(stream, X.device))
    if st != FLCE_OK:
        raise FLCEError(st, "flce_pair_fwd")
    return float(loss.value), float(nll.value)


def flce_kto_workspace_bytes(n_seq: int, T: int, H: int, V: int, dtype: int,
                             chunk_seqs: int = 0) -> int:
    return int(_load().flce_kto_workspace_bytes(n_seq, T, H, V, dtype, chunk_seqs))


def _kto_args(X, W, labels, n_seq, desirable, ref_logp, workspace, logp, reward):
    N, H = X.shape
    V = W.shape[0]
    if n_seq <= 0 or N % n_seq != 0:
        raise ValueError(f"X has {N} rows: not n_seq = {n_seq} equal sequences")
    _dev(X, "X")
    _dev(W, "W", X.dtype, (V, H))
    _dev(labels, "labels", torch.int64, (N,))
    _dev(desirable, "desirable", torch.int32, (n_seq,))
    _dev(ref_logp, "ref_logp", torch.float32, (n_seq,))
    _dev(workspace, "workspace")
    for t, name in ((logp, "logp"), (reward, "reward")):
        _dev(t, name, torch.float32, (n_seq,))
    return N // n_seq, H, V, _dtype_code(X)


def flce_kto_fwd_bwd(X: torch.Tensor, W: torch.Tensor, labels: torch.Tensor, n_seq: int,
                     ignore_index: int, desirable: torch.Tensor, ref_logp: torch.Tensor,
                     beta: float, z0: float, lambda_d: float, lambda_u: float, chunk_seqs: int,
                     dX: torch.Tensor, dW: torch.Tensor, workspace: torch.Tensor,
                     logp: torch.Tensor | None = None, reward: torch.Tensor | None = None,
                     stream=None) -> float:
    """Call libflce's flce_kto_fwd_bwd; returns the loss."""
    T, H, V, dt = _kto_args(X, W, labels, n_seq, desirable, ref_logp, workspace, logp, reward)
    _dev(dX, "dX", X.dtype, tuple(X.shape))
    _dev(dW, "dW", torch.float32, (V, H))
    loss = ctypes.c_float(0.0)
    st = _load().flce_kto_fwd_bwd(_ptr(X), _ptr(W), _ptr(labels), n_seq, T, H, V, dt,
                                  ignore_index, _ptr(desirable), _ptr(ref_logp), float(beta),
                                  float(z0), float(lambda_d), float(lambda_u), chunk_seqs,
                                  ctypes.byref(loss), _ptr(dX), _ptr(dW), _ptr(logp),
                                  _ptr(reward), _ptr(workspace), workspace.numel(),
                                  _stream(stream, X.device))
    if st != FLCE_OK:
        raise FLCEError(st, "flce_kto_fwd_bwd")
    return float(loss.value)


def flce_kto_fwd(X: torch.Tensor, W: torch.Tensor, labels: torch.Tensor, n_seq: int,
                 ignore_index: int, desirable: torch.Tensor, ref_logp: torch.Tensor, beta: float,
                 z0: float, lambda_d: float, lambda_u: float, chunk_seqs: int,
                 workspace: torch.Tensor, logp: torch.Tensor | None = None,
                 reward: torch.Tensor | None = None, stream=None) -> float:
    """Call libflce's flce_kto_fwd; returns the loss."""
    T, H, V, dt = _kto_args(X, W, labels, n_seq, desirable, ref_logp, workspace, logp, reward)
    loss = ctypes.c_float(0.0)
    st = _load().flce_kto_fwd(_ptr(X), _ptr(W), _ptr(labels), n_seq, T, H, V, dt, ignore_index,
                              _ptr(desirable), _ptr(ref_logp), float(beta), float(z0),
                              float(lambda_d), float(lambda_u), chunk_seqs, ctypes.byref(loss),
                              _ptr(logp), _ptr(reward), _ptr(workspace), workspace.numel(),
                              _stream(stream, X.device))
    if st != FLCE_OK:
        raise FLCEError(st, "flce_kto_fwd")
    return float(loss.value)


def flce_kto_reference_point(X: torch.Tensor, W: torch.Tensor, labels: torch.Tensor, n_seq: int,
                             ignore_index: int, ref_logp: torch.Tensor, chunk_seqs: int,
                             workspace: torch.Tensor, logp: torch.Tensor | None = None,
                             reward: torch.Tensor | None = None, stream=None) -> float:
    """Call libflce's flce_kto_reference_point; returns z0."""
    N, H = X.shape
    V = W.shape[0]
    if n_seq <= 0 or N % n_seq != 0:
        raise ValueError(f"X has {N} rows: not n_seq = {n_seq} equal sequences")
    _dev(X, "X")
    _dev(W, "W", X.dtype, (V, H))
    _dev(labels, "labels", torch.int64, (N,))
    _dev(ref_logp, "ref_logp", torch.float32, (n_seq,))
    _dev(workspace, "workspace")
    for t, name in ((logp, "logp"), (reward, "reward")):
        _dev(t, name, torch.float32, (n_seq,))
    z0 = ctypes.c_float(0.0)
    st = _load().flce_kto_reference_point(_ptr(X), _ptr(W), _ptr(labels), n_seq, N // n_seq, H, V,
                                          _dtype_code(X), ignore_index, _ptr(ref_logp), chunk_seqs,
                                          ctypes.byref(z0), _ptr(logp), _ptr(reward),
                                          _ptr(workspace), workspace.numel(),
                                          _stream(stream, X.device))
    if st != FLCE_OK:
        raise FLCEError(st, "flce_kto_reference_point")
    return float(z0.value)


def flce_scale_inplace(buf: torch.Tensor, scale: torch.Tensor, stream=None) -> None:
    """buf *= scale (a one-element fp32 device tensor), in place, on the stream."""
    _dev(buf, "buf")
    _dev(scale, "scale", torch.float32)
    if scale.numel() != 1:
        raise ValueError("scale must hold one element")
    st = _load().flce_scale_inplace(_ptr(buf), buf.numel(), _dtype_code(buf), _ptr(scale),
                                    _stream(stream, buf.device))
    if st != FLCE_OK:
        raise FLCEError(st, "flce_scale_inplace")


def _consume_once(ctx):
    """The backward functions below scale the gradients saved by the forward
    in place by the upstream gradient, so a second backward through the same
    graph (retain_graph=True) would see them already scaled: refuse it."""
    if getattr(ctx, "consumed", False):
        raise RuntimeError("the fused loss's saved gradients were already used by a backward "
                           "pass; recompute the loss to differentiate it again")
    ctx.consumed = True


# ------------------------------------------------------------------ autograd

class _FLCEFunction(torch.autograd.Function):
    """Mean or sum: the gradients are computed with the loss (one call) and
    scaled by the upstream gradient in backward."""

    @staticmethod
    def forward(ctx, weight, input, target, ignore_index, chunk_tokens, reduction):
        N, H = input.shape
        V = weight.shape[0]
        dt = _dtype_code(input)
        ws = workspace(N, H, V, dt, chunk_tokens, device=input.device)
        need = ctx.needs_input_grad[0] or ctx.needs_input_grad[1]
        if need:
            dX = torch.empty_like(input)
            dW = torch.empty((V, H), dtype=torch.float32, device=input.device)
            val = flce_fwd_bwd_ex(input, weight, target, ignore_index, chunk_tokens, dX, dW, ws,
                                  reduction=reduction)
            ctx.save_for_backward(dX, dW)
        else:
            val = flce_fwd_ex(input, weight, target, ignore_index, chunk_tokens, ws,
                              reduction=reduction)
        ctx.wdtype = weight.dtype
        return torch.tensor(val, dtype=torch.float32, device=input.device)

    @staticmethod
    def backward(ctx, grad_out):
        _consume_once(ctx)
        dX, dW = ctx.saved_tensors
        g = grad_out.detach().to(torch.float32).reshape(1).contiguous()
        flce_scale_inplace(dX, g)
        flce_scale_inplace(dW, g)
        gw = dW if ctx.wdtype == torch.float32 else dW.to(ctx.wdtype)
        return gw, dX, None, None, None, None


class _FLCETokenFunction(torch.autograd.Function):
    """Per-token losses: the forward returns the loss vector; the backward
    runs the fused forward and backward again with the upstream gradient of
    each token as its weight."""

    @staticmethod
    def forward(ctx, weight, input, target, ignore_index, chunk_tokens):
        N, H = input.shape
        V = weight.shape[0]
        ws = workspace(N, H, V, _dtype_code(input), chunk_tokens, device=input.device)
        row = torch.empty(N, dtype=torch.float32, device=input.device)
        flce_fwd_ex(input, weight, target, ignore_index, chunk_tokens, ws, reduction="none",
                    row_loss=row)
        ctx.save_for_backward(weight, input, target)
        ctx.ignore_index, ctx.chunk_tokens = ignore_index, chunk_tokens
        return row

    @staticmethod
    def backward(ctx, grad_rows):
        weight, input, target = ctx.saved_tensors
        N, H = input.shape
        V = weight.shape[0]
        ws = workspace(N, H, V, _dtype_code(input), ctx.chunk_tokens, device=input.device)
        dX = torch.empty_like(input)
        dW = torch.empty((V, H), dtype=torch.float32, device=input.device)
        row = torch.empty(N, dtype=torch.float32, device=input.device)
        g = grad_rows.detach().to(torch.float32).contiguous()
        flce_fwd_bwd_ex(input, weight, target, ctx.ignore_index, ctx.chunk_tokens, dX, dW, ws,
                        reduction="none", grad_rows=g, row_loss=row)
        gw = dW if weight.dtype == torch.float32 else dW.to(weight.dtype)
        return gw, dX, None, None, None


def loss(weight: torch.Tensor, input: torch.Tensor, target: torch.Tensor,
         ignore_index: int = -100, chunk_tokens: int = 0,
         reduction: str = "mean") -> torch.Tensor:
    """Cross-entropy of input @ weight.T against target, fused and chunked.

    weight [V, H], input [N, H] (both bf16 or both fp32, contiguous, on the
    GPU), target [N] int64.  reduction "mean" (over tokens whose target is not
    ignore_index) or "sum" returns a scalar; "none" returns the per-token
    losses [N] (0 on ignored tokens).  Gradients flow to weight and input."""
    _reduction_code(reduction)
    if reduction == "none":
        return _FLCETokenFunction.apply(weight, input, target, ignore_index, chunk_tokens)
    return _FLCEFunction.apply(weight, input, target, ignore_index, chunk_tokens, reduction)


class FusedLinearCrossEntropyLoss(torch.nn.Module):
    """Module form of :func:`loss`: ``loss_fn(weight, input, target)``."""

    def __init__(self, ignore_index: int = -100, chunk_tokens: int = 0, reduction: str = "mean"):
        super().__init__()
        self.ignore_index = ignore_index
        self.chunk_tokens = chunk_tokens
        self.reduction = reduction

    def forward(self, weight, input, target):
        return loss(weight, input, target, self.ignore_index, self.chunk_tokens, self.reduction)


class _CEFunction(torch.autograd.Function):
    """Cross-entropy on given logits, mean or sum.  With gradients, the
    logits buffer (or its copy, when not in place) receives dL/dlogits in
    the forward; backward scales it by the upstream gradient."""

    @staticmethod
    def forward(ctx, logits, target, ignore_index, reduction, inplace):
        N = logits.shape[0]
        ws = torch.empty(flce_ce_workspace_bytes(N), dtype=torch.uint8, device=logits.device)
        if ctx.needs_input_grad[0]:
            buf = logits if inplace else logits.detach().clone()
            val = flce_ce_fwd_bwd(buf, target, ignore_index, ws, reduction=reduction)
            ctx.save_for_backward(buf)
        else:
            val = flce_ce_fwd(logits, target, ignore_index, ws, reduction=reduction)
        return torch.tensor(val, dtype=torch.float32, device=logits.device)

    @staticmethod
    def backward(ctx, grad_out):
        _consume_once(ctx)
        (buf,) = ctx.saved_tensors
        g = grad_out.detach().to(torch.float32).reshape(1).contiguous()
        flce_scale_inplace(buf, g)
        return buf, None, None, None, None


def cross_entropy(logits: torch.Tensor, target: torch.Tensor, ignore_index: int = -100,
                  reduction: str = "mean", inplace: bool = True) -> torch.Tensor:
    """Cross-entropy of given logits [N, V] (bf16 or fp32) against target [N].

    reduction "mean" or "sum".  With inplace (the default, as the pages'
    in-place operations), a logits tensor that requires grad is overwritten
    with its own gradient during the forward, so it must not be used again."""
    if reduction not in ("mean", "sum"):
        raise ValueError("cross_entropy supports reduction 'mean' or 'sum'")
    return _CEFunction.apply(logits, target, ignore_index, reduction, inplace)


class _ORPOFunction(torch.autograd.Function):
    """Odds-ratio preference loss: the gradients are computed with the loss
    (one call) and scaled by the upstream gradient in backward."""

    @staticmethod
    def forward(ctx, weight, input, target, n_pairs, ignore_index, beta, chunk_pairs):
        N, H = input.shape
        V = weight.shape[0]
        T = N // (2 * n_pairs) if n_pairs > 0 else 0
        nbytes = flce_orpo_workspace_bytes(n_pairs, T, H, V, _dtype_code(input), chunk_pairs)
        if nbytes == 0:
            raise FLCEError(FLCE_EINVAL, "flce_orpo_workspace_bytes")
        ws = torch.empty(nbytes, dtype=torch.uint8, device=input.device)
        if ctx.needs_input_grad[0] or ctx.needs_input_grad[1]:
            dX = torch.empty_like(input)
            dW = torch.empty((V, H), dtype=torch.float32, device=input.device)
            val, _ = flce_orpo_fwd_bwd(input, weight, target, n_pairs, ignore_index, beta,
                                       chunk_pairs, dX, dW, ws)
            ctx.save_for_backward(dX, dW)
        else:
            val, _ = flce_orpo_fwd(input, weight, target, n_pairs, ignore_index, beta,
                                   chunk_pairs, ws)
        ctx.wdtype = weight.dtype
        return torch.tensor(val, dtype=torch.float32, device=input.device)

    @staticmethod
    def backward(ctx, grad_out):
        _consume_once(ctx)
        dX, dW = ctx.saved_tensors
        g = grad_out.detach().to(torch.float32).reshape(1).contiguous()
        flce_scale_inplace(dX, g)
        flce_scale_inplace(dW, g)
        gw = dW if ctx.wdtype == torch.float32 else dW.to(ctx.wdtype)
        return gw, dX, None, None, None, None, None


def orpo_loss(weight: torch.Tensor, input: torch.Tensor, target: torch.Tensor,
              ignore_index: int = -100, beta: float = 0.1, chunk_pairs: int = 0) -> torch.Tensor:
    """ORPO loss in the pages' call form orpo_loss(lm_head.weight, x, target).

    input [2B, T, H] (or [2B * T, H] with target [2B, T]): the B chosen
    sequences, then the B rejected ones; target [2B, T] with ignore_index on
    unscored tokens.  Returns NLL of the chosen tokens + beta * mean over pairs
    of -log sigmoid(log odds ratio)."""
    if target.dim() != 2 or target.shape[0] % 2 != 0:
        raise ValueError("target must be [2B, T] (chosen sequences first)")
    n_pairs = target.shape[0] // 2
    x = input.reshape(-1, input.shape[-1])
    if x.shape[0] != target.numel():
        raise ValueError(f"input has {x.shape[0]} rows, target {target.numel()} tokens")
    return _ORPOFunction.apply(weight, x, target.reshape(-1).contiguous(), n_pairs, ignore_index,
                               beta, chunk_pairs)


class FusedLinearORPOLoss(torch.nn.Module):
    """Module form: FusedLinearORPOLoss(beta)(lm_head.weight, x, target)."""

    def __init__(self, ignore_index: int = -100, beta: float = 0.1, chunk_pairs: int = 0):
        super().__init__()
        self.ignore_index, self.beta, self.chunk_pairs = ignore_index, beta, chunk_pairs

    def forward(self, weight, input, target):
        return orpo_loss(weight, input, target, self.ignore_index, self.beta, self.chunk_pairs)


class _PairFunction(torch.autograd.Function):
    """A pairwise preference loss: gradients computed with the loss (one
    call), scaled by the upstream gradient in backward."""

    @staticmethod
    def forward(ctx, weight, input, target, kind, n_pairs, ignore_index, beta, gamma, alpha,
                ref_c, ref_r, chunk_pairs):
        N, H = input.shape
        V = weight.shape[0]
        T = N // (2 * n_pairs) if n_pairs > 0 else 0
        nbytes = flce_pair_workspace_bytes(n_pairs, T, H, V, _dtype_code(input), chunk_pairs)
        if nbytes == 0:
            raise FLCEError(FLCE_EINVAL, "flce_pair_workspace_bytes")
        ws = torch.empty(nbytes, dtype=torch.uint8, device=input.device)
        if ctx.needs_input_grad[0] or ctx.needs_input_grad[1]:
            dX = torch.empty_like(input)
            dW = torch.empty((V, H), dtype=torch.float32, device=input.device)
            val, _ = flce_pair_fwd_bwd(kind, input, weight, target, n_pairs, ignore_index, beta,
                                       gamma, alpha, chunk_pairs, dX, dW, ws, ref_c, ref_r)
            ctx.save_for_backward(dX, dW)
        else:
            val, _ = flce_pair_fwd(kind, input, weight, target, n_pairs, ignore_index, beta,
                                   gamma, alpha, chunk_pairs, ws, ref_c, ref_r)
        ctx.wdtype = weight.dtype
        return torch.tensor(val, dtype=torch.float32, device=input.device)

    @staticmethod
    def backward(ctx, grad_out):
        _consume_once(ctx)
        dX, dW = ctx.saved_tensors
        g = grad_out.detach().to(torch.float32).reshape(1).contiguous()
        flce_scale_inplace(dX, g)
        flce_scale_inplace(dW, g)
        gw = dW if ctx.wdtype == torch.float32 else dW.to(ctx.wdtype)
        return gw, dX, None, None, None, None, None, None, None, None, None, None


def _pair_rows(input, target):
    if target.dim() != 2 or target.shape[0] % 2 != 0:
        raise ValueError("target must be [2B, T] (chosen sequences first)")
    x = input.reshape(-1, input.shape[-1])
    if x.shape[0] != target.numel():
        raise ValueError(f"input has {x.shape[0]} rows, target {target.numel()} tokens")
    return x, target.reshape(-1).contiguous(), target.shape[0] // 2


def preference_loss(kind: str, weight: torch.Tensor, input: torch.Tensor, target: torch.Tensor,
                    beta: float, gamma: float = 0.0, alpha: float = 0.0,
                    ref_chosen_logp: torch.Tensor | None = None,
                    ref_rejected_logp: torch.Tensor | None = None, ignore_index: int = -100,
                    chunk_pairs: int = 0) -> torch.Tensor:
    """A pairwise preference loss ("orpo", "simpo", "cpo", "dpo") of the B
    chosen sequences then the B rejected ones in input [2B, T, H] (or
    [2B * T, H]), target [2B, T]; see flce_pair_fwd_bwd in include/flce.h."""
    x, y, n_pairs = _pair_rows(input, target)
    if kind == "orpo":
        return _ORPOFunction.apply(weight, x, y, n_pairs, ignore_index, beta, chunk_pairs)
    return _PairFunction.apply(weight, x, y, kind, n_pairs, ignore_index, beta, gamma, alpha,
                               ref_chosen_logp, ref_rejected_logp, chunk_pairs)


@torch.no_grad()
def sequence_logps(weight: torch.Tensor, input: torch.Tensor, target: torch.Tensor,
                   ignore_index: int = -100, chunk_pairs: int = 0):
    """Sums of log p(y_t) over each chosen and each rejected sequence's scored
    tokens (forward only), e.g. a reference model's for DPO: (chosen [B],
    rejected [B]) fp32."""
    x, y, n_pairs = _pair_rows(input, target)
    N, H = x.shape
    nbytes = flce_pair_workspace_bytes(n_pairs, N // (2 * n_pairs), H, weight.shape[0],
                                       _dtype_code(x), chunk_pairs)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
    c = torch.empty(n_pairs, dtype=torch.float32, device=x.device)
    r = torch.empty(n_pairs, dtype=torch.float32, device=x.device)
    flce_pair_fwd("cpo", x.contiguous(), weight.contiguous(), y, n_pairs, ignore_index, 0.0, 0.0,
                  0.0, chunk_pairs, ws, chosen_logp=c, rejected_logp=r)
    return c, r


class FusedLinearSimPOLoss(torch.nn.Module):
    """SimPO: -log sigmoid(beta (a_c - a_r) - gamma) with a the mean token
    log-probability, plus alpha times the chosen NLL."""

    def __init__(self, beta: float = 2.0, gamma: float = 1.0, alpha: float = 0.0,
                 ignore_index: int = -100, chunk_pairs: int = 0):
        super().__init__()
        self.beta, self.gamma, self.alpha = beta, gamma, alpha
        self.ignore_index, self.chunk_pairs = ignore_index, chunk_pairs

    def forward(self, weight, input, target):
        return preference_loss("simpo", weight, input, target, self.beta, self.gamma, self.alpha,
                               ignore_index=self.ignore_index, chunk_pairs=self.chunk_pairs)


class FusedLinearCPOLoss(torch.nn.Module):
    """CPO: -log sigmoid(beta (S_c - S_r)) with S the summed token
    log-probability, plus alpha times the chosen NLL."""

    def __init__(self, beta: float = 0.1, alpha: float = 1.0, ignore_index: int = -100,
                 chunk_pairs: int = 0):
        super().__init__()
        self.beta, self.alpha = beta, alpha
        self.ignore_index, self.chunk_pairs = ignore_index, chunk_pairs

    def forward(self, weight, input, target):
        return preference_loss("cpo", weight, input, target, self.beta, 0.0, self.alpha,
                               ignore_index=self.ignore_index, chunk_pairs=self.chunk_pairs)


class FusedLinearDPOLoss(torch.nn.Module):
    """DPO: -log sigmoid(beta ((S_c - R_c) - (S_r - R_r))), R the reference
    model's summed log-probabilities: given directly, or computed (forward
    only) from ref_weight and ref_input (default: input)."""

    def __init__(self, beta: float = 0.1, alpha: float = 0.0, ignore_index: int = -100,
                 chunk_pairs: int = 0):
        super().__init__()
        self.beta, self.alpha = beta, alpha
        self.ignore_index, self.chunk_pairs = ignore_index, chunk_pairs

    def forward(self, weight, input, target, ref_weight=None, ref_input=None,
                ref_chosen_logp=None, ref_rejected_logp=None):
        if ref_chosen_logp is None or ref_rejected_logp is None:
            if ref_weight is None:
                raise ValueError("DPO needs ref_weight or the reference log-probabilities")
            ref_chosen_logp, ref_rejected_logp = sequence_logps(
                ref_weight.detach(), (input if ref_input is None else ref_input).detach(), target,
                self.ignore_index, self.chunk_pairs)
        return preference_loss("dpo", weight, input, target, self.beta, 0.0, self.alpha,
                               ref_chosen_logp, ref_rejected_logp, self.ignore_index,
                               self.chunk_pairs)


def _kto_ws(x, weight, n_seq, chunk_seqs):
    N, H = x.shape
    nbytes = flce_kto_workspace_bytes(n_seq, N // n_seq, H, weight.shape[0], _dtype_code(x),
                                      chunk_seqs)
    if nbytes == 0:
        raise FLCEError(FLCE_EINVAL, "flce_kto_workspace_bytes")
    return torch.empty(nbytes, dtype=torch.uint8, device=x.device)


class _KTOFunction(torch.autograd.Function):
    """KTO: gradients computed with the loss (one call), scaled by the
    upstream gradient in backward."""

    @staticmethod
    def forward(ctx, weight, input, target, n_seq, desirable, ref_logp, ignore_index, beta, z0,
                lambda_d, lambda_u, chunk_seqs):
        ws = _kto_ws(input, weight, n_seq, chunk_seqs)
        args = (input, weight, target, n_seq, ignore_index, desirable, ref_logp, beta, z0,
                lambda_d, lambda_u, chunk_seqs)
        if ctx.needs_input_grad[0] or ctx.needs_input_grad[1]:
            dX = torch.empty_like(input)
            dW = torch.empty(tuple(weight.shape), dtype=torch.float32, device=input.device)
            val = flce_kto_fwd_bwd(*args, dX, dW, ws)
            ctx.save_for_backward(dX, dW)
        else:
            val = flce_kto_fwd(*args, ws)
        ctx.wdtype = weight.dtype
        return torch.tensor(val, dtype=torch.float32, device=input.device)

    @staticmethod
    def backward(ctx, grad_out):
        _consume_once(ctx)
        dX, dW = ctx.saved_tensors
        g = grad_out.detach().to(torch.float32).reshape(1).contiguous()
        flce_scale_inplace(dX, g)
        flce_scale_inplace(dW, g)
        gw = dW if ctx.wdtype == torch.float32 else dW.to(ctx.wdtype)
        return (gw, dX) + (None,) * 10


def _kto_rows(input, target, desirable):
    if target.dim() != 2:
        raise ValueError("target must be [n_seq, T]")
    x = input.reshape(-1, input.shape[-1])
    if x.shape[0] != target.numel():
        raise ValueError(f"input has {x.shape[0]} rows, target {target.numel()} tokens")
    des = desirable.to(torch.int32).contiguous()
    return x, target.reshape(-1).contiguous(), target.shape[0], des


def kto_loss(weight: torch.Tensor, input: torch.Tensor, target: torch.Tensor,
             desirable: torch.Tensor, ref_logp: torch.Tensor, beta: float = 0.1, z0: float = 0.0,
             lambda_d: float = 1.0, lambda_u: float = 1.0, ignore_index: int = -100,
             chunk_seqs: int = 0) -> torch.Tensor:
    """KTO loss of input [n_seq, T, H] (or [n_seq * T, H]) against target
    [n_seq, T]; desirable [n_seq] (bool or int), ref_logp [n_seq] the
    reference model's summed log-probabilities, z0 the reference point."""
    x, y, n_seq, des = _kto_rows(input, target, desirable)
    return _KTOFunction.apply(weight, x, y, n_seq, des, ref_logp.float().contiguous(),
                              ignore_index, beta, z0, lambda_d, lambda_u, chunk_seqs)


@torch.no_grad()
def kto_reference_point(weight: torch.Tensor, input: torch.Tensor, target: torch.Tensor,
                        ref_logp: torch.Tensor, ignore_index: int = -100,
                        chunk_seqs: int = 0) -> float:
    """KTO's reference point from a batch of mismatched completions: input
    [n_seq, T, H] (or [n_seq * T, H]) holds the hidden states of n_seq
    completions each under a prompt that is not its own, target [n_seq, T]
    their tokens, ref_logp [n_seq] the reference model's summed
    log-probabilities of the same completions.  Returns z0 = max(0, mean of
    S - ref_logp) with S the policy's sums, computed on the device by
    flce_kto_reference_point, as a host float for kto_loss."""
    if target.dim() != 2:
        raise ValueError("target must be [n_seq, T]")
    if ref_logp.numel() != target.shape[0]:
        raise ValueError(f"ref_logp has {ref_logp.numel()} values for {target.shape[0]} sequences")
    x = input.reshape(-1, input.shape[-1]).contiguous()
    if x.shape[0] != target.numel():
        raise ValueError(f"input has {x.shape[0]} rows, target {target.numel()} tokens")
    n_seq = target.shape[0]
    w = weight.detach().contiguous()
    return flce_kto_reference_point(x.detach(), w, target.reshape(-1).contiguous(), n_seq,
                                    ignore_index, ref_logp.detach().reshape(-1).float().contiguous(),
                                    chunk_seqs, _kto_ws(x, w, n_seq, chunk_seqs))


class FusedLinearKTOLoss(torch.nn.Module):
    """Module form of kto_loss; the reference log-probabilities are given, or
    computed (forward only) from ref_weight and ref_input (default: input)."""

    def __init__(self, beta: float = 0.1, lambda_d: float = 1.0, lambda_u: float = 1.0,
                 ignore_index: int = -100, chunk_seqs: int = 0):
        super().__init__()
        self.beta, self.lambda_d, self.lambda_u = beta, lambda_d, lambda_u
        self.ignore_index, self.chunk_seqs = ignore_index, chunk_seqs

    def forward(self, weight, input, target, desirable, z0: float = 0.0, ref_logp=None,
                ref_weight=None, ref_input=None):
        if ref_logp is None:
            if ref_weight is None:
                raise ValueError("KTO needs ref_weight or the reference log-probabilities")
            with torch.no_grad():
                src = (input if ref_input is None else ref_input).detach()
                x, y, n_seq, des = _kto_rows(src, target, desirable)
                ref_logp = torch.empty(n_seq, dtype=torch.float32, device=x.device)
                zeros = torch.zeros(n_seq, dtype=torch.float32, device=x.device)
                flce_kto_fwd(x.contiguous(), ref_weight.detach().contiguous(), y, n_seq,
                             self.ignore_index, des, zeros, self.beta, 0.0, 1.0, 1.0,
                             self.chunk_seqs, _kto_ws(x, ref_weight, n_seq, self.chunk_seqs),
                             logp=ref_logp)
        return kto_loss(weight, input, target, desirable, ref_logp, self.beta, z0, self.lambda_d,
                        self.lambda_u, self.ignore_index, self.chunk_seqs)
