"""Python binding of libkla (ctypes).  Argument marshalling only: every step
of the scan runs in the HIP kernels of ``libkla.so``.

PyTorch supplies device memory and the current stream.  There is no CPU
fallback: without the built library every call raises.
"""

from __future__ import annotations

import ctypes
import os
import threading

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libkla.so")

KLA_OK = 0
KLA_DTYPE_F32 = 0
KLA_DTYPE_BF16 = 1
_DTYPES = {torch.float32: KLA_DTYPE_F32, torch.bfloat16: KLA_DTYPE_BF16}

_lock = threading.Lock()
_lib = None


class KlaError(RuntimeError):
    """A libkla call returned an error status."""

    def __init__(self, status: int, name: str, detail: str):
        super().__init__("%s: %s" % (name, detail))
        self.status = status
        self.name = name
        self.detail = detail


def library() -> ctypes.CDLL:
    """Loads libkla.so (built by ``python -m linear_attention_sequence_kla_amd.build``)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIBRARY):
            raise RuntimeError(
                "libkla.so is not built (%s); run __graft_entry__.build() or "
                "python -m linear_attention_sequence_kla_amd.build" % LIBRARY)
        lib = ctypes.CDLL(LIBRARY)
        vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
        lib.kla_scan_fwd_workspace_size.argtypes = [i64, i64, i64, i64, ctypes.c_int]
        lib.kla_scan_fwd_workspace_size.restype = sz
        lib.kla_scan_fwd.argtypes = [vp, vp, vp, vp, ctypes.c_int, vp, vp, vp, vp,
                                     i64, i64, i64, i64, vp, sz, vp]
        lib.kla_scan_fwd.restype = ctypes.c_int
        lib.kla_workspace_health.argtypes = [vp, ctypes.POINTER(ctypes.c_uint32), vp]
        lib.kla_workspace_health.restype = ctypes.c_int
        lib.kla_status_string.argtypes = [ctypes.c_int]
        lib.kla_status_string.restype = ctypes.c_char_p
        lib.kla_last_error_detail.argtypes = []
        lib.kla_last_error_detail.restype = ctypes.c_char_p
        _lib = lib
        return lib


def _check(status: int):
    if status != KLA_OK:
        lib = library()
        raise KlaError(status, lib.kla_status_string(status).decode(),
                       lib.kla_last_error_detail().decode())


def workspace_size(B: int, H: int, T: int, D: int, dtype=torch.float32) -> int:
    """Bytes of workspace kla_scan_fwd needs (0 for an empty problem)."""
    return int(library().kla_scan_fwd_workspace_size(B, H, T, D, _DTYPES[dtype]))


# Workspaces are zero-filled once and then reused: libkla leaves them ready
# for the next call.  One per (device, stream), so calls on different streams
# never share one.
_workspaces: dict = {}


def get_workspace(nbytes: int, device: torch.device, stream) -> torch.Tensor:
    key = (device.index, stream.cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def scan_fwd(a: torch.Tensor, p: torch.Tensor, phi: torch.Tensor, b: torch.Tensor,
             lam0: torch.Tensor | None = None, eta0: torch.Tensor | None = None,
             out: tuple | None = None, workspace: torch.Tensor | None = None):
    """Forward KLA scan on the current stream.

    a, p, phi, b: [B, H, T, D] contiguous tensors on one GPU, all float32 or
    all bfloat16.  lam0, eta0: [B, H, D] float32 (None: 1 and 0).
    Returns (lam, eta), float32 [B, H, T, D].  ``out`` may supply the two
    output tensors; ``workspace`` a zero-initialised uint8 tensor of at least
    ``workspace_size`` bytes that only this stream uses.
    """
    gates = (a, p, phi, b)
    if a.dim() != 4:
        raise ValueError("gates must be [B, H, T, D], got shape %s" % (tuple(a.shape),))
    for name, t in zip(("a", "p", "phi", "b"), gates):
        if t.shape != a.shape:
            raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(a.shape)))
        if t.dtype != a.dtype:
            raise ValueError("all gates must share one dtype (%s is %s)" % (name, t.dtype))
        if not t.is_cuda or t.device != a.device:
            raise ValueError("%s must be on the same GPU as a" % name)
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
    if a.dtype not in _DTYPES:
        raise ValueError("gate dtype must be float32 or bfloat16, got %s" % a.dtype)
    B, H, T, D = a.shape
    for name, t in (("lam0", lam0), ("eta0", eta0)):
        if t is not None:
            if t.shape != (B, H, D) or t.dtype != torch.float32 or t.device != a.device:
                raise ValueError("%s must be float32 [B, H, D] on a's device" % name)
            if not t.is_contiguous():
                raise ValueError("%s must be contiguous" % name)
    if out is None:
        lam = torch.empty(a.shape, dtype=torch.float32, device=a.device)
        eta = torch.empty(a.shape, dtype=torch.float32, device=a.device)
    else:
        lam, eta = out
        for t in (lam, eta):
            if (t.shape != a.shape or t.dtype != torch.float32 or t.device != a.device
                    or not t.is_contiguous()):
                raise ValueError("outputs must be contiguous float32 [B, H, T, D] on a's device")
    stream = torch.cuda.current_stream(a.device)
    nbytes = workspace_size(B, H, T, D, a.dtype)
    if workspace is None:
        workspace = get_workspace(nbytes, a.device, stream)
    _check(library().kla_scan_fwd(
        _ptr(a), _ptr(p), _ptr(phi), _ptr(b), _DTYPES[a.dtype], _ptr(lam0), _ptr(eta0),
        _ptr(lam), _ptr(eta), B, H, T, D, _ptr(workspace), workspace.numel(),
        ctypes.c_void_p(stream.cuda_stream)))
    return lam, eta


def workspace_health(workspace: torch.Tensor) -> int:
    """Reads and clears the workspace's health word (0: every call ran normally)."""
    out = ctypes.c_uint32(0)
    stream = torch.cuda.current_stream(workspace.device)
    _check(library().kla_workspace_health(_ptr(workspace), ctypes.byref(out),
                                          ctypes.c_void_p(stream.cuda_stream)))
    return int(out.value)
