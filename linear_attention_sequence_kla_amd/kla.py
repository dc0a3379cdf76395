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
KLA_ERR_HIP_HEALTH = 4  # reported with the status of a HIP error
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
        if _lib is None:
            _lib = load_library(LIBRARY)
        return _lib


def load_library(path: str) -> ctypes.CDLL:
    """Loads a build of libkla from `path` and declares its entry points."""
    if not os.path.exists(path):
        raise RuntimeError(
            "%s is not built; run __graft_entry__.build() or "
            "python -m linear_attention_sequence_kla_amd.build" % path)
    lib = ctypes.CDLL(path)
    vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    lib.kla_scan_fwd_workspace_size.argtypes = [i64, i64, i64, i64, ctypes.c_int]
    lib.kla_scan_fwd_workspace_size.restype = sz
    lib.kla_scan_fwd.argtypes = [vp, vp, vp, vp, ctypes.c_int, vp, vp, vp, vp,
                                 i64, i64, i64, i64, vp, sz, vp]
    lib.kla_scan_fwd.restype = ctypes.c_int
    lib.kla_scan_fwd_noalloc.argtypes = [vp, vp, vp, vp, ctypes.c_int, vp, vp, vp, vp,
                                         i64, i64, i64, i64, vp]
    lib.kla_scan_fwd_noalloc.restype = ctypes.c_int
    lib.kla_scan_fwd_noalloc_max_workspace.argtypes = []
    lib.kla_scan_fwd_noalloc_max_workspace.restype = sz
    lib.kla_scan_states_size.argtypes = [i64, i64, i64, i64]
    lib.kla_scan_states_size.restype = sz
    lib.kla_scan_fwd_states.argtypes = [vp, vp, vp, vp, ctypes.c_int, vp, vp, vp, vp, vp,
                                        i64, i64, i64, i64, vp, sz, vp]
    lib.kla_scan_fwd_states.restype = ctypes.c_int
    lib.kla_scan_bwd_states_workspace_size.argtypes = [i64, i64, i64, i64, ctypes.c_int]
    lib.kla_scan_bwd_states_workspace_size.restype = sz
    lib.kla_scan_bwd_states.argtypes = [vp, vp, vp, vp, ctypes.c_int] + [vp] * 11 + [i64] * 4 + [
        vp, sz, vp]
    lib.kla_scan_bwd_states.restype = ctypes.c_int
    lib.kla_scan_bwd_workspace_size.argtypes = [i64, i64, i64, i64, ctypes.c_int]
    lib.kla_scan_bwd_workspace_size.restype = sz
    lib.kla_scan_bwd.argtypes = [vp, vp, ctypes.c_int] + [vp] * 12 + [i64] * 4 + [vp, sz, vp]
    lib.kla_scan_bwd.restype = ctypes.c_int
    lib.kla_mixer_fwd_workspace_size.argtypes = [i64, i64, i64, i64, ctypes.c_int]
    lib.kla_mixer_fwd_workspace_size.restype = sz
    lib.kla_mixer_fwd.argtypes = [vp, vp, vp, vp, ctypes.c_int] + [vp] * 9 + [i64] * 4 + [
        vp, sz, vp]
    lib.kla_mixer_fwd.restype = ctypes.c_int
    lib.kla_mixer_states_size.argtypes = [i64, i64, i64, i64]
    lib.kla_mixer_states_size.restype = sz
    lib.kla_scan_lti_fwd_workspace_size.argtypes = [i64, i64, i64, i64, ctypes.c_int]
    lib.kla_scan_lti_fwd_workspace_size.restype = sz
    lib.kla_scan_lti_fwd.argtypes = [vp, vp, vp, vp, ctypes.c_int, vp, vp, vp, vp,
                                     i64, i64, i64, i64, vp, sz, vp]
    lib.kla_scan_lti_fwd.restype = ctypes.c_int
    lib.kla_mixer_bwd_workspace_size.argtypes = [i64, i64, i64, i64, ctypes.c_int]
    lib.kla_mixer_bwd_workspace_size.restype = sz
    lib.kla_mixer_bwd.argtypes = [vp, vp, vp, vp, ctypes.c_int] + [vp] * 15 + [i64] * 4 + [
        vp, sz, vp]
    lib.kla_mixer_bwd.restype = ctypes.c_int
    lib.kla_decode_step.argtypes = [vp, vp, vp, vp, ctypes.c_int, vp, vp, i64, vp]
    lib.kla_decode_step.restype = ctypes.c_int
    lib.kla_mixer_decode_step.argtypes = [vp, vp, vp, vp, ctypes.c_int] + [vp] * 6 + [
        i64, i64, vp]
    lib.kla_mixer_decode_step.restype = ctypes.c_int
    lib.kla_workspace_health.argtypes = [vp, ctypes.POINTER(ctypes.c_uint32), vp]
    lib.kla_workspace_health.restype = ctypes.c_int
    lib.kla_status_string.argtypes = [ctypes.c_int]
    lib.kla_status_string.restype = ctypes.c_char_p
    lib.kla_last_error_detail.argtypes = []
    lib.kla_last_error_detail.restype = ctypes.c_char_p
    return lib


def _check(status: int):
    if status != KLA_OK:
        lib = library()
        raise KlaError(status, lib.kla_status_string(status).decode(),
                       lib.kla_last_error_detail().decode())


class KlaHealthError(KlaError):
    """A kernel gave up waiting for a predecessor's carry (its outputs are
    wrong); raised only when health checks are on."""


# Health checks: off by default.  When on, every call that uses a workspace
# is followed by kla_workspace_health on it, which synchronizes the stream
# and copies 4 bytes to the host (a few microseconds plus the wait for the
# call to finish, so launches no longer overlap the host); a nonzero word
# raises KlaHealthError.  A give-up needs a predecessor tile that never
# publishes its carry for about 2^20 polls, which only a fault elsewhere
# causes; the kernels still terminate and the word records it either way.
_health_checks = os.environ.get("KLA_CHECK_HEALTH", "0") not in ("", "0")


def set_health_checks(enabled: bool) -> bool:
    """Turns the per-call health check on or off; returns the previous
    setting.  The environment variable KLA_CHECK_HEALTH=1 turns it on at
    import."""
    global _health_checks
    prev = _health_checks
    _health_checks = bool(enabled)
    return prev


def health_checks_enabled() -> bool:
    return _health_checks


def _after_call(name: str, workspace: torch.Tensor):
    """With health checks on: reads and clears the workspace's health word
    after the call and raises if a wait gave up."""
    if not _health_checks:
        return
    word = workspace_health(workspace)
    if word != 0:
        raise KlaHealthError(KLA_ERR_HIP_HEALTH, name,
                             "a chunk gave up waiting for its predecessor's carry "
                             "(health word 0x%x); the outputs of this call are wrong" % word)


def workspace_size(B: int, H: int, T: int, D: int, dtype=torch.float32) -> int:
    """Bytes of workspace kla_scan_fwd needs (0 for an empty problem)."""
    return int(library().kla_scan_fwd_workspace_size(B, H, T, D, _DTYPES[dtype]))


def bwd_workspace_size(B: int, H: int, T: int, D: int, dtype=torch.float32) -> int:
    """Bytes of workspace kla_scan_bwd needs (0 for an empty problem)."""
    return int(library().kla_scan_bwd_workspace_size(B, H, T, D, _DTYPES[dtype]))


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
    if workspace is None:
        workspace = get_workspace(workspace_size(B, H, T, D, a.dtype), a.device, stream)
    _check(library().kla_scan_fwd(
        _ptr(a), _ptr(p), _ptr(phi), _ptr(b), _DTYPES[a.dtype], _ptr(lam0), _ptr(eta0),
        _ptr(lam), _ptr(eta), B, H, T, D, _ptr(workspace), workspace.numel(),
        ctypes.c_void_p(stream.cuda_stream)))
    _after_call("kla_scan_fwd", workspace)
    return lam, eta


def scan_fwd_noalloc(a: torch.Tensor, p: torch.Tensor, phi: torch.Tensor, b: torch.Tensor,
                     lam0: torch.Tensor | None = None, eta0: torch.Tensor | None = None,
                     out: tuple | None = None):
    """kla_scan_fwd_noalloc on the current stream: the forward scan with the
    library's own per-GPU workspace (no workspace argument; calls that overlap
    on one GPU race).  Arguments and results as for ``scan_fwd``; with ``out``
    given nothing is allocated at all."""
    if a.dim() != 4:
        raise ValueError("gates must be [B, H, T, D], got shape %s" % (tuple(a.shape),))
    for name, t in zip(("a", "p", "phi", "b"), (a, p, phi, b)):
        if t.shape != a.shape or t.dtype != a.dtype:
            raise ValueError("%s must match a in shape and dtype" % name)
        if not t.is_cuda or t.device != a.device or not t.is_contiguous():
            raise ValueError("%s must be contiguous on a's GPU" % name)
    if a.dtype not in _DTYPES:
        raise ValueError("gate dtype must be float32 or bfloat16, got %s" % a.dtype)
    B, H, T, D = a.shape
    for name, t in (("lam0", lam0), ("eta0", eta0)):
        _check_f32(name, t, (B, H, D), a.device)
    if out is None:
        out = (torch.empty(a.shape, dtype=torch.float32, device=a.device),
               torch.empty(a.shape, dtype=torch.float32, device=a.device))
    lam, eta = out
    for name, t in (("lam", lam), ("eta", eta)):
        if t is None:
            raise ValueError("%s output is required" % name)
        _check_f32(name, t, a.shape, a.device)
    stream = torch.cuda.current_stream(a.device)
    _check(library().kla_scan_fwd_noalloc(
        _ptr(a), _ptr(p), _ptr(phi), _ptr(b), _DTYPES[a.dtype], _ptr(lam0), _ptr(eta0),
        _ptr(lam), _ptr(eta), B, H, T, D, ctypes.c_void_p(stream.cuda_stream)))
    return lam, eta


def _check_gates(a, p, phi, b):
    if a.dim() != 4:
        raise ValueError("gates must be [B, H, T, D], got shape %s" % (tuple(a.shape),))
    for name, t in zip(("a", "p", "phi", "b"), (a, p, phi, b)):
        if t is None:
            raise ValueError("%s is required" % name)
        if t.shape != a.shape or t.dtype != a.dtype:
            raise ValueError("%s must match a in shape and dtype" % name)
        if not t.is_cuda or t.device != a.device or not t.is_contiguous():
            raise ValueError("%s must be contiguous on a's GPU" % name)
    if a.dtype not in _DTYPES:
        raise ValueError("gate dtype must be float32 or bfloat16, got %s" % a.dtype)


def _check_f32(name, t, shape, device):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or t.dtype != torch.float32 or t.device != device:
        raise ValueError("%s must be float32 %s on %s" % (name, tuple(shape), device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def scan_bwd(a: torch.Tensor, p: torch.Tensor, lam: torch.Tensor, eta: torch.Tensor,
             g_lam: torch.Tensor | None, g_eta: torch.Tensor | None,
             lam0: torch.Tensor | None = None, eta0: torch.Tensor | None = None,
             need_state_grads: bool = True, workspace: torch.Tensor | None = None,
             out: tuple | None = None):
    """Backward KLA scan on the current stream (kla_scan_bwd).

    a, p: the forward gates; lam, eta: the forward outputs; g_lam, g_eta:
    upstream gradients (None: zero); lam0, eta0: the forward initial state.
    Returns (g_a, g_p, g_phi, g_b, g_lam0, g_eta0), float32; the last two are
    None unless need_state_grads.  ``out`` may supply the four [B, H, T, D]
    gate-gradient tensors.
    """
    if a.dim() != 4 or p.shape != a.shape or p.dtype != a.dtype:
        raise ValueError("a and p must be [B, H, T, D] tensors of one dtype")
    if a.dtype not in _DTYPES:
        raise ValueError("gate dtype must be float32 or bfloat16, got %s" % a.dtype)
    for name, t in (("a", a), ("p", p)):
        if not t.is_cuda or t.device != a.device or not t.is_contiguous():
            raise ValueError("%s must be contiguous on a's GPU" % name)
    B, H, T, D = a.shape
    dev = a.device
    for name, t in (("lam", lam), ("eta", eta), ("g_lam", g_lam), ("g_eta", g_eta)):
        _check_f32(name, t, a.shape, dev)
    if lam is None or eta is None:
        raise ValueError("the forward outputs lam and eta are required")
    for name, t in (("lam0", lam0), ("eta0", eta0)):
        _check_f32(name, t, (B, H, D), dev)
    if out is None:
        g_a, g_p, g_phi, g_b = (torch.empty(a.shape, dtype=torch.float32, device=dev)
                                for _ in range(4))
    else:
        g_a, g_p, g_phi, g_b = out
        for name, t in zip(("g_a", "g_p", "g_phi", "g_b"), out):
            if t is None:
                raise ValueError("%s output is required" % name)
            _check_f32(name, t, a.shape, dev)
    g_lam0 = g_eta0 = None
    if need_state_grads:
        g_lam0 = torch.empty((B, H, D), dtype=torch.float32, device=dev)
        g_eta0 = torch.empty((B, H, D), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    if workspace is None:
        workspace = get_workspace(max(bwd_workspace_size(B, H, T, D, a.dtype),
                                      workspace_size(B, H, T, D, a.dtype)), dev, stream)
    _check(library().kla_scan_bwd(
        _ptr(a), _ptr(p), _DTYPES[a.dtype], _ptr(lam0), _ptr(eta0), _ptr(lam), _ptr(eta),
        _ptr(g_lam), _ptr(g_eta), _ptr(g_a), _ptr(g_p), _ptr(g_phi), _ptr(g_b),
        _ptr(g_lam0), _ptr(g_eta0), B, H, T, D, _ptr(workspace), workspace.numel(),
        ctypes.c_void_p(stream.cuda_stream)))
    _after_call("kla_scan_bwd", workspace)
    return g_a, g_p, g_phi, g_b, g_lam0, g_eta0


def scan_states_shape(B: int, H: int, T: int, D: int) -> tuple:
    """Shape of the float64 tensor of scan states (kla_scan_fwd_states'
    `states`): the (lam, eta) of every channel after every 8th token."""
    C = B * H * D
    n = int(library().kla_scan_states_size(B, H, T, D))
    return (n // (16 * C) if C else 0, C, 2)


def _check_scan_states(states, shape4, dev):
    if states is None:
        return
    want = scan_states_shape(*shape4)
    if (tuple(states.shape) != want or states.dtype != torch.float64 or not states.is_cuda
            or states.device != dev or not states.is_contiguous()):
        raise ValueError("states must be a contiguous float64 %s tensor on %s" % (want, dev))


def scan_fwd_states(a: torch.Tensor, p: torch.Tensor, phi: torch.Tensor, b: torch.Tensor,
                    lam0: torch.Tensor | None = None, eta0: torch.Tensor | None = None,
                    states: torch.Tensor | None = None, out: tuple | None = None,
                    workspace: torch.Tensor | None = None):
    """kla_scan_fwd_states: the forward scan that also keeps the float64 state
    after every 8th token for ``scan_bwd_states``.  Arguments as for
    ``scan_fwd``; ``states`` (float64, ``scan_states_shape``) is allocated
    when None.  Returns (lam, eta, states)."""
    _check_gates(a, p, phi, b)
    B, H, T, D = a.shape
    for name, t in (("lam0", lam0), ("eta0", eta0)):
        _check_f32(name, t, (B, H, D), a.device)
    if out is None:
        out = (torch.empty(a.shape, dtype=torch.float32, device=a.device),
               torch.empty(a.shape, dtype=torch.float32, device=a.device))
    lam, eta = out
    for name, t in (("lam", lam), ("eta", eta)):
        if t is None:
            raise ValueError("%s output is required" % name)
        _check_f32(name, t, a.shape, a.device)
    if states is None:
        states = torch.empty(scan_states_shape(B, H, T, D), dtype=torch.float64,
                             device=a.device)
    _check_scan_states(states, (B, H, T, D), a.device)
    stream = torch.cuda.current_stream(a.device)
    if workspace is None:
        workspace = get_workspace(workspace_size(B, H, T, D, a.dtype), a.device, stream)
    _check(library().kla_scan_fwd_states(
        _ptr(a), _ptr(p), _ptr(phi), _ptr(b), _DTYPES[a.dtype], _ptr(lam0), _ptr(eta0),
        _ptr(lam), _ptr(eta), _ptr(states), B, H, T, D, _ptr(workspace), workspace.numel(),
        ctypes.c_void_p(stream.cuda_stream)))
    _after_call("kla_scan_fwd_states", workspace)
    return lam, eta, states


def bwd_states_workspace_size(B: int, H: int, T: int, D: int, dtype=torch.float32) -> int:
    """Bytes of workspace kla_scan_bwd_states needs (0 for an empty problem)."""
    return int(library().kla_scan_bwd_states_workspace_size(B, H, T, D, _DTYPES[dtype]))


def scan_bwd_states(a: torch.Tensor, p: torch.Tensor, phi: torch.Tensor, b: torch.Tensor,
                    g_lam: torch.Tensor | None, g_eta: torch.Tensor | None,
                    lam0: torch.Tensor | None = None, eta0: torch.Tensor | None = None,
                    states: torch.Tensor | None = None, need_state_grads: bool = True,
                    workspace: torch.Tensor | None = None, out: tuple | None = None):
    """kla_scan_bwd_states: the backward scan from float64 states (exact also
    where the forward outputs overflow float32).  ``states``: what
    ``scan_fwd_states`` kept for these inputs, or None (recomputed).  Returns
    (g_a, g_p, g_phi, g_b, g_lam0, g_eta0) as ``scan_bwd``."""
    _check_gates(a, p, phi, b)
    B, H, T, D = a.shape
    dev = a.device
    for name, t in (("g_lam", g_lam), ("g_eta", g_eta)):
        _check_f32(name, t, a.shape, dev)
    for name, t in (("lam0", lam0), ("eta0", eta0)):
        _check_f32(name, t, (B, H, D), dev)
    _check_scan_states(states, (B, H, T, D), dev)
    if out is None:
        out = tuple(torch.empty(a.shape, dtype=torch.float32, device=dev) for _ in range(4))
    for name, t in zip(("g_a", "g_p", "g_phi", "g_b"), out):
        if t is None:
            raise ValueError("%s output is required" % name)
        _check_f32(name, t, a.shape, dev)
    g_a, g_p, g_phi, g_b = out
    g_lam0 = g_eta0 = None
    if need_state_grads:
        g_lam0 = torch.empty((B, H, D), dtype=torch.float32, device=dev)
        g_eta0 = torch.empty((B, H, D), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    if workspace is None:
        workspace = get_workspace(max(bwd_states_workspace_size(B, H, T, D, a.dtype),
                                      workspace_size(B, H, T, D, a.dtype)), dev, stream)
    _check(library().kla_scan_bwd_states(
        _ptr(a), _ptr(p), _ptr(phi), _ptr(b), _DTYPES[a.dtype], _ptr(lam0), _ptr(eta0),
        _ptr(states), _ptr(g_lam), _ptr(g_eta), _ptr(g_a), _ptr(g_p), _ptr(g_phi), _ptr(g_b),
        _ptr(g_lam0), _ptr(g_eta0), B, H, T, D, _ptr(workspace), workspace.numel(),
        ctypes.c_void_p(stream.cuda_stream)))
    _after_call("kla_scan_bwd_states", workspace)
    return g_a, g_p, g_phi, g_b, g_lam0, g_eta0


class KLAScan(torch.autograd.Function):
    """Differentiable forward scan: kla_scan_fwd_states forward, which also
    keeps the float64 state after every 8th token (about 2 bytes per
    element), and kla_scan_bwd_states backward from those states (defined on
    the whole domain, also where lam or eta overflow float32).

    Gradients are float32 and are cast to each input's dtype.
    """

    @staticmethod
    def forward(ctx, a, p, phi, b, lam0, eta0):
        if any(ctx.needs_input_grad):
            lam, eta, states = scan_fwd_states(a, p, phi, b, lam0, eta0)
        else:
            (lam, eta), states = scan_fwd(a, p, phi, b, lam0, eta0), None
        ctx.save_for_backward(a, p, phi, b, lam0, eta0, states)
        return lam, eta

    @staticmethod
    def backward(ctx, g_lam, g_eta):
        a, p, phi, b, lam0, eta0, states = ctx.saved_tensors
        g_lam = None if g_lam is None else g_lam.contiguous().float()
        g_eta = None if g_eta is None else g_eta.contiguous().float()
        need = ctx.needs_input_grad
        g_a, g_p, g_phi, g_b, g_lam0, g_eta0 = scan_bwd_states(
            a, p, phi, b, g_lam, g_eta, lam0, eta0, states=states,
            need_state_grads=need[4] or need[5])
        cast = (lambda g, x: g.to(x.dtype))  # noqa: E731
        return (cast(g_a, a), cast(g_p, p), cast(g_phi, phi), cast(g_b, b),
                g_lam0 if need[4] else None, g_eta0 if need[5] else None)


def kla_scan(a, p, phi, b, lam0=None, eta0=None):
    """Differentiable KLA scan: returns (lam, eta); see KLAScan."""
    return KLAScan.apply(a, p, phi, b, lam0, eta0)


def lti_workspace_size(B: int, H: int, T: int, D: int, dtype=torch.float32) -> int:
    """Bytes of workspace kla_scan_lti_fwd needs (0 for an empty problem)."""
    return int(library().kla_scan_lti_fwd_workspace_size(B, H, T, D, _DTYPES[dtype]))


def scan_lti_fwd(a: torch.Tensor, p: torch.Tensor, phi: torch.Tensor, b: torch.Tensor,
                 lam0: torch.Tensor | None = None, eta0: torch.Tensor | None = None,
                 out: tuple | None = None, workspace: torch.Tensor | None = None):
    """Forward KLA scan with time-invariant gates (kla_scan_lti_fwd).

    a, p, phi: [H, D] float32; b: [B, H, T, D] contiguous float32 or
    bfloat16; lam0, eta0: [B, H, D] float32 (None: 1 and 0).  Returns
    (lam, eta), float32 [B, H, T, D].
    """
    if b.dim() != 4:
        raise ValueError("b must be [B, H, T, D], got shape %s" % (tuple(b.shape),))
    if b.dtype not in _DTYPES:
        raise ValueError("b must be float32 or bfloat16, got %s" % b.dtype)
    if not b.is_cuda or not b.is_contiguous():
        raise ValueError("b must be a contiguous GPU tensor")
    B, H, T, D = b.shape
    dev = b.device
    for name, t in (("a", a), ("p", p), ("phi", phi)):
        if t is None:
            raise ValueError("%s is required" % name)
        _check_f32(name, t, (H, D), dev)
    for name, t in (("lam0", lam0), ("eta0", eta0)):
        _check_f32(name, t, (B, H, D), dev)
    if out is None:
        lam = torch.empty(b.shape, dtype=torch.float32, device=dev)
        eta = torch.empty(b.shape, dtype=torch.float32, device=dev)
    else:
        lam, eta = out
        for name, t in (("lam", lam), ("eta", eta)):
            if t is None:
                raise ValueError("%s output is required" % name)
            _check_f32(name, t, b.shape, dev)
    stream = torch.cuda.current_stream(dev)
    if workspace is None:
        workspace = get_workspace(lti_workspace_size(B, H, T, D, b.dtype), dev, stream)
    _check(library().kla_scan_lti_fwd(
        _ptr(a), _ptr(p), _ptr(phi), _ptr(b), _DTYPES[b.dtype], _ptr(lam0), _ptr(eta0),
        _ptr(lam), _ptr(eta), B, H, T, D, _ptr(workspace), workspace.numel(),
        ctypes.c_void_p(stream.cuda_stream)))
    _after_call("kla_scan_lti_fwd", workspace)
    return lam, eta


def mixer_workspace_size(B: int, H: int, T: int, D: int, dtype=torch.float32) -> int:
    """Bytes of workspace kla_mixer_fwd needs (0 for an empty problem)."""
    return int(library().kla_mixer_fwd_workspace_size(B, H, T, D, _DTYPES[dtype]))


def mixer_fwd(k: torch.Tensor, v: torch.Tensor, lam_v: torch.Tensor, q: torch.Tensor,
              a: torch.Tensor, p: torch.Tensor, lam0: torch.Tensor | None = None,
              eta0: torch.Tensor | None = None, want_var: bool = True,
              want_state: bool = False, out: torch.Tensor | None = None,
              var: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
              states: torch.Tensor | None = None):
    """Fused KLA mixer forward on the current stream (kla_mixer_fwd).

    k, v, lam_v, q: [B, H, T, D] contiguous, all float32 or all bfloat16 (the
    observation operator, the value, its precision and the readout operator).
    a, p: [H, D] float32 state decay and process noise.  lam0, eta0: [B, H, D]
    float32 (None: 1 and 0).  Returns (out, var, lam_T, eta_T): the readout
    q * eta / lam, the posterior variance 1 / lam (None unless want_var) and
    the final state (None unless want_state), float32.  ``states``, a float64
    tensor of ``mixer_states_shape(B, H, T, D)`` on k's GPU, receives the
    state after every 8th token for ``mixer_bwd``.
    """
    ins = (k, v, lam_v, q)
    if k.dim() != 4:
        raise ValueError("token inputs must be [B, H, T, D], got shape %s" % (tuple(k.shape),))
    for name, t in zip(("k", "v", "lam_v", "q"), ins):
        if t.shape != k.shape or t.dtype != k.dtype:
            raise ValueError("%s must match k in shape and dtype" % name)
        if not t.is_cuda or t.device != k.device or not t.is_contiguous():
            raise ValueError("%s must be contiguous on k's GPU" % name)
    if k.dtype not in _DTYPES:
        raise ValueError("token dtype must be float32 or bfloat16, got %s" % k.dtype)
    B, H, T, D = k.shape
    dev = k.device
    for name, t in (("a", a), ("p", p)):
        if t is None:
            raise ValueError("%s is required" % name)
        _check_f32(name, t, (H, D), dev)
    for name, t in (("lam0", lam0), ("eta0", eta0)):
        _check_f32(name, t, (B, H, D), dev)
    if out is None:
        out = torch.empty(k.shape, dtype=torch.float32, device=dev)
    _check_f32("out", out, k.shape, dev)
    if want_var and var is None:
        var = torch.empty(k.shape, dtype=torch.float32, device=dev)
    if not want_var:
        var = None
    _check_f32("var", var, k.shape, dev)
    lam_T = eta_T = None
    if want_state:
        lam_T = torch.empty((B, H, D), dtype=torch.float32, device=dev)
        eta_T = torch.empty((B, H, D), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    _check_states(states, (B, H, T, D), dev)
    if workspace is None:
        workspace = get_workspace(mixer_workspace_size(B, H, T, D, k.dtype), dev, stream)
    _check(library().kla_mixer_fwd(
        _ptr(k), _ptr(v), _ptr(lam_v), _ptr(q), _DTYPES[k.dtype], _ptr(a), _ptr(p), _ptr(lam0),
        _ptr(eta0), _ptr(out), _ptr(var), _ptr(lam_T), _ptr(eta_T), _ptr(states), B, H, T, D,
        _ptr(workspace), workspace.numel(), ctypes.c_void_p(stream.cuda_stream)))
    _after_call("kla_mixer_fwd", workspace)
    return out, var, lam_T, eta_T


def mixer_states_shape(B: int, H: int, T: int, D: int) -> tuple:
    """Shape of the float64 tensor of mixer states (kla_mixer_fwd's `states`):
    the (lam, eta) of every channel after every 8th token."""
    C = B * H * D
    n = int(library().kla_mixer_states_size(B, H, T, D))
    return (n // (16 * C) if C else 0, C, 2)


def _check_states(states, shape4, dev):
    if states is None:
        return
    want = mixer_states_shape(*shape4)
    if (tuple(states.shape) != want or states.dtype != torch.float64 or not states.is_cuda
            or states.device != dev or not states.is_contiguous()):
        raise ValueError("states must be a contiguous float64 %s tensor on %s" % (want, dev))


def mixer_bwd_workspace_size(B: int, H: int, T: int, D: int, dtype=torch.float32) -> int:
    """Bytes of workspace kla_mixer_bwd needs (0 for an empty problem)."""
    return int(library().kla_mixer_bwd_workspace_size(B, H, T, D, _DTYPES[dtype]))


def mixer_bwd(k: torch.Tensor, v: torch.Tensor, lam_v: torch.Tensor, q: torch.Tensor,
              a: torch.Tensor, p: torch.Tensor, g_out: torch.Tensor,
              g_var: torch.Tensor | None = None, lam0: torch.Tensor | None = None,
              eta0: torch.Tensor | None = None, need_state_grads: bool = True,
              workspace: torch.Tensor | None = None, out: tuple | None = None,
              states: torch.Tensor | None = None):
    """Fused KLA mixer backward on the current stream (kla_mixer_bwd).

    Inputs as for ``mixer_fwd``; g_out, g_var: float32 [B, H, T, D] upstream
    gradients of the readout and the variance (g_var None: zero).  Returns
    (g_k, g_v, g_lam_v, g_q, g_a, g_p, g_lam0, g_eta0), float32; the last two
    are None unless need_state_grads.  ``out`` may supply the first six.
    ``states``: the tensor ``mixer_fwd`` filled for these inputs (the forward
    states are then not recomputed), or None.
    """
    if k.dim() != 4:
        raise ValueError("token inputs must be [B, H, T, D], got shape %s" % (tuple(k.shape),))
    for name, t in zip(("k", "v", "lam_v", "q"), (k, v, lam_v, q)):
        if t.shape != k.shape or t.dtype != k.dtype:
            raise ValueError("%s must match k in shape and dtype" % name)
        if not t.is_cuda or t.device != k.device or not t.is_contiguous():
            raise ValueError("%s must be contiguous on k's GPU" % name)
    if k.dtype not in _DTYPES:
        raise ValueError("token dtype must be float32 or bfloat16, got %s" % k.dtype)
    B, H, T, D = k.shape
    dev = k.device
    for name, t in (("a", a), ("p", p)):
        if t is None:
            raise ValueError("%s is required" % name)
        _check_f32(name, t, (H, D), dev)
    if g_out is None:
        raise ValueError("g_out is required")
    for name, t in (("g_out", g_out), ("g_var", g_var)):
        _check_f32(name, t, k.shape, dev)
    for name, t in (("lam0", lam0), ("eta0", eta0)):
        _check_f32(name, t, (B, H, D), dev)
    if out is None:
        g_k, g_v, g_lam_v, g_q = (torch.empty(k.shape, dtype=torch.float32, device=dev)
                                  for _ in range(4))
        g_a = torch.empty((H, D), dtype=torch.float32, device=dev)
        g_p = torch.empty((H, D), dtype=torch.float32, device=dev)
    else:
        g_k, g_v, g_lam_v, g_q, g_a, g_p = out
        for name, t, sh in (("g_k", g_k, k.shape), ("g_v", g_v, k.shape),
                            ("g_lam_v", g_lam_v, k.shape), ("g_q", g_q, k.shape),
                            ("g_a", g_a, (H, D)), ("g_p", g_p, (H, D))):
            if t is None:
                raise ValueError("%s output is required" % name)
            _check_f32(name, t, sh, dev)
    g_lam0 = g_eta0 = None
    if need_state_grads:
        g_lam0 = torch.empty((B, H, D), dtype=torch.float32, device=dev)
        g_eta0 = torch.empty((B, H, D), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    _check_states(states, (B, H, T, D), dev)
    if workspace is None:
        workspace = get_workspace(mixer_bwd_workspace_size(B, H, T, D, k.dtype), dev, stream)
    _check(library().kla_mixer_bwd(
        _ptr(k), _ptr(v), _ptr(lam_v), _ptr(q), _DTYPES[k.dtype], _ptr(a), _ptr(p), _ptr(lam0),
        _ptr(eta0), _ptr(states), _ptr(g_out), _ptr(g_var), _ptr(g_k), _ptr(g_v), _ptr(g_lam_v), _ptr(g_q),
        _ptr(g_a), _ptr(g_p), _ptr(g_lam0), _ptr(g_eta0), B, H, T, D, _ptr(workspace),
        workspace.numel(), ctypes.c_void_p(stream.cuda_stream)))
    _after_call("kla_mixer_bwd", workspace)
    return g_k, g_v, g_lam_v, g_q, g_a, g_p, g_lam0, g_eta0


class KLAMixer(torch.autograd.Function):
    """Differentiable fused mixer: kla_mixer_fwd forward, which also keeps the
    float64 state after every 8th token (about 2 bytes per element), and
    kla_mixer_bwd backward from those states.  Returns (out, var).  Gradients
    are float32 and are cast to each input's dtype."""

    @staticmethod
    def forward(ctx, k, v, lam_v, q, a, p, lam0, eta0):
        states = None
        if any(ctx.needs_input_grad):
            states = torch.empty(mixer_states_shape(*k.shape), dtype=torch.float64,
                                 device=k.device)
        out, var, _, _ = mixer_fwd(k, v, lam_v, q, a, p, lam0, eta0, states=states)
        ctx.save_for_backward(k, v, lam_v, q, a, p, lam0, eta0, states)
        return out, var

    @staticmethod
    def backward(ctx, g_out, g_var):
        k, v, lam_v, q, a, p, lam0, eta0, states = ctx.saved_tensors
        need = ctx.needs_input_grad
        if g_out is None:
            g_out = torch.zeros(k.shape, dtype=torch.float32, device=k.device)
        g = mixer_bwd(k, v, lam_v, q, a, p, g_out.contiguous().float(),
                      None if g_var is None else g_var.contiguous().float(), lam0, eta0,
                      need_state_grads=need[6] or need[7], states=states)
        cast = (lambda t, x: t.to(x.dtype))  # noqa: E731
        return (cast(g[0], k), cast(g[1], v), cast(g[2], lam_v), cast(g[3], q), g[4], g[5],
                g[6] if need[6] else None, g[7] if need[7] else None)


def kla_mixer(k, v, lam_v, q, a, p, lam0=None, eta0=None):
    """Differentiable fused KLA mixer: returns (out, var); see KLAMixer."""
    return KLAMixer.apply(k, v, lam_v, q, a, p, lam0, eta0)


def decode_step(a: torch.Tensor, p: torch.Tensor, phi: torch.Tensor, b: torch.Tensor,
                lam: torch.Tensor, eta: torch.Tensor):
    """One-token update of the running state (lam, eta), in place, on the
    current stream (kla_decode_step).  Gates: one token, any shape, all of one
    dtype (float32 or bfloat16); lam, eta: float32 of the same shape.
    Returns (lam, eta)."""
    for name, t in (("a", a), ("p", p), ("phi", phi), ("b", b)):
        if t.shape != a.shape or t.dtype != a.dtype or t.device != a.device:
            raise ValueError("%s must match a in shape, dtype and device" % name)
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("%s must be a contiguous GPU tensor" % name)
    if a.dtype not in _DTYPES:
        raise ValueError("gate dtype must be float32 or bfloat16, got %s" % a.dtype)
    for name, t in (("lam", lam), ("eta", eta)):
        _check_f32(name, t, a.shape, a.device)
        if t is None:
            raise ValueError("%s is required" % name)
    stream = torch.cuda.current_stream(a.device)
    _check(library().kla_decode_step(_ptr(a), _ptr(p), _ptr(phi), _ptr(b), _DTYPES[a.dtype],
                                     _ptr(lam), _ptr(eta), a.numel(),
                                     ctypes.c_void_p(stream.cuda_stream)))
    return lam, eta


def mixer_decode_step(k: torch.Tensor, v: torch.Tensor, lam_v: torch.Tensor, q: torch.Tensor,
                      a: torch.Tensor, p: torch.Tensor, lam: torch.Tensor, eta: torch.Tensor,
                      want_var: bool = True, out: torch.Tensor | None = None,
                      var: torch.Tensor | None = None):
    """One token of the fused mixer on the running state (lam, eta), in place,
    on the current stream (kla_mixer_decode_step).  k, v, lam_v, q: [B, H, D]
    contiguous, all float32 or all bfloat16; a, p: [H, D] float32; lam, eta:
    [B, H, D] float32.  Returns (out, var, lam, eta): the readout q eta / lam
    and the variance 1 / lam of the new state (var None unless want_var)."""
    if k.dim() != 3:
        raise ValueError("token inputs must be [B, H, D], got shape %s" % (tuple(k.shape),))
    for name, t in zip(("k", "v", "lam_v", "q"), (k, v, lam_v, q)):
        if t.shape != k.shape or t.dtype != k.dtype:
            raise ValueError("%s must match k in shape and dtype" % name)
        if not t.is_cuda or t.device != k.device or not t.is_contiguous():
            raise ValueError("%s must be contiguous on k's GPU" % name)
    if k.dtype not in _DTYPES:
        raise ValueError("token dtype must be float32 or bfloat16, got %s" % k.dtype)
    B, H, D = k.shape
    dev = k.device
    for name, t in (("a", a), ("p", p)):
        if t is None:
            raise ValueError("%s is required" % name)
        _check_f32(name, t, (H, D), dev)
    for name, t in (("lam", lam), ("eta", eta)):
        if t is None:
            raise ValueError("%s is required" % name)
        _check_f32(name, t, k.shape, dev)
    if out is None:
        out = torch.empty(k.shape, dtype=torch.float32, device=dev)
    _check_f32("out", out, k.shape, dev)
    if want_var and var is None:
        var = torch.empty(k.shape, dtype=torch.float32, device=dev)
    if not want_var:
        var = None
    _check_f32("var", var, k.shape, dev)
    stream = torch.cuda.current_stream(dev)
    _check(library().kla_mixer_decode_step(
        _ptr(k), _ptr(v), _ptr(lam_v), _ptr(q), _DTYPES[k.dtype], _ptr(a), _ptr(p), _ptr(lam),
        _ptr(eta), _ptr(out), _ptr(var), k.numel(), H * D, ctypes.c_void_p(stream.cuda_stream)))
    return out, var, lam, eta


def workspace_health(workspace: torch.Tensor) -> int:
    """Reads and clears the workspace's health word (0: every call ran normally)."""
    out = ctypes.c_uint32(0)
    stream = torch.cuda.current_stream(workspace.device)
    _check(library().kla_workspace_health(_ptr(workspace), ctypes.byref(out),
                                          ctypes.c_void_p(stream.cuda_stream)))
    return int(out.value)
