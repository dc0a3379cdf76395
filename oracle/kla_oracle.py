"""ctypes wrapper around ``kla_oracle.c`` (the float64 covariance-form filter).

TEST INFRASTRUCTURE ONLY (see the package docstring).  The arithmetic lives
in ``kla_oracle.c``; this module only converts arrays and calls it.

The filter follows the "KLA Part 1" primer, section 5.1 (one predict and one
update per token, a missing observation being zero precision) applied per
channel as the Pith review of arXiv 2602.10743 prescribes for the diagonal
model ("Load-bearing premise").
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "kla_oracle.c")
LIBRARY = os.path.join(_HERE, "libkla_oracle.so")

GCC_FLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
             "-shared", "-fPIC", "-std=c99"]


def build_oracle(out: str = LIBRARY, src: str = SOURCE) -> str:
    """Compiles an oracle source into a shared library with gcc; returns its path."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *GCC_FLAGS, src, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


class OracleLibrary:
    """One loaded copy of the oracle shared library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.kla_oracle_scan.argtypes = [dp] * 9 + [ctypes.c_int64] * 4 + [ctypes.c_int]
        lib.kla_oracle_scan.restype = ctypes.c_int
        lib.kla_oracle_scan_bwd.argtypes = [dp] * 20 + [ctypes.c_int64] * 4 + [ctypes.c_int]
        lib.kla_oracle_scan_bwd.restype = ctypes.c_int
        lib.kla_oracle_mixer.argtypes = [dp] * 13 + [ctypes.c_int64] * 4 + [ctypes.c_int]
        lib.kla_oracle_mixer.restype = ctypes.c_int
        lib.kla_oracle_mixer_bwd.argtypes = [dp] * 26 + [ctypes.c_int64] * 4 + [ctypes.c_int]
        lib.kla_oracle_mixer_bwd.restype = ctypes.c_int
        lib.kla_oracle_threads.argtypes = [ctypes.c_int]
        lib.kla_oracle_threads.restype = ctypes.c_int
        self._lib = lib
        self.path = path

    def threads(self, nthreads: int | None = None) -> int:
        return int(self._lib.kla_oracle_threads(int(nthreads or 0)))

    def scan(self, a, p, phi, b, lam0=None, eta0=None, nthreads: int | None = None):
        """Runs the float64 filter.

        a, p, phi, b: array-likes of shape [B, H, T, D] (any float dtype; the
        values are upcast to float64 exactly).  lam0, eta0: [B, H, D],
        default 1 and 0.  Returns (lam, eta, eta_abs), float64 [B, H, T, D].
        """
        a = _as_f64(a)
        if a.ndim != 4:
            raise ValueError("gates must be [B, H, T, D]")
        B, H, T, D = a.shape
        shape = (B, H, T, D)
        p, phi, b = (_as_f64(x, shape) for x in (p, phi, b))
        lam0 = _as_f64(np.ones((B, H, D)) if lam0 is None else lam0, (B, H, D))
        eta0 = _as_f64(np.zeros((B, H, D)) if eta0 is None else eta0, (B, H, D))
        lam, eta, eta_abs = np.empty(shape), np.empty(shape), np.empty(shape)
        rc = self._lib.kla_oracle_scan(
            _ptr(a), _ptr(p), _ptr(phi), _ptr(b), _ptr(lam0), _ptr(eta0),
            _ptr(lam), _ptr(eta), _ptr(eta_abs), B, H, T, D, int(nthreads or 0))
        if rc != 0:
            raise ValueError("oracle rejected the sizes")
        return lam, eta, eta_abs

    def scan_bwd(self, a, p, phi, b, lam0, eta0, g_lam, g_eta, nthreads: int | None = None):
        """Runs the float64 backward pass (vector-Jacobian product).

        Gates and upstream gradients g_lam, g_eta: [B, H, T, D]; lam0, eta0:
        [B, H, D] (None: 1 and 0).  Returns (grads, mags): two dicts with keys
        a, p, phi, b ([B, H, T, D]) and lam0, eta0 ([B, H, D]); grads are the
        gradients of sum(g_lam * lam + g_eta * eta) with respect to each
        input, mags their cancellation-free magnitudes.
        """
        a = _as_f64(a)
        if a.ndim != 4:
            raise ValueError("gates must be [B, H, T, D]")
        B, H, T, D = a.shape
        shape = (B, H, T, D)
        p, phi, b, g_lam, g_eta = (_as_f64(x, shape) for x in (p, phi, b, g_lam, g_eta))
        lam0 = _as_f64(np.ones((B, H, D)) if lam0 is None else lam0, (B, H, D))
        eta0 = _as_f64(np.zeros((B, H, D)) if eta0 is None else eta0, (B, H, D))
        names = ("a", "p", "phi", "b")
        grads = {k: np.empty(shape) for k in names}
        mags = {k: np.empty(shape) for k in names}
        for k in ("lam0", "eta0"):
            grads[k] = np.empty((B, H, D))
            mags[k] = np.empty((B, H, D))
        rc = self._lib.kla_oracle_scan_bwd(
            _ptr(a), _ptr(p), _ptr(phi), _ptr(b), _ptr(lam0), _ptr(eta0),
            _ptr(g_lam), _ptr(g_eta),
            *(_ptr(grads[k]) for k in names), _ptr(grads["lam0"]), _ptr(grads["eta0"]),
            *(_ptr(mags[k]) for k in names), _ptr(mags["lam0"]), _ptr(mags["eta0"]),
            B, H, T, D, int(nthreads or 0))
        if rc != 0:
            raise ValueError("backward oracle failed (%d)" % rc)
        return grads, mags


    def mixer(self, k, v, lam_v, q, a, p, lam0=None, eta0=None, nthreads: int | None = None):
        """Runs the float64 fused-mixer filter.

        k, v, lam_v, q: [B, H, T, D]; a, p: [H, D]; lam0, eta0: [B, H, D]
        (None: 1 and 0).  Returns a dict: out (q times the posterior mean),
        var (posterior variance), mu_abs (a bound on |mean|), [B, H, T, D];
        lam_T, eta_T (final precision and information mean), [B, H, D].
        """
        k = _as_f64(k)
        if k.ndim != 4:
            raise ValueError("token inputs must be [B, H, T, D]")
        B, H, T, D = k.shape
        shape = (B, H, T, D)
        v, lam_v, q = (_as_f64(x, shape) for x in (v, lam_v, q))
        a, p = (_as_f64(x, (H, D)) for x in (a, p))
        lam0 = _as_f64(np.ones((B, H, D)) if lam0 is None else lam0, (B, H, D))
        eta0 = _as_f64(np.zeros((B, H, D)) if eta0 is None else eta0, (B, H, D))
        res = {n: np.empty(shape) for n in ("out", "var", "mu_abs")}
        res["lam_T"], res["eta_T"] = np.empty((B, H, D)), np.empty((B, H, D))
        rc = self._lib.kla_oracle_mixer(
            _ptr(k), _ptr(v), _ptr(lam_v), _ptr(q), _ptr(a), _ptr(p), _ptr(lam0), _ptr(eta0),
            _ptr(res["out"]), _ptr(res["var"]), _ptr(res["mu_abs"]), _ptr(res["lam_T"]),
            _ptr(res["eta_T"]), B, H, T, D, int(nthreads or 0))
        if rc != 0:
            raise ValueError("oracle rejected the sizes")
        return res


    def mixer_bwd(self, k, v, lam_v, q, a, p, lam0, eta0, g_out, g_var,
                  nthreads: int | None = None):
        """Runs the float64 fused-mixer backward pass.

        Inputs as for ``mixer`` plus the upstream gradients g_out, g_var
        ([B, H, T, D]; g_var None means zero).  Returns (grads, mags): dicts
        with keys k, v, lam_v, q ([B, H, T, D]), a, p ([H, D], summed over the
        batch) and lam0, eta0 ([B, H, D]); mags are the cancellation-free
        magnitudes of the same sums.
        """
        k = _as_f64(k)
        if k.ndim != 4:
            raise ValueError("token inputs must be [B, H, T, D]")
        B, H, T, D = k.shape
        shape = (B, H, T, D)
        v, lam_v, q, g_out = (_as_f64(x, shape) for x in (v, lam_v, q, g_out))
        g_var = _as_f64(np.zeros(shape) if g_var is None else g_var, shape)
        a, p = (_as_f64(x, (H, D)) for x in (a, p))
        lam0 = _as_f64(np.ones((B, H, D)) if lam0 is None else lam0, (B, H, D))
        eta0 = _as_f64(np.zeros((B, H, D)) if eta0 is None else eta0, (B, H, D))
        names = ("k", "v", "lam_v", "q")
        grads = {n: np.empty(shape) for n in names}
        mags = {n: np.empty(shape) for n in names}
        for n, sh in (("a", (H, D)), ("p", (H, D)), ("lam0", (B, H, D)), ("eta0", (B, H, D))):
            grads[n] = np.empty(sh)
            mags[n] = np.empty(sh)
        rc = self._lib.kla_oracle_mixer_bwd(
            _ptr(k), _ptr(v), _ptr(lam_v), _ptr(q), _ptr(a), _ptr(p), _ptr(lam0), _ptr(eta0),
            _ptr(g_out), _ptr(g_var),
            *(_ptr(grads[n]) for n in names), _ptr(grads["a"]), _ptr(grads["p"]),
            _ptr(grads["lam0"]), _ptr(grads["eta0"]),
            *(_ptr(mags[n]) for n in names), _ptr(mags["a"]), _ptr(mags["p"]),
            _ptr(mags["lam0"]), _ptr(mags["eta0"]), B, H, T, D, int(nthreads or 0))
        if rc != 0:
            raise ValueError("mixer backward oracle failed (%d)" % rc)
        return grads, mags


def _as_f64(x, shape=None):
    if hasattr(x, "detach"):  # a torch tensor: copy to host, upcast exactly
        x = x.detach().to("cpu")
        x = x.double().numpy() if x.dtype.is_floating_point else x.numpy()
    arr = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    if shape is not None and arr.shape != tuple(shape):
        raise ValueError("expected shape %s, got %s" % (tuple(shape), arr.shape))
    return arr


def _ptr(arr):
    return arr.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


_lock = threading.Lock()
_default = None


def _library() -> OracleLibrary:
    global _default
    with _lock:
        if _default is None:
            if (not os.path.exists(LIBRARY)
                    or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE)):
                build_oracle()
            _default = OracleLibrary(LIBRARY)
        return _default


def oracle_threads(nthreads: int | None = None) -> int:
    """Threads the oracle's parallel loop uses for a given request."""
    return _library().threads(nthreads)


def oracle_scan(a, p, phi, b, lam0=None, eta0=None, nthreads: int | None = None):
    """The float64 oracle; see ``OracleLibrary.scan``."""
    return _library().scan(a, p, phi, b, lam0, eta0, nthreads)


def oracle_mixer(k, v, lam_v, q, a, p, lam0=None, eta0=None, nthreads: int | None = None):
    """The float64 fused-mixer oracle; see ``OracleLibrary.mixer``."""
    return _library().mixer(k, v, lam_v, q, a, p, lam0, eta0, nthreads)


def oracle_mixer_bwd(k, v, lam_v, q, a, p, lam0, eta0, g_out, g_var,
                     nthreads: int | None = None):
    """The float64 fused-mixer backward oracle; see ``OracleLibrary.mixer_bwd``."""
    return _library().mixer_bwd(k, v, lam_v, q, a, p, lam0, eta0, g_out, g_var, nthreads)


def oracle_scan_bwd(a, p, phi, b, lam0, eta0, g_lam, g_eta, nthreads: int | None = None):
    """The float64 backward oracle; see ``OracleLibrary.scan_bwd``."""
    return _library().scan_bwd(a, p, phi, b, lam0, eta0, g_lam, g_eta, nthreads)
