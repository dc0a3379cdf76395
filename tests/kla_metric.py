"""Parity metric between fp32 scan outputs and the float64 oracle.

Readings of "maximum relative error" for this scan (the pages print none):

* lam (posterior precision, always > 0, a sum of non-negative terms):
  max |lam_hat - lam| / lam.
* eta (information mean) is a signed sum that can cancel to near zero, so a
  plain relative error is ill-posed there.  Its error is divided by the
  cancellation-free magnitude eta_abs (the same recursion with |b| and a
  non-negative start), floored at lam * 2^-126 so that only posterior means
  |eta| / lam below fp32's normal range are forgiven:
  max |eta_hat - eta| / max(eta_abs, lam * 2^-126).
* Range: where the exact value rounds to an fp32 overflow, the output must be
  the infinity of the same sign; everywhere else it must be finite.  Any NaN
  fails.

The plain |eta_hat - eta| / |eta| over elements that do not cancel
(|eta| >= 0.1 eta_abs) is reported too, without a gate.
"""

from __future__ import annotations

import numpy as np

TINY = 2.0 ** -126

TOL_F32 = 1e-4   # fp32 gate inputs
TOL_BF16 = 2e-2  # bf16 gate inputs (oracle runs on the same bf16 values)
# Regression bound of the forward paths, checked next to the bars above: the
# kernels carry float64 from the very input values the oracle reads, so their
# only error of note is the final float32 rounding (~6e-8).  A slip that moves
# a gate by one token or one channel shows up far above it.
TOL_REGRESSION = 1e-5


def _np(x):
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        return (x.double() if x.dtype.is_floating_point else x).numpy()
    return np.asarray(x)


def compare(lam_hat, eta_hat, lam, eta, eta_abs) -> dict:
    """Returns the error report of fp32 outputs against float64 oracle values."""
    lam_hat = _np(lam_hat).astype(np.float64)
    eta_hat = _np(eta_hat).astype(np.float64)
    lam, eta, eta_abs = (np.asarray(x, dtype=np.float64) for x in (lam, eta, eta_abs))
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        lam32 = lam.astype(np.float32)
        eta32 = eta.astype(np.float32)
        lam_over = np.isinf(lam32)
        eta_over = np.isinf(eta32)

        rep = {"n": int(lam.size)}
        rep["nan"] = int(np.isnan(lam_hat).sum() + np.isnan(eta_hat).sum())
        # overflow rule
        bad_inf = (lam_over & (lam_hat != np.inf)).sum()
        bad_inf += (eta_over & (eta_hat != np.sign(eta) * np.inf)).sum()
        bad_inf += (~lam_over & ~np.isfinite(lam_hat)).sum()
        bad_inf += (~eta_over & ~np.isfinite(eta_hat)).sum()
        rep["range_violations"] = int(bad_inf)
        rep["lam_overflow"] = int(lam_over.sum())
        rep["eta_overflow"] = int(eta_over.sum())

        ok = ~lam_over & np.isfinite(lam_hat)
        lam_err = np.abs(lam_hat - lam) / lam
        rep["lam_max_rel"] = float(lam_err[ok].max()) if ok.any() else 0.0

        ok = ~eta_over & ~lam_over & np.isfinite(eta_hat)
        den = np.maximum(eta_abs, lam * TINY)
        eta_err = np.abs(eta_hat - eta) / den
        rep["eta_max_scaled"] = float(eta_err[ok].max()) if ok.any() else 0.0

        plain = ok & (np.abs(eta) >= 0.1 * eta_abs) & (eta != 0)
        rel = np.abs(eta_hat - eta) / np.abs(eta)
        rep["eta_max_rel_noncancel"] = float(rel[plain].max()) if plain.any() else 0.0
    return rep


_MAX_KEYS = ("lam_max_rel", "eta_max_scaled", "eta_max_rel_noncancel")
_SUM_KEYS = ("n", "nan", "range_violations", "lam_overflow", "eta_overflow")


def merge_reports(reps) -> dict:
    """One report for the union of the elements of several reports (counts
    add, maxima take the largest)."""
    out = {k: 0 for k in _SUM_KEYS}
    out.update({k: 0.0 for k in _MAX_KEYS})
    for r in reps:
        for k in _SUM_KEYS:
            out[k] += r[k]
        for k in _MAX_KEYS:
            out[k] = max(out[k], r[k])
    return out


_COUNT_KEYS = _SUM_KEYS + ("zero_q_nonzero_out",)


def merge_any(reps) -> dict:
    """merge_reports for any of the reports of this module (compare_mixer's,
    compare_grads'): count keys add, every other key takes the largest."""
    out: dict = {}
    for r in reps:
        for k, v in r.items():
            out[k] = out.get(k, 0) + v if k in _COUNT_KEYS else max(out.get(k, 0.0), v)
    return out


def assert_parity(rep: dict, tol: float, what: str = ""):
    msg = "%s %r" % (what, rep)
    assert rep["nan"] == 0, msg
    assert rep["range_violations"] == 0, msg
    assert rep["lam_max_rel"] <= tol, msg
    assert rep["eta_max_scaled"] <= tol, msg


GRAD_FLOOR = 2.0 ** -100


def compare_grads(got: dict, grads: dict, mags: dict) -> dict:
    """Per-input error of fp32 gradients against the float64 backward oracle:
    max |g_hat - g| / max(m, 2^-100), m the cancellation-free magnitude of the
    same sum (a gradient is a signed sum that can cancel), with the fp32
    overflow rule and no NaN, as for the forward outputs."""
    rep = {"nan": 0, "range_violations": 0}
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        for k, ref in grads.items():
            if k not in got or got[k] is None:
                continue
            g = _np(got[k]).astype(np.float64)
            ref = np.asarray(ref, dtype=np.float64)
            m = np.asarray(mags[k], dtype=np.float64)
            over = np.isinf(ref.astype(np.float32))
            rep["nan"] += int(np.isnan(g).sum())
            rep["range_violations"] += int((over & (g != np.sign(ref) * np.inf)).sum())
            rep["range_violations"] += int((~over & ~np.isfinite(g)).sum())
            ok = ~over & np.isfinite(g)
            err = np.abs(g - ref) / np.maximum(m, GRAD_FLOOR)
            rep[k] = float(err[ok].max()) if ok.any() else 0.0
    return rep


def assert_grad_parity(rep: dict, tol: float, what: str = ""):
    msg = "%s %r" % (what, rep)
    assert rep["nan"] == 0, msg
    assert rep["range_violations"] == 0, msg
    for k, v in rep.items():
        if k not in ("nan", "range_violations"):
            assert v <= tol, msg


def compare_mixer(out_hat, var_hat, q, out, var, mu_abs) -> dict:
    """Error report of the fused mixer's fp32 outputs against the float64
    oracle.  The readout q * mean is a signed quantity that can cancel, so its
    error is divided by |q| times the cancellation-free magnitude of the mean
    (floored at 2^-126); where q is 0 the output must be exactly 0.  The
    variance is positive: plain relative error, floored at 2^-126.  The fp32
    overflow rule and the NaN rule are those of ``compare``."""
    out_hat = _np(out_hat).astype(np.float64)
    q = _np(q).astype(np.float64)
    out, mu_abs = (np.asarray(x, dtype=np.float64) for x in (out, mu_abs))
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        out_over = np.isinf(out.astype(np.float32))
        rep = {"n": int(out.size)}
        rep["nan"] = int(np.isnan(out_hat).sum())
        bad = (out_over & (out_hat != np.sign(out) * np.inf)).sum()
        bad += (~out_over & ~np.isfinite(out_hat)).sum()
        ok = ~out_over & np.isfinite(out_hat)
        den = np.abs(q) * np.maximum(mu_abs, TINY)
        zero_q = den == 0
        rep["zero_q_nonzero_out"] = int((zero_q & (out_hat != 0)).sum())
        err = np.abs(out_hat - out) / np.where(zero_q, 1.0, den)
        rep["out_max_scaled"] = float(err[ok & ~zero_q].max()) if (ok & ~zero_q).any() else 0.0
        if var_hat is not None:
            var_hat = _np(var_hat).astype(np.float64)
            var = np.asarray(var, dtype=np.float64)
            rep["nan"] += int(np.isnan(var_hat).sum())
            bad += (~np.isfinite(var_hat)).sum()
            vok = np.isfinite(var_hat)
            verr = np.abs(var_hat - var) / np.maximum(var, TINY)
            rep["var_max_rel"] = float(verr[vok].max()) if vok.any() else 0.0
        rep["range_violations"] = int(bad)
    return rep


def assert_mixer_parity(rep: dict, tol: float, what: str = ""):
    msg = "%s %r" % (what, rep)
    assert rep["nan"] == 0, msg
    assert rep["range_violations"] == 0, msg
    assert rep["zero_q_nonzero_out"] == 0, msg
    assert rep["out_max_scaled"] <= tol, msg
    assert rep.get("var_max_rel", 0.0) <= tol, msg
