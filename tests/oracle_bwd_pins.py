"""Pins of the float64 backward oracle (gradients of the scan).

Each pin takes ``scan_bwd(a, p, phi, b, lam0, eta0, g_lam, g_eta) -> (grads,
mags)`` and ``scan(a, p, phi, b, lam0, eta0) -> (lam, eta, eta_abs)`` (the
forward oracle, pinned separately) and raises AssertionError on a mismatch.

  * autograd: torch's reverse-mode differentiation (float64, CPU) of the
    information-form recursion of the Pith review of arXiv 2602.10743
    ("Circularity check", Theorems 1 and 2) -- an independent derivation of
    every partial derivative and of the index conventions;
  * finite differences: central differences of the *forward* oracle along
    random directions;
  * closed forms: p = 0, a = 1 (precisions and informations add, so every
    adjoint is a suffix sum of the upstream gradients);
  * magnitudes: |gradient| <= magnitude always, with equality when no term
    can be negative.
"""

from __future__ import annotations

import numpy as np
import torch

from oracle_pins import gates_np, state_np


def upstream(shape, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal(shape), rng.standard_normal(shape)


def loss_of(out, g_lam, g_eta):
    lam, eta = out[0], out[1]
    return float(np.sum(g_lam * lam) + np.sum(g_eta * eta))


def _close(name, got, ref, mag, tol):
    err = np.max(np.abs(got - ref) / np.maximum(mag, 1e-300)) if got.size else 0.0
    assert err <= tol, "%s: scaled error %.3g > %.1g" % (name, err, tol)


def autograd_grads(a, p, phi, b, lam0, eta0, g_lam, g_eta):
    """torch.autograd of the information-form forward, float64 on the CPU."""
    ts = [torch.tensor(x, dtype=torch.float64, requires_grad=True)
          for x in (a, p, phi, b, lam0, eta0)]
    ta, tp, tphi, tb, tl0, te0 = ts
    lam, eta = tl0, te0
    loss = torch.zeros((), dtype=torch.float64)
    for t in range(a.shape[2]):
        at, pt = ta[:, :, t], tp[:, :, t]
        den = at * at + pt * lam
        # lam / den written as 1 / (a^2 / lam + p): the same value, but its
        # derivative in lam (a^2 / den^2) comes out without the cancellation
        # 1/den - p lam/den^2 that autograd of lam / den would compute
        lam_new = 1.0 / (at * at / lam + pt) + tphi[:, :, t]
        eta = (at / den) * eta + tb[:, :, t]
        lam = lam_new
        loss = loss + (torch.tensor(g_lam[:, :, t]) * lam).sum() + \
            (torch.tensor(g_eta[:, :, t]) * eta).sum()
    grads = torch.autograd.grad(loss, ts)
    return dict(zip(("a", "p", "phi", "b", "lam0", "eta0"), (g.numpy() for g in grads)))


def pin_bwd_autograd(scan_bwd, scan):
    for shape, fam, seed in (((2, 2, 60, 3), "std", 61), ((1, 2, 80, 4), "slow", 62),
                             ((3, 1, 40, 2), "hard", 63)):
        a, p, phi, b = gates_np(shape, fam, seed)
        lam0, eta0 = state_np(shape[0], shape[1], shape[3], seed=seed)
        g_lam, g_eta = upstream(shape, seed)
        grads, mags = scan_bwd(a, p, phi, b, lam0, eta0, g_lam, g_eta)
        ref = autograd_grads(a, p, phi, b, lam0, eta0, g_lam, g_eta)
        for k in ref:
            _close("autograd %s (%s)" % (k, fam), grads[k], ref[k], mags[k], 1e-11)


def pin_bwd_finite_differences(scan_bwd, scan):
    """<grad, v> equals the central difference of the forward oracle's loss
    along a random direction v (relative step 1e-5; error O(h^2))."""
    rng = np.random.default_rng(71)
    shape = (1, 2, 24, 3)
    a, p, phi, b = gates_np(shape, "std", 71)
    lam0, eta0 = state_np(1, 2, 3, seed=71)
    g_lam, g_eta = upstream(shape, 72)
    grads, mags = scan_bwd(a, p, phi, b, lam0, eta0, g_lam, g_eta)
    x = {"a": a, "p": p, "phi": phi, "b": b, "lam0": lam0, "eta0": eta0}
    for trial in range(6):
        v = {k: rng.standard_normal(x[k].shape) * np.abs(x[k]) for k in x}
        h = 1e-5

        def shifted(s):
            return {k: x[k] + s * h * v[k] for k in x}
        up, dn = shifted(1.0), shifted(-1.0)
        f_up = loss_of(scan(up["a"], up["p"], up["phi"], up["b"], up["lam0"], up["eta0"]),
                       g_lam, g_eta)
        f_dn = loss_of(scan(dn["a"], dn["p"], dn["phi"], dn["b"], dn["lam0"], dn["eta0"]),
                       g_lam, g_eta)
        fd = (f_up - f_dn) / (2 * h)
        an = sum(float(np.sum(grads[k] * v[k])) for k in x)
        scale = sum(float(np.sum(mags[k] * np.abs(v[k]))) for k in x)
        assert abs(fd - an) <= 1e-7 * scale, ("finite differences", trial, fd, an, scale)


def pin_bwd_static_state(scan_bwd, scan):
    """p = 0, a = 1: lam_t = lam0 + sum phi, eta_t = eta0 + sum b, so the
    adjoints are suffix sums S_lam(s) = sum_{t>=s} g_lam[t] (likewise eta):
    g_phi = S_lam, g_b = S_eta, g_lam0 = S_lam(1), g_eta0 = S_eta(1),
    g_a[s] = -2 lam_{s-1} S_lam(s) - eta_{s-1} S_eta(s),
    g_p[s] = -lam_{s-1}^2 S_lam(s) - lam_{s-1} eta_{s-1} S_eta(s)."""
    shape = (2, 1, 50, 3)
    _, _, phi, b = gates_np(shape, "std", 81)
    a = np.ones(shape)
    p = np.zeros(shape)
    lam0, eta0 = state_np(2, 1, 3, seed=81)
    g_lam, g_eta = upstream(shape, 81)
    grads, mags = scan_bwd(a, p, phi, b, lam0, eta0, g_lam, g_eta)
    S_lam = np.flip(np.cumsum(np.flip(g_lam, 2), 2), 2)
    S_eta = np.flip(np.cumsum(np.flip(g_eta, 2), 2), 2)
    lam = lam0[:, :, None, :] + np.cumsum(phi, 2)
    eta = eta0[:, :, None, :] + np.cumsum(b, 2)
    lam_prev = np.concatenate([lam0[:, :, None, :], lam[:, :, :-1]], 2)
    eta_prev = np.concatenate([eta0[:, :, None, :], eta[:, :, :-1]], 2)
    ref = {"phi": S_lam, "b": S_eta, "lam0": S_lam[:, :, 0], "eta0": S_eta[:, :, 0],
           "a": -2 * lam_prev * S_lam - eta_prev * S_eta,
           "p": -lam_prev ** 2 * S_lam - lam_prev * eta_prev * S_eta}
    for k in ref:
        _close("static %s" % k, grads[k], ref[k], mags[k], 1e-12)


def pin_bwd_magnitudes(scan_bwd, scan):
    """|g| <= m always; |g| == m when every term is non-negative in size and
    sign-consistent: p = 0 (no eta-lambda coupling), g_lam, g_eta >= 0,
    b >= 0 and eta0 >= 0."""
    shape = (2, 2, 70, 3)
    a, p, phi, b = gates_np(shape, "std", 91)
    lam0, eta0 = state_np(2, 2, 3, seed=91)
    g_lam, g_eta = upstream(shape, 91)
    grads, mags = scan_bwd(a, p, phi, b, lam0, eta0, g_lam, g_eta)
    for k in grads:
        assert np.all(np.abs(grads[k]) <= mags[k] * (1 + 1e-12) + 1e-300), k
    p0 = np.zeros(shape)
    grads, mags = scan_bwd(a, p0, phi, np.abs(b), lam0, np.abs(eta0), np.abs(g_lam),
                           np.abs(g_eta))
    for k in grads:
        np.testing.assert_allclose(np.abs(grads[k]), mags[k], rtol=1e-12, atol=1e-300,
                                   err_msg="magnitude equality %s" % k)


ALL_BWD_PINS = [pin_bwd_autograd, pin_bwd_finite_differences, pin_bwd_static_state,
                pin_bwd_magnitudes]
