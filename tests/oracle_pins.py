"""Pins that tie the float64 oracle to facts fixed outside it.

Every pin takes ``scan(a, p, phi, b, lam0, eta0) -> (lam, eta, eta_abs)``
(numpy float64 arrays, [B, H, T, D] gates, [B, H, D] initial state) and raises
AssertionError when the oracle disagrees with the fact it checks.  They are
used on the real oracle (test_oracle_pins.py) and on planted mutants of it
(test_oracle_mutants.py), where at least one pin must fail.

What pins what:
  * exact marginal posterior (rational arithmetic): the filter's output is the
    marginal of x_t under the joint Gaussian of x_0..x_t given y_1..y_t, the
    inference statement of the "KLA Part 1" primer (section 3, statement B)
    on the model of its section 2 (eqs. 2.1-2.5).  Computed by Gaussian
    elimination on the tridiagonal joint precision -- no recursion shared
    with the oracle.
  * information form: the Moebius precision recursion and the affine
    information-mean recursion of the Pith review of arXiv 2602.10743
    ("What carries the argument", "Circularity check": predict
    lam_prior = lam / (a^2 + p lam), update lam = lam_prior + phi); the
    forget gate a / (a^2 + p lam_{t-1}) is the precision ratio of its "Core
    claim".
  * composition: prefix products of the 2x2 matrices M_t (same page) applied
    to lam0, affine prefixes, the 3x3 homogeneous lift, and the same under
    random bracketings (associativity axiom of the same page).
  * special cases with closed forms: p = 0 (the process-noise ablation on the
    same page), phi = 0 (missing observation, primer section 5.1), constant
    gates (fixed point of the Riccati map and powers of M).
  * invariants: lam > 0, the update never lowers precision below the prior,
    the posterior mean is a convex combination of prediction and observation
    (primer section 5.1), and the forget gate falls as precision grows (Pith
    review, "If this is right").
"""

from __future__ import annotations

import math
import random
from fractions import Fraction

import numpy as np

from kla_inputs import make_gates, make_initial_state


def _np(t):
    return t.detach().to("cpu").double().numpy()


def gates_np(shape, family="std", seed=0, dtype="f32"):
    g = make_gates(shape, family, dtype, seed)
    return tuple(_np(g[k]) for k in ("a", "p", "phi", "b"))


def state_np(B, H, D, random_state=True, seed=0):
    lam0, eta0 = make_initial_state(B, H, D, random=random_state, seed=seed)
    return _np(lam0), _np(eta0)


def _check_close(lam, eta, lam_ref, eta_ref, scale, tol, what):
    lam_err = np.max(np.abs(lam - lam_ref) / lam_ref)
    eta_err = np.max(np.abs(eta - eta_ref) / scale)
    assert lam_err <= tol and eta_err <= tol, (
        "%s: lam rel err %.3g, eta scaled err %.3g (tol %.1g)" % (what, lam_err, eta_err, tol))


# ---------------------------------------------------------------------------
# Exact marginal posterior by rational Gaussian elimination
# ---------------------------------------------------------------------------

def _solve_exact(K, rhs):
    """Solves K X = rhs exactly (K symmetric positive definite, Fractions)."""
    n = len(K)
    M = [list(K[i]) + [r[i] for r in rhs] for i in range(n)]
    m = len(rhs)
    for col in range(n):
        piv = M[col][col]
        for r in range(col + 1, n):
            fac = M[r][col] / piv
            if fac:
                for c in range(col, n + m):
                    M[r][c] -= fac * M[col][c]
    X = [[Fraction(0)] * n for _ in range(m)]
    for j in range(m):
        for i in range(n - 1, -1, -1):
            s = M[i][n + j] - sum(M[i][c] * X[j][c] for c in range(i + 1, n))
            X[j][i] = s / M[i][i]
    return X


def exact_marginal_filter(a, p, phi, b, lam0, eta0):
    """Exact (lam_t, eta_t), t = 1..T, of one channel, for p_t > 0.

    Joint information form of x_0..x_t: the prior on x_0 contributes
    (lam0, eta0); the transition x_s = a_s x_{s-1} + w_s with Var(w_s) = p_s
    contributes (x_s - a_s x_{s-1})^2 / p_s; the observation with precision
    phi_s and information b_s contributes phi_s to J[s, s] and b_s to h[s].
    The marginal of x_t is the Schur complement onto its row.
    """
    T = len(a)
    out_lam, out_eta = [], []
    for t in range(1, T + 1):
        n = t + 1
        J = [[Fraction(0)] * n for _ in range(n)]
        h = [Fraction(0)] * n
        J[0][0] += lam0
        h[0] += eta0
        for s in range(1, t + 1):
            q = 1 / p[s - 1]
            J[s][s] += q
            J[s - 1][s - 1] += a[s - 1] * a[s - 1] * q
            J[s - 1][s] -= a[s - 1] * q
            J[s][s - 1] -= a[s - 1] * q
            J[s][s] += phi[s - 1]
            h[s] += b[s - 1]
        K = [row[:t] for row in J[:t]]
        cols = [[J[i][t] for i in range(t)], h[:t]]
        X = _solve_exact(K, cols)
        out_lam.append(J[t][t] - sum(J[t][i] * X[0][i] for i in range(t)))
        out_eta.append(h[t] - sum(J[t][i] * X[1][i] for i in range(t)))
    return out_lam, out_eta


def pin_exact_marginal(scan, T=6, D=3, families=("std", "slow"), seed=11):
    for fam in families:
        a, p, phi, b = gates_np((1, 1, T, D), fam, seed)
        lam0, eta0 = state_np(1, 1, D, seed=seed)
        lam, eta, eta_abs = scan(a, p, phi, b, lam0, eta0)
        for d in range(D):
            F = lambda x: [Fraction(float(v)) for v in x]  # noqa: E731  exact binary values
            lam_x, eta_x = exact_marginal_filter(
                F(a[0, 0, :, d]), F(p[0, 0, :, d]), F(phi[0, 0, :, d]), F(b[0, 0, :, d]),
                Fraction(float(lam0[0, 0, d])), Fraction(float(eta0[0, 0, d])))
            lam_x = np.array([float(v) for v in lam_x])
            eta_x = np.array([float(v) for v in eta_x])
            scale = np.maximum(eta_abs[0, 0, :, d], np.abs(eta_x))
            _check_close(lam[0, 0, :, d], eta[0, 0, :, d], lam_x, eta_x, scale, 1e-13,
                         "exact marginal (%s, d=%d)" % (fam, d))


def pin_hand_worked(scan):
    """Two tokens worked by hand from the predict/update cycle.

    lam0 = 1, eta0 = 0 (P = 1, mu = 0).
    Token 1: a = 1, p = 1, phi = 1, b = 1: Ppred = 2, S = 3, mu = 2/3,
      P = 2/3 -> lam = 3/2, eta = 1.
    Token 2: a = 1/2, p = 1/4, phi = 2, b = -1: Ppred = 1/6 + 1/4 = 5/12,
      mupred = 1/3, S = 1 + 10/12 = 11/6, mu = (1/3 - 5/12) * 6/11 = -1/22,
      P = (5/12) * (6/11) = 5/22 -> lam = 22/5, eta = -1/5.
    (Information form check: lam_prior = 1.5 / 0.625 = 2.4, 2.4 + 2 = 4.4;
    f = 0.5 / 0.625 = 0.8, 0.8 * 1 - 1 = -0.2.)
    """
    a = np.array([1.0, 0.5]).reshape(1, 1, 2, 1)
    p = np.array([1.0, 0.25]).reshape(1, 1, 2, 1)
    phi = np.array([1.0, 2.0]).reshape(1, 1, 2, 1)
    b = np.array([1.0, -1.0]).reshape(1, 1, 2, 1)
    lam, eta, eta_abs = scan(a, p, phi, b, np.ones((1, 1, 1)), np.zeros((1, 1, 1)))
    np.testing.assert_allclose(lam.ravel(), [1.5, 4.4], rtol=1e-15)
    np.testing.assert_allclose(eta.ravel(), [1.0, -0.2], rtol=1e-15, atol=1e-16)
    # eta_abs: 0.8 * 1 + |-1| = 1.8
    np.testing.assert_allclose(eta_abs.ravel(), [1.0, 1.8], rtol=1e-15)


# ---------------------------------------------------------------------------
# Information form (Moebius precision, affine information mean)
# ---------------------------------------------------------------------------

def info_form(a, p, phi, b, lam0, eta0):
    """Information-form recursion over the T axis (axis 2), vectorised."""
    T = a.shape[2]
    lam = np.empty_like(a)
    eta = np.empty_like(a)
    l, e = lam0.astype(np.float64), eta0.astype(np.float64)
    for t in range(T):
        at, pt, ft, bt = a[:, :, t], p[:, :, t], phi[:, :, t], b[:, :, t]
        den = at * at + pt * l
        f = at / den
        l = l / den + ft
        e = f * e + bt
        lam[:, :, t] = l
        eta[:, :, t] = e
    return lam, eta


def pin_info_form(scan, cases=None):
    cases = cases or [((1, 1, 256, 16), "std", 0), ((2, 3, 300, 5), "slow", 1),
                      ((4, 2, 512, 8), "hard", 4)]
    for shape, fam, seed in cases:
        a, p, phi, b = gates_np(shape, fam, seed)
        lam0, eta0 = state_np(shape[0], shape[1], shape[3], seed=seed)
        lam, eta, eta_abs = scan(a, p, phi, b, lam0, eta0)
        lam_i, eta_i = info_form(a, p, phi, b, lam0, eta0)
        _check_close(lam, eta, lam_i, eta_i, np.maximum(eta_abs, lam * 2.0 ** -126),
                     1e-12, "information form (%s)" % fam)


def pin_eta_abs(scan):
    """eta_abs is eta of the same filter fed |b| and |eta0| (f does not depend
    on b), and equals eta when no term is negative."""
    a, p, phi, b = gates_np((2, 2, 200, 6), "std", 5)
    lam0, eta0 = state_np(2, 2, 6, seed=5)
    _, _, eta_abs = scan(a, p, phi, b, lam0, eta0)
    _, eta_pos, eta_abs_pos = scan(a, p, phi, np.abs(b), lam0, np.abs(eta0))
    np.testing.assert_allclose(eta_abs, eta_pos, rtol=1e-13)
    np.testing.assert_allclose(eta_abs_pos, eta_pos, rtol=1e-13)


# ---------------------------------------------------------------------------
# Composition: 2x2 Moebius matrices, affine maps, the 3x3 lift
# ---------------------------------------------------------------------------

def moebius(at, pt, phit):
    """M_t = [[1 + p phi, a^2 phi], [p, a^2]] (Pith review, Theorem 1)."""
    return np.array([[1.0 + pt * phit, at * at * phit], [pt, at * at]])


def lift(at, pt, phit, bt):
    """3x3 map on homogeneous (lam, eta, 1): rows lam, eta, 1."""
    a2 = at * at
    return np.array([[1.0 + pt * phit, 0.0, a2 * phit],
                     [bt * pt, at, bt * a2],
                     [pt, 0.0, a2]])


def _apply2(M, l):
    return (M[0, 0] * l + M[0, 1]) / (M[1, 0] * l + M[1, 1])


def _normalise(M):
    return M / np.max(np.abs(M))


def pin_prefix_products(scan, T=40, D=4):
    """Brute force: for every t the product M_t ... M_1 is formed afresh and
    applied to lam0; the affine maps (f_t, b_t) and the 3x3 lift likewise."""
    for fam, seed in (("std", 2), ("hard", 3), ("slow", 4)):
        a, p, phi, b = gates_np((1, 1, T, D), fam, seed)
        lam0, eta0 = state_np(1, 1, D, seed=seed)
        lam, eta, eta_abs = scan(a, p, phi, b, lam0, eta0)
        for d in range(D):
            at, pt, ft, bt = a[0, 0, :, d], p[0, 0, :, d], phi[0, 0, :, d], b[0, 0, :, d]
            l0, e0 = lam0[0, 0, d], eta0[0, 0, d]
            lam_prev = np.concatenate([[l0], lam[0, 0, :-1, d]])
            f = at / (at * at + pt * lam_prev)
            for t in range(T):
                M = np.eye(2)
                N = np.eye(3)
                F, Bv = 1.0, 0.0
                for s in range(t + 1):
                    M = _normalise(moebius(at[s], pt[s], ft[s]) @ M)
                    N = _normalise(lift(at[s], pt[s], ft[s], bt[s]) @ N)
                    F, Bv = f[s] * F, f[s] * Bv + bt[s]
                ref_l = _apply2(M, l0)
                v = N @ np.array([l0, e0, 1.0])
                scale = max(eta_abs[0, 0, t, d], lam[0, 0, t, d] * 2.0 ** -126)
                lt, et = lam[0, 0, t, d], eta[0, 0, t, d]
                assert abs(lt - ref_l) <= 1e-12 * ref_l, ("2x2 prefix", fam, d, t, lt, ref_l)
                assert abs(lt - v[0] / v[2]) <= 1e-12 * lt, ("3x3 lift lam", fam, d, t)
                assert abs(et - v[1] / v[2]) <= 1e-12 * scale, ("3x3 lift eta", fam, d, t)
                assert abs(et - (F * e0 + Bv)) <= 1e-12 * scale, ("affine prefix", fam, d, t)


def _random_tree_product(mats, rng, combine):
    """Multiplies mats (later maps on the left) under a random bracketing."""
    items = list(mats)
    while len(items) > 1:
        i = rng.randrange(len(items) - 1)
        items[i:i + 2] = [combine(items[i + 1], items[i])]
    return items[0]


def pin_random_bracketings(scan, T=64, D=3, trials=8, seed=7):
    """Associativity: any bracketing of the T maps gives the oracle's final
    state (2x2 Moebius, affine (f, b) with f from the oracle's lam, 3x3 lift)."""
    rng = random.Random(seed)
    for fam, s in (("std", 8), ("hard", 9)):
        a, p, phi, b = gates_np((1, 1, T, D), fam, s)
        lam0, eta0 = state_np(1, 1, D, seed=s)
        lam, eta, eta_abs = scan(a, p, phi, b, lam0, eta0)
        for d in range(D):
            at, pt, ft, bt = a[0, 0, :, d], p[0, 0, :, d], phi[0, 0, :, d], b[0, 0, :, d]
            l0, e0 = lam0[0, 0, d], eta0[0, 0, d]
            lam_prev = np.concatenate([[l0], lam[0, 0, :-1, d]])
            f = at / (at * at + pt * lam_prev)
            Ms = [moebius(at[t], pt[t], ft[t]) for t in range(T)]
            Ns = [lift(at[t], pt[t], ft[t], bt[t]) for t in range(T)]
            As = [(f[t], bt[t]) for t in range(T)]
            lT, eT = lam[0, 0, -1, d], eta[0, 0, -1, d]
            scale = max(eta_abs[0, 0, -1, d], lT * 2.0 ** -126)
            for _ in range(trials):
                M = _random_tree_product(Ms, rng, lambda x, y: _normalise(x @ y))
                N = _random_tree_product(Ns, rng, lambda x, y: _normalise(x @ y))
                F, Bv = _random_tree_product(
                    As, rng, lambda x, y: (x[0] * y[0], x[0] * y[1] + x[1]))
                assert abs(_apply2(M, l0) - lT) <= 1e-12 * lT, ("2x2 bracketing", fam, d)
                v = N @ np.array([l0, e0, 1.0])
                assert abs(v[0] / v[2] - lT) <= 1e-12 * lT, ("3x3 bracketing lam", fam, d)
                assert abs(v[1] / v[2] - eT) <= 1e-12 * scale, ("3x3 bracketing eta", fam, d)
                assert abs(F * e0 + Bv - eT) <= 1e-12 * scale, ("affine bracketing", fam, d)


# ---------------------------------------------------------------------------
# Special cases with closed forms
# ---------------------------------------------------------------------------

def pin_static_state(scan):
    """p = 0, a = 1: precisions and informations add (recursive least squares):
    lam_t = lam0 + sum phi, eta_t = eta0 + sum b."""
    shape = (2, 1, 300, 4)
    _, _, phi, b = gates_np(shape, "std", 21)
    a = np.ones(shape)
    p = np.zeros(shape)
    lam0, eta0 = state_np(2, 1, 4, seed=21)
    lam, eta, eta_abs = scan(a, p, phi, b, lam0, eta0)
    lam_x = lam0[:, :, None, :] + np.cumsum(phi, axis=2)
    eta_x = eta0[:, :, None, :] + np.cumsum(b, axis=2)
    _check_close(lam, eta, lam_x, eta_x, eta_abs, 1e-13, "p=0, a=1")


def pin_no_process_noise(scan):
    """p = 0, general a: with A_t = prod_{s<=t} a_s^2 and G_t = prod_{s<=t} a_s,
    lam_t A_t = lam0 + sum_{s<=t} phi_s A_s and eta_t G_t = eta0 + sum b_s G_s
    (lam_prior = lam / a^2, forget gate 1 / a)."""
    shape = (1, 2, 60, 4)
    a, _, phi, b = gates_np(shape, "std", 22)
    p = np.zeros(shape)
    lam0, eta0 = state_np(1, 2, 4, seed=22)
    lam, eta, eta_abs = scan(a, p, phi, b, lam0, eta0)
    A = np.cumprod(a * a, axis=2)
    G = np.cumprod(a, axis=2)
    lam_x = (lam0[:, :, None, :] + np.cumsum(phi * A, axis=2)) / A
    eta_x = (eta0[:, :, None, :] + np.cumsum(b * G, axis=2)) / G
    _check_close(lam, eta, lam_x, eta_x, eta_abs, 1e-12, "p=0")


def pin_no_observation(scan):
    """phi = 0, b = 0 (every observation missing): P_t = a_t^2 P_{t-1} + p_t and
    mu_t = mu0 prod a_s, so lam_t = 1 / P_t and eta_t = mu_t / P_t.  With
    a = 1: lam_t = 1 / (1 / lam0 + sum p)."""
    shape = (2, 2, 120, 3)
    a, p, _, _ = gates_np(shape, "std", 23)
    phi = np.zeros(shape)
    b = np.zeros(shape)
    lam0, eta0 = state_np(2, 2, 3, seed=23)
    lam, eta, eta_abs = scan(a, p, phi, b, lam0, eta0)
    A = np.cumprod(a * a, axis=2)
    # P_t = A_t (P0 + sum_{s<=t} p_s / A_s)
    P = A * (1.0 / lam0[:, :, None, :] + np.cumsum(p / A, axis=2))
    mu = (eta0 / lam0)[:, :, None, :] * np.cumprod(a, axis=2)
    _check_close(lam, eta, 1.0 / P, mu / P, np.maximum(eta_abs, np.abs(mu / P)), 1e-12,
                 "phi=0")
    ones = np.ones(shape)
    lam1, eta1, _ = scan(ones, p, phi, b, lam0, eta0)
    lam_x = 1.0 / (1.0 / lam0[:, :, None, :] + np.cumsum(p, axis=2))
    np.testing.assert_allclose(lam1, lam_x, rtol=1e-13)
    np.testing.assert_allclose(eta1, lam_x * (eta0 / lam0)[:, :, None, :], rtol=1e-13,
                               atol=1e-300)


def pin_constant_gates(scan):
    """Constant gates: lam_t = M^t(lam0) with M^t from the eigen-decomposition
    of M; lam_t tends to the positive root of p l^2 + (a^2 - 1 - p phi) l -
    a^2 phi = 0 and eta_t to b / (1 - f*), f* = a / (a^2 + p lam*)."""
    for (av, pv, fv, bv) in ((0.9, 0.3, 0.7, 0.4), (0.99, 0.01, 2.0, -1.5),
                             (0.5, 2.0, 0.1, 0.25)):
        T, D = 3000, 2
        shape = (1, 1, T, D)
        a = np.full(shape, av)
        p = np.full(shape, pv)
        phi = np.full(shape, fv)
        b = np.full(shape, bv)
        lam0 = np.array([[[0.3, 5.0]]])
        eta0 = np.array([[[1.0, -2.0]]])
        lam, eta, _ = scan(a, p, phi, b, lam0, eta0)
        M = moebius(av, pv, fv)
        w, V = np.linalg.eig(M)
        Vi = np.linalg.inv(V)
        for t in (1, 5, 17, 100):
            Mt = (V * w ** t) @ Vi
            for d in range(D):
                ref = _apply2(Mt, lam0[0, 0, d])
                assert abs(lam[0, 0, t - 1, d] - ref) <= 1e-11 * ref, ("M^t", av, t, d)
        c = 1.0 + pv * fv - av * av
        lam_star = (c + math.sqrt(c * c + 4.0 * pv * av * av * fv)) / (2.0 * pv)
        f_star = av / (av * av + pv * lam_star)
        np.testing.assert_allclose(lam[0, 0, -1], lam_star, rtol=1e-12)
        np.testing.assert_allclose(eta[0, 0, -1], bv / (1.0 - f_star), rtol=1e-11)


def _causal_convolution_fft(x, kernel):
    """y[t] = sum_{s <= t} kernel[t - s] x[s] along the last axis, by a
    zero-padded real FFT (the frequency-domain evaluation of the convolutional
    form)."""
    T = x.shape[-1]
    n = 1 << (2 * T - 1).bit_length()
    X = np.fft.rfft(x, n=n)
    K = np.fft.rfft(kernel, n=n)
    return np.fft.irfft(X * K, n=n)[..., :T]


def pin_lti_convolution(scan):
    """Time-invariant gates (the linear time-invariant case of the review's
    minor comment on Theorem 3).  Started from the stationary precision
    lam* (positive root of p l^2 + (a^2 - 1 - p phi) l - a^2 phi = 0) the
    precision stays lam* and eta is the causal convolution of b with the
    kernel f*^j (f* = a / (a^2 + p lam*)) plus f*^t eta0, evaluated here by
    FFT.  With p = 0 (a deterministic state) and a >= 1 the precision is
    a^-2t lam0 + phi sum_j a^-2j and the kernel of eta is a^-j, from any
    lam0."""
    rng = np.random.default_rng(23)
    T, D = 700, 5
    av = rng.uniform(0.3, 1.0, D)
    pv = rng.uniform(0.05, 2.0, D)
    fv = rng.uniform(0.1, 3.0, D)
    c = 1.0 + pv * fv - av * av
    lam_star = (c + np.sqrt(c * c + 4.0 * pv * av * av * fv)) / (2.0 * pv)
    f_star = av / (av * av + pv * lam_star)
    b = rng.normal(size=(1, 1, T, D)) * fv
    eta0 = rng.normal(size=(1, 1, D))
    full = lambda v: np.broadcast_to(v, (1, 1, T, D)).copy()  # noqa: E731
    lam, eta, eta_abs = scan(full(av), full(pv), full(fv), b, lam_star[None, None, :], eta0)
    np.testing.assert_allclose(lam[0, 0], np.broadcast_to(lam_star, (T, D)), rtol=1e-12)
    j = np.arange(T)
    for d in range(D):
        kern = f_star[d] ** j
        ref = _causal_convolution_fft(b[0, 0, :, d], kern) + f_star[d] ** (j + 1) * eta0[0, 0, d]
        err = np.abs(eta[0, 0, :, d] - ref) / eta_abs[0, 0, :, d]
        assert err.max() <= 1e-10, ("stationary LTI convolution", d, err.max())
    # deterministic state: p = 0, a >= 1
    av = rng.uniform(1.0, 1.05, D)
    fv = rng.uniform(0.1, 3.0, D)
    lam0 = rng.uniform(0.5, 2.0, (1, 1, D))
    lam, eta, eta_abs = scan(full(av), np.zeros((1, 1, T, D)), full(fv), b, lam0, eta0)
    for d in range(D):
        t = j + 1
        lam_ref = av[d] ** (-2.0 * t) * lam0[0, 0, d] + fv[d] * _causal_convolution_fft(
            np.ones(T), av[d] ** (-2.0 * j))
        np.testing.assert_allclose(lam[0, 0, :, d], lam_ref, rtol=1e-11)
        ref = _causal_convolution_fft(b[0, 0, :, d], av[d] ** (-1.0 * j)) + \
            av[d] ** (-1.0 * t) * eta0[0, 0, d]
        err = np.abs(eta[0, 0, :, d] - ref) / eta_abs[0, 0, :, d]
        assert err.max() <= 1e-10, ("deterministic LTI convolution", d, err.max())


# ---------------------------------------------------------------------------
# Invariants
# ---------------------------------------------------------------------------

def check_invariants(a, p, phi, b, lam0, eta0, lam, eta, eta_abs, rtol=1e-12):
    lam_prev = np.concatenate([lam0[:, :, None, :], lam[:, :, :-1]], axis=2)
    eta_prev = np.concatenate([eta0[:, :, None, :], eta[:, :, :-1]], axis=2)
    assert np.all(lam > 0), "lam must stay positive"
    # the update adds phi to the prior precision: lam_t > phi_t (strictly)
    assert np.all(lam > phi * (1 - rtol)), "update: lam_t > phi_t"
    with np.errstate(divide="ignore"):
        cap = np.minimum(lam_prev / (a * a), np.where(p > 0, 1.0 / p, np.inf))
    assert np.all(lam <= (phi + cap) * (1 + rtol)), "lam_t <= phi_t + min(lam/a^2, 1/p)"
    # posterior mean between the predicted mean and the observation
    mu_prev = eta_prev / lam_prev
    mu_pred = a * mu_prev
    mu = eta / lam
    obs = phi > 0
    y = np.where(obs, b / np.where(obs, phi, 1.0), 0.0)
    lo = np.minimum(mu_pred, y)
    hi = np.maximum(mu_pred, y)
    slack = rtol * (np.abs(mu_pred) + np.abs(y) + np.abs(mu)) + 1e-300
    assert np.all(~obs | ((mu >= lo - slack) & (mu <= hi + slack))), "convex combination"
    miss = ~obs & (b == 0)
    assert np.all(np.abs(mu - mu_pred)[miss] <= (rtol * np.abs(mu_pred) + 1e-300)[miss]), \
        "missing observation keeps the predicted mean"
    assert np.all(eta_abs >= np.abs(eta) * (1 - rtol)), "eta_abs bounds |eta|"


def pin_invariants(scan):
    for shape, fam, seed in (((2, 2, 400, 8), "std", 31), ((8, 2, 512, 4), "hard", 32),
                             ((1, 2, 2000, 3), "slow", 33)):
        a, p, phi, b = gates_np(shape, fam, seed)
        lam0, eta0 = state_np(shape[0], shape[1], shape[3], seed=seed)
        out = scan(a, p, phi, b, lam0, eta0)
        check_invariants(a, p, phi, b, lam0, eta0, *out)


def pin_forget_gate_falls(scan):
    """One token, b = 0, eta0 = 1: eta_1 = f_1, and f falls as the prior
    precision lam0 grows whenever p > 0."""
    a, p, phi, _ = gates_np((1, 1, 1, 64), "std", 41)
    b = np.zeros_like(a)
    lam_lo = np.full((1, 1, 64), 0.5)
    lam_hi = np.full((1, 1, 64), 4.0)
    _, f_lo, _ = scan(a, p, phi, b, lam_lo, lam_lo)      # eta0 = lam0 -> mu0 = 1
    _, f_hi, _ = scan(a, p, phi, b, lam_hi, lam_hi)
    f_lo = f_lo / lam_lo[:, :, None, :]
    f_hi = f_hi / lam_hi[:, :, None, :]
    assert np.all(f_hi < f_lo), "forget gate must fall as precision grows"
    # and equals a / (a^2 + p lam0) exactly in this one-step case
    np.testing.assert_allclose(f_lo, a / (a * a + p * 0.5), rtol=1e-14)


def pin_segmenting(scan):
    """Two calls chained through (lam_T1, eta_T1) equal one call."""
    shape = (2, 2, 257, 5)
    a, p, phi, b = gates_np(shape, "std", 51)
    lam0, eta0 = state_np(2, 2, 5, seed=51)
    lam, eta, _ = scan(a, p, phi, b, lam0, eta0)
    k = 100
    l1, e1, _ = scan(a[:, :, :k], p[:, :, :k], phi[:, :, :k], b[:, :, :k], lam0, eta0)
    l2, e2, _ = scan(a[:, :, k:], p[:, :, k:], phi[:, :, k:], b[:, :, k:],
                     l1[:, :, -1], e1[:, :, -1])
    np.testing.assert_allclose(np.concatenate([l1, l2], axis=2), lam, rtol=1e-13)
    np.testing.assert_allclose(np.concatenate([e1, e2], axis=2), eta, rtol=1e-12, atol=1e-13)


ALL_PINS = [pin_exact_marginal, pin_hand_worked, pin_info_form, pin_eta_abs,
            pin_prefix_products, pin_random_bracketings, pin_static_state,
            pin_no_process_noise, pin_no_observation, pin_constant_gates,
            pin_lti_convolution, pin_invariants, pin_forget_gate_falls, pin_segmenting]
