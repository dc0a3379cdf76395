"""Pins that tie the float64 fused-mixer oracle to facts fixed outside it.

Every pin takes ``mixer(k, v, lam_v, q, a, p, lam0, eta0) -> dict`` (numpy
float64 arrays: token inputs [B, H, T, D], channel gates [H, D], initial
state [B, H, D]; the dict holds out, var, mu_abs, lam_T, eta_T) and raises
AssertionError when the oracle disagrees with the fact it checks.  Used on the
real oracle (test_oracle_pins.py) and on planted mutants of it
(test_oracle_mutants.py), where at least one pin must fail.

The model is the scalar state-space model of the "KLA Part 1" primer
(section 2) with an observation operator: x_t = a x_{t-1} + w_t (Var p),
v_t = k_t x_t + e_t (precision lam_v_t), prior x_0 with precision lam0 and
information mean eta0; the mixer reads out q_t times the posterior mean and
the posterior variance (Pith review of arXiv 2602.10743: explicit belief-state
uncertainty; free-parameter ledger: time-invariant decay, learned process
noise, value precision and observation/readout operators from the input).

What pins what:
  * dense Gaussian conditioning: mean and variance of x_t given v_1..v_t from
    the joint covariance of (x_0..x_T) and the observations, by numpy linear
    solves -- the inference statement of the primer (section 3), no recursion;
  * static state (a = 1, p = 0): the posterior mean is the weighted least
    squares estimate of a constant from the prior and the observations
    (numpy lstsq), its variance the inverse of the normal matrix;
  * no observations (k = 0 or lam_v = 0): pure prediction in closed form;
  * the information form of the review ("Circularity check"): the scan
    oracle fed with phi = k^2 lam_v and b = k lam_v v gives lam = 1 / var and
    eta = mean / var;
  * the readout is q times one mean (linear in q); the magnitude bounds the
    mean and equals it when every contribution is non-negative;
  * the final state equals the last token's posterior, and two calls chained
    through it equal one call.
"""

from __future__ import annotations

import numpy as np


def _rng(seed):
    return np.random.default_rng(seed)


def _inputs(rng, B, H, T, D, missing=0.0):
    shape = (B, H, T, D)
    k = rng.normal(size=shape)
    v = rng.normal(size=shape)
    lv = np.log1p(np.exp(rng.normal(size=shape)))
    if missing:
        lv[rng.random(size=shape) < missing] = 0.0
    q = rng.normal(size=shape)
    a = rng.uniform(0.3, 1.2, size=(H, D))
    p = rng.uniform(0.0, 0.5, size=(H, D))
    lam0 = rng.uniform(0.5, 2.0, size=(B, H, D))
    eta0 = rng.normal(size=(B, H, D))
    return k, v, lv, q, a, p, lam0, eta0


def _dense_posterior(k, v, lv, a, p, lam0, eta0):
    """Mean and variance of x_t given the observations up to t (t = 1..T) for
    one channel, by conditioning the joint Gaussian with dense solves."""
    T = len(k)
    # x_t = a^t x_0 + sum_{s<=t} a^{t-s} w_s: x = m + G w
    G = np.zeros((T + 1, T + 1))
    for t in range(T + 1):
        for s in range(t + 1):
            G[t, s] = a ** (t - s)
    w_var = np.array([1.0 / lam0] + [p] * T)
    Sxx = G @ np.diag(w_var) @ G.T
    m = np.array([a ** t * (eta0 / lam0) for t in range(T + 1)])
    means, variances = np.empty(T), np.empty(T)
    for t in range(1, T + 1):
        obs = [s for s in range(1, t + 1) if lv[s - 1] > 0]
        if not obs:
            means[t - 1], variances[t - 1] = m[t], Sxx[t, t]
            continue
        Hm = np.zeros((len(obs), T + 1))
        for j, s in enumerate(obs):
            Hm[j, s] = k[s - 1]
        Svv = Hm @ Sxx @ Hm.T + np.diag([1.0 / lv[s - 1] for s in obs])
        Sxv = Sxx[t] @ Hm.T
        resid = np.array([v[s - 1] for s in obs]) - Hm @ m
        means[t - 1] = m[t] + Sxv @ np.linalg.solve(Svv, resid)
        variances[t - 1] = Sxx[t, t] - Sxv @ np.linalg.solve(Svv, Sxv)
    return means, variances


def _check_mean(got_mean, want_mean, mu_abs, tol, what):
    err = np.abs(got_mean - want_mean) / np.maximum(mu_abs, 1e-300)
    assert err.max() <= tol, "%s: mean error %.3g" % (what, err.max())


def pin_dense_gaussian_conditioning(mixer):
    for seed, missing in ((1, 0.0), (2, 0.3)):
        rng = _rng(seed)
        k, v, lv, q, a, p, lam0, eta0 = _inputs(rng, 2, 2, 9, 3, missing)
        res = mixer(k, v, lv, q, a, p, lam0, eta0)
        for b in range(2):
            for h in range(2):
                for d in range(3):
                    mean, var = _dense_posterior(k[b, h, :, d], v[b, h, :, d], lv[b, h, :, d],
                                                 a[h, d], p[h, d], lam0[b, h, d], eta0[b, h, d])
                    got = res["out"][b, h, :, d] / q[b, h, :, d]
                    scale = np.maximum(res["mu_abs"][b, h, :, d], np.abs(mean))
                    _check_mean(got, mean, scale, 1e-9, "dense conditioning")
                    rel = np.abs(res["var"][b, h, :, d] - var) / var
                    assert rel.max() <= 1e-9, "dense conditioning: variance error %.3g" % rel.max()


def pin_static_least_squares(mixer):
    rng = _rng(3)
    B, H, T, D = 1, 1, 12, 4
    k, v, lv, q, _, _, lam0, eta0 = _inputs(rng, B, H, T, D)
    a = np.ones((H, D))
    p = np.zeros((H, D))
    res = mixer(k, v, lv, q, a, p, lam0, eta0)
    for d in range(D):
        l0, mu0 = lam0[0, 0, d], eta0[0, 0, d] / lam0[0, 0, d]
        for t in range(1, T + 1):
            w = np.sqrt(np.concatenate([[l0], lv[0, 0, :t, d]]))
            A = (w * np.concatenate([[1.0], k[0, 0, :t, d]]))[:, None]
            y = w * np.concatenate([[mu0], v[0, 0, :t, d]])
            est = np.linalg.lstsq(A, y, rcond=None)[0][0]
            var = 1.0 / (A[:, 0] @ A[:, 0])
            got = res["out"][0, 0, t - 1, d] / q[0, 0, t - 1, d]
            assert abs(got - est) <= 1e-11 * max(res["mu_abs"][0, 0, t - 1, d], abs(est)), \
                "static least squares: mean %r vs %r" % (got, est)
            assert abs(res["var"][0, 0, t - 1, d] - var) <= 1e-12 * var, "static: variance"


def pin_no_observation_prediction(mixer):
    rng = _rng(4)
    B, H, T, D = 1, 1, 10, 3
    k, v, lv, q, a, p, lam0, eta0 = _inputs(rng, B, H, T, D)
    lv[..., :2] = 0.0  # channels 0, 1: no observation precision
    k[..., 2] = 0.0    # channel 2: no observation operator
    res = mixer(k, v, lv, q, a, p, lam0, eta0)
    for d in range(D):
        ad, pd = a[0, d], p[0, d]
        P0, mu0 = 1.0 / lam0[0, 0, d], eta0[0, 0, d] / lam0[0, 0, d]
        for t in range(1, T + 1):
            mean = ad ** t * mu0
            var = ad ** (2 * t) * P0 + pd * sum(ad ** (2 * j) for j in range(t))
            got = res["out"][0, 0, t - 1, d] / q[0, 0, t - 1, d]
            assert abs(got - mean) <= 1e-13 * max(abs(mean), 1e-300) + 1e-300, "prediction mean"
            assert abs(res["var"][0, 0, t - 1, d] - var) <= 1e-13 * var, "prediction variance"


def pin_information_form(mixer):
    """The review's information-form update with phi = k^2 lam_v, b = k lam_v v."""
    from oracle import oracle_scan
    rng = _rng(5)
    B, H, T, D = 2, 3, 40, 4
    k, v, lv, q, a, p, lam0, eta0 = _inputs(rng, B, H, T, D, missing=0.1)
    res = mixer(k, v, lv, q, a, p, lam0, eta0)
    ab = np.broadcast_to(a[None, :, None, :], k.shape)
    pb = np.broadcast_to(p[None, :, None, :], k.shape)
    lam, eta, eta_abs = oracle_scan(ab, pb, k * k * lv, k * lv * v, lam0, eta0)
    rel = np.abs(1.0 / res["var"] - lam) / lam
    assert rel.max() <= 1e-12, "information form: precision %.3g" % rel.max()
    _check_mean(res["out"] / q, eta / lam, eta_abs / lam, 1e-12, "information form")
    rel = np.abs(res["mu_abs"] - eta_abs / lam) / (eta_abs / lam)
    assert rel.max() <= 1e-12, "information form: magnitude"


def pin_readout_and_magnitude(mixer):
    rng = _rng(6)
    B, H, T, D = 1, 2, 30, 3
    k, v, lv, q, a, p, lam0, eta0 = _inputs(rng, B, H, T, D)
    ones = np.ones_like(q)
    r1 = mixer(k, v, lv, ones, a, p, lam0, eta0)
    rq = mixer(k, v, lv, q, a, p, lam0, eta0)
    assert np.allclose(rq["out"], q * r1["out"], rtol=1e-15, atol=0), "readout is q * mean"
    assert np.array_equal(rq["var"], r1["var"]), "variance does not depend on q"
    assert np.all(np.abs(r1["out"]) <= r1["mu_abs"] * (1 + 1e-12)), "|mean| <= magnitude"
    # every contribution non-negative: magnitude == mean
    rp = mixer(np.abs(k), np.abs(v), lv, ones, a, p, lam0, np.abs(eta0))
    assert np.allclose(rp["out"], rp["mu_abs"], rtol=1e-12, atol=0), "magnitude of a positive sum"


def pin_final_state_and_segments(mixer):
    rng = _rng(7)
    B, H, T, D = 2, 1, 24, 3
    k, v, lv, q, a, p, lam0, eta0 = _inputs(rng, B, H, T, D)
    whole = mixer(k, v, lv, q, a, p, lam0, eta0)
    lam_last = 1.0 / whole["var"][:, :, -1]
    assert np.allclose(whole["lam_T"], lam_last, rtol=1e-15, atol=0), "final precision"
    mean_last = whole["out"][:, :, -1] / q[:, :, -1]
    assert np.allclose(whole["eta_T"], mean_last * lam_last, rtol=1e-12, atol=1e-300), \
        "final information mean"
    s = 10
    first = mixer(k[:, :, :s], v[:, :, :s], lv[:, :, :s], q[:, :, :s], a, p, lam0, eta0)
    second = mixer(k[:, :, s:], v[:, :, s:], lv[:, :, s:], q[:, :, s:], a, p,
                   first["lam_T"], first["eta_T"])
    for name in ("out", "var"):
        both = np.concatenate([first[name], second[name]], axis=2)
        assert np.allclose(both, whole[name], rtol=1e-12, atol=1e-300), "segments: " + name


ALL_MIXER_PINS = [
    pin_dense_gaussian_conditioning,
    pin_static_least_squares,
    pin_no_observation_prediction,
    pin_information_form,
    pin_readout_and_magnitude,
    pin_final_state_and_segments,
]
