"""Pins that tie the float64 fused-mixer backward oracle to facts fixed
outside it.

Every pin takes ``mixer_bwd(k, v, lam_v, q, a, p, lam0, eta0, g_out, g_var)
-> (grads, mags)`` and ``mixer(...) -> dict`` (the forward oracle) and raises
AssertionError on a disagreement.  Used on the real oracle and on planted
mutants of it (test_oracle_mutants.py).

What pins what:
  * automatic differentiation: a float64 torch implementation of the mixer
    written here from the review's information form (Theorems 1 and 2 as the
    Pith review states them: predict lam / (a^2 + p lam), add k^2 lam_v; the
    information mean with the precision-ratio gate and increment k lam_v v;
    readout q eta / lam and variance 1 / lam), differentiated by
    torch.autograd;
  * central finite differences of the forward oracle;
  * the magnitudes bound the gradients;
  * the channel-gate gradients are sums over the batch of per-sequence
    gradients.
"""

from __future__ import annotations

import numpy as np
import torch


def _inputs(seed, B=2, H=2, T=12, D=3):
    rng = np.random.default_rng(seed)
    shape = (B, H, T, D)
    return dict(
        k=rng.normal(size=shape), v=rng.normal(size=shape),
        lam_v=np.log1p(np.exp(rng.normal(size=shape))), q=rng.normal(size=shape),
        a=rng.uniform(0.4, 1.1, size=(H, D)), p=rng.uniform(0.01, 0.6, size=(H, D)),
        lam0=rng.uniform(0.5, 2.0, size=(B, H, D)), eta0=rng.normal(size=(B, H, D)),
        g_out=rng.normal(size=shape), g_var=rng.normal(size=shape))


def _torch_mixer_loss(x):
    """Loss sum(g_out * out + g_var * var) of the information-form mixer."""
    k, v, lv, q = x["k"], x["v"], x["lam_v"], x["q"]
    B, H, T, D = k.shape
    a = x["a"][None]   # [1, H, D]
    p = x["p"][None]
    lam, eta = x["lam0"], x["eta0"]
    loss = torch.zeros((), dtype=torch.float64)
    for t in range(T):
        kt, vt, lvt, qt = k[:, :, t], v[:, :, t], lv[:, :, t], q[:, :, t]
        den = a * a + p * lam
        eta = a * eta / den + kt * lvt * vt
        lam = 1.0 / (a * a / lam + p) + kt * kt * lvt
        out = qt * eta / lam
        var = 1.0 / lam
        loss = loss + (x["g_out"][:, :, t] * out).sum() + (x["g_var"][:, :, t] * var).sum()
    return loss


NAMES = ("k", "v", "lam_v", "q", "a", "p", "lam0", "eta0")


def _check(grads, mags, ref, tol, what):
    for n in NAMES:
        err = np.abs(grads[n] - ref[n]) / np.maximum(mags[n], 1e-300)
        assert err.max() <= tol, "%s: %s error %.3g" % (what, n, err.max())


def pin_autograd(mixer_bwd, mixer):
    for seed in (1, 2):
        x = _inputs(seed)
        grads, mags = mixer_bwd(**x)
        leaves = {n: torch.tensor(x[n], dtype=torch.float64, requires_grad=n in NAMES)
                  for n in x}
        _torch_mixer_loss(leaves).backward()
        ref = {n: leaves[n].grad.numpy() for n in NAMES}
        _check(grads, mags, ref, 1e-10, "autograd")


def pin_finite_differences(mixer_bwd, mixer):
    x = _inputs(3, B=1, H=2, T=8, D=2)
    grads, mags = mixer_bwd(**x)

    def loss(xx):
        r = mixer(xx["k"], xx["v"], xx["lam_v"], xx["q"], xx["a"], xx["p"], xx["lam0"],
                  xx["eta0"])
        return float((xx["g_out"] * r["out"]).sum() + (xx["g_var"] * r["var"]).sum())

    rng = np.random.default_rng(4)
    for n in NAMES:
        for _ in range(3):
            idx = tuple(int(rng.integers(0, s)) for s in x[n].shape)
            h = 1e-6 * max(1.0, abs(x[n][idx]))
            xp = {m: val.copy() for m, val in x.items()}
            xm = {m: val.copy() for m, val in x.items()}
            xp[n][idx] += h
            xm[n][idx] -= h
            fd = (loss(xp) - loss(xm)) / (2 * h)
            err = abs(fd - grads[n][idx]) / max(mags[n][idx], 1e-12)
            assert err <= 1e-6, "finite differences: %s%s %r vs %r" % (n, idx, grads[n][idx], fd)


def pin_magnitudes_bound(mixer_bwd, mixer):
    x = _inputs(5, B=2, H=1, T=30, D=4)
    grads, mags = mixer_bwd(**x)
    for n in NAMES:
        assert np.all(np.abs(grads[n]) <= mags[n] * (1 + 1e-12) + 1e-300), "magnitude " + n


def pin_batch_sum(mixer_bwd, mixer):
    x = _inputs(6, B=3, H=2, T=10, D=2)
    grads, _ = mixer_bwd(**x)
    ga = np.zeros_like(x["a"])
    gp = np.zeros_like(x["p"])
    for b in range(3):
        xb = {n: (val[b:b + 1] if val.ndim >= 3 else val) for n, val in x.items()}
        gb, _ = mixer_bwd(**xb)
        ga += gb["a"]
        gp += gb["p"]
        for n in ("k", "v", "lam_v", "q"):
            np.testing.assert_allclose(gb[n][0], grads[n][b], rtol=1e-13, atol=1e-300)
    np.testing.assert_allclose(grads["a"], ga, rtol=1e-12)
    np.testing.assert_allclose(grads["p"], gp, rtol=1e-12)


ALL_MIXER_BWD_PINS = [pin_autograd, pin_finite_differences, pin_magnitudes_bound, pin_batch_sum]
