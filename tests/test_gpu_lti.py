"""GPU parity of the time-invariant-gate scan (kla_scan_lti_fwd through the
C ABI) against the float64 oracle fed the same gates broadcast over time, and
against the convolutional (FFT) form in the stationary case.  Bar: the
kla_metric rules, 1e-4 for fp32 inputs, 2e-2 for bf16."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from kla_inputs import (LTI_WORKLOADS, broadcast_lti, make_initial_state, make_lti_inputs,
                        make_lti_workload)
from kla_metric import TOL_BF16, TOL_F32, TOL_REGRESSION, assert_parity, compare, merge_reports
from oracle import oracle_scan

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)


def run_gpu(g, use_state=True):
    from linear_attention_sequence_kla_amd import scan_lti_fwd
    lam0 = g["lam0"].to(DEV) if use_state else None
    eta0 = g["eta0"].to(DEV) if use_state else None
    lam, eta = scan_lti_fwd(g["a"].to(DEV), g["p"].to(DEV), g["phi"].to(DEV), g["b"].to(DEV),
                            lam0, eta0)
    torch.cuda.synchronize(DEV)
    return lam, eta


def health():
    from linear_attention_sequence_kla_amd import get_workspace, workspace_health
    return workspace_health(get_workspace(0, DEV, torch.cuda.current_stream(DEV)))


def full_parity(g, tol, what, use_state=True):
    lam, eta = run_gpu(g, use_state)
    assert health() == 0, what
    f = broadcast_lti(g)
    ref = oracle_scan(f["a"], f["p"], f["phi"], f["b"], g["lam0"] if use_state else None,
                      g["eta0"] if use_state else None)
    rep = compare(lam.cpu(), eta.cpu(), *ref)
    _say("%s: %s" % (what, rep))
    assert_parity(rep, tol, what)
    return rep


@pytest.mark.parametrize("key", [0, 1])
def test_lti_workload_full(key):
    w = LTI_WORKLOADS[key]
    _say("LTI workload %s" % w.describe())
    full_parity(make_lti_workload(key), TOL_F32, w.describe())


@pytest.mark.parametrize("key", [2, 3])
def test_lti_workload_full_size_sampled(key):
    """Full size in the benchmark's launch configuration; the oracle checks a
    sample of (b, h) slabs with all their channels and the whole sequence."""
    w = LTI_WORKLOADS[key]
    _say("LTI workload %s (full size, sampled slabs)" % w.describe())
    g = make_lti_inputs(w.shape, w.gates, w.dtype, w.seed, device=DEV)
    g["lam0"], g["eta0"] = make_initial_state(w.B, w.H, w.D, random=True, seed=w.seed,
                                              device=DEV)
    lam, eta = run_gpu(g)
    assert health() == 0
    rng = np.random.default_rng(w.seed)
    slabs = sorted(set(rng.choice(w.B * w.H, size=min(3, w.B * w.H), replace=False).tolist())
                   | {w.B * w.H - 1})
    for s in slabs:
        bi, hi = divmod(s, w.H)
        sub = {n: g[n][hi:hi + 1].cpu() for n in ("a", "p", "phi")}
        sub["b"] = g["b"][bi:bi + 1, hi:hi + 1].cpu()
        f = broadcast_lti(sub)
        ref = oracle_scan(f["a"], f["p"], f["phi"], f["b"], g["lam0"][bi:bi + 1, hi:hi + 1].cpu(),
                          g["eta0"][bi:bi + 1, hi:hi + 1].cpu())
        rep = compare(lam[bi:bi + 1, hi:hi + 1].cpu(), eta[bi:bi + 1, hi:hi + 1].cpu(), *ref)
        _say("slab (%d, %d): %s" % (bi, hi, rep))
        assert_parity(rep, TOL_BF16 if w.dtype == "bf16" else TOL_F32, "slab %d" % s)


@pytest.mark.parametrize("key", [2, 3])
def test_lti_workload_every_element(key):
    """A full-size workload drawn on the GPU exactly as the benchmark draws it,
    in the benchmark's launch; the oracle runs on host copies, a batch of
    (b, h) slabs at a time with the gates of those h broadcast over time, and
    every output element is compared."""
    w = LTI_WORKLOADS[key]
    _say("LTI workload %s (every element)" % w.describe())
    g = make_lti_workload(key, device=DEV)
    lam, eta = run_gpu(g)
    assert health() == 0
    B, H, T, D = w.shape
    per = max(1, min(H, (1 << 25) // (T * D)))
    reps = []
    for b in range(B):
        for h0 in range(0, H, per):
            h1 = min(H, h0 + per)
            sub = {n: g[n][h0:h1].cpu() for n in ("a", "p", "phi")}
            sub["b"] = g["b"][b:b + 1, h0:h1].cpu()
            f = broadcast_lti(sub)
            ref = oracle_scan(f["a"], f["p"], f["phi"], f["b"], g["lam0"][b:b + 1, h0:h1].cpu(),
                              g["eta0"][b:b + 1, h0:h1].cpu())
            reps.append(compare(lam[b:b + 1, h0:h1].cpu(), eta[b:b + 1, h0:h1].cpu(), *ref))
            del sub, f, ref
    rep = merge_reports(reps)
    _say("%s: %s" % (w.describe(), rep))
    assert rep["n"] == w.elements
    assert_parity(rep, TOL_BF16 if w.dtype == "bf16" else TOL_F32, w.describe())
    assert max(rep["lam_max_rel"], rep["eta_max_scaled"]) <= TOL_REGRESSION, rep


SHAPES = [(1, 1, 1, 1), (1, 1, 5, 3), (2, 3, 113, 7), (1, 2, 337, 64), (3, 1, 450, 65),
          (2, 2, 1000, 33), (1, 1, 2049, 128), (4, 3, 96, 40), (3, 3, 700, 128)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_lti_shapes(shape):
    g = make_lti_inputs(shape, "std", "f32", seed=sum(shape))
    g["lam0"], g["eta0"] = make_initial_state(shape[0], shape[1], shape[3], random=True,
                                              seed=sum(shape))
    full_parity(g, TOL_F32, "shape %s" % (shape,))


def test_lti_bf16_and_default_state():
    shape = (2, 2, 700, 48)
    g = make_lti_inputs(shape, "std", "bf16", seed=5)
    g["lam0"], g["eta0"] = make_initial_state(2, 2, 48)
    full_parity(g, TOL_BF16, "bf16 %s" % (shape,), use_state=False)


# LTI tiles hold 64 rows x 4 waves; bfloat16 rows are packed two to a register
@pytest.mark.parametrize("shape", [(1, 2, 256, 64), (2, 1, 257, 33), (1, 1, 63, 5),
                                   (2, 3, 1001, 128), (2, 2, 1, 9)],
                         ids=lambda s: "x".join(map(str, s)))
def test_lti_bf16_tile_boundaries(shape):
    g = make_lti_inputs(shape, "slow", "bf16", seed=sum(shape))
    g["lam0"], g["eta0"] = make_initial_state(shape[0], shape[1], shape[3], random=True,
                                              seed=sum(shape))
    full_parity(g, TOL_BF16, "bf16 %s" % (shape,))


def test_lti_matches_general_scan():
    """The same problem through kla_scan_fwd with the gates materialised."""
    from linear_attention_sequence_kla_amd import scan_fwd
    shape = (2, 4, 600, 64)
    g = make_lti_inputs(shape, "slow", "f32", seed=8)
    g["lam0"], g["eta0"] = make_initial_state(2, 4, 64, random=True, seed=8)
    lam, eta = run_gpu(g)
    full = {n: g[n][None, :, None, :].expand(shape).contiguous().to(DEV)
            for n in ("a", "p", "phi")}
    lam2, eta2 = scan_fwd(full["a"], full["p"], full["phi"], g["b"].to(DEV),
                          g["lam0"].to(DEV), g["eta0"].to(DEV))
    torch.cuda.synchronize(DEV)
    assert torch.equal(lam, lam2)
    assert torch.allclose(eta, eta2, rtol=1e-6, atol=1e-6)


def test_lti_stationary_convolution():
    """From the stationary precision the output is the FFT convolution of b
    with f*^j (plus f*^t eta0) and the precision stays lam*."""
    B, H, T, D = 1, 2, 4096, 64
    g = make_lti_inputs((B, H, T, D), "std", "f32", seed=31)
    a, p, phi = (g[n].double().numpy() for n in ("a", "p", "phi"))
    c = 1.0 + p * phi - a * a
    lam_star = (c + np.sqrt(c * c + 4.0 * p * a * a * phi)) / (2.0 * p)
    f_star = a / (a * a + p * lam_star)
    g["lam0"] = torch.tensor(lam_star[None], dtype=torch.float32)
    g["eta0"] = torch.zeros((B, H, D), dtype=torch.float32)
    # start exactly at the float32 value of lam*
    lam_star32 = g["lam0"].double().numpy()[0]
    lam, eta = run_gpu(g)
    lam, eta = lam.cpu().double().numpy()[0], eta.cpu().double().numpy()[0]
    b = g["b"].double().numpy()[0]
    n = 1 << (2 * T - 1).bit_length()
    j = np.arange(T)
    for h in range(H):
        np.testing.assert_allclose(lam[h], np.broadcast_to(lam_star32[h], (T, D)), rtol=1e-5)
        kern = f_star[h][None, :] ** j[:, None]
        ref = np.fft.irfft(np.fft.rfft(b[h], n=n, axis=0) * np.fft.rfft(kern, n=n, axis=0),
                           n=n, axis=0)[:T]
        mag = np.fft.irfft(np.fft.rfft(np.abs(b[h]), n=n, axis=0) *
                           np.fft.rfft(kern, n=n, axis=0), n=n, axis=0)[:T]
        err = np.abs(eta[h] - ref) / mag
        _say("head %d: max scaled error %.3g" % (h, err.max()))
        assert err.max() < 1e-4


def test_lti_argument_errors_on_device():
    from linear_attention_sequence_kla_amd import scan_lti_fwd
    g = {n: v.to(DEV) for n, v in make_lti_inputs((1, 2, 8, 4), "std", "f32", seed=1).items()}
    with pytest.raises(ValueError):
        scan_lti_fwd(g["a"][:1].contiguous(), g["p"], g["phi"], g["b"])
    with pytest.raises(ValueError):
        scan_lti_fwd(g["a"], g["p"], g["phi"].double(), g["b"])
    with pytest.raises(ValueError):
        scan_lti_fwd(g["a"], g["p"], g["phi"], g["b"].double())
