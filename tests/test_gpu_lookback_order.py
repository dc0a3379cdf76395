"""The carry protocol under adversarial timing.  libkla_debug.so is libkla
built with a pseudo-random pause (0 to ~50 microseconds) before every carry
flag is published, so tiles meet their predecessors in every state -- not yet
published, aggregate only, inclusive late -- and walk back over several
tiles.  Every entry point that scans must still match the oracle.  (The
pauses are bounded and every wait is bounded, so the kernels always end.)"""

from __future__ import annotations

import os

import numpy as np
import pytest
import torch

from kla_inputs import (broadcast_lti, make_gates, make_initial_state, make_lti_inputs,
                        make_mixer_inputs)
from kla_metric import (TOL_F32, assert_grad_parity, assert_mixer_parity, assert_parity,
                        compare, compare_grads, compare_mixer)
from oracle import oracle_mixer, oracle_mixer_bwd, oracle_scan, oracle_scan_bwd

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
# a few columns with long chains of tiles, and many columns
SHAPES = [(1, 2, 9000, 64), (2, 2, 3000, 96), (3, 3, 2000, 128),
          (1, 1, 70000, 64)]  # the tall tiles of long sequences


@pytest.fixture
def debug_build(monkeypatch):
    from linear_attention_sequence_kla_amd import kla
    lib = kla.load_library(os.path.join(kla.HERE, "libkla_debug.so"))
    monkeypatch.setattr(kla, "_lib", lib)
    monkeypatch.setattr(kla, "_workspaces", {})
    yield lib


def _health():
    from linear_attention_sequence_kla_amd import get_workspace, workspace_health
    return workspace_health(get_workspace(0, DEV, torch.cuda.current_stream(DEV)))


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_scan_forward_and_backward(debug_build, shape):
    from linear_attention_sequence_kla_amd import scan_bwd, scan_fwd
    B, H, T, D = shape
    g = make_gates(shape, "std", "f32", seed=T)
    g["lam0"], g["eta0"] = make_initial_state(B, H, D, random=True, seed=T)
    d = {n: v.to(DEV) for n, v in g.items()}
    for _ in range(2):  # twice: the second call runs on a reused workspace
        lam, eta = scan_fwd(d["a"], d["p"], d["phi"], d["b"], d["lam0"], d["eta0"])
        torch.cuda.synchronize(DEV)
    assert _health() == 0
    ref = oracle_scan(g["a"], g["p"], g["phi"], g["b"], g["lam0"], g["eta0"])
    assert_parity(compare(lam.cpu(), eta.cpu(), *ref), TOL_F32, "forward %s" % (shape,))

    gen = torch.Generator().manual_seed(3)
    g_lam, g_eta = torch.randn(shape, generator=gen), torch.randn(shape, generator=gen)
    out = scan_bwd(d["a"], d["p"], lam, eta, g_lam.to(DEV), g_eta.to(DEV), d["lam0"], d["eta0"])
    torch.cuda.synchronize(DEV)
    assert _health() == 0
    grads, mags = oracle_scan_bwd(g["a"], g["p"], g["phi"], g["b"], g["lam0"], g["eta0"],
                                  g_lam, g_eta)
    got = dict(zip(("a", "p", "phi", "b", "lam0", "eta0"), (t.cpu() for t in out)))
    assert_grad_parity(compare_grads(got, grads, mags), TOL_F32, "backward %s" % (shape,))

    # the training pair: forward keeping float64 states, backward from them
    from linear_attention_sequence_kla_amd import scan_bwd_states, scan_fwd_states
    _, _, states = scan_fwd_states(d["a"], d["p"], d["phi"], d["b"], d["lam0"], d["eta0"])
    out = scan_bwd_states(d["a"], d["p"], d["phi"], d["b"], g_lam.to(DEV), g_eta.to(DEV),
                          d["lam0"], d["eta0"], states=states)
    torch.cuda.synchronize(DEV)
    assert _health() == 0
    got = dict(zip(("a", "p", "phi", "b", "lam0", "eta0"), (t.cpu() for t in out)))
    assert_grad_parity(compare_grads(got, grads, mags), TOL_F32,
                       "backward from states %s" % (shape,))


@pytest.mark.parametrize("shape", [(1, 2, 9000, 128), (3, 3, 2000, 256)],
                         ids=lambda s: "x".join(map(str, s)))
def test_scan_forward_bf16(debug_build, shape):
    """bfloat16 gates on whole rows (D = 128) and on paired quarter rows."""
    from kla_metric import TOL_BF16
    from linear_attention_sequence_kla_amd import scan_fwd
    B, H, T, D = shape
    g = make_gates(shape, "std", "bf16", seed=T + 1)
    g["lam0"], g["eta0"] = make_initial_state(B, H, D, random=True, seed=T + 1)
    d = {n: v.to(DEV) for n, v in g.items()}
    for _ in range(2):
        lam, eta = scan_fwd(d["a"], d["p"], d["phi"], d["b"], d["lam0"], d["eta0"])
        torch.cuda.synchronize(DEV)
    assert _health() == 0
    ref = oracle_scan(g["a"], g["p"], g["phi"], g["b"], g["lam0"], g["eta0"])
    assert_parity(compare(lam.cpu(), eta.cpu(), *ref), TOL_BF16, "bf16 forward %s" % (shape,))


@pytest.mark.parametrize("shape", [(1, 2, 9000, 128), (2, 2, 3000, 64)],
                         ids=lambda s: "x".join(map(str, s)))
def test_scan_training_pair_bf16(debug_build, shape):
    """bfloat16 gates through the forward keeping states and the backward
    from them (the backward's bfloat16 tiles: 4 waves, 5 per SIMD)."""
    from kla_metric import TOL_BF16
    from linear_attention_sequence_kla_amd import scan_bwd_states, scan_fwd_states
    B, H, T, D = shape
    g = make_gates(shape, "std", "bf16", seed=T + 2)
    g["lam0"], g["eta0"] = make_initial_state(B, H, D, random=True, seed=T + 2)
    d = {n: v.to(DEV) for n, v in g.items()}
    gen = torch.Generator().manual_seed(11)
    g_lam, g_eta = torch.randn(shape, generator=gen), torch.randn(shape, generator=gen)
    _, _, states = scan_fwd_states(d["a"], d["p"], d["phi"], d["b"], d["lam0"], d["eta0"])
    out = scan_bwd_states(d["a"], d["p"], d["phi"], d["b"], g_lam.to(DEV), g_eta.to(DEV),
                          d["lam0"], d["eta0"], states=states)
    torch.cuda.synchronize(DEV)
    assert _health() == 0
    grads, mags = oracle_scan_bwd(g["a"], g["p"], g["phi"], g["b"], g["lam0"], g["eta0"],
                                  g_lam, g_eta)
    got = dict(zip(("a", "p", "phi", "b", "lam0", "eta0"), (t.cpu() for t in out)))
    assert_grad_parity(compare_grads(got, grads, mags), TOL_BF16, "bf16 training pair")
    assert_grad_parity(compare_grads(got, grads, mags), TOL_F32, "bf16 training pair")


@pytest.mark.parametrize("shape", [(1, 2, 6000, 64), (2, 4, 1500, 128)],
                         ids=lambda s: "x".join(map(str, s)))
def test_mixer_forward_and_backward(debug_build, shape):
    from linear_attention_sequence_kla_amd import mixer_bwd, mixer_fwd, mixer_states_shape
    g = make_mixer_inputs(shape, "f32", seed=4)
    g["lam0"], g["eta0"] = make_initial_state(shape[0], shape[1], shape[3], random=True, seed=4)
    d = {n: v.to(DEV) for n, v in g.items()}
    states = torch.empty(mixer_states_shape(*shape), dtype=torch.float64, device=DEV)
    out, var, _, _ = mixer_fwd(d["k"], d["v"], d["lam_v"], d["q"], d["a"], d["p"], d["lam0"],
                               d["eta0"], states=states)
    torch.cuda.synchronize(DEV)
    assert _health() == 0
    ref = oracle_mixer(g["k"], g["v"], g["lam_v"], g["q"], g["a"], g["p"], g["lam0"], g["eta0"])
    assert_mixer_parity(compare_mixer(out.cpu(), var.cpu(), g["q"], ref["out"], ref["var"],
                                      ref["mu_abs"]), TOL_F32, "mixer forward")
    gen = torch.Generator().manual_seed(5)
    g_out, g_var = torch.randn(shape, generator=gen), torch.randn(shape, generator=gen)
    res = mixer_bwd(d["k"], d["v"], d["lam_v"], d["q"], d["a"], d["p"], g_out.to(DEV),
                    g_var.to(DEV), d["lam0"], d["eta0"])
    torch.cuda.synchronize(DEV)
    assert _health() == 0
    grads, mags = oracle_mixer_bwd(g["k"], g["v"], g["lam_v"], g["q"], g["a"], g["p"],
                                   g["lam0"], g["eta0"], g_out, g_var)
    got = dict(zip(("k", "v", "lam_v", "q", "a", "p", "lam0", "eta0"), (t.cpu() for t in res)))
    assert_grad_parity(compare_grads(got, grads, mags), TOL_F32, "mixer backward")
    # from the states the forward kept: bitwise the same gradients
    kept = mixer_bwd(d["k"], d["v"], d["lam_v"], d["q"], d["a"], d["p"], g_out.to(DEV),
                     g_var.to(DEV), d["lam0"], d["eta0"], states=states)
    torch.cuda.synchronize(DEV)
    assert _health() == 0
    for x, y in zip(res, kept):
        assert torch.equal(x, y)


def test_lti(debug_build):
    from linear_attention_sequence_kla_amd import scan_lti_fwd
    shape = (2, 1, 12000, 64)
    g = make_lti_inputs(shape, "std", "f32", seed=6)
    g["lam0"], g["eta0"] = make_initial_state(2, 1, 64, random=True, seed=6)
    d = {n: v.to(DEV) for n, v in g.items()}
    lam, eta = scan_lti_fwd(d["a"], d["p"], d["phi"], d["b"], d["lam0"], d["eta0"])
    torch.cuda.synchronize(DEV)
    assert _health() == 0
    f = broadcast_lti(g)
    ref = oracle_scan(f["a"], f["p"], f["phi"], f["b"], g["lam0"], g["eta0"])
    assert_parity(compare(lam.cpu(), eta.cpu(), *ref), TOL_F32, "lti")
    assert np.isfinite(lam.cpu().numpy()).all()
