"""GPU parity of the decode steps (kla_decode_step, kla_mixer_decode_step):
one token applied to a running state equals the oracle's one-token filter
(or mixer) from that state, and a scan (mixer) prefix followed by decode
steps continues the oracle's sequence."""

from __future__ import annotations

import pytest
import torch

from kla_inputs import make_gates, make_initial_state
from kla_metric import TOL_BF16, TOL_F32, assert_parity, compare
from oracle import oracle_scan

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.mark.parametrize("fam,dtype", [("std", "f32"), ("slow", "f32"), ("hard", "f32"),
                                       ("std", "bf16")])
def test_decode_one_token(fam, dtype):
    from linear_attention_sequence_kla_amd import decode_step
    B, H, D = 4, 8, 67
    g = make_gates((B, H, 1, D), fam, dtype, seed=31)
    lam0, eta0 = make_initial_state(B, H, D, random=True, seed=31)
    lam, eta = lam0.clone().to(DEV), eta0.clone().to(DEV)
    tok = {k: g[k][:, :, 0].contiguous().to(DEV) for k in ("a", "p", "phi", "b")}
    decode_step(tok["a"], tok["p"], tok["phi"], tok["b"], lam, eta)
    torch.cuda.synchronize(DEV)
    ref = oracle_scan(g["a"], g["p"], g["phi"], g["b"], lam0, eta0)
    rep = compare(lam.cpu()[:, :, None], eta.cpu()[:, :, None], *ref)
    assert_parity(rep, TOL_BF16 if dtype == "bf16" else TOL_F32, "decode %s %s" % (fam, dtype))


def test_decode_continues_scan():
    from linear_attention_sequence_kla_amd import decode_step, scan_fwd
    B, H, T, D = 2, 4, 300, 64
    k = 250
    g = make_gates((B, H, T, D), "std", "f32", seed=41)
    g["lam0"], g["eta0"] = make_initial_state(B, H, D, random=True, seed=41)
    d = {n: v.to(DEV) for n, v in g.items()}
    cut = lambda t, s: t[:, :, s].contiguous()  # noqa: E731
    lam, eta = scan_fwd(*(cut(d[n], slice(0, k)) for n in ("a", "p", "phi", "b")),
                        d["lam0"], d["eta0"])
    state_l = lam[:, :, -1].contiguous()
    state_e = eta[:, :, -1].contiguous()
    outs_l, outs_e = [], []
    for t in range(k, T):
        decode_step(*(cut(d[n], t) for n in ("a", "p", "phi", "b")), state_l, state_e)
        outs_l.append(state_l.clone())
        outs_e.append(state_e.clone())
    torch.cuda.synchronize(DEV)
    lam_ref, eta_ref, eta_abs = oracle_scan(g["a"], g["p"], g["phi"], g["b"], g["lam0"],
                                            g["eta0"])
    got_l = torch.stack(outs_l, 2).cpu()
    got_e = torch.stack(outs_e, 2).cpu()
    rep = compare(got_l, got_e, lam_ref[:, :, k:], eta_ref[:, :, k:], eta_abs[:, :, k:])
    assert_parity(rep, TOL_F32, "scan prefix + decode")


def test_decode_errors():
    from linear_attention_sequence_kla_amd import KlaError, decode_step, library
    x = torch.ones(8, device=DEV)
    with pytest.raises(KlaError):
        decode_step(x, x.clone(), x.clone(), x.clone(), x, torch.ones(8, device=DEV))
    with pytest.raises(ValueError):
        decode_step(x, x.clone(), x.clone(), x.clone(), torch.ones(4, device=DEV),
                    torch.ones(8, device=DEV))
    assert library().kla_decode_step(None, None, None, None, 0, None, None, 0, None) == 0


def _mixer_token_reference(g, lam0, eta0):
    """The oracle's mixer (readout, variance) and its scan form (the state with
    its magnitude) for one token from the state (lam0, eta0)."""
    from oracle import oracle_mixer
    ref = oracle_mixer(g["k"], g["v"], g["lam_v"], g["q"], g["a"], g["p"], lam0, eta0)
    k, v, lv = (g[n].double() for n in ("k", "v", "lam_v"))
    shape = k.shape
    a = g["a"].double()[None, :, None, :].expand(shape)
    p = g["p"].double()[None, :, None, :].expand(shape)
    state = oracle_scan(a, p, k * k * lv, k * lv * v, lam0, eta0)
    return ref, state


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mixer_decode_one_token(dtype):
    from kla_inputs import make_mixer_inputs
    from kla_metric import assert_mixer_parity, compare_mixer
    from linear_attention_sequence_kla_amd import mixer_decode_step
    B, H, D = 3, 5, 67
    g = make_mixer_inputs((B, H, 1, D), dtype, seed=51)
    lam0, eta0 = make_initial_state(B, H, D, random=True, seed=51)
    d = {n: (g[n][:, :, 0] if g[n].dim() == 4 else g[n]).contiguous().to(DEV) for n in g}
    lam, eta = lam0.clone().to(DEV), eta0.clone().to(DEV)
    out, var, _, _ = mixer_decode_step(d["k"], d["v"], d["lam_v"], d["q"], d["a"], d["p"],
                                       lam, eta)
    torch.cuda.synchronize(DEV)
    ref, state = _mixer_token_reference(g, lam0, eta0)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    assert_mixer_parity(compare_mixer(out.cpu()[:, :, None], var.cpu()[:, :, None], g["q"],
                                      ref["out"], ref["var"], ref["mu_abs"]), tol,
                        "mixer decode %s" % dtype)
    assert_parity(compare(lam.cpu()[:, :, None], eta.cpu()[:, :, None], *state), tol,
                  "mixer decode state %s" % dtype)


def test_mixer_decode_continues_mixer():
    """kla_mixer_fwd over a prefix, then decode steps from its final state,
    follow the oracle's mixer over the whole sequence."""
    from kla_inputs import make_mixer_inputs
    from kla_metric import assert_mixer_parity, compare_mixer
    from linear_attention_sequence_kla_amd import mixer_decode_step, mixer_fwd
    from oracle import oracle_mixer
    B, H, T, D = 2, 3, 300, 48
    k0 = 260
    g = make_mixer_inputs((B, H, T, D), "f32", seed=52)
    g["lam0"], g["eta0"] = make_initial_state(B, H, D, random=True, seed=52)
    d = {n: v.to(DEV) for n, v in g.items()}
    cut = lambda t, s: t[:, :, s].contiguous()  # noqa: E731
    tok = ("k", "v", "lam_v", "q")
    _, _, lam, eta = mixer_fwd(*(cut(d[n], slice(0, k0)) for n in tok), d["a"], d["p"],
                               d["lam0"], d["eta0"], want_state=True)
    outs, vars_ = [], []
    for t in range(k0, T):
        out, var, _, _ = mixer_decode_step(*(cut(d[n], t) for n in tok), d["a"], d["p"], lam, eta)
        outs.append(out.clone())
        vars_.append(var.clone())
    torch.cuda.synchronize(DEV)
    ref = oracle_mixer(g["k"], g["v"], g["lam_v"], g["q"], g["a"], g["p"], g["lam0"], g["eta0"])
    rep = compare_mixer(torch.stack(outs, 2).cpu(), torch.stack(vars_, 2).cpu(),
                        g["q"][:, :, k0:], ref["out"][:, :, k0:], ref["var"][:, :, k0:],
                        ref["mu_abs"][:, :, k0:])
    assert_mixer_parity(rep, TOL_F32, "mixer prefix + decode")


def test_mixer_decode_errors():
    from linear_attention_sequence_kla_amd import KlaError, library, mixer_decode_step
    x = torch.ones((2, 3, 4), device=DEV)
    a = torch.full((3, 4), 0.9, device=DEV)
    with pytest.raises(ValueError):  # channel gates of the wrong shape
        mixer_decode_step(x, x.clone(), x.clone(), x.clone(), a[:2].contiguous(), a,
                          x.clone(), x.clone())
    with pytest.raises(KlaError):  # the state overlaps the readout
        lam = torch.ones((2, 3, 4), device=DEV)
        mixer_decode_step(x, x.clone(), x.clone(), x.clone(), a, a.clone(), lam,
                          torch.ones_like(lam), out=lam)
    assert library().kla_mixer_decode_step(None, None, None, None, 0, None, None, None, None,
                                           None, None, 0, 4, None) == 0
