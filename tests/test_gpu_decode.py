"""GPU parity of the decode step (kla_decode_step): one token applied to a
running state equals the oracle's one-token filter from that state, and a
scan prefix followed by decode steps continues the oracle's sequence."""

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
