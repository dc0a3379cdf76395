"""GPU parity of the backward scan (kla_scan_bwd, through the C ABI and the
autograd Function) against the float64 backward oracle.

The oracle differentiates the exact float64 filter; the kernel uses the
forward outputs (float32) as its states, so the bar is the same 1e-4 (2e-2
for bf16 gates) on errors scaled by each gradient's cancellation-free
magnitude.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from kla_inputs import WORKLOADS, make_gates, make_initial_state, make_workload
from kla_metric import TOL_BF16, TOL_F32, assert_grad_parity, compare_grads
from oracle import oracle_scan_bwd

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)


def upstream(shape, seed, device="cpu"):
    gen = torch.Generator(device=device)
    gen.manual_seed(seed + 4242)
    return (torch.randn(shape, generator=gen, device=device),
            torch.randn(shape, generator=gen, device=device))


def gpu_grads(g, g_lam, g_eta, use_state=True):
    from linear_attention_sequence_kla_amd import scan_bwd, scan_fwd
    d = {k: v.to(DEV) for k, v in g.items()}
    lam0 = d["lam0"] if use_state else None
    eta0 = d["eta0"] if use_state else None
    lam, eta = scan_fwd(d["a"], d["p"], d["phi"], d["b"], lam0, eta0)
    out = scan_bwd(d["a"], d["p"], lam, eta,
                   None if g_lam is None else g_lam.to(DEV),
                   None if g_eta is None else g_eta.to(DEV), lam0, eta0)
    torch.cuda.synchronize(DEV)
    names = ("a", "p", "phi", "b", "lam0", "eta0")
    return dict(zip(names, (x.cpu() for x in out))), lam, eta


def oracle_grads(g, g_lam, g_eta):
    zero = np.zeros(g["a"].shape)
    return oracle_scan_bwd(g["a"], g["p"], g["phi"], g["b"], g["lam0"], g["eta0"],
                           zero if g_lam is None else g_lam, zero if g_eta is None else g_eta)


def health():
    from linear_attention_sequence_kla_amd import get_workspace, workspace_health
    return workspace_health(get_workspace(0, DEV, torch.cuda.current_stream(DEV)))


SHAPES = [
    (1, 1, 1, 1, "std", "f32"),
    (1, 1, 113, 1, "std", "f32"),       # one row past one backward tile
    (2, 3, 1000, 7, "std", "f32"),
    (3, 2, 517, 100, "slow", "f32"),
    (1, 2, 333, 64, "hard", "f32"),
    (2, 2, 300, 128, "std", "bf16"),
    (1, 1, 2500, 65, "slow", "bf16"),
    (3, 3, 700, 128, "std", "f32"),     # row halves paired per XCD, partial last block
    (2, 5, 300, 256, "slow", "bf16"),
    (2, 1, 112, 40, "std", "f32"),      # exactly one backward tile (14 rows x 8 waves)
    (1, 3, 14, 9, "hard", "f32"),       # exactly one wave's rows
    (2, 2, 15, 3, "std", "bf16"),       # one row into a second wave, bf16
    (1, 1, 225, 64, "slow", "f32"),     # one row into a third tile
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s[:4])) + s[4] + s[5])
def test_backward_shapes(shape):
    B, H, T, D, fam, dtype = shape
    _say("backward shape %s" % (shape,))
    g = make_gates((B, H, T, D), fam, dtype, seed=B * 7 + T)
    g["lam0"], g["eta0"] = make_initial_state(B, H, D, random=True, seed=T)
    g_lam, g_eta = upstream((B, H, T, D), T)
    got, lam, eta = gpu_grads(g, g_lam, g_eta)
    assert health() == 0
    grads, mags = oracle_grads(g, g_lam, g_eta)
    # gradients are specified where the forward outputs of the channel are
    # finite (they are the backward's states); compare those channels
    ok = (torch.isfinite(lam) & torch.isfinite(eta)).all(dim=2).cpu().numpy()  # [B, H, D]
    assert ok.any()
    if not ok.all():
        _say("%d of %d channels overflowed in the forward pass" % ((~ok).sum(), ok.size))
        sel4 = np.broadcast_to(ok[:, :, None, :], g["a"].shape)
        for dct in (got, grads, mags):
            for k in list(dct):
                v = np.asarray(dct[k].numpy() if hasattr(dct[k], "numpy") else dct[k])
                dct[k] = v[sel4] if v.ndim == 4 else v[ok]
    rep = compare_grads(got, grads, mags)
    _say("%s: %s" % (shape, rep))
    assert_grad_parity(rep, TOL_BF16 if dtype == "bf16" else TOL_F32, str(shape))


@pytest.mark.parametrize("key", [0, 1])
def test_backward_workload_full(key):
    w = WORKLOADS[key]
    _say("backward workload %s" % w.describe())
    g = make_workload(key, device="cpu")
    g_lam, g_eta = upstream(w.shape, key)
    got, _, _ = gpu_grads(g, g_lam, g_eta)
    assert health() == 0
    grads, mags = oracle_grads(g, g_lam, g_eta)
    rep = compare_grads(got, grads, mags)
    _say("%s: %s" % (w.describe(), rep))
    assert_grad_parity(rep, TOL_F32, w.describe())


def _gather(x, D, q):
    B, H, T, _ = x.shape
    flat = x.reshape(B * H, T, D)
    slab = torch.as_tensor(q // D, device=x.device)
    d = torch.as_tensor(q % D, device=x.device)
    return flat[slab, :, d].transpose(0, 1).reshape(1, 1, T, len(q)).contiguous()


@pytest.mark.parametrize("key", [4])
def test_backward_workload_sampled(key):
    """Full-size backward launch on the hard gates; the oracle checks whole
    sampled channels whose forward outputs stay finite (this entry point
    takes its states from the float32 outputs; the backward from float64
    states covers every channel)."""
    from linear_attention_sequence_kla_amd import scan_bwd, scan_fwd
    w = WORKLOADS[key]
    _say("backward workload %s (sampled channels)" % w.describe())
    g = make_workload(key, device=DEV)
    g_lam, g_eta = upstream(w.shape, key, device=DEV)
    lam, eta = scan_fwd(g["a"], g["p"], g["phi"], g["b"], g["lam0"], g["eta0"])
    out = scan_bwd(g["a"], g["p"], lam, eta, g_lam, g_eta, g["lam0"], g["eta0"])
    torch.cuda.synchronize(DEV)
    assert health() == 0
    finite = (torch.isfinite(lam) & torch.isfinite(eta)).all(dim=2).reshape(-1)
    cand = np.nonzero(finite.cpu().numpy())[0]
    rng = np.random.default_rng(key)
    q = np.sort(rng.choice(cand, size=min(256, len(cand)), replace=False))
    gs = {k: _gather(g[k], w.D, q).cpu() for k in ("a", "p", "phi", "b")}
    sel = torch.as_tensor(q, device=DEV)
    gs["lam0"] = g["lam0"].reshape(-1)[sel].reshape(1, 1, -1).cpu()
    gs["eta0"] = g["eta0"].reshape(-1)[sel].reshape(1, 1, -1).cpu()
    grads, mags = oracle_grads(gs, _gather(g_lam, w.D, q).cpu(), _gather(g_eta, w.D, q).cpu())
    names = ("a", "p", "phi", "b")
    got = {k: _gather(v, w.D, q).cpu() for k, v in zip(names, out[:4])}
    got["lam0"] = out[4].reshape(-1)[sel].reshape(1, 1, -1).cpu()
    got["eta0"] = out[5].reshape(-1)[sel].reshape(1, 1, -1).cpu()
    rep = compare_grads(got, grads, mags)
    _say("%s: %s" % (w.describe(), rep))
    assert_grad_parity(rep, TOL_BF16 if w.dtype == "bf16" else TOL_F32, w.describe())


@pytest.mark.parametrize("key", [2, 3])
def test_backward_workload_every_element(key):
    """kla_scan_bwd at full size in the benchmark's launch, from the float32
    outputs of the forward call (finite everywhere on these gates); every
    gradient element against the oracle, a batch of slabs at a time."""
    from linear_attention_sequence_kla_amd import scan_bwd, scan_fwd
    w = WORKLOADS[key]
    _say("backward workload %s (every element)" % w.describe())
    g = make_workload(key, device=DEV)
    g_lam, g_eta = upstream(w.shape, key, device=DEV)
    lam, eta = scan_fwd(g["a"], g["p"], g["phi"], g["b"], g["lam0"], g["eta0"])
    out = scan_bwd(g["a"], g["p"], lam, eta, g_lam, g_eta, g["lam0"], g["eta0"])
    torch.cuda.synchronize(DEV)
    assert health() == 0
    assert bool(torch.isfinite(lam).all()) and bool(torch.isfinite(eta).all())
    del lam, eta
    got = dict(zip(("a", "p", "phi", "b", "lam0", "eta0"), out))
    rep = compare_grads_by_slabs(g, g_lam, g_eta, got, w.shape)
    _say("%s: %s" % (w.describe(), rep))
    assert_grad_parity(rep, TOL_BF16 if w.dtype == "bf16" else TOL_F32, w.describe())
    del g, g_lam, g_eta, out, got
    torch.cuda.empty_cache()


def test_backward_largest_offsets():
    """The backward pass at the largest per-wave address span the library
    accepts (D = 1: a wave's 64 channels in 64 slabs of T tokens, 63 T just
    under 2^30); the oracle checks whole channels including the farthest."""
    from linear_attention_sequence_kla_amd import scan_bwd, scan_fwd
    B, H, T, D = 8, 8, 17_000_000, 1
    _say("backward, largest offsets %s" % ((B, H, T, D),))
    g = make_gates((B, H, T, D), "std", "f32", seed=78, device=DEV)
    g["lam0"], g["eta0"] = make_initial_state(B, H, D, random=True, seed=78, device=DEV)
    g_lam, g_eta = upstream((B, H, T, D), 78, device=DEV)
    lam, eta = scan_fwd(g["a"], g["p"], g["phi"], g["b"], g["lam0"], g["eta0"])
    out = scan_bwd(g["a"], g["p"], lam, eta, g_lam, g_eta, g["lam0"], g["eta0"])
    torch.cuda.synchronize(DEV)
    assert health() == 0
    q = np.array([0, 1, 31, 62, 63])
    gs = {k: _gather(g[k], D, q).cpu() for k in ("a", "p", "phi", "b")}
    sel = torch.as_tensor(q, device=DEV)
    gs["lam0"] = g["lam0"].reshape(-1)[sel].reshape(1, 1, -1).cpu()
    gs["eta0"] = g["eta0"].reshape(-1)[sel].reshape(1, 1, -1).cpu()
    grads, mags = oracle_grads(gs, _gather(g_lam, D, q).cpu(), _gather(g_eta, D, q).cpu())
    got = {k: _gather(v, D, q).cpu() for k, v in zip(("a", "p", "phi", "b"), out[:4])}
    got["lam0"] = out[4].reshape(-1)[sel].reshape(1, 1, -1).cpu()
    got["eta0"] = out[5].reshape(-1)[sel].reshape(1, 1, -1).cpu()
    rep = compare_grads(got, grads, mags)
    _say("backward, largest offsets: %s" % rep)
    assert_grad_parity(rep, TOL_F32, "backward, largest offsets")
    del g, g_lam, g_eta, lam, eta, out
    torch.cuda.empty_cache()


def test_null_upstream_and_no_state_grads():
    """g_eta = NULL means zero; g_lam0/g_eta0 may be skipped."""
    from linear_attention_sequence_kla_amd import scan_bwd, scan_fwd
    g = make_gates((2, 2, 400, 40), "std", "f32", seed=5)
    g["lam0"], g["eta0"] = make_initial_state(2, 2, 40, random=True, seed=5)
    g_lam, _ = upstream((2, 2, 400, 40), 5)
    got, _, _ = gpu_grads(g, g_lam, None)
    grads, mags = oracle_grads(g, g_lam, None)
    assert_grad_parity(compare_grads(got, grads, mags), TOL_F32, "g_eta=None")
    d = {k: v.to(DEV) for k, v in g.items()}
    lam, eta = scan_fwd(d["a"], d["p"], d["phi"], d["b"], d["lam0"], d["eta0"])
    out = scan_bwd(d["a"], d["p"], lam, eta, g_lam.to(DEV), None, d["lam0"], d["eta0"],
                   need_state_grads=False)
    torch.cuda.synchronize(DEV)
    assert out[4] is None and out[5] is None
    assert torch.equal(out[0].cpu(), got["a"])


def test_autograd_function_and_segments():
    """The autograd Function matches the oracle, and gradients through two
    chained segments (the carry passed as lam0/eta0) equal one call's."""
    from linear_attention_sequence_kla_amd import kla_scan
    shape = (2, 2, 900, 64)
    g = make_gates(shape, "std", "f32", seed=21)
    g["lam0"], g["eta0"] = make_initial_state(2, 2, 64, random=True, seed=21)
    g_lam, g_eta = upstream(shape, 21)

    def leaves():
        return {k: g[k].to(DEV).clone().requires_grad_(True) for k in g}

    x = leaves()
    lam, eta = kla_scan(x["a"], x["p"], x["phi"], x["b"], x["lam0"], x["eta0"])
    ((lam * g_lam.to(DEV)).sum() + (eta * g_eta.to(DEV)).sum()).backward()
    got = {k: x[k].grad.cpu() for k in x}
    grads, mags = oracle_grads(g, g_lam, g_eta)
    assert_grad_parity(compare_grads(got, grads, mags), TOL_F32, "autograd")

    y = leaves()
    k = 377
    cut = lambda t, s: t[:, :, s].contiguous()  # noqa: E731
    l1, e1 = kla_scan(*(cut(y[n], slice(0, k)) for n in ("a", "p", "phi", "b")),
                      y["lam0"], y["eta0"])
    l2, e2 = kla_scan(*(cut(y[n], slice(k, None)) for n in ("a", "p", "phi", "b")),
                      l1[:, :, -1].contiguous(), e1[:, :, -1].contiguous())
    lam_s = torch.cat([l1, l2], 2)
    eta_s = torch.cat([e1, e2], 2)
    ((lam_s * g_lam.to(DEV)).sum() + (eta_s * g_eta.to(DEV)).sum()).backward()
    seg = {k: y[k].grad.cpu() for k in y}
    assert_grad_parity(compare_grads(seg, grads, mags), TOL_F32, "segmented autograd")


def test_backward_argument_errors():
    from linear_attention_sequence_kla_amd import KlaError, scan_bwd
    g = make_gates((1, 2, 100, 8), "std", "f32", seed=3)
    d = {k: v.to(DEV) for k, v in g.items()}
    small = torch.zeros(64, dtype=torch.uint8, device=DEV)
    with pytest.raises(KlaError) as e:
        scan_bwd(d["a"], d["p"], d["a"].clone(), d["a"].clone(), None, None, workspace=small)
    assert e.value.name == "KLA_ERR_WORKSPACE"
    with pytest.raises(ValueError):
        scan_bwd(d["a"], d["p"], None, d["a"].clone(), None, None)


# ---------------------------------------------------------------------------
# The backward pass from float64 states (kla_scan_fwd_states /
# kla_scan_bwd_states): defined on the whole domain, so every channel is
# compared, also where lam or eta overflow float32 (hard gates).

STATE_SHAPES = SHAPES + [
    (2, 3, 8, 5, "hard", "f32"),        # exactly one state block
    (1, 2, 9, 7, "hard", "bf16"),       # one row past a state block
    (2, 1, 64, 9, "hard", "f32"),       # exactly one backward tile (8 rows x 8 waves)
    (2, 1, 65, 9, "std", "f32"),        # one row into a second tile
    (1, 3, 129, 40, "hard", "f32"),
    (4, 2, 600, 32, "hard", "f32"),     # hard gates: lam overflows float32 in places
    (2, 1, 32, 9, "std", "f32"),        # exactly one short-sequence tile (8 rows x 4 waves)
    (2, 1, 33, 9, "hard", "bf16"),      # one row into a second one
    (1, 1, 8191, 5, "slow", "f32"),     # the longest sequence with 4-wave tiles
    (1, 2, 8192, 70, "hard", "f32"),    # the first with 8-wave tiles
    (1, 1, 8200, 64, "std", "bf16"),
]


def _bwd_states(g, g_lam, g_eta, keep_states):
    from linear_attention_sequence_kla_amd import scan_bwd_states, scan_fwd_states
    d = {k: v.to(DEV) for k, v in g.items()}
    states = None
    if keep_states:
        _, _, states = scan_fwd_states(d["a"], d["p"], d["phi"], d["b"], d["lam0"], d["eta0"])
    out = scan_bwd_states(d["a"], d["p"], d["phi"], d["b"],
                          None if g_lam is None else g_lam.to(DEV),
                          None if g_eta is None else g_eta.to(DEV), d["lam0"], d["eta0"],
                          states=states)
    torch.cuda.synchronize(DEV)
    return dict(zip(("a", "p", "phi", "b", "lam0", "eta0"), out))


@pytest.mark.parametrize("shape", STATE_SHAPES,
                         ids=lambda s: "x".join(map(str, s[:4])) + s[4] + s[5])
def test_backward_states_shapes(shape):
    """Every channel, hard gates included; kept states and recomputed states
    give identical bits."""
    B, H, T, D, fam, dtype = shape
    _say("backward from states, shape %s" % (shape,))
    g = make_gates((B, H, T, D), fam, dtype, seed=B * 11 + T)
    g["lam0"], g["eta0"] = make_initial_state(B, H, D, random=True, seed=T + 1)
    g_lam, g_eta = upstream((B, H, T, D), T + 1)
    kept = _bwd_states(g, g_lam, g_eta, keep_states=True)
    again = _bwd_states(g, g_lam, g_eta, keep_states=False)
    assert health() == 0
    for k in kept:
        assert torch.equal(kept[k], again[k]), k
    grads, mags = oracle_grads(g, g_lam, g_eta)
    rep = compare_grads({k: v.cpu() for k, v in kept.items()}, grads, mags)
    _say("%s: %s" % (shape, rep))
    assert_grad_parity(rep, TOL_BF16 if dtype == "bf16" else TOL_F32, str(shape))


def compare_grads_by_slabs(g, g_lam, g_eta, got, shape, max_elements=1 << 23):
    """Every gradient element against the backward oracle, a batch of (b, h)
    slabs at a time (inputs copied to the host per batch)."""
    B, H, T, D = shape
    S = B * H
    per = max(1, min(S, max_elements // max(1, T * D)))
    rep = {"nan": 0, "range_violations": 0}
    for s0 in range(0, S, per):
        s1 = min(S, s0 + per)

        def cut(x):
            return x.reshape(S, T, D)[s0:s1].cpu().reshape(1, s1 - s0, T, D)

        def cut3(x):
            return x.reshape(S, D)[s0:s1].cpu().reshape(1, s1 - s0, D)

        host = {k: cut(g[k]) for k in ("a", "p", "phi", "b")}
        host["lam0"], host["eta0"] = cut3(g["lam0"]), cut3(g["eta0"])
        grads, mags = oracle_grads(host, cut(g_lam), cut(g_eta))
        mine = {k: cut(got[k]) for k in ("a", "p", "phi", "b")}
        mine["lam0"], mine["eta0"] = cut3(got["lam0"]), cut3(got["eta0"])
        r = compare_grads(mine, grads, mags)
        for k, v in r.items():
            rep[k] = rep.get(k, 0) + v if k in ("nan", "range_violations") else max(
                rep.get(k, 0.0), v)
        del host, grads, mags, mine
    return rep


@pytest.mark.parametrize("key", [0, 1, 2, 3, 4])
def test_backward_states_workload_every_element(key):
    """A workload at full size, drawn on the GPU as the benchmark draws it,
    through the training pair (forward keeping the states, backward from
    them); every gradient element of every channel against the oracle."""
    from linear_attention_sequence_kla_amd import scan_bwd_states, scan_fwd_states
    w = WORKLOADS[key]
    _say("backward from states, workload %s (every element)" % w.describe())
    g = make_workload(key, device=DEV)
    g_lam, g_eta = upstream(w.shape, key, device=DEV)
    _, _, states = scan_fwd_states(g["a"], g["p"], g["phi"], g["b"], g["lam0"], g["eta0"])
    out = scan_bwd_states(g["a"], g["p"], g["phi"], g["b"], g_lam, g_eta, g["lam0"], g["eta0"],
                          states=states)
    torch.cuda.synchronize(DEV)
    assert health() == 0
    del states
    got = dict(zip(("a", "p", "phi", "b", "lam0", "eta0"), out))
    rep = compare_grads_by_slabs(g, g_lam, g_eta, got, w.shape)
    _say("%s: %s" % (w.describe(), rep))
    assert_grad_parity(rep, TOL_BF16 if w.dtype == "bf16" else TOL_F32, w.describe())
    del g, g_lam, g_eta, out, got
    torch.cuda.empty_cache()


def test_autograd_hard_gates_every_channel():
    """The autograd Function (forward keeping states, backward from them) on
    hard gates whose forward outputs overflow float32 in places: every
    channel matches the oracle."""
    from linear_attention_sequence_kla_amd import kla_scan
    shape = (8, 4, 2048, 32)
    g = make_gates(shape, "hard", "f32", seed=44)
    g["lam0"], g["eta0"] = make_initial_state(8, 4, 32, random=True, seed=44)
    g_lam, g_eta = upstream(shape, 44)
    x = {k: g[k].to(DEV).clone().requires_grad_(True) for k in g}
    lam, eta = kla_scan(x["a"], x["p"], x["phi"], x["b"], x["lam0"], x["eta0"])
    assert not bool(torch.isfinite(lam).all())  # the overflow case is exercised
    # one backward pass for both outputs (the gradient of
    # sum(g_lam * lam + g_eta * eta)): two separate passes would add two
    # float32 results that can overflow with opposite signs where their sum
    # does not
    torch.autograd.backward([lam, eta], [g_lam.to(DEV), g_eta.to(DEV)])
    torch.cuda.synchronize(DEV)
    got = {k: x[k].grad.cpu() for k in x}
    grads, mags = oracle_grads(g, g_lam, g_eta)
    rep = compare_grads(got, grads, mags)
    _say("autograd, hard gates: %s" % rep)
    assert_grad_parity(rep, TOL_F32, "autograd, hard gates")


def test_backward_states_argument_errors():
    from linear_attention_sequence_kla_amd import KlaError, scan_bwd_states, scan_fwd_states
    g = make_gates((1, 2, 100, 8), "std", "f32", seed=3)
    d = {k: v.to(DEV) for k, v in g.items()}
    small = torch.zeros(64, dtype=torch.uint8, device=DEV)
    with pytest.raises(KlaError) as e:
        scan_bwd_states(d["a"], d["p"], d["phi"], d["b"], None, None, workspace=small)
    assert e.value.name == "KLA_ERR_WORKSPACE"
    with pytest.raises(ValueError):  # states of the wrong shape
        scan_bwd_states(d["a"], d["p"], d["phi"], d["b"], None, None,
                        states=torch.zeros((3, 16, 2), dtype=torch.float64, device=DEV))
    with pytest.raises(KlaError) as e:  # states overlapping an output
        lam = torch.empty((1, 2, 100, 8), device=DEV)
        scan_fwd_states(d["a"], d["p"], d["phi"], d["b"], out=(lam, torch.empty_like(lam)),
                        states=lam.view(torch.float64).reshape(-1)[:13 * 16 * 2].reshape(13, 16, 2))
    assert e.value.name == "KLA_ERR_INVALID_ARG"
