"""Scan launches captured in a HIP graph (torch.cuda.CUDAGraph) replay
correctly: several replays, with eager calls on the same workspace and host
synchronisations between them, each match the eager results and the oracle.
(The kernels keep their epoch in the workspace and record no memset.)"""

from __future__ import annotations

import pytest
import torch

from kla_inputs import make_gates, make_initial_state
from kla_metric import TOL_F32, assert_parity, compare
from oracle import oracle_scan

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def test_graph_replays_match_eager():
    from linear_attention_sequence_kla_amd import (
        bwd_workspace_size, scan_bwd, scan_fwd, workspace_health, workspace_size)
    shape = (2, 4, 1500, 64)
    sets = []
    for k in range(2):
        g = make_gates(shape, "std", "f32", seed=100 + k)
        g["lam0"], g["eta0"] = make_initial_state(2, 4, 64, random=True, seed=100 + k)
        sets.append(g)
    dev = [{n: v.to(DEV) for n, v in g.items()} for g in sets]
    nbytes = max(workspace_size(*shape), bwd_workspace_size(*shape))
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    outs = [(torch.empty(shape, device=DEV), torch.empty(shape, device=DEV)) for _ in sets]
    g_lam = torch.randn(shape, device=DEV)

    # eager reference
    eager = [scan_fwd(d["a"], d["p"], d["phi"], d["b"], d["lam0"], d["eta0"], workspace=ws)
             for d in dev]
    eager_bwd = scan_bwd(dev[0]["a"], dev[0]["p"], eager[0][0], eager[0][1], g_lam, None,
                         dev[0]["lam0"], dev[0]["eta0"], workspace=ws)
    torch.cuda.synchronize(DEV)

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for d, o in zip(dev, outs):
            scan_fwd(d["a"], d["p"], d["phi"], d["b"], d["lam0"], d["eta0"], out=o, workspace=ws)
        gb = scan_bwd(dev[0]["a"], dev[0]["p"], outs[0][0], outs[0][1], g_lam, None,
                      dev[0]["lam0"], dev[0]["eta0"], workspace=ws)
    torch.cuda.synchronize(DEV)

    refs = [oracle_scan(g["a"], g["p"], g["phi"], g["b"], g["lam0"], g["eta0"]) for g in sets]
    for replay in range(3):
        for o in outs:
            o[0].fill_(float("nan"))
            o[1].fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize(DEV)
        for k, (o, e, ref) in enumerate(zip(outs, eager, refs)):
            assert torch.equal(o[0], e[0]) and torch.equal(o[1], e[1]), (replay, k)
            assert_parity(compare(o[0].cpu(), o[1].cpu(), *ref), TOL_F32, "replay %d" % replay)
        for x, y in zip(gb[:4], eager_bwd[:4]):
            assert torch.equal(x, y), replay
        # eager work on the same workspace between replays
        scan_fwd(dev[1]["a"], dev[1]["p"], dev[1]["phi"], dev[1]["b"], workspace=ws)
        torch.cuda.synchronize(DEV)
    assert workspace_health(ws) == 0


def test_graph_replays_mixer_and_lti():
    """The fused mixer and the time-invariant scan captured together in one
    graph on one workspace (kla_mixer_fwd and kla_scan_lti_fwd), replayed
    three times with eager calls in between."""
    from kla_inputs import make_lti_inputs, make_mixer_inputs
    from linear_attention_sequence_kla_amd import (lti_workspace_size, mixer_fwd,
                                                   mixer_workspace_size, scan_lti_fwd,
                                                   workspace_health)
    shape = (2, 3, 900, 40)
    mx = {n: v.to(DEV) for n, v in make_mixer_inputs(shape, "f32", seed=41).items()}
    lt = {n: v.to(DEV) for n, v in make_lti_inputs(shape, "std", "f32", seed=42).items()}
    nbytes = max(mixer_workspace_size(*shape), lti_workspace_size(*shape))
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    outs = [torch.empty(shape, device=DEV) for _ in range(4)]
    e_out, e_var, _, _ = mixer_fwd(mx["k"], mx["v"], mx["lam_v"], mx["q"], mx["a"], mx["p"],
                                   workspace=ws)
    e_lam, e_eta = scan_lti_fwd(lt["a"], lt["p"], lt["phi"], lt["b"], workspace=ws)
    torch.cuda.synchronize(DEV)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mixer_fwd(mx["k"], mx["v"], mx["lam_v"], mx["q"], mx["a"], mx["p"], out=outs[0],
                  var=outs[1], workspace=ws)
        scan_lti_fwd(lt["a"], lt["p"], lt["phi"], lt["b"], out=(outs[2], outs[3]), workspace=ws)
    torch.cuda.synchronize(DEV)
    for replay in range(3):
        for o in outs:
            o.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize(DEV)
        # bitwise: every look-back path gives the same carry (see test_gpu_determinism)
        for got, want in zip(outs, (e_out, e_var, e_lam, e_eta)):
            assert torch.equal(got, want), replay
        scan_lti_fwd(lt["a"], lt["p"], lt["phi"], lt["b"], workspace=ws)
        torch.cuda.synchronize(DEV)
    assert workspace_health(ws) == 0


def test_graph_replays_mixer_training_step():
    """A mixer training step -- kla_mixer_fwd keeping its states, kla_mixer_bwd
    from them -- and a recomputing kla_mixer_bwd, captured in one graph on one
    workspace and replayed three times with eager calls in between; every
    replay equals the eager results bit for bit."""
    from linear_attention_sequence_kla_amd import (mixer_bwd, mixer_bwd_workspace_size,
                                                   mixer_fwd, mixer_states_shape,
                                                   workspace_health)
    from kla_inputs import make_initial_state, make_mixer_inputs
    shape = (2, 2, 700, 48)
    mx = {n: v.to(DEV) for n, v in make_mixer_inputs(shape, "f32", seed=43).items()}
    lam0, eta0 = (x.to(DEV) for x in make_initial_state(2, 2, 48, random=True, seed=43))
    gen = torch.Generator(device=DEV).manual_seed(44)
    g_out = torch.randn(shape, generator=gen, device=DEV)
    g_var = torch.randn(shape, generator=gen, device=DEV)
    ws = torch.zeros(mixer_bwd_workspace_size(*shape), dtype=torch.uint8, device=DEV)
    tok = (mx["k"], mx["v"], mx["lam_v"], mx["q"], mx["a"], mx["p"])

    def grads_out():
        return tuple(torch.empty(shape, device=DEV) for _ in range(4)) + tuple(
            torch.empty((2, 48), device=DEV) for _ in range(2))

    states = torch.empty(mixer_states_shape(*shape), dtype=torch.float64, device=DEV)
    e_out, e_var, _, _ = mixer_fwd(*tok, lam0, eta0, workspace=ws, states=states)
    e_kept = mixer_bwd(*tok, g_out, g_var, lam0, eta0, workspace=ws, states=states,
                       need_state_grads=False)
    e_again = mixer_bwd(*tok, g_out, g_var, lam0, eta0, workspace=ws, need_state_grads=False)
    torch.cuda.synchronize(DEV)
    fo, fv = torch.empty(shape, device=DEV), torch.empty(shape, device=DEV)
    kept, again = grads_out(), grads_out()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mixer_fwd(*tok, lam0, eta0, out=fo, var=fv, workspace=ws, states=states)
        mixer_bwd(*tok, g_out, g_var, lam0, eta0, workspace=ws, states=states, out=kept,
                  need_state_grads=False)
        mixer_bwd(*tok, g_out, g_var, lam0, eta0, workspace=ws, out=again,
                  need_state_grads=False)
    torch.cuda.synchronize(DEV)
    for replay in range(3):
        for t in (fo, fv, states) + kept + again:
            t.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize(DEV)
        assert torch.equal(fo, e_out) and torch.equal(fv, e_var), replay
        for got, want in zip(kept + again, e_kept[:6] + e_again[:6]):
            assert torch.equal(got, want), replay
        mixer_fwd(*tok, workspace=ws)  # eager work on the same workspace
        torch.cuda.synchronize(DEV)
    assert workspace_health(ws) == 0
