"""GPU parity of the fused mixer's backward pass (kla_mixer_bwd through the C
ABI, and the KLAMixer autograd Function) against the float64 mixer backward
oracle.  Bar: kla_metric.compare_grads (error over the cancellation-free
magnitude) within 1e-4 for fp32 inputs, 2e-2 for bf16, no NaN."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from kla_inputs import MIXER_WORKLOADS, make_initial_state, make_mixer_inputs, make_mixer_workload
from kla_metric import (TOL_BF16, TOL_F32, TOL_REGRESSION, assert_grad_parity, compare_grads,
                        merge_any)
from oracle import oracle_mixer_bwd

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
TOKEN = ("k", "v", "lam_v", "q")
NAMES = ("k", "v", "lam_v", "q", "a", "p", "lam0", "eta0")


def _say(msg):
    print(msg, flush=True)


def _case(shape, dtype="f32", seed=0, random_state=True, with_var=True):
    g = make_mixer_inputs(shape, dtype, seed=seed)
    g["lam0"], g["eta0"] = make_initial_state(shape[0], shape[1], shape[3],
                                              random=random_state, seed=seed)
    gen = torch.Generator().manual_seed(seed + 99)
    g["g_out"] = torch.randn(shape, generator=gen)
    g["g_var"] = torch.randn(shape, generator=gen) if with_var else None
    return g


def run_gpu(g, need_state=True):
    from linear_attention_sequence_kla_amd import get_workspace, mixer_bwd, workspace_health
    d = {n: (None if t is None else t.to(DEV)) for n, t in g.items()}
    res = mixer_bwd(*(d[n] for n in TOKEN), d["a"], d["p"], d["g_out"], d["g_var"], d["lam0"],
                    d["eta0"], need_state_grads=need_state)
    torch.cuda.synchronize(DEV)
    assert workspace_health(get_workspace(0, DEV, torch.cuda.current_stream(DEV))) == 0
    return dict(zip(NAMES, res))


def oracle(g):
    return oracle_mixer_bwd(*(g[n] for n in TOKEN), g["a"], g["p"], g["lam0"], g["eta0"],
                            g["g_out"], g["g_var"])


def parity(g, tol, what, need_state=True):
    got = run_gpu(g, need_state)
    grads, mags = oracle(g)
    rep = compare_grads({n: (None if t is None else t.cpu()) for n, t in got.items()}, grads,
                        mags)
    _say("%s: %s" % (what, rep))
    assert_grad_parity(rep, tol, what)
    return rep


@pytest.mark.parametrize("key", [0, 1])
def test_mixer_bwd_workload(key):
    w = MIXER_WORKLOADS[key]
    _say("mixer backward, workload %s" % w.describe())
    parity(_case(w.shape, w.dtype, seed=w.seed), TOL_F32, w.describe())


SHAPES = [(1, 1, 1, 1), (1, 1, 7, 3), (2, 3, 113, 7), (1, 2, 337, 64), (3, 1, 450, 65),
          (2, 2, 1000, 33), (1, 1, 2049, 128), (3, 3, 300, 128),
          # a state is kept after every 8th token; a tile holds 64 rows
          (2, 3, 8, 5), (1, 2, 9, 7), (2, 1, 64, 9), (2, 1, 65, 9), (1, 3, 129, 40),
          # 8-row waves: 4 per workgroup below T = 8192, 8 from there on
          (2, 1, 32, 9), (2, 1, 33, 9), (1, 1, 8191, 5), (1, 2, 8192, 70),
          # g_a, g_p are summed in slices of 64 (b, chunk) pairs, then over
          # the slices by the workgroup that finishes last: 9 slices of 564
          # pairs, the last one short; at most 128 slices, so 8750 pairs
          # give slices of 69 and leave the last one empty
          (3, 1, 6000, 64), (70, 1, 4000, 2)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_mixer_bwd_shapes(shape):
    parity(_case(shape, seed=sum(shape)), TOL_F32, "shape %s" % (shape,))


def test_mixer_bwd_bf16_no_var_default_state():
    g = _case((2, 2, 600, 48), "bf16", seed=3, random_state=False, with_var=False)
    parity(g, TOL_BF16, "bf16, g_var NULL, default state", need_state=False)


@pytest.mark.parametrize("key", [2, 3])
def test_mixer_bwd_full_size_sampled(key):
    """A full-size workload in the benchmark's launch (inputs drawn on the GPU
    as the benchmark draws them); the oracle runs on a sample of whole (h, d)
    channels with every batch entry b, so it checks the token-input and
    initial-state gradients of those channels and the channel-gate gradients
    g_a[h, d], g_p[h, d] (sums over b and t) themselves."""
    from linear_attention_sequence_kla_amd import mixer_bwd
    w = MIXER_WORKLOADS[key]
    _say("mixer backward, workload %s (sampled (h, d) channels, every b)" % w.describe())
    g = make_mixer_inputs(w.shape, w.dtype, w.seed, device=DEV)
    g["lam0"], g["eta0"] = make_initial_state(w.B, w.H, w.D, random=True, seed=w.seed,
                                              device=DEV)
    gen = torch.Generator(device=DEV).manual_seed(5)
    g["g_out"] = torch.randn(w.shape, generator=gen, device=DEV)
    g["g_var"] = torch.randn(w.shape, generator=gen, device=DEV)
    res = dict(zip(NAMES, mixer_bwd(*(g[n] for n in TOKEN), g["a"], g["p"], g["g_out"],
                                    g["g_var"], g["lam0"], g["eta0"])))
    torch.cuda.synchronize(DEV)
    HD = w.H * w.D
    rng = np.random.default_rng(key)
    hd = np.array(sorted(set(rng.choice(HD, 192, replace=False).tolist()) | {0, HD - 1}))
    hd_dev = torch.as_tensor(hd, device=DEV)
    h_idx, d_idx = hd_dev // w.D, hd_dev % w.D

    def tok(x):  # [B, H, T, D] -> [B, 1, T, n]: the sampled channels of every b
        return x[:, h_idx, :, d_idx].permute(1, 2, 0).unsqueeze(1).contiguous()

    def st(x):  # [B, H, D] -> [B, 1, n]
        return x[:, h_idx, d_idx].unsqueeze(1).contiguous()

    sub = {n: tok(g[n]).cpu() for n in TOKEN + ("g_out", "g_var")}
    sub["a"] = g["a"].reshape(-1)[hd_dev].reshape(1, -1).cpu()
    sub["p"] = g["p"].reshape(-1)[hd_dev].reshape(1, -1).cpu()
    sub["lam0"] = st(g["lam0"]).cpu()
    sub["eta0"] = st(g["eta0"]).cpu()
    grads, mags = oracle(sub)
    got = {n: tok(res[n]).cpu() for n in TOKEN}
    got["lam0"] = st(res["lam0"]).cpu()
    got["eta0"] = st(res["eta0"]).cpu()
    got["a"] = res["a"].reshape(-1)[hd_dev].reshape(1, -1).cpu()
    got["p"] = res["p"].reshape(-1)[hd_dev].reshape(1, -1).cpu()
    rep = compare_grads(got, grads, mags)
    _say("sampled: %s" % rep)
    assert_grad_parity(rep, TOL_BF16 if w.dtype == "bf16" else TOL_F32, w.describe())
    assert bool(torch.isfinite(res["a"]).all()) and bool(torch.isfinite(res["p"]).all())
    del g, res
    torch.cuda.empty_cache()


@pytest.mark.parametrize("key", [2, 3])
def test_mixer_bwd_workload_every_element(key):
    """A full-size workload drawn on the GPU as the benchmark draws it, the
    backward in the benchmark's launch (recomputing the states); the oracle
    runs on host copies of every batch entry b of a range of heads at a time,
    so that it also forms the channel-gate gradients g_a, g_p (sums over b
    and t) of those heads, and every gradient element is compared."""
    from linear_attention_sequence_kla_amd import mixer_bwd
    w = MIXER_WORKLOADS[key]
    _say("mixer backward, workload %s (every element)" % w.describe())
    g = make_mixer_workload(key, device=DEV)
    gen = torch.Generator(device=DEV).manual_seed(7)
    g["g_out"] = torch.randn(w.shape, generator=gen, device=DEV)
    g["g_var"] = torch.randn(w.shape, generator=gen, device=DEV)
    res = dict(zip(NAMES, mixer_bwd(*(g[n] for n in TOKEN), g["a"], g["p"], g["g_out"],
                                    g["g_var"], g["lam0"], g["eta0"])))
    torch.cuda.synchronize(DEV)
    from linear_attention_sequence_kla_amd import get_workspace, workspace_health
    assert workspace_health(get_workspace(0, DEV, torch.cuda.current_stream(DEV))) == 0
    B, H, T, D = w.shape
    per = max(1, min(H, (1 << 24) // (B * T * D)))
    reps = []
    for h0 in range(0, H, per):
        h1 = min(H, h0 + per)
        sub = {n: g[n][:, h0:h1].cpu() for n in TOKEN + ("g_out", "g_var", "lam0", "eta0")}
        sub["a"], sub["p"] = g["a"][h0:h1].cpu(), g["p"][h0:h1].cpu()
        grads, mags = oracle(sub)
        got = {n: res[n][:, h0:h1].cpu() for n in TOKEN + ("lam0", "eta0")}
        got["a"], got["p"] = res["a"][h0:h1].cpu(), res["p"][h0:h1].cpu()
        reps.append(compare_grads(got, grads, mags))
        del sub, grads, mags, got
    rep = merge_any(reps)
    _say("%s: %s" % (w.describe(), rep))
    assert_grad_parity(rep, TOL_BF16 if w.dtype == "bf16" else TOL_F32, w.describe())
    # float64 arithmetic from float32 kept states on the very values the
    # oracle reads: errors of a few float32 roundings (2e-7 measured)
    assert_grad_parity(rep, TOL_REGRESSION, w.describe())
    del g, res
    torch.cuda.empty_cache()


def test_kla_mixer_autograd():
    """torch.autograd through KLAMixer equals the oracle's gradients of
    sum(g_out * out + g_var * var)."""
    from linear_attention_sequence_kla_amd import kla_mixer
    shape = (2, 3, 500, 24)
    g = _case(shape, seed=12)
    leaves = {n: g[n].to(DEV).clone().requires_grad_(True) for n in NAMES}
    out, var = kla_mixer(*(leaves[n] for n in NAMES))
    ((out * g["g_out"].to(DEV)).sum() + (var * g["g_var"].to(DEV)).sum()).backward()
    torch.cuda.synchronize(DEV)
    grads, mags = oracle(g)
    rep = compare_grads({n: leaves[n].grad.cpu() for n in NAMES}, grads, mags)
    _say("autograd: %s" % rep)
    assert_grad_parity(rep, TOL_F32, "autograd")


def test_workspace_left_dirty_by_other_calls():
    """Past its header a shared workspace may hold another call's leftovers,
    the channel-gate reduction's arrival counts among them (the backward
    kernel clears those before the reduction runs): filled with 0xFF bytes
    between two calls of a shape whose g_a, g_p take two slices, the mixer
    backward gives the same gradients bit for bit, healthy and equal to the
    oracle."""
    from linear_attention_sequence_kla_amd import (mixer_bwd, mixer_bwd_workspace_size,
                                                   workspace_health)
    shape = (3, 2, 1000, 33)
    g = _case(shape, seed=21)
    d = {n: (None if t is None else t.to(DEV)) for n, t in g.items()}
    ws = torch.zeros(mixer_bwd_workspace_size(*shape, torch.float32), dtype=torch.uint8,
                     device=DEV)
    args = (*(d[n] for n in TOKEN), d["a"], d["p"], d["g_out"], d["g_var"], d["lam0"], d["eta0"])
    first = mixer_bwd(*args, workspace=ws)
    torch.cuda.synchronize(DEV)
    ws[256:].fill_(255)
    again = mixer_bwd(*args, workspace=ws)
    torch.cuda.synchronize(DEV)
    assert workspace_health(ws) == 0
    for n, x, y in zip(NAMES, first, again):
        assert torch.equal(x, y), n
    grads, mags = oracle(g)
    rep = compare_grads(dict(zip(NAMES, (t.cpu() for t in again))), grads, mags)
    _say("dirty workspace: %s" % rep)
    assert_grad_parity(rep, TOL_F32, "dirty workspace")


@pytest.mark.parametrize("shape,dtype", [((2, 3, 500, 24), "f32"), ((3, 3, 300, 128), "f32"),
                                         ((2, 2, 601, 48), "bf16"), ((1, 1, 7, 3), "f32"),
                                         ((2, 1, 289, 40), "bf16")],
                         ids=lambda x: "x".join(map(str, x)) if isinstance(x, tuple) else x)
def test_saved_states_equal_recompute(shape, dtype):
    """States kept by kla_mixer_fwd give the backward bitwise the gradients of
    its own recompute (the same kernel writes the same float64 states), and
    those match the oracle."""
    from linear_attention_sequence_kla_amd import mixer_bwd, mixer_fwd, mixer_states_shape
    g = _case(shape, dtype, seed=sum(shape))
    d = {n: (None if t is None else t.to(DEV)) for n, t in g.items()}
    states = torch.full(mixer_states_shape(*shape), float("nan"), dtype=torch.float64,
                        device=DEV)
    mixer_fwd(*(d[n] for n in TOKEN), d["a"], d["p"], d["lam0"], d["eta0"], states=states)
    args = (*(d[n] for n in TOKEN), d["a"], d["p"], d["g_out"], d["g_var"], d["lam0"], d["eta0"])
    kept = mixer_bwd(*args, states=states)
    again = mixer_bwd(*args)
    torch.cuda.synchronize(DEV)
    # every state the backward reads was written (all blocks but the last)
    assert bool(torch.isfinite(states[:-1]).all())
    for n, x, y in zip(NAMES, kept, again):
        assert torch.equal(x, y), n
    grads, mags = oracle(g)
    rep = compare_grads(dict(zip(NAMES, (t.cpu() for t in kept))), grads, mags)
    _say("saved states %s %s: %s" % (shape, dtype, rep))
    assert_grad_parity(rep, TOL_BF16 if dtype == "bf16" else TOL_F32, "saved states")


def test_mixer_bwd_argument_errors_on_device():
    from linear_attention_sequence_kla_amd import mixer_bwd
    g = {n: (None if t is None else t.to(DEV)) for n, t in _case((1, 2, 8, 4), seed=1).items()}
    with pytest.raises(ValueError):
        mixer_bwd(g["k"], g["v"], g["lam_v"], g["q"], g["a"], g["p"], None)
    with pytest.raises(ValueError):
        mixer_bwd(g["k"], g["v"], g["lam_v"], g["q"], g["a"], g["p"],
                  g["g_out"][:, :, :4].contiguous())
    with pytest.raises(ValueError):
        mixer_bwd(g["k"], g["v"], g["lam_v"], g["q"], g["a"][:1].contiguous(), g["p"],
                  g["g_out"])
    with pytest.raises(ValueError):  # states of the wrong shape
        mixer_bwd(g["k"], g["v"], g["lam_v"], g["q"], g["a"], g["p"], g["g_out"],
                  states=torch.zeros((2, 8, 2), dtype=torch.float64, device=DEV))
