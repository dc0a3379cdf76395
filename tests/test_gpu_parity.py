"""GPU parity: libkla's scan (through the C ABI) against the float64 oracle.

Both sides get the same seeded tensors from kla_inputs.  The bar is the
metric of kla_metric: max relative error 1e-4 on lam and 1e-4 on eta scaled
by its cancellation-free magnitude for fp32 gates, 2e-2 for bf16 gates, the
fp32 overflow rule, and no NaN.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from kla_inputs import WORKLOADS, make_gates, make_initial_state, make_workload
from kla_metric import TOL_BF16, TOL_F32, TOL_REGRESSION, assert_parity, compare, merge_reports
from oracle import oracle_scan

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)


def run_gpu(g, use_state=True):
    from linear_attention_sequence_kla_amd import scan_fwd
    lam0 = g["lam0"].to(DEV) if use_state else None
    eta0 = g["eta0"].to(DEV) if use_state else None
    lam, eta = scan_fwd(g["a"].to(DEV), g["p"].to(DEV), g["phi"].to(DEV), g["b"].to(DEV),
                        lam0, eta0)
    torch.cuda.synchronize(DEV)
    return lam, eta


def health():
    from linear_attention_sequence_kla_amd import get_workspace, workspace_health
    return workspace_health(get_workspace(0, DEV, torch.cuda.current_stream(DEV)))


def full_parity(g, tol, what):
    lam, eta = run_gpu(g)
    assert health() == 0, what
    ref = oracle_scan(g["a"], g["p"], g["phi"], g["b"], g["lam0"], g["eta0"])
    rep = compare(lam.cpu(), eta.cpu(), *ref)
    _say("%s: %s" % (what, rep))
    assert_parity(rep, tol, what)
    assert max(rep["lam_max_rel"], rep["eta_max_scaled"]) <= TOL_REGRESSION, (what, rep)
    return rep


def test_workload_tiny():
    """The tiny reference workload, drawn on the CPU."""
    w = WORKLOADS[0]
    _say("workload %s" % w.describe())
    full_parity(make_workload(0, device="cpu"), TOL_F32, w.describe())


def _sample_channels(C, n, seed):
    rng = np.random.default_rng(seed)
    picks = set(rng.choice(C, size=min(n, C), replace=False).tolist())
    picks.update({0, C - 1, min(63, C - 1), min(64, C - 1)})
    return np.array(sorted(picks))


def _gather(x, D, q):
    """x: [B, H, T, D] on any device -> [1, 1, T, len(q)] (channels q)."""
    B, H, T, _ = x.shape
    flat = x.reshape(B * H, T, D)
    slab = torch.as_tensor(q // D, device=x.device)
    d = torch.as_tensor(q % D, device=x.device)
    return flat[slab, :, d].transpose(0, 1).reshape(1, 1, T, len(q)).contiguous()


def compare_by_slabs(g, lam, eta, shape, max_elements=1 << 25):
    """Every output element against the oracle, a batch of (b, h) slabs at a
    time: the batch's inputs are copied to the host, the oracle runs on them
    and the GPU outputs of the same slabs are compared.  Host memory stays
    bounded whatever the size of the workload."""
    B, H, T, D = shape
    S = B * H
    per = max(1, min(S, max_elements // max(1, T * D)))
    slabs = lambda x: x.reshape(S, T, D)  # noqa: E731
    reps = []
    for s0 in range(0, S, per):
        s1 = min(S, s0 + per)
        host = {k: slabs(g[k])[s0:s1].cpu().reshape(1, s1 - s0, T, D)
                for k in ("a", "p", "phi", "b")}
        st = {k: g[k].reshape(S, D)[s0:s1].cpu().reshape(1, s1 - s0, D) for k in ("lam0", "eta0")}
        ref = oracle_scan(host["a"], host["p"], host["phi"], host["b"], st["lam0"], st["eta0"])
        reps.append(compare(slabs(lam)[s0:s1].cpu().reshape(1, s1 - s0, T, D),
                            slabs(eta)[s0:s1].cpu().reshape(1, s1 - s0, T, D), *ref))
        del host, ref
    return merge_reports(reps)


@pytest.mark.parametrize("key", [1, 2, 3, 4])
def test_workload_every_element(key):
    """A workload at full size, drawn on the GPU exactly as the benchmark
    draws it (same generator, same seed) and run in the benchmark's launch;
    the oracle runs on host copies of those very tensors, a batch of slabs at
    a time, and every output element is compared."""
    from linear_attention_sequence_kla_amd import scan_fwd
    w = WORKLOADS[key]
    _say("workload %s (every element)" % w.describe())
    g = make_workload(key, device=DEV)
    lam, eta = scan_fwd(g["a"], g["p"], g["phi"], g["b"], g["lam0"], g["eta0"])
    torch.cuda.synchronize(DEV)
    assert health() == 0
    rep = compare_by_slabs(g, lam, eta, w.shape)
    _say("%s: %s" % (w.describe(), rep))
    assert rep["n"] == w.elements
    assert_parity(rep, TOL_BF16 if w.dtype == "bf16" else TOL_F32, w.describe())
    assert max(rep["lam_max_rel"], rep["eta_max_scaled"]) <= TOL_REGRESSION, rep
    if key == 4:
        # the hard gates do overflow fp32 somewhere: the rule was exercised
        assert rep["lam_overflow"] > 0 and rep["eta_overflow"] > 0
    else:
        assert rep["lam_overflow"] == 0 and rep["eta_overflow"] == 0
    del g, lam, eta
    torch.cuda.empty_cache()


def test_largest_offsets():
    """The largest per-wave address span the library accepts: D = 1, so the
    64 channels of a wave lie in 64 slabs of T elements, and T just under the
    limit of 32-bit per-wave byte offsets (63 T < 2^30; 4.35 GB per float32
    tensor).  The oracle checks whole channels, including the first and the
    last (the farthest slab)."""
    from linear_attention_sequence_kla_amd import scan_fwd
    B, H, T, D = 8, 8, 17_000_000, 1
    _say("largest offsets %s" % ((B, H, T, D),))
    g = make_gates((B, H, T, D), "std", "f32", seed=77, device=DEV)
    lam0, eta0 = make_initial_state(B, H, D, random=True, seed=77, device=DEV)
    lam, eta = scan_fwd(g["a"], g["p"], g["phi"], g["b"], lam0, eta0)
    torch.cuda.synchronize(DEV)
    assert health() == 0
    q = _sample_channels(B * H * D, 3, seed=77)
    gs = {k: _gather(g[k], D, q).cpu() for k in ("a", "p", "phi", "b")}
    qd = torch.as_tensor(q, device=DEV)
    ref = oracle_scan(gs["a"], gs["p"], gs["phi"], gs["b"],
                      lam0.reshape(-1)[qd].reshape(1, 1, -1).cpu(),
                      eta0.reshape(-1)[qd].reshape(1, 1, -1).cpu())
    rep = compare(_gather(lam, D, q).cpu(), _gather(eta, D, q).cpu(), *ref)
    _say("largest offsets: %s" % rep)
    assert_parity(rep, TOL_F32, "largest offsets")
    assert bool(torch.isfinite(lam).all()) and bool(torch.isfinite(eta).all())
    del g, lam, eta
    torch.cuda.empty_cache()


def test_long_single_sequence():
    """One sequence of 17M tokens at D = 64 (1.09G elements, 4.35 GB per
    float32 tensor): with D a multiple of 64 the per-wave offsets stay within
    a wave's rows, so such a sequence runs in one call.  The oracle checks
    whole channels (the first, one in the middle, the last)."""
    from linear_attention_sequence_kla_amd import scan_fwd
    B, H, T, D = 1, 1, 17_000_000, 64
    _say("long single sequence %s" % ((B, H, T, D),))
    g = make_gates((B, H, T, D), "slow", "f32", seed=79, device=DEV)
    lam0, eta0 = make_initial_state(B, H, D, random=True, seed=79, device=DEV)
    lam, eta = scan_fwd(g["a"], g["p"], g["phi"], g["b"], lam0, eta0)
    torch.cuda.synchronize(DEV)
    assert health() == 0
    q = np.array([0, 31, 63])
    gs = {k: _gather(g[k], D, q).cpu() for k in ("a", "p", "phi", "b")}
    qd = torch.as_tensor(q, device=DEV)
    ref = oracle_scan(gs["a"], gs["p"], gs["phi"], gs["b"],
                      lam0.reshape(-1)[qd].reshape(1, 1, -1).cpu(),
                      eta0.reshape(-1)[qd].reshape(1, 1, -1).cpu())
    rep = compare(_gather(lam, D, q).cpu(), _gather(eta, D, q).cpu(), *ref)
    _say("long single sequence: %s" % rep)
    assert_parity(rep, TOL_F32, "long single sequence")
    assert max(rep["lam_max_rel"], rep["eta_max_scaled"]) <= TOL_REGRESSION, rep
    assert bool(torch.isfinite(lam).all()) and bool(torch.isfinite(eta).all())
    del g, lam, eta
    torch.cuda.empty_cache()


SHAPES = [
    # (B, H, T, D, gates, dtype)
    (1, 1, 1, 1, "std", "f32"),          # a single token, a single channel
    (1, 1, 111, 1, "std", "f32"),        # T below one tile (28 rows x 4 waves), D below a wave
    (1, 1, 112, 64, "std", "f32"),       # exactly one tile
    (1, 1, 113, 64, "std", "f32"),       # one row into a second tile
    (1, 2, 28, 3, "hard", "f32"),        # exactly one wave's rows
    (2, 1, 29, 3, "slow", "f32"),        # one row into a second wave
    (2, 3, 1000, 7, "std", "f32"),       # ragged everything
    (3, 2, 517, 100, "slow", "f32"),     # column groups straddle slabs
    (1, 2, 4099, 33, "hard", "f32"),     # long ragged T with hard gates
    (2, 2, 300, 128, "std", "bf16"),     # bf16
    (1, 1, 5000, 200, "slow", "bf16"),   # bf16, ragged D > 64
    (5, 1, 64, 13, "hard", "f32"),       # T below one wave's rows
    (3, 3, 1000, 128, "hard", "f32"),    # row halves paired per XCD, partial last block
    (2, 5, 400, 256, "std", "bf16"),     # paired quarter rows, bf16
    (3, 1, 777, 6, "hard", "bf16"),      # bf16, small even D, hard gates
    (2, 3, 250, 2, "slow", "bf16"),      # bf16, D = 2
    (1, 2, 96, 64, "std", "bf16"),       # exactly one bf16 tile (24 rows x 4 waves)
    (2, 1, 97, 64, "slow", "bf16"),      # one row into a second bf16 tile
    (1, 1, 23, 5, "hard", "bf16"),       # bf16, T below one wave's rows (odd)
    (2, 2, 1153, 70, "std", "bf16"),     # bf16, many tiles, odd rows in the last wave
    (2, 3, 1, 40, "hard", "bf16"),       # bf16, a single token
    (1, 1, 2, 1, "std", "bf16"),         # bf16, two tokens, one channel
    # long float32 sequences take the tall tiles (18 rows x 8 waves = 144 rows)
    (1, 1, 65535, 3, "hard", "f32"),     # one token below the tall-tile length
    (1, 1, 65536, 3, "hard", "f32"),     # the first tall length, ragged last tile
    (1, 2, 65664, 64, "std", "f32"),     # exactly 456 tall tiles
    (2, 1, 65665, 100, "slow", "f32"),   # one row into a tall tile, groups straddle slabs
    (1, 1, 65553, 128, "std", "f32"),    # paired row halves, rows into the last tile's 2nd wave
    (1, 1, 70000, 64, "std", "bf16"),    # bf16 keeps its 4-wave tiles at any length
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s[:4])) + s[4] + s[5])
def test_shapes(shape):
    B, H, T, D, fam, dtype = shape
    _say("shape %s" % (shape,))
    g = make_gates((B, H, T, D), fam, dtype, seed=B * 1000 + T)
    g["lam0"], g["eta0"] = make_initial_state(B, H, D, random=True, seed=T)
    full_parity(g, TOL_BF16 if dtype == "bf16" else TOL_F32, str(shape))


def test_default_initial_state():
    """NULL lam0/eta0 means lam0 = 1, eta0 = 0."""
    g = make_gates((2, 2, 300, 40), "std", "f32", seed=5)
    lam, eta = run_gpu(g, use_state=False)
    ones, zeros = make_initial_state(2, 2, 40)
    ref = oracle_scan(g["a"], g["p"], g["phi"], g["b"], ones, zeros)
    assert_parity(compare(lam.cpu(), eta.cpu(), *ref), TOL_F32, "default state")


def test_segmenting_matches_one_call():
    """Passing the last row of one call as the initial state of the next
    continues the sequence."""
    from linear_attention_sequence_kla_amd import scan_fwd
    g = make_gates((2, 4, 3000, 64), "std", "f32", seed=9)
    gd = {k: v.to(DEV) for k, v in g.items()}
    lam0, eta0 = (x.to(DEV) for x in make_initial_state(2, 4, 64, random=True, seed=9))
    lam, eta = scan_fwd(gd["a"], gd["p"], gd["phi"], gd["b"], lam0, eta0)
    k = 1111
    part = lambda x, s: x[:, :, s].contiguous()  # noqa: E731
    l1, e1 = scan_fwd(*(part(gd[n], slice(0, k)) for n in ("a", "p", "phi", "b")), lam0, eta0)
    l2, e2 = scan_fwd(*(part(gd[n], slice(k, None)) for n in ("a", "p", "phi", "b")),
                      l1[:, :, -1].contiguous(), e1[:, :, -1].contiguous())
    torch.cuda.synchronize(DEV)
    lam_s = torch.cat([l1, l2], dim=2)
    eta_s = torch.cat([e1, e2], dim=2)
    assert torch.allclose(lam_s, lam, rtol=2e-6, atol=0)
    assert torch.allclose(eta_s, eta, rtol=2e-6, atol=2e-6 * float(eta.abs().max()))


def test_repeated_calls_reuse_workspace():
    """The workspace resets itself: many calls in a row, and a call with a
    different shape in between, all stay exact and healthy."""
    g = make_gates((4, 4, 2048, 64), "std", "f32", seed=13)
    g["lam0"], g["eta0"] = make_initial_state(4, 4, 64, random=True, seed=13)
    first = run_gpu(g)
    small = make_gates((1, 1, 300, 5), "std", "f32", seed=14)
    run_gpu(small, use_state=False)
    for _ in range(5):
        again = run_gpu(g)
    assert health() == 0
    ref = oracle_scan(g["a"], g["p"], g["phi"], g["b"], g["lam0"], g["eta0"])
    assert_parity(compare(again[0].cpu(), again[1].cpu(), *ref), TOL_F32, "repeat")
    assert torch.allclose(first[0], again[0], rtol=1e-6)


def test_workspace_left_dirty_by_other_calls():
    """Past its header a shared workspace may hold another call's leftovers
    (flags of other tags, records, counts): filled with 0xFF bytes between two
    calls, the forward gives the same outputs bit for bit, healthy and equal
    to the oracle."""
    from linear_attention_sequence_kla_amd import scan_fwd, workspace_health, workspace_size
    shape = (2, 3, 1500, 64)
    g = make_gates(shape, "std", "f32", seed=23)
    g["lam0"], g["eta0"] = make_initial_state(2, 3, 64, random=True, seed=23)
    d = {k: v.to(DEV) for k, v in g.items()}
    ws = torch.zeros(workspace_size(*shape, torch.float32), dtype=torch.uint8, device=DEV)
    first = scan_fwd(d["a"], d["p"], d["phi"], d["b"], d["lam0"], d["eta0"], workspace=ws)
    torch.cuda.synchronize(DEV)
    ws[256:].fill_(255)
    again = scan_fwd(d["a"], d["p"], d["phi"], d["b"], d["lam0"], d["eta0"], workspace=ws)
    torch.cuda.synchronize(DEV)
    assert workspace_health(ws) == 0
    assert torch.equal(first[0], again[0]) and torch.equal(first[1], again[1])
    ref = oracle_scan(g["a"], g["p"], g["phi"], g["b"], g["lam0"], g["eta0"])
    assert_parity(compare(again[0].cpu(), again[1].cpu(), *ref), TOL_F32, "dirty workspace")


def test_side_stream():
    """The call runs on the caller's current stream."""
    g = make_gates((2, 2, 700, 64), "std", "f32", seed=17)
    g["lam0"], g["eta0"] = make_initial_state(2, 2, 64, random=True, seed=17)
    s = torch.cuda.Stream(DEV)
    with torch.cuda.stream(s):
        gd = {k: v.to(DEV) for k, v in g.items()}
        from linear_attention_sequence_kla_amd import scan_fwd
        lam, eta = scan_fwd(gd["a"], gd["p"], gd["phi"], gd["b"], gd["lam0"], gd["eta0"])
    s.synchronize()
    ref = oracle_scan(g["a"], g["p"], g["phi"], g["b"], g["lam0"], g["eta0"])
    assert_parity(compare(lam.cpu(), eta.cpu(), *ref), TOL_F32, "side stream")


def test_concurrent_streams():
    """Four scans in flight at once on four streams (default priority), each
    with its own workspace: the carry protocols of concurrent launches do not
    interfere, and every result matches the oracle."""
    from linear_attention_sequence_kla_amd import scan_fwd, workspace_health, workspace_size
    shapes = [(2, 2, 3000, 64), (1, 3, 2500, 40), (4, 1, 1800, 96), (3, 2, 2222, 33)]
    cases = []
    for k, shape in enumerate(shapes):
        g = make_gates(shape, "std", "f32", seed=60 + k)
        g["lam0"], g["eta0"] = make_initial_state(shape[0], shape[1], shape[3], random=True,
                                                  seed=60 + k)
        cases.append(g)
    streams = [torch.cuda.Stream(DEV) for _ in shapes]
    outs, wss = [], []
    torch.cuda.synchronize(DEV)
    for g, s, shape in zip(cases, streams, shapes):
        with torch.cuda.stream(s):
            gd = {n: v.to(DEV, non_blocking=False) for n, v in g.items()}
            ws = torch.zeros(workspace_size(*shape), dtype=torch.uint8, device=DEV)
            for _ in range(3):  # repeated calls on the same workspace and stream
                out = scan_fwd(gd["a"], gd["p"], gd["phi"], gd["b"], gd["lam0"], gd["eta0"],
                               workspace=ws)
            outs.append(out)
            wss.append(ws)
    torch.cuda.synchronize(DEV)
    for g, (lam, eta), ws, shape in zip(cases, outs, wss, shapes):
        assert workspace_health(ws) == 0
        ref = oracle_scan(g["a"], g["p"], g["phi"], g["b"], g["lam0"], g["eta0"])
        assert_parity(compare(lam.cpu(), eta.cpu(), *ref), TOL_F32, "stream %s" % (shape,))


@pytest.mark.parametrize("shape", [(1, 1, 200000, 1), (1, 4096, 1, 512)],
                         ids=["one-channel-long", "many-channels-one-token"])
def test_extreme_aspect(shape):
    """One channel over a long sequence (a chain of ~1800 tiles in one column)
    and two million channels of one token (one tile per column)."""
    g = make_gates(shape, "std", "f32", seed=71)
    g["lam0"], g["eta0"] = make_initial_state(shape[0], shape[1], shape[3], random=True,
                                              seed=71)
    full_parity(g, TOL_F32, "shape %s" % (shape,))


def test_argument_errors_on_device():
    """Host-side validation with real device buffers: nothing is launched."""
    from linear_attention_sequence_kla_amd import KlaError, scan_fwd
    g = make_gates((1, 2, 100, 8), "std", "f32", seed=3)
    gd = {k: v.to(DEV) for k, v in g.items()}
    small_ws = torch.zeros(64, dtype=torch.uint8, device=DEV)
    with pytest.raises(KlaError) as e:
        scan_fwd(gd["a"], gd["p"], gd["phi"], gd["b"], workspace=small_ws)
    assert e.value.name == "KLA_ERR_WORKSPACE"
    with pytest.raises(KlaError) as e:
        scan_fwd(gd["a"], gd["p"], gd["phi"], gd["b"], out=(gd["a"], torch.empty_like(gd["a"])))
    assert e.value.name == "KLA_ERR_INVALID_ARG"
    with pytest.raises(ValueError):
        scan_fwd(gd["a"], gd["p"].double(), gd["phi"], gd["b"])
