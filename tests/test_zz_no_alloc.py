"""kla_scan_fwd_noalloc (the forward scan with the library's own per-GPU
workspace array) through the C ABI, against kla_scan_fwd with a caller-owned
workspace on the same inputs, and against the oracle: two calls in a row, the
second with a smaller problem, then the first shape again."""

from __future__ import annotations

import ctypes

import pytest
import torch

from kla_inputs import make_gates, make_initial_state
from kla_metric import TOL_BF16, TOL_F32, TOL_REGRESSION, assert_parity, compare
from oracle import oracle_scan

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)


def _case(shape, fam, dtype, seed):
    g = make_gates(shape, fam, dtype, seed=seed)
    g["lam0"], g["eta0"] = make_initial_state(shape[0], shape[1], shape[3], random=True,
                                              seed=seed)
    return g


def _both(g):
    """(noalloc outputs, kla_scan_fwd outputs) on the same device inputs."""
    from linear_attention_sequence_kla_amd import scan_fwd, scan_fwd_noalloc
    d = {k: v.to(DEV) for k, v in g.items()}
    lam_n, eta_n = scan_fwd_noalloc(d["a"], d["p"], d["phi"], d["b"], d["lam0"], d["eta0"])
    ws = torch.zeros(max(256, _ws_size(g)), dtype=torch.uint8, device=DEV)
    lam_w, eta_w = scan_fwd(d["a"], d["p"], d["phi"], d["b"], d["lam0"], d["eta0"], workspace=ws)
    torch.cuda.synchronize(DEV)
    return (lam_n, eta_n), (lam_w, eta_w)


def _ws_size(g):
    from linear_attention_sequence_kla_amd import workspace_size
    return workspace_size(*g["a"].shape, g["a"].dtype)


def test_noalloc_matches_workspace_entry_point():
    cases = [((2, 4, 3000, 64), "std", "f32", 31),   # several tiles per column
             ((1, 2, 700, 40), "hard", "bf16", 32),  # a smaller problem right after
             ((2, 4, 3000, 64), "slow", "f32", 33)]  # the first shape again
    for shape, fam, dtype, seed in cases:
        _say("noalloc %s %s %s" % (shape, fam, dtype))
        g = _case(shape, fam, dtype, seed)
        (lam_n, eta_n), (lam_w, eta_w) = _both(g)
        # the same kernels on the same inputs: identical bits
        assert torch.equal(lam_n, lam_w) and torch.equal(eta_n, eta_w), shape
        ref = oracle_scan(g["a"], g["p"], g["phi"], g["b"], g["lam0"], g["eta0"])
        rep = compare(lam_n.cpu(), eta_n.cpu(), *ref)
        _say("  %s" % rep)
        assert_parity(rep, TOL_BF16 if dtype == "bf16" else TOL_F32, str(shape))
        assert max(rep["lam_max_rel"], rep["eta_max_scaled"]) <= TOL_REGRESSION, rep


def test_noalloc_rejects_oversize_before_launch():
    """A problem whose workspace exceeds the array is refused with
    KLA_ERR_WORKSPACE, and the outputs are left untouched."""
    from linear_attention_sequence_kla_amd import library, workspace_size
    lib = library()
    limit = int(lib.kla_scan_fwd_noalloc_max_workspace())
    B, H, T, D = 1, 8, 131072, 128
    assert workspace_size(B, H, T, D) > limit
    x = torch.ones(16, device=DEV)
    out = torch.full((16,), 7.0, device=DEV)
    p = ctypes.c_void_p(x.data_ptr())
    st = lib.kla_scan_fwd_noalloc(p, p, p, p, 0, None, None, ctypes.c_void_p(out.data_ptr()),
                                  ctypes.c_void_p(out.data_ptr() + 32), B, H, T, D, None)
    torch.cuda.synchronize(DEV)
    assert lib.kla_status_string(st).decode() == "KLA_ERR_WORKSPACE"
    assert b"kla_scan_fwd_noalloc" in lib.kla_last_error_detail()
    assert bool((out == 7.0).all())
