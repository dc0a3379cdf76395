"""Host-side logic of bench.py (no GPU): the refusal of more than one GPU,
the algorithmic byte counts per direction, the source hash that guards the
committed counter records, and the traffic arithmetic of
--summarize-counters on synthetic rocprofv3 tables."""

from __future__ import annotations

import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("direction,f32,bf16", [
    ("fwd", 24, 16),            # 4 gate reads, lam and eta written
    ("bwd", 40, 36),            # a, p; lam, eta, g_lam, g_eta; 4 gradients written
    ("decode", 32, 24),         # 4 gates, state read and written
    ("mixer", 24, 16),          # k, v, lam_v, q; readout and variance
    ("lti", 12, 10),            # b; lam and eta
    ("mixer_bwd", 56, 42),      # recompute (3 token reads + 2 B of states) + kernel
    ("mixer_train", 68, 52),    # forward with states (4 + 8 + 2) + backward kernel
    ("mixer_decode", 40, 32),   # 4 token inputs, state in place, readout and variance
])
def test_bytes_per_element(direction, f32, bf16):
    assert bench.bytes_per_element("f32", direction) == f32
    assert bench.bytes_per_element("bf16", direction) == bf16


def test_mixer_backward_kernel_bytes():
    # k, v, lam_v, q + 2 B of boundary state + g_out, g_var + 4 gradients
    assert bench.kernel_bytes_per_element("f32", "mixer_bwd") == 42
    assert bench.kernel_bytes_per_element("bf16", "mixer_bwd") == 34
    assert bench.kernel_bytes_per_element("f32", "fwd") == 24


def test_code_hash_ignores_comments():
    code = "int f(int x) {\n    return x + 1;  // one more\n}\n"
    assert bench._code_only(code) == bench._code_only(
        "/* header */\nint f(int x) {\n\n    return x + 1;\n}\n// end\n")
    assert bench._code_only(code) != bench._code_only(code.replace("+ 1", "+ 2"))


def test_workload_tables():
    for d in ("fwd", "bwd", "decode"):
        assert bench.workloads_for(d)[1].name == "small-lm-layer"
    for d in ("mixer", "mixer_bwd", "mixer_train", "mixer_decode"):
        assert bench.workloads_for(d)[1].name == "mixer-small-lm-layer"
    assert bench.workloads_for("lti")[1].name == "lti-small-lm-layer"


def _write_csv(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_summarize_counters_arithmetic(tmp_path, monkeypatch):
    """FETCH_SIZE and WRITE_SIZE are scaled by what they read for a plain copy
    of known size; the record and summary land in <root>/profiles."""
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    name = "void kla::(anonymous namespace)::kla_scan_kernel<float, 28, 4, (kla::(anonymous " \
           "namespace)::Mode)0>(kla::FwdArgs)"
    other = "void kla::(anonymous namespace)::kla_scan_kernel<float, 28, 4, (kla::(anonymous " \
            "namespace)::Mode)1>(kla::FwdArgs)"
    copy = "__amd_rocclr_copyBuffer"
    trace = tmp_path / "stats.csv"
    _write_csv(trace, ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs",
                       "MaxNs", "StdDev"],
               [[name, 10, 800000, 80000, 90, 79000, 81000, 1], [other, 3, 3, 1, 1, 1, 1, 0]])
    cols = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    fetch = tmp_path / "fetch.csv"
    _write_csv(fetch, cols, [[name, "FETCH_SIZE", 100000], [name, "FETCH_SIZE", 110000],
                             [other, "FETCH_SIZE", 5]])
    write = tmp_path / "write.csv"
    _write_csv(write, cols, [[name, "WRITE_SIZE", 130000], [other, "WRITE_SIZE", 7]])
    cfetch = tmp_path / "cfetch.csv"
    _write_csv(cfetch, cols, [[copy, "FETCH_SIZE", 512 * 1024]])   # half the copy's bytes
    cwrite = tmp_path / "cwrite.csv"
    _write_csv(cwrite, cols, [[copy, "WRITE_SIZE", 1024 * 1024]])  # all of them
    args = bench.argparse.Namespace(
        direction="fwd", workload=1, trace=str(trace), fetch=str(fetch), write=str(write),
        copy_fetch=str(cfetch), copy_write=str(cwrite), copy_mib=1024, commands=["cmd"])
    assert bench.summarize_counters(args) == 0
    rec = json.load(open(tmp_path / "profiles" / "traffic_workload1.json"))
    assert rec["fetch_scale"] == pytest.approx(2.0) and rec["write_scale"] == pytest.approx(1.0)
    assert rec["fetch_kib_per_dispatch"] == pytest.approx(105000)
    assert rec["hbm_bytes_per_launch"] == pytest.approx((105000 * 2.0 + 130000) * 1024)
    assert rec["algorithmic_bytes_per_launch"] == 16777216 * 24
    assert rec["trace_avg_ns"] == 80000 and rec["kernel"] == name
    assert rec["kernel_sha256_16"] == bench.kernel_hash("fwd")
    assert bench.load_traffic(1, "fwd") == pytest.approx(rec["hbm_bytes_per_launch"])
    md = open(tmp_path / "profiles" / "kla_scan_kernel_small-lm-layer.md").read()
    assert "cmd" in md and "80000" in md


@pytest.mark.parametrize("direction", ["fwd", "bwd", "bwd_states", "scan_train", "lti", "mixer",
                                       "mixer_bwd", "mixer_train", "decode", "mixer_decode"])
def test_cpu_baseline_every_direction(direction):
    """The oracle timing of every bench direction runs on the tiny workload's
    inputs as the bench builds them (host tensors here), with a short budget,
    and reports a positive rate over the whole sample and on one thread."""
    import torch
    from kla_inputs import (make_gates, make_lti_workload, make_mixer_inputs,
                            make_mixer_workload, make_workload)
    w = bench.workloads_for(direction)[0]
    if direction in ("mixer", "mixer_bwd", "mixer_train"):
        g = make_mixer_workload(0)
        g["g_out"], g["g_var"] = torch.randn(w.shape), torch.randn(w.shape)
    elif direction == "lti":
        g = make_lti_workload(0)
    elif direction == "decode":
        g = {n: v[:, :, 0].contiguous()
             for n, v in make_gates((w.B, w.H, 1, w.D), w.gates, w.dtype, 1).items()}
    elif direction == "mixer_decode":
        g = {n: (v[:, :, 0] if v.dim() == 4 else v).contiguous()
             for n, v in make_mixer_inputs((w.B, w.H, 1, w.D), w.dtype, 1).items()}
    else:
        g = make_workload(0)
        g["g_lam"], g["g_eta"] = torch.randn(w.shape), torch.randn(w.shape)
    rec = bench.cpu_baseline(w, g, direction, budget_s=0.05)
    assert rec["kind"] == "oracle" and rec["cores"] >= 1
    assert rec["value"] > 0 and rec["value_1thread"] > 0
    assert ("one token" in rec["sample"]) == direction.endswith("decode")
