"""Benchmark of the KLA scan (libkla) on one MI355X.

The headline (default) is the forward scan on the long-context workload
(B=1, H=32, T=131072, D=128, float32 gates; the largest one): a step is one
kla_scan_fwd call over one batch of synthetic gates, the whole scan (chunk
matrices, carry look-back, replay and output writes) in a single kernel
launch.  The small-LM-layer and 1B-scale-layer workloads are measured the
same way in the same process and reported under per_config.  --direction
selects the backward scan, the fused mixer (forward, backward, a training
step of both, or its decode step), the time-invariant form or the scan's
decode step instead.  The K timed steps are
captured once into a HIP graph and replayed (--no-graph launches them one by
one).  Inputs are generated on the GPU and are resident in HBM before timing;
two input/output sets alternate so that the 256 MB Infinity Cache cannot
serve one step from the previous one.

Prints one JSON line: throughput in scanned elements (B*H*T*D) per second,
the roofline of the kernel (HBM bound; for the forward scan the algorithmic
bytes are 4 gate reads + 2 float32 writes per element), the HBM traffic from
the committed rocprofv3 counters when they match the kernel source, and the
float64 CPU oracle timed on a sample of the same workload as a baseline.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
CSRC = os.path.join(ROOT, "linear_attention_sequence_kla_amd", "csrc")
KERNEL_SOURCES = {"fwd": ("kla_scan_fwd.hip", "kla_lookback.h", "kla_internal.h"),
                  "bwd": ("kla_scan_bwd.hip", "kla_lookback.h", "kla_internal.h"),
                  "decode": ("kla_decode.hip", "kla_lookback.h", "kla_internal.h"),
                  "mixer_decode": ("kla_decode.hip", "kla_lookback.h", "kla_internal.h"),
                  "mixer": ("kla_scan_fwd.hip", "kla_lookback.h", "kla_internal.h"),
                  "lti": ("kla_scan_fwd.hip", "kla_lookback.h", "kla_internal.h"),
                  "mixer_bwd": ("kla_scan_bwd.hip", "kla_lookback.h", "kla_internal.h"),
                  "bwd_states": ("kla_scan_bwd.hip", "kla_lookback.h", "kla_internal.h"),
                  "scan_train": ("kla_scan_bwd.hip", "kla_lookback.h", "kla_internal.h"),
                  "mixer_train": ("kla_scan_bwd.hip", "kla_lookback.h", "kla_internal.h")}
KERNEL_NAMES = {"fwd": "kla_scan_kernel", "bwd": "kla_scan_bwd_kernel",
                "decode": "kla_decode_kernel", "mixer_decode": "kla_mixer_decode_kernel",
                "mixer": "kla_scan_kernel",
                "lti": "kla_scan_kernel", "mixer_bwd": "kla_state_bwd_kernel",
                "mixer_train": "kla_state_bwd_kernel", "bwd_states": "kla_state_bwd_kernel",
                "scan_train": "kla_state_bwd_kernel"}
# the forward kernel template's last parameter is its mode (scan, mixer, LTI)
KERNEL_SUFFIX = {"fwd": "Mode)0>", "mixer": "Mode)1>", "lti": "Mode)2>",
                 "mixer_bwd": "StateBwdMode)0>", "mixer_train": "StateBwdMode)0>",
                 "bwd_states": "StateBwdMode)1>", "scan_train": "StateBwdMode)1>"}
PROFILE_NAMES = {"fwd": "kla_scan_kernel", "bwd": "kla_scan_bwd_kernel",
                 "decode": "kla_decode_kernel", "mixer_decode": "kla_mixer_decode_kernel",
                 "mixer": "kla_scan_kernel_mixer",
                 "lti": "kla_scan_kernel_lti", "mixer_bwd": "kla_state_bwd_kernel_mixer",
                 "mixer_train": "kla_state_bwd_kernel_mixer",
                 "bwd_states": "kla_state_bwd_kernel_scan", "scan_train": "kla_state_bwd_kernel_scan"}


def is_kernel(name: str, direction: str) -> bool:
    """Whether a rocprofv3 kernel name is the kernel a direction times."""
    return (name.startswith("void kla::(anonymous namespace)::%s<" % KERNEL_NAMES[direction])
            and KERNEL_SUFFIX.get(direction, ">") in name)


def _code_only(text: str) -> str:
    """Source text without comments and blank lines (what the compiler sees)."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def kernel_hash(direction: str = "fwd") -> str:
    """Hash of the code (comments excluded) of the sources a direction's kernel
    is built from; counter records taken from other code do not apply."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[direction]:
        with open(os.path.join(CSRC, name)) as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def bytes_per_element(dtype: str, direction: str = "fwd") -> int:
    """Algorithmic HBM bytes per scanned element.  Forward: 4 gate reads and
    2 float32 writes.  Backward: reads a, p, the saved lam, eta and the
    upstream g_lam, g_eta; writes 4 float32 gradients."""
    gate = 4 if dtype == "f32" else 2
    if direction == "fwd":
        return 4 * gate + 2 * 4
    if direction == "decode":  # 4 gates, state read and written in place
        return 4 * gate + 2 * 4 + 2 * 4
    if direction == "mixer_decode":  # 4 token inputs, state in place, readout and variance
        return 4 * gate + 2 * 4 + 2 * 4 + 2 * 4
    if direction == "mixer":  # k, v, lam_v, q read; readout and variance written
        return 4 * gate + 2 * 4
    if direction == "lti":  # b read (gates once per channel); lam, eta written
        return gate + 2 * 4
    if direction == "mixer_bwd":  # the whole call: recompute (k, v, lam_v read, boundary
        # states written), backward kernel, reduction
        return 3 * gate + 2 + kernel_bytes_per_element(dtype, direction)
    if direction == "mixer_train":  # forward keeping the boundary states, then the backward
        # from them (no recompute)
        return 4 * gate + 2 * 4 + 2 + kernel_bytes_per_element(dtype, "mixer_bwd")
    if direction == "bwd_states":  # the backward kernel from kept states
        return kernel_bytes_per_element(dtype, "bwd_states")
    if direction == "scan_train":  # forward keeping the states, then the backward from them
        return 4 * gate + 2 * 4 + 2 + kernel_bytes_per_element(dtype, "bwd_states")
    return 2 * gate + 4 * 4 + 4 * 4


def kernel_bytes_per_element(dtype: str, direction: str = "fwd") -> int:
    """Algorithmic bytes per element of the direction's dominant kernel.  For
    mixer_bwd that is the backward kernel alone: k, v, lam_v, q, the float64
    boundary state (16 bytes per 8 rows) and the upstream g_out, g_var read;
    g_k, g_v, g_lam_v, g_q written."""
    if direction in ("mixer_bwd", "mixer_train", "bwd_states", "scan_train"):
        # mixer: k, v, lam_v, q, the states, g_out, g_var read; g_k, g_v,
        # g_lam_v, g_q written.  scan: a, p, phi, b, the states, g_lam, g_eta
        # read; g_a, g_p, g_phi, g_b written.
        gate = 4 if dtype == "f32" else 2
        return 4 * gate + 2 + 2 * 4 + 4 * 4
    return bytes_per_element(dtype, direction)


def traffic_path(workload_key: int, direction: str) -> str:
    # a training step's dominant kernel is the mixer backward kernel
    direction = {"mixer_train": "mixer_bwd", "scan_train": "bwd_states"}.get(direction, direction)
    suffix = {"fwd": "", "bwd": "_bwd"}.get(direction, "_" + direction)
    return os.path.join(ROOT, "profiles", "traffic_workload%d%s.json" % (workload_key, suffix))


def load_traffic(workload_key: int, direction: str = "fwd"):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the kernel source changed since the counters were taken."""
    try:
        with open(traffic_path(workload_key, direction)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_sha256_16") != kernel_hash(direction):
        return None
    return rec.get("hbm_bytes_per_launch")


def _counter_kib(path: str, counter: str, match):
    """Mean per-dispatch value (KiB) of a rocprofv3 --pmc counter for kernels
    whose name satisfies match(name), and the number of dispatches."""
    import csv
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(path))
            if r["Counter_Name"] == counter and match(r["Kernel_Name"])]
    if not vals:
        raise SystemExit("no %s rows in %s" % (counter, path))
    return sum(vals) / len(vals), len(vals)


def summarize_counters(args):
    """Writes profiles/traffic_workload<k>.json and a markdown summary from
    rocprofv3 outputs: the kernel-trace stats of the bench command, its
    FETCH_SIZE and WRITE_SIZE runs, and the same two counters on a plain
    device copy of known size (the scale factors)."""
    import csv
    d = args.direction
    w = workloads_for(d)[args.workload]

    def scan(name):
        return is_kernel(name, d)

    def copy(name):
        return name.startswith("__amd_rocclr_copyBuffer")

    stats = [r for r in csv.DictReader(open(args.trace)) if scan(r["Name"])]
    if len(stats) != 1:
        raise SystemExit("expected one scan kernel row in %s" % args.trace)
    st = stats[0]
    fetch, n_f = _counter_kib(args.fetch, "FETCH_SIZE", scan)
    write, n_w = _counter_kib(args.write, "WRITE_SIZE", scan)
    copy_bytes = args.copy_mib << 20
    cf, _ = _counter_kib(args.copy_fetch, "FETCH_SIZE", copy)
    cw, _ = _counter_kib(args.copy_write, "WRITE_SIZE", copy)
    f_fetch = copy_bytes / (cf * 1024.0)
    f_write = copy_bytes / (cw * 1024.0)
    traffic = fetch * 1024.0 * f_fetch + write * 1024.0 * f_write
    algo = w.elements * kernel_bytes_per_element(w.dtype, d)
    avg_ns = float(st["AverageNs"])
    rec = {"workload": w.describe(), "kernel": st["Name"], "kernel_sha256_16": kernel_hash(d),
           "hbm_bytes_per_launch": traffic, "algorithmic_bytes_per_launch": algo,
           "fetch_kib_per_dispatch": fetch, "write_kib_per_dispatch": write,
           "dispatches": [n_f, n_w], "copy_fetch_kib": cf, "copy_write_kib": cw,
           "copy_bytes": copy_bytes, "fetch_scale": f_fetch, "write_scale": f_write,
           "trace_calls": int(st["Calls"]), "trace_avg_ns": avg_ns,
           "trace_min_ns": float(st["MinNs"]), "trace_max_ns": float(st["MaxNs"])}
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(traffic_path(args.workload, d), "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    md = os.path.join(ROOT, "profiles", "%s_%s.md" % (PROFILE_NAMES[d], w.name))
    with open(md, "w") as f:
        f.write("# %s on %s\n\n" % (PROFILE_NAMES[d], w.describe()))
        f.write("Kernel: `%s`  (source sha256/16 `%s`)\n\n" % (st["Name"], kernel_hash(d)))
        f.write("## Kernel trace (rocprofv3 --kernel-trace --stats)\n\n")
        f.write("| calls | average ns | min ns | max ns |\n|---|---|---|---|\n")
        f.write("| %s | %.0f | %s | %s |\n\n" % (st["Calls"], avg_ns, st["MinNs"], st["MaxNs"]))
        f.write("Algorithmic bytes per launch: %d (%d elements x %d B); at the average "
                "duration: %.0f GB/s = %.3f of 8 TB/s.\n\n"
                % (algo, w.elements, kernel_bytes_per_element(w.dtype, d), algo / avg_ns,
                   algo / avg_ns / HBM_PEAK_GBS))
        f.write("## HBM counters (rocprofv3 --pmc, one counter per run)\n\n")
        f.write("| counter | scan KiB/dispatch | plain copy of %d MiB, KiB | scale |\n"
                "|---|---|---|---|\n" % args.copy_mib)
        f.write("| FETCH_SIZE | %.0f | %.0f | %.3f |\n" % (fetch, cf, f_fetch))
        f.write("| WRITE_SIZE | %.0f | %.0f | %.3f |\n\n" % (write, cw, f_write))
        f.write("HBM traffic per launch = FETCH*scale + WRITE*scale = %.0f bytes = %.3f x "
                "algorithmic.\n\n" % (traffic, traffic / algo))
        f.write("## Commands\n\n```\n")
        for line in args.commands:
            f.write(line + "\n")
        f.write("```\n")
    print(md)
    return 0


def per_config_entry(m, direction: str) -> dict:
    """One workload's line of the per-config table: the timed step and the
    kernel time per launch (HIP events on the launch stream), with the
    algorithmic bandwidth and its fraction of the HBM peak."""
    w = m["w"]
    k_avg = sum(m["kernel_ms"]) / len(m["kernel_ms"])
    steps = len(m["kernel_ms"])
    gbs = w.elements * bytes_per_element(w.dtype, direction) / (k_avg * 1e-3) / 1e9
    return {"workload": w.describe(), "elements": w.elements,
            "bytes_per_element": bytes_per_element(w.dtype, direction),
            "ms_per_step": m["wall"] * 1e3 / steps, "kernel_ms_avg": k_avg,
            "kernel_ms_min": min(m["kernel_ms"]), "achieved_GBps": gbs,
            "frac": gbs / HBM_PEAK_GBS, "elements_per_sec": w.elements / (k_avg * 1e-3),
            "eager_launch_ms_median": m["eager_ms"][len(m["eager_ms"]) // 2],
            "health": m["health"]}


def workloads_for(direction: str):
    from kla_inputs import LTI_WORKLOADS, MIXER_WORKLOADS, WORKLOADS
    return {"mixer": MIXER_WORKLOADS, "mixer_bwd": MIXER_WORKLOADS,
            "mixer_train": MIXER_WORKLOADS, "mixer_decode": MIXER_WORKLOADS,
            "lti": LTI_WORKLOADS}.get(direction, WORKLOADS)


def cpu_baseline(w, g_dev, direction: str = "fwd", budget_s: float = 10.0):
    """Times the float64 oracle of a direction on the host, on a bounded sample
    of the workload (its leading (b, h) slabs with every channel and the full
    sequence; every channel for the decode steps), scaled to the direction's
    unit.  The backward and training-step directions time the backward
    oracle, which runs the forward recursion and then the adjoint one."""
    from oracle import (oracle_mixer, oracle_mixer_bwd, oracle_scan, oracle_scan_bwd,
                        oracle_threads)
    d = direction
    threads = len(os.sched_getaffinity(0))
    used = oracle_threads(threads)
    decoding = d in ("decode", "mixer_decode")
    S, T = w.B * w.H, (1 if decoding else w.T)
    per_slab = T * w.D
    # about 10 s of oracle work at its rate on the machine's host cores, and at
    # least one slab per thread (the oracle runs its slabs in parallel)
    cap = 2e8 if d in ("fwd", "lti", "mixer") else 5e7
    n = S if decoding else max(1, min(S, max(used, int(cap // max(per_slab, 1)))))
    heads = np.arange(n) % w.H  # slab s is (b, h) = divmod(s, H)

    def tok(name):  # the sampled slabs of a [B, H, T, D] input, [1, n, T, D] float64
        return (g_dev[name].reshape(S, T, w.D)[:n].to("cpu").double().numpy()
                .reshape(1, n, T, w.D))

    def head(name):  # a per-(h, d) input for the sampled slabs, [n, D]
        return np.ascontiguousarray(g_dev[name].to("cpu").double().numpy()[heads])

    def init(name):  # the sampled slabs' initial state, [1, n, D], or None (1 and 0)
        x = g_dev.get(name)
        return None if x is None else (x.reshape(S, w.D)[:n].to("cpu").double().numpy()
                                       .reshape(1, n, w.D))

    def cut(x, sl):
        return None if x is None else x[:, sl]

    lam0, eta0 = init("lam0"), init("eta0")
    if d in ("mixer", "mixer_decode", "mixer_bwd", "mixer_train"):
        tokens = [tok(k) for k in ("k", "v", "lam_v", "q")]
        a, p = head("a"), head("p")
        if d in ("mixer_bwd", "mixer_train"):
            go, gv = tok("g_out"), tok("g_var")

            def run(sl, nt):
                oracle_mixer_bwd(*(t[:, sl] for t in tokens), a[sl], p[sl], cut(lam0, sl),
                                 cut(eta0, sl), go[:, sl], gv[:, sl], nthreads=nt)
        else:
            def run(sl, nt):
                oracle_mixer(*(t[:, sl] for t in tokens), a[sl], p[sl], cut(lam0, sl),
                             cut(eta0, sl), nthreads=nt)
    else:
        if d == "lti":  # the channel gates broadcast over the sequence, as the oracle reads them
            b = tok("b")
            gates = [np.ascontiguousarray(np.broadcast_to(head(k)[None, :, None, :], b.shape))
                     for k in ("a", "p", "phi")] + [b]
        else:
            gates = [tok(k) for k in ("a", "p", "phi", "b")]
        if d in ("bwd", "bwd_states", "scan_train"):
            gl, ge = tok("g_lam"), tok("g_eta")

            def run(sl, nt):
                oracle_scan_bwd(*(t[:, sl] for t in gates), cut(lam0, sl), cut(eta0, sl),
                                gl[:, sl], ge[:, sl], nthreads=nt)
        else:
            def run(sl, nt):
                oracle_scan(*(t[:, sl] for t in gates), cut(lam0, sl), cut(eta0, sl),
                            nthreads=nt)

    reps, t_total = 0, 0.0
    while t_total < budget_s and reps < 100000:
        t0 = time.perf_counter()
        run(slice(0, n), used)
        t_total += time.perf_counter() - t0
        reps += 1
    # one thread, on one slab
    reps1, t1 = 0, 0.0
    while t1 < budget_s / 4 and reps1 < 100000:
        t0 = time.perf_counter()
        run(slice(0, 1), 1)
        t1 += time.perf_counter() - t0
        reps1 += 1
    what = "one token" if decoding else "full T=%d" % w.T
    return {"value": n * per_slab * reps / t_total, "unit": "elements/sec", "cores": used,
            "kind": "oracle",
            "sample": "%d of %d slabs (all %d channels, %s), %d runs, %.1f s"
                      % (n, S, w.D, what, reps, t_total),
            "value_1thread": per_slab * reps1 / t1,
            "sample_1thread": "1 slab, %d runs, %.1f s, 1 thread" % (reps1, t1)}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=3,
                    help="0..4; the headline is 3 (long context, the largest)")
    ap.add_argument("--per-config", type=lambda x: [int(v) for v in x.split(",") if v],
                    default=[1, 2, 3],
                    help="forward only: workloads measured the same way after the "
                         "headline and reported in per_config (comma list; empty: none)")
    ap.add_argument("--sets", type=int, default=2, help="input/output sets to rotate")
    ap.add_argument("--direction",
                    choices=("fwd", "bwd", "bwd_states", "scan_train", "decode", "mixer",
                             "mixer_bwd", "mixer_train", "mixer_decode", "lti"),
                    default="fwd",
                    help="fwd: kla_scan_fwd (the headline); bwd: kla_scan_bwd; bwd_states: "
                         "kla_scan_bwd_states from the states kla_scan_fwd_states kept; "
                         "scan_train: kla_scan_fwd_states then kla_scan_bwd_states (one "
                         "training step of the scan); decode: "
                         "kla_decode_step on one token of every channel of the workload; "
                         "mixer: kla_mixer_fwd on the mixer workload of the same key; "
                         "mixer_bwd: kla_mixer_bwd on the mixer workload; "
                         "mixer_train: kla_mixer_fwd keeping its states, then kla_mixer_bwd "
                         "from them (one training step of the layer); mixer_decode: "
                         "kla_mixer_decode_step on one token of every channel; "
                         "lti: kla_scan_lti_fwd on the time-invariant workload of that key")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", dest="graph", action="store_false",
                    help="launch the timed steps one by one instead of replaying them "
                         "from a captured HIP graph")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the scan, run torch's plain device copy of MIB MiB "
                         "(known bytes, to scale rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    ap.add_argument("--summarize-counters", action="store_true",
                    help="write profiles/ summaries from rocprofv3 csv files (no GPU)")
    ap.add_argument("--trace"), ap.add_argument("--fetch"), ap.add_argument("--write")
    ap.add_argument("--copy-fetch"), ap.add_argument("--copy-write")
    ap.add_argument("--copy-mib", type=int, default=1024)
    ap.add_argument("--commands", nargs="*", default=[])
    args = ap.parse_args(argv)

    if args.summarize_counters:
        return summarize_counters(args)

    if args.gpus != 1:
        print("bench.py measures one GPU: the scan's channels are independent, so each "
              "GPU of a data-parallel job runs this same kernel on its own share; "
              "--gpus %d is not supported here" % args.gpus, file=sys.stderr)
        return 2

    import torch

    TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}
    if args.copy_calibration:
        n = args.copy_calibration << 18  # float32 elements in MIB MiB
        src = torch.ones(n, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n * 4, "launches": max(1, args.steps)}))
        return 0

    from kla_inputs import make_lti_workload, make_mixer_workload, make_workload
    from linear_attention_sequence_kla_amd import (
        bwd_workspace_size, decode_step, get_workspace, lti_workspace_size, mixer_bwd,
        mixer_bwd_workspace_size, mixer_decode_step, mixer_fwd, mixer_states_shape, scan_bwd,
        scan_fwd, scan_lti_fwd, workspace_health, workspace_size, bwd_states_workspace_size,
        scan_bwd_states, scan_fwd_states, scan_states_shape)

    d = args.direction
    if args.workload not in workloads_for(d):
        print("no workload %d for --direction %s (workloads: %s)"
              % (args.workload, d, ", ".join(map(str, sorted(workloads_for(d))))),
              file=sys.stderr)
        return 2
    def run_one(key):
        """Times K launches of direction d on workload `key` (warm-up first);
        returns the timings and the first input set."""
        w = workloads_for(d)[key]
        dev = torch.device("cuda:0")
        torch.cuda.set_device(dev)
        stream = torch.cuda.current_stream(dev)
        ws = get_workspace(max(workspace_size(*w.shape, TORCH_DTYPE[w.dtype]),
                               bwd_workspace_size(*w.shape, TORCH_DTYPE[w.dtype]),
                               bwd_states_workspace_size(*w.shape, TORCH_DTYPE[w.dtype]),
                               lti_workspace_size(*w.shape, TORCH_DTYPE[w.dtype]),
                               mixer_bwd_workspace_size(*w.shape, TORCH_DTYPE[w.dtype])), dev, stream)
        sets = []
        decoding = d in ("decode", "mixer_decode")
        for k in range(args.sets if not decoding else 0):
            make = {"mixer": make_mixer_workload, "mixer_bwd": make_mixer_workload,
                    "mixer_train": make_mixer_workload, "lti": make_lti_workload}.get(d, make_workload)
            g = make(key, device=dev, seed=w.seed + 1000 * k)
            lam = torch.empty(w.shape, dtype=torch.float32, device=dev)
            eta = torch.empty(w.shape, dtype=torch.float32, device=dev)
            if d in ("bwd_states", "scan_train"):
                g["states"] = torch.empty(scan_states_shape(*w.shape), dtype=torch.float64,
                                          device=dev)
                scan_fwd_states(g["a"], g["p"], g["phi"], g["b"], g["lam0"], g["eta0"],
                                states=g["states"], out=(lam, eta))
            if d in ("bwd", "bwd_states", "scan_train"):
                # the forward outputs are the saved states; upstream gradients ~ N(0, 1)
                scan_fwd(g["a"], g["p"], g["phi"], g["b"], g["lam0"], g["eta0"], out=(lam, eta))
                gen = torch.Generator(device=dev)
                gen.manual_seed(w.seed + 77 + k)
                g["g_lam"] = torch.randn(w.shape, generator=gen, device=dev)
                g["g_eta"] = torch.randn(w.shape, generator=gen, device=dev)
            if d in ("mixer_bwd", "mixer_train"):
                # upstream gradients of the readout and the variance ~ N(0, 1)
                gen = torch.Generator(device=dev)
                gen.manual_seed(w.seed + 77 + k)
                g["g_out"] = torch.randn(w.shape, generator=gen, device=dev)
                g["g_var"] = torch.randn(w.shape, generator=gen, device=dev)
            if d == "mixer_train":
                g["states"] = torch.empty(mixer_states_shape(*w.shape), dtype=torch.float64,
                                          device=dev)
            sets.append((g, (lam, eta)))
        if d == "decode":
            # one token per channel; the state is updated in place each step
            from kla_inputs import make_gates, make_initial_state
            for k in range(args.sets):
                g = make_gates((w.B, w.H, 1, w.D), w.gates, w.dtype, w.seed + 1000 * k, dev)
                g = {n: v[:, :, 0].contiguous() for n, v in g.items()}
                sets.append((g, tuple(x.clone() for x in make_initial_state(
                    w.B, w.H, w.D, random=True, seed=k, device=dev))))
        if d == "mixer_decode":
            # one mixer token per channel; the state is updated in place each step
            from kla_inputs import make_initial_state, make_mixer_inputs
            for k in range(args.sets):
                g = make_mixer_inputs((w.B, w.H, 1, w.D), w.dtype, w.seed + 1000 * k, dev)
                g = {n: (v[:, :, 0] if v.dim() == 4 else v).contiguous() for n, v in g.items()}
                g["out"] = torch.empty((w.B, w.H, w.D), dtype=torch.float32, device=dev)
                g["var"] = torch.empty((w.B, w.H, w.D), dtype=torch.float32, device=dev)
                sets.append((g, tuple(x.clone() for x in make_initial_state(
                    w.B, w.H, w.D, random=True, seed=k, device=dev))))
        grads = None
        if d in ("bwd", "bwd_states", "scan_train"):
            grads = tuple(torch.empty(w.shape, dtype=torch.float32, device=dev) for _ in range(4))
        if d in ("mixer_bwd", "mixer_train"):
            grads = tuple(torch.empty(w.shape, dtype=torch.float32, device=dev) for _ in range(4)) + \
                tuple(torch.empty((w.H, w.D), dtype=torch.float32, device=dev) for _ in range(2))
        torch.cuda.synchronize(dev)

        def step(i):
            g, out = sets[i % len(sets)]
            if d == "decode":
                decode_step(g["a"], g["p"], g["phi"], g["b"], out[0], out[1])
            elif d == "mixer_decode":
                mixer_decode_step(g["k"], g["v"], g["lam_v"], g["q"], g["a"], g["p"], out[0], out[1],
                                  out=g["out"], var=g["var"])
            elif d == "fwd":
                scan_fwd(g["a"], g["p"], g["phi"], g["b"], g["lam0"], g["eta0"], out=out,
                         workspace=ws)
            elif d == "lti":
                scan_lti_fwd(g["a"], g["p"], g["phi"], g["b"], g["lam0"], g["eta0"], out=out,
                             workspace=ws)
            elif d == "mixer_bwd":
                mixer_bwd(g["k"], g["v"], g["lam_v"], g["q"], g["a"], g["p"], g["g_out"], g["g_var"],
                          g["lam0"], g["eta0"], need_state_grads=False, workspace=ws, out=grads)
            elif d == "bwd_states":
                scan_bwd_states(g["a"], g["p"], g["phi"], g["b"], g["g_lam"], g["g_eta"],
                                g["lam0"], g["eta0"], states=g["states"], need_state_grads=False,
                                workspace=ws, out=grads)
            elif d == "scan_train":
                scan_fwd_states(g["a"], g["p"], g["phi"], g["b"], g["lam0"], g["eta0"],
                                states=g["states"], out=out, workspace=ws)
                scan_bwd_states(g["a"], g["p"], g["phi"], g["b"], g["g_lam"], g["g_eta"],
                                g["lam0"], g["eta0"], states=g["states"], need_state_grads=False,
                                workspace=ws, out=grads)
            elif d == "mixer":
                mixer_fwd(g["k"], g["v"], g["lam_v"], g["q"], g["a"], g["p"], g["lam0"], g["eta0"],
                          out=out[0], var=out[1], workspace=ws)
            elif d == "mixer_train":
                mixer_fwd(g["k"], g["v"], g["lam_v"], g["q"], g["a"], g["p"], g["lam0"], g["eta0"],
                          out=out[0], var=out[1], workspace=ws, states=g["states"])
                mixer_bwd(g["k"], g["v"], g["lam_v"], g["q"], g["a"], g["p"], g["g_out"], g["g_var"],
                          g["lam0"], g["eta0"], need_state_grads=False, workspace=ws, out=grads,
                          states=g["states"])
            else:
                scan_bwd(g["a"], g["p"], out[0], out[1], g["g_lam"], g["g_eta"], g["lam0"],
                         g["eta0"], workspace=ws, out=grads)

        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize(dev)

        if args.graph:
            # The K timed launches are captured once into a HIP graph and replayed:
            # the kernels read their epoch from the workspace, so replays need no
            # host work (and the graph holds no memset).
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for i in range(args.steps):
                    step(i)
            torch.cuda.synchronize(dev)
            start = torch.cuda.Event(enable_timing=True)
            end = torch.cuda.Event(enable_timing=True)
            t0 = time.perf_counter()
            start.record(stream)
            graph.replay()
            end.record(stream)
            torch.cuda.synchronize(dev)
            wall = time.perf_counter() - t0
            kernel_ms = [start.elapsed_time(end) / args.steps] * args.steps
        else:
            starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
            ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
            torch.cuda.synchronize(dev)
            t0 = time.perf_counter()
            for i in range(args.steps):
                starts[i].record(stream)
                step(i)
                ends[i].record(stream)
            torch.cuda.synchronize(dev)
            wall = time.perf_counter() - t0
            kernel_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
        # outside the timed region: the per-launch distribution of eager launches
        n_eager = min(20, max(1, args.steps))
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n_eager)]
        for i, (e0, e1) in enumerate(ev):
            e0.record(stream)
            step(i)
            e1.record(stream)
        torch.cuda.synchronize(dev)
        eager_ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
        health = workspace_health(ws)
        if health != 0:
            print("warning: workspace health word %#x" % health, file=sys.stderr)
        return {"w": w, "kernel_ms": kernel_ms, "wall": wall, "eager_ms": eager_ms,
                "n_eager": n_eager, "health": health, "decoding": decoding,
                "first_set": sets[0][0] if sets else None}

    m = run_one(args.workload)
    w, kernel_ms, wall, eager_ms = m["w"], m["kernel_ms"], m["wall"], m["eager_ms"]
    n_eager, health, decoding = m["n_eager"], m["health"], m["decoding"]
    n = w.elements if not decoding else w.channels
    ms_step = wall * 1e3 / args.steps
    k_avg = sum(kernel_ms) / len(kernel_ms)
    bpe = bytes_per_element(w.dtype, d)
    achieved = n * bpe / (k_avg * 1e-3) / 1e9
    traffic = load_traffic(args.workload, d)
    rec = {
        "metric": "KLA scan elements (B·H·T·D)/sec and achieved HBM GB/s vs peak, 1 MI355X",
        "value": n / (ms_step * 1e-3),
        "unit": "elements/sec",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic",
        "config": {"workload": w.describe(), "B": w.B, "H": w.H, "T": w.T, "D": w.D,
                   "io_dtype": w.dtype, "elements": n, "parallelism": "single GPU",
                   "direction": d},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": KERNEL_NAMES[d], "kernel_ms_avg": k_avg,
                     "kernel_ms_min": min(kernel_ms), "bytes_per_element": bpe},
        "health": health,
        "launch": "hip graph of %d launches" % args.steps if args.graph else "eager",
        "eager_launch_ms": {"median": eager_ms[len(eager_ms) // 2], "min": eager_ms[0],
                            "max": eager_ms[-1], "launches": n_eager},
    }
    if d == "bwd":
        rec["metric"] = "KLA backward scan elements (B·H·T·D)/sec and achieved HBM GB/s vs peak"
    if d == "bwd_states":
        rec["metric"] = ("KLA backward scan from float64 states, elements (B·H·T·D)/sec and "
                         "achieved HBM GB/s vs peak")
    if d == "scan_train":
        rec["roofline"]["scope"] = ("the whole step (forward keeping the states, backward "
                                    "from them); traffic is the backward kernel's alone")
        rec["metric"] = ("KLA scan training step (forward keeping states + backward) elements "
                         "(B·H·T·D)/sec and achieved HBM GB/s vs peak")
    if d == "lti":
        rec["metric"] = ("KLA scan with time-invariant gates, elements (B·H·T·D)/sec and "
                         "achieved HBM GB/s vs peak")
    if d == "mixer_bwd":
        rec["roofline"]["scope"] = ("the whole call (state recompute, backward kernel, "
                                    "reduction); traffic is the backward kernel's alone")
        rec["metric"] = ("KLA fused mixer backward elements (B·H·T·D)/sec and achieved HBM GB/s "
                         "vs peak (the whole call: state recompute, adjoint scan, reduction)")
    if d == "mixer_train":
        rec["roofline"]["scope"] = ("the whole step (mixer forward keeping the states, "
                                    "backward kernel, reduction); traffic is the backward "
                                    "kernel's alone")
        rec["metric"] = ("KLA fused mixer training step (forward + backward) elements "
                         "(B·H·T·D)/sec and achieved HBM GB/s vs peak")
    if d == "mixer":
        rec["metric"] = ("KLA fused mixer elements (B·H·T·D)/sec and achieved HBM GB/s vs peak "
                         "(gates, scan, readout and variance in one pass)")
    if d == "decode":
        rec["metric"] = "KLA decode step channel updates (B·H·D)/sec, one token per step"
        rec["config"]["elements"] = n
    if d == "mixer_decode":
        rec["metric"] = ("KLA fused mixer decode step channel updates (B·H·D)/sec, one token "
                         "per step (readout and variance written)")
        rec["config"]["elements"] = n
    if d == "fwd" and args.per_config:
        # the other target workloads, each measured the same way in this process
        rec["per_config"] = [per_config_entry(m, d)]
        for key in args.per_config:
            if key != args.workload:
                rec["per_config"].append(per_config_entry(run_one(key), d))
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, m["first_set"], d)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
