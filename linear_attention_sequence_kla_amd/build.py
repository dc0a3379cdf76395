"""Builds libkla.so (the HIP kernels and the C ABI) in-tree for gfx950, and
libkla_debug.so, the same library with pseudo-random pauses before every
carry flag is published and before each slice of the mixer's channel-gate
reduction counts itself (a test build that forces the look-back through all
its orders and the reduction's last arrival onto other workgroups; see
kla_lookback.h).

    python -m linear_attention_sequence_kla_amd.build
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(HERE, "csrc", f)
           for f in ("kla_api.cpp", "kla_scan_fwd.hip", "kla_scan_bwd.hip", "kla_decode.hip",
                     "kla_noalloc.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(HERE, "libkla.so")
DEBUG_LIBRARY = os.path.join(HERE, "libkla_debug.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
    "-fvisibility=hidden",
    # no packed fp32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build(out: str = LIBRARY, extra=(), verbose: bool = False) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-I", INCLUDE, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build_debug(verbose: bool = False) -> str:
    return build(DEBUG_LIBRARY, extra=("-DKLA_DEBUG_DELAYS",), verbose=verbose)


COPY_SOURCE = os.path.join(ROOT, "bench_copy.hip")
COPY_BINARY = os.path.join(ROOT, "bench_copy")


def build_copy_bench(verbose: bool = False) -> str:
    """Builds bench_copy (the standalone copy prototypes of the forward
    scan's memory structure, a measurement tool outside the library)."""
    tmp = COPY_BINARY + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", COPY_SOURCE, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, COPY_BINARY)
    return COPY_BINARY


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_debug(verbose=True))
    print(build_copy_bench(verbose=True))
    sys.exit(0)
