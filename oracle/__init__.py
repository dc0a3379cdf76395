"""CPU float64 oracle for the KLA scan (forward, backward) and the fused mixer.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this package.  It shares no code with
the HIP library under ``linear_attention_sequence_kla_amd`` and never imports
it.  Every function here is pinned by ``tests/test_oracle_pins.py``.
"""

from .kla_oracle import (  # noqa: F401
    LIBRARY, SOURCE, OracleLibrary, build_oracle, oracle_mixer, oracle_mixer_bwd, oracle_scan,
    oracle_scan_bwd, oracle_threads)
