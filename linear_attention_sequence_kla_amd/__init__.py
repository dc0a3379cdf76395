"""libkla: the Kalman Linear Attention (KLA) scan on AMD MI355X (gfx950):
forward and backward scan, time-invariant-gate scan, fused mixer (forward
and backward), decode steps of the scan and of the mixer.

The work happens in ``libkla.so`` (HIP kernels behind a C ABI declared in
``include/kla.h``); ``kla`` is its ctypes binding.
"""

from .kla import (  # noqa: F401
    KLAMixer, KLAScan, KlaError, KlaHealthError, LIBRARY, bwd_workspace_size, decode_step,
    get_workspace, health_checks_enabled, set_health_checks,
    kla_mixer, kla_scan, library, lti_workspace_size, mixer_bwd, mixer_bwd_workspace_size,
    mixer_decode_step, mixer_fwd, mixer_states_shape, mixer_workspace_size, scan_bwd, scan_fwd,
    scan_fwd_noalloc, scan_lti_fwd, workspace_health, workspace_size, scan_fwd_states,
    scan_bwd_states, scan_states_shape, bwd_states_workspace_size)
