"""libkla: forward Kalman Linear Attention (KLA) scan on AMD MI355X (gfx950).

The work happens in ``libkla.so`` (HIP kernels behind a C ABI declared in
``include/kla.h``); ``kla`` is its ctypes binding.
"""

from .kla import (  # noqa: F401
    KlaError, LIBRARY, get_workspace, library, scan_fwd, workspace_health, workspace_size)
