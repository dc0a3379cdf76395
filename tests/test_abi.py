"""The C ABI on the CPU: the library loads, exports what include/kla.h
declares, sizes its workspace, and rejects bad arguments before touching the
GPU (none of these calls launch anything)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kla.h")


@pytest.fixture(scope="module")
def lib():
    from linear_attention_sequence_kla_amd import library
    return library()


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"KLA_API\s+[\w\s\*]*?\b(kla_\w+)\s*\(", text)


def test_header_declares_entry_points():
    names = declared_functions()
    assert {"kla_scan_fwd", "kla_scan_fwd_workspace_size", "kla_status_string",
            "kla_last_error_detail", "kla_workspace_health"} <= set(names)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code, name in enumerate(["KLA_OK", "KLA_ERR_INVALID_ARG", "KLA_ERR_UNSUPPORTED",
                                 "KLA_ERR_WORKSPACE", "KLA_ERR_HIP"]):
        assert lib.kla_status_string(code).decode() == name


def test_workspace_size(lib):
    ws = lib.kla_scan_fwd_workspace_size
    assert ws(0, 1, 1, 1, 0) == 0          # empty problem
    assert ws(-1, 1, 1, 1, 0) == 0         # invalid
    assert ws(1, 1, 1, 1, 7) == 0          # unknown dtype
    assert ws(2 ** 40, 2 ** 40, 1, 1, 0) == 0  # overflow
    small = ws(1, 1, 256, 16, 0)
    assert small > 256 and small % 8 == 0
    # grows with the number of tiles: bfloat16 tiles are shorter (96 rows
    # against 112), so the same problem has more of them
    assert ws(8, 16, 2048, 64, 0) > small
    assert ws(8, 16, 2048, 64, 1) > ws(8, 16, 2048, 64, 0)
    assert ws(8, 16, 96 * 22, 64, 1) == ws(8, 16, 112 * 22, 64, 0)


def _call(lib, a=1, p=1, phi=1, b=1, dtype=0, lam=0x1000000, eta=0x2000000,
          shape=(1, 1, 4, 4), ws=0x4000000, ws_bytes=1 << 20):
    vp = ctypes.c_void_p
    B, H, T, D = shape
    st = lib.kla_scan_fwd(vp(a * 0x100000), vp(p * 0x200000), vp(phi * 0x300000),
                          vp(b * 0x400000), dtype, None, None, vp(lam), vp(eta),
                          B, H, T, D, vp(ws), ws_bytes, None)
    return st, lib.kla_last_error_detail().decode()


def test_argument_errors_before_launch(lib):
    # Fake pointers: safe only where no GPU could run a launch that slipped through.
    import torch
    if torch.cuda.is_available():
        pytest.skip("uses fake device pointers; argument errors are tested on GPUs elsewhere")
    # null gate
    st, msg = _call(lib, a=0)
    assert st == 1 and "a is NULL" in msg
    # negative size
    st, msg = _call(lib, shape=(1, -1, 4, 4))
    assert st == 1 and "negative" in msg
    # unknown dtype
    st, _ = _call(lib, dtype=5)
    assert st == 2
    # null workspace / too small / misaligned
    st, _ = _call(lib, ws=0)
    assert st == 3
    st, msg = _call(lib, ws_bytes=16)
    assert st == 3 and "needs" in msg
    st, _ = _call(lib, ws=0x4000010)
    assert st == 3
    # output overlapping an input
    st, msg = _call(lib, lam=0x100000)
    assert st == 1 and "overlaps" in msg
    # misaligned output
    st, _ = _call(lib, lam=0x1000002)
    assert st == 2
    # outputs overlapping each other, and the workspace
    st, msg = _call(lib, eta=0x1000004)
    assert st == 1 and "overlaps" in msg
    st, msg = _call(lib, ws=0x1000000 - 256)
    assert st == 1 and "overlaps" in msg
    # empty problem: nothing to do, no pointer needed
    st, _ = _call(lib, a=0, shape=(1, 1, 0, 4))
    assert st == 0
    # a wave's 64 channels straddle slabs (D not a multiple of 64) too far
    # apart for 32-bit offsets
    st, msg = _call(lib, shape=(1, 1, 1 << 25, 65), ws_bytes=1 << 62)
    assert st == 2 and "too large" in msg
    # with D a multiple of 64 the offsets stay within the wave's rows: any T
    # passes the size checks (here the fake buffers then overlap)
    st, msg = _call(lib, shape=(1, 1, 1 << 25, 64), ws_bytes=1 << 62)
    assert st == 1 and "overlaps" in msg


def test_health_rejects_null(lib):
    out = ctypes.c_uint32(0)
    assert lib.kla_workspace_health(None, ctypes.byref(out), None) == 3


def _mixer_call(lib, k=1, a=0x500000, out=0x1000000, var=0x2000000, lam_T=0, eta_T=0,
                states=0, shape=(2, 1, 4, 4), ws=0x4000000, ws_bytes=1 << 20):
    vp = ctypes.c_void_p
    B, H, T, D = shape
    st = lib.kla_mixer_fwd(vp(k * 0x100000), vp(0x200000), vp(0x300000), vp(0x400000), 0,
                           vp(a), vp(0x600000), None, None, vp(out), vp(var), vp(lam_T),
                           vp(eta_T), vp(states), B, H, T, D, vp(ws), ws_bytes, None)
    return st, lib.kla_last_error_detail().decode()


def test_mixer_workspace_size(lib):
    """float32 mixer tiles equal the scan's (28 rows x 4 waves); bfloat16
    mixer tiles hold 36 rows per wave against the scan's 24, so a bfloat16
    mixer over 144 * n rows needs what a bfloat16 scan over 96 * n rows does."""
    for shape in ((1, 1, 256, 16), (8, 16, 2048, 64), (3, 5, 77, 9)):
        assert (lib.kla_mixer_fwd_workspace_size(*shape, 0)
                == lib.kla_scan_fwd_workspace_size(*shape, 0))
        assert 0 < lib.kla_mixer_fwd_workspace_size(*shape, 1) <= \
            lib.kla_scan_fwd_workspace_size(*shape, 1)
    for n in (1, 7, 30):
        assert (lib.kla_mixer_fwd_workspace_size(2, 3, 144 * n, 40, 1)
                == lib.kla_scan_fwd_workspace_size(2, 3, 96 * n, 40, 1))
    assert lib.kla_mixer_fwd_workspace_size(0, 3, 144, 40, 1) == 0
    assert lib.kla_mixer_fwd_workspace_size(1, 3, 144, 40, 5) == 0


def test_mixer_argument_errors_before_launch(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("uses fake device pointers; argument errors are tested on GPUs elsewhere")
    st, msg = _mixer_call(lib, k=0)
    assert st == 1 and "k is NULL" in msg
    st, msg = _mixer_call(lib, a=0)
    assert st == 1 and "a is NULL" in msg
    st, msg = _mixer_call(lib, out=0)
    assert st == 1 and "out is NULL" in msg
    st, msg = _mixer_call(lib, lam_T=0x3000000)
    assert st == 1 and "both" in msg
    st, msg = _mixer_call(lib, var=0x100000)
    assert st == 1 and "overlaps" in msg
    st, msg = _mixer_call(lib, lam_T=0x3000000, eta_T=0x3000010)
    assert st == 1 and "overlaps" in msg
    st, msg = _mixer_call(lib, ws_bytes=16)
    assert st == 3 and "needs" in msg
    st, msg = _mixer_call(lib, states=0x3000008)
    assert st == 2 and "16-byte" in msg
    st, msg = _mixer_call(lib, states=0x1000000 - 64)  # runs into out
    assert st == 1 and "overlaps" in msg
    st, _ = _mixer_call(lib, k=0, shape=(1, 1, 0, 4))
    assert st == 0


def test_mixer_states_size(lib):
    sz = lib.kla_mixer_states_size
    assert sz(0, 1, 1, 1) == 0 and sz(-1, 1, 1, 1) == 0 and sz(2 ** 40, 2 ** 40, 1, 1) == 0
    # float64 (lam, eta) of every channel after every 8th token
    for B, H, T, D in ((1, 1, 1, 1), (2, 3, 8, 5), (2, 3, 9, 5), (8, 16, 2048, 64)):
        assert sz(B, H, T, D) == ((T + 7) // 8) * B * H * D * 16


def test_lti_workspace_size(lib):
    ws = lib.kla_scan_lti_fwd_workspace_size
    assert ws(0, 1, 1, 1, 0) == 0
    assert ws(1, 1, 1, 1, 7) == 0
    assert 256 < ws(8, 16, 2048, 64, 0) <= lib.kla_scan_fwd_workspace_size(8, 16, 2048, 64, 0)


def test_lti_argument_errors_before_launch(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("uses fake device pointers; argument errors are tested on GPUs elsewhere")
    vp = ctypes.c_void_p

    def call(a=0x100000, b=0x400000, lam=0x1000000, ws_bytes=1 << 20):
        st = lib.kla_scan_lti_fwd(vp(a), vp(0x200000), vp(0x300000), vp(b), 0, None, None,
                                  vp(lam), vp(0x2000000), 2, 1, 4, 4, vp(0x4000000), ws_bytes,
                                  None)
        return st, lib.kla_last_error_detail().decode()
    st, msg = call(a=0)
    assert st == 1 and "a is NULL" in msg
    st, msg = call(b=0)
    assert st == 1 and "b is NULL" in msg
    st, msg = call(lam=0x400000)
    assert st == 1 and "overlaps" in msg
    st, msg = call(ws_bytes=16)
    assert st == 3


def test_mixer_bwd_workspace_size(lib):
    ws = lib.kla_mixer_bwd_workspace_size
    assert ws(0, 1, 1, 1, 0) == 0
    assert ws(1, 1, 1, 1, 9) == 0
    n = 8 * 16 * 2048 * 64
    big = ws(8, 16, 2048, 64, 0)
    # holds the recomputed float64 states after every 8th row (2 bytes per
    # element) and the carry records
    assert big >= 2 * n + lib.kla_scan_fwd_workspace_size(8, 16, 2048, 64, 0)
    assert big < 4 * n + lib.kla_scan_fwd_workspace_size(8, 16, 2048, 64, 0)
    assert big % 256 == 0


def test_mixer_bwd_argument_errors_before_launch(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("uses fake device pointers; argument errors are tested on GPUs elsewhere")
    vp = ctypes.c_void_p
    shape = (2, 1, 4, 4)
    need = lib.kla_mixer_bwd_workspace_size(*shape, 0)

    def call(k=0x100000, g_out=0x700000, g_k=0x1000000, g_a=0x1800000, ws=0x4000000,
             ws_bytes=need, states=0):
        st = lib.kla_mixer_bwd(vp(k), vp(0x200000), vp(0x300000), vp(0x400000), 0,
                               vp(0x500000), vp(0x600000), None, None, vp(states), vp(g_out),
                               None,
                               vp(g_k), vp(0x1100000), vp(0x1200000), vp(0x1300000), vp(g_a),
                               vp(0x1900000), None, None, *shape, vp(ws), ws_bytes, None)
        return st, lib.kla_last_error_detail().decode()
    st, msg = call(k=0)
    assert st == 1 and "k is NULL" in msg
    st, msg = call(g_out=0)
    assert st == 1 and "g_out is NULL" in msg
    st, msg = call(g_a=0)
    assert st == 1 and "g_a is NULL" in msg
    st, msg = call(g_k=0x700000)
    assert st == 1 and "overlaps" in msg
    st, msg = call(ws_bytes=need - 8)
    assert st == 3 and "needs" in msg
    st, _ = call(ws=0x4000010)
    assert st == 3
    st, msg = call(states=0x3000008)
    assert st == 2 and "16-byte" in msg
    st, msg = call(states=0x1000000 - 64)  # g_k is written over the states
    assert st == 1 and "overlaps" in msg


def test_mixer_decode_argument_errors_before_launch(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("uses fake device pointers; argument errors are tested on GPUs elsewhere")
    vp = ctypes.c_void_p

    def call(k=0x100000, n=24, hd=12, out=0x1000000, lam=0x800000, var=0):
        st = lib.kla_mixer_decode_step(vp(k), vp(0x200000), vp(0x300000), vp(0x400000), 0,
                                       vp(0x500000), vp(0x600000), vp(lam), vp(0x900000),
                                       vp(out), vp(var), n, hd, None)
        return st, lib.kla_last_error_detail().decode()
    st, msg = call(k=0)
    assert st == 1 and "k is NULL" in msg
    st, msg = call(out=0)
    assert st == 1 and "out is NULL" in msg
    st, msg = call(n=25)
    assert st == 1 and "multiple" in msg
    st, msg = call(hd=0)
    assert st == 1
    st, msg = call(n=-1)
    assert st == 1
    st, msg = call(out=0x800000 + 16)  # the readout runs into the state
    assert st == 1 and "overlaps" in msg
    st, msg = call(var=0x100000 + 8)   # the variance would overwrite k
    assert st == 1 and "overlaps" in msg
    st, _ = call(k=0, n=0)
    assert st == 0


def test_states_sizes(lib):
    """The scan's float64 states: 16 bytes per channel per 8 tokens, as the
    mixer's; the backward-from-states workspace holds them and the carry
    records."""
    for shape in ((1, 1, 256, 16), (8, 16, 2048, 64), (3, 5, 77, 9)):
        B, H, T, D = shape
        assert lib.kla_scan_states_size(*shape) == ((T + 7) // 8) * B * H * D * 16
        assert lib.kla_scan_states_size(*shape) == lib.kla_mixer_states_size(*shape)
        ws = lib.kla_scan_bwd_states_workspace_size(*shape, 0)
        assert ws >= lib.kla_scan_states_size(*shape) and ws % 256 == 0
        assert ws >= lib.kla_scan_fwd_workspace_size(*shape, 0)
    assert lib.kla_scan_states_size(0, 1, 8, 1) == 0
    assert lib.kla_scan_bwd_states_workspace_size(1, 1, 8, 1, 9) == 0


def test_states_argument_errors_before_launch(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("uses fake device pointers; argument errors are tested on GPUs elsewhere")
    vp = ctypes.c_void_p
    shape = (2, 1, 40, 4)
    fwd_need = lib.kla_scan_fwd_workspace_size(*shape, 0)
    bwd_need = lib.kla_scan_bwd_states_workspace_size(*shape, 0)

    def fwd(states=0x3000000, lam=0x1000000):
        st = lib.kla_scan_fwd_states(vp(0x100000), vp(0x200000), vp(0x300000), vp(0x400000), 0,
                                     None, None, vp(lam), vp(0x2000000), vp(states), *shape,
                                     vp(0x4000000), fwd_need, None)
        return st, lib.kla_last_error_detail().decode()

    st, msg = fwd(states=0)
    assert st == 1 and "states is NULL" in msg
    st, msg = fwd(states=0x3000008)
    assert st == 2 and "16-byte" in msg
    st, msg = fwd(states=0x1000000 - 64)  # lam is written over the states
    assert st == 1 and "overlaps" in msg

    def bwd(a=0x100000, g_a=0x1000000, states=0, ws_bytes=bwd_need, g_lam=0x700000):
        st = lib.kla_scan_bwd_states(vp(a), vp(0x200000), vp(0x300000), vp(0x400000), 0, None,
                                     None, vp(states), vp(g_lam), None, vp(g_a),
                                     vp(0x1100000), vp(0x1200000), vp(0x1300000), None, None,
                                     *shape, vp(0x4000000), ws_bytes, None)
        return st, lib.kla_last_error_detail().decode()

    st, msg = bwd(a=0)
    assert st == 1 and "a is NULL" in msg
    st, msg = bwd(g_a=0)
    assert st == 1 and "g_a is NULL" in msg
    st, msg = bwd(ws_bytes=bwd_need - 8)
    assert st == 3 and "needs" in msg
    st, msg = bwd(g_a=0x700000)  # a gradient over the upstream gradient
    assert st == 1 and "overlaps" in msg
    st, msg = bwd(states=0x3000008)
    assert st == 2 and "16-byte" in msg
    # empty problem: nothing to do
    st = lib.kla_scan_bwd_states(None, None, None, None, 0, None, None, None, None, None, None,
                                 None, None, None, None, None, 1, 1, 0, 4, None, 0, None)
    assert st == 0
