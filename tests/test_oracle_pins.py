"""The float64 oracle against its pins (CPU only)."""

import numpy as np
import pytest

import oracle_pins
from oracle import oracle_scan


def scan(a, p, phi, b, lam0, eta0):
    return oracle_scan(a, p, phi, b, lam0, eta0)


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(scan)


def test_threads_reported():
    from oracle import oracle_threads
    assert oracle_threads(2) == 2
    assert oracle_threads(1) == 1


def test_default_initial_state():
    a = np.full((1, 1, 1, 1), 1.0)
    lam, eta, eta_abs = oracle_scan(a, a, a, a)  # lam0 = 1, eta0 = 0
    # P = 1 -> Ppred = 2, S = 3, mu = 2/3, P = 2/3
    assert lam.item() == pytest.approx(1.5, rel=1e-15)
    assert eta.item() == pytest.approx(1.0, rel=1e-15)
    assert eta_abs.item() == pytest.approx(1.0, rel=1e-15)


def test_empty_time_axis():
    a = np.zeros((2, 1, 0, 3))
    lam, eta, eta_abs = oracle_scan(a, a, a, a)
    assert lam.shape == (2, 1, 0, 3)


def test_regression_fixture():
    """The oracle still reproduces tests/golden/oracle_regression.json, and the
    fixture itself agrees with the information-form recursion."""
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "oracle_regression.json")
    fx = json.load(open(path))
    inp = fx["input"]
    T, D = len(inp["a"]), len(inp["a"][0])
    g = [np.array(inp[k], dtype=np.float64).reshape(1, 1, T, D) for k in ("a", "p", "phi", "b")]
    lam0 = np.array(inp["lam0"]).reshape(1, 1, D)
    eta0 = np.array(inp["eta0"]).reshape(1, 1, D)
    lam, eta, eta_abs = oracle_scan(*g, lam0, eta0)
    np.testing.assert_allclose(lam.reshape(T, D), fx["lam"], rtol=1e-15)
    np.testing.assert_allclose(eta.reshape(T, D), fx["eta"], rtol=1e-15, atol=1e-300)
    np.testing.assert_allclose(eta_abs.reshape(T, D), fx["eta_abs"], rtol=1e-15)
    lam_i, eta_i = oracle_pins.info_form(*g, lam0, eta0)
    np.testing.assert_allclose(lam_i.reshape(T, D), fx["lam"], rtol=1e-13)
    np.testing.assert_allclose(eta_i.reshape(T, D), fx["eta"], rtol=1e-13, atol=1e-12)


import oracle_bwd_pins  # noqa: E402
from oracle import oracle_scan_bwd  # noqa: E402


@pytest.mark.parametrize("pin", oracle_bwd_pins.ALL_BWD_PINS, ids=lambda f: f.__name__)
def test_bwd_pin(pin):
    pin(oracle_scan_bwd, scan)


import oracle_mixer_pins  # noqa: E402


@pytest.mark.parametrize("pin", oracle_mixer_pins.ALL_MIXER_PINS, ids=lambda f: f.__name__)
def test_mixer_pin(pin):
    from oracle import oracle_mixer
    pin(oracle_mixer)


import oracle_mixer_bwd_pins  # noqa: E402


@pytest.mark.parametrize("pin", oracle_mixer_bwd_pins.ALL_MIXER_BWD_PINS,
                         ids=lambda f: f.__name__)
def test_mixer_bwd_pin(pin):
    from oracle import oracle_mixer, oracle_mixer_bwd
    pin(oracle_mixer_bwd, oracle_mixer)
