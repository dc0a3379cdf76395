"""Planted mistakes in the oracle must be caught by its pins.

Each case copies ``oracle/kla_oracle.c``, plants one plausible mistake by a
textual substitution (a dropped term, a wrong sign, a wrong operand or index),
builds the copy into a temporary library on the CPU and runs every pin on it:
at least one pin must fail.  The real oracle is never modified.
"""

import pytest

import oracle_pins
from oracle import SOURCE, OracleLibrary, build_oracle

MUTANTS = {
    "dropped-square-in-predict": ("at * at * P + pt", "at * P + pt"),
    "dropped-process-noise": ("at * at * P + pt;", "at * at * P;"),
    "mean-not-propagated": ("mupred = at * mu;", "mupred = mu;"),
    "stale-variance-in-gain": ("1.0 + phit * Ppred", "1.0 + phit * P"),
    "wrong-sign-of-evidence": ("(mupred + Ppred * bt)", "(mupred - Ppred * bt)"),
    "posterior-variance-not-updated": ("P = Ppred / S;", "P = Ppred;"),
    "eta-scaled-wrong-way": ("eta[i] = mu / P;", "eta[i] = mu * P;"),
    "forget-gate-transposed": ("f = at * P / Ppred;", "f = at * Ppred / P;"),
    "magnitude-without-forgetting": ("mag = f * mag + fabs(bt);", "mag = mag + fabs(bt);"),
    "signed-magnitude": ("mag = f * mag + fabs(bt);", "mag = f * mag + bt;"),
    "gate-read-one-token-late": ("const double at = a[i];",
                                 "const double at = a[t + 1 < T ? i + stride : i];"),
    "initial-mean-ignored": ("double mu = eta0 / lam0;", "double mu = 0.0;"),
    "initial-precision-as-variance": ("double P = 1.0 / lam0;", "double P = lam0;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SOURCE).read()
    assert src.count(old) >= 1, "mutation site vanished: %r" % old
    mutant_src = tmp_path / "mutant.c"
    mutant_src.write_text(src.replace(old, new, 1))
    lib = OracleLibrary(build_oracle(str(tmp_path / "libmutant.so"), str(mutant_src)))

    def scan(a, p, phi, b, lam0, eta0):
        return lib.scan(a, p, phi, b, lam0, eta0)

    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(scan)
        except (AssertionError, FloatingPointError, ValueError, ZeroDivisionError) as e:
            caught.append((pin.__name__, str(e)[:80]))
    assert caught, "no pin caught mutant %s" % name
