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


import oracle_bwd_pins  # noqa: E402

BWD_MUTANTS = {
    "bwd-dropped-square-in-lambda-chain": ("const double dl_dlp = at * at / d2;",
                                           "const double dl_dlp = at / d2;"),
    "bwd-wrong-sign-of-coupling": ("const double de_dlp = -at * pt * ep / d2;",
                                   "const double de_dlp = at * pt * ep / d2;"),
    "bwd-state-one-token-late": ("const double lp = LAM[t - 1];", "const double lp = LAM[t];"),
    "bwd-eta-carry-without-gate": ("ce = de_dep * Eta;", "ce = Eta;"),
    "bwd-decay-grad-missing-eta-term": ("g_a[i] = Lam * dl_da + Eta * de_da;",
                                        "g_a[i] = Lam * dl_da;"),
    "bwd-lambda-carry-missing-coupling": ("cl = dl_dlp * Lam + de_dlp * Eta;",
                                          "cl = dl_dlp * Lam;"),
    "bwd-wrong-sign-in-decay-derivative": ("ep * (pt * lp - at * at) / d2",
                                           "ep * (pt * lp + at * at) / d2"),
    "bwd-noise-derivative-missing-square": ("const double dl_dp = -lp * lp / d2;",
                                            "const double dl_dp = -lp / d2;"),
    "bwd-upstream-ignored-in-total": ("const double Lam = g_lam[i] + cl;",
                                      "const double Lam = cl;"),
    "bwd-magnitude-missing-term": (
        "m_a[i] = MLam * fabs(dl_da) + MEta * eap * (pt * lp + at * at) / d2;",
        "m_a[i] = MLam * fabs(dl_da);"),
    "bwd-initial-gradient-from-magnitude": ("me = de_dep * MEta;\n    }\n    *g_lam0 = cl;",
                                            "me = de_dep * MEta;\n    }\n    *g_lam0 = ml;"),
}


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_bwd_mutant_is_caught(name, tmp_path):
    old, new = BWD_MUTANTS[name]
    src = open(SOURCE).read()
    assert src.count(old) == 1, "mutation site not unique: %r" % old
    mutant_src = tmp_path / "mutant.c"
    mutant_src.write_text(src.replace(old, new, 1))
    lib = OracleLibrary(build_oracle(str(tmp_path / "libmutant.so"), str(mutant_src)))

    def scan(a, p, phi, b, lam0, eta0):
        return lib.scan(a, p, phi, b, lam0, eta0)

    def scan_bwd(a, p, phi, b, lam0, eta0, g_lam, g_eta):
        return lib.scan_bwd(a, p, phi, b, lam0, eta0, g_lam, g_eta)

    caught = []
    for pin in oracle_bwd_pins.ALL_BWD_PINS:
        try:
            pin(scan_bwd, scan)
        except (AssertionError, FloatingPointError, ValueError, ZeroDivisionError) as e:
            caught.append((pin.__name__, str(e)[:80]))
    assert caught, "no pin caught mutant %s" % name


import oracle_mixer_pins  # noqa: E402

MIXER_MUTANTS = {
    "mixer-gain-without-operator": ("const double K = Ppred * kt * lv[i] / S;",
                                    "const double K = Ppred * lv[i] / S;"),
    "mixer-innovation-ignores-operator": ("(v[i] - kt * mupred)", "(v[i] - mupred)"),
    "mixer-precision-linear-in-operator": ("1.0 + kt * kt * lv[i] * Ppred",
                                           "1.0 + kt * lv[i] * Ppred"),
    "mixer-readout-without-q": ("out[i] = q[i] * MU[t + 1];", "out[i] = MU[t + 1];"),
    "mixer-variance-not-updated": ("mu = mupred + K * (v[i] - kt * mupred);\n        P = Ppred / S;",
                                   "mu = mupred + K * (v[i] - kt * mupred);\n        P = Ppred;"),
    "mixer-decay-not-squared": ("const double Ppred = a * a * P + p;",
                                "const double Ppred = a * P + p;"),
    "mixer-noise-dropped": ("const double Ppred = a * a * P + p;",
                            "const double Ppred = a * a * P;"),
    "mixer-final-precision-as-variance": ("*lamT = 1.0 / PV[T];", "*lamT = PV[T];"),
    "mixer-signed-magnitude": ("fabs(kt * lv[i] * v[i])", "(kt * lv[i] * v[i])"),
    "mixer-wrong-channel-gates": ("(slab % H) * D + d;\n            const int64_t base = slab * T * D + d;\n            double *PV",
                                  "(slab / H) * D + d;\n            const int64_t base = slab * T * D + d;\n            double *PV"),
    "mixer-variance-one-token-early": ("var[i] = PV[t + 1];", "var[i] = PV[t];"),
    "mixer-prior-mean-ignored": ("    double mu = eta0 / lam0;\n    double mag = fabs(eta0);\n    PV[0] = P;",
                                 "    double mu = 0.0;\n    double mag = fabs(eta0);\n    PV[0] = P;"),
}


@pytest.mark.parametrize("name", sorted(MIXER_MUTANTS))
def test_mixer_mutant_is_caught(name, tmp_path):
    old, new = MIXER_MUTANTS[name]
    src = open(SOURCE).read()
    assert src.count(old) == 1, "mutation site not unique: %r" % old
    mutant_src = tmp_path / "mutant.c"
    mutant_src.write_text(src.replace(old, new, 1))
    lib = OracleLibrary(build_oracle(str(tmp_path / "libmutant.so"), str(mutant_src)))

    def mixer(k, v, lam_v, q, a, p, lam0, eta0):
        return lib.mixer(k, v, lam_v, q, a, p, lam0, eta0)

    caught = []
    for pin in oracle_mixer_pins.ALL_MIXER_PINS:
        try:
            pin(mixer)
        except (AssertionError, FloatingPointError, ValueError, ZeroDivisionError) as e:
            caught.append((pin.__name__, str(e)[:80]))
    assert caught, "no pin caught mutant %s" % name


import oracle_mixer_bwd_pins  # noqa: E402

MIXER_BWD_MUTANTS = {
    "mbwd-readout-precision-adjoint-sign": ("const double gl_dir = -(g_out[i] * qt * eta + g_var[i])",
                                            "const double gl_dir = (g_out[i] * qt * eta + g_var[i])"),
    "mbwd-variance-adjoint-dropped": ("-(g_out[i] * qt * eta + g_var[i]) / (lam * lam)",
                                      "-(g_out[i] * qt * eta) / (lam * lam)"),
    "mbwd-operator-grad-missing-2": ("g_k[i] = Lam * 2.0 * kt * lvt", "g_k[i] = Lam * kt * lvt"),
    "mbwd-readout-grad-unscaled": ("g_q[i] = g_out[i] * eta / lam;", "g_q[i] = g_out[i] * eta;"),
    "mbwd-eta-carry-without-gate": ("ce = a / d * Eta;", "ce = Eta;"),
    "mbwd-batch-sum-overwrites": ("g_a[hd] += part[4 * c];", "g_a[hd] = part[4 * c];"),
    "mbwd-precision-grad-missing-term": ("g_lv[i] = Lam * kt * kt + Eta * kt * vt;",
                                         "g_lv[i] = Lam * kt * kt;"),
    "mbwd-noise-grad-sign": ("gp += Lam * (-lp * lp / d2)", "gp += Lam * (lp * lp / d2)"),
    "mbwd-value-grad-missing-precision": ("g_v[i] = Eta * kt * lvt;", "g_v[i] = Eta * kt;"),
    "mbwd-coupling-dropped": ("cl = a * a / d2 * Lam - a * p * ep / d2 * Eta;",
                              "cl = a * a / d2 * Lam;"),
}


@pytest.mark.parametrize("name", sorted(MIXER_BWD_MUTANTS))
def test_mixer_bwd_mutant_is_caught(name, tmp_path):
    old, new = MIXER_BWD_MUTANTS[name]
    src = open(SOURCE).read()
    assert src.count(old) == 1, "mutation site not unique: %r" % old
    mutant_src = tmp_path / "mutant.c"
    mutant_src.write_text(src.replace(old, new, 1))
    lib = OracleLibrary(build_oracle(str(tmp_path / "libmutant.so"), str(mutant_src)))

    def mixer_bwd(**kw):
        return lib.mixer_bwd(**kw)

    def mixer(*args):
        return lib.mixer(*args)

    caught = []
    for pin in oracle_mixer_bwd_pins.ALL_MIXER_BWD_PINS:
        try:
            pin(mixer_bwd, mixer)
        except (AssertionError, FloatingPointError, ValueError, ZeroDivisionError) as e:
            caught.append((pin.__name__, str(e)[:80]))
    assert caught, "no pin caught mutant %s" % name
