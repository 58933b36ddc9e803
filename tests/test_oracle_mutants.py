"""The oracle's pins must catch plausible mistakes.

Each case below plants one mistake in a temporary copy of the oracle's C
source (a dropped term, a wrong sign, a wrong operand or index, a wrong
order), compiles it, and runs the pin suite against it in a subprocess; the
pin suite must fail.  The unmodified source must pass the same run.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "gdn_oracle.c")

MUTANTS = {
    "decay_dropped": ("S[(size_t)c * dk + j] = a * (s - bt * Sk[c] * k[j])",
                      "S[(size_t)c * dk + j] = (s - bt * Sk[c] * k[j])"),
    "erase_sign_flipped": ("a * (s - bt * Sk[c] * k[j])", "a * (s + bt * Sk[c] * k[j])"),
    "erase_beta_dropped": ("a * (s - bt * Sk[c] * k[j])", "a * (s - Sk[c] * k[j])"),
    "write_term_dropped": ("+ bt * v[c] * k[j];", ";"),
    "gate_not_exponentiated": ("exp(gval(J, J->g, b, j, h))", "(1.0 + gval(J, J->g, b, j, h))"),
    "readout_uses_key": ("gdn_readout(Si, d->dv, d->dk, qvec(J, b, i, kh), o);",
                         "gdn_readout(Si, d->dv, d->dk, kvec(J, b, i, kh), o);"),
    "head_map_modulo": ("int kh = h / (d->Hv / d->Hk);", "int kh = h % d->Hk;"),
    "memo_ignores_parent": ("const double *Sp = par[i] < 0 ? S0 : Sall + (size_t)par[i] * ss;",
                            "const double *Sp = S0;"),
    "memo_uses_previous_node": ("const double *Sp = par[i] < 0 ? S0 : Sall + (size_t)par[i] * ss;",
                                "const double *Sp = i == 0 ? S0 : Sall + (size_t)(i - 1) * ss;"),
    "readout_before_update": ("gdn_readout(Si, d->dv, d->dk, qvec(J, b, i, kh), o);",
                              "gdn_readout(Sp, d->dv, d->dk, qvec(J, b, i, kh), o);"),
    "commit_stops_at_parent": ("for (int t = 0; t < len; ++t) step_node(J, S, b, path[t], h, kh, Sk);\n        }\n        memcpy(Snew",
                               "for (int t = 0; t + 1 < len; ++t) step_node(J, S, b, path[t], h, kh, Sk);\n        }\n        memcpy(Snew"),
    "value_head_swapped": ("return J->v + (((size_t)b * d->N + i) * d->Hv + h) * d->dv;",
                           "return J->v + (((size_t)b * d->N + i) * d->Hv + (d->Hv - 1 - h)) * d->dv;"),
    "ancestor_depth_off_by_one": ("depth[(size_t)b * N + i] = d;", "depth[(size_t)b * N + i] = d - 1;"),
}


def run_pins(lib_path):
    env = dict(os.environ, GDN_ORACLE_LIB_OVERRIDE=lib_path, PYTHONDONTWRITEBYTECODE="1")
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                          env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)


def build_variant(tmp_path, name, text):
    src = tmp_path / f"{name}.c"
    src.write_text(text)
    return oracle.build(str(src), str(tmp_path / f"lib{name}.so"))


def test_unmodified_source_passes(tmp_path):
    lib = build_variant(tmp_path, "clean", open(SRC).read())
    r = run_pins(lib)
    assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(tmp_path, name):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    lib = build_variant(tmp_path, name, text.replace(old, new))
    r = run_pins(lib)
    assert r.returncode != 0, f"pins did not catch mutant {name}"
