"""The pins must reject a broken oracle.

Each case plants one plausible slip in a copy of oracle/oracle.c (on the
CPU), builds it, and runs the pin suite against it in a subprocess; the
suite must fail.  The real oracle is never modified.
"""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, text in oracle.c, replacement)
MUTANTS = [
    ("assembly_sign_of_psi", "double im = wl - pw;", "double im = wl + pw;"),
    ("assembly_drops_g_reactance", "im = im + zi * gi;", "im = im;"),
    ("assembly_g_into_wrong_part", "re = zr * gi;", "re = zi * gi;"),
    ("gepp_rhs_not_exchanged", "RE(y, a) = RE(y, b); IM(y, a) = IM(y, b);",
     "(void)b;"),
    ("gepp_update_sign", "ai[2 * j] = ai[2 * j] - mr;", "ai[2 * j] = ai[2 * j] + mr;"),
    ("gepp_no_pivoting", "if (m > best) { best = m; p = i; }",
     "if (i == k) { best = m; p = i; }"),
    ("forward_subst_imag_cross_term", "si = si - (ar * vi + aim * vr);",
     "si = si - (ar * vi - aim * vr);"),
    ("smith_division_sign", "*ei = (b - a * r) / den;", "*ei = (a * r - b) / den;"),
    ("residual_uncompensated", "*c = *c + (ep + es);", "*c = *c;"),
    ("residual_imag_sign", "dot2_acc(&si, &ci, -b, xr);", "dot2_acc(&si, &ci, b, xr);"),
    ("lu_nopivot_update_sign", "ai[2 * j] = ai[2 * j] - (lr * ur - li * ui);",
     "ai[2 * j] = ai[2 * j] + (lr * ur - li * ui);"),
    ("norm_l1_modulus", "s = s + hypot(RE(Z, k), IM(Z, k));",
     "s = s + fabs(RE(Z, k)) + fabs(IM(Z, k));"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_reject_mutant(name, old, new, tmp_path):
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation site missing: " + name
    mutated = src.replace(old, new, 1)
    csrc = tmp_path / "oracle_mut.c"
    csrc.write_text(mutated)
    lib = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
                    "-std=c11", str(csrc), "-o", str(lib), "-lm"], check=True)
    env = dict(os.environ, ORACLE_LIB_OVERRIDE=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, "pins accepted a broken oracle (%s)\n%s" % (name, r.stdout[-2000:])
