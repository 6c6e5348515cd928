"""The oracle's stored full-size solutions (tests/golden/oracle_*.npz, written
by golden/make_oracle_solutions.py) hold what the GPU tests rely on: every
frequency the oracle solves, a backward error <= 1e-14 for each solution
(the acceptance rule of the oracle's direct solve), the oracle's own
reciprocity (Z^T = Z) to 1e-12, and the frequencies of the workload.  At
n = 4096 the inputs are regenerated and matched by digest, and a few stored
solutions are re-checked against the oracle's compensated residual."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from golden_io import input_digest, load_oracle_solutions

NAMES = ["n8000_1freq", "n4096_41freq_resonance", "n16384_8freq"]


def frequencies_for(spec):
    return list(spec.oracle_freq) if spec.oracle_freq is not None else list(range(spec.nfreq))


@pytest.mark.parametrize("name", NAMES)
def test_stored_solutions_are_complete_and_accepted(name):
    spec = workloads.config_by_name(name)
    gold = load_oracle_solutions(name)
    assert gold is not None, "missing tests/golden/oracle_%s.npz" % name
    assert str(gold["workload"]) == name and int(gold["n"]) == spec.n
    idx = [int(f) for f in gold["omega_index"]]
    assert idx == frequencies_for(spec)
    omega = np.linspace(spec.omega_lo, spec.omega_hi, spec.nfreq)
    assert np.array_equal(gold["omega"], omega[idx])
    nrhs = 1 if spec.rhs == "random" else len(spec.unit_index)
    assert gold["X"].shape == (len(idx), nrhs, spec.n)
    assert np.all(np.isfinite(gold["X"]))
    assert np.all(gold["eta"] <= 1e-14)
    assert np.all(gold["recip"] <= 1e-12)
    # row 1-norms as stated
    assert np.allclose(gold["x_norm1"], np.abs(gold["X"]).sum(axis=2), rtol=1e-12, atol=0)


def test_stored_n4096_solutions_match_inputs_and_oracle_residual():
    wl = workloads.make_workload(workloads.config_by_name("n4096_41freq_resonance"))
    gold = load_oracle_solutions(wl.spec.name)
    assert gold is not None
    assert str(gold["digest"]) == input_digest(wl)
    for i in (0, 20, 40):
        f = int(gold["omega_index"][i])
        Z = oracle.assemble(wl.omega[f], wl.zs[f], wl.L, wl.Psi, wl.g)
        assert oracle.norm_inf_mat(Z) == gold["z_norm_inf"][i]
        assert np.all(oracle.eta(Z, gold["X"][i], wl.B) <= 1e-14)
