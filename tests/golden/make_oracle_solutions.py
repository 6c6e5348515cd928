"""Writes the oracle's direct solutions of the full-size workloads to
tests/golden/oracle_<workload>.npz.

At these sizes the oracle's complex128 LU with partial pivoting takes from a
minute (n = 8000) to half an hour (n = 16384) per frequency on a host, too
long to repeat inside every GPU test run, so its answers are stored.  This
script calls only the seeded input generator (``workloads``) and the oracle
(``oracle``); nothing here touches the GPU library.

For every stored frequency the file holds:

* ``X`` -- the oracle's solution, complex128, one row per right-hand side;
* ``eta`` -- the oracle's own normwise backward error of that solution
  (compensated residual), which must be <= 1e-14 to be accepted;
* ``x_norm1`` -- the 1-norm of each solution row; for a unit right-hand
  side e_k and a symmetric Z this is the 1-norm of row k of Z^-1, which
  bounds how far a residual can move entry k of any other solution;
* ``z_norm_inf`` -- ||Z(w)||_inf;
* ``recip`` -- the oracle's own reciprocity defect over the pairs of unit
  right-hand sides (Z^T = Z makes it zero in exact arithmetic);
* a SHA-256 digest of the generated L, Psi, g and B, so a test can check
  that its generator produced the same inputs.

The frequencies are those the oracle is asked to solve: all of them, except
for the n = 16384 workload, where it solves the two end frequencies.

Usage (from the repository root):
    python tests/golden/make_oracle_solutions.py n8000_1freq n4096_41freq_resonance
    python tests/golden/make_oracle_solutions.py n16384_8freq

The output is rewritten after every frequency, so an interrupted run keeps
what it finished and a rerun continues from there.
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
TESTS = os.path.dirname(HERE)
ROOT = os.path.dirname(TESTS)
for p in (ROOT, TESTS):
    if p not in sys.path:
        sys.path.insert(0, p)

import oracle      # noqa: E402
import workloads   # noqa: E402
from golden_io import input_digest, oracle_solutions_path as golden_path   # noqa: E402

ETA_ACCEPT = 1e-14


def frequencies_for(spec) -> list:
    if spec.oracle_freq is not None:
        return list(spec.oracle_freq)
    return list(range(spec.nfreq))


def load_partial(path: str, digest: str):
    if not os.path.exists(path):
        return {}
    with np.load(path, allow_pickle=False) as d:
        if str(d["digest"]) != digest:
            return {}
        out = {}
        for i, f in enumerate(d["omega_index"]):
            out[int(f)] = (d["X"][i], d["eta"][i], d["x_norm1"][i],
                           float(d["z_norm_inf"][i]), float(d["recip"][i]))
        return out


def save(path: str, name: str, digest: str, done: dict, wl) -> None:
    idx = sorted(done)
    tmp = path + ".tmp.npz"
    np.savez(tmp,
             workload=np.array(name),
             digest=np.array(digest),
             n=np.array(wl.n, dtype=np.int64),
             omega_index=np.array(idx, dtype=np.int64),
             omega=np.array([wl.omega[f] for f in idx], dtype=np.float64),
             X=np.stack([done[f][0] for f in idx]).astype(np.complex128),
             eta=np.stack([done[f][1] for f in idx]).astype(np.float64),
             x_norm1=np.stack([done[f][2] for f in idx]).astype(np.float64),
             z_norm_inf=np.array([done[f][3] for f in idx], dtype=np.float64),
             recip=np.array([done[f][4] for f in idx], dtype=np.float64))
    os.replace(tmp, path)


def make(name: str) -> None:
    spec = workloads.config_by_name(name)
    t0 = time.time()
    wl = workloads.make_workload(spec)
    digest = input_digest(wl)
    path = golden_path(name)
    done = load_partial(path, digest)
    print("%s: inputs generated in %.1f s, %d of %d frequencies already stored"
          % (name, time.time() - t0, len(done), len(frequencies_for(spec))), flush=True)
    for f in frequencies_for(spec):
        if f in done:
            continue
        t = time.time()
        Z = oracle.assemble(wl.omega[f], wl.zs[f], wl.L, wl.Psi, wl.g)
        X = oracle.solve(Z, wl.B)
        eta = oracle.eta(Z, X, wl.B)
        if not np.all(eta <= ETA_ACCEPT):
            raise RuntimeError("%s w[%d]: oracle backward error %s above %g"
                               % (name, f, eta, ETA_ACCEPT))
        x1 = np.abs(X).sum(axis=1)
        zn = oracle.norm_inf_mat(Z)
        rc = oracle.reciprocity(X, wl.unit_cols) if len(wl.unit_cols) > 1 else 0.0
        done[f] = (X, eta, x1, zn, rc)
        save(path, name, digest, done, wl)
        print("%s w[%d]=%.6f: oracle solve %.1f s, eta %s, reciprocity %.3g"
              % (name, f, wl.omega[f], time.time() - t, np.array2string(eta, precision=3), rc),
              flush=True)
        del Z


if __name__ == "__main__":
    names = sys.argv[1:] or ["n8000_1freq", "n4096_41freq_resonance", "n16384_8freq"]
    for nm in names:
        make(nm)
