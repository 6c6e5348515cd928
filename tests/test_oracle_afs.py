"""Pins of the reduced-order sweep oracle (oracle/afs.py) against facts that
the page and the mathematics fix, not against a retyping of its formulas.

Page "Solving Dense Matrices Fast in the Browser", section "Fewer frequency
points: adaptive frequency sampling": the reduced model matches the exact
solution at the frequencies solved exactly, and the reduced matrix is
symmetric because the basis is real.
"""
import numpy as np

import oracle
import workloads
from oracle import afs


def _direct(L, Psi, g, w, zs, B):
    return oracle.solve(oracle.assemble(w, zs, L, Psi, g), B)


def test_basis_is_orthonormal_and_spans_its_inputs():
    rng = np.random.default_rng(3)
    n = 40
    X = rng.standard_normal((3, n)) + 1j * rng.standard_normal((3, n))
    V = afs.extend_basis(np.zeros((0, n)), X)
    assert V.shape == (6, n)
    assert np.abs(V @ V.T - np.eye(6)).max() < 1e-14
    # every real and imaginary part lies in the span: its projection is itself
    for part in np.concatenate([X.real, X.imag]):
        assert np.linalg.norm(part - (V @ part) @ V) < 1e-13 * np.linalg.norm(part)
    # a vector already in the span adds nothing
    V2 = afs.extend_basis(V, (X[0] + 2.0 * X[1]).reshape(1, n))
    assert V2.shape == V.shape


def test_reduced_matrix_is_symmetric():
    rng = np.random.default_rng(5)
    n = 30
    L, Psi, g, _ = workloads.make_matrices(n, seed=2)
    X = rng.standard_normal((4, n)) + 1j * rng.standard_normal((4, n))
    V = afs.extend_basis(np.zeros((0, n)), X)
    Zr = afs.reduced_matrix(1.3, 0.01 + 0.01j, V @ L @ V.T, V @ Psi @ V.T, (V * g) @ V.T)
    assert np.abs(Zr - Zr.T).max() <= 1e-14 * np.abs(Zr).max()
    assert np.abs(Zr - np.conj(Zr.T)).max() > 1e-3 * np.abs(Zr).max()   # symmetric, not Hermitian


def test_galerkin_exact_at_solved_frequencies():
    wl = workloads.make_quasistatic_workload(64, nfreq=17)
    B = np.vstack([wl.B, np.arange(64) % 5 - 2.0 + 0.5j])
    r = afs.afs(wl.L, wl.Psi, wl.g, wl.omega, wl.zs, B)
    assert r["exact"][:2] == [0, 16]
    for f in r["exact"]:
        xe = _direct(wl.L, wl.Psi, wl.g, wl.omega[f], wl.zs[f], B)
        assert oracle.forward_error(r["X"][f], xe).max() < 1e-11
        assert r["estimate"][f] < 1e-10


def test_full_basis_reproduces_every_direct_solve():
    # n = 6: three exact solves give 2 x 3 = 6 independent real directions,
    # so V spans R^6 and the reduced model is exact at every frequency
    wl = workloads.make_workload(workloads.config(0), n=6, nfreq=9)
    r = afs.afs(wl.L, wl.Psi, wl.g, wl.omega, wl.zs, wl.B, tol=0.0, max_exact=3)
    assert len(r["exact"]) == 3 and r["q"] == 6
    for f in range(9):
        xe = _direct(wl.L, wl.Psi, wl.g, wl.omega[f], wl.zs[f], wl.B)
        assert oracle.forward_error(r["X"][f], xe).max() < 1e-10
        assert r["estimate"][f] < 1e-12


def test_diagonal_closed_form():
    # L = Psi = I: Z is diagonal, z_i(w) = j (w - 1/w) + Zs(w) g_i, and with
    # b = e_0 + 2 e_3 every solution lies in span{e_0, e_3}: two directions,
    # reached by the first exact solve, after which every estimate is ~0
    n, nf = 8, 7
    rng = np.random.default_rng(11)
    g = rng.uniform(0.5, 1.5, n)
    om = np.linspace(0.5, 2.0, nf)
    zs = workloads.zs_values(om, 0.01)
    b = np.zeros((1, n), complex)
    b[0, 0], b[0, 3] = 1.0, 2.0
    r = afs.afs(np.eye(n), np.eye(n), g, om, zs, b)
    assert r["exact"] == [0, nf - 1] and r["q"] == 2
    for f in range(nf):
        z = 1j * (om[f] - 1.0 / om[f]) + zs[f] * g
        x = b[0] / z
        assert np.abs(r["X"][f, 0] - x).max() <= 1e-14 * np.abs(x).max()
        assert r["estimate"][f] < 1e-14


def test_quasistatic_sweep_needs_few_exact_solves():
    # below the first resonance the response is smooth: few exact solves
    # reach the page's stopping residual at every candidate
    wl = workloads.make_quasistatic_workload(128, nfreq=41)
    r = afs.afs(wl.L, wl.Psi, wl.g, wl.omega, wl.zs, wl.B)
    assert len(r["exact"]) <= 8
    assert r["estimate"].max() <= 1e-4
    for f in range(0, 41, 5):
        xe = _direct(wl.L, wl.Psi, wl.g, wl.omega[f], wl.zs[f], wl.B)
        assert oracle.forward_error(r["X"][f], xe).max() < 1e-3


def test_cap_on_exact_solves():
    wl = workloads.make_quasistatic_workload(48, nfreq=11)
    r = afs.afs(wl.L, wl.Psi, wl.g, wl.omega, wl.zs, wl.B, tol=0.0, max_exact=2)
    assert r["exact"] == [0, 10]
    r1 = afs.afs(wl.L, wl.Psi, wl.g, wl.omega[:1], wl.zs[:1], wl.B)
    assert r1["exact"] == [0] and r1["X"].shape == (1, 1, 48)


def _galerkin_error(monkeypatch, attr, fn):
    monkeypatch.setattr(afs, attr, fn)
    wl = workloads.make_quasistatic_workload(48, nfreq=9)
    r = afs.afs(wl.L, wl.Psi, wl.g, wl.omega, wl.zs, wl.B, tol=0.0, max_exact=3)
    f = r["exact"][-1]
    xe = _direct(wl.L, wl.Psi, wl.g, wl.omega[f], wl.zs[f], wl.B)
    return oracle.forward_error(r["X"][f], xe).max()


def test_pins_reject_a_wrong_sign_in_the_reduced_matrix(monkeypatch):
    bad = lambda w, zs, VLV, VPV, VGV: 1j * w * VLV + 1j * VPV / w + complex(zs) * VGV
    assert _galerkin_error(monkeypatch, "reduced_matrix", bad) > 1e-6


def test_pins_reject_a_basis_without_imaginary_parts(monkeypatch):
    good = afs.extend_basis
    bad = lambda V, X: good(V, np.atleast_2d(X).real + 0j)
    assert _galerkin_error(monkeypatch, "extend_basis", bad) > 1e-6
