"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: hand-worked
fixtures, Cramer's rule, exact rational elimination, closed forms, invariants
and manufactured solutions.  A plausible slip in the oracle (a dropped term,
a sign, a transposed operand, a missed row exchange in the right-hand side)
fails at least one of them.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest

import exact
import golden_io
import oracle
import workloads

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def _cplx(re, im) -> np.ndarray:
    return golden_io.as_float(re) + 1j * golden_io.as_float(im)


# ---------------------------------------------------------------- assembly

def test_assembly_golden_2x2_bit_exact():
    d = golden_io.load("assembly_solve_2x2.txt")
    L = golden_io.as_float(d["L"])
    Psi = golden_io.as_float(d["Psi"])
    g = golden_io.as_float(d["g"])
    zs = complex(float(d["zs_re"]), float(d["zs_im"]))
    Z = oracle.assemble(float(d["omega"]), zs, L, Psi, g)
    Zg = _cplx(d["Z_re"], d["Z_im"])
    assert np.array_equal(Z, Zg)


def test_assembly_diagonal_closed_form_bit_exact():
    d = golden_io.load("diagonal_closed_form.txt")
    n = int(d["n"])
    I = np.eye(n)
    g = golden_io.as_float(d["g"])
    zs = complex(float(d["zs_re"]), float(d["zs_im"]))
    Z = oracle.assemble(float(d["omega"]), zs, I, I, g)
    assert np.array_equal(Z, _cplx(d["Z_re"], d["Z_im"]))


def test_assembly_resonance_leaves_only_zs_g():
    # L = Psi and w = 1: the reactive part w L - Psi / w vanishes exactly,
    # leaving Z = Zs G (diagonal).
    rng = np.random.default_rng(3)
    n = 7
    S = rng.standard_normal((n, n))
    S = S + S.T
    g = rng.uniform(0.5, 1.5, n)
    zs = 0.3 - 0.7j
    Z = oracle.assemble(1.0, zs, S, S, g)
    expect = np.diag(zs.real * g + 1j * (zs.imag * g))
    assert np.array_equal(Z, expect)


def test_assembly_terms_separately():
    # Each term of the model equation alone, at w = 4 (a power of two, so
    # scaling by w and 1/w is exact): jwL, then -jPsi/w, then Zs G.
    rng = np.random.default_rng(5)
    n = 6
    A = rng.standard_normal((n, n))
    A = A + A.T
    zero = np.zeros((n, n))
    g0 = np.zeros(n)
    w = 4.0
    Z1 = oracle.assemble(w, 0j, A, zero, g0)
    assert np.array_equal(Z1.real, np.zeros((n, n)))
    assert np.array_equal(Z1.imag, 4.0 * A)
    Z2 = oracle.assemble(w, 0j, zero, A, g0)
    assert np.array_equal(Z2.real, np.zeros((n, n)))
    assert np.array_equal(Z2.imag, -0.25 * A)
    g = rng.uniform(0.5, 1.5, n)
    Z3 = oracle.assemble(w, 2.0 + 0.5j, zero, zero, g)
    assert np.array_equal(Z3, np.diag(2.0 * g + 1j * 0.5 * g))


def test_assembly_symmetric_and_real_part_diagonal():
    wl = workloads.make_workload(workloads.config(0), n=64, nfreq=3)
    for w, zs in zip(wl.omega, wl.zs):
        Z = oracle.assemble(w, zs, wl.L, wl.Psi, wl.g)
        assert np.array_equal(Z, Z.T)
        off = ~np.eye(64, dtype=bool)
        assert np.all(Z.real[off] == 0.0)
        assert np.all(Z.real.diagonal() > 0.0)


# ------------------------------------------------------------ direct solve

def test_solve_golden_2x2():
    d = golden_io.load("assembly_solve_2x2.txt")
    Z = _cplx(d["Z_re"], d["Z_im"])
    b = _cplx(d["b_re"], d["b_im"]).reshape(1, -1)
    xg = _cplx(d["x_re"], d["x_im"])
    x = oracle.solve(Z, b)[0]
    assert np.max(np.abs(x - xg)) <= 4 * np.finfo(float).eps * np.max(np.abs(xg))


def test_solve_diagonal_closed_form():
    d = golden_io.load("diagonal_closed_form.txt")
    Z = _cplx(d["Z_re"], d["Z_im"])
    b = _cplx(d["b_re"], d["b_im"]).reshape(1, -1)
    xg = _cplx(d["x_re"], d["x_im"])
    x = oracle.solve(Z, b)[0]
    assert np.max(np.abs(x - xg)) <= 4 * np.finfo(float).eps


@pytest.mark.parametrize("n", [1, 2, 3, 4])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_solve_matches_cramer(n, seed):
    rng = np.random.default_rng(100 + seed)
    Z = rng.standard_normal((n, n)) + 1j * rng.standard_normal((n, n))
    b = rng.standard_normal(n) + 1j * rng.standard_normal(n)
    x = oracle.solve(Z, b.reshape(1, n))[0]
    xc = exact.cramer_solve(Z, b)
    kappa = np.linalg.cond(Z)
    assert np.max(np.abs(x - xc)) <= 50 * kappa * np.finfo(float).eps * np.max(np.abs(xc))


@pytest.mark.parametrize("n", [2, 3, 5, 6])
def test_solve_matches_exact_rationals(n):
    # dyadic inputs (k / 8): exactly representable, so the exact solution of
    # the binary system is the reference, rounded once at the end
    rng = np.random.default_rng(200 + n)
    Z = (rng.integers(-16, 17, (n, n)) + 1j * rng.integers(-16, 17, (n, n))) / 8.0
    Z += np.diag(np.full(n, 0.125))
    b = (rng.integers(-8, 9, n) + 1j * rng.integers(-8, 9, n)) / 8.0
    xe = [exact.to_complex(v) for v in exact.gauss_solve(exact.matrix(Z), exact.vector(b))]
    xe = np.array(xe)
    x = oracle.solve(Z, b.reshape(1, n))[0]
    kappa = np.linalg.cond(Z)
    assert np.max(np.abs(x - xe)) <= 20 * n * kappa * np.finfo(float).eps * np.max(np.abs(xe))


def test_solve_needs_row_exchange():
    # a zero leading pivot: elimination without row exchanges would divide by
    # zero; the oracle must exchange rows (in the right-hand side too)
    Z = np.array([[0, 1, 0], [1, 0, 0], [0, 0, 2]], dtype=np.complex128)
    B = np.array([[3 + 1j, 5 - 2j, 4j]])
    x = oracle.solve(Z, B)[0]
    assert np.array_equal(x, np.array([5 - 2j, 3 + 1j, 2j]))


def test_solve_pivot_order_first_maximum():
    # |a_00| < |a_10|: the row with the largest modulus goes first.  The
    # result is the same either way in exact arithmetic; with 1e-20 on the
    # diagonal, elimination without the exchange loses every digit.
    Z = np.array([[1e-20, 1], [1, 1]], dtype=np.complex128)
    b = np.array([[1.0 + 0j, 2.0 + 0j]])
    x = oracle.solve(Z, b)[0]
    xe = np.array([1.0 / (1 - 1e-20), (1 - 2e-20) / (1 - 1e-20)])
    assert np.max(np.abs(x - xe)) <= 4e-16


def test_solve_singular_detected():
    Z = np.array([[1, 2], [2, 4]], dtype=np.complex128)
    with pytest.raises(oracle.SingularError):
        oracle.solve(Z, np.array([[1, 0]], dtype=np.complex128))


def test_solve_manufactured_solution_exact_rhs():
    # b = Z x_true computed exactly in rationals, rounded once
    n = 12
    wl = workloads.make_workload(workloads.config(0), n=n, nfreq=2)
    Z = oracle.assemble(wl.omega[1], wl.zs[1], wl.L, wl.Psi, wl.g)
    rng = np.random.default_rng(9)
    xt = rng.standard_normal(n) + 1j * rng.standard_normal(n)
    bq = exact.matvec(exact.matrix(Z), exact.vector(xt))
    b = np.array([exact.to_complex(v) for v in bq])
    x = oracle.solve(Z, b.reshape(1, n))[0]
    kappa = np.linalg.cond(Z)
    err = np.max(np.abs(x - xt)) / np.max(np.abs(xt))
    assert err <= 10 * n * kappa * np.finfo(float).eps
    assert oracle.eta(Z, x.reshape(1, n), b.reshape(1, n))[0] <= 1e-15


def test_solve_reciprocity_and_backward_error_config0():
    # Z^T = Z, so (Z^-1)_mk = (Z^-1)_km: solutions for e_k and e_m agree at
    # the swapped indices.
    wl = workloads.make_workload(workloads.config(0))
    cols = [0, 17, 128, 255]
    B = np.zeros((len(cols), wl.n), dtype=np.complex128)
    for r, k in enumerate(cols):
        B[r, k] = 1.0
    for w, zs in zip(wl.omega, wl.zs):
        Z = oracle.assemble(w, zs, wl.L, wl.Psi, wl.g)
        X = oracle.solve(Z, B)
        assert oracle.reciprocity(X, cols) <= 1e-13
        assert np.all(oracle.eta(Z, X, B) <= 1e-14)


def test_solve_agrees_with_lapack_config0():
    # test-only cross-check against LAPACK (zgesv), within the conditioning
    wl = workloads.make_workload(workloads.config(0))
    for w, zs in zip(wl.omega, wl.zs):
        Z = oracle.assemble(w, zs, wl.L, wl.Psi, wl.g)
        X = oracle.solve(Z, wl.B)
        Xl = np.linalg.solve(Z, wl.B.T).T
        kappa = np.linalg.cond(Z)
        assert oracle.forward_error(X, Xl)[0] <= 10 * kappa * np.finfo(float).eps


def test_solve_multiple_rhs_independent():
    wl = workloads.make_workload(workloads.config(0), n=40, nfreq=1)
    Z = oracle.assemble(wl.omega[0], wl.zs[0], wl.L, wl.Psi, wl.g)
    B = workloads.random_rhs(np.random.default_rng(4), 40, 3)
    X = oracle.solve(Z, B)
    for r in range(3):
        assert np.array_equal(X[r], oracle.solve(Z, B[r:r + 1])[0])


def test_solve_permutation_equivariance():
    # P Z P^T (P x) = P b: relabelling the unknowns permutes the answer
    wl = workloads.make_workload(workloads.config(0), n=30, nfreq=1)
    Z = oracle.assemble(wl.omega[0], wl.zs[0], wl.L, wl.Psi, wl.g)
    b = workloads.random_rhs(np.random.default_rng(8), 30, 1)
    p = np.random.default_rng(6).permutation(30)
    x = oracle.solve(Z, b)[0]
    xp = oracle.solve(Z[np.ix_(p, p)], b[:, p])[0]
    assert np.max(np.abs(xp - x[p])) <= 1e-13 * np.max(np.abs(x))


# ---------------------------------------------- LU without row exchanges

def _integer_factors(n, rng):
    Lt = np.tril(rng.integers(-2, 3, (n, n)), -1) + np.eye(n)
    Ut = np.triu(rng.integers(-3, 4, (n, n)), 1) + np.diag(2.0 ** rng.integers(0, 3, n))
    Lt = Lt + 1j * np.tril(rng.integers(-1, 2, (n, n)), -1)
    Ut = Ut + 1j * np.triu(rng.integers(-1, 2, (n, n)), 1)
    return Lt.astype(np.complex128), Ut.astype(np.complex128)


def test_lu_nopivot_exact_integer_factors():
    rng = np.random.default_rng(11)
    n = 9
    Lt, Ut = _integer_factors(n, rng)
    A = Lt @ Ut                            # exact: small integers
    F = oracle.lu_nopivot(A)
    packed = np.tril(Lt, -1) + Ut
    assert np.array_equal(F, packed)


def test_lu_nopivot_reconstructs_and_symmetric_structure():
    # an unpivoted LU of a symmetric matrix has U = diag(U) L^T
    wl = workloads.make_workload(workloads.config(0), n=96, nfreq=1)
    Z = oracle.assemble(wl.omega[0], wl.zs[0], wl.L, wl.Psi, wl.g)
    F = oracle.lu_nopivot(Z)
    Lf = np.tril(F, -1) + np.eye(96)
    Uf = np.triu(F)
    assert np.max(np.abs(Lf @ Uf - Z)) <= 1e-13 * np.max(np.abs(Z))
    Ud = np.diag(np.diag(Uf)) @ Lf.T
    assert np.max(np.abs(Ud - Uf)) <= 1e-12 * np.max(np.abs(Uf))


def test_lu_nopivot_reports_zero_pivot():
    A = np.array([[0, 1], [1, 0]], dtype=np.complex128)
    with pytest.raises(oracle.SingularError):
        oracle.lu_nopivot(A)


def test_lu_solve_exact_integer_systems():
    rng = np.random.default_rng(12)
    n = 10
    Lt, Ut = _integer_factors(n, rng)
    xt = rng.integers(-4, 5, (2, n)) + 1j * rng.integers(-4, 5, (2, n))
    B = (Lt @ Ut @ xt.T).T                   # exact integers
    packed = np.tril(Lt, -1) + Ut
    X = oracle.lu_solve(packed, B)
    assert np.array_equal(X, xt.astype(np.complex128))


def test_lu_solve_matches_gepp_when_no_exchange_needed():
    # diagonally dominant: partial pivoting keeps the natural order
    rng = np.random.default_rng(13)
    n = 50
    A = rng.standard_normal((n, n)) + 1j * rng.standard_normal((n, n))
    A += np.diag(np.full(n, 4.0 * n))
    b = workloads.random_rhs(rng, n, 2)
    x1 = oracle.lu_solve(oracle.lu_nopivot(A), b)
    x2 = oracle.solve(A, b)
    assert np.max(np.abs(x1 - x2)) <= 1e-15 * np.max(np.abs(x2))


# --------------------------------------------------------------- residual

def test_residual_exact_on_integers():
    rng = np.random.default_rng(14)
    n = 31
    Z = (rng.integers(-50, 51, (n, n)) + 1j * rng.integers(-50, 51, (n, n))).astype(np.complex128)
    X = (rng.integers(-50, 51, (2, n)) + 1j * rng.integers(-50, 51, (2, n))).astype(np.complex128)
    B = (rng.integers(-500, 501, (2, n)) + 1j * rng.integers(-500, 501, (2, n))).astype(np.complex128)
    R = oracle.residual(Z, X, B)
    Ri = B - (Z.astype(np.complex128) @ X.T).T   # integer-valued, exact in float64 here
    assert np.array_equal(R, Ri)


def test_residual_compensated_under_cancellation():
    # b = Z x rounded, so b - Z x is a tiny number left after cancelling
    # terms of size ~1; plain float64 summation loses most of its digits,
    # the compensated residual must match the exact rational result.
    rng = np.random.default_rng(15)
    n = 16
    Z = rng.standard_normal((n, n)) + 1j * rng.standard_normal((n, n))
    x = rng.standard_normal(n) + 1j * rng.standard_normal(n)
    b = Z @ x
    R = oracle.residual(Z, x.reshape(1, n), b.reshape(1, n))[0]
    Zq, xq, bq = exact.matrix(Z), exact.vector(x), exact.vector(b)
    zx = exact.matvec(Zq, xq)
    re = np.array([exact.to_complex(exact.sub(bi, zi)) for bi, zi in zip(bq, zx)])
    scale = np.abs(Z) @ np.abs(x)
    # Dot2: error <= u |exact| + gamma^2 sum |terms|, far below plain summation
    assert np.all(np.abs(R - re) <= 2 * np.finfo(float).eps * np.abs(re) + 1e-28 * scale)
    assert np.max(np.abs(re)) > 0


def test_residual_of_exact_solution_vanishes_for_diagonal():
    d = golden_io.load("diagonal_closed_form.txt")
    Z = _cplx(d["Z_re"], d["Z_im"])
    b = _cplx(d["b_re"], d["b_im"]).reshape(1, -1)
    # x_1 = -1/2 + j/2 is exact in binary: its residual component is zero
    x = np.array([[0j, -0.5 + 0.5j]])
    R = oracle.residual(Z, x, b)[0]
    assert R[1] == 0
    assert R[0] == b[0, 0]


# ------------------------------------------------------------------ norms

def test_norms_closed_forms():
    n = 5
    ones = np.ones((n, n), dtype=np.complex128) * (3 + 4j)    # |3+4j| = 5
    assert oracle.norm_inf_mat(ones) == 25.0
    M = np.diag(np.arange(1, n + 1)).astype(np.complex128)
    M[0, :] = 1j
    assert oracle.norm_inf_mat(M) == 5.0
    v = np.array([1, -7j, 3 + 4j, 0.5])
    assert oracle.norm_inf_vec(v) == 7.0


def test_eta_special_values():
    wl = workloads.make_workload(workloads.config(0), n=20, nfreq=1)
    Z = oracle.assemble(wl.omega[0], wl.zs[0], wl.L, wl.Psi, wl.g)
    b = workloads.random_rhs(np.random.default_rng(1), 20, 1)
    # x = 0: r = b, so eta = ||b|| / ||b|| = 1 exactly
    assert oracle.eta(Z, np.zeros_like(b), b)[0] == 1.0
    x = oracle.solve(Z, b)
    e = oracle.eta(Z, x, b)[0]
    # scaling Z and b by a power of two leaves eta unchanged exactly
    assert oracle.eta(4.0 * Z, x, 4.0 * b)[0] == e
    assert e <= 1e-15


def test_forward_error_and_reciprocity_definitions():
    x = np.array([[1 + 0j, 2j, -4]])
    y = np.array([[1 + 0j, 2j, -4 + 1j]])
    assert oracle.forward_error(y, x)[0] == 0.25
    X = np.array([[1, 2 + 1j, 3], [2 + 1j, 5, 6], [3, 6, 9]], dtype=np.complex128)
    assert oracle.reciprocity(X, [0, 1, 2]) == 0.0
    X[1, 0] = 2
    # pair (0, 1): |(2 + j) - 2| / max(3, 6)
    assert oracle.reciprocity(X, [0, 1, 2]) == pytest.approx(1.0 / 6.0)
