"""Parity of the device fallback solve (msolve_gepp_solve_c128, complex128
LU with partial pivoting on the GPU) with the oracle's direct solve (needs a
GPU).  Page "Solving Dense Matrices Fast in the Browser", section
"Double-precision answers from a GPU without double precision": a frequency
whose refinement fails is solved directly in double precision.

Both sides are backward stable complex128 eliminations with partial
pivoting, so their answers agree to about cond(Z) u, and each answer's
backward error is a small multiple of u.  The orders span one panel of 32,
several panels with a ragged tail, and the update tiles of 64.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ms():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mixed_precision_refinement_amd import msolve
    return msolve


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def gepp(ms, Z, B):
    X = ms.gepp_solve_c128(dev(Z), dev(B))
    torch.cuda.synchronize()
    return X.cpu().numpy()


@pytest.mark.parametrize("n,nrhs", [(1, 1), (7, 2), (32, 1), (64, 3), (130, 2), (700, 2)])
def test_random_systems_match_oracle(ms, n, nrhs):
    rng = np.random.default_rng(n)
    Z = (rng.standard_normal((n, n)) + 1j * rng.standard_normal((n, n))) / np.sqrt(n)
    B = workloads.random_rhs(rng, n, nrhs)
    print("gepp n=%d nrhs=%d" % (n, nrhs), flush=True)
    X = gepp(ms, Z, B)
    Xo = oracle.solve(Z, B)
    cond = np.linalg.cond(Z)
    assert np.all(oracle.forward_error(X, Xo) <= 1e-14 * cond), oracle.forward_error(X, Xo)
    assert np.all(oracle.eta(Z, X, B) <= 1e-14)


@pytest.mark.parametrize("n", [96, 333])
def test_model_matrix_matches_oracle(ms, n):
    # the configs' construction, at a frequency in the band (resonant, so
    # ill conditioned: the refinement's hard case)
    wl = workloads.make_workload(workloads.config(1), n=n, nfreq=3)
    B = workloads.random_rhs(np.random.default_rng(1), n, 2)
    for w, zs in zip(wl.omega, wl.zs):
        Z = oracle.assemble(w, zs, wl.L, wl.Psi, wl.g)
        X = gepp(ms, Z, B)
        assert np.all(oracle.forward_error(X, oracle.solve(Z, B)) <= 1e-14 * np.linalg.cond(Z))
        assert np.all(oracle.eta(Z, X, B) <= 1e-14)


def test_pivoting_is_needed_and_done(ms):
    # z_00 = 0 and tiny leading entries: no-pivot elimination fails or loses
    # every digit; partial pivoting solves it to full accuracy
    n = 150
    rng = np.random.default_rng(4)
    Z = (rng.standard_normal((n, n)) + 1j * rng.standard_normal((n, n))) / np.sqrt(n)
    Z[np.arange(n), np.arange(n)] = 1e-14
    Z[0, 0] = 0.0
    B = workloads.random_rhs(rng, n, 1)
    X = gepp(ms, Z, B)
    assert np.all(oracle.eta(Z, X, B) <= 1e-14)
    assert np.all(oracle.forward_error(X, oracle.solve(Z, B)) <= 1e-14 * np.linalg.cond(Z))


def test_permutation_matrix_is_solved_exactly(ms):
    # Z = P D with D diagonal (powers of two times 1 + j): every multiplier
    # is zero, so x_i = b_(p(i)) / d_i up to the rounding of one division
    n = 100
    rng = np.random.default_rng(8)
    perm = rng.permutation(n)
    d = 2.0 ** rng.integers(-3, 4, n) * (1.0 + 1j)
    Z = np.zeros((n, n), complex)
    Z[perm, np.arange(n)] = d
    B = workloads.random_rhs(rng, n, 2)
    X = gepp(ms, Z, B)
    x = B[:, perm] / d
    assert np.all(np.abs(X - x) <= 4e-16 * np.abs(x))


def test_in_place_right_hand_side(ms):
    n = 90
    rng = np.random.default_rng(9)
    Z = (rng.standard_normal((n, n)) + 1j * rng.standard_normal((n, n))) / np.sqrt(n)
    B = workloads.random_rhs(rng, n, 2)
    Bd = dev(B)
    Xd = ms.gepp_solve_c128(dev(Z), Bd, X=Bd)
    torch.cuda.synchronize()
    assert Xd.data_ptr() == Bd.data_ptr()
    assert np.all(oracle.eta(Z, Xd.cpu().numpy(), B) <= 1e-14)


@pytest.mark.parametrize("case", ["zero column", "nan entry"])
def test_singular_matrix_is_reported(ms, case):
    n = 70
    rng = np.random.default_rng(6)
    Z = (rng.standard_normal((n, n)) + 1j * rng.standard_normal((n, n))) / np.sqrt(n)
    if case == "zero column":
        Z[:, 40] = 0.0
    else:
        Z[13, 5] = np.nan
    with pytest.raises(ms.MsolveError) as e:
        gepp(ms, Z, workloads.random_rhs(rng, n, 1))
    assert e.value.status == ms.E_FALLBACK
    # the library stays usable after the report
    X = gepp(ms, np.eye(3, dtype=complex), np.ones((1, 3), complex))
    assert np.array_equal(X, np.ones((1, 3), complex))


def test_bench_matrix_at_full_size(ms):
    # the matrix and launch the bench times: Z of the n = 2157 workload's
    # first frequency, one right-hand side
    wl = workloads.make_workload(workloads.config(1))
    Z = oracle.assemble(wl.omega[0], wl.zs[0], wl.L, wl.Psi, wl.g)
    B = wl.B[:1]
    X = gepp(ms, Z, B)
    assert np.all(oracle.eta(Z, X, B) <= 1e-14)
    assert np.all(oracle.forward_error(X, oracle.solve(Z, B)) <= 1e-12)
