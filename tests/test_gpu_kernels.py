"""Per-kernel parity of the HIP path against the CPU oracle (needs a GPU).

Inputs come from the seeded generator or are built here on the host; every
expected value comes from the oracle or from exact arithmetic, never from
the HIP path.  Sizes span several 64-blocks and a ragged tail.
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


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def inputs(n, spec=0, nfreq=3, seed=0):
    return workloads.make_workload(workloads.config(spec), n=n, nfreq=nfreq, seed=seed)


# ---------------------------------------------------------------- assembly

@pytest.mark.parametrize("n", [1, 7, 64, 130, 256, 1000])
def test_assembly_bit_exact(ms, n):
    wl = inputs(n)
    L, P, g = dev(wl.L), dev(wl.Psi), dev(wl.g)
    for w, zs in zip(wl.omega, wl.zs):
        print("assemble n=%d w=%g" % (n, w), flush=True)
        Z128, Z64, zrow = ms.assemble(L, P, g, w, zs)
        Zo = oracle.assemble(w, zs, wl.L, wl.Psi, wl.g)
        assert np.array_equal(host(Z128), Zo)
        assert np.array_equal(host(Z64), Zo.astype(np.complex64))
        rows = np.abs(Zo).sum(axis=1)
        assert np.allclose(host(zrow), rows, rtol=1e-13, atol=0)


def test_assembly_golden_2x2(ms):
    import golden_io
    d = golden_io.load("assembly_solve_2x2.txt")
    L = golden_io.as_float(d["L"])
    P = golden_io.as_float(d["Psi"])
    g = golden_io.as_float(d["g"])
    zs = complex(float(d["zs_re"]), float(d["zs_im"]))
    Z128, _, _ = ms.assemble(dev(L), dev(P), dev(g), float(d["omega"]), zs)
    expect = golden_io.as_float(d["Z_re"]) + 1j * golden_io.as_float(d["Z_im"])
    assert np.array_equal(host(Z128), expect)


# ---------------------------------------------------------------- residual

@pytest.mark.parametrize("n,nrhs", [(1, 1), (100, 1), (257, 2), (500, 3), (640, 4), (300, 6)])
def test_residual_against_compensated_oracle(ms, n, nrhs):
    rng = np.random.default_rng(n + nrhs)
    Z = rng.standard_normal((n, n)) + 1j * rng.standard_normal((n, n))
    X = workloads.random_rhs(rng, n, nrhs)
    B = workloads.random_rhs(rng, n, nrhs)
    R, norms = ms.residual_c128(dev(Z), dev(B), dev(X))
    R = host(R)
    Ro = oracle.residual(Z, X, B)
    # |fl(r) - r| <= gamma_{2n+2} (|b| + |Z| |x|) elementwise (fp64 dot products)
    u = np.finfo(float).eps / 2
    bound = (2 * n + 4) * u / (1 - (2 * n + 4) * u) * (np.abs(B) + (np.abs(Z) @ np.abs(X).T).T)
    assert np.all(np.abs(R - Ro) <= bound)
    nn = host(norms)
    for k in range(nrhs):
        assert nn[k] == pytest.approx(oracle.norm_inf_vec(Ro[k]), rel=1e-12)
        assert nn[nrhs + k] == oracle.norm_inf_vec(X[k]) or \
            nn[nrhs + k] == pytest.approx(oracle.norm_inf_vec(X[k]), rel=1e-15)


def test_residual_exact_on_integers(ms):
    rng = np.random.default_rng(4)
    n = 333
    Z = (rng.integers(-9, 10, (n, n)) + 1j * rng.integers(-9, 10, (n, n))).astype(np.complex128)
    X = (rng.integers(-9, 10, (2, n)) + 1j * rng.integers(-9, 10, (2, n))).astype(np.complex128)
    B = (rng.integers(-99, 100, (2, n)) + 1j * rng.integers(-99, 100, (2, n))).astype(np.complex128)
    R, _ = ms.residual_c128(dev(Z), dev(B), dev(X))
    assert np.array_equal(host(R), oracle.residual(Z, X, B))


# --------------------------------------------------------------- factorisation

def _structured_exact_factors(n, rng):
    """Unit-lower L (full first column and first subdiagonal) and upper U
    (unit-modulus diagonal 1, -1, j, -j; full first row and first
    superdiagonal), all entries small Gaussian integers.  The inverses of
    their diagonal blocks have small Gaussian-integer entries and every
    partial sum of the blocked algorithm stays an integer below 2^24, so a
    single-precision factorisation of A = L U (and a solve with its factors)
    is exact."""
    units = np.array([1.0, -1.0, 1j, -1j])
    Lt = np.eye(n, dtype=np.complex128)
    Lt[1:, 0] = rng.choice([-1.0, 1.0], n - 1) + 1j * rng.choice([-1.0, 0.0, 1.0], n - 1)
    idx = np.arange(2, n)
    Lt[idx, idx - 1] = rng.choice(np.array([-1.0, 0.0, 1.0, 1j]), n - 2)
    Ut = np.diag(rng.choice(units, n)).astype(np.complex128)
    Ut[0, 1:] = rng.integers(-2, 3, n - 1) + 1j * rng.integers(-1, 2, n - 1)
    idx = np.arange(1, n - 1)
    Ut[idx, idx + 1] = rng.choice(np.array([-1.0, 0.0, 1.0, -1j]), n - 2)
    return Lt, Ut


def host_dinv(Lt, Ut, nb, exact=False):
    """Dinv as the factorisation lays it out, built on the host: per 64-block
    the inverses of its unit-lower and upper parts (identity padding), then
    per pair of blocks (2t, 2t+1) the coupling blocks of the pair's inverses,
    X = -Li1 L[2t+1][2t] Li0 and Y = -Ui0 U[2t][2t+1] Ui1 (zero padding).
    exact: round the block inverses to the Gaussian integers they are (for
    factors with unit determinants), so every entry is exact."""
    n = Lt.shape[0]
    nblk = -(-n // nb)
    npair = nblk // 2
    D = np.zeros((nblk + npair, 2, nb, nb), dtype=np.complex128)
    for b in range(nblk):
        k0, k1 = b * nb, min(n, (b + 1) * nb)
        m = k1 - k0
        Li = np.linalg.inv(Lt[k0:k1, k0:k1])
        Ui = np.linalg.inv(Ut[k0:k1, k0:k1])
        if exact:
            Li, Ui = np.round(Li), np.round(Ui)
            assert np.array_equal(Li @ Lt[k0:k1, k0:k1], np.eye(m))
            assert np.array_equal(Ui @ Ut[k0:k1, k0:k1], np.eye(m))
        D[b, 0] = np.eye(nb)
        D[b, 1] = np.eye(nb)
        D[b, 0, :m, :m] = Li
        D[b, 1, :m, :m] = Ui
    for t in range(npair):
        k0, k1 = 2 * t * nb, (2 * t + 1) * nb
        e1 = min(n, k1 + nb)
        M = np.zeros((nb, nb), dtype=np.complex128)
        N = np.zeros((nb, nb), dtype=np.complex128)
        M[:e1 - k1, :] = Lt[k1:e1, k0:k1]
        N[:, :e1 - k1] = Ut[k0:k1, k1:e1]
        D[nblk + t, 0] = -D[2 * t + 1, 0] @ M @ D[2 * t, 0]
        D[nblk + t, 1] = -D[2 * t, 1] @ N @ D[2 * t + 1, 1]
    return D


def pair_inverses_ok(D, Lg, Ug, nb, tol):
    """The 128 x 128 inverses assembled from Dinv invert the pairs' triangles."""
    n = Lg.shape[0]
    nblk = -(-n // nb)
    for t in range(nblk // 2):
        k0, e1 = 2 * t * nb, min(n, (2 * t + 2) * nb)
        m = e1 - k0
        Li = np.zeros((2 * nb, 2 * nb), dtype=np.complex128)
        Ui = np.zeros((2 * nb, 2 * nb), dtype=np.complex128)
        Li[:nb, :nb], Li[nb:, nb:], Li[nb:, :nb] = D[2 * t, 0], D[2 * t + 1, 0], D[nblk + t, 0]
        Ui[:nb, :nb], Ui[nb:, nb:], Ui[:nb, nb:] = D[2 * t, 1], D[2 * t + 1, 1], D[nblk + t, 1]
        if np.max(np.abs(Li[:m, :m] @ Lg[k0:e1, k0:e1] - np.eye(m))) > tol:
            return False
        if np.max(np.abs(Ui[:m, :m] @ Ug[k0:e1, k0:e1] - np.eye(m))) > tol:
            return False
    return True


@pytest.mark.parametrize("n", [5, 64, 65, 200, 300, 384, 450, 700, 833])
def test_factor_exact_structured(ms, n):
    rng = np.random.default_rng(n)
    Lt, Ut = _structured_exact_factors(n, rng)
    A = Lt @ Ut
    packed = np.tril(Lt, -1) + Ut
    # the oracle's unpivoted LU recovers the factors exactly (pins the case)
    assert np.array_equal(oracle.lu_nopivot(A), packed)
    Ad = dev(A.astype(np.complex64))
    _, Dinv, info = ms.factor_c64(Ad)
    assert int(host(info)[0]) == 0
    assert np.array_equal(host(Ad), packed.astype(np.complex64))


@pytest.mark.parametrize("n", [64, 129, 256, 511, 700, 1030])
def test_factor_matches_oracle_unpivoted_lu(ms, n):
    wl = inputs(n, nfreq=2)
    for w, zs in zip(wl.omega, wl.zs):
        Zo = oracle.assemble(w, zs, wl.L, wl.Psi, wl.g)
        Z64 = Zo.astype(np.complex64)
        F = oracle.lu_nopivot(Z64.astype(np.complex128))   # exact-arithmetic target in fp64
        Ad = dev(Z64)
        _, Dinv, info = ms.factor_c64(Ad)
        G = host(Ad).astype(np.complex128)
        assert int(host(info)[0]) == 0
        # elementwise within single-precision error growth
        scale = np.max(np.abs(F))
        assert np.max(np.abs(G - F)) <= 2e-4 * scale
        # backward stability of the computed factors
        Lg = np.tril(G, -1) + np.eye(n)
        Ug = np.triu(G)
        assert np.max(np.abs(Lg @ Ug - Z64)) <= 64 * n * 6e-8 * np.max(np.abs(Z64))
        # symmetric input: U = diag(U) L^T up to rounding
        assert np.max(np.abs(np.diag(np.diag(Ug)) @ Lg.T - Ug)) <= 1e-4 * np.max(np.abs(Ug))
        # inverted diagonal blocks, and the inverses of the pairs of blocks
        nb = ms.block_size(n)
        D = host(Dinv).view(np.complex64).reshape(-1, 2, nb, nb).astype(np.complex128)
        nblk = -(-n // nb)
        assert D.shape[0] == nblk + nblk // 2
        assert pair_inverses_ok(D, Lg, Ug, nb, 1e-4)
        for b in range(nblk):
            k0, k1 = b * nb, min(n, (b + 1) * nb)
            m = k1 - k0
            Lb = Lg[k0:k1, k0:k1]
            Ub = Ug[k0:k1, k0:k1]
            assert np.max(np.abs(D[b, 0, :m, :m] @ Lb - np.eye(m))) <= 1e-4
            assert np.max(np.abs(D[b, 1, :m, :m] @ Ub - np.eye(m))) <= 1e-4


@pytest.mark.parametrize("n", [5, 64, 65, 200, 384, 833, 1030])
def test_factor_sym_exact_structured(ms, n):
    # A = L D L^T with the exact structured L and a unit-modulus diagonal D:
    # the unpivoted factors are L and U = D L^T, and every step of the
    # symmetric factorisation stays in small Gaussian integers, so the
    # result is exact.  The strict upper triangle is NaN: it must not be read.
    rng = np.random.default_rng(3 * n + 1)
    Lt, Ut = _structured_exact_factors(n, rng)
    Ut = np.diag(np.diag(Ut)) @ Lt.T
    A = Lt @ Ut
    assert np.array_equal(A, A.T)
    packed = np.tril(Lt, -1) + Ut
    assert np.array_equal(oracle.lu_nopivot(A), packed)          # pins the case
    A64 = A.astype(np.complex64)
    A64[np.triu_indices(n, 1)] = np.complex64(complex(np.nan, np.nan))
    Ad = dev(A64)
    _, Dinv, info = ms.factor_c64(Ad, sym=True)
    assert int(host(info)[0]) == 0
    assert np.array_equal(host(Ad), packed.astype(np.complex64))


@pytest.mark.parametrize("n", [129, 700, 2157])
def test_factor_sym_matches_oracle(ms, n):
    wl = inputs(n, nfreq=1)
    Zo = oracle.assemble(wl.omega[0], wl.zs[0], wl.L, wl.Psi, wl.g)
    assert np.array_equal(Zo, Zo.T)             # the model's Z is complex symmetric
    Z64 = Zo.astype(np.complex64)
    F = oracle.lu_nopivot(Z64.astype(np.complex128))
    Zin = Z64.copy()
    Zin[np.triu_indices(n, 1)] = np.complex64(complex(np.nan, np.nan))
    Ad = dev(Zin)
    _, Dinv, info = ms.factor_c64(Ad, sym=True)
    G = host(Ad).astype(np.complex128)
    assert int(host(info)[0]) == 0
    assert np.all(np.isfinite(G))
    scale = np.max(np.abs(F))
    assert np.max(np.abs(G - F)) <= 2e-4 * scale
    Lg = np.tril(G, -1) + np.eye(n)
    Ug = np.triu(G)
    assert np.max(np.abs(Lg @ Ug - Z64)) <= 64 * n * 6e-8 * np.max(np.abs(Z64))
    # right of each diagonal block, U = D L^T to single-precision rounding
    nb = ms.block_size(n)
    d = np.diag(Ug)
    for k0 in range(0, n - nb, nb):
        want = d[k0:k0 + nb, None] * Lg[k0 + nb:, k0:k0 + nb].T
        got = Ug[k0:k0 + nb, k0 + nb:]
        assert np.max(np.abs(got - want)) <= 1e-6 * max(1.0, np.max(np.abs(want)))
    D = host(Dinv).view(np.complex64).reshape(-1, 2, nb, nb).astype(np.complex128)
    assert pair_inverses_ok(D, Lg, Ug, nb, 1e-4)
    # inside each diagonal block too the factors are those of one L D L^T:
    # u_rc = d_r l_cr with each product rounded on its own in float32, and
    # the stored U^-1 is L^-T D^-1 from the stored L^-1
    G32 = host(Ad)
    for k0 in range(0, n, nb):
        k1 = min(n, k0 + nb)
        blk = G32[k0:k1, k0:k1]
        dd = np.diag(blk)
        lo = np.tril(blk, -1)
        for r in range(k1 - k0):
            for c in range(r + 1, k1 - k0):
                a, b = dd[r], lo[c, r]
                re = np.float32(np.float32(a.real) * np.float32(b.real)) - np.float32(np.float32(a.imag) * np.float32(b.imag))
                im = np.float32(np.float32(a.real) * np.float32(b.imag)) + np.float32(np.float32(a.imag) * np.float32(b.real))
                assert blk[r, c] == np.complex64(complex(re, im)), (k0, r, c)
        m = k1 - k0
        Li = D[k0 // nb, 0][:m, :m]
        Ui = D[k0 // nb, 1][:m, :m]
        want = Li.T / dd.astype(np.complex128)[None, :]
        assert np.max(np.abs(Ui - want)) <= 1e-6 * max(1.0, np.max(np.abs(want)))
    # solving with the factors
    B = workloads.random_rhs(np.random.default_rng(n), n, 2).astype(np.complex64)
    RHS = dev(B)
    ms.lu_solve_c64(Ad, Dinv, RHS)
    X = host(RHS).astype(np.complex128)
    Xo = oracle.solve(Zo, B.astype(np.complex128))
    kappa = np.linalg.cond(Zo)
    assert np.max(oracle.forward_error(X, Xo)) <= 10 * kappa * 6e-8 * 8


@pytest.mark.parametrize("n,sym", [(300, False), (300, True), (900, False), (900, True)])
def test_factor_batch_equals_single_calls(ms, n, sym):
    # msolve_factor_c64_batch on three matrices gives bit for bit the
    # factors, inverses and pivot reports of three single calls
    wl = inputs(n, nfreq=3, seed=2)
    Zs = [oracle.assemble(w, zs, wl.L, wl.Psi, wl.g).astype(np.complex64)
          for w, zs in zip(wl.omega, wl.zs)]
    Ab = dev(np.stack(Zs))
    _, Db, ib = ms.factor_c64_batch(Ab, sym=sym)
    Ab, Db, ib = host(Ab), host(Db), host(ib)
    for f, Z in enumerate(Zs):
        Ad = dev(Z)
        _, D1, i1 = ms.factor_c64(Ad, sym=sym)
        assert np.array_equal(Ab[f], host(Ad))
        assert np.array_equal(Db[f], host(D1))
        assert int(ib[f]) == int(host(i1)[0]) == 0


def test_factor_reports_zero_pivot(ms):
    n = 100
    A = np.eye(n, dtype=np.complex64) * 2
    A[0, 0] = 0
    A[0, 1] = A[1, 0] = 1
    Ad = dev(A)
    _, _, info = ms.factor_c64(Ad)
    assert int(host(info)[0]) == 1
    A = np.eye(n, dtype=np.complex64) * 2
    A[70, 70] = 0
    Ad = dev(A)
    _, _, info = ms.factor_c64(Ad)
    assert int(host(info)[0]) == 71


# ------------------------------------------------------- triangular solves

@pytest.mark.parametrize("n,nrhs", [(5, 1), (64, 2), (200, 3), (300, 4), (257, 5)])
def test_lu_solve_exact_structured(ms, n, nrhs):
    rng = np.random.default_rng(7 * n)
    Lt, Ut = _structured_exact_factors(n, rng)
    packed = (np.tril(Lt, -1) + Ut).astype(np.complex64)
    nb = ms.block_size(n)
    # inverted diagonal blocks and pair couplings computed on the host; the
    # exact inverses are Gaussian integers (unit determinants), so rounding
    # removes the ~1e-17 noise of the floating-point inversion, which would
    # otherwise survive the cast to complex64 and make the result depend on
    # the summation order
    D = host_dinv(Lt, Ut, nb, exact=True)
    assert pair_inverses_ok(D, Lt, Ut, nb, 0.0)
    Dd = dev(D.astype(np.complex64).view(np.float32).ravel())
    xt = (rng.integers(-3, 4, (nrhs, n)) + 1j * rng.integers(-3, 4, (nrhs, n))).astype(np.complex128)
    B = (Lt @ Ut @ xt.T).T
    assert np.array_equal(oracle.lu_solve(np.tril(Lt, -1) + Ut, B), xt)   # pins the case
    RHS = dev(B.astype(np.complex64))
    ms.lu_solve_c64(dev(packed), Dd, RHS)
    assert np.array_equal(host(RHS), xt.astype(np.complex64))


def test_lu_solve_nan_input_and_workspace_reuse(ms):
    # The solves hand values between workgroups through their outputs, which
    # start out as a "pending" bit pattern (a NaN).  A NaN in one right-hand
    # side must come out as NaN without being mistaken for a pending value
    # (which would stall the solve), the other right-hand sides must stay
    # exact, and a later call on the same workspace must start clean.
    n, nrhs = 300, 3
    rng = np.random.default_rng(11)
    Lt, Ut = _structured_exact_factors(n, rng)
    packed = dev((np.tril(Lt, -1) + Ut).astype(np.complex64))
    D = host_dinv(Lt, Ut, ms.block_size(n), exact=True)
    Dd = dev(D.astype(np.complex64).view(np.float32).ravel())
    work = ms.workspace(ms.refine_workspace_bytes(n, nrhs))
    xt = (rng.integers(-3, 4, (nrhs, n)) + 1j * rng.integers(-3, 4, (nrhs, n))).astype(np.complex128)
    B = (Lt @ Ut @ xt.T).T.astype(np.complex64)
    for nan_at in (0, n // 2, n - 1):
        print("lu_solve nan at row %d" % nan_at, flush=True)
        Bn = B.copy()
        Bn[1, nan_at] = np.complex64(complex(np.nan, 0.0))
        RHS = dev(Bn)
        ms.lu_solve_c64(packed, Dd, RHS, work=work)
        X = host(RHS)
        assert np.array_equal(X[0], xt[0].astype(np.complex64))
        assert np.array_equal(X[2], xt[2].astype(np.complex64))
        # forward substitution spreads the NaN from its row on; the back
        # substitution then reaches every row
        assert np.all(np.isnan(X[1].real) | np.isnan(X[1].imag))
    RHS = dev(B)
    ms.lu_solve_c64(packed, Dd, RHS, work=work)
    assert np.array_equal(host(RHS), xt.astype(np.complex64))


@pytest.mark.parametrize("n,nrhs", [(130, 1), (256, 2), (700, 4)])
def test_lu_solve_matches_oracle_substitution(ms, n, nrhs):
    # factors made on the host (oracle LU of a config matrix, rounded to c64)
    wl = inputs(n, nfreq=1)
    Zo = oracle.assemble(wl.omega[0], wl.zs[0], wl.L, wl.Psi, wl.g)
    F = oracle.lu_nopivot(Zo).astype(np.complex64)
    Fd = F.astype(np.complex128)
    nb = ms.block_size(n)
    Lf = np.tril(Fd, -1) + np.eye(n)
    Uf = np.triu(Fd)
    D = host_dinv(Lf, Uf, nb)
    B = workloads.random_rhs(np.random.default_rng(n), n, nrhs).astype(np.complex64)
    RHS = dev(B)
    ms.lu_solve_c64(dev(F), dev(D.astype(np.complex64).view(np.float32).ravel()), RHS)
    X = host(RHS).astype(np.complex128)
    Xo = oracle.lu_solve(Fd, B.astype(np.complex128))
    kappa = np.linalg.cond(Zo)
    assert np.max(oracle.forward_error(X, Xo)) <= 10 * kappa * 6e-8 * 8


# ------------------------------------------------------- refinement

@pytest.mark.parametrize("n,nrhs", [(256, 1), (300, 2), (500, 4), (130, 6)])
def test_refine_matches_oracle(ms, n, nrhs):
    wl = inputs(n, nfreq=2)
    B = workloads.random_rhs(np.random.default_rng(n), n, nrhs)
    L, P, g = dev(wl.L), dev(wl.Psi), dev(wl.g)
    Bd = dev(B)
    for w, zs in zip(wl.omega, wl.zs):
        print("refine n=%d nrhs=%d w=%g" % (n, nrhs, w), flush=True)
        Z128, Z64, zrow = ms.assemble(L, P, g, w, zs)
        _, Dinv, info = ms.factor_c64(Z64)
        X, rinfo = ms.refine(Z128, Z64, Dinv, Bd, tol=1e-13, max_iter=10, zrowabs=zrow)
        X = host(X)
        Zo = oracle.assemble(w, zs, wl.L, wl.Psi, wl.g)
        Xo = oracle.solve(Zo, B)
        assert all(r.converged and not r.fallback for r in rinfo), rinfo
        assert np.all(oracle.forward_error(X, Xo) <= 1e-10)
        assert np.all(oracle.eta(Zo, X, B) <= 1e-13)
        # the device's own stop test agrees with the oracle's backward error
        for k, r in enumerate(rinfo):
            assert r.eta <= 1e-13


def test_refine_forward_estimate_stops_the_loop(ms):
    # With a loose backward-error bound (tol = 1e-6, met after the first
    # pass), the loop still runs until the estimated forward error is below
    # the library's bound: the answers are as accurate as with tol = 1e-13,
    # each converged right-hand side reports an estimate <= FWD_TOL, and the
    # estimate is not below the oracle's forward error by more than a small
    # factor.  The earliest stop is after three passes.
    n = 300
    wl = inputs(n, nfreq=1)
    B = workloads.random_rhs(np.random.default_rng(11), n, 2)
    Z128, Z64, zrow = ms.assemble(dev(wl.L), dev(wl.Psi), dev(wl.g), wl.omega[0], wl.zs[0])
    _, Dinv, _ = ms.factor_c64(Z64)
    X, rinfo = ms.refine(Z128, Z64, Dinv, dev(B), tol=1e-6, max_iter=10, zrowabs=zrow)
    Zo = oracle.assemble(wl.omega[0], wl.zs[0], wl.L, wl.Psi, wl.g)
    fe = oracle.forward_error(host(X), oracle.solve(Zo, B))
    for k, r in enumerate(rinfo):
        assert r.converged and not r.fallback, r
        assert r.iters >= 3, r
        assert r.fwd_est <= ms.FWD_TOL, r
        assert fe[k] <= 4.0 * r.fwd_est + 1e-13, (fe[k], r.fwd_est)
    assert np.all(fe <= 1e-10)


def test_refine_forward_estimate_not_met_falls_back(ms):
    # tol = 1e-6 is met after the first pass, but two passes give no usable
    # forward-error estimate: the system has not converged at max_iter = 2
    # and is solved directly (complex128 LU with partial pivoting)
    n = 256
    wl = inputs(n, nfreq=1)
    B = workloads.random_rhs(np.random.default_rng(12), n, 1)
    Z128, Z64, zrow = ms.assemble(dev(wl.L), dev(wl.Psi), dev(wl.g), wl.omega[0], wl.zs[0])
    _, Dinv, _ = ms.factor_c64(Z64)
    X, rinfo = ms.refine(Z128, Z64, Dinv, dev(B), tol=1e-6, max_iter=2, zrowabs=zrow)
    Zo = oracle.assemble(wl.omega[0], wl.zs[0], wl.L, wl.Psi, wl.g)
    assert all(r.fallback and not r.converged for r in rinfo), rinfo
    assert all(np.isnan(r.fwd_est) for r in rinfo)
    assert np.all(oracle.forward_error(host(X), oracle.solve(Zo, B)) <= 1e-12)


def test_refine_without_zrowabs(ms):
    wl = inputs(200, nfreq=1)
    B = workloads.random_rhs(np.random.default_rng(1), 200, 1)
    Z128, Z64, _ = ms.assemble(dev(wl.L), dev(wl.Psi), dev(wl.g), wl.omega[0], wl.zs[0])
    _, Dinv, _ = ms.factor_c64(Z64)
    X, rinfo = ms.refine(Z128, Z64, Dinv, dev(B))
    Zo = oracle.assemble(wl.omega[0], wl.zs[0], wl.L, wl.Psi, wl.g)
    assert oracle.forward_error(host(X), oracle.solve(Zo, B))[0] <= 1e-10


@pytest.mark.parametrize("tol,max_iter", [(0.0, 10), (1e-13, 0), (1e-13, 1)])
def test_refine_forced_fallback(ms, tol, max_iter):
    wl = inputs(256, nfreq=1)
    B = workloads.random_rhs(np.random.default_rng(5), 256, 2)
    Z128, Z64, zrow = ms.assemble(dev(wl.L), dev(wl.Psi), dev(wl.g), wl.omega[0], wl.zs[0])
    _, Dinv, _ = ms.factor_c64(Z64)
    X, rinfo = ms.refine(Z128, Z64, Dinv, dev(B), tol=tol, max_iter=max_iter, zrowabs=zrow)
    Zo = oracle.assemble(wl.omega[0], wl.zs[0], wl.L, wl.Psi, wl.g)
    assert all(r.fallback and not r.converged for r in rinfo)
    assert np.all(oracle.forward_error(host(X), oracle.solve(Zo, B)) <= 1e-12)


def test_sweep_zero_leading_pivot_falls_back(ms):
    # L = Psi = I except a [[0,1],[1,0]] leading block of L at w = 1 with no
    # real part there: Z[0,0] = 0, so the unpivoted factorisation meets a
    # zero pivot; the frequency must fall back and still match the oracle.
    n = 150
    L = np.eye(n)
    L[0, 0] = L[1, 1] = 0.0
    L[0, 1] = L[1, 0] = 1.0
    Psi = np.eye(n)
    Psi[0, 0] = Psi[1, 1] = 0.0
    g = np.ones(n)
    g[0] = g[1] = 0.0
    omega = np.array([2.0])
    zs = np.array([0.01 + 0.01j])
    B = workloads.random_rhs(np.random.default_rng(2), n, 1)
    X, finfo, rinfo = ms.sweep(dev(L), dev(Psi), dev(g), omega, zs, dev(B))
    assert finfo[0].pivot_info == 1 and finfo[0].fallback
    Zo = oracle.assemble(2.0, zs[0], L, Psi, g)
    assert oracle.forward_error(host(X)[0], oracle.solve(Zo, B))[0] <= 1e-13


def test_sweep_small_matches_oracle(ms):
    spec = workloads.config(0)
    wl = workloads.make_workload(spec)
    X, finfo, rinfo = ms.sweep(dev(wl.L), dev(wl.Psi), dev(wl.g), wl.omega, wl.zs, dev(wl.B),
                               tol=spec.tol, max_iter=spec.max_iter)
    X = host(X)
    for f, (w, zs) in enumerate(zip(wl.omega, wl.zs)):
        Zo = oracle.assemble(w, zs, wl.L, wl.Psi, wl.g)
        Xo = oracle.solve(Zo, wl.B)
        assert not finfo[f].fallback and finfo[f].status == 0
        assert np.all(oracle.forward_error(X[f], Xo) <= 1e-10)
        assert np.all(oracle.eta(Zo, X[f], wl.B) <= 1e-13)


@pytest.mark.parametrize("n", [300, 900])
def test_sweep_asymmetric_model_matches_oracle(ms, n):
    # L and Psi not symmetric: Z(w) is not symmetric, so the sweep must not
    # use the symmetric factorisation (which would factorise the mirror of
    # the lower triangle); the answers still match the oracle's
    wl = inputs(n, nfreq=3)
    rng = np.random.default_rng(n)
    L = wl.L + np.triu(0.05 * rng.standard_normal((n, n)) / np.sqrt(n), 1)
    P = wl.Psi.copy()
    P[0, n - 1] += 0.1
    X, finfo, rinfo = ms.sweep(dev(L), dev(P), dev(wl.g), wl.omega, wl.zs, dev(wl.B),
                               tol=1e-13, max_iter=10)
    X = host(X)
    for f, (w, zs) in enumerate(zip(wl.omega, wl.zs)):
        Zo = oracle.assemble(w, zs, L, P, wl.g)
        assert not np.array_equal(Zo, Zo.T)
        Xo = oracle.solve(Zo, wl.B)
        assert not finfo[f].fallback and finfo[f].status == 0
        assert finfo[f].iters_max <= 4
        assert np.all(oracle.forward_error(X[f], Xo) <= 1e-10)
        assert np.all(oracle.eta(Zo, X[f], wl.B) <= 1e-13)


def test_deterministic(ms):
    wl = inputs(300, nfreq=2)
    B = workloads.random_rhs(np.random.default_rng(9), 300, 2)
    outs = []
    for _ in range(2):
        X, _, _ = ms.sweep(dev(wl.L), dev(wl.Psi), dev(wl.g), wl.omega, wl.zs, dev(B))
        outs.append(host(X))
    assert np.array_equal(outs[0], outs[1])


# ------------------------------------------------------- frequency batches

@pytest.mark.parametrize("n,nrhs", [(300, 2), (900, 2), (300, 6)])
def test_sweep_batch_equals_single_frequency_calls(ms, n, nrhs):
    # a batch of three frequencies (one launch per step for all three) gives
    # bit for bit the answers of assembling, factorising and refining each
    # frequency on its own; n = 900 also takes the look-ahead schedule, and
    # six right-hand sides take the on-the-fly residual in a group of four
    # (two frequencies per workgroup) and a group of two (four per
    # workgroup).  L and Psi are symmetric, so the sweep factorises with the
    # symmetric factorisation.
    wl = inputs(n, nfreq=3, seed=4)
    B = workloads.random_rhs(np.random.default_rng(n + 1), n, nrhs)
    L, P, g, Bd = dev(wl.L), dev(wl.Psi), dev(wl.g), dev(B)
    assert ms.sweep_batch(n, nrhs, 3) == 3
    X, finfo, rinfo = ms.sweep(L, P, g, wl.omega, wl.zs, Bd, tol=1e-13, max_iter=10)
    X = host(X)
    for f, (w, zs) in enumerate(zip(wl.omega, wl.zs)):
        print("batch vs single n=%d f=%d" % (n, f), flush=True)
        Z128, Z64, zrow = ms.assemble(L, P, g, w, zs)
        _, Dinv, _ = ms.factor_c64(Z64, sym=True)
        Xs, rs = ms.refine(Z128, Z64, Dinv, Bd, tol=1e-13, max_iter=10, zrowabs=zrow)
        assert np.array_equal(X[f], host(Xs))
        assert [r.iters for r in rinfo[f]] == [r.iters for r in rs]
        assert [r.eta for r in rinfo[f]] == [r.eta for r in rs]


def test_sweep_two_batches_match_oracle(ms):
    n, nfreq = 96, 40
    wl = inputs(n, nfreq=nfreq, seed=3)
    assert ms.sweep_batch(n, 1, nfreq) == 20      # two batches of 20
    B = workloads.random_rhs(np.random.default_rng(8), n, 1)
    X, finfo, rinfo = ms.sweep(dev(wl.L), dev(wl.Psi), dev(wl.g), wl.omega, wl.zs, dev(B))
    X = host(X)
    for f in range(nfreq):
        Zo = oracle.assemble(wl.omega[f], wl.zs[f], wl.L, wl.Psi, wl.g)
        assert not finfo[f].fallback and finfo[f].status == 0
        assert oracle.forward_error(X[f], oracle.solve(Zo, B))[0] <= 1e-10
        assert oracle.eta(Zo, X[f], B)[0] <= 1e-13


@pytest.mark.parametrize("n", [96, 900])
def test_sweep_batches_equal_separate_sweeps(ms, n):
    # a sweep of several batches (each next batch assembled and factorised
    # on another stream while the current one is refined, into a second
    # set of per-frequency arrays) gives bit for bit the answers of sweeping
    # each batch's frequencies in a call of its own
    nfreq = 40 if n == 96 else 3 * ms.sweep_batch(n, 1, 1000)
    wl = inputs(n, nfreq=nfreq, seed=6)
    nb = ms.sweep_batch(n, 1, nfreq)
    assert nb < nfreq
    B = workloads.random_rhs(np.random.default_rng(n + 2), n, 1)
    L, P, g, Bd = dev(wl.L), dev(wl.Psi), dev(wl.g), dev(B)
    X, finfo, _ = ms.sweep(L, P, g, wl.omega, wl.zs, Bd)
    X = host(X)
    for f0 in range(0, nfreq, nb):
        om, zz = wl.omega[f0:f0 + nb], wl.zs[f0:f0 + nb]
        assert ms.sweep_batch(n, 1, len(om)) == len(om)
        Xs, fs, _ = ms.sweep(L, P, g, om, zz, Bd)
        print("batches vs separate n=%d f0=%d" % (n, f0), flush=True)
        assert np.array_equal(X[f0:f0 + nb], host(Xs))
        assert [f.iters_max for f in finfo[f0:f0 + nb]] == [f.iters_max for f in fs]


def test_sweep_batch_isolates_a_fallback(ms):
    # Z[0,0] = j (w - 1/w) vanishes at w = 1 only (L00 = Psi00 = 1, g0 = 0);
    # the coupling L01 = L10 = 1 keeps Z nonsingular there.  In a batch of
    # three, only w = 1 meets the zero pivot and falls back; the other two
    # converge, and all three match the oracle.
    n = 200
    L = np.eye(n)
    L[0, 1] = L[1, 0] = 1.0
    Psi = np.eye(n)
    Psi[1, 1] = 0.0
    g = np.ones(n)
    g[0] = g[1] = 0.0
    omega = np.array([0.7, 1.0, 2.0])
    zs = 0.01 * (1 + 1j) * np.sqrt(omega)
    B = workloads.random_rhs(np.random.default_rng(6), n, 2)
    X, finfo, rinfo = ms.sweep(dev(L), dev(Psi), dev(g), omega, zs, dev(B))
    X = host(X)
    assert [f.pivot_info for f in finfo] == [0, 1, 0]
    assert [f.fallback for f in finfo] == [False, True, False]
    assert all(r.converged for r in rinfo[0] + rinfo[2])
    for f, w in enumerate(omega):
        Zo = oracle.assemble(w, zs[f], L, Psi, g)
        assert np.all(oracle.forward_error(X[f], oracle.solve(Zo, B)) <= 1e-10)
        assert np.all(oracle.eta(Zo, X[f], B) <= 1e-13)


def test_sweep_singular_frequency_does_not_stop_later_batches(ms):
    # L = Psi = M and Zs = 0 at w = 1 make Z(1) = j(M - M) = 0 exactly
    # singular; at every other frequency Z = j(w - 1/w) M + Zs G is
    # nonsingular.  40 frequencies go in two batches of 20, with w = 1 in the
    # first: its direct solve reports the singular matrix, its answers are
    # NaN, and every other frequency (the second batch included) still
    # matches the oracle.
    n, nfreq, bad = 96, 40, 5
    M = inputs(n, nfreq=1, seed=3).L
    g = np.linspace(0.5, 1.5, n)
    omega = np.linspace(0.5, 2.0, nfreq)
    omega[bad] = 1.0
    zs = 0.01 * (1 + 1j) * np.sqrt(omega)
    zs[bad] = 0.0
    assert ms.sweep_batch(n, 1, nfreq) == 20
    B = workloads.random_rhs(np.random.default_rng(12), n, 1)
    with pytest.raises(ms.FallbackError) as e:
        ms.sweep(dev(M), dev(M), dev(g), omega, zs, dev(B))
    assert e.value.status == ms.E_FALLBACK
    Xd, finfo, rinfo = e.value.result
    X = host(Xd)
    assert finfo[bad].status == ms.E_FALLBACK and finfo[bad].fallback
    assert rinfo[bad][0].status == ms.E_FALLBACK
    assert np.all(np.isnan(X[bad]))
    for f in range(nfreq):
        if f == bad:
            continue
        assert finfo[f].status == 0 and not finfo[f].fallback, f
        Zo = oracle.assemble(omega[f], zs[f], M, M, g)
        assert oracle.forward_error(X[f], oracle.solve(Zo, B))[0] <= 1e-10, f
    # the binding returns the same results without raising when asked to
    X2, finfo2, _ = ms.sweep(dev(M), dev(M), dev(g), omega, zs, dev(B), check=False)
    assert [f.status for f in finfo2] == [f.status for f in finfo]
    assert np.array_equal(host(X2)[:bad], X[:bad])


@pytest.mark.parametrize("device_fallback", [True, False])
def test_refine_fallback_device_or_host(ms, device_fallback):
    # the fallback's direct solve runs in the caller's workspace on the
    # device when it is large enough, otherwise on the host; both match
    # the oracle
    n = 300
    wl = inputs(n, nfreq=1, seed=7)
    B = workloads.random_rhs(np.random.default_rng(13), n, 3)
    Z128, Z64, zrow = ms.assemble(dev(wl.L), dev(wl.Psi), dev(wl.g), wl.omega[0], wl.zs[0])
    _, Dinv, _ = ms.factor_c64(Z64)
    X, rinfo = ms.refine(Z128, Z64, Dinv, dev(B), tol=0.0, zrowabs=zrow,
                         device_fallback=device_fallback)
    assert all(r.fallback and r.status == 0 for r in rinfo)
    Zo = oracle.assemble(wl.omega[0], wl.zs[0], wl.L, wl.Psi, wl.g)
    assert np.all(oracle.forward_error(host(X), oracle.solve(Zo, B)) <= 1e-12)
    assert np.all(oracle.eta(Zo, host(X), B) <= 1e-14)
    # Z128 is the caller's and must come back unchanged
    assert np.array_equal(host(Z128), Zo)


def test_refine_singular_matrix_reports_fallback(ms):
    n = 70
    Z = np.zeros((n, n), dtype=np.complex128)
    Z64 = dev(Z.astype(np.complex64))
    _, Dinv, info = ms.factor_c64(Z64)
    B = workloads.random_rhs(np.random.default_rng(14), n, 1)
    X = torch.zeros((1, n), dtype=torch.complex128, device="cuda")
    # max_iter = 0 hands the matrix straight to the direct solve
    with pytest.raises(ms.MsolveError) as e:
        ms.refine(dev(Z), Z64, Dinv, dev(B), X=X, max_iter=0)
    assert e.value.status == ms.E_FALLBACK
    assert np.all(np.isnan(host(X)))
