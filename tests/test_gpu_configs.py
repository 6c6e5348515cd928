"""Full-size workloads through msolve_sweep (the launch configuration the
benchmark times), checked against the CPU oracle.

Every frequency the oracle is asked to solve is compared with the oracle's
complex128 direct solve (forward error <= 1e-10): all frequencies of the
n = 256, 2157, 8000 and 4096 workloads, and the two end frequencies of the
n = 16384 workload.  Above n = 2157 those solutions are stored under
tests/golden/ by ``golden/make_oracle_solutions.py`` (which calls only the
oracle and the seeded generator); a digest of the generated inputs ties each
file to the inputs the test generates.

At every frequency the backward error comes from the oracle's compensated
residual (<= 1e-13).  Between unit right-hand sides e_k, e_m, reciprocity
(Z^T = Z, so Z^-1 is symmetric) is checked against the bound the residuals
fix: with r_k = e_k - Z x_k,

    x_k[m] - x_m[k] = (Z^-1 r_m)[k] - (Z^-1 r_k)[m],
    |x_k[m] - x_m[k]| <= ||Z^-1 e_k||_1 ||r_m||_inf + ||Z^-1 e_m||_1 ||r_k||_inf,

because row k of the symmetric Z^-1 is the solution for e_k.  The 1-norms
are the oracle's where it solved the frequency, else those of the computed
solutions (within n * 1e-10 relative of the exact ones).  The asymmetry of
a refined answer is therefore whatever its stopping residual leaves, not a
fixed fraction of the forward-error bar.  The oracle's own solutions must
be reciprocal to 1e-12.
"""
from __future__ import annotations

import time

import numpy as np
import pytest

import oracle
import workloads
from golden_io import input_digest, load_oracle_solutions

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

FWD_TOL = 1e-10     # forward error bar
ETA_TOL = 1e-13     # backward error bar
ORACLE_RECIP_TOL = 1e-12
U64 = 2.0 ** -53


@pytest.fixture(scope="module")
def ms():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mixed_precision_refinement_amd import msolve
    return msolve


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run_sweep(ms, wl, B=None, omega=None, zs=None):
    B = wl.B if B is None else B
    omega = wl.omega if omega is None else omega
    zs = wl.zs if zs is None else zs
    t = time.perf_counter()
    X, finfo, rinfo = ms.sweep(dev(wl.L), dev(wl.Psi), dev(wl.g), omega, zs, dev(B),
                               tol=wl.spec.tol, max_iter=wl.spec.max_iter)
    torch.cuda.synchronize()
    print("%s: sweep of %d frequencies in %.2f s, iterations %s, fallbacks %d"
          % (wl.spec.name, len(omega), time.perf_counter() - t,
             [f.iters_max for f in finfo], sum(f.fallback for f in finfo)), flush=True)
    return X.cpu().numpy(), finfo, rinfo


def manufactured_rhs(wl, f, seed):
    """b = Z x_true with x_true seeded; Z x is formed by the oracle's
    compensated residual (0 - Z(-x)), accurate to about one rounding."""
    rng = np.random.default_rng(seed)
    xt = workloads.random_rhs(rng, wl.n, 1)
    Z = oracle.assemble(wl.omega[f], wl.zs[f], wl.L, wl.Psi, wl.g)
    b = oracle.residual(Z, -xt, np.zeros_like(xt))
    return Z, xt, b


def stored_solutions(wl):
    """The oracle's stored solutions of this workload, keyed by frequency."""
    gold = load_oracle_solutions(wl.spec.name)
    assert gold is not None, "tests/golden/oracle_%s.npz is missing" % wl.spec.name
    assert str(gold["digest"]) == input_digest(wl), "generated inputs differ from the stored ones"
    assert np.all(gold["eta"] <= 1e-14)
    assert np.all(gold["recip"] <= ORACLE_RECIP_TOL)
    return {int(f): (gold["X"][i], gold["x_norm1"][i]) for i, f in enumerate(gold["omega_index"])}


def reciprocity_within_residual_bound(X, R, unit_cols, x_norm1):
    """Largest |x_k[m] - x_m[k]| / bound over the pairs of unit right-hand
    sides (must be <= 1; see the module docstring)."""
    worst = 0.0
    for a in range(len(unit_cols)):
        for b in range(a + 1, len(unit_cols)):
            k, m = unit_cols[a], unit_cols[b]
            d = abs(X[a, m] - X[b, k])
            rk, rm = np.abs(R[a]).max(), np.abs(R[b]).max()
            bound = 1.01 * (x_norm1[a] * rm + x_norm1[b] * rk) + 4 * U64 * abs(X[a, m])
            worst = max(worst, d / bound if bound > 0 else (0.0 if d == 0 else np.inf))
    return worst


def check_all_frequencies(wl, X, finfo, direct, rinfo=None):
    """direct: {frequency: (oracle solution, its row 1-norms)} compared for
    forward error; every frequency gets the backward error and reciprocity.
    With rinfo, the refinement's own forward-error estimate of every refined
    answer is checked against the oracle: it is what the stop test relies on
    (a converged answer has estimate <= FWD_TOL of the library), so it must
    not understate the true error by much."""
    worst_fe, worst_eta, worst_recip, worst_ratio = 0.0, 0.0, 0.0, 0.0
    fe_per_freq = {}
    for f in range(wl.nfreq):
        assert finfo[f].status == 0
        Z = oracle.assemble(wl.omega[f], wl.zs[f], wl.L, wl.Psi, wl.g)
        R = oracle.residual(Z, X[f], wl.B)
        zn = oracle.norm_inf_mat(Z)
        eta = max(oracle.norm_inf_vec(R[k]) / (zn * oracle.norm_inf_vec(X[f][k]) +
                                               oracle.norm_inf_vec(wl.B[k]))
                  for k in range(wl.nrhs))
        worst_eta = max(worst_eta, eta)
        assert eta <= ETA_TOL, (f, eta)
        if f in direct:
            Xo, x1 = direct[f]
            fe = oracle.forward_error(X[f], Xo).max()
            fe_per_freq[f] = fe
            worst_fe = max(worst_fe, fe)
            assert fe <= FWD_TOL, (f, fe)
            if rinfo is not None and not finfo[f].fallback:
                for k in range(wl.nrhs):
                    r = rinfo[f][k]
                    fek = oracle.forward_error(X[f][k:k + 1], Xo[k:k + 1])[0]
                    assert r.converged and r.fwd_est <= ms_fwd_tol(), (f, k, r.fwd_est)
                    # the estimate tracks the error within a small factor
                    # down to the floor the double-precision residual leaves
                    # (about cond(Z) u64, a few 1e-12 near resonance), which
                    # the corrections do not see
                    assert fek <= 4.0 * r.fwd_est + 1e-11, (f, k, fek, r.fwd_est)
        else:
            x1 = np.abs(X[f]).sum(axis=1)
        if len(wl.unit_cols) > 1:
            worst_recip = max(worst_recip, oracle.reciprocity(X[f], wl.unit_cols))
            ratio = reciprocity_within_residual_bound(X[f], R, wl.unit_cols, x1)
            worst_ratio = max(worst_ratio, ratio)
            assert ratio <= 1.0, (f, ratio)
        del Z
    print("%s: worst forward error %.3g over %d oracle-solved frequencies, worst eta %.3g"
          % (wl.spec.name, worst_fe, len(direct), worst_eta), flush=True)
    if len(wl.unit_cols) > 1:
        print("%s: worst reciprocity defect %.3g, at most %.3g of its residual bound"
              % (wl.spec.name, worst_recip, worst_ratio), flush=True)
    return fe_per_freq


def ms_fwd_tol():
    from mixed_precision_refinement_amd import msolve
    return msolve.FWD_TOL


def oracle_direct(wl, freqs):
    out = {}
    for f in freqs:
        Z = oracle.assemble(wl.omega[f], wl.zs[f], wl.L, wl.Psi, wl.g)
        Xo = oracle.solve(Z, wl.B)
        out[f] = (Xo, np.abs(Xo).sum(axis=1))
        assert oracle.reciprocity(Xo, wl.unit_cols) <= ORACLE_RECIP_TOL
    return out


@pytest.mark.timeout(300)
def test_config0_n256_5_frequencies(ms):
    wl = workloads.make_workload(workloads.config(0))
    X, finfo, rinfo = run_sweep(ms, wl)
    check_all_frequencies(wl, X, finfo, oracle_direct(wl, range(wl.nfreq)), rinfo)


@pytest.mark.timeout(600)
def test_config1_n2157_21_frequencies(ms):
    wl = workloads.make_workload(workloads.config(1))
    X, finfo, rinfo = run_sweep(ms, wl)
    check_all_frequencies(wl, X, finfo, oracle_direct(wl, range(wl.nfreq)), rinfo)


@pytest.mark.timeout(900)
def test_config4_n4096_resonance_41_frequencies(ms):
    wl = workloads.make_workload(workloads.config(4))
    X, finfo, rinfo = run_sweep(ms, wl)
    fe = check_all_frequencies(wl, X, finfo, stored_solutions(wl), rinfo)
    assert sorted(fe) == list(range(wl.nfreq))
    order = sorted(fe, key=lambda f: -fe[f])
    print("n4096 resonance: largest forward errors %s" %
          ", ".join("w=%.4f %.3g (%d passes)" % (wl.omega[f], fe[f], finfo[f].iters_max)
                    for f in order[:6]), flush=True)
    print("n4096 resonance: passes per frequency %s" % [f.iters_max for f in finfo], flush=True)
    # near resonance some frequencies may need the LU retry after the
    # symmetric factorisation, but none needs the direct solve
    assert sum(f.fallback for f in finfo) == 0


@pytest.mark.timeout(900)
def test_config2_n8000_random_rhs(ms):
    wl = workloads.make_workload(workloads.config(2))
    X, finfo, _ = run_sweep(ms, wl)
    check_all_frequencies(wl, X, finfo, stored_solutions(wl))
    # manufactured solution at the same frequency: exact answer known
    Z, xt, b = manufactured_rhs(wl, 0, seed=11)
    Xm, finfo_m, _ = run_sweep(ms, wl, B=b)
    fe = oracle.forward_error(Xm[0], xt)[0]
    print("n8000 manufactured solution forward error %.3g" % fe, flush=True)
    assert fe <= FWD_TOL
    assert oracle.eta(Z, Xm[0], b)[0] <= ETA_TOL


@pytest.mark.timeout(1200)
def test_config3_n16384_8_frequencies_4_rhs(ms):
    spec = workloads.config(3)
    wl = workloads.make_workload(spec)
    X, finfo, _ = run_sweep(ms, wl)
    direct = stored_solutions(wl)
    assert sorted(direct) == sorted(spec.oracle_freq)
    # every frequency: backward error and reciprocity over the 6 pairs of
    # unit right-hand sides; the two end frequencies against the oracle's
    # direct solve, and against a manufactured solution
    check_all_frequencies(wl, X, finfo, direct)
    for f in spec.oracle_freq:
        Z, xt, b = manufactured_rhs(wl, f, seed=20 + f)
        Xm, _, _ = run_sweep(ms, wl, B=b, omega=wl.omega[f:f + 1], zs=wl.zs[f:f + 1])
        fe = oracle.forward_error(Xm[0], xt)[0]
        print("n16384 w=%.3f manufactured solution forward error %.3g" % (wl.omega[f], fe),
              flush=True)
        assert fe <= FWD_TOL
        del Z
