"""The seeded input generator: structure, seeds, draw order, sizes."""
from __future__ import annotations

import math

import numpy as np

import workloads


def test_matrices_exactly_symmetric_and_shifted():
    L, Psi, g, _ = workloads.make_matrices(50, seed=0)
    assert np.array_equal(L, L.T)
    assert np.array_equal(Psi, Psi.T)
    assert L.dtype == np.float64 and g.shape == (50,)
    assert np.all((g >= 0.5) & (g < 1.5))
    # diagonal about 2, off-diagonal entries of size ~ 1/sqrt(2n)
    assert abs(np.mean(np.diag(L)) - 2.0) < 0.1
    off = L[~np.eye(50, dtype=bool)]
    assert abs(np.std(off) * math.sqrt(2 * 50) - 1.0) < 0.1


def test_draw_order_and_seed():
    n = 8
    rng = np.random.default_rng(0)
    b1 = rng.standard_normal((n, n))
    b2 = rng.standard_normal((n, n))
    u = rng.uniform(0.5, 1.5, n)
    L, Psi, g, _ = workloads.make_matrices(n, seed=0)
    d = 2.0 * math.sqrt(n)
    assert np.array_equal(L, (b1 + b1.T) / d + 2.0 * np.eye(n))
    assert np.array_equal(Psi, (b2 + b2.T) / d + 2.0 * np.eye(n))
    assert np.array_equal(g, u)
    L2, _, _, _ = workloads.make_matrices(n, seed=1)
    assert not np.array_equal(L, L2)


def test_configs_shapes_and_rhs():
    c = workloads.CONFIGS
    assert [s.n for s in c] == [256, 2157, 8000, 16384, 4096]
    assert [s.nfreq for s in c] == [5, 21, 1, 8, 41]
    wl = workloads.make_workload(c[1], n=2157, nfreq=21)
    assert wl.unit_cols == [0, 1078]
    assert wl.B.shape == (2, 2157) and wl.B[1, 1078] == 1.0
    assert wl.omega[0] == 0.5 and wl.omega[-1] == 2.0 and len(wl.omega) == 21
    assert np.allclose(wl.zs, 0.01 * (1 + 1j) * np.sqrt(wl.omega))
    spec3 = c[3]
    assert [workloads._unit_index(s, 16384) for s in spec3.unit_index] == [0, 1, 8192, 16383]
    w4 = workloads.make_workload(c[4], n=64)
    assert 1.0 in w4.omega      # the resonance point w = 1 is on the grid
    assert np.allclose(w4.zs, 1e-4 * (1 + 1j) * np.sqrt(w4.omega))


def test_random_rhs_drawn_after_matrices():
    n = 16
    wl = workloads.make_workload(workloads.config(2), n=n)
    _, _, _, rng = workloads.make_matrices(n, seed=0)
    br = rng.standard_normal(n)
    bi = rng.standard_normal(n)
    assert np.array_equal(wl.B[0], (br + 1j * bi) / math.sqrt(2.0))
    assert wl.omega.tolist() == [1.3]


def test_quasistatic_workload_resonances_above_the_band():
    wl = workloads.make_quasistatic_workload(64, nfreq=41)
    L0, Psi0, g0, _ = workloads.make_matrices(64, seed=0)
    assert np.array_equal(wl.L, 0.05 * L0) and np.array_equal(wl.Psi, Psi0) and np.array_equal(wl.g, g0)
    assert wl.omega[0] == 0.5 and wl.omega[-1] == 2.0 and wl.B.shape == (1, 64) and wl.B[0, 0] == 1.0
    # w^2 L x = Psi x: every resonance lies above w = 2
    w2 = np.linalg.eigvals(np.linalg.solve(wl.L, wl.Psi)).real
    assert np.sqrt(w2.min()) > 2.0
