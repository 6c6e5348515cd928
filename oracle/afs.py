"""Adaptive frequency sampling (reduced-order sweep) -- TEST INFRASTRUCTURE
ONLY, part of the CPU oracle (see ``oracle/__init__.py`` for who may import
it).  Shares no code with the GPU library.

Page "Solving Dense Matrices Fast in the Browser", section "Fewer frequency
points: adaptive frequency sampling".  Since L, Psi and G do not depend on
the frequency, the solutions at a few frequencies span a small space on which
Z(w) can be projected.  The steps, in the section's order:

  1. solve exactly at a few frequencies; orthonormalise the real and the
     imaginary parts of the solutions into a real basis V (n x q);
  2. the reduced matrix Z_r(w) = jw V^T L V - j V^T Psi V / w + Zs(w) V^T G V
     (q x q), solved for y at any frequency; the sweep's answer is x = V y;
  3. estimate the residual ||Z(w) V y - b|| at every candidate frequency and
     solve exactly next where it is largest;
  4. stop once every candidate's residual is below the tolerance (1e-4).

Readings where the section is silent (each is also listed with the design
notes of this repository):
  * the first exact frequencies are the two ends of the candidate list;
  * the basis takes the real and imaginary part of every right-hand side's
    solution, orthonormalised by modified Gram-Schmidt applied twice; a part
    whose remaining 2-norm falls below 1e-10 of its own is left out;
  * the residual is the 2-norm relative to ||b||_2, per right-hand side, and
    a frequency's estimate is the largest over its right-hand sides;
  * the next exact frequency is the candidate with the largest estimate
    (the lowest index among equal ones), frequencies already solved exactly
    left out;
  * the reduced systems are solved by complex128 LU with partial pivoting
    (the oracle's direct solve).

Here the residual is evaluated from its definition: Z(w) is assembled and
multiplied by V y in complex128 (slow, obviously correct).  Exact solves use
the oracle's pivoted direct solve.

Parity: pinned by ``tests/test_oracle_afs.py`` (Galerkin exactness at the
exactly solved frequencies, a full basis reproducing every direct solve, the
diagonal closed form, symmetry of the reduced matrix).
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from . import assemble, solve

DROP_TOL = 1e-10


def extend_basis(V: np.ndarray, X: np.ndarray) -> np.ndarray:
    """Append the real and imaginary parts of the rows of X (complex, k x n)
    to the orthonormal rows of V (q x n, real), each orthogonalised against
    every row before it by two passes of modified Gram-Schmidt and dropped
    when less than DROP_TOL of its norm remains."""
    rows = [v for v in V]
    for x in np.atleast_2d(X):
        for part in (x.real, x.imag):
            u = np.array(part, dtype=np.float64)
            n0 = np.linalg.norm(u)
            if n0 == 0.0:
                continue
            for _ in range(2):
                for v in rows:
                    u = u - np.dot(v, u) * v
            nu = np.linalg.norm(u)
            if nu > DROP_TOL * n0:
                rows.append(u / nu)
    return np.array(rows, dtype=np.float64).reshape(len(rows), X.shape[-1])


def reduced_matrix(omega: float, zs: complex, VLV: np.ndarray, VPV: np.ndarray,
                   VGV: np.ndarray) -> np.ndarray:
    """Z_r = jw V^T L V - j V^T Psi V / w + Zs V^T G V (step 2)."""
    return 1j * omega * VLV - 1j * VPV / omega + complex(zs) * VGV


def reduced_solve(omega: float, zs: complex, V: np.ndarray, L: np.ndarray,
                  Psi: np.ndarray, g: np.ndarray, B: np.ndarray) -> np.ndarray:
    """y (nrhs x q) with Z_r(w) y = V^T b for every right-hand side."""
    VLV = V @ L @ V.T
    VPV = V @ Psi @ V.T
    VGV = (V * g) @ V.T
    Zr = reduced_matrix(omega, zs, VLV, VPV, VGV)
    Br = np.atleast_2d(B) @ V.T            # rows: V^T b
    return solve(Zr, Br)


def residual_estimate(omega: float, zs: complex, V: np.ndarray, Y: np.ndarray,
                      L: np.ndarray, Psi: np.ndarray, g: np.ndarray,
                      B: np.ndarray) -> np.ndarray:
    """||Z(w) V y - b||_2 / ||b||_2 per right-hand side, from the definition
    (step 3)."""
    Z = assemble(omega, zs, L, Psi, g)
    B = np.atleast_2d(B)
    out = np.empty(B.shape[0])
    for k in range(B.shape[0]):
        x = Y[k] @ V
        out[k] = np.linalg.norm(Z @ x - B[k]) / np.linalg.norm(B[k])
    return out


def afs(L: np.ndarray, Psi: np.ndarray, g: np.ndarray, omegas: Sequence[float],
        zs: Sequence[complex], B: np.ndarray, tol: float = 1e-4,
        max_exact: Optional[int] = None) -> dict:
    """Reduced-order sweep over the candidate frequencies ``omegas`` (steps
    1-4).  Returns X (nfreq x nrhs x n, x = V y at every candidate), the
    exactly solved indices in the order they were chosen, the final residual
    estimates (largest over the right-hand sides), the basis size, and the
    basis V (q x n) and reduced solutions Y (nfreq x nrhs x q) themselves."""
    omegas = [float(w) for w in omegas]
    zs = [complex(z) for z in zs]
    B = np.atleast_2d(np.asarray(B, dtype=np.complex128))
    nf, n = len(omegas), L.shape[0]
    cap = nf if max_exact is None else max(1, min(int(max_exact), nf))
    exact = [0] if nf == 1 else [0, nf - 1]
    exact = exact[:cap]
    V = np.zeros((0, n))
    new = list(exact)
    while True:
        for f in new:
            V = extend_basis(V, solve(assemble(omegas[f], zs[f], L, Psi, g), B))
        Y = [reduced_solve(omegas[f], zs[f], V, L, Psi, g, B) for f in range(nf)]
        est = np.array([residual_estimate(omegas[f], zs[f], V, Y[f], L, Psi, g, B).max()
                        for f in range(nf)])
        rest = [f for f in range(nf) if f not in exact]
        if not rest or len(exact) >= cap:
            break
        f_next = max(rest, key=lambda f: (est[f], -f))
        if est[f_next] <= tol:
            break
        exact.append(f_next)
        new = [f_next]
    X = np.stack([Y[f] @ V for f in range(nf)])
    return {"X": X, "exact": exact, "estimate": est, "q": V.shape[0], "V": V, "Y": np.stack(Y)}
