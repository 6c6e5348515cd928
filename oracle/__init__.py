"""CPU oracle for Z(w) x = b -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check in ``__graft_entry__`` and the CPU-baseline
leg of ``bench.py`` may import this package.  It shares no code with the GPU
library (``mixed_precision_refinement_amd``) and never imports it.

The arithmetic lives in ``oracle.c`` (plain C, float64 / complex128, built by
``build.py`` with gcc); this module marshals numpy arrays to it and adds the
metrics used to judge a solution:

* ``assemble``      -- Z(w) = jwL - jPsi/w + Zs(w)G (page "Solving Dense
  Matrices Fast in the Browser", section "Fewer frequency points: adaptive
  frequency sampling", model equation);
* ``solve``         -- complex128 LU with partial pivoting and substitution,
  the double-precision direct solve the refined answer must agree with
  (same page, sections "Measure first: the ceiling of JavaScript" and
  "Double-precision answers from a GPU without double precision");
* ``lu_nopivot`` / ``lu_solve`` -- the unpivoted factorisation and the
  substitutions that steps 1, 2 and 4 of the refinement list apply, here in
  complex128;
* ``residual``      -- r = b - Z x (step 3 of that list), compensated so it
  is accurate to about one rounding of the result;
* ``eta``, ``forward_error``, ``reciprocity`` -- acceptance metrics.

Every function here is pinned by ``tests/test_oracle_pins.py``; the parity
status of each is listed in its docstring.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib: Optional[ctypes.CDLL] = None

_i64 = ctypes.c_int64
_dbl = ctypes.c_double
_ptr = ctypes.c_void_p


def _load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    # ORACLE_LIB_OVERRIDE lets the mutation tests load a deliberately broken
    # copy of the oracle and check that the pins reject it.
    path = os.environ.get("ORACLE_LIB_OVERRIDE", _LIB_PATH)
    if path == _LIB_PATH and not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(path)
    lib.orc_set_threads.argtypes = [ctypes.c_int]
    lib.orc_set_threads.restype = None
    lib.orc_get_threads.argtypes = []
    lib.orc_get_threads.restype = ctypes.c_int
    lib.orc_assemble.argtypes = [_i64, _dbl, _dbl, _dbl, _ptr, _ptr, _ptr, _ptr]
    lib.orc_assemble.restype = None
    lib.orc_gepp_solve.argtypes = [_i64, _i64, _ptr, _ptr, _ptr]
    lib.orc_gepp_solve.restype = ctypes.c_int
    lib.orc_lu_nopivot.argtypes = [_i64, _ptr]
    lib.orc_lu_nopivot.restype = ctypes.c_int
    lib.orc_lu_solve.argtypes = [_i64, _i64, _ptr, _ptr, _ptr]
    lib.orc_lu_solve.restype = None
    lib.orc_residual.argtypes = [_i64, _i64, _ptr, _ptr, _ptr, _ptr]
    lib.orc_residual.restype = None
    lib.orc_norm_inf_mat.argtypes = [_i64, _ptr]
    lib.orc_norm_inf_mat.restype = _dbl
    lib.orc_norm_inf_vec.argtypes = [_i64, _ptr]
    lib.orc_norm_inf_vec.restype = _dbl
    _lib = lib
    return lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a: np.ndarray) -> int:
    return a.ctypes.data


def set_threads(n: int) -> None:
    """Number of OpenMP threads the oracle uses (0 leaves the default)."""
    _load().orc_set_threads(int(n))


def get_threads() -> int:
    return int(_load().orc_get_threads())


class SingularError(RuntimeError):
    pass


def assemble(omega: float, zs: complex, L: np.ndarray, Psi: np.ndarray,
             g: np.ndarray) -> np.ndarray:
    """Z(w) in complex128 with the operation order fixed (pinned: golden 2x2,
    structure and special cases in tests)."""
    L = _c(L, np.float64)
    Psi = _c(Psi, np.float64)
    g = _c(g, np.float64)
    n = L.shape[0]
    Z = np.empty((n, n), dtype=np.complex128)
    zs = complex(zs)
    _load().orc_assemble(n, float(omega), zs.real, zs.imag, _p(L), _p(Psi), _p(g), _p(Z))
    return Z


def solve(Z: np.ndarray, B: np.ndarray) -> np.ndarray:
    """X (rows) with Z X^T = B^T by complex128 GEPP (pinned: Cramer, exact
    rationals, closed forms, manufactured solutions, reciprocity, LAPACK)."""
    A = np.array(Z, dtype=np.complex128, order="C", copy=True)
    B = np.atleast_2d(_c(B, np.complex128))
    n = A.shape[0]
    nrhs = B.shape[0]
    X = np.empty_like(B)
    info = _load().orc_gepp_solve(n, nrhs, _p(A), _p(B), _p(X))
    if info != 0:
        raise SingularError("oracle GEPP: zero pivot at step %d" % (info - 1))
    return X


def lu_nopivot(A: np.ndarray) -> np.ndarray:
    """Packed L\\U of A without row exchanges, complex128 (pinned: exact
    integer factors, reconstruction, symmetric structure U = diag(U) L^T)."""
    F = np.array(A, dtype=np.complex128, order="C", copy=True)
    info = _load().orc_lu_nopivot(F.shape[0], _p(F))
    if info != 0:
        raise SingularError("oracle LU: zero pivot at step %d" % (info - 1))
    return F


def lu_solve(LU: np.ndarray, B: np.ndarray) -> np.ndarray:
    """Forward (unit lower) then back (upper) substitution with packed
    factors, complex128 (pinned: exact integer triangular systems)."""
    LU = _c(LU, np.complex128)
    B = np.atleast_2d(_c(B, np.complex128))
    X = np.empty_like(B)
    _load().orc_lu_solve(LU.shape[0], B.shape[0], _p(LU), _p(B), _p(X))
    return X


def residual(Z: np.ndarray, X: np.ndarray, B: np.ndarray) -> np.ndarray:
    """R = B - Z X (rows), compensated Dot2 (pinned: exact integer cases and
    cancellation cases against exact rationals)."""
    Z = _c(Z, np.complex128)
    X = np.atleast_2d(_c(X, np.complex128))
    B = np.atleast_2d(_c(B, np.complex128))
    R = np.empty_like(B)
    _load().orc_residual(Z.shape[0], X.shape[0], _p(Z), _p(X), _p(B), _p(R))
    return R


def norm_inf_mat(Z: np.ndarray) -> float:
    Z = _c(Z, np.complex128)
    return float(_load().orc_norm_inf_mat(Z.shape[0], _p(Z)))


def norm_inf_vec(v: np.ndarray) -> float:
    v = _c(v, np.complex128).ravel()
    return float(_load().orc_norm_inf_vec(v.shape[0], _p(v)))


def eta(Z: np.ndarray, X: np.ndarray, B: np.ndarray,
        znorm: Optional[float] = None) -> np.ndarray:
    """Normwise backward error per right-hand side,
    eta = ||b - Z x||_inf / (||Z||_inf ||x||_inf + ||b||_inf)."""
    X = np.atleast_2d(X)
    B = np.atleast_2d(B)
    R = residual(Z, X, B)
    zn = norm_inf_mat(Z) if znorm is None else float(znorm)
    out = np.empty(X.shape[0])
    for k in range(X.shape[0]):
        out[k] = norm_inf_vec(R[k]) / (zn * norm_inf_vec(X[k]) + norm_inf_vec(B[k]))
    return out


def forward_error(x: np.ndarray, x_ref: np.ndarray) -> np.ndarray:
    """||x - x_ref||_inf / ||x_ref||_inf per row."""
    x = np.atleast_2d(x)
    x_ref = np.atleast_2d(x_ref)
    out = np.empty(x.shape[0])
    for k in range(x.shape[0]):
        out[k] = norm_inf_vec(x[k] - x_ref[k]) / norm_inf_vec(x_ref[k])
    return out


def reciprocity(X: np.ndarray, unit_cols: Sequence[int]) -> float:
    """Largest |x^(k)_m - x^(m)_k| / max(||x^(k)||, ||x^(m)||) over pairs of
    unit right-hand sides e_k, e_m (Z^T = Z implies Z^-1 is symmetric)."""
    worst = 0.0
    for a in range(len(unit_cols)):
        for b in range(a + 1, len(unit_cols)):
            k, m = unit_cols[a], unit_cols[b]
            d = abs(X[a, m] - X[b, k])
            s = max(norm_inf_vec(X[a]), norm_inf_vec(X[b]))
            worst = max(worst, d / s)
    return worst
