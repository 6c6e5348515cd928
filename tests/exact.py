"""Exact complex-rational arithmetic used to pin the oracle.

Independent of the oracle: a complex number is a pair of Fractions, a
matrix a list of rows of such pairs.  Used only by tests.
"""
from __future__ import annotations

import itertools
from fractions import Fraction
from typing import List, Sequence, Tuple

import numpy as np

C = Tuple[Fraction, Fraction]


def cq(z) -> C:
    """Exact complex rational from a Python/numpy complex (binary value kept)."""
    z = complex(z)
    return (Fraction(z.real), Fraction(z.imag))


def add(a: C, b: C) -> C:
    return (a[0] + b[0], a[1] + b[1])


def sub(a: C, b: C) -> C:
    return (a[0] - b[0], a[1] - b[1])


def mul(a: C, b: C) -> C:
    return (a[0] * b[0] - a[1] * b[1], a[0] * b[1] + a[1] * b[0])


def div(a: C, b: C) -> C:
    d = b[0] * b[0] + b[1] * b[1]
    return ((a[0] * b[0] + a[1] * b[1]) / d, (a[1] * b[0] - a[0] * b[1]) / d)


def to_complex(a: C) -> complex:
    return complex(float(a[0]), float(a[1]))


def matrix(Z: np.ndarray) -> List[List[C]]:
    return [[cq(Z[i, j]) for j in range(Z.shape[1])] for i in range(Z.shape[0])]


def vector(b: np.ndarray) -> List[C]:
    return [cq(v) for v in np.ravel(b)]


def gauss_solve(A: List[List[C]], b: List[C]) -> List[C]:
    """Exact Gaussian elimination (any nonzero pivot; exact arithmetic makes
    the choice irrelevant)."""
    n = len(A)
    M = [list(r) + [b[i]] for i, r in enumerate(A)]
    zero = (Fraction(0), Fraction(0))
    for k in range(n):
        p = next(i for i in range(k, n) if M[i][k] != zero)
        M[k], M[p] = M[p], M[k]
        for i in range(k + 1, n):
            if M[i][k] == zero:
                continue
            f = div(M[i][k], M[k][k])
            for j in range(k, n + 1):
                M[i][j] = sub(M[i][j], mul(f, M[k][j]))
    x = [zero] * n
    for i in range(n - 1, -1, -1):
        s = M[i][n]
        for j in range(i + 1, n):
            s = sub(s, mul(M[i][j], x[j]))
        x[i] = div(s, M[i][i])
    return x


def matvec(A: List[List[C]], x: Sequence[C]) -> List[C]:
    out = []
    for row in A:
        s = (Fraction(0), Fraction(0))
        for a, v in zip(row, x):
            s = add(s, mul(a, v))
        out.append(s)
    return out


def _perm_sign(p) -> int:
    s = 1
    p = list(p)
    for i in range(len(p)):
        while p[i] != i:
            j = p[i]
            p[i], p[j] = p[j], p[i]
            s = -s
    return s


def leibniz_det(Z: np.ndarray) -> complex:
    """det by the Leibniz permutation expansion, in complex128."""
    n = Z.shape[0]
    total = 0j
    for p in itertools.permutations(range(n)):
        term = complex(_perm_sign(p))
        for i in range(n):
            term *= complex(Z[i, p[i]])
        total += term
    return total


def cramer_solve(Z: np.ndarray, b: np.ndarray) -> np.ndarray:
    """x_i = det(Z with column i replaced by b) / det(Z), complex128."""
    n = Z.shape[0]
    d = leibniz_det(Z)
    x = np.empty(n, dtype=np.complex128)
    for i in range(n):
        Zi = np.array(Z, dtype=np.complex128, copy=True)
        Zi[:, i] = b
        x[i] = leibniz_det(Zi) / d
    return x
