"""Seeded synthetic workloads for repeated solves of Z(w) x = b.

This module only draws the frequency-independent inputs of the method (the
real symmetric matrices L and Psi, the diagonal g of G, the frequencies, the
surface-impedance values Zs(w) and the right-hand sides).  It holds none of
the method's arithmetic: the assembly of Z(w), the factorisation, the
residual and the refinement live elsewhere.  Both the GPU path and the CPU
oracle take their inputs from here.

Construction (page "Solving Dense Matrices Fast in the Browser", section
"Fewer frequency points: adaptive frequency sampling", the model equation
Z(w) = jwL - jPsi/w + Zs(w)G with L, Psi, G independent of frequency; the
pages give neither the form of Zs nor the structure of G, so they are fixed
here):

* ``rng = numpy.random.default_rng(seed)`` (PCG64), seed 0 by default;
* draw order ``B1 = rng.standard_normal((n, n))``,
  ``B2 = rng.standard_normal((n, n))``, ``u = rng.uniform(0.5, 1.5, n)``,
  and for a random right-hand side ``br = rng.standard_normal(n)``,
  ``bi = rng.standard_normal(n)``;
* ``S = (B + B.T) / (2 sqrt(n))`` (exactly symmetric),
  ``L = S1 + 2I``, ``Psi = S2 + 2I``, ``G = diag(u)``;
* ``Zs(w) = c (1 + j) sqrt(w)`` with ``c = 0.01`` (``1e-4`` for the
  near-resonance sweep);
* frequencies ``numpy.linspace(lo, hi, nfreq)`` (end points included);
* unit right-hand sides ``e_k`` use 0-based k, ``e_{N/2}`` means ``N // 2``;
  a random right-hand side is ``(br + j bi) / sqrt(2)``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np


@dataclasses.dataclass(frozen=True)
class ConfigSpec:
    """Shape of one workload: matrix order, frequency grid and right-hand sides."""

    name: str
    n: int
    omega_lo: float
    omega_hi: float
    nfreq: int
    rhs: str                      # "unit" or "random"
    unit_index: Sequence[str]     # symbolic indices for unit right-hand sides
    zs_scale: float = 0.01
    tol: float = 1e-13
    max_iter: int = 10
    oracle_freq: Optional[Sequence[int]] = None   # frequency subset the oracle solves


CONFIGS: List[ConfigSpec] = [
    ConfigSpec("n256_5freq", 256, 0.5, 2.0, 5, "unit", ("0",)),
    ConfigSpec("n2157_21freq", 2157, 0.5, 2.0, 21, "unit", ("0", "n/2")),
    ConfigSpec("n8000_1freq", 8000, 1.3, 1.3, 1, "random", ()),
    ConfigSpec("n16384_8freq", 16384, 0.5, 2.0, 8, "unit", ("0", "1", "n/2", "n-1"),
               oracle_freq=(0, 7)),
    ConfigSpec("n4096_41freq_resonance", 4096, 0.9, 1.1, 41, "unit", ("0",),
               zs_scale=1e-4),
]


def _unit_index(sym: str, n: int) -> int:
    if sym == "n/2":
        return n // 2
    if sym == "n-1":
        return n - 1
    return int(sym)


@dataclasses.dataclass
class Workload:
    """All inputs of one sweep, in float64 / complex128 host arrays."""

    spec: ConfigSpec
    L: np.ndarray          # (n, n) float64, exactly symmetric
    Psi: np.ndarray        # (n, n) float64, exactly symmetric
    g: np.ndarray          # (n,) float64, diagonal of G
    omega: np.ndarray      # (nfreq,) float64
    zs: np.ndarray         # (nfreq,) complex128, Zs(omega)
    B: np.ndarray          # (nrhs, n) complex128, right-hand sides as rows
    unit_cols: List[int]   # column index of each unit right-hand side (empty if random)

    @property
    def n(self) -> int:
        return self.L.shape[0]

    @property
    def nrhs(self) -> int:
        return self.B.shape[0]

    @property
    def nfreq(self) -> int:
        return self.omega.shape[0]


def symmetric_pair(rng: np.random.Generator, n: int):
    """Draw two symmetric matrices S1, S2 = (B + B^T) / (2 sqrt(n))."""
    b1 = rng.standard_normal((n, n))
    b2 = rng.standard_normal((n, n))
    d = 2.0 * math.sqrt(n)
    s1 = (b1 + b1.T) / d
    s2 = (b2 + b2.T) / d
    return s1, s2


def make_matrices(n: int, seed: int = 0):
    """L, Psi, g and the generator state after drawing them (draw order fixed)."""
    rng = np.random.default_rng(seed)
    s1, s2 = symmetric_pair(rng, n)
    u = rng.uniform(0.5, 1.5, n)
    idx = np.arange(n)
    s1[idx, idx] += 2.0
    s2[idx, idx] += 2.0
    return s1, s2, u, rng


def zs_values(omega: np.ndarray, scale: float) -> np.ndarray:
    """Zs(w) = scale * (1 + j) * sqrt(w) for every frequency."""
    r = scale * np.sqrt(omega)
    return r + 1j * r


def make_workload(spec: ConfigSpec, seed: int = 0, n: Optional[int] = None,
                  nfreq: Optional[int] = None) -> Workload:
    """Build the inputs of ``spec``; ``n``/``nfreq`` override its sizes (for small cases)."""
    n = spec.n if n is None else int(n)
    nf = spec.nfreq if nfreq is None else int(nfreq)
    L, Psi, g, rng = make_matrices(n, seed)
    omega = np.linspace(spec.omega_lo, spec.omega_hi, nf)
    zs = zs_values(omega, spec.zs_scale)
    unit_cols: List[int] = []
    if spec.rhs == "random":
        br = rng.standard_normal(n)
        bi = rng.standard_normal(n)
        B = ((br + 1j * bi) / math.sqrt(2.0)).reshape(1, n)
    else:
        unit_cols = [_unit_index(s, n) for s in spec.unit_index]
        B = np.zeros((len(unit_cols), n), dtype=np.complex128)
        for r, k in enumerate(unit_cols):
            B[r, k] = 1.0
    return Workload(spec, L, Psi, g, omega, zs, np.ascontiguousarray(B), unit_cols)


def make_quasistatic_workload(n: int, nfreq: int = 41, seed: int = 0,
                              alpha: float = 0.05) -> Workload:
    """A smooth sweep for the reduced-order (adaptive frequency sampling)
    path: the configs' construction with L scaled by ``alpha``, so every
    resonance of w^2 L = Psi lies above the band w in [0.5, 2] (the response
    is smooth there, as for a structure below its first resonance).  Zs(w) =
    0.01 (1 + j) sqrt(w), ``nfreq`` candidate frequencies, b = e_0."""
    L, Psi, g, _ = make_matrices(n, seed)
    L = alpha * L
    omega = np.linspace(0.5, 2.0, nfreq)
    zs = zs_values(omega, 0.01)
    B = np.zeros((1, n), dtype=np.complex128)
    B[0, 0] = 1.0
    spec = ConfigSpec(name="n%d_%dfreq_quasistatic" % (n, nfreq), n=n, nfreq=nfreq, omega_lo=0.5,
                      omega_hi=2.0, zs_scale=0.01, rhs="unit", unit_index=("0",), tol=1e-13, max_iter=10)
    return Workload(spec, np.ascontiguousarray(L), Psi, g, omega, zs, B, [0])


def config(i: int) -> ConfigSpec:
    return CONFIGS[i]


def config_by_name(name: str) -> ConfigSpec:
    for c in CONFIGS:
        if c.name == name:
            return c
    raise KeyError(name)


def random_rhs(rng: np.random.Generator, n: int, nrhs: int) -> np.ndarray:
    """nrhs rows of iid (N(0,1) + j N(0,1)) / sqrt(2) entries."""
    br = rng.standard_normal((nrhs, n))
    bi = rng.standard_normal((nrhs, n))
    return (br + 1j * bi) / math.sqrt(2.0)


def make_matrices_device(n: int, seed: int = 0, device="cuda"):
    """L, Psi, g with the construction above drawn by torch's generator on
    the device (for timing runs at large n, where numpy's draws would take
    longer than the measurement; the values differ from make_matrices')."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    d = 2.0 * math.sqrt(n)
    out = []
    for _ in range(2):
        b = torch.randn((n, n), generator=gen, dtype=torch.float64, device=device)
        s = (b + b.T) / d
        del b
        s.diagonal().add_(2.0)
        out.append(s.contiguous())
    u = torch.rand(n, generator=gen, dtype=torch.float64, device=device) + 0.5
    return out[0], out[1], u
