"""Thin Python binding of libmsolve.so (argument marshalling only).

Every function here forwards to the C-ABI entry point of the same name
(declared in include/msolve.h); all arithmetic runs in the library's HIP
kernels (or, for ``host_solve_c128`` and the fallback, in its host code).
PyTorch provides device memory and the current stream.  If the library is
missing the import fails: there is no other code path.

Layouts: complex matrices are contiguous row-major torch tensors of dtype
complex128 / complex64; right-hand sides and solutions are rows
(``nrhs x n``).
"""
from __future__ import annotations

import collections
import ctypes
import dataclasses
import os
from typing import List, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmsolve.so")

_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_dbl = ctypes.c_double
_ptr = ctypes.c_void_p
_sz = ctypes.c_size_t

OK = 0
E_ARG = -1
E_HIP = -2
E_WORKSPACE = -3
E_FALLBACK = -4
E_DEVICE = -5

# MSOLVE_FWD_TOL of msolve.h: the refinement's bound on its forward error estimate
FWD_TOL = 5e-11

(K_ASSEMBLE, K_LU_DIAG, K_LU_PANEL, K_LU_UPDATE, K_TRSV_FWD, K_TRSV_BWD, K_RESIDUAL,
 K_LU_BULK) = range(8)
KERNEL_NAMES = ["assemble", "lu_diag", "lu_panel", "lu_update", "trsv_fwd", "trsv_bwd", "residual",
                "lu_bulk", "afs_project", "gepp_update"]


class RhsInfo(ctypes.Structure):
    _fields_ = [("iters", _i32), ("converged", _i32), ("fallback", _i32), ("status", _i32),
                ("eta", _dbl), ("eta_first", _dbl), ("fwd_est", _dbl)]


class FreqInfo(ctypes.Structure):
    _fields_ = [("iters_max", _i32), ("fallback", _i32), ("status", _i32), ("pivot_info", _i32),
                ("eta_max", _dbl), ("t_assemble_ms", _dbl), ("t_factor_ms", _dbl),
                ("t_refine_ms", _dbl)]


class MsolveError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("msolve status %d: %s" % (status, msg))
        self.status = status


class FallbackError(MsolveError):
    """A sweep in which the direct solve found some frequency's Z singular.
    ``result`` holds what the call returned for every frequency (the
    singular ones have status E_FALLBACK and NaN solutions)."""

    def __init__(self, status: int, msg: str, result):
        super().__init__(status, msg)
        self.result = result


EXPORTS = {
    "msolve_version": (_i32, []),
    "msolve_last_error": (ctypes.c_char_p, []),
    "msolve_block_size": (_i64, [_i64]),
    "msolve_dinv_floats": (_sz, [_i64]),
    "msolve_factor_workspace_bytes": (_sz, [_i64]),
    "msolve_refine_workspace_bytes": (_sz, [_i64, _i64]),
    "msolve_factor_batch_workspace_bytes": (_sz, [_i64, _i64]),
    "msolve_lu_solve_noalloc_max_bytes": (_sz, []),
    "msolve_lu_solve_c64_noalloc": (ctypes.c_int, [_i64, _i64, _ptr, _ptr, _ptr, _ptr]),
    "msolve_sweep_batch": (_i64, [_i64, _i64, _i64]),
    "msolve_sweep_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "msolve_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "msolve_assemble": (ctypes.c_int, [_i64, _dbl, _dbl, _dbl, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr,
                                       _ptr]),
    "msolve_factor_c64": (ctypes.c_int, [_i64, _ptr, _ptr, _ptr, _ptr, _sz, _ptr]),
    "msolve_factor_c64_sym": (ctypes.c_int, [_i64, _ptr, _ptr, _ptr, _ptr, _sz, _ptr]),
    "msolve_factor_c64_batch": (ctypes.c_int, [_i64, _i64, _ptr, _i64, _ptr, _i64, _ptr, ctypes.c_int32,
                                               _ptr, _sz, _ptr]),
    "msolve_lu_solve_c64": (ctypes.c_int, [_i64, _i64, _ptr, _ptr, _ptr, _ptr, _sz, _ptr]),
    "msolve_residual_c128": (ctypes.c_int, [_i64, _i64, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr]),
    "msolve_refine": (ctypes.c_int, [_i64, _i64, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _dbl, _i32,
                                     _ptr, _sz, _ptr, _ptr]),
    "msolve_sweep": (ctypes.c_int, [_i64, _i64, _ptr, _ptr, _ptr, _ptr, _ptr, _i64, _ptr, _ptr,
                                    _dbl, _i32, _ptr, _sz, _ptr, _ptr, _ptr]),
    "msolve_afs_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32]),
    "msolve_afs": (ctypes.c_int, [_i64, _i64, _ptr, _ptr, _ptr, _ptr, _ptr, _i64, _ptr, _ptr, _dbl, _i32,
                                  _dbl, _i32, _ptr, _ptr, _ptr, _ptr, _ptr, _sz, _ptr]),
    "msolve_host_solve_c128": (ctypes.c_int, [_i64, _i64, _ptr, _ptr, _ptr]),
    "msolve_gepp_workspace_bytes": (_sz, [_i64]),
    "msolve_gepp_solve_c128": (ctypes.c_int, [_i64, _i64, _ptr, _ptr, _ptr, _ptr, _sz, _ptr]),
    "msolve_profile_enable": (ctypes.c_int, [_i32]),
    "msolve_profile_reset": (ctypes.c_int, []),
    "msolve_profile_query": (ctypes.c_int, [_i32, ctypes.POINTER(_i64), ctypes.POINTER(_dbl),
                                            ctypes.POINTER(_dbl)]),
}


def _load() -> ctypes.CDLL:
    # torch first: its extension libraries ask for the HIP runtime by a name
    # that does not match the library's own request (libamdhip64.so versus
    # libamdhip64.so.7), so loading this library first would put a second
    # HIP runtime in the process, one that then finds no device.  Loaded
    # after torch, the library binds to torch's runtime and shares its
    # device memory and streams.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError("libmsolve.so is not built (%s); run "
                          "`python mixed_precision_refinement_amd/build.py`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in EXPORTS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def last_error() -> str:
    return lib.msolve_last_error().decode(errors="replace")


def _check(status: int) -> None:
    if status != OK:
        raise MsolveError(status, last_error())


# ---------------------------------------------------------------- helpers

def _torch():
    import torch
    return torch


def _stream(stream=None) -> int:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _dev_ptr(t, dtype, shape: Optional[Tuple[int, ...]] = None, name: str = "tensor") -> int:
    if t is None:
        return 0
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if t.dtype != dtype:
        raise ValueError("%s must have dtype %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, shape, tuple(t.shape)))
    return int(t.data_ptr())


def workspace(nbytes: int, device=None):
    torch = _torch()
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8,
                       device=device if device is not None else "cuda")


def version() -> int:
    return int(lib.msolve_version())


def block_size(n: int) -> int:
    return int(lib.msolve_block_size(n))


def dinv_floats(n: int) -> int:
    return int(lib.msolve_dinv_floats(n))


def workspace_bytes(n: int, nrhs: int, nfreq: int = 1) -> int:
    return int(lib.msolve_workspace_bytes(n, nrhs, nfreq))


def factor_workspace_bytes(n: int) -> int:
    return int(lib.msolve_factor_workspace_bytes(n))


def factor_batch_workspace_bytes(n: int, nf: int) -> int:
    return int(lib.msolve_factor_batch_workspace_bytes(n, nf))


def refine_workspace_bytes(n: int, nrhs: int) -> int:
    return int(lib.msolve_refine_workspace_bytes(n, nrhs))


def sweep_batch(n: int, nrhs: int, nfreq: int) -> int:
    return int(lib.msolve_sweep_batch(n, nrhs, nfreq))


def sweep_workspace_bytes(n: int, nrhs: int, nfreq: int) -> int:
    return int(lib.msolve_sweep_workspace_bytes(n, nrhs, nfreq))


# ------------------------------------------------------------ entry points

def assemble(L, Psi, g, omega: float, zs: complex, Z128=None, Z64=None, zrowabs=None,
             want=("z128", "z64", "zrowabs"), stream=None):
    """msolve_assemble: returns (Z128, Z64, zrowabs); outputs not in ``want``
    and not given are None."""
    torch = _torch()
    n = int(L.shape[0])
    dev = L.device
    if Z128 is None and "z128" in want:
        Z128 = torch.empty((n, n), dtype=torch.complex128, device=dev)
    if Z64 is None and "z64" in want:
        Z64 = torch.empty((n, n), dtype=torch.complex64, device=dev)
    if zrowabs is None and "zrowabs" in want:
        zrowabs = torch.empty(n, dtype=torch.float64, device=dev)
    zs = complex(zs)
    _check(lib.msolve_assemble(n, float(omega), zs.real, zs.imag,
                               _dev_ptr(L, torch.float64, (n, n), "L"),
                               _dev_ptr(Psi, torch.float64, (n, n), "Psi"),
                               _dev_ptr(g, torch.float64, (n,), "g"),
                               _dev_ptr(Z128, torch.complex128, (n, n), "Z128"),
                               _dev_ptr(Z64, torch.complex64, (n, n), "Z64"),
                               _dev_ptr(zrowabs, torch.float64, (n,), "zrowabs"),
                               _stream(stream)))
    return Z128, Z64, zrowabs


def factor_c64(A, Dinv=None, d_info=None, work=None, stream=None, sym=False):
    """msolve_factor_c64 (sym: msolve_factor_c64_sym) in place on A (complex64
    n x n); returns (A, Dinv, d_info)."""
    torch = _torch()
    n = int(A.shape[0])
    if Dinv is None:
        Dinv = torch.empty(dinv_floats(n), dtype=torch.float32, device=A.device)
    if d_info is None:
        d_info = torch.zeros(1, dtype=torch.int32, device=A.device)
    wb = factor_workspace_bytes(n)
    if work is None:
        work = workspace(wb, A.device)
    fn = lib.msolve_factor_c64_sym if sym else lib.msolve_factor_c64
    _check(fn(n, _dev_ptr(A, torch.complex64, (n, n), "A"),
              _dev_ptr(Dinv, torch.float32, (dinv_floats(n),), "Dinv"),
              _dev_ptr(d_info, torch.int32, (1,), "d_info"),
              int(work.data_ptr()), int(work.numel()), _stream(stream)))
    return A, Dinv, d_info


def factor_c64_batch(A, sym=False, Dinv=None, d_info=None, work=None, stream=None):
    """msolve_factor_c64_batch in place on A (complex64 nf x n x n, contiguous);
    returns (A, Dinv (nf x dinv_floats(n) float32), d_info (nf int32))."""
    torch = _torch()
    nf, n = int(A.shape[0]), int(A.shape[1])
    if Dinv is None:
        Dinv = torch.empty((nf, dinv_floats(n)), dtype=torch.float32, device=A.device)
    if d_info is None:
        d_info = torch.zeros(nf, dtype=torch.int32, device=A.device)
    if work is None:
        work = workspace(factor_batch_workspace_bytes(n, nf), A.device)
    _check(lib.msolve_factor_c64_batch(n, nf, _dev_ptr(A, torch.complex64, (nf, n, n), "A"), 2 * n * n,
                                       _dev_ptr(Dinv, torch.float32, (nf, dinv_floats(n)), "Dinv"),
                                       dinv_floats(n), _dev_ptr(d_info, torch.int32, (nf,), "d_info"),
                                       1 if sym else 0, int(work.data_ptr()), int(work.numel()),
                                       _stream(stream)))
    return A, Dinv, d_info


def lu_solve_c64(LU, Dinv, RHS, work=None, stream=None):
    """msolve_lu_solve_c64: RHS (complex64 nrhs x n) is overwritten with the solution."""
    torch = _torch()
    n = int(LU.shape[0])
    nrhs = int(RHS.shape[0])
    if work is None:
        work = workspace(refine_workspace_bytes(n, nrhs), LU.device)
    _check(lib.msolve_lu_solve_c64(n, nrhs, _dev_ptr(LU, torch.complex64, (n, n), "LU"),
                                   _dev_ptr(Dinv, torch.float32, None, "Dinv"),
                                   _dev_ptr(RHS, torch.complex64, (nrhs, n), "RHS"),
                                   int(work.data_ptr()), int(work.numel()), _stream(stream)))
    return RHS


def lu_solve_noalloc_max_bytes() -> int:
    return int(lib.msolve_lu_solve_noalloc_max_bytes())


def lu_solve_c64_noalloc(LU, Dinv, RHS, stream=None):
    """msolve_lu_solve_c64_noalloc: as lu_solve_c64, with the library's
    fixed per-device scratch instead of a workspace (nothing is allocated)."""
    torch = _torch()
    n = int(LU.shape[0])
    nrhs = int(RHS.shape[0])
    _check(lib.msolve_lu_solve_c64_noalloc(n, nrhs, _dev_ptr(LU, torch.complex64, (n, n), "LU"),
                                           _dev_ptr(Dinv, torch.float32, None, "Dinv"),
                                           _dev_ptr(RHS, torch.complex64, (nrhs, n), "RHS"),
                                           _stream(stream)))
    return RHS


def residual_c128(Z128, B, X, R=None, norms=None, stream=None):
    """msolve_residual_c128: returns (R, norms) with norms = [||r_k||..., ||x_k||...]."""
    torch = _torch()
    n = int(Z128.shape[0])
    nrhs = int(B.shape[0])
    if R is None:
        R = torch.empty((nrhs, n), dtype=torch.complex128, device=Z128.device)
    if norms is None:
        norms = torch.empty(2 * nrhs, dtype=torch.float64, device=Z128.device)
    _check(lib.msolve_residual_c128(n, nrhs, _dev_ptr(Z128, torch.complex128, (n, n), "Z128"),
                                    _dev_ptr(B, torch.complex128, (nrhs, n), "B"),
                                    _dev_ptr(X, torch.complex128, (nrhs, n), "X"),
                                    _dev_ptr(R, torch.complex128, (nrhs, n), "R"),
                                    _dev_ptr(norms, torch.float64, (2 * nrhs,), "norms"),
                                    _stream(stream)))
    return R, norms


@dataclasses.dataclass
class RhsResult:
    iters: int
    converged: bool
    fallback: bool
    status: int
    eta: float
    eta_first: float
    fwd_est: float


def _rhs(r: RhsInfo) -> RhsResult:
    return RhsResult(int(r.iters), bool(r.converged), bool(r.fallback), int(r.status),
                     float(r.eta), float(r.eta_first), float(r.fwd_est))


def refine(Z128, LU, Dinv, B, X=None, tol: float = 1e-13, max_iter: int = 10, zrowabs=None,
           work=None, stream=None, device_fallback: bool = True):
    """msolve_refine: returns (X, [RhsResult per right-hand side]).  Without
    ``work``, the workspace allocated here also holds the device direct
    solve's buffers when ``device_fallback`` is true (else that solve runs on
    the host)."""
    torch = _torch()
    n = int(Z128.shape[0])
    nrhs = int(B.shape[0])
    if X is None:
        X = torch.empty((nrhs, n), dtype=torch.complex128, device=Z128.device)
    if work is None:
        nb = refine_workspace_bytes(n, nrhs)
        if device_fallback:
            nb += gepp_workspace_bytes(n)
        work = workspace(nb, Z128.device)
    info = (RhsInfo * nrhs)()
    _check(lib.msolve_refine(n, nrhs, _dev_ptr(Z128, torch.complex128, (n, n), "Z128"),
                             _dev_ptr(zrowabs, torch.float64, (n,), "zrowabs"),
                             _dev_ptr(LU, torch.complex64, (n, n), "LU"),
                             _dev_ptr(Dinv, torch.float32, None, "Dinv"),
                             _dev_ptr(B, torch.complex128, (nrhs, n), "B"),
                             _dev_ptr(X, torch.complex128, (nrhs, n), "X"),
                             float(tol), int(max_iter), int(work.data_ptr()), int(work.numel()),
                             info, _stream(stream)))
    return X, [_rhs(r) for r in info]


@dataclasses.dataclass
class FreqResult:
    iters_max: int
    fallback: bool
    status: int
    pivot_info: int
    eta_max: float
    t_assemble_ms: float
    t_factor_ms: float
    t_refine_ms: float


def sweep(L, Psi, g, omega: Sequence[float], zs: Sequence[complex], B, tol: float = 1e-13,
          max_iter: int = 10, X=None, work=None, stream=None, check: bool = True):
    """msolve_sweep: returns (X[nfreq, nrhs, n], [FreqResult], [[RhsResult]]).
    If the direct solve finds some frequency singular, every other frequency
    is still solved; with ``check`` a FallbackError carrying those results is
    raised, without it they are returned (the singular frequencies have
    status E_FALLBACK)."""
    torch = _torch()
    n = int(L.shape[0])
    nrhs = int(B.shape[0])
    om = np.ascontiguousarray(np.asarray(omega, dtype=np.float64))
    nfreq = int(om.shape[0])
    zsa = np.ascontiguousarray(np.asarray(zs, dtype=np.complex128))
    if zsa.shape[0] != nfreq:
        raise ValueError("zs must have one value per frequency")
    if X is None:
        X = torch.empty((nfreq, nrhs, n), dtype=torch.complex128, device=L.device)
    if work is None:
        work = workspace(max(sweep_workspace_bytes(n, nrhs, nfreq), 256), L.device)
    finfo = (FreqInfo * max(nfreq, 1))()
    rinfo = (RhsInfo * max(nfreq * nrhs, 1))()
    st = int(lib.msolve_sweep(n, nfreq, om.ctypes.data, zsa.ctypes.data,
                              _dev_ptr(L, torch.float64, (n, n), "L"),
                              _dev_ptr(Psi, torch.float64, (n, n), "Psi"),
                              _dev_ptr(g, torch.float64, (n,), "g"), nrhs,
                              _dev_ptr(B, torch.complex128, (nrhs, n), "B"),
                              _dev_ptr(X, torch.complex128, (nfreq, nrhs, n), "X"),
                              float(tol), int(max_iter), int(work.data_ptr()), int(work.numel()),
                              finfo, rinfo, _stream(stream)))
    if st != OK and st != E_FALLBACK:
        _check(st)
    fr = [FreqResult(int(f.iters_max), bool(f.fallback), int(f.status), int(f.pivot_info),
                     float(f.eta_max), float(f.t_assemble_ms), float(f.t_factor_ms),
                     float(f.t_refine_ms)) for f in finfo[:nfreq]]
    rr = [[_rhs(rinfo[f * nrhs + k]) for k in range(nrhs)] for f in range(nfreq)]
    if st == E_FALLBACK and check:
        raise FallbackError(st, last_error(), (X, fr, rr))
    return X, fr, rr


def afs_workspace_bytes(n: int, nrhs: int, nfreq: int, max_exact: int) -> int:
    return int(lib.msolve_afs_workspace_bytes(n, nrhs, nfreq, max_exact))


AfsResult = collections.namedtuple("AfsResult", "exact estimate q")


def afs(L, Psi, g, omega: Sequence[float], zs: Sequence[complex], B, tol: float = 1e-4,
        max_exact: Optional[int] = None, solve_tol: float = 1e-13, solve_max_iter: int = 10,
        X=None, work=None, stream=None):
    """msolve_afs (reduced-order sweep): returns (X[nfreq, nrhs, n], AfsResult).
    max_exact defaults to min(nfreq, 64): the workspace holds a basis of
    2 nrhs max_exact vectors and their Gram matrix."""
    torch = _torch()
    n = int(L.shape[0])
    nrhs = int(B.shape[0])
    om = np.ascontiguousarray(np.asarray(omega, dtype=np.float64))
    nfreq = int(om.shape[0])
    zsa = np.ascontiguousarray(np.asarray(zs, dtype=np.complex128))
    if zsa.shape[0] != nfreq:
        raise ValueError("zs must have one value per frequency")
    cap = min(nfreq, 64) if max_exact is None else int(max_exact)
    if X is None:
        X = torch.empty((nfreq, nrhs, n), dtype=torch.complex128, device=L.device)
    if work is None:
        work = workspace(max(afs_workspace_bytes(n, nrhs, max(nfreq, 1), max(cap, 1)), 256), L.device)
    exact = np.zeros(max(nfreq, 1), dtype=np.int32)
    est = np.zeros(max(nfreq, 1), dtype=np.float64)
    n_exact = ctypes.c_int32(0)
    q = ctypes.c_int32(0)
    _check(lib.msolve_afs(n, nfreq, om.ctypes.data, zsa.ctypes.data,
                          _dev_ptr(L, torch.float64, (n, n), "L"),
                          _dev_ptr(Psi, torch.float64, (n, n), "Psi"),
                          _dev_ptr(g, torch.float64, (n,), "g"), nrhs,
                          _dev_ptr(B, torch.complex128, (nrhs, n), "B"),
                          _dev_ptr(X, torch.complex128, (nfreq, nrhs, n), "X"),
                          float(tol), cap, float(solve_tol), int(solve_max_iter),
                          exact.ctypes.data, ctypes.byref(n_exact), est.ctypes.data, ctypes.byref(q),
                          int(work.data_ptr()), int(work.numel()), _stream(stream)))
    return X, AfsResult([int(v) for v in exact[:n_exact.value]], est[:nfreq].copy(), int(q.value))


def gepp_workspace_bytes(n: int) -> int:
    return int(lib.msolve_gepp_workspace_bytes(int(n)))


def gepp_solve_c128(Z, B, X=None, work=None, stream=None):
    """msolve_gepp_solve_c128: X = Z^-1 B on the device (complex128 LU with
    partial pivoting); Z is complex128 n x n, B complex128 nrhs x n."""
    torch = _torch()
    n = int(Z.shape[0])
    nrhs = int(B.shape[0])
    if X is None:
        X = torch.empty((nrhs, n), dtype=torch.complex128, device=Z.device)
    if work is None:
        work = workspace(gepp_workspace_bytes(n), Z.device)
    _check(lib.msolve_gepp_solve_c128(n, nrhs, _dev_ptr(Z, torch.complex128, (n, n), "Z"),
                                      _dev_ptr(B, torch.complex128, (nrhs, n), "B"),
                                      _dev_ptr(X, torch.complex128, (nrhs, n), "X"),
                                      int(work.data_ptr()), int(work.numel()), _stream(stream)))
    return X


def host_solve_c128(Z: np.ndarray, B: np.ndarray) -> np.ndarray:
    """msolve_host_solve_c128 (host arrays): the fallback direct solve alone."""
    Z = np.ascontiguousarray(Z, dtype=np.complex128)
    B = np.ascontiguousarray(np.atleast_2d(B), dtype=np.complex128)
    n = Z.shape[0]
    X = np.empty_like(B)
    _check(lib.msolve_host_solve_c128(n, B.shape[0], Z.ctypes.data, B.ctypes.data, X.ctypes.data))
    return X


# ---------------------------------------------------------------- timing

def profile_enable(on: bool = True) -> None:
    _check(lib.msolve_profile_enable(1 if on else 0))


def profile_reset() -> None:
    _check(lib.msolve_profile_reset())


def profile_query(kernel: int) -> Tuple[int, float, float]:
    """(launches, total_ms, algorithmic flops-or-bytes) for one kernel id."""
    n = _i64(0)
    ms = _dbl(0.0)
    work = _dbl(0.0)
    _check(lib.msolve_profile_query(int(kernel), ctypes.byref(n), ctypes.byref(ms),
                                    ctypes.byref(work)))
    return int(n.value), float(ms.value), float(work.value)
