"""msolve_lu_solve_c64_noalloc (the triangular solves with the library's fixed
per-device scratch) against msolve_lu_solve_c64 (the same solves with a
caller-owned workspace), through the C-ABI: two calls in a row, the second
with a smaller system, each bit-identical to the workspace entry point, and
no device memory taken by the second."""
from __future__ import annotations

import ctypes

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


def factors(ms, n, seed):
    wl = workloads.make_workload(workloads.config(0), n=n, nfreq=1, seed=seed)
    _, Z64, _ = ms.assemble(dev(wl.L), dev(wl.Psi), dev(wl.g), wl.omega[0], wl.zs[0], want=("z64",))
    _, Dinv, info = ms.factor_c64(Z64)
    torch.cuda.synchronize()
    assert int(info.item()) == 0
    return Z64, Dinv


def test_noalloc_solve_matches_workspace_solve_twice(ms):
    lib = ms.lib
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for call, (n, nrhs, seed) in enumerate([(300, 3, 1), (130, 2, 2)]):
        print("noalloc call %d: n=%d nrhs=%d" % (call, n, nrhs), flush=True)
        LU, Dinv = factors(ms, n, seed)
        B = workloads.random_rhs(np.random.default_rng(100 + call), n, nrhs).astype(np.complex64)
        R1 = dev(B)
        work = ms.workspace(ms.refine_workspace_bytes(n, nrhs))
        st = lib.msolve_lu_solve_c64(n, nrhs, LU.data_ptr(), Dinv.data_ptr(), R1.data_ptr(),
                                     work.data_ptr(), work.numel(), stream)
        assert st == ms.OK, ms.last_error()
        torch.cuda.synchronize()
        R2 = dev(B)
        free_before = torch.cuda.mem_get_info()[0]
        st = lib.msolve_lu_solve_c64_noalloc(n, nrhs, LU.data_ptr(), Dinv.data_ptr(), R2.data_ptr(), stream)
        assert st == ms.OK, ms.last_error()
        torch.cuda.synchronize()
        if call > 0:
            # (the first call may map the library's code object that holds
            # the scratch array, once per process and device)
            assert torch.cuda.mem_get_info()[0] == free_before
        x1, x2 = R1.cpu().numpy(), R2.cpu().numpy()
        assert np.array_equal(x1.view(np.uint32), x2.view(np.uint32))
        # and both are the solution with these factors (the oracle's
        # complex128 substitution, within single-precision rounding)
        F = LU.cpu().numpy().astype(np.complex128)
        xo = oracle.lu_solve(F, B.astype(np.complex128))
        assert np.max(oracle.forward_error(x2.astype(np.complex128), xo)) <= 1e-3


def test_noalloc_rejects_problems_beyond_its_scratch(ms):
    cap = ms.lu_solve_noalloc_max_bytes()
    assert cap == 8 << 20
    n, nrhs = 1 << 16, 8
    assert ms.refine_workspace_bytes(n, nrhs) > cap
    st = ms.lib.msolve_lu_solve_c64_noalloc(n, nrhs, 1, 1, 1, None)
    assert st == ms.E_WORKSPACE
    assert "scratch" in ms.last_error()
