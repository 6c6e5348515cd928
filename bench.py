"""Benchmark: frequency solves per second of the full refinement path.

One step = one frequency sweep of the workload (every stage of the path:
Z(w) assembly, complex64 LU, triangular solves, complex128 residual, the
refinement loop with its stop test and fallback), with L, Psi, g and the
right-hand sides already resident on the GPU.  Default workload: n = 2157,
21 frequencies in [0.5, 2], right-hand sides e_0 and e_1078.

Prints ONE JSON line.  ``value`` is the number of frequencies over the
median time of one sweep (each of the K timed sweeps is timed on its own;
the K sweeps together are bracketed by device synchronisations).  It counts
only if the timed answers pass the accuracy bars: every frequency converged
without error with a device backward error <= 1e-13, and every frequency the
CPU oracle solves (all of them by default) agrees with the oracle to a
forward error <= 1e-10 and a backward error <= 1e-13; otherwise ``value`` is
null and ``invalid`` says why.  Besides the throughput the line reports, for
the kernel that takes the most time, its achieved rate against the MI355X
roofline (from HIP events bracketing every launch inside the timed region),
a per-kernel breakdown, the general LU's rate at n = 2157 (batch), 8000 and
16384, and the oracle itself timed on the same frequencies.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "frequency solves/s at N=2157 (fp64-accurate); LU TFLOP/s as % FP32 MFMA peak"
PEAK_FP32_MFMA_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0

# kernel id -> (bound, unit) of its roofline
ROOFLINE = {
    0: ("hbm", "GB/s"),     # assemble
    1: ("alu", "TFLOP/s"),  # lu_diag (serial, one workgroup)
    2: ("mfma", "TFLOP/s"),  # lu_panel
    3: ("mfma", "TFLOP/s"),  # lu_update
    4: ("hbm", "GB/s"),     # trsv_fwd
    5: ("hbm", "GB/s"),     # trsv_bwd
    6: ("hbm", "GB/s"),     # residual
    7: ("mfma", "TFLOP/s"),  # lu_bulk (the bulk trailing updates)
    8: ("hbm", "GB/s"),     # afs_project (reduced-order sweep: L V, Psi V)
    9: ("alu", "TFLOP/s"),  # gepp_update (device fallback: fp64 trailing updates)
}
# fp32 vector peak without packed instructions: 256 CU x 64 lanes x 2 flop x 2.4 GHz
PEAK_FP32_VALU_TFLOPS = 78.6
# fp64 vector FMA runs at the same rate: 256 CU x 64 lanes x 2 flop x 2.4 GHz
PEAK_FP64_VALU_TFLOPS = 78.6

# HBM bytes per launch from rocprofv3 --pmc runs of this same command
# (FETCH_SIZE and WRITE_SIZE, each scaled by its reading for a plain copy of
# known size), per kernel and workload, with the summary they come from and
# the SHA-256 prefix of the kernel's source file when the counters were
# taken.  A figure whose source file has changed since is reported as null
# (the kernel it measured no longer exists); a kernel missing here has not
# been measured in its current version.
MEASURED_TRAFFIC = {
    # profiles/sweep_n2157_21freq_hbm_traffic.md (FETCH_SIZE x 2.0, WRITE_SIZE x 1.0);
    # the sweep's kernels (symmetric factorisation) per launch over the whole
    # batch (the refinement's empty launches of a pass queued after the last
    # system stopped excluded)
    ("n2157_21freq", "lu_bulk"): (627730000, "lu.hip", "ae89b56f34125c62"),
    ("n2157_21freq", "lu_update"): (80818000, "lu.hip", "ae89b56f34125c62"),
    ("n2157_21freq", "lu_panel"): (39061000, "lu.hip", "ae89b56f34125c62"),
    ("n2157_21freq", "lu_diag"): (2701000, "lu.hip", "ae89b56f34125c62"),
    ("n2157_21freq", "trsv_fwd"): (428800000, "trsv.hip", "6ea50d6778772e65"),
    ("n2157_21freq", "trsv_bwd"): (439750000, "trsv.hip", "6ea50d6778772e65"),
    ("n2157_21freq", "residual"): (90561000, "residual.hip", "a5748f4bf30c2098"),
    ("n2157_21freq", "assemble"): (505721000, "assemble.hip", "013250d86983f92c"),
    # the same passes: the stored-Z residual at n = 8000 (23 launches); the
    # reduced-order sweep's projection at n = 2157 (30 launches) from the
    # earlier passes of the summary, whose afs.hip is the current one
    ("n8000_gemv", "residual"): (1025749000, "residual.hip", "a5748f4bf30c2098"),
    ("n2157_quasistatic", "afs_project"): (75779676, "afs.hip", "eb2f87cd4a688bc5"),
}
CSRC = os.path.join(ROOT, "mixed_precision_refinement_amd", "csrc")
TRAFFIC_SOURCE = "profiles/sweep_n2157_21freq_hbm_traffic.md, profiles/lu_factorisation_mfma_counters.md"


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def measured_traffic(workload, kernel):
    """The measured HBM bytes per launch, or None if unmeasured or stale."""
    import hashlib
    entry = MEASURED_TRAFFIC.get((workload, kernel))
    if entry is None:
        return None
    nbytes, src, sha = entry
    with open(os.path.join(CSRC, src), "rb") as f:
        if hashlib.sha256(f.read()).hexdigest()[:16] != sha:
            return None
    return nbytes


FWD_TOL = 1e-10     # forward error bar against the oracle
ETA_TOL = 1e-13     # backward error bar


def parse():
    p = argparse.ArgumentParser(description=__doc__)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=7)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--config", type=int, default=1, help="workload index (default 1: n=2157)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-freqs", type=int, default=0,
                   help="frequencies of the workload the oracle solves for the baseline and the "
                        "accuracy check (0: all)")
    p.add_argument("--no-afs", action="store_true",
                   help="skip the reduced-order sweep measurement")
    p.add_argument("--no-fallback-solve", action="store_true",
                   help="skip the measurement of the device fallback direct solve")
    p.add_argument("--no-gemv", action="store_true",
                   help="skip the stored-Z residual measurement at n = 8000")
    p.add_argument("--lu-sizes", type=str, default="8000,16384",
                   help="orders of the single-matrix factorisation timings (comma separated; "
                        "empty: none)")
    p.add_argument("--no-copy-bw", action="store_true",
                   help="skip the plain-copy bandwidth measurement (1 GiB device copy)")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="after the run, one device-to-device copy of MIB MiB (a plain copy kernel "
                        "of known traffic, to scale hardware byte counters)")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: the solver runs on one GPU; --gpus %d is not supported "
              "(a sweep would shard its frequencies one batch per GPU, with no exchange "
              "between GPUs)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import workloads
    from mixed_precision_refinement_amd import msolve

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    spec = workloads.config(args.config)
    wl = workloads.make_workload(spec)
    n, nrhs, nfreq = wl.n, wl.nrhs, wl.nfreq
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    L, P, g, B = dev(wl.L), dev(wl.Psi), dev(wl.g), dev(wl.B)
    X = torch.empty((nfreq, nrhs, n), dtype=torch.complex128, device="cuda")
    work = msolve.workspace(msolve.sweep_workspace_bytes(n, nrhs, nfreq))
    stream = torch.cuda.current_stream()

    def step():
        return msolve.sweep(L, P, g, wl.omega, wl.zs, B, tol=spec.tol, max_iter=spec.max_iter,
                            X=X, work=work)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region 1: throughput.  msolve_sweep returns once its answers
    # are complete, so each sweep is timed on its own by the host clock
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    finfo = None
    step_s = []
    all_ok = True
    dev_eta_max = 0.0
    for _ in range(args.steps):
        t1 = time.perf_counter()
        _, finfo, rinfo = step()
        step_s.append(time.perf_counter() - t1)
        all_ok = all_ok and all(f.status == 0 for f in finfo)
        dev_eta_max = max(dev_eta_max, max(f.eta_max for f in finfo))
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    median_s = float(np.median(step_s))
    ms_per_step = 1000.0 * median_s
    value = nfreq / median_s

    # timed region 2: the same steps with every kernel launch bracketed by
    # HIP events on the stream it runs on
    msolve.profile_reset()
    msolve.profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall_prof = time.perf_counter() - t0
    msolve.profile_enable(False)
    kernels = {}
    for k, name in enumerate(msolve.KERNEL_NAMES):
        cnt, ms, work_units = msolve.profile_query(k)
        if cnt == 0:
            continue
        bound, unit = ROOFLINE[k]
        rate = work_units / (ms * 1e-3)
        kernels[name] = {
            "launches_per_step": cnt / args.steps,
            "ms_per_step": ms / args.steps,
            "avg_launch_us": 1000.0 * ms / cnt,
            "work_per_launch": work_units / cnt,
            "achieved": rate / 1e12 if unit == "TFLOP/s" else rate / 1e9,
            "unit": unit,
            "bound": bound,
        }
    msolve.profile_reset()
    dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    dk = kernels[dom]
    peak = {"mfma": PEAK_FP32_MFMA_TFLOPS, "hbm": PEAK_HBM_GBS,
            "alu": PEAK_FP32_VALU_TFLOPS}[dk["bound"]]
    roofline = {
        "kernel": dom,
        "bound": dk["bound"],
        "achieved": round(dk["achieved"], 3),
        "peak": peak,
        "unit": dk["unit"],
        "frac": round(dk["achieved"] / peak, 4),
        "traffic": measured_traffic(spec.name, dom),
        "traffic_source": TRAFFIC_SOURCE if measured_traffic(spec.name, dom) else None,
        "avg_launch_us": round(dk["avg_launch_us"], 3),
        "work_per_launch": dk["work_per_launch"],
    }
    # the sweep's factorisation (HIP events around the factorisation of each
    # batch of frequencies on the caller's stream; its kernels overlap on two
    # streams, so summed kernel times would overstate it).  L and Psi are
    # symmetric here, so every Z(w) is complex symmetric and the sweep uses
    # the symmetric factorisation: 4 n^3 / 3 flop per matrix (half of LU's).
    batch = msolve.sweep_batch(n, nrhs, nfreq)
    sym = bool(np.array_equal(wl.L, wl.L.T) and np.array_equal(wl.Psi, wl.Psi.T))
    fact_batch_ms = [float(finfo[f0].t_factor_ms) for f0 in range(0, nfreq, batch)]
    fact_wall_ms = float(sum(fact_batch_ms))
    fact_flop = (4.0 if sym else 8.0) * n ** 3 / 3.0
    fact_tflops = fact_flop * nfreq / (fact_wall_ms * 1e-3) / 1e12 if fact_wall_ms > 0 else None

    # the general LU (msolve_factor_c64_batch, sym = 0) of the same batch of
    # matrices, 8 n^3 / 3 flop per matrix, timed alone: the median of three
    # runs, each bracketed by HIP events on the caller's stream (which the
    # factorisation joins at its end)
    A0 = torch.empty((batch, n, n), dtype=torch.complex64, device="cuda")
    for f in range(batch):
        msolve.assemble(L, P, g, float(wl.omega[f]), complex(wl.zs[f]), Z64=A0[f], want=("z64",))
    A = torch.empty_like(A0)
    fwork = msolve.workspace(msolve.factor_workspace_bytes(n))
    Dl = torch.empty((batch, msolve.dinv_floats(n)), dtype=torch.float32, device="cuda")
    dl = torch.zeros(batch, dtype=torch.int32, device="cuda")
    lu_runs = []
    for rep in range(4):
        A.copy_(A0)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        msolve.factor_c64_batch(A, sym=False, Dinv=Dl, d_info=dl, work=fwork)
        e1.record(stream)
        torch.cuda.synchronize()
        if rep > 0:                      # the first run warms up
            lu_runs.append(e0.elapsed_time(e1))
    lu_ms = float(np.median(lu_runs))
    lu_tflops = 8.0 * n ** 3 / 3.0 * batch / (lu_ms * 1e-3) / 1e12
    lu_pivots_ok = bool(int(dl.abs().sum().item()) == 0)
    # the same LU once more with every factorisation launch event-timed: the
    # rate over the summed kernel durations (the look-ahead stream's kernels
    # overlap the bulk products, so the sum exceeds the wall time)
    A.copy_(A0)
    torch.cuda.synchronize()
    msolve.profile_reset()
    msolve.profile_enable(True)
    msolve.factor_c64_batch(A, sym=False, Dinv=Dl, d_info=dl, work=fwork)
    torch.cuda.synchronize()
    msolve.profile_enable(False)
    lu_kernel_ms = sum(msolve.profile_query(msolve.KERNEL_NAMES.index(k))[1]
                       for k in ("lu_diag", "lu_panel", "lu_update", "lu_bulk"))
    msolve.profile_reset()
    del A0, A, Dl

    # accuracy of the timed answers and the CPU baseline (oracle): the
    # oracle solves the chosen frequencies (all by default) on the host's
    # cores, timed, and its answers check the last timed sweep's
    Xh = X.cpu().numpy()
    acc = {}
    cpu = None
    invalid = []
    if not all_ok:
        invalid.append("a frequency returned a nonzero status")
    if not dev_eta_max <= ETA_TOL:
        invalid.append("device backward error %.3g above %g" % (dev_eta_max, ETA_TOL))
    if not args.no_cpu_baseline:
        import oracle
        threads = len(os.sched_getaffinity(0))
        oracle.set_threads(threads)
        nch = nfreq if args.cpu_freqs <= 0 else min(args.cpu_freqs, nfreq)
        pick = np.unique(np.linspace(0, nfreq - 1, nch).round().astype(int))
        fe, etas = [], []
        t_or = 0.0
        for f in pick:
            t1 = time.perf_counter()
            Z = oracle.assemble(wl.omega[f], wl.zs[f], wl.L, wl.Psi, wl.g)
            Xo = oracle.solve(Z, wl.B)
            t_or += time.perf_counter() - t1
            fe.append(float(oracle.forward_error(Xh[f], Xo).max()))
            etas.append(float(oracle.eta(Z, Xh[f], wl.B).max()))
        cpu = {
            "value": round(len(pick) / t_or, 4),
            "unit": "solves/s",
            "cores": oracle.get_threads(),
            "nproc": os.cpu_count(),
            "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": "%d of the %d frequencies%s, n=%d, %d right-hand sides each: "
                      "oracle assembly + complex128 GEPP + substitution, %.1f s"
                      % (len(pick), nfreq, "" if len(pick) == nfreq else " (indices %s)" % pick.tolist(),
                         n, nrhs, t_or),
        }
        acc = {"forward_error_max": max(fe), "eta_max": max(etas),
               "frequencies_checked": len(pick)}
        if not max(fe) <= FWD_TOL:
            invalid.append("forward error %.3g above %g" % (max(fe), FWD_TOL))
        if not max(etas) <= ETA_TOL:
            invalid.append("oracle-measured backward error %.3g above %g" % (max(etas), ETA_TOL))
    else:
        invalid.append("accuracy not checked against the oracle (--no-cpu-baseline)")
    acc["device_eta_max"] = dev_eta_max

    # the general LU of one matrix at the large orders (n = 8000 is the
    # single large factorisation, n = 16384 the large-n workload's order),
    # and the symmetric factorisation of the same matrix: inputs drawn on the
    # device with the workloads' construction (torch's generator), Z at the
    # workload's first frequency; median of three runs after one warm-up,
    # HIP events on the caller's stream (which the factorisation joins)
    def lu_rate(nn, omega, zsv, sym):
        Ld, Pd, gd = workloads.make_matrices_device(nn, seed=0)
        _, Z0, _ = msolve.assemble(Ld, Pd, gd, omega, zsv, want=("z64",))
        del Ld, Pd, gd
        Zw = torch.empty_like(Z0)
        Dv = torch.empty(msolve.dinv_floats(nn), dtype=torch.float32, device="cuda")
        di = torch.zeros(1, dtype=torch.int32, device="cuda")
        fw = msolve.workspace(msolve.factor_workspace_bytes(nn))
        runs = []
        for rep_ in range(4):
            Zw.copy_(Z0)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            msolve.factor_c64(Zw, Dinv=Dv, d_info=di, work=fw, sym=sym)
            e1.record(stream)
            torch.cuda.synchronize()
            if rep_ > 0:
                runs.append(e0.elapsed_time(e1))
        ok = int(di.item()) == 0
        del Z0, Zw, Dv
        t = float(np.median(runs))
        flop = (4.0 if sym else 8.0) * nn ** 3 / 3.0
        return {"n": nn, "ms": round(t, 4), "tflops": round(flop / (t * 1e-3) / 1e12, 3),
                "frac_fp32_mfma_peak": round(flop / (t * 1e-3) / 1e12 / PEAK_FP32_MFMA_TFLOPS, 4),
                "flop": flop, "pivots_ok": ok}

    lu_large = []
    for tok in [t for t in args.lu_sizes.split(",") if t.strip()]:
        nn = int(tok)
        ws = workloads.config(2) if nn == 8000 else workloads.config(3)
        om = float(np.linspace(ws.omega_lo, ws.omega_hi, ws.nfreq)[0])
        zsv = complex(workloads.zs_values(np.array([om]), ws.zs_scale)[0])
        lu_large.append({"general": lu_rate(nn, om, zsv, False), "symmetric": lu_rate(nn, om, zsv, True)})
        torch.cuda.empty_cache()

    # a plain device-to-device copy of 1 GiB (torch's copy kernel, HIP events
    # on the current stream, median of five after one warm-up): the
    # bandwidth a streaming kernel can reach in practice, read + write
    copy_bw = None
    if not args.no_copy_bw:
        nbytes = 1 << 30
        src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        cts = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            dst.copy_(src)
            e1.record()
            torch.cuda.synchronize()
            cts.append(e0.elapsed_time(e1))
        cms = float(np.median(cts))
        copy_bw = {"bytes_read": nbytes, "bytes_written": nbytes, "ms": round(cms, 4),
                   "GB/s": round(2.0 * nbytes / (cms * 1e-3) / 1e9, 1)}
        del src, dst
        torch.cuda.empty_cache()
        for v in kernels.values():
            if v["unit"] == "GB/s":
                v["frac_of_copy"] = v["achieved"] / copy_bw["GB/s"]

    # the residual GEMV that streams a stored complex128 Z (msolve_residual_c128,
    # the refinement's step 3 as msolve_refine runs it) at the order of the
    # single large system (n = 8000, one right-hand side: 1.02 GB of Z)
    gemv = None
    if not args.no_gemv:
        gspec = workloads.config(2)
        gn = gspec.n
        gw = workloads.make_workload(gspec)
        Zg, _, _ = msolve.assemble(dev(gw.L), dev(gw.Psi), dev(gw.g), gw.omega[0], gw.zs[0],
                                   want=("z128",))
        Bg = dev(gw.B)
        Xg = Bg.clone()
        for _ in range(3):
            msolve.residual_c128(Zg, Bg, Xg)
        torch.cuda.synchronize()
        msolve.profile_reset()
        msolve.profile_enable(True)
        for _ in range(20):
            msolve.residual_c128(Zg, Bg, Xg)
        torch.cuda.synchronize()
        msolve.profile_enable(False)
        cnt, ms, byt = msolve.profile_query(msolve.KERNEL_NAMES.index("residual"))
        msolve.profile_reset()
        rate = byt / (ms * 1e-3) / 1e9
        gemv = {"kernel": "residual (stored Z)", "n": gn, "nrhs": int(Bg.shape[0]),
                "avg_launch_us": round(1000.0 * ms / cnt, 3), "bytes_per_launch": byt / cnt,
                "achieved": round(rate, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(rate / PEAK_HBM_GBS, 4),
                "frac_of_copy": round(rate / copy_bw["GB/s"], 4) if copy_bw else None,
                "traffic": measured_traffic("n8000_gemv", "residual")}
        del Zg
    # the reduced-order sweep (adaptive frequency sampling, msolve_afs) on the
    # quasi-static stand-in of the same order, with 41 and with 1001 candidate
    # frequencies, against the exact sweep of the same candidates
    # (msolve_sweep); medians of three runs after one warm-up each (one run
    # for the exact sweep of 1001)
    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            t1 = time.perf_counter()
            r = fn()
            torch.cuda.synchronize()
            ts.append(1000.0 * (time.perf_counter() - t1))
        return float(np.median(ts)), r

    def measure_afs(nq, cap, full_reps):
        qw = workloads.make_quasistatic_workload(n, nfreq=nq)
        qL, qP, qg, qB = dev(qw.L), dev(qw.Psi), dev(qw.g), dev(qw.B)
        awork = msolve.workspace(msolve.afs_workspace_bytes(n, 1, nq, cap))
        swork = msolve.workspace(msolve.sweep_workspace_bytes(n, 1, nq))
        Xa = torch.empty((nq, 1, n), dtype=torch.complex128, device="cuda")
        Xs = torch.empty_like(Xa)
        run_afs = lambda: msolve.afs(qL, qP, qg, qw.omega, qw.zs, qB, tol=1e-4, max_exact=cap, X=Xa,
                                     work=awork)
        run_full = lambda: msolve.sweep(qL, qP, qg, qw.omega, qw.zs, qB, tol=qw.spec.tol,
                                        max_iter=qw.spec.max_iter, X=Xs, work=swork)
        afs_ms, (_, ares) = timed(run_afs, 3)
        # the exact sweep of every candidate is the comparison; above n = 8192
        # it would take minutes at 1001 candidates and is left out
        full_ms = timed(run_full, full_reps)[0] if nq * n ** 3 <= 1001 * 8192 ** 3 else None
        msolve.profile_reset()
        msolve.profile_enable(True)
        run_afs()
        torch.cuda.synchronize()
        msolve.profile_enable(False)
        pcnt, pms, pbytes = msolve.profile_query(msolve.KERNEL_NAMES.index("afs_project"))
        msolve.profile_reset()
        xa, xs = Xa.cpu().numpy(), Xs.cpu().numpy()
        ferr = (max(float(np.abs(xa[f] - xs[f]).max() / np.abs(xs[f]).max()) for f in range(nq))
                if full_ms is not None else None)
        prate = pbytes / (pms * 1e-3) / 1e9 if pcnt else None
        return {"workload": qw.spec.name, "candidates": nq, "max_exact": cap, "tol": 1e-4,
                "exact_solves": len(ares.exact), "exact": ares.exact, "basis_size": ares.q,
                "max_estimate": float(ares.estimate.max()),
                "afs_ms": round(afs_ms, 3),
                "exact_sweep_ms": round(full_ms, 3) if full_ms is not None else None,
                "speedup_vs_exact_sweep": round(full_ms / afs_ms, 3) if full_ms is not None else None,
                "max_forward_error_vs_exact_sweep": ferr,
                "project_kernel": None if not pcnt else {
                    "launches": pcnt, "avg_launch_us": round(1000.0 * pms / pcnt, 3),
                    "bytes_per_launch": pbytes / pcnt, "achieved": round(prate, 1),
                    "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(prate / PEAK_HBM_GBS, 4),
                    "traffic": measured_traffic("n%d_quasistatic" % n, "afs_project")}}

    afs = None
    if not args.no_afs:
        afs = [measure_afs(41, 41, 3), measure_afs(1001, 64, 1)]
    def measure_fallback_solve():
        # the direct solve a failed frequency gets: Z of the workload's first
        # frequency, one right-hand side; the host solver beside it up to n = 4096
        Zf, _, _ = msolve.assemble(L, P, g, float(wl.omega[0]), complex(wl.zs[0]), want=("z128",))
        Bf = dev(wl.B[:1])
        gwork = msolve.workspace(msolve.gepp_workspace_bytes(n))
        Xf = torch.empty((1, n), dtype=torch.complex128, device="cuda")
        run = lambda: msolve.gepp_solve_c128(Zf, Bf, X=Xf, work=gwork)
        dev_ms = timed(run, 3)[0]
        msolve.profile_reset()
        msolve.profile_enable(True)
        run()
        torch.cuda.synchronize()
        msolve.profile_enable(False)
        ucnt, ums, uflop = msolve.profile_query(msolve.KERNEL_NAMES.index("gepp_update"))
        msolve.profile_reset()
        host_ms, herr = None, None
        if n <= 4096:
            Zh, Bh = Zf.cpu().numpy(), wl.B[:1].astype(np.complex128)
            t1 = time.perf_counter()
            Xh = msolve.host_solve_c128(Zh, Bh)
            host_ms = 1000.0 * (time.perf_counter() - t1)
            xd = Xf.cpu().numpy()
            herr = float(np.abs(xd - Xh).max() / np.abs(Xh).max())
        urate = uflop / (ums * 1e-3) / 1e12 if ucnt else None
        return {"kind": "complex128 LU with partial pivoting and substitution on the device "
                        "(msolve_gepp_solve_c128)",
                "n": n, "nrhs": 1, "device_ms": round(dev_ms, 3),
                "host_ms": round(host_ms, 3) if host_ms is not None else None,
                "speedup_vs_host": round(host_ms / dev_ms, 3) if host_ms is not None else None,
                "max_difference_vs_host": herr,
                "tflops": round(8.0 * n ** 3 / 3.0 / (dev_ms * 1e-3) / 1e12, 3),
                "update_kernel": None if not ucnt else {
                    "launches": ucnt, "avg_launch_us": round(1000.0 * ums / ucnt, 3),
                    "flop_per_launch": uflop / ucnt, "achieved": round(urate, 3),
                    "peak": PEAK_FP64_VALU_TFLOPS, "unit": "TFLOP/s", "bound": "alu",
                    "frac": round(urate / PEAK_FP64_VALU_TFLOPS, 4)}}

    fallback_solve = None if args.no_fallback_solve else measure_fallback_solve()
    acc["iters_max"] = max(f.iters_max for f in finfo)
    acc["fallbacks"] = int(sum(f.fallback for f in finfo))

    out = {
        "metric": METRIC,
        "value": round(value, 3) if not invalid else None,
        "unit": "solves/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "c64+c128",
        "data": "synthetic",
        "config": {"workload": spec.name, "n": n, "nfreq": nfreq, "nrhs": nrhs,
                   "omega": [float(wl.omega[0]), float(wl.omega[-1])], "tol": spec.tol,
                   "max_iter": spec.max_iter, "frequencies_per_batch": batch,
                   "parallelism": "single-gpu"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "invalid": invalid or None,
        "measured_value": round(value, 3),
        "mean_ms_per_step": round(1000.0 * wall / args.steps, 3),
        "step_ms": [round(1000.0 * t, 3) for t in step_s],
        "lu": {"kind": "general unpivoted LU of one batch (msolve_factor_c64_batch)",
               "tflops": round(lu_tflops, 3),
               "frac_fp32_mfma_peak": round(lu_tflops / PEAK_FP32_MFMA_TFLOPS, 4),
               "flop_per_matrix": 8.0 * n ** 3 / 3.0, "factor_wall_ms": round(lu_ms, 4),
               "kernel_ms_sum": round(lu_kernel_ms, 4),
               "tflops_over_kernel_sum": round(8.0 * n ** 3 / 3.0 * batch / (lu_kernel_ms * 1e-3) / 1e12, 3),
               "n": n, "matrices": batch, "pivots_ok": lu_pivots_ok},
        "lu_single_matrix": lu_large,
        "sweep_factorisation": {"kind": "symmetric" if sym else "general LU",
                                "tflops": round(fact_tflops, 3) if fact_tflops else None,
                                "frac_fp32_mfma_peak": (round(fact_tflops / PEAK_FP32_MFMA_TFLOPS, 4)
                                                        if fact_tflops else None),
                                "flop_per_matrix": fact_flop,
                                "factor_wall_ms_per_sweep": round(fact_wall_ms, 4)},
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in kernels.items()},
        "copy_bandwidth": copy_bw,
        "residual_gemv": gemv,
        "reduced_order_sweep": afs,
        "fallback_direct_solve": fallback_solve,
        "accuracy": acc,
        "gpu_event_ms_per_step": round(gpu_ms / args.steps, 3),
        "profiled_ms_per_step": round(1000.0 * wall_prof / args.steps, 3),
    }
    print(json.dumps(out), flush=True)

    if args.copy_calibration > 0:
        nbytes = args.copy_calibration << 20
        src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print("copy calibration: %d bytes read, %d bytes written" % (nbytes, nbytes), file=sys.stderr)


if __name__ == "__main__":
    main()
