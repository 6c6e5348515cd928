// Mixed-precision iterative refinement (the four-step list of the section
// "Double-precision answers from a GPU without double precision", page
// "Solving Dense Matrices Fast in the Browser"), the per-frequency fallback
// to a direct solve (paragraph after that list), and the frequency sweep.
//
// The loop starts from x0 = 0, r0 = b, so its first pass is step 2 (solve
// with the single-precision factors) and every later pass is steps 3-4:
//   d = U^-1 L^-1 fl32(r)   (two persistent triangular-solve launches, the
//                            second also adds d to x in complex128)
//   r = b - Z x             (complex128 residual, norms folded in)
// then the stop test on the host with the normwise backward error
//   eta = ||r||_inf / (||Z||_inf ||x||_inf + ||b||_inf).
// A right-hand side whose eta is not finite, rises while above tol, or stays
// above tol after max_iter passes sends the whole frequency to the host
// complex128 LU with partial pivoting.
#include <algorithm>
#include <atomic>
#include <chrono>
#include <mutex>
#include <string>
#include <thread>
#include <cmath>
#include <limits>
#include <vector>

#include "common.hpp"

namespace msolve {
namespace {

constexpr int kRhsPerLaunch = 4;

double bits_to_double(uint64_t b)
{
    double d;
    static_assert(sizeof(d) == sizeof(b), "size");
    __builtin_memcpy(&d, &b, sizeof(d));
    return d;
}

struct RefineBuffers {
    RefineLayout lay;
    double *R;
    float *Y, *D;
    uint64_t *norms;
    uint32_t *flags_fwd, *flags_bwd, *cnt_fwd, *cnt_bwd;
    uint64_t *err;
};

RefineBuffers carve(int64_t n, int64_t nrhs, char *work)
{
    RefineBuffers b;
    b.lay = refine_layout(n, nrhs);
    b.R = reinterpret_cast<double *>(work + b.lay.r128);
    b.Y = reinterpret_cast<float *>(work + b.lay.y64);
    b.D = reinterpret_cast<float *>(work + b.lay.d64);
    b.norms = reinterpret_cast<uint64_t *>(work + b.lay.norms);
    uint32_t *f = reinterpret_cast<uint32_t *>(work + b.lay.flags);
    b.flags_fwd = f;
    b.flags_bwd = f + b.lay.nblk;
    b.cnt_fwd = f + 2 * b.lay.nblk;
    b.cnt_bwd = b.cnt_fwd + 1;
    b.err = b.norms + norm_slot_err(nrhs);
    return b;
}

// d = U^-1 L^-1 fl32(r) for every right-hand side, in groups of four; X += d
// when X is not NULL.  r is complex128 (r128) or complex64 (r64), rows of n.
int solve_corrections(int64_t n, int64_t nrhs, const float *LU, const float *Dinv,
                      const double *r128, const float *r64, double *X, RefineBuffers &b,
                      uint32_t &epoch, hipStream_t s)
{
    const int64_t npad = b.lay.npad;
    for (int64_t k0 = 0; k0 < nrhs; k0 += kRhsPerLaunch) {
        const int64_t nr = std::min<int64_t>(kRhsPerLaunch, nrhs - k0);
        ++epoch;
        const double *r128k = r128 ? r128 + size_t(k0) * size_t(n) * 2 : nullptr;
        const float *r64k = r64 ? r64 + size_t(k0) * size_t(n) * 2 : nullptr;
        float *Yk = b.Y + size_t(k0) * size_t(npad) * 2;
        float *Dk = b.D + size_t(k0) * size_t(npad) * 2;
        double *Xk = X ? X + size_t(k0) * size_t(n) * 2 : nullptr;
        MS_TRY(launch_trsv_fwd(n, nr, LU, Dinv, r128k, r64k, Yk, b.flags_fwd, b.cnt_fwd, epoch,
                               b.err, s));
        MS_TRY(launch_trsv_bwd(n, nr, LU, Dinv, Yk, Dk, Xk, b.flags_bwd, b.cnt_bwd, epoch, b.err,
                               s));
    }
    return MSOLVE_OK;
}

int reset_flags(RefineBuffers &b, hipStream_t s)
{
    return launch_fill_u32(b.flags_fwd, size_t(2 * b.lay.nblk + 2), 0u, s);
}

int host_fallback(int64_t n, int64_t nrhs, const double *Z128, const double *B, double *X,
                  hipStream_t s)
{
    std::vector<double> hz(size_t(2) * size_t(n) * size_t(n));
    std::vector<double> hb(size_t(2) * size_t(n) * size_t(nrhs)), hx(hb.size());
    MS_HIP(hipMemcpyAsync(hz.data(), Z128, sizeof(double) * hz.size(), hipMemcpyDeviceToHost, s));
    MS_HIP(hipMemcpyAsync(hb.data(), B, sizeof(double) * hb.size(), hipMemcpyDeviceToHost, s));
    MS_HIP(hipStreamSynchronize(s));
    const int st = host_gepp_solve(n, nrhs, hz.data(), hb.data(), hx.data());
    if (st != MSOLVE_OK) return fail(st, "fallback direct solve: matrix is singular");
    MS_HIP(hipMemcpyAsync(X, hx.data(), sizeof(double) * hx.size(), hipMemcpyHostToDevice, s));
    MS_HIP(hipStreamSynchronize(s));
    return MSOLVE_OK;
}

}  // namespace

// The refinement loop.  pivot_info (device, nullable): when the factorisation
// met a zero or non-finite pivot the factors are unusable and the loop is
// skipped in favour of the fallback.
int refine_impl(int64_t n, int64_t nrhs, const double *Z128, const double *zrowabs,
                const float *LU, const float *Dinv, const double *B, double *X, double tol,
                int32_t max_iter, char *work, msolve_rhs_info *info, const int32_t *pivot_info,
                int32_t *pivot_info_host, hipStream_t s)
{
    RefineBuffers b = carve(n, nrhs, work);
    const size_t nslots = norm_slots(nrhs);
    std::vector<uint64_t> h(nslots, 0);

    MS_TRY(reset_flags(b, s));
    MS_TRY(launch_fill_u32(reinterpret_cast<uint32_t *>(b.norms), 2 * nslots, 0u, s));
    MS_TRY(launch_fill_f64(X, size_t(2) * size_t(n) * size_t(nrhs), 0.0, s));
    MS_TRY(launch_vec_norms(n, nrhs, B, b.norms + norm_slot_b(nrhs, 0), s));
    if (zrowabs) {
        MS_TRY(launch_max_reduce(n, zrowabs, b.norms + norm_slot_z(nrhs), s));
    } else {
        MS_TRY(launch_row_abs_sums(n, Z128, b.R, s));   // R as n-double scratch
        MS_TRY(launch_max_reduce(n, b.R, b.norms + norm_slot_z(nrhs), s));
    }
    int32_t piv = 0;
    if (pivot_info)
        MS_HIP(hipMemcpyAsync(&piv, pivot_info, sizeof(piv), hipMemcpyDeviceToHost, s));
    MS_HIP(hipMemcpyAsync(h.data(), b.norms, sizeof(uint64_t) * nslots, hipMemcpyDeviceToHost, s));
    MS_HIP(hipStreamSynchronize(s));
    if (pivot_info_host) *pivot_info_host = piv;
    const double znorm = bits_to_double(h[norm_slot_z(nrhs)]);
    std::vector<double> bnorm(nrhs), prev(nrhs, std::numeric_limits<double>::infinity());
    for (int64_t k = 0; k < nrhs; ++k) {
        bnorm[size_t(k)] = bits_to_double(h[norm_slot_b(nrhs, k)]);
        info[k] = msolve_rhs_info{0, 0, 0, 0, std::numeric_limits<double>::infinity(),
                                  std::numeric_limits<double>::infinity()};
    }

    bool converged = false;
    uint32_t epoch = 0;
    for (int32_t it = 1; it <= max_iter && piv == 0; ++it) {
        // it == 1: r = b (x = 0); afterwards r is the last residual
        MS_TRY(solve_corrections(n, nrhs, LU, Dinv, it == 1 ? B : b.R, nullptr, X, b, epoch, s));
        MS_TRY(launch_fill_u32(reinterpret_cast<uint32_t *>(b.norms), size_t(4 * nrhs), 0u, s));
        MS_TRY(launch_residual(n, nrhs, Z128, B, X, b.R, b.norms + norm_slot_r(0),
                               b.norms + norm_slot_x(nrhs, 0), s));
        MS_HIP(hipMemcpyAsync(h.data(), b.norms, sizeof(uint64_t) * nslots, hipMemcpyDeviceToHost, s));
        MS_HIP(hipStreamSynchronize(s));
        if (h[norm_slot_err(nrhs)] != 0)
            return fail(MSOLVE_E_DEVICE, "msolve_refine: triangular solve wait timed out");
        bool all_done = true, give_up = false;
        for (int64_t k = 0; k < nrhs; ++k) {
            const double rn = bits_to_double(h[norm_slot_r(k)]);
            const double xn = bits_to_double(h[norm_slot_x(nrhs, k)]);
            const double eta = rn / (znorm * xn + bnorm[size_t(k)]);
            msolve_rhs_info &in = info[k];
            in.iters = it;
            in.eta = eta;
            if (it == 1) in.eta_first = eta;
            if (!std::isfinite(eta)) {
                give_up = true;
            } else if (!(eta <= tol)) {
                all_done = false;
                if (eta > prev[size_t(k)]) give_up = true;
            }
            prev[size_t(k)] = eta;
        }
        if (all_done && !give_up) {
            converged = true;
            break;
        }
        if (give_up) break;
    }
    for (int64_t k = 0; k < nrhs; ++k) info[k].converged = converged ? 1 : 0;
    if (converged) return MSOLVE_OK;

    // per-frequency fallback: direct solve on the host
    const int st = host_fallback(n, nrhs, Z128, B, X, s);
    for (int64_t k = 0; k < nrhs; ++k) {
        info[k].fallback = 1;
        info[k].status = st;
    }
    if (st != MSOLVE_OK) return st;
    // report the backward error of the fallback answer
    MS_TRY(launch_fill_u32(reinterpret_cast<uint32_t *>(b.norms), size_t(4 * nrhs), 0u, s));
    MS_TRY(launch_residual(n, nrhs, Z128, B, X, b.R, b.norms + norm_slot_r(0),
                           b.norms + norm_slot_x(nrhs, 0), s));
    MS_HIP(hipMemcpyAsync(h.data(), b.norms, sizeof(uint64_t) * nslots, hipMemcpyDeviceToHost, s));
    MS_HIP(hipStreamSynchronize(s));
    for (int64_t k = 0; k < nrhs; ++k) {
        const double rn = bits_to_double(h[norm_slot_r(k)]);
        const double xn = bits_to_double(h[norm_slot_x(nrhs, k)]);
        info[k].eta = rn / (znorm * xn + bnorm[size_t(k)]);
    }
    return MSOLVE_OK;
}

}  // namespace msolve

using namespace msolve;

extern "C" int msolve_lu_solve_c64(int64_t n, int64_t nrhs, const float *LU, const float *Dinv,
                                   float *RHS, void *work, size_t work_bytes, void *stream)
{
    if (n < 1 || nrhs < 1) return fail(MSOLVE_E_ARG, "msolve_lu_solve_c64: n and nrhs must be >= 1");
    if (!LU || !Dinv || !RHS || !work) return fail(MSOLVE_E_ARG, "msolve_lu_solve_c64: null pointer");
    if (work_bytes < msolve_refine_workspace_bytes(n, nrhs))
        return fail(MSOLVE_E_WORKSPACE, "msolve_lu_solve_c64: workspace too small");
    hipStream_t s = static_cast<hipStream_t>(stream);
    RefineBuffers b = carve(n, nrhs, static_cast<char *>(work));
    MS_TRY(reset_flags(b, s));
    MS_TRY(launch_fill_u32(reinterpret_cast<uint32_t *>(b.err), 2, 0u, s));
    uint32_t epoch = 0;
    MS_TRY(solve_corrections(n, nrhs, LU, Dinv, nullptr, RHS, nullptr, b, epoch, s));
    return launch_copy_c64_rows(n, nrhs, b.D, b.lay.npad, RHS, n, s);
}

extern "C" int msolve_refine(int64_t n, int64_t nrhs, const double *Z128, const double *zrowabs,
                             const float *LU, const float *Dinv, const double *B, double *X,
                             double tol, int32_t max_iter, void *work, size_t work_bytes,
                             msolve_rhs_info *info, void *stream)
{
    if (n < 1 || nrhs < 1) return fail(MSOLVE_E_ARG, "msolve_refine: n and nrhs must be >= 1");
    if (!Z128 || !LU || !Dinv || !B || !X || !work || !info)
        return fail(MSOLVE_E_ARG, "msolve_refine: null pointer");
    if (!(tol >= 0.0) || max_iter < 0) return fail(MSOLVE_E_ARG, "msolve_refine: tol >= 0 and max_iter >= 0 required");
    if (work_bytes < msolve_refine_workspace_bytes(n, nrhs))
        return fail(MSOLVE_E_WORKSPACE, "msolve_refine: workspace too small");
    return refine_impl(n, nrhs, Z128, zrowabs, LU, Dinv, B, X, tol, max_iter,
                       static_cast<char *>(work), info, nullptr, nullptr,
                       static_cast<hipStream_t>(stream));
}

extern "C" int msolve_sweep(int64_t n, int64_t nfreq, const double *omega, const double *zs,
                            const double *L, const double *Psi, const double *g, int64_t nrhs,
                            const double *B, double *X, double tol, int32_t max_iter, void *work,
                            size_t work_bytes, msolve_freq_info *finfo, msolve_rhs_info *rinfo,
                            void *stream)
{
    if (n < 1 || nrhs < 1 || nfreq < 0) return fail(MSOLVE_E_ARG, "msolve_sweep: bad sizes");
    if (!omega || !zs || !L || !Psi || !g || !B || !X || !work || !finfo)
        return fail(MSOLVE_E_ARG, "msolve_sweep: null pointer");
    if (!(tol >= 0.0) || max_iter < 0) return fail(MSOLVE_E_ARG, "msolve_sweep: tol >= 0 and max_iter >= 0 required");
    for (int64_t f = 0; f < nfreq; ++f)
        if (!std::isfinite(omega[f]) || omega[f] == 0.0)
            return fail(MSOLVE_E_ARG, "msolve_sweep: every omega must be finite and nonzero");
    if (work_bytes < msolve_sweep_workspace_bytes(n, nrhs))
        return fail(MSOLVE_E_WORKSPACE, "msolve_sweep: workspace too small");
    hipStream_t s = static_cast<hipStream_t>(stream);
    char *w = static_cast<char *>(work);
    const SweepLayout lay = sweep_layout(n, nrhs);
    const int nw = int(std::min<int64_t>(lay.workers, std::max<int64_t>(nfreq, 1)));
    int device = 0;
    MS_HIP(hipGetDevice(&device));
    // the workers' streams start after the caller's stream has written the inputs
    hipEvent_t in_ready = nullptr;
    MS_HIP(hipEventCreateWithFlags(&in_ready, hipEventDisableTiming));
    if (hipEventRecord(in_ready, s) != hipSuccess) {
        (void)hipEventDestroy(in_ready);
        return fail(MSOLVE_E_HIP, "msolve_sweep: hipEventRecord failed");
    }

    std::atomic<int64_t> next{0};
    std::atomic<int> first_status{MSOLVE_OK};
    std::mutex err_mu;
    std::string err_msg;

    // Worker p: its own stream (default priority) and slot; frequencies are
    // taken from a shared counter.  Each frequency is assembled, factorised
    // and refined in order on the worker's stream (the refinement blocks on
    // its own stream only), so up to nw frequencies are in flight at once.
    auto worker = [&](int p) {
        auto record_failure = [&](int st) {
            int expect = MSOLVE_OK;
            if (first_status.compare_exchange_strong(expect, st)) {
                std::lock_guard<std::mutex> g(err_mu);
                err_msg = msolve_last_error();
            }
        };
        if (hipSetDevice(device) != hipSuccess) {
            set_error("msolve_sweep: hipSetDevice failed in a worker");
            record_failure(MSOLVE_E_HIP);
            return;
        }
        hipStream_t ws = nullptr, wla = nullptr;
        hipEvent_t ev[3] = {nullptr, nullptr, nullptr};
        bool ok = hipStreamCreateWithFlags(&ws, hipStreamNonBlocking) == hipSuccess;
        // large n: a look-ahead stream for the factorisation (the bulk
        // trailing update is long enough to hide the diagonal steps)
        if (ok && n > 4096) ok = hipStreamCreateWithFlags(&wla, hipStreamNonBlocking) == hipSuccess;
        for (auto &e : ev) ok = ok && hipEventCreate(&e) == hipSuccess;
        ok = ok && hipStreamWaitEvent(ws, in_ready, 0) == hipSuccess;
        if (!ok) {
            set_error("msolve_sweep: stream or event creation failed in a worker");
            record_failure(MSOLVE_E_HIP);
        }
        const SweepSlot &sl = lay.slot[p];
        double *Z128 = reinterpret_cast<double *>(w + sl.z128);
        float *Z64 = reinterpret_cast<float *>(w + sl.z64);
        float *Dinv = reinterpret_cast<float *>(w + sl.dinv);
        double *zrow = reinterpret_cast<double *>(w + sl.zrow);
        int32_t *dinfo = reinterpret_cast<int32_t *>(w + sl.info);
        std::vector<msolve_rhs_info> ri(nrhs);
        while (ok && first_status.load() == MSOLVE_OK) {
            const int64_t f = next.fetch_add(1);
            if (f >= nfreq) break;
            msolve_freq_info &fi = finfo[f];
            fi = msolve_freq_info{0, 0, 0, 0, 0.0, 0.0, 0.0, 0.0};
            int st = MSOLVE_OK;
            if (hipEventRecord(ev[0], ws) != hipSuccess) st = hip_fail(hipErrorUnknown, "hipEventRecord");
            if (st == MSOLVE_OK)
                st = launch_assemble(n, omega[f], zs[2 * f], zs[2 * f + 1], L, Psi, g, Z128, Z64,
                                     zrow, ws);
            if (st == MSOLVE_OK && hipEventRecord(ev[1], ws) != hipSuccess)
                st = hip_fail(hipErrorUnknown, "hipEventRecord");
            if (st == MSOLVE_OK) st = launch_factor(n, Z64, Dinv, dinfo, ws, wla);
            if (st == MSOLVE_OK && hipEventRecord(ev[2], ws) != hipSuccess)
                st = hip_fail(hipErrorUnknown, "hipEventRecord");
            const auto t0 = std::chrono::steady_clock::now();
            int32_t piv = 0;
            if (st == MSOLVE_OK)
                st = refine_impl(n, nrhs, Z128, zrow, Z64, Dinv, B,
                                 X + size_t(f) * size_t(nrhs) * size_t(n) * 2, tol, max_iter,
                                 w + sl.refine, ri.data(), dinfo, &piv, ws);
            const auto t1 = std::chrono::steady_clock::now();
            float ta = 0.0f, tf = 0.0f;
            (void)hipEventElapsedTime(&ta, ev[0], ev[1]);
            (void)hipEventElapsedTime(&tf, ev[1], ev[2]);
            fi.t_assemble_ms = ta;
            fi.t_factor_ms = tf;
            fi.t_refine_ms = std::chrono::duration<double, std::milli>(t1 - t0).count();
            fi.pivot_info = piv;
            fi.status = st;
            for (int64_t r = 0; r < nrhs; ++r) {
                fi.iters_max = std::max(fi.iters_max, ri[size_t(r)].iters);
                fi.fallback |= ri[size_t(r)].fallback;
                fi.eta_max = std::max(fi.eta_max, ri[size_t(r)].eta);
                if (rinfo) rinfo[size_t(f) * size_t(nrhs) + size_t(r)] = ri[size_t(r)];
            }
            if (st != MSOLVE_OK) record_failure(st);
        }
        if (ws) {
            (void)hipStreamSynchronize(ws);
            (void)hipStreamDestroy(ws);
        }
        if (wla) {
            (void)hipStreamSynchronize(wla);
            (void)hipStreamDestroy(wla);
        }
        for (auto &e : ev)
            if (e) (void)hipEventDestroy(e);
    };

    std::vector<std::thread> pool;
    for (int p = 1; p < nw; ++p) pool.emplace_back(worker, p);
    worker(0);
    for (auto &t : pool) t.join();
    (void)hipEventDestroy(in_ready);
    const int status = first_status.load();
    if (status != MSOLVE_OK) set_error(err_msg);
    return status;
}
