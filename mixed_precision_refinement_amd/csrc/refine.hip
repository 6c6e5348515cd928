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
// then the stop test with the normwise backward error
//   eta = ||r||_inf / (||Z||_inf ||x||_inf + ||b||_inf).
// A right-hand side whose eta is not finite, rises while above tol, or stays
// above tol after max_iter passes sends the whole frequency to the host
// complex128 LU with partial pivoting.
//
// The loop runs on a batch of systems at once (a sweep's frequencies, or a
// single system): every launch covers the batch.  The stop test runs on the
// device after each residual; it drops systems that have converged or been
// handed to the fallback from the active mask that every later launch
// reads, and counts the systems still refining.  The host reads that count
// one pass behind, while the next pass already runs, so the device never
// waits for the host between passes; a pass queued after the last system
// has stopped finds the mask empty and does nothing.
#include <algorithm>
#include <chrono>
#include <cmath>
#include <limits>
#include <mutex>
#include <string>
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

// Operands of the refinement of nf systems of order n: system f uses
// Z128 + f sZ, zrow + f sRow, B + f sB, X + f sX (doubles; sB = 0 shares
// the right-hand sides), LU + f sLU, Dinv + f sD (floats), pivot_info + f.
// With a model (model != NULL) the matrices are not stored: the residuals
// form Z from the model, Z128 is one spare slot into which a frequency that
// falls back is assembled, and zrow is required.
struct RefineBatch {
    int64_t n, nrhs, nf;
    double *Z128;
    int64_t sZ;
    const ZModel *model;
    const double *zrow;
    int64_t sRow;
    const float *LU;
    int64_t sLU;
    const float *Dinv;
    int64_t sD;
    const double *B;
    int64_t sB;
    double *X;
    int64_t sX;
    const int32_t *pivot_info;   // device, nullable
    // The direct solve of a frequency that falls back.  With a model, Z128 is
    // the spare slot the frequency is assembled into, and the solve factors
    // it in place with fb_aux (gepp_aux_bytes) for pivots and candidates.
    // Without one, Z128 is the caller's and is not written: fb_work (nullable)
    // holds gepp_workspace_bytes(n) for a factor copy on the device, else the
    // solve runs on the host.
    void *fb_aux;
    void *fb_work;
    // nullable: the factors are the symmetric factorisation's (msolve_sweep
    // with a model); a frequency that does not converge with them is
    // assembled, factorised with LU and refined again before any host
    // fallback
    const struct LuRetry *retry;
    // start from the X given instead of 0 (a first residual is formed before
    // the first pass)
    bool warm;
    // nullable: a stream for the set-up that needs no factor (norms of b and
    // Z, buffers), which starts after prep_after (the assembly) and so runs
    // beside the factorisation
    hipStream_t prep;
    hipEvent_t prep_after;
};

struct LuRetry {
    float *Z64;         // the factors' slots (rb.LU, writable), stride sZ64
    int64_t sZ64;
    float *Dinv;        // stride sD
    int64_t sD;
    int32_t *dinfo;     // pivot reports
    uint32_t *fflags;   // the factorisation's workspace
    hipStream_t sla;    // look-ahead stream (nullable)
};

// Per right-hand side state of the loop (device).
struct RhsState {
    double eta, eta_first, prev;
    double dprev;     // ||d|| of the previous pass (0 before the first)
    double fwd_est;   // estimated relative forward error of x after this pass
    int32_t iters, pad;
};
static_assert(sizeof(RhsState) == kRhsStateBytes, "state layout");

struct RefineBuffers {
    RefineLayout lay;
    double *R;
    float *Y, *D;
    uint64_t *norms;
    uint32_t *cnt_fwd, *cnt_bwd;
    uint32_t *active, *fate, *poll;   // nf, nf, 4 (two pass slots of {live, timed out})
    int32_t *piv;                     // nf: copy of the pivot reports
    RhsState *st;
    uint64_t *err;
};

RefineBuffers carve(int64_t n, int64_t nrhs, int64_t nf, char *work)
{
    RefineBuffers b;
    b.lay = refine_layout(n, nrhs, nf);
    b.R = reinterpret_cast<double *>(work + b.lay.r128);
    b.Y = reinterpret_cast<float *>(work + b.lay.y64);
    b.D = reinterpret_cast<float *>(work + b.lay.d64);
    b.norms = reinterpret_cast<uint64_t *>(work + b.lay.norms);
    b.cnt_fwd = reinterpret_cast<uint32_t *>(work + b.lay.tickets);
    b.cnt_bwd = b.cnt_fwd + 1;
    b.active = reinterpret_cast<uint32_t *>(work + b.lay.active);
    b.fate = b.active + nf;
    b.poll = b.fate + nf;
    b.piv = reinterpret_cast<int32_t *>(b.poll + 4);
    b.st = reinterpret_cast<RhsState *>(work + b.lay.state);
    b.err = b.norms + norm_slot_err(nrhs);   // system 0's slot, shared by the batch
    return b;
}

// d = U^-1 L^-1 fl32(r) for every right-hand side of every active system, in
// groups of four; X += d when X is not NULL.  r is complex128 (r128, system
// stride sR doubles) or complex64 (r64, stride sR floats), rows of n.
int solve_corrections(const RefineBatch &rb, const double *r128, const float *r64, int64_t sR,
                      double *X, RefineBuffers &b, const uint32_t *active, hipStream_t s)
{
    const int64_t n = rb.n, npad = b.lay.npad;
    for (int64_t k0 = 0; k0 < rb.nrhs; k0 += kRhsPerLaunch) {
        const int64_t nr = std::min<int64_t>(kRhsPerLaunch, rb.nrhs - k0);
        const double *r128k = r128 ? r128 + size_t(k0) * size_t(n) * 2 : nullptr;
        const float *r64k = r64 ? r64 + size_t(k0) * size_t(n) * 2 : nullptr;
        float *Yk = b.Y + size_t(k0) * size_t(npad) * 2;
        float *Dk = b.D + size_t(k0) * size_t(npad) * 2;
        double *Xk = X ? X + size_t(k0) * size_t(n) * 2 : nullptr;
        TrsvBatch fw;
        fw.nf = rb.nf; fw.sLU = rb.sLU; fw.sD = rb.sD; fw.sSrc = sR; fw.sOut = b.lay.yd_stride;
        fw.sX = 0; fw.active = active;
        MS_TRY(launch_trsv_fwd(n, nr, fw, rb.LU, rb.Dinv, r128k, r64k, Yk, Dk, b.cnt_fwd, b.err, s));
        TrsvBatch bw = fw;
        bw.sSrc = b.lay.yd_stride;
        bw.sX = rb.sX;
        bw.dnorm = X ? b.norms + norm_slot_d(rb.nrhs, k0) : nullptr;
        bw.sN = b.lay.norm_stride;
        MS_TRY(launch_trsv_bwd(n, nr, bw, rb.LU, rb.Dinv, Yk, Dk, Xk, b.cnt_bwd, b.err, s));
    }
    return MSOLVE_OK;
}

// r = b - Z x and the norms of r and x for every active system
int residuals(const RefineBatch &rb, RefineBuffers &b, hipStream_t s)
{
    ResidualBatch rsb;
    rsb.nf = rb.nf; rsb.sZ = rb.sZ; rsb.sB = rb.sB; rsb.sX = rb.sX; rsb.sR = b.lay.r_stride;
    rsb.sN = b.lay.norm_stride; rsb.active = b.active;
    uint64_t *rn = b.norms + norm_slot_r(0), *xn = b.norms + norm_slot_x(rb.nrhs, 0);
    if (rb.model)
        return launch_residual_model(rb.n, rb.nrhs, *rb.model, rsb, rb.B, rb.X, b.R, rn, xn, s);
    return launch_residual(rb.n, rb.nrhs, rsb, rb.Z128, rb.B, rb.X, b.R, rn, xn, s);
}

// the start of a sequence of solves: zero ticket counters, y and d pending
int reset_solves(RefineBuffers &b, hipStream_t s)
{
    MS_TRY(launch_fill_u32(b.cnt_fwd, 2, 0u, s));
    const size_t words = 2 * (b.lay.d64 - b.lay.y64) / sizeof(uint32_t);   // y then d
    return launch_fill_u32(reinterpret_cast<uint32_t *>(b.Y), words, kTrsvPendingWord, s);
}

// ------------------------------------------------ device stop test

__device__ inline double as_double(uint64_t b) { return __longlong_as_double(static_cast<long long>(b)); }

static_assert(kMaxBatch <= 64, "the stop test gives each system one lane of a wave");

// Start of the loop for nf <= 64 systems (one wave, lane f = system f):
// every norm slot zeroed, the per right-hand side state reset, and the
// systems whose factorisation met a bad pivot (or all, when max_iter is 0)
// handed to the fallback at once.
// parts: 1 clears the norm slots and states, 2 reads the pivot reports
// (which the factorisation must have written)
__global__ __launch_bounds__(64) void refine_init_kernel(int64_t nf, int64_t nrhs, int32_t max_iter,
                                                         const int32_t *pivot_info, uint64_t *norms,
                                                         int64_t sN, uint32_t *active, uint32_t *fate,
                                                         int32_t *piv, RhsState *st, int parts)
{
    const int f = threadIdx.x;
    if (parts & 1) {
        for (int64_t i = f; i < nf * sN; i += 64) norms[i] = 0;
        for (int64_t i = f; i < nf * nrhs; i += 64) {
            const double inf = __builtin_inf();
            st[i] = RhsState{inf, inf, inf, 0.0, inf, 0, 0};
        }
    }
    if ((parts & 2) && f < nf) {
        piv[f] = pivot_info ? pivot_info[f] : 0;
        const bool ok = piv[f] == 0 && max_iter > 0;
        fate[f] = ok ? 0u : 2u;
        active[f] = ok ? 1u : 0u;
    }
}

// zero the residual and solution norm slots of every system (lane f = system f)
__global__ __launch_bounds__(64) void clear_rx_kernel(int64_t nf, int64_t nrhs, uint64_t *norms, int64_t sN)
{
    const int f = threadIdx.x;
    if (f >= nf) return;
    for (int64_t k = 0; k < nrhs; ++k) {
        norms[size_t(f) * size_t(sN) + norm_slot_r(k)] = 0;
        norms[size_t(f) * size_t(sN) + norm_slot_x(nrhs, k)] = 0;
        norms[size_t(f) * size_t(sN) + norm_slot_d(nrhs, k)] = 0;
    }
}

// The stop test after the residual of pass `it`, for every active system:
// eta_k = ||r_k|| / (||Z|| ||x_k|| + ||b_k||) (each operation rounded on its
// own), and an estimate of the relative forward error of x_k from the sizes
// of the last two corrections: with rho = ||d_it|| / ||d_it-1|| (the
// contraction of the iteration), ||x - x_k|| ~ min(rho, 1) ||d_it||.  The
// first correction is not used as a denominator (it is x_1 itself, and its
// ratio to the next says little about the later contraction), so the
// estimate needs three passes.  The system converges when every
// eta_k <= tol and every estimate <= fwd_tol ||x_k||; it goes to the fallback
// when some eta_k is not finite, or rises while above tol, or when it has not
// converged at the last pass.  The residual, solution and correction norm
// slots are cleared for the next pass.  poll[0] = systems still refining, poll[1] = 1 after a
// triangular-solve wait time-out (which stops every system).
__global__ __launch_bounds__(64) void refine_check_kernel(int64_t nf, int64_t nrhs, int32_t it,
                                                          int32_t max_iter, double tol, double fwd_tol,
                                                          uint64_t *norms, int64_t sN, const uint64_t *err,
                                                          uint32_t *active, uint32_t *fate,
                                                          RhsState *st, uint32_t *poll)
{
#pragma clang fp contract(off)
    const int f = threadIdx.x;
    const bool timed_out = *err != 0;
    bool live = false;
    if (f < nf && active[f] != 0) {
        uint64_t *nm = norms + size_t(f) * size_t(sN);
        const double zn = as_double(nm[norm_slot_z(nrhs)]);
        bool all_done = true, give_up = false, fwd_wait = false;
        for (int64_t k = 0; k < nrhs; ++k) {
            const double rn = as_double(nm[norm_slot_r(k)]);
            const double xn = as_double(nm[norm_slot_x(nrhs, k)]);
            const double bn = as_double(nm[norm_slot_b(nrhs, k)]);
            const double dn = as_double(nm[norm_slot_d(nrhs, k)]);
            const double eta = rn / (zn * xn + bn);
            RhsState &r = st[size_t(f) * size_t(nrhs) + size_t(k)];
            // rho is +inf in the first two passes (dprev = 0), NaN only when
            // both corrections are 0, and then the estimate is 0
            const double est = fmin(dn / r.dprev, 1.0) * dn;
            r.iters = it;
            r.eta = eta;
            r.fwd_est = est / xn;
            r.dprev = it >= 2 ? dn : 0.0;
            if (it == 1) r.eta_first = eta;
            if (!isfinite(eta)) {
                give_up = true;
            } else if (!(eta <= tol)) {
                all_done = false;
                if (eta > r.prev) give_up = true;
            } else if (!(est <= fwd_tol * xn)) {
                fwd_wait = true;
            }
            r.prev = eta;
            nm[norm_slot_r(k)] = 0;
            nm[norm_slot_x(nrhs, k)] = 0;
            nm[norm_slot_d(nrhs, k)] = 0;
        }
        if (timed_out) {
            active[f] = 0;
        } else if (all_done && !give_up && !fwd_wait) {
            fate[f] = 1;
            active[f] = 0;
        } else if (give_up || it == max_iter) {
            fate[f] = 2;
            active[f] = 0;
        } else {
            live = true;
        }
    }
    const uint64_t mask = __ballot(live);
    if (f == 0) {
        poll[0] = uint32_t(__popcll(mask));
        poll[1] = timed_out ? 1u : 0u;
    }
}

// The direct solve of a frequency whose refinement failed: complex128 LU
// with partial pivoting on the device, in the buffers the caller's workspace
// provides (see RefineBatch), else on the host.  No device memory is
// allocated here.
int host_fallback(int64_t n, int64_t nrhs, const double *Z128, const double *B, double *X,
                  hipStream_t s);

int direct_fallback(const RefineBatch &rb, double *Zf, const double *B, double *X, hipStream_t s)
{
    if (rb.model && rb.fb_aux) return device_gepp_solve_inplace(rb.n, rb.nrhs, Zf, B, X, rb.fb_aux, s);
    if (rb.fb_work) return device_gepp_solve(rb.n, rb.nrhs, Zf, B, X, rb.fb_work, s);
    return host_fallback(rb.n, rb.nrhs, Zf, B, X, s);
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

// The refinement loop of a batch.  info: host, nf * nrhs entries (system
// major); piv_host (nullable): host, nf pivot reports.  When the
// factorisation of a system met a zero or non-finite pivot its factors are
// unusable and the loop skips it in favour of the fallback.
int refine_batch(const RefineBatch &rb, double tol, int32_t max_iter, char *work,
                 msolve_rhs_info *info, int32_t *piv_host, hipStream_t s)
{
    const int64_t n = rb.n, nrhs = rb.nrhs, nf = rb.nf;
    RefineBuffers b = carve(n, nrhs, nf, work);
    const int64_t ns = b.lay.norm_stride;

    // the set-up that needs no factor: on rb.prep after rb.prep_after when
    // given (beside the factorisation), else on s
    hipStream_t ps = rb.prep ? rb.prep : s;
    if (rb.prep) MS_HIP(hipStreamWaitEvent(ps, rb.prep_after, 0));
    MS_TRY(reset_solves(b, ps));
    if (!rb.warm) MS_TRY(launch_fill_f64_batch(rb.X, size_t(2) * size_t(n) * size_t(nrhs), rb.sX, nf, 0.0, ps));
    hipLaunchKernelGGL(refine_init_kernel, dim3(1), dim3(64), 0, ps, nf, nrhs, max_iter,
                       rb.pivot_info, b.norms, ns, b.active, b.fate, b.piv, b.st, 1);
    MS_HIP(hipGetLastError());
    MS_TRY(launch_vec_norms(n, nrhs, nf, rb.B, rb.sB, b.norms + norm_slot_b(nrhs, 0), ns, ps));
    if (rb.zrow) {
        MS_TRY(launch_max_reduce(n, nf, rb.zrow, rb.sRow, b.norms + norm_slot_z(nrhs), ns, ps));
    } else {
        for (int64_t f = 0; f < nf; ++f) {
            double *scratch = b.R + size_t(f) * size_t(b.lay.r_stride);   // n doubles
            MS_TRY(launch_row_abs_sums(n, rb.Z128 + size_t(f) * size_t(rb.sZ), scratch, ps));
        }
        MS_TRY(launch_max_reduce(n, nf, b.R, b.lay.r_stride, b.norms + norm_slot_z(nrhs), ns, ps));
    }
    if (rb.prep) {
        hipEvent_t ready = nullptr;
        MS_HIP(hipEventCreateWithFlags(&ready, hipEventDisableTiming));
        const hipError_t e1 = hipEventRecord(ready, ps);
        const hipError_t e2 = e1 == hipSuccess ? hipStreamWaitEvent(s, ready, 0) : e1;
        (void)hipEventDestroy(ready);
        MS_HIP(e2);
    }
    // the pivot reports, once the factorisation has written them
    hipLaunchKernelGGL(refine_init_kernel, dim3(1), dim3(64), 0, s, nf, nrhs, max_iter,
                       rb.pivot_info, b.norms, ns, b.active, b.fate, b.piv, b.st, 2);
    MS_HIP(hipGetLastError());
    if (rb.warm) {
        // r = b - Z x for the first pass; its norms are not needed
        MS_TRY(residuals(rb, b, s));
        hipLaunchKernelGGL(clear_rx_kernel, dim3(1), dim3(64), 0, s, nf, nrhs, b.norms, ns);
        MS_HIP(hipGetLastError());
    }

    // passes, the host one pass behind: after queueing pass it it reads the
    // count of pass it - 1 (on the poll stream, which waits only for that
    // pass's stop test) and stops queueing once nothing is left to refine
    hipStream_t sp = nullptr;
    MS_TRY(poll_stream(&sp));
    hipEvent_t ev[2] = {nullptr, nullptr};
    // timing registry: the work of a pass's launches is scaled to the
    // systems active in it once the host knows their number
    std::vector<int64_t> tags;
    auto loop = [&]() -> int {
        for (auto &e : ev) MS_HIP(hipEventCreateWithFlags(&e, hipEventDisableTiming));
        for (int32_t it = 1; it <= max_iter; ++it) {
            tags.push_back(prof_new_tag());
            prof_set_tag(tags.back());
            // it == 1 from x = 0: r = b; otherwise r is the last residual
            int st = it == 1 && !rb.warm
                         ? solve_corrections(rb, rb.B, nullptr, rb.sB, rb.X, b, b.active, s)
                         : solve_corrections(rb, b.R, nullptr, b.lay.r_stride, rb.X, b, b.active, s);
            if (st == MSOLVE_OK) st = residuals(rb, b, s);
            prof_set_tag(0);
            MS_TRY(st);
            hipLaunchKernelGGL(refine_check_kernel, dim3(1), dim3(64), 0, s, nf, nrhs, it, max_iter,
                               tol, MSOLVE_FWD_TOL, b.norms, ns, b.err, b.active, b.fate, b.st, b.poll + 2 * (it & 1));
            MS_HIP(hipGetLastError());
            MS_HIP(hipEventRecord(ev[it & 1], s));
            if (it == 1) continue;
            uint32_t pw[2] = {0, 0};
            MS_HIP(hipStreamWaitEvent(sp, ev[(it - 1) & 1], 0));
            MS_HIP(hipMemcpyAsync(pw, b.poll + 2 * ((it - 1) & 1), sizeof(pw), hipMemcpyDeviceToHost, sp));
            MS_HIP(hipStreamSynchronize(sp));
            prof_scale_tag(tags.back(), double(pw[0]) / double(nf));
            if (pw[1] != 0) break;
            if (pw[0] == 0) break;
        }
        return MSOLVE_OK;
    };
    const int lst = loop();
    for (auto &e : ev)
        if (e) (void)hipEventDestroy(e);
    MS_TRY(lst);

    // the outcome of every system and right-hand side: norms, masks, pivot
    // reports and states in one copy
    const size_t span = b.lay.state + kRhsStateBytes * size_t(nf) * size_t(nrhs) - b.lay.norms;
    std::vector<uint64_t> rep((span + 7) / 8);
    MS_HIP(hipMemcpyAsync(rep.data(), b.norms, span, hipMemcpyDeviceToHost, s));
    MS_HIP(hipStreamSynchronize(s));
    const char *base = reinterpret_cast<const char *>(rep.data());
    const auto at = [&](void *dev) { return base + (static_cast<char *>(dev) - reinterpret_cast<char *>(b.norms)); };
    std::vector<uint64_t> h(reinterpret_cast<const uint64_t *>(base),
                            reinterpret_cast<const uint64_t *>(base) + size_t(ns * nf));
    const uint32_t *fate = reinterpret_cast<const uint32_t *>(at(b.fate));
    const int32_t *piv = reinterpret_cast<const int32_t *>(at(b.piv));
    const RhsState *st = reinterpret_cast<const RhsState *>(at(b.st));
    if (h[norm_slot_err(nrhs)] != 0)
        return fail(MSOLVE_E_DEVICE, "refinement: triangular solve wait timed out");
    if (piv_host) std::copy(piv, piv + nf, piv_host);
    if (!tags.empty())
        prof_scale_tag(tags.front(), double(std::count(piv, piv + nf, 0)) / double(nf));
    std::vector<double> znorm(static_cast<size_t>(nf)), bnorm(static_cast<size_t>(nf * nrhs));
    for (int64_t f = 0; f < nf; ++f) {
        const uint64_t *hf = h.data() + size_t(f * ns);
        znorm[size_t(f)] = bits_to_double(hf[norm_slot_z(nrhs)]);
        for (int64_t k = 0; k < nrhs; ++k) {
            bnorm[size_t(f * nrhs + k)] = bits_to_double(hf[norm_slot_b(nrhs, k)]);
            const RhsState &r = st[size_t(f * nrhs + k)];
            info[f * nrhs + k] = msolve_rhs_info{r.iters, 0, 0, 0, r.eta, r.eta_first, r.fwd_est};
        }
    }

    // A frequency that did not converge with the symmetric factors (and
    // whose factorisation met no bad pivot) is factorised again with LU --
    // the page's fallback from LDL^T to LU (section "Measure first: the
    // ceiling of JavaScript") -- and refined again on its own, with its own
    // host fallback.  Its info then describes that second refinement.  (The
    // nested call reuses the start of the workspace; every value still
    // needed here was copied to the host above.)
    std::vector<uint8_t> retried(static_cast<size_t>(nf), 0);
    if (rb.retry && rb.model) {
        const LuRetry &lr = *rb.retry;
        const ZModel &m = *rb.model;
        for (int64_t f = 0; f < nf; ++f) {
            if (fate[f] == 1u || piv[f] != 0) continue;
            float *z64 = lr.Z64 + size_t(f) * size_t(lr.sZ64);
            float *dv = lr.Dinv + size_t(f) * size_t(lr.sD);
            int32_t *di = lr.dinfo + f;
            MS_TRY(launch_assemble(n, 1, m.w + f, m.zr + f, m.zi + f, m.L, m.Psi, m.g, nullptr, 0, z64, 0,
                                   nullptr, 0, s));
            MS_TRY(launch_factor(n, 1, z64, 0, dv, 0, di, false, lr.fflags, s, lr.sla));
            const ZModel m1{m.L, m.Psi, m.g, m.w + f, m.zr + f, m.zi + f};
            RefineBatch r1 = rb;
            r1.nf = 1;
            r1.model = &m1;
            r1.zrow = rb.zrow + size_t(f) * size_t(rb.sRow);
            r1.LU = z64;
            r1.Dinv = dv;
            r1.B = rb.B + size_t(f) * size_t(rb.sB);
            r1.X = rb.X + size_t(f) * size_t(rb.sX);
            r1.pivot_info = di;
            r1.retry = nullptr;
            r1.prep = nullptr;
            // a frequency that met the backward-error bar and failed only the
            // forward-error estimate continues from its answer; otherwise the
            // second refinement starts again from x = 0
            r1.warm = true;
            for (int64_t k = 0; k < nrhs; ++k) r1.warm = r1.warm && st[size_t(f * nrhs + k)].eta <= tol;
            int32_t p1 = 0;
            const int st1 = refine_batch(r1, tol, max_iter, work, info + f * nrhs, &p1, s);
            if (st1 != MSOLVE_OK && st1 != MSOLVE_E_FALLBACK) return st1;
            if (piv_host) piv_host[f] = p1;
            retried[size_t(f)] = 1;
        }
    }

    // per-frequency fallback: complex128 direct solve, then the backward
    // error of the fallback answers
    int status = MSOLVE_OK;
    std::vector<uint32_t> fb(static_cast<size_t>(nf), 0);
    bool any_fb = false;
    for (int64_t f = 0; f < nf; ++f) {
        if (retried[size_t(f)]) {
            for (int64_t k = 0; k < nrhs; ++k)
                if (info[f * nrhs + k].status != MSOLVE_OK && status == MSOLVE_OK) status = info[f * nrhs + k].status;
            continue;
        }
        const bool conv = fate[f] == 1u;
        for (int64_t k = 0; k < nrhs; ++k) info[f * nrhs + k].converged = conv ? 1 : 0;
        if (conv) continue;
        double *zf = rb.Z128 + size_t(f) * size_t(rb.sZ);
        if (rb.model) {
            const ZModel &m = *rb.model;
            MS_TRY(launch_assemble(n, 1, m.w + f, m.zr + f, m.zi + f, m.L, m.Psi, m.g, rb.Z128, 0,
                                   nullptr, 0, nullptr, 0, s));
            zf = rb.Z128;
        }
        double *xf = rb.X + size_t(f) * size_t(rb.sX);
        const int st = direct_fallback(rb, zf, rb.B + size_t(f) * size_t(rb.sB), xf, s);
        // a frequency the direct solve finds singular has no answer: its
        // solutions are set to NaN rather than left half permuted
        if (st == MSOLVE_E_FALLBACK)
            MS_TRY(launch_fill_f64(xf, size_t(2) * size_t(n) * size_t(nrhs), __builtin_nan(""), s));
        for (int64_t k = 0; k < nrhs; ++k) {
            info[f * nrhs + k].fallback = 1;
            info[f * nrhs + k].status = st;
            info[f * nrhs + k].fwd_est = __builtin_nan("");
        }
        if (st == MSOLVE_OK) {
            fb[size_t(f)] = 1;
            any_fb = true;
        } else if (status == MSOLVE_OK) {
            status = st;
        }
    }
    if (!any_fb) return status;
    MS_HIP(hipMemcpyAsync(b.active, fb.data(), sizeof(uint32_t) * fb.size(), hipMemcpyHostToDevice, s));
    hipLaunchKernelGGL(clear_rx_kernel, dim3(1), dim3(64), 0, s, nf, nrhs, b.norms, ns);
    MS_HIP(hipGetLastError());
    const int64_t ftag = prof_new_tag();
    prof_set_tag(ftag);
    const int rst = residuals(rb, b, s);
    prof_set_tag(0);
    MS_TRY(rst);
    prof_scale_tag(ftag, double(std::count(fb.begin(), fb.end(), 1u)) / double(nf));
    MS_HIP(hipMemcpyAsync(h.data(), b.norms, sizeof(uint64_t) * h.size(), hipMemcpyDeviceToHost, s));
    MS_HIP(hipStreamSynchronize(s));
    for (int64_t f = 0; f < nf; ++f) {
        if (!fb[size_t(f)]) continue;
        const uint64_t *hf = h.data() + size_t(f * ns);
        for (int64_t k = 0; k < nrhs; ++k) {
            const double rn = bits_to_double(hf[norm_slot_r(k)]);
            const double xn = bits_to_double(hf[norm_slot_x(nrhs, k)]);
            info[f * nrhs + k].eta = rn / (znorm[size_t(f)] * xn + bnorm[size_t(f * nrhs + k)]);
        }
    }
    return status;
}

}  // namespace
}  // namespace msolve

using namespace msolve;

namespace msolve {
namespace {
// steps 2 and 4 with the refinement workspace at `work`
int lu_solve_in(int64_t n, int64_t nrhs, const float *LU, const float *Dinv, float *RHS, char *work,
                hipStream_t s)
{
    RefineBuffers b = carve(n, nrhs, 1, work);
    MS_TRY(reset_solves(b, s));
    MS_TRY(launch_fill_u32(reinterpret_cast<uint32_t *>(b.err), 2, 0u, s));
    RefineBatch rb{};
    rb.n = n; rb.nrhs = nrhs; rb.nf = 1; rb.LU = LU; rb.Dinv = Dinv;
    MS_TRY(solve_corrections(rb, nullptr, RHS, 0, nullptr, b, nullptr, s));
    return launch_copy_c64_rows(n, nrhs, b.D, b.lay.npad, RHS, n, s);
}

// The scratch of msolve_lu_solve_c64_noalloc: a fixed array on every device
// the library runs on, held until the process ends.  Its name is only a
// host-side handle: host code uses the device address that
// hipGetSymbolAddress returns for the current device (noalloc_scratch).
constexpr size_t kNoAllocScratchBytes = size_t(8) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

// the device address of `scratch` on the current device, looked up once per
// device
int noalloc_scratch(char **out)
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static char *addr[kMaxDevices] = {};
    int dev = 0;
    MS_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) return fail(MSOLVE_E_ARG, "msolve_lu_solve_c64_noalloc: device index out of range");
    std::lock_guard<std::mutex> g(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        MS_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        if (!p) return fail(MSOLVE_E_HIP, "msolve_lu_solve_c64_noalloc: no device address for the scratch array");
        addr[dev] = static_cast<char *>(p);
    }
    *out = addr[dev];
    return MSOLVE_OK;
}
}  // namespace
}  // namespace msolve

extern "C" int msolve_lu_solve_c64(int64_t n, int64_t nrhs, const float *LU, const float *Dinv,
                                   float *RHS, void *work, size_t work_bytes, void *stream)
{
    if (n < 1 || nrhs < 1) return fail(MSOLVE_E_ARG, "msolve_lu_solve_c64: n and nrhs must be >= 1");
    if (!LU || !Dinv || !RHS || !work) return fail(MSOLVE_E_ARG, "msolve_lu_solve_c64: null pointer");
    if (work_bytes < msolve_refine_workspace_bytes(n, nrhs))
        return fail(MSOLVE_E_WORKSPACE, "msolve_lu_solve_c64: workspace too small");
    return lu_solve_in(n, nrhs, LU, Dinv, RHS, static_cast<char *>(work), static_cast<hipStream_t>(stream));
}

extern "C" size_t msolve_lu_solve_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

extern "C" int msolve_lu_solve_c64_noalloc(int64_t n, int64_t nrhs, const float *LU, const float *Dinv,
                                           float *RHS, void *stream)
{
    if (n < 1 || nrhs < 1) return fail(MSOLVE_E_ARG, "msolve_lu_solve_c64_noalloc: n and nrhs must be >= 1");
    if (!LU || !Dinv || !RHS) return fail(MSOLVE_E_ARG, "msolve_lu_solve_c64_noalloc: null pointer");
    const size_t need = msolve_refine_workspace_bytes(n, nrhs);
    if (need > kNoAllocScratchBytes)
        return fail(MSOLVE_E_WORKSPACE, "msolve_lu_solve_c64_noalloc: n = " + std::to_string(n) + " with " +
                                            std::to_string(nrhs) + " right-hand sides needs " +
                                            std::to_string(need) + " bytes of scratch, more than the " +
                                            std::to_string(kNoAllocScratchBytes) + " the library holds");
    char *ptr = nullptr;
    MS_TRY(noalloc_scratch(&ptr));
    return lu_solve_in(n, nrhs, LU, Dinv, RHS, ptr, static_cast<hipStream_t>(stream));
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
    RefineBatch rb{};
    rb.n = n; rb.nrhs = nrhs; rb.nf = 1;
    rb.Z128 = const_cast<double *>(Z128); rb.zrow = zrowabs; rb.LU = LU; rb.Dinv = Dinv; rb.B = B; rb.X = X;
    // a workspace that also holds the device direct solve's buffers gets the
    // fallback on the device; otherwise it runs on the host
    const size_t rbytes = align256(msolve_refine_workspace_bytes(n, nrhs));
    if (work_bytes >= rbytes + gepp_workspace_bytes(n)) rb.fb_work = static_cast<char *>(work) + rbytes;
    return refine_batch(rb, tol, max_iter, static_cast<char *>(work), info, nullptr,
                        static_cast<hipStream_t>(stream));
}

// The sweep: equal batches of at most msolve_sweep_batch frequencies, each
// assembled, factorised and refined with launches that cover the batch, on
// the caller's stream (plus the look-ahead stream for the factorisation).
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
    if (nfreq == 0) return MSOLVE_OK;
    if (work_bytes < msolve_sweep_workspace_bytes(n, nrhs, nfreq))
        return fail(MSOLVE_E_WORKSPACE, "msolve_sweep: workspace too small");
    hipStream_t s = static_cast<hipStream_t>(stream);
    char *w = static_cast<char *>(work);
    const int64_t nb = msolve_sweep_batch(n, nrhs, nfreq);
    const int64_t nbatch = (nfreq + nb - 1) / nb;
    // with more than one batch, batch b + 1 is assembled and factorised (on
    // the front stream, into the other set of per-frequency arrays) while
    // batch b is refined on s
    const int64_t sets = nbatch > 1 ? 2 : 1;
    const SweepLayout lay = sweep_layout(n, nrhs, nb, sets);
    double *Z128 = reinterpret_cast<double *>(w + lay.z128);
    void *gepp_aux = w + lay.gepp_aux;
    struct Set {
        float *Z64, *Dinv;
        double *zrow;
        int32_t *dinfo;
        uint32_t *fflags;
        std::vector<double> zr, zi;
        hipEvent_t ev[3];
    };
    Set set[2];
    for (int64_t k = 0; k < sets; ++k) {
        char *base = w + size_t(k) * lay.set_bytes;
        set[k].Z64 = reinterpret_cast<float *>(base + lay.z64);
        set[k].Dinv = reinterpret_cast<float *>(base + lay.dinv);
        set[k].zrow = reinterpret_cast<double *>(base + lay.zrow);
        set[k].dinfo = reinterpret_cast<int32_t *>(base + lay.info);
        set[k].fflags = reinterpret_cast<uint32_t *>(base + lay.fflags);
        set[k].zr.assign(static_cast<size_t>(nb), 0.0);
        set[k].zi.assign(static_cast<size_t>(nb), 0.0);
        for (auto &e : set[k].ev) e = nullptr;
    }

    hipStream_t sla = nullptr, sf = s;
    int status = MSOLVE_OK;
    auto body = [&]() -> int {
        if (nblocks(n) >= 12) MS_TRY(lookahead_stream(&sla));
        MS_TRY(front_stream(&sf));
        for (int64_t k = 0; k < sets; ++k)
            for (auto &e : set[k].ev) MS_HIP(hipEventCreate(&e));
        std::vector<msolve_rhs_info> ri(static_cast<size_t>(nb * nrhs));
        std::vector<int32_t> piv(static_cast<size_t>(nb));
        // Z(w) is complex symmetric when L and Psi are symmetric (G is
        // diagonal), and then the factorisation uses the symmetry (the
        // pivot-report words hold the check's flag until the first one)
        // (the check's flag lives in a word the first factorisation's pivot
        // reports overwrite, and the first assembly runs while the host
        // waits for it)
        uint32_t asym = 0;
        uint32_t *flag = reinterpret_cast<uint32_t *>(set[0].dinfo);
        MS_TRY(launch_fill_u32(flag, 1, 0u, s));
        MS_TRY(launch_sym_check(n, L, Psi, flag, s));
        bool sym = false;
        // batch b's assembly, then its factorisation, into its set on stream fs.
        // The symmetric factorisation reads only the lower triangle and
        // writes U over the upper one, so that triangle is not assembled:
        // the first batch's assembly reads the check's word on the device
        // (the host learns it only afterwards), the later ones know `sym`.
        int64_t asm_tag = 0;
        auto assemble_batch = [&](int64_t b, hipStream_t fs) -> int {
            Set &S = set[b % sets];
            const int64_t f0 = b * nb, nf = std::min<int64_t>(nb, nfreq - f0);
            for (int64_t f = 0; f < nf; ++f) {
                S.zr[size_t(f)] = zs[2 * (f0 + f)];
                S.zi[size_t(f)] = zs[2 * (f0 + f) + 1];
            }
            MS_HIP(hipEventRecord(S.ev[0], fs));
            if (b == 0) {
                asm_tag = prof_new_tag();
                prof_set_tag(asm_tag);
            }
            const int st = launch_assemble(n, nf, omega + f0, S.zr.data(), S.zi.data(), L, Psi, g, nullptr, 0,
                                           S.Z64, lay.z64_stride, S.zrow, lay.zrow_stride, fs, b > 0 && sym,
                                           b == 0 ? flag : nullptr);
            prof_set_tag(0);
            MS_TRY(st);
            MS_HIP(hipEventRecord(S.ev[1], fs));
            return MSOLVE_OK;
        };
        auto factor_batch = [&](int64_t b, hipStream_t fs) -> int {
            Set &S = set[b % sets];
            const int64_t nf = std::min<int64_t>(nb, nfreq - b * nb);
            MS_TRY(launch_factor(n, nf, S.Z64, lay.z64_stride, S.Dinv, lay.dinv_stride, S.dinfo, sym, S.fflags,
                                 fs, sla));
            MS_HIP(hipEventRecord(S.ev[2], fs));
            return MSOLVE_OK;
        };
        auto front = [&](int64_t b, hipStream_t fs) -> int {
            MS_TRY(assemble_batch(b, fs));
            return factor_batch(b, fs);
        };
        // the first batch's assembly is queued behind the check, and the
        // flag is copied on the poll stream, which waits for the check only
        {
            hipStream_t sp = nullptr;
            MS_TRY(poll_stream(&sp));
            hipEvent_t checked = nullptr;
            MS_HIP(hipEventCreateWithFlags(&checked, hipEventDisableTiming));
            auto copy_flag = [&]() -> int {
                MS_HIP(hipEventRecord(checked, s));
                MS_TRY(assemble_batch(0, s));
                MS_HIP(hipStreamWaitEvent(sp, checked, 0));
                MS_HIP(hipMemcpyAsync(&asym, flag, sizeof(asym), hipMemcpyDeviceToHost, sp));
                MS_HIP(hipStreamSynchronize(sp));
                return MSOLVE_OK;
            };
            const int st0 = copy_flag();
            (void)hipEventDestroy(checked);
            MS_TRY(st0);
        }
        sym = asym == 0;
        if (sym) {
            // the first assembly wrote the lower triangles only
            const double nn = double(n) * double(n), nfb = double(std::min<int64_t>(nb, nfreq));
            const double full = 16.0 * nn + (8.0 * nn + 8.0 * double(n)) * nfb + 8.0 * double(n);
            const double low = 16.0 * nn + (4.0 * double(n) * double(n + 1) + 8.0 * double(n)) * nfb + 8.0 * double(n);
            prof_scale_tag(asm_tag, low / full);
        }
        MS_TRY(factor_batch(0, s));
        for (int64_t b = 0; b < nbatch; ++b) {
            Set &S = set[b % sets];
            const int64_t f0 = b * nb, nf = std::min<int64_t>(nb, nfreq - f0);
            // the next batch's front goes ahead on its own stream (its set
            // was last used by batch b - 1, whose refinement has finished)
            if (b + 1 < nbatch) {
                MS_HIP(hipStreamWaitEvent(sf, S.ev[2], 0));
                MS_TRY(front(b + 1, sf));
            }
            if (b > 0) MS_HIP(hipStreamWaitEvent(s, S.ev[2], 0));
            const ZModel model{L, Psi, g, omega + f0, S.zr.data(), S.zi.data()};
            RefineBatch rb{};
            rb.n = n; rb.nrhs = nrhs; rb.nf = nf;
            rb.Z128 = Z128; rb.sZ = 0; rb.model = &model;
            rb.zrow = S.zrow; rb.sRow = lay.zrow_stride;
            rb.LU = S.Z64; rb.sLU = lay.z64_stride;
            rb.Dinv = S.Dinv; rb.sD = lay.dinv_stride;
            rb.B = B; rb.sB = 0;
            rb.X = X + size_t(f0) * size_t(nrhs) * size_t(n) * 2;
            rb.sX = nrhs * n * 2;
            rb.pivot_info = S.dinfo;
            rb.fb_aux = gepp_aux;
            const LuRetry retry{S.Z64, lay.z64_stride, S.Dinv, lay.dinv_stride, S.dinfo, S.fflags, sla};
            rb.retry = sym ? &retry : nullptr;
            if (nbatch == 1) {
                // the refinement's set-up runs on the (otherwise idle) front
                // stream beside the factorisation
                rb.prep = sf;
                rb.prep_after = S.ev[1];
            }
            const auto t0 = std::chrono::steady_clock::now();
            const int st = refine_batch(rb, tol, max_iter, w + lay.refine, ri.data(), piv.data(), s);
            const auto t1 = std::chrono::steady_clock::now();
            if (st != MSOLVE_OK && st != MSOLVE_E_FALLBACK) return st;
            // a singular frequency does not stop the sweep: the later batches
            // still run, and the first such status is returned at the end
            if (st != MSOLVE_OK && status == MSOLVE_OK) status = st;
            float ta = 0.0f, tf = 0.0f;
            MS_HIP(hipEventElapsedTime(&ta, S.ev[0], S.ev[1]));
            MS_HIP(hipEventElapsedTime(&tf, S.ev[1], S.ev[2]));
            const double trf = std::chrono::duration<double, std::milli>(t1 - t0).count();
            for (int64_t f = 0; f < nf; ++f) {
                msolve_freq_info &fi = finfo[f0 + f];
                fi = msolve_freq_info{0, 0, 0, 0, 0.0, 0.0, 0.0, 0.0};
                fi.t_assemble_ms = ta;
                fi.t_factor_ms = tf;
                fi.t_refine_ms = trf;
                fi.pivot_info = piv[size_t(f)];
                for (int64_t r = 0; r < nrhs; ++r) {
                    const msolve_rhs_info &x = ri[size_t(f * nrhs + r)];
                    fi.iters_max = std::max(fi.iters_max, x.iters);
                    fi.fallback |= x.fallback;
                    fi.eta_max = std::max(fi.eta_max, x.eta);
                    if (x.status != MSOLVE_OK) fi.status = x.status;
                    if (rinfo) rinfo[size_t(f0 + f) * size_t(nrhs) + size_t(r)] = x;
                }
            }
        }
        return status;
    };
    const int rc = body();
    // an error may leave the front stream's work queued: finish it before
    // the workspace is handed back
    if (sf != s) (void)hipStreamSynchronize(sf);
    for (int64_t k = 0; k < sets; ++k)
        for (auto &e : set[k].ev)
            if (e) (void)hipEventDestroy(e);
    return rc;
}
