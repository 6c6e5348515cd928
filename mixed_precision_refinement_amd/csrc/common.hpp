// Internal helpers shared by the msolve HIP sources (not part of the C-ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <string>

#include "msolve.h"

namespace msolve {

// ---------------------------------------------------------------- errors

void set_error(const std::string &msg);
int fail(int status, const std::string &msg);
int hip_fail(hipError_t e, const char *what);

#define MS_HIP(call)                                   \
    do {                                               \
        hipError_t e_ = (call);                        \
        if (e_ != hipSuccess) return ::msolve::hip_fail(e_, #call); \
    } while (0)

#define MS_TRY(call)                                   \
    do {                                               \
        int s_ = (call);                               \
        if (s_ != MSOLVE_OK) return s_;                \
    } while (0)

// ------------------------------------------------------------ constants

// Block size of the factorisation and of the triangular solves that use its
// inverted diagonal blocks.
constexpr int kNB = 64;

inline int64_t nblocks(int64_t n) { return (n + kNB - 1) / kNB; }
inline int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }
inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// ------------------------------------------------------------ workspace

// Layout of the refinement workspace (offsets in bytes from `work`).
struct RefineLayout {
    size_t r128;      // complex128 nrhs x n: current residual
    size_t y64;       // complex64 nrhs x npad: forward-solve result
    size_t d64;       // complex64 nrhs x npad: correction
    size_t norms;     // uint64 slots: rnorm[nrhs], xnorm[nrhs], bnorm[nrhs], znorm, err
    size_t flags;     // uint32 fwd[nb] then bwd[nb] ready flags, 2 counters
    size_t total;
    int64_t npad;
    int64_t nblk;
};
RefineLayout refine_layout(int64_t n, int64_t nrhs);

// The sweep runs sweep_workers(n) frequencies at once (one host thread and
// stream per worker); each worker owns one slot.
constexpr int kMaxWorkers = 4;
inline int sweep_workers(int64_t n) { return n <= 4096 ? 4 : 2; }

struct SweepSlot {
    size_t z128;      // complex128 n x n
    size_t z64;       // complex64 n x n (factorised in place)
    size_t dinv;      // msolve_dinv_floats(n) floats
    size_t zrow;      // n doubles
    size_t info;      // int32 pivot info
    size_t refine;    // RefineLayout region
};
struct SweepLayout {
    int workers;
    SweepSlot slot[kMaxWorkers];
    size_t total;
};
SweepLayout sweep_layout(int64_t n, int64_t nrhs);

// slots inside the norms region
inline size_t norm_slot_r(int64_t k) { return size_t(k); }
inline size_t norm_slot_x(int64_t nrhs, int64_t k) { return size_t(nrhs + k); }
inline size_t norm_slot_b(int64_t nrhs, int64_t k) { return size_t(2 * nrhs + k); }
inline size_t norm_slot_z(int64_t nrhs) { return size_t(3 * nrhs); }
inline size_t norm_slot_err(int64_t nrhs) { return size_t(3 * nrhs + 1); }
inline size_t norm_slots(int64_t nrhs) { return size_t(3 * nrhs + 2); }

// --------------------------------------------------------------- timing

// Event-bracketed launches for the timing registry; no-ops when disabled.
struct ProfScope {
    int kernel;
    hipStream_t stream;
    double work;
    void *ev0;
    ProfScope(int k, hipStream_t s, double w);
    ~ProfScope();
};

// ------------------------------------------------------------- launchers
// (each returns MSOLVE_OK or a negative status; asynchronous on `s`)

int launch_assemble(int64_t n, double w, double zr, double zi, const double *L,
                    const double *Psi, const double *g, double *Z128, float *Z64,
                    double *zrowabs, hipStream_t s);

int launch_factor(int64_t n, float *A, float *Dinv, int32_t *d_info, hipStream_t s,
                  hipStream_t sla = nullptr);

// forward solve L y = fl32(r) (r complex128 or complex64) and back solve
// U d = y, optionally X += d (complex128).  `epoch` must be fresh per launch
// for the flags region (flags zeroed at the start of each sequence).
int launch_trsv_fwd(int64_t n, int64_t nrhs, const float *LU, const float *Dinv,
                    const double *r128, const float *r64, float *y, uint32_t *flags,
                    uint32_t *counter, uint32_t epoch, uint64_t *err, hipStream_t s);
int launch_trsv_bwd(int64_t n, int64_t nrhs, const float *LU, const float *Dinv,
                    const float *y, float *d, double *X128, uint32_t *flags,
                    uint32_t *counter, uint32_t epoch, uint64_t *err, hipStream_t s);

int launch_residual(int64_t n, int64_t nrhs, const double *Z, const double *B,
                    const double *X, double *R, uint64_t *rnorm_bits,
                    uint64_t *xnorm_bits, hipStream_t s);

// small vector kernels
int launch_fill_u32(uint32_t *p, size_t count, uint32_t v, hipStream_t s);
int launch_fill_f64(double *p, size_t count, double v, hipStream_t s);
int launch_copy_c64_rows(int64_t n, int64_t nrhs, const float *src, int64_t ld_src, float *dst,
                         int64_t ld_dst, hipStream_t s);
int launch_vec_norms(int64_t n, int64_t nrhs, const double *B, uint64_t *out_bits,
                     hipStream_t s);
int launch_max_reduce(int64_t n, const double *v, uint64_t *out_bits, hipStream_t s);
int launch_row_abs_sums(int64_t n, const double *Z128, double *out, hipStream_t s);

// host fallback (complex128 GEPP); returns MSOLVE_OK or MSOLVE_E_FALLBACK
int host_gepp_solve(int64_t n, int64_t nrhs, const double *Z, const double *B, double *X);

}  // namespace msolve
