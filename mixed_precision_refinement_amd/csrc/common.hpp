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

// Batches: a sweep factorises and refines up to kMaxBatch frequencies in
// lockstep, every launch covering the whole batch.
constexpr int64_t kMaxBatch = 32;

// Layout of the refinement workspace for a batch of nf systems (offsets in
// bytes from `work`; per-system regions at constant strides).
struct RefineLayout {
    size_t r128;      // complex128 nrhs x n per system: current residual
    size_t y64;       // complex64 nrhs x npad per system: forward-solve result
    size_t d64;       // complex64 nrhs x npad per system: correction
    size_t norms;     // uint64 norm slots per system (see norm_slot_*)
    size_t tickets;   // uint32: the ticket counters of the forward and back solves
    size_t active;    // uint32: active[nf] (1 while refining), fate[nf], 4 poll words, pivot reports[nf]
    size_t state;     // kRhsStateBytes per system and right-hand side
    size_t total;
    int64_t npad, nblk, nf;
    int64_t r_stride;     // doubles between systems' residuals
    int64_t yd_stride;    // floats between systems' y (and d) vectors
    int64_t norm_stride;  // uint64 slots between systems
};
RefineLayout refine_layout(int64_t n, int64_t nrhs, int64_t nf = 1);
constexpr size_t kRhsStateBytes = 48;   // eta, eta_first, previous eta, previous ||d||, estimate, count

// Systems per batch that the sweep uses for order n (bounded by memory).
int64_t sweep_batch_max(int64_t n, int64_t nrhs);

// Layout of the sweep workspace for batches of nf frequencies.  With two
// sets the per-frequency arrays (and the factorisation's workspace) exist
// twice, so that the next batch is assembled and factorised while the
// current one is refined.
struct SweepLayout {
    int64_t nf, sets;
    size_t z128;           // one complex128 n x n slot for a frequency that falls back
    size_t z64, dinv, zrow, info;   // per-frequency arrays at the strides below (set 0)
    int64_t z128_stride;   // doubles (the slot's size)
    int64_t z64_stride;    // floats
    int64_t dinv_stride;   // floats
    int64_t zrow_stride;   // doubles
    size_t fflags;         // the factorisation's workspace (hand-off words of its diagonal steps)
    size_t set_bytes;      // offset of set 1's arrays from set 0's (z64, dinv, zrow, info, fflags)
    size_t gepp_aux;       // pivots and candidates of the direct solve in the spare slot
    size_t refine;         // RefineLayout for nf systems
    size_t total;
};
SweepLayout sweep_layout(int64_t n, int64_t nrhs, int64_t nf, int64_t sets);

// slots inside one system's norms region
__host__ __device__ inline size_t norm_slot_r(int64_t k) { return size_t(k); }
__host__ __device__ inline size_t norm_slot_x(int64_t nrhs, int64_t k) { return size_t(nrhs + k); }
__host__ __device__ inline size_t norm_slot_b(int64_t nrhs, int64_t k) { return size_t(2 * nrhs + k); }
__host__ __device__ inline size_t norm_slot_z(int64_t nrhs) { return size_t(3 * nrhs); }
__host__ __device__ inline size_t norm_slot_err(int64_t nrhs) { return size_t(3 * nrhs + 1); }
// ||d_k||, the correction the back solve has just added to x_k
__host__ __device__ inline size_t norm_slot_d(int64_t nrhs, int64_t k) { return size_t(3 * nrhs + 2 + k); }
__host__ __device__ inline size_t norm_slots(int64_t nrhs) { return size_t(4 * nrhs + 2); }

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
// Launches recorded while a tag is set carry it; their work can be scaled
// afterwards (a refinement pass learns how many of its systems were active
// only after it was queued).  Tag 0: none.
int64_t prof_new_tag();
void prof_set_tag(int64_t tag);
void prof_scale_tag(int64_t tag, double factor);

// psi / w, rounded to nearest like the division itself (Z, whether
// assembled or formed on the fly by the residual, must be the same bit for
// bit).  With y = 1 / w rounded to nearest, q = psi y is within two
// ulps of the quotient; one correction q + (psi - w q) y, the remainder
// formed exactly by a fused multiply-add, makes it faithful, and a second
// one makes it the rounded quotient (Markstein's theorem for the last step
// of a Newton-Raphson division: y within half an ulp of 1 / w, q faithful).
// The theorem needs every value normal and no overflow: with |w| in
// [2^-64, 2^64] (checked on the host) that holds for |psi| in [2^-900,
// 2^900]; psi = 0 gives psi y (a zero of the quotient's sign), and any
// other psi (tiny, huge, infinite, NaN) takes the division.
__device__ __forceinline__ double psi_over_w(double psi, double w, double y, bool by_inv)
{
#pragma clang fp contract(off)
    const double a = fabs(psi);
    if (by_inv && a >= 0x1p-900 && a <= 0x1p900) {
        double q = psi * y;
        double r = fma(-q, w, psi);
        q = fma(r, y, q);
        r = fma(-q, w, psi);
        return fma(r, y, q);
    }
    if (by_inv && a == 0.0) return psi * y;
    return psi / w;
}

// ------------------------------------------------------------- launchers
// (each returns MSOLVE_OK or a negative status; asynchronous on `s`)

// Z(w_f) for a batch of nf frequencies (w, zr, zi: host arrays of nf);
// frequency f writes Z128 + f sZ128, Z64 + f sZ64, zrowabs + f sRow (any of
// the three outputs may be NULL).  lower: write only the lower triangle
// (j <= i) of Z128 and Z64; sym_flag (device, nullable): the same when
// *sym_flag == 0 at the time the kernel runs (the symmetry check's word).
// zrowabs always covers whole rows.
int launch_assemble(int64_t n, int64_t nf, const double *w, const double *zr, const double *zi,
                    const double *L, const double *Psi, const double *g, double *Z128,
                    int64_t sZ128, float *Z64, int64_t sZ64, double *zrowabs, int64_t sRow,
                    hipStream_t s, bool lower = false, const uint32_t *sym_flag = nullptr);

// *flag |= 1 unless L and Psi (device, n x n) are both exactly symmetric
int launch_sym_check(int64_t n, const double *L, const double *Psi, uint32_t *flag, hipStream_t s);

// Factorisation of nf matrices at A + f sA (floats); Dinv at Dinv + f sD,
// pivot reports at d_info + f.  sym: the matrices are complex symmetric
// (only their entries on and below the diagonal are read).  flags: nf words
// of device scratch for the general diagonal steps (unused when sym).  sla
// (nullable): look-ahead stream for the diagonal and panel steps; s joins it
// at the end.
int launch_factor(int64_t n, int64_t nf, float *A, int64_t sA, float *Dinv, int64_t sD,
                  int32_t *d_info, bool sym, uint32_t *flags, hipStream_t s, hipStream_t sla);
// the look-ahead stream of the current device (created on first use, kept
// for the life of the process)
int lookahead_stream(hipStream_t *out);
// the stream on which the refinement reads its per-pass counts (same life)
int poll_stream(hipStream_t *out);
// the stream on which a sweep assembles and factorises its next batch while
// the current one is refined (created on first use, kept for the process)
int front_stream(hipStream_t *out);

// Strides of a batch of triangular solves (system f: LU + f sLU and
// Dinv + f sD floats, source + f sSrc elements, output + f sOut floats,
// X128 + f sX doubles); `active` (nullable) skips systems whose entry is 0.
struct TrsvBatch {
    int64_t nf = 1;
    int64_t sLU = 0, sD = 0, sSrc = 0, sOut = 0, sX = 0;
    const uint32_t *active = nullptr;
    // back solve with X: nullable, the bits of ||d_k||_inf (modulus; atomic
    // max, so zero beforehand) for right-hand side k at dnorm[f sN + k]
    uint64_t *dnorm = nullptr;
    int64_t sN = 0;
};

// forward solve L y = fl32(r) (r complex128 or complex64) and back solve
// U d = y, optionally X += d (complex128) and ||d||, for up to four right-hand sides
// (y and d: complex64 rows of npad at the batch's sOut stride).  The solves
// hand values between workgroups through y and d themselves: both must hold
// kTrsvPendingWord in every 32-bit word before the first forward solve of a
// sequence; each launch leaves them so for the next (the forward solve resets
// d, the back solve y).  counter: a ticket counter, zero at the first launch
// (each launch leaves it zero).
constexpr uint32_t kTrsvPendingWord = 0xFFFFFFFFu;
int launch_trsv_fwd(int64_t n, int64_t nrhs, const TrsvBatch &tb, const float *LU,
                    const float *Dinv, const double *r128, const float *r64, float *y, float *d,
                    uint32_t *counter, uint64_t *err, hipStream_t s);
int launch_trsv_bwd(int64_t n, int64_t nrhs, const TrsvBatch &tb, const float *LU,
                    const float *Dinv, float *y, float *d, double *X128, uint32_t *counter,
                    uint64_t *err, hipStream_t s);

// Strides of a batch of residuals (doubles; norm slots sN); `active`
// (nullable) skips systems whose entry is 0.
struct ResidualBatch {
    int64_t nf = 1;
    int64_t sZ = 0, sB = 0, sX = 0, sR = 0, sN = 0;
    const uint32_t *active = nullptr;
};
int launch_residual(int64_t n, int64_t nrhs, const ResidualBatch &rb, const double *Z,
                    const double *B, const double *X, double *R, uint64_t *rnorm_bits,
                    uint64_t *xnorm_bits, hipStream_t s);

// The model of a batch's matrices: Z(w_f) = j w_f L - j Psi / w_f + (zr_f +
// j zi_f) diag(g), with w, zr, zi host arrays of the batch's frequencies.
struct ZModel {
    const double *L, *Psi, *g;
    const double *w, *zr, *zi;
};
// the residual of a batch with Z formed on the fly from the model (bit for
// bit the assembled Z, same summation order as launch_residual); rb.sZ is
// not used
int launch_residual_model(int64_t n, int64_t nrhs, const ZModel &zm, const ResidualBatch &rb,
                          const double *B, const double *X, double *R, uint64_t *rnorm_bits,
                          uint64_t *xnorm_bits, hipStream_t s);

// small vector kernels
int launch_fill_u32(uint32_t *p, size_t count, uint32_t v, hipStream_t s);
int launch_fill_f64(double *p, size_t count, double v, hipStream_t s);
// p + f stride, f < nsys: count doubles each set to v (one launch)
int launch_fill_f64_batch(double *p, size_t count, int64_t stride, int64_t nsys, double v,
                          hipStream_t s);
int launch_copy_c64_rows(int64_t n, int64_t nrhs, const float *src, int64_t ld_src, float *dst,
                         int64_t ld_dst, hipStream_t s);
int launch_vec_norms(int64_t n, int64_t nrhs, int64_t nf, const double *B, int64_t sB,
                     uint64_t *out_bits, int64_t sOut, hipStream_t s);
int launch_max_reduce(int64_t n, int64_t nf, const double *v, int64_t sv, uint64_t *out_bits,
                      int64_t sOut, hipStream_t s);
int launch_row_abs_sums(int64_t n, const double *Z128, double *out, hipStream_t s);

// host fallback (complex128 GEPP); returns MSOLVE_OK or MSOLVE_E_FALLBACK
int host_gepp_solve(int64_t n, int64_t nrhs, const double *Z, const double *B, double *X);

// device fallback (complex128 GEPP on the GPU, blocking on `s`): work holds
// gepp_workspace_bytes(n); returns MSOLVE_OK, MSOLVE_E_FALLBACK on a zero or
// non-finite pivot, or a HIP status
size_t gepp_workspace_bytes(int64_t n);
int device_gepp_solve(int64_t n, int64_t nrhs, const double *Z, const double *B, double *X,
                      void *work, hipStream_t s);
// the same solve with the factors overwriting Zf (complex128 n x n, row
// major); aux holds gepp_aux_bytes(n) (pivots, report word, pivot candidates)
size_t gepp_aux_bytes(int64_t n);
int device_gepp_solve_inplace(int64_t n, int64_t nrhs, double *Zf, const double *B, double *X,
                              void *aux, hipStream_t s);

}  // namespace msolve
