/*
 * msolve -- repeated dense complex-symmetric solves Z(w) x = b to double
 * precision by single-precision LU plus double-precision iterative
 * refinement, on one AMD Instinct MI355X (gfx950).
 *
 * The method (page "Solving Dense Matrices Fast in the Browser -- Adaptive
 * Frequency Sampling and Mixed Precision on WebGPU", section "Double-precision
 * answers from a GPU without double precision", its four-step refinement
 * list):
 *   1. factorise Z in single precision (no row exchanges);
 *   2. solve with those factors for an approximate x;
 *   3. form r = b - Z x in double precision;
 *   4. solve for a correction with the single-precision factors, add it to x,
 *      and repeat from 3;
 * a frequency whose refinement does not converge is solved again by a direct
 * solve on the CPU (same section, paragraph after the list).  Z itself is
 *   Z(w) = j w L - j Psi / w + Zs(w) G
 * with L, Psi, G independent of frequency (same page, section "Fewer
 * frequency points: adaptive frequency sampling", model equation).
 *
 * Conventions for every entry point:
 *   - extern "C", reentrant; no function keeps state between calls except the
 *     optional timing registry (msolve_profile_*), which is process-wide, and
 *     two non-blocking streams per device, created on first use and kept
 *     until the process ends: the factorisation's look-ahead stream (n > 704)
 *     and the stream on which the refinement reads its per-pass counts.
 *   - Pointers are DEVICE pointers unless the argument says "host".
 *   - Matrices are row-major and contiguous with leading dimension n.
 *     Complex numbers are interleaved (re, im): a complex128 matrix of order n
 *     is 2*n*n doubles, a complex64 one 2*n*n floats.  Right-hand sides and
 *     solutions are stored as rows: B and X are nrhs x n complex arrays.
 *   - The caller owns every buffer, including the device workspace `work`;
 *     the library allocates device memory in one place only: the fallback
 *     direct solve of a frequency whose refinement failed takes a factor
 *     buffer of 16 n^2 bytes (+ 4 n) with hipMalloc and frees it before it
 *     returns (when the allocation fails it solves on the host, allocating
 *     host memory instead).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *   - Return value: MSOLVE_OK (0) or a negative status.  Argument errors are
 *     detected before any HIP call.  The text of the last error of the calling
 *     thread is returned by msolve_last_error().
 *   - Numerical outcomes are not errors: they are reported in the info
 *     structures (non-convergence => fallback = 1, status = 0).
 */
#ifndef MSOLVE_H
#define MSOLVE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    MSOLVE_OK = 0,
    MSOLVE_E_ARG = -1,        /* invalid argument (size, null pointer, tol, ...) */
    MSOLVE_E_HIP = -2,        /* a HIP runtime call failed; text in msolve_last_error */
    MSOLVE_E_WORKSPACE = -3,  /* work_bytes smaller than the matching *_workspace_bytes */
    MSOLVE_E_FALLBACK = -4,   /* the direct solve found Z singular (zero or
                                 non-finite pivot) */
    MSOLVE_E_DEVICE = -5      /* device kernel reported an internal failure (wait time-out) */
};

/*
 * The refinement's second stop condition (see msolve_refine): besides
 * eta <= tol, the estimated relative forward error of x must be at most this.
 * The backward error bounds the forward error only up to the condition
 * number, which near a resonance is large enough that eta <= 1e-13 leaves
 * forward errors above 1e-10; the bound here is half of that, since the
 * estimate is only an estimate.
 */
#define MSOLVE_FWD_TOL 5e-11

/* Per right-hand side outcome of msolve_refine. */
typedef struct {
    int32_t iters;      /* residual evaluations performed (one per correction) */
    int32_t converged;  /* 1 if eta <= tol was reached by the refinement */
    int32_t fallback;   /* 1 if the answer came from the direct solve */
    int32_t status;     /* 0, or a negative status of the fallback */
    double eta;         /* final normwise backward error (see msolve_refine) */
    double eta_first;   /* backward error after the first solve */
    double fwd_est;     /* estimated relative forward error at the stop (see
                           msolve_refine); NaN for an answer of the direct solve */
} msolve_rhs_info;

/* Per frequency outcome of msolve_sweep. */
typedef struct {
    int32_t iters_max;  /* largest iteration count over the right-hand sides */
    int32_t fallback;   /* 1 if this frequency was solved by the direct solve */
    int32_t status;     /* 0, or the negative status of this frequency */
    int32_t pivot_info; /* 0, or 1-based index of the first zero / non-finite pivot */
    double eta_max;     /* largest final backward error over the right-hand sides */
    double t_assemble_ms, t_factor_ms, t_refine_ms;  /* host wall-clock phases */
} msolve_freq_info;

/* Library version (major*10000 + minor*100 + patch). */
int32_t msolve_version(void);

/* Text of the last negative status returned to the calling thread. */
const char *msolve_last_error(void);

/* Block size of the factorisation for order n (the diagonal blocks whose
 * inverses msolve_factor_c64 returns). */
int64_t msolve_block_size(int64_t n);

/* Number of floats of the Dinv output of msolve_factor_c64 for order n:
 * 2 * (nblocks + nblocks / 2) * 2 * nb * nb with nblocks = ceil(n / nb)
 * (see msolve_factor_c64 for the layout). */
size_t msolve_dinv_floats(int64_t n);

/* Frequencies that msolve_sweep factorises and refines together (one batch)
 * for a sweep of nfreq frequencies of order n with nrhs right-hand sides:
 * the sweep is cut into ceil(nfreq / bmax) equal batches, where bmax (at most
 * 32) is the number of frequencies whose matrices fit in 24 GiB of
 * workspace.  0 for invalid sizes. */
int64_t msolve_sweep_batch(int64_t n, int64_t nrhs, int64_t nfreq);

/* Device workspace sizes in bytes, each already a multiple of 256.  The
 * factorisation's workspace holds one hand-off word per matrix for the two
 * workgroups that factorise each general diagonal block (batch: nf words). */
size_t msolve_factor_workspace_bytes(int64_t n);
size_t msolve_factor_batch_workspace_bytes(int64_t n, int64_t nf);
size_t msolve_refine_workspace_bytes(int64_t n, int64_t nrhs);
size_t msolve_sweep_workspace_bytes(int64_t n, int64_t nrhs, int64_t nfreq);
/* The largest of the three: enough for every call (nfreq: the largest
 * sweep that will be run). */
size_t msolve_workspace_bytes(int64_t n, int64_t nrhs, int64_t nfreq);

/*
 * Assembly of Z(w) = j w L - j Psi / w + Zs(w) G (model equation, section
 * "Fewer frequency points: adaptive frequency sampling").  With Zs = zs_re +
 * j zs_im and G = diag(g):
 *   Re Z_ij = (i == j) ? zs_re * g_i : 0
 *   Im Z_ij = w * L_ij - Psi_ij / w  (+ zs_im * g_i on the diagonal)
 * each operation rounded separately, in that order (IEEE division, no fused
 * multiply-add), so Z128 is bit-identical to the plain formula.
 *   L, Psi : n*n doubles (real, any matrix; the method uses symmetric ones)
 *   g      : n doubles
 *   Z128   : out, complex128 n x n, or NULL
 *   Z64    : out, complex64 n x n = round-to-nearest of Z128, or NULL
 *   zrowabs: out, n doubles, sum_j |Z_ij| (|.| = modulus), or NULL
 * Asynchronous on `stream`.  Errors: n < 1, omega not finite or zero, a null
 * input pointer, or all three outputs NULL -> MSOLVE_E_ARG.
 */
int msolve_assemble(int64_t n, double omega, double zs_re, double zs_im,
                    const double *L, const double *Psi, const double *g,
                    double *Z128, float *Z64, double *zrowabs, void *stream);

/*
 * Step 1 of the refinement list: unpivoted blocked LU of a complex64 matrix,
 * in place.  On return A holds L\U (unit lower L strictly below the diagonal,
 * U on and above it, A = L U up to single-precision rounding).  Dinv holds,
 * all nb x nb complex64 row-major (nb = msolve_block_size(n)):
 *   - for every diagonal block b, the inverse Li_b of its unit-lower block
 *     followed by the inverse Ui_b of its upper block (the last block padded
 *     with the identity);
 *   - then, for every pair of blocks (2t, 2t+1), the blocks that couple the
 *     pair in the inverses of its 2nb x 2nb triangles:
 *     X_t = -Li_{2t+1} L_{2t+1,2t} Li_{2t} (lower left of the unit-lower
 *     inverse) followed by Y_t = -Ui_{2t} U_{2t,2t+1} Ui_{2t+1} (upper right
 *     of the upper inverse), padded with zeros.
 *   A     : in/out complex64 n x n
 *   Dinv  : out, msolve_dinv_floats(n) floats
 *   d_info: out, one int32: 0, or the 1-based index of the first pivot that
 *           was zero or not finite (factors are then not usable)
 *   work  : msolve_factor_workspace_bytes(n) bytes of device scratch
 * Asynchronous on `stream` (for n > 704 the diagonal and panel steps run on
 * the library's look-ahead stream, ordered after the work already queued on
 * `stream`, and `stream` waits for them before its next command).  Two
 * workgroups factorise each diagonal block with the same elimination, one
 * sweeping L^-1, the other U^-1; the first overwrites the block only after
 * the second has read it (a bounded wait through the workspace; a wait that
 * times out reports the block's first pivot in d_info).  Calls that overlap
 * on one workspace race.
 */
int msolve_factor_c64(int64_t n, float *A, float *Dinv, int32_t *d_info,
                      void *work, size_t work_bytes, void *stream);

/*
 * msolve_factor_c64 for a complex-symmetric matrix (A^T = A, not Hermitian;
 * page "Solving Dense Matrices Fast in the Browser", section "Measure first:
 * the ceiling of JavaScript": Z is complex symmetric and a factorisation that
 * uses the symmetry needs half the work).  Only the entries of A on and
 * below the diagonal are read.  The trailing updates touch only those
 * entries, and each block row of U right of a diagonal block is formed as
 * D L^T (D = diag(U)) from the block column of L below it, as A = L U and
 * A^T = A give U = D L^T.  The outputs have the layout and meaning of
 * msolve_factor_c64 (L\U in A, Dinv, d_info), so msolve_lu_solve_c64 and
 * msolve_refine take them unchanged.  Each diagonal block is factorised as
 * L D L^T as well: its upper triangle holds U = D L^T (u_rc = d_r l_cr) and
 * its entry of Dinv the inverses L^-1 and U^-1 = L^-T D^-1, so every stored
 * factor is that of one L D L^T.  Arguments, workspace and errors as
 * msolve_factor_c64.
 * For a matrix that is not symmetric the factors are those of the matrix
 * whose upper triangle mirrors the lower one.
 */
int msolve_factor_c64_sym(int64_t n, float *A, float *Dinv, int32_t *d_info,
                          void *work, size_t work_bytes, void *stream);

/*
 * msolve_factor_c64 (sym == 0) or msolve_factor_c64_sym (sym != 0) for nf
 * matrices of order n in one go, as msolve_sweep factorises a batch of
 * frequencies: every launch covers all nf matrices.
 *   A     : in/out, matrix f at A + f * stride_A floats (stride_A >= 2 n^2)
 *   Dinv  : out, matrix f's at Dinv + f * stride_D floats
 *           (stride_D >= msolve_dinv_floats(n))
 *   d_info: out, nf int32 (matrix f's pivot report at d_info[f])
 *   work  : msolve_factor_batch_workspace_bytes(n, nf) bytes
 * Asynchronous as msolve_factor_c64.  Errors: n < 1, nf outside 1..65535,
 * a null pointer or a stride smaller than one matrix -> MSOLVE_E_ARG; a
 * small workspace -> MSOLVE_E_WORKSPACE.
 */
int msolve_factor_c64_batch(int64_t n, int64_t nf, float *A, int64_t stride_A, float *Dinv,
                            int64_t stride_D, int32_t *d_info, int32_t sym, void *work,
                            size_t work_bytes, void *stream);

/*
 * Steps 2 and 4 of the refinement list: solve L U x = rhs with the
 * single-precision factors, for nrhs right-hand sides in place.
 *   LU, Dinv: outputs of msolve_factor_c64
 *   RHS     : in/out complex64 nrhs x n
 *   work    : msolve_refine_workspace_bytes(n, nrhs) bytes
 * Asynchronous on `stream`.  A device wait time-out is reported by the next
 * synchronising call of the library that reads the same workspace.
 */
int msolve_lu_solve_c64(int64_t n, int64_t nrhs, const float *LU, const float *Dinv,
                        float *RHS, void *work, size_t work_bytes, void *stream);

/*
 * msolve_lu_solve_c64 for callers that cannot allocate device memory (code
 * being captured into a HIP graph, tight serving loops, harnesses that
 * forbid allocation): the same kernels, with the workspace taken from a
 * fixed array of msolve_lu_solve_noalloc_max_bytes() bytes (8 MiB) that the
 * library holds on every device it runs on until the process ends.  The
 * call allocates nothing.  A problem whose workspace
 * (msolve_refine_workspace_bytes(n, nrhs)) exceeds the array returns
 * MSOLVE_E_WORKSPACE; so do sizes beyond that (about n * nrhs > 260000).
 * Every call on one device shares that device's array (each call re-clears
 * what it needs), so calls that overlap on one device -- on two streams, or
 * from two host threads -- race and must not be issued.  Arguments, layout,
 * asynchrony and errors otherwise as msolve_lu_solve_c64.
 */
size_t msolve_lu_solve_noalloc_max_bytes(void);
int msolve_lu_solve_c64_noalloc(int64_t n, int64_t nrhs, const float *LU, const float *Dinv,
                                float *RHS, void *stream);

/*
 * Step 3 of the refinement list: R = B - Z X in double precision for nrhs
 * right-hand sides, streaming Z once.
 *   Z128 : complex128 n x n;  B, X : complex128 nrhs x n;  R : out, same shape
 *   norms: out, NULL or 2*nrhs doubles: ||r_k||_inf then ||x_k||_inf (modulus)
 * Asynchronous on `stream`.
 */
int msolve_residual_c128(int64_t n, int64_t nrhs, const double *Z128, const double *B,
                         const double *X, double *R, double *norms, void *stream);

/*
 * The refinement loop for one matrix (steps 2-4 of the list, with x0 = 0 so
 * that the first pass is step 2):
 *   for it = 1..max_iter:
 *     d = U^-1 L^-1 fl32(r);  x += d;  r = b - Z x (float64)
 *     eta_k = ||r_k|| / (||Z|| ||x_k|| + ||b_k||)   (infinity norms, modulus)
 *     est_k = min(rho, 1) ||d_k||,  rho = ||d_k|| / ||d_k of the pass before||
 *   stop when every eta_k <= tol and every est_k <= MSOLVE_FWD_TOL ||x_k||.
 * est_k estimates ||x - x_k||: the iteration contracts the error by about rho
 * per pass.  The first correction (x_1 itself) is never the denominator, so
 * the earliest stop is after three passes.
 * A right-hand side whose eta is not finite, or grows while above tol, or has
 * not met both bounds after max_iter iterations sends the whole matrix to the
 * direct solve (LU with partial pivoting in complex128), which then provides
 * X; info[k].fallback is set.  The direct solve runs on the device (see
 * msolve_gepp_solve_c128) when the workspace also holds its buffers, else on
 * the host (complex128 copies of Z and B, allocated and freed in the call).
 * The library allocates no device memory here.
 *   Z128    : complex128 n x n (the matrix in double precision)
 *   zrowabs : NULL or n doubles from msolve_assemble (row sums of |Z|)
 *   LU, Dinv: outputs of msolve_factor_c64 for fl32(Z)
 *   B       : complex128 nrhs x n;  X : out, complex128 nrhs x n
 *   tol     : > 0 bound on eta (0 forces the fallback); max_iter >= 0
 *   info    : host, nrhs entries
 *   work    : at least msolve_refine_workspace_bytes(n, nrhs) bytes; with
 *             msolve_refine_workspace_bytes(n, nrhs) +
 *             msolve_gepp_workspace_bytes(n) bytes or more, the tail holds
 *             the device direct solve's factor copy (16 n^2 B) and pivots
 * A matrix the direct solve finds singular returns MSOLVE_E_FALLBACK with
 * info[k].status set and X filled with NaN.
 * The stop test runs on the device after every residual and drops the
 * systems that have stopped from the later launches; the host reads the
 * count of systems still refining one pass behind (on the library's poll
 * stream, which waits only for that pass), so passes follow each other on
 * `stream` without waiting for the host, and a pass queued after the last
 * system stopped does nothing.  Blocking: returns when X and info are final.
 */
int msolve_refine(int64_t n, int64_t nrhs, const double *Z128, const double *zrowabs,
                  const float *LU, const float *Dinv, const double *B, double *X,
                  double tol, int32_t max_iter, void *work, size_t work_bytes,
                  msolve_rhs_info *info, void *stream);

/*
 * A frequency sweep: for each w_f, assemble Z(w_f) from L, Psi, g (the model
 * equation of the section "Fewer frequency points: adaptive frequency
 * sampling"), factorise fl32(Z) and refine every right-hand side (the
 * refinement list of the section "Double-precision answers from a GPU
 * without double precision"), with the per-frequency fallback to a direct
 * solve that the paragraph after that list describes; the page runs the
 * frequencies of its sweeps one after another, each with its own solve.
 * The frequencies go in batches of msolve_sweep_batch(n, nrhs, nfreq): every
 * kernel launch of the assembly, the factorisation and the refinement covers
 * the whole batch (the refinement loop runs until every frequency of the
 * batch has converged or been handed to the fallback; converged frequencies
 * are not updated further).  The results are those of msolve_assemble,
 * msolve_factor_c64 and msolve_refine applied to each frequency, except that
 * when L and Psi are exactly symmetric (checked on the device at the start
 * of the call), every Z(w) is complex symmetric and msolve_factor_c64_sym's
 * factorisation is used instead; a frequency whose refinement does not
 * converge with those factors (and whose factorisation met no bad pivot) is
 * then factorised with msolve_factor_c64 and refined again, before any host
 * fallback, and its info describes that second refinement (which continues
 * from the first one's answer when that met eta <= tol and failed only the
 * forward-error estimate, and starts from x = 0 otherwise).  No
 * complex128 copy of Z is stored: the residual forms each entry from L, Psi
 * and g with the assembly's operations, bit-identical to it, and a
 * frequency that falls back has its complex128 matrix assembled on demand
 * into one spare slot of the workspace, where the device direct solve
 * factorises it in place (no device memory is allocated by the call).
 * A frequency that the direct solve finds singular does not stop the sweep:
 * its finfo/rinfo status is MSOLVE_E_FALLBACK, its rows of X are NaN, every
 * other frequency (later batches included) is solved as usual, and the call
 * returns MSOLVE_E_FALLBACK at the end.
 *   omega : host, nfreq doubles;  zs : host, 2*nfreq doubles (re, im of Zs(w_f))
 *   L, Psi: n*n doubles;  g : n doubles
 *   B     : complex128 nrhs x n (the same right-hand sides at every frequency)
 *   X     : out, complex128 nfreq x nrhs x n
 *   finfo : host, nfreq entries (the t_*_ms times are those of the batch
 *           the frequency belongs to);  rinfo : host, nfreq*nrhs entries, or NULL
 *   work  : msolve_sweep_workspace_bytes(n, nrhs, nfreq) bytes
 * Runs on `stream`, for n > 704 also on the library's look-ahead stream,
 * and with more than one batch also on its front stream: batch b + 1 is
 * assembled and factorised there (into a second set of per-frequency
 * arrays) while batch b is refined on `stream`.  Blocking: returns when X
 * is complete.  Other negative statuses (arguments, workspace, HIP errors)
 * stop the call at once.
 */
int msolve_sweep(int64_t n, int64_t nfreq, const double *omega, const double *zs,
                 const double *L, const double *Psi, const double *g,
                 int64_t nrhs, const double *B, double *X, double tol, int32_t max_iter,
                 void *work, size_t work_bytes, msolve_freq_info *finfo,
                 msolve_rhs_info *rinfo, void *stream);

/*
 * Reduced-order frequency sweep (adaptive frequency sampling; page "Solving
 * Dense Matrices Fast in the Browser", section "Fewer frequency points:
 * adaptive frequency sampling").  Solves exactly (with msolve_sweep) at the
 * first and last candidate frequency, builds a real orthonormal basis V from
 * the real and imaginary parts of the solutions, and at every candidate w_f
 * solves the q x q reduced system
 *     (jw V^T L V - j V^T Psi V / w + Zs(w) V^T G V) y = V^T b,
 * taking x = V y.  The candidate whose residual ||Z(w) V y - b||_2 /
 * ||b||_2 (largest over the right-hand sides) is largest is solved exactly
 * next and its solution joins the basis, until every estimate is <= tol or
 * max_exact frequencies have been solved exactly.
 * Readings of the section (it leaves these open): the first exact
 * frequencies are the two ends of the list; each new real or imaginary part
 * is orthogonalised by two passes of modified Gram-Schmidt and left out when
 * less than 1e-10 of its 2-norm remains; equal estimates go to the lowest
 * index.
 *   omega, zs, L, Psi, g, B : as msolve_sweep (every row of B nonzero)
 *   X        : out, device complex128 nfreq x nrhs x n: V y at every candidate
 *   tol      : stop once every estimate is <= tol (the section uses 1e-4)
 *   max_exact: at most this many exact solves (>= 1; capped at nfreq)
 *   solve_tol, solve_max_iter : the refinement settings of the exact solves
 *   exact    : host out, int32[nfreq]: the exactly solved indices in the
 *              order they were chosen (the first *n_exact are set)
 *   estimate : host out, double[nfreq]: the final residual estimates
 *   q_out    : host out: the basis size q
 *   work     : msolve_afs_workspace_bytes(n, nrhs, nfreq, max_exact) bytes
 * The residual needs no product with Z: with A = L V, P = Psi V, Q = G V
 * (device products, L and Psi read once per batch of new basis vectors),
 * ||M y - b||^2 for M = jw A - j P / w + Zs Q comes from the inner products
 * of V, A, P, Q and b (one device Gram launch per exact solve).  The q x q
 * systems are solved on the host (complex128 Gaussian elimination with
 * partial pivoting, candidates spread over host threads); an exactly
 * singular one returns MSOLVE_E_FALLBACK.
 * Blocking; runs on `stream` (and the streams msolve_sweep uses).
 */
size_t msolve_afs_workspace_bytes(int64_t n, int64_t nrhs, int64_t nfreq, int32_t max_exact);
int msolve_afs(int64_t n, int64_t nfreq, const double *omega, const double *zs,
               const double *L, const double *Psi, const double *g, int64_t nrhs,
               const double *B, double *X, double tol, int32_t max_exact, double solve_tol,
               int32_t solve_max_iter, int32_t *exact, int32_t *n_exact, double *estimate,
               int32_t *q_out, void *work, size_t work_bytes, void *stream);

/*
 * The fallback direct solve on its own (HOST pointers): X = Z^-1 B by
 * complex128 LU with partial pivoting (the CPU direct solve of the section
 * "Double-precision answers from a GPU without double precision").
 *   Z: host complex128 n x n (not modified);  B, X: host complex128 nrhs x n
 * Returns MSOLVE_E_FALLBACK if a pivot is exactly zero.
 */
int msolve_host_solve_c128(int64_t n, int64_t nrhs, const double *Z, const double *B,
                           double *X);

/*
 * The fallback direct solve on the device: X = Z^-1 B by complex128 LU with
 * partial pivoting (the double-precision direct solve of the section
 * "Double-precision answers from a GPU without double precision", which the
 * page runs on the CPU; the pivoting rule is that of the section "Measure
 * first: the ceiling of JavaScript").  The refinement's per-frequency
 * fallback calls it with a buffer of its own.
 *   Z    : complex128 n x n (not modified)
 *   B    : complex128 nrhs x n;  X : out, complex128 nrhs x n (X == B is
 *          allowed, otherwise the two must not overlap)
 *   work : msolve_gepp_workspace_bytes(n) bytes: the factors (a copy of Z,
 *          overwritten by L and U), the pivot rows, a status word and one
 *          pivot candidate per workgroup of the column step
 * Pivot of column j: the row i >= j of largest |Re z_ij| + |Im z_ij| (the
 * lowest i among equal ones), whole rows exchanged.  nrhs <= 65535.
 * Returns MSOLVE_E_FALLBACK if a pivot is zero or not finite (X then holds
 * no answer).  Blocking: the call waits on `stream` for the status word.
 */
size_t msolve_gepp_workspace_bytes(int64_t n);
int msolve_gepp_solve_c128(int64_t n, int64_t nrhs, const double *Z, const double *B, double *X,
                           void *work, size_t work_bytes, void *stream);

/*
 * Optional timing registry (instrumentation).  When enabled, every launch of
 * the kernels below is bracketed by HIP events on the stream it runs on;
 * msolve_profile_query synchronises those events and returns the number of
 * launches and their summed duration.  Process-wide; not thread-safe against
 * concurrent enable/reset.
 */
enum {
    MSOLVE_K_ASSEMBLE = 0,
    MSOLVE_K_LU_DIAG = 1,
    MSOLVE_K_LU_PANEL = 2,
    MSOLVE_K_LU_UPDATE = 3,
    MSOLVE_K_TRSV_FWD = 4,
    MSOLVE_K_TRSV_BWD = 5,
    MSOLVE_K_RESIDUAL = 6,
    MSOLVE_K_LU_BULK = 7,     /* the bulk trailing updates (large tiles); other
                                 updates are MSOLVE_K_LU_UPDATE */
    MSOLVE_K_AFS_PROJECT = 8, /* L V, Psi V, G V of msolve_afs (bytes: L and Psi) */
    MSOLVE_K_GEPP_UPDATE = 9, /* trailing updates of msolve_gepp_solve_c128
                                 (real flops: 8 m^2 w per panel) */
    MSOLVE_K_COUNT = 10
};
int msolve_profile_enable(int32_t on);
int msolve_profile_reset(void);
int msolve_profile_query(int32_t kernel, int64_t *launches, double *total_ms,
                         double *flops_or_bytes);

#ifdef __cplusplus
}
#endif

#endif /* MSOLVE_H */
