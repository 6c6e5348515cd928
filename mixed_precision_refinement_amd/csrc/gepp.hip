// Device fallback: complex128 LU with partial pivoting, then substitution,
// all on the GPU.
//
// Page "Solving Dense Matrices Fast in the Browser", section "Double-precision
// answers from a GPU without double precision": a frequency whose refinement
// does not converge is solved directly in double precision (LU with partial
// pivoting, section "Measure first: the ceiling of JavaScript").  The page
// runs that solve on the CPU; this device has native fp64, so the same solve
// runs here and Z never leaves HBM.  The host solver stays as the last
// resort when the workspace cannot be allocated.
//
// Layout: Z row major (row i at Z + 2 i n), B and X right-hand-side major
// (right-hand side k at X + 2 k n), complex128 interleaved.  The factors
// overwrite a copy of Z in the workspace; X is copied from B and permuted in
// place as the pivot rows are found.
//
// Right-looking factorisation in column panels of kGW:
//   per column j of the panel: gepp_pivot_kernel (one workgroup: pivot
//   search, whole-row swap of the factors and of X), gepp_column_kernel
//   (multipliers of column j, rank-1 update of the panel's later columns);
//   per panel: gepp_trsm_kernel (U12 = L11^-1 A12, one thread per column),
//   gepp_update_kernel (A22 -= L21 U12, 64 x 64 tiles in LDS, fp64 FMA).
// Substitution in row blocks of kGW: a one-wave diagonal-block solve per
// right-hand side, then a matrix-vector update of the rows not yet solved.
#include <algorithm>
#include <cfloat>

#include "common.hpp"

namespace msolve {
namespace {

constexpr int kGW = 32;        // panel width = substitution block
constexpr int kPivThreads = 256;

__device__ __forceinline__ double2 cmul(double2 a, double2 b)
{
    return make_double2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}

__device__ __forceinline__ double2 cfma(double2 a, double2 b, double2 c)
{
    return make_double2(fma(a.x, b.x, fma(-a.y, b.y, c.x)), fma(a.x, b.y, fma(a.y, b.x, c.y)));
}

// a / b with both scaled by |Re b| + |Im b| first (no overflow of |b|^2)
__device__ __forceinline__ double2 cdiv(double2 a, double2 b)
{
    const double s = fabs(b.x) + fabs(b.y);
    const double br = b.x / s, bi = b.y / s, ar = a.x / s, ai = a.y / s;
    const double d = br * br + bi * bi;
    return make_double2((ar * br + ai * bi) / d, (ai * br - ar * bi) / d);
}

__device__ __forceinline__ double2 csub(double2 a, double2 b)
{
    return make_double2(a.x - b.x, a.y - b.y);
}

// Pivot of column j: the row p >= j of largest |Re| + |Im| (the BLAS
// convention; the lowest index among equal ones), then rows j and p swapped
// over all n columns of the factors and in every right-hand side.  A zero or
// non-finite pivot records column j + 1 in info[0] (the first one only) and
// swaps nothing.  One workgroup of kPivThreads.  With np > 0 the column was
// last updated by gepp_column_kernel, which left one candidate per workgroup
// (pv: its largest |Re| + |Im|, +inf if one was not finite, -1 if it had no
// row; pi: the row); the search then reduces those np candidates.
__global__ __launch_bounds__(kPivThreads) void gepp_pivot_kernel(
    int64_t n, int64_t j, double2 *__restrict__ A, int64_t nrhs, double2 *__restrict__ X,
    int32_t *__restrict__ piv, int32_t *__restrict__ info, const double *__restrict__ pv,
    const int64_t *__restrict__ pi, int64_t np)
{
    __shared__ double sv[kPivThreads / 64];
    __shared__ int64_t si[kPivThreads / 64];
    const int t = threadIdx.x;
    if (j == 0 && t == 0) info[0] = 0;
    double best = -1.0;
    int64_t bi = n;
    int bad = 0;
    if (np > 0) {
        for (int64_t q = t; q < np; q += kPivThreads) {
            const double m = pv[q];
            if (m > best) { best = m; bi = pi[q]; }
        }
    } else {
        for (int64_t i = j + t; i < n; i += kPivThreads) {
            const double2 a = A[i * n + j];
            const double m = fabs(a.x) + fabs(a.y);
            if (!(m <= DBL_MAX)) bad = 1;
            else if (m > best) { best = m; bi = i; }
        }
    }
    // largest value, lowest index among equal ones: across the wave by
    // shuffles, then across the waves through LDS
    for (int m = 32; m > 0; m >>= 1) {
        const double ov = __shfl_xor(best, m, 64);
        const int64_t oi = __shfl_xor(bi, m, 64);
        if (ov > best || (ov == best && oi < bi)) { best = ov; bi = oi; }
    }
    if ((t & 63) == 0) { sv[t >> 6] = best; si[t >> 6] = bi; }
    bad = __syncthreads_or(bad);
    best = sv[0];
    bi = si[0];
    for (int q = 1; q < kPivThreads / 64; ++q)
        if (sv[q] > best || (sv[q] == best && si[q] < bi)) { best = sv[q]; bi = si[q]; }
    const bool ok = !bad && best > 0.0 && best <= DBL_MAX;
    const int64_t p = ok ? bi : j;
    if (t == 0) {
        piv[j] = int32_t(p);
        if (!ok && info[0] == 0) info[0] = int32_t(j + 1);
    }
    if (p == j) return;
    for (int64_t c = t; c < n; c += kPivThreads) {
        const double2 a = A[j * n + c];
        A[j * n + c] = A[p * n + c];
        A[p * n + c] = a;
    }
    for (int64_t k = t; k < nrhs; k += kPivThreads) {
        const double2 a = X[k * n + j];
        X[k * n + j] = X[k * n + p];
        X[k * n + p] = a;
    }
}

// Rows i in (j, n): l_ij = a_ij / a_jj stored in column j, and the panel's
// later columns c in (j, p1) take a_ic -= l_ij a_jc.  8 rows of 32 lanes per
// workgroup; lane 0 of a row forms its multiplier.  When column j + 1 is in
// the panel, each workgroup also leaves its pivot candidate for that column
// in pv[blockIdx.x], pi[blockIdx.x] (see gepp_pivot_kernel).
__global__ __launch_bounds__(256) void gepp_column_kernel(int64_t n, int64_t j, int64_t p1,
                                                          double2 *__restrict__ A,
                                                          double *__restrict__ pv,
                                                          int64_t *__restrict__ pi)
{
    __shared__ double2 ls[8];
    __shared__ double mv[8];
    const int r = threadIdx.x >> 5, cl = threadIdx.x & 31;
    const int64_t i = j + 1 + int64_t(blockIdx.x) * 8 + r;
    if (i < n && cl == 0) ls[r] = cdiv(A[i * n + j], A[j * n + j]);
    if (cl == 1) mv[r] = -1.0;
    __syncthreads();
    if (i < n) {
        if (cl == 0) {
            A[i * n + j] = ls[r];
        } else if (j + cl < p1) {
            const double2 l = ls[r], u = A[j * n + j + cl];
            const double2 v = cfma(make_double2(-l.x, -l.y), u, A[i * n + j + cl]);
            A[i * n + j + cl] = v;
            if (cl == 1) {
                const double m = fabs(v.x) + fabs(v.y);
                mv[r] = m <= DBL_MAX ? m : __builtin_inf();
            }
        }
    }
    if (j + 1 >= p1) return;
    __syncthreads();
    if (threadIdx.x == 0) {
        double best = -1.0;
        int64_t bi = n;
        for (int q = 0; q < 8; ++q)
            if (mv[q] > best) { best = mv[q]; bi = j + 1 + int64_t(blockIdx.x) * 8 + q; }
        pv[blockIdx.x] = best;
        pi[blockIdx.x] = bi;
    }
}

// U12 = L11^-1 A12 for the panel rows [p0, p0 + w) and the columns
// [p0 + w, n): one thread per column, L11 (unit lower) in LDS.
__global__ __launch_bounds__(256) void gepp_trsm_kernel(int64_t n, int64_t p0, int w,
                                                        double2 *__restrict__ A)
{
    __shared__ double2 Ls[kGW][kGW];
    for (int e = threadIdx.x; e < w * w; e += 256) {
        const int r = e / w, s = e % w;
        Ls[r][s] = A[(p0 + r) * n + p0 + s];
    }
    __syncthreads();
    const int64_t c = p0 + w + int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (c >= n) return;
    double2 u[kGW];
#pragma unroll
    for (int r = 0; r < kGW; ++r) {
        if (r < w) {
            double2 v = A[(p0 + r) * n + c];
#pragma unroll
            for (int s = 0; s < r; ++s) v = cfma(make_double2(-Ls[r][s].x, -Ls[r][s].y), u[s], v);
            u[r] = v;
            A[(p0 + r) * n + c] = v;
        }
    }
}

// A22 -= L21 U12 over the rows and columns [p0 + w, n): 64 x 64 tiles, the
// K = w products in two LDS slices of 16; each of the 256 threads owns 4 x 4
// outputs (rows ty + 16 a, columns tx + 16 b).
__global__ __launch_bounds__(256) void gepp_update_kernel(int64_t n, int64_t p0, int w,
                                                          double2 *__restrict__ A)
{
    __shared__ double2 Lt[64][17];
    __shared__ double2 Ut[16][64];
    const int t = threadIdx.x, tx = t & 15, ty = t >> 4;
    const int64_t base = p0 + w;
    const int64_t i0 = base + int64_t(blockIdx.y) * 64, c0 = base + int64_t(blockIdx.x) * 64;
    double2 acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = make_double2(0.0, 0.0);
    for (int k0 = 0; k0 < w; k0 += 16) {
        for (int e = t; e < 64 * 16; e += 256) {
            const int r = e >> 4, s = e & 15;
            const int64_t i = i0 + r;
            Lt[r][s] = (i < n && k0 + s < w) ? A[i * n + p0 + k0 + s] : make_double2(0.0, 0.0);
        }
        for (int e = t; e < 16 * 64; e += 256) {
            const int s = e >> 6, cc = e & 63;
            const int64_t c = c0 + cc;
            Ut[s][cc] = (c < n && k0 + s < w) ? A[(p0 + k0 + s) * n + c] : make_double2(0.0, 0.0);
        }
        __syncthreads();
#pragma unroll 4
        for (int s = 0; s < 16; ++s) {
            double2 l[4], u[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) l[a] = Lt[ty + 16 * a][s];
#pragma unroll
            for (int b = 0; b < 4; ++b) u[b] = Ut[s][tx + 16 * b];
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b) acc[a][b] = cfma(l[a], u[b], acc[a][b]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int64_t i = i0 + ty + 16 * a;
        if (i >= n) continue;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int64_t c = c0 + tx + 16 * b;
            if (c < n) A[i * n + c] = csub(A[i * n + c], acc[a][b]);
        }
    }
}

__device__ __forceinline__ double2 sum_lanes(double2 v, int width)
{
    for (int m = width / 2; m > 0; m >>= 1) {
        v.x += __shfl_xor(v.x, m, width);
        v.y += __shfl_xor(v.y, m, width);
    }
    return v;
}

// Diagonal block [r0, r0 + w) of the substitution, one wave per right-hand
// side (blockIdx.x): forward with the unit lower factor, or backward with the
// upper factor.  Lane s holds x_{r0+s}; each row's sum over the block is a
// wave reduction.
template <bool kForward>
__global__ __launch_bounds__(64) void gepp_subst_diag_kernel(int64_t n, int64_t r0, int w,
                                                             const double2 *__restrict__ A,
                                                             double2 *__restrict__ X)
{
    const int lane = threadIdx.x;
    double2 *x = X + int64_t(blockIdx.x) * n;
    // lane s holds column s of the block (a_{r0+r, r0+s} for every row r)
    // and b_{r0+s}, loaded before the dependent chain starts
    double2 col[kGW];
#pragma unroll
    for (int r = 0; r < kGW; ++r)
        col[r] = (r < w && lane < w) ? A[(r0 + r) * n + r0 + lane] : make_double2(0.0, 0.0);
    const double2 xb = lane < w ? x[r0 + lane] : make_double2(0.0, 0.0);
    double2 xs = make_double2(0.0, 0.0);
#pragma unroll
    for (int q = 0; q < kGW; ++q) {
        const int r = kForward ? q : kGW - 1 - q;
        if (r < w) {
            const bool use = kForward ? lane < r : (lane > r && lane < w);
            double2 v = use ? cmul(col[r], xs) : make_double2(0.0, 0.0);
            v = sum_lanes(v, 64);
            if (lane == r) {
                const double2 y = csub(xb, v);
                xs = kForward ? y : cdiv(y, col[r]);
            }
        }
    }
    if (lane < w) x[r0 + lane] = xs;
}

// Rows not yet solved take x_i -= sum_s A[i][r0 + s] x_{r0+s} over the block
// just solved: rows [r0 + w, n) going forward, rows [0, r0) going backward.
// 8 rows of 32 lanes per workgroup, lane s reads A[i][r0 + s].
template <bool kForward>
__global__ __launch_bounds__(256) void gepp_subst_update_kernel(int64_t n, int64_t r0, int w,
                                                                const double2 *__restrict__ A,
                                                                int64_t nrhs,
                                                                double2 *__restrict__ X)
{
    const int r = threadIdx.x >> 5, s = threadIdx.x & 31;
    const int64_t lo = kForward ? r0 + w : 0, hi = kForward ? n : r0;
    const int64_t i = lo + int64_t(blockIdx.x) * 8 + r;
    const bool row = i < hi;
    const double2 l = (row && s < w) ? A[i * n + r0 + s] : make_double2(0.0, 0.0);
    for (int64_t k = 0; k < nrhs; ++k) {
        double2 *x = X + k * n;
        const double2 xv = s < w ? x[r0 + s] : make_double2(0.0, 0.0);
        const double2 v = sum_lanes(cmul(l, xv), 32);
        if (row && s == 0) x[i] = csub(x[i], v);
    }
}

inline unsigned grid_of(int64_t items, int64_t per) { return unsigned((items + per - 1) / per); }

}  // namespace

size_t gepp_aux_bytes(int64_t n)
{
    const size_t cand = align256(8 * size_t(n / 8 + 2));
    return align256(sizeof(int32_t) * size_t(n)) + 256 + 2 * cand;
}

size_t gepp_workspace_bytes(int64_t n)
{
    return align256(sizeof(double2) * size_t(n) * size_t(n)) + gepp_aux_bytes(n);
}

int device_gepp_solve(int64_t n, int64_t nrhs, const double *Z, const double *B, double *X,
                      void *work, hipStream_t s)
{
    auto *A = static_cast<double *>(work);
    MS_HIP(hipMemcpyAsync(A, Z, sizeof(double2) * size_t(n) * size_t(n), hipMemcpyDeviceToDevice, s));
    return device_gepp_solve_inplace(n, nrhs, A, B, X,
                                     static_cast<char *>(work) + align256(sizeof(double2) * size_t(n) * size_t(n)),
                                     s);
}

int device_gepp_solve_inplace(int64_t n, int64_t nrhs, double *Zf, const double *B, double *X,
                              void *aux, hipStream_t s)
{
    auto *A = reinterpret_cast<double2 *>(Zf);
    char *p = static_cast<char *>(aux);
    auto *piv = reinterpret_cast<int32_t *>(p);
    auto *dinfo = reinterpret_cast<int32_t *>(p + align256(sizeof(int32_t) * size_t(n)));
    const size_t cand = align256(8 * size_t(n / 8 + 2));
    auto *pv = reinterpret_cast<double *>(reinterpret_cast<char *>(dinfo) + 256);
    auto *pi = reinterpret_cast<int64_t *>(reinterpret_cast<char *>(pv) + cand);
    auto *Xc = reinterpret_cast<double2 *>(X);
    if (X != B)
        MS_HIP(hipMemcpyAsync(X, B, sizeof(double2) * size_t(n) * size_t(nrhs), hipMemcpyDeviceToDevice, s));

    for (int64_t p0 = 0; p0 < n; p0 += kGW) {
        const int w = int(std::min<int64_t>(kGW, n - p0));
        const int64_t p1 = p0 + w;
        for (int64_t j = p0; j < p1; ++j) {
            // column j's candidates were left by the column step of j - 1
            // (its grid_of(n - j, 8) workgroups) unless j opens the panel
            const int64_t np = j > p0 ? int64_t(grid_of(n - j, 8)) : 0;
            hipLaunchKernelGGL(gepp_pivot_kernel, dim3(1), dim3(kPivThreads), 0, s, n, j, A, nrhs, Xc,
                               piv, dinfo, pv, pi, np);
            if (j + 1 < n)
                hipLaunchKernelGGL(gepp_column_kernel, dim3(grid_of(n - j - 1, 8)), dim3(256), 0, s, n,
                                   j, p1, A, pv, pi);
        }
        const int64_t m = n - p1;
        if (m > 0) {
            hipLaunchKernelGGL(gepp_trsm_kernel, dim3(grid_of(m, 256)), dim3(256), 0, s, n, p0, w, A);
            ProfScope prof(MSOLVE_K_GEPP_UPDATE, s, 8.0 * double(m) * double(m) * double(w));
            hipLaunchKernelGGL(gepp_update_kernel, dim3(grid_of(m, 64), grid_of(m, 64)), dim3(256), 0,
                               s, n, p0, w, A);
        }
        MS_HIP(hipGetLastError());
    }
    for (int64_t r0 = 0; r0 < n; r0 += kGW) {
        const int w = int(std::min<int64_t>(kGW, n - r0));
        hipLaunchKernelGGL(gepp_subst_diag_kernel<true>, dim3(unsigned(nrhs)), dim3(64), 0, s, n, r0,
                           w, A, Xc);
        if (r0 + w < n)
            hipLaunchKernelGGL(gepp_subst_update_kernel<true>, dim3(grid_of(n - r0 - w, 8)), dim3(256),
                               0, s, n, r0, w, A, nrhs, Xc);
    }
    for (int64_t r0 = (n - 1) / kGW * kGW; r0 >= 0; r0 -= kGW) {
        const int w = int(std::min<int64_t>(kGW, n - r0));
        hipLaunchKernelGGL(gepp_subst_diag_kernel<false>, dim3(unsigned(nrhs)), dim3(64), 0, s, n, r0,
                           w, A, Xc);
        if (r0 > 0)
            hipLaunchKernelGGL(gepp_subst_update_kernel<false>, dim3(grid_of(r0, 8)), dim3(256), 0, s,
                               n, r0, w, A, nrhs, Xc);
    }
    MS_HIP(hipGetLastError());
    int32_t info = 0;
    MS_HIP(hipMemcpyAsync(&info, dinfo, sizeof(info), hipMemcpyDeviceToHost, s));
    MS_HIP(hipStreamSynchronize(s));
    if (info != 0)
        return fail(MSOLVE_E_FALLBACK, "device direct solve: zero or non-finite pivot in column " +
                                           std::to_string(info - 1));
    return MSOLVE_OK;
}

}  // namespace msolve

extern "C" size_t msolve_gepp_workspace_bytes(int64_t n)
{
    return n > 0 ? msolve::gepp_workspace_bytes(n) : 0;
}

extern "C" int msolve_gepp_solve_c128(int64_t n, int64_t nrhs, const double *Z, const double *B,
                                      double *X, void *work, size_t work_bytes, void *stream)
{
    using namespace msolve;
    if (n <= 0 || nrhs <= 0 || nrhs > 65535 || n > (int64_t(1) << 31) - 1 || !Z || !B || !X || !work)
        return fail(MSOLVE_E_ARG, "msolve_gepp_solve_c128: bad size or null pointer");
    if (work_bytes < gepp_workspace_bytes(n))
        return fail(MSOLVE_E_WORKSPACE, "msolve_gepp_solve_c128: workspace too small");
    return device_gepp_solve(n, nrhs, Z, B, X, work, static_cast<hipStream_t>(stream));
}
