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
// overwrite a copy of Z in the workspace; X is copied from B and takes each
// panel's interchanges after the panel.
//
// Right-looking factorisation in column panels of kGW, the panel's rows left
// in place while it is factorised:
//   gepp_cand_kernel: each of up to 256 workgroups leaves the pivot candidate
//   of its rows for the panel's first column;
//   per column j: gepp_step_kernel, one launch: every workgroup reduces the
//   candidates to the same pivot row, then updates its rows not yet pivoted
//   (multipliers of column j, rank-1 update of the panel's later columns) and
//   leaves its candidate for column j + 1; the rows' logical positions (the
//   order the interchanges so far give them) are tracked per row;
//   per panel: gepp_swap_kernel (the panel's interchanges in order, over all
//   columns and every right-hand side), gepp_trsm_kernel (U12 = L11^-1 A12,
//   one thread per column), gepp_update_kernel (A22 -= L21 U12, 64 x 64
//   tiles in LDS, fp64 FMA).
// The arithmetic on every entry, the pivots and their order are those of
// swapping whole rows at each column.
// Substitution in row blocks of kGW: a one-wave diagonal-block solve per
// right-hand side, then a matrix-vector update of the rows not yet solved.
#include <algorithm>
#include <cfloat>
#include <cstdint>

#include "common.hpp"

namespace msolve {
namespace {

constexpr int kGW = 32;        // panel width = substitution block
constexpr int kStepThreads = 256;
constexpr int kStepGroups = 256;  // workgroups of a column step (at most; one candidate per thread)
constexpr int kStepPre = 4;       // rows per lane a column step loads before its pivot is known

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

// A workgroup's pivot candidate: its largest |Re| + |Im| (+inf when an
// entry is not finite, -1 when it has no row), that row's logical position
// (its place in the order the panel's interchanges so far give the rows) and
// the row itself.  The pivot is the largest, the lowest position among equal
// ones (the BLAS convention).
struct Cand {
    double v;
    int32_t pos, row;
};
__device__ __forceinline__ bool cand_before(double v, int32_t pos, double bv, int32_t bpos)
{
    return v > bv || (v == bv && pos < bpos);
}
// the best of every thread's (v, pos, row) in a workgroup of 256, in all
// threads
__device__ __forceinline__ Cand cand_reduce(double v, int32_t pos, int32_t row, Cand *scratch)
{
    for (int m = 32; m > 0; m >>= 1) {
        const double ov = __shfl_xor(v, m, 64);
        const int32_t op = __shfl_xor(pos, m, 64), orow = __shfl_xor(row, m, 64);
        if (cand_before(ov, op, v, pos)) {
            v = ov;
            pos = op;
            row = orow;
        }
    }
    if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = Cand{v, pos, row};
    __syncthreads();
    Cand b = scratch[0];
    for (int q = 1; q < kStepThreads / 64; ++q)
        if (cand_before(scratch[q].v, scratch[q].pos, b.v, b.pos)) b = scratch[q];
    return b;
}

// First column p0 of a panel: workgroup g scans its rows [p0 + g R, p0 +
// (g + 1) R) and leaves its candidate; the rows' logical positions start as
// the rows themselves (the earlier panels' interchanges are applied).
__global__ __launch_bounds__(kStepThreads) void gepp_cand_kernel(int64_t n, int64_t p0, int64_t R,
                                                                 const double2 *__restrict__ A,
                                                                 int32_t *__restrict__ pos,
                                                                 Cand *__restrict__ cand,
                                                                 int32_t *__restrict__ info)
{
    __shared__ Cand sc[kStepThreads / 64];
    if (p0 == 0 && blockIdx.x == 0 && threadIdx.x == 0) info[0] = 0;
    const int64_t lo = p0 + int64_t(blockIdx.x) * R, hi = min(n, lo + R);
    double bv = -1.0;
    int32_t bpos = INT32_MAX, brow = -1;
    for (int64_t i = lo + threadIdx.x; i < hi; i += kStepThreads) {
        pos[i] = int32_t(i);
        const double2 a = A[i * n + p0];
        double m = fabs(a.x) + fabs(a.y);
        if (!(m <= DBL_MAX)) m = __builtin_inf();
        if (cand_before(m, int32_t(i), bv, bpos)) {
            bv = m;
            bpos = int32_t(i);
            brow = int32_t(i);
        }
    }
    const Cand b = cand_reduce(bv, bpos, brow, sc);
    if (threadIdx.x == 0) cand[blockIdx.x] = b;
}

// Column step j of the panel [p0, p1), rows left in place: the pivot row pr
// from the ncin candidates (identical in every workgroup); piv[j] = its
// logical position (LAPACK's interchange of rows j and piv[j]); a zero or
// non-finite pivot records column j + 1 in info[0] (the first one only).
// Workgroup g takes its rows [p0 + g R, ...) that are not yet pivoted
// (pos_in >= j) other than pr: l = a_ij / a_pr,j stored in column j, and the
// panel's later columns c take a_ic -= l a_pr,c.  The pivot row is only read.
// Logical positions move to pos_out (pr to j, the row at position j to pr's
// old one), and each workgroup leaves its candidate for column j + 1.  8 rows
// of 32 lanes per pass: lane c works on column j + c.
__global__ __launch_bounds__(kStepThreads) void gepp_step_kernel(
    int64_t n, int64_t j, int64_t p0, int64_t p1, int64_t R, double2 *__restrict__ A,
    const int32_t *__restrict__ pos_in, int32_t *__restrict__ pos_out, const Cand *__restrict__ cin,
    int ncin, Cand *__restrict__ cout, int32_t *__restrict__ piv, int32_t *__restrict__ info)
{
    __shared__ Cand sc[kStepThreads / 64], sc2[kStepThreads / 64];   // the two reductions' own
    const int t = threadIdx.x;
    const int r = t >> 5, cl = t & 31;
    const int64_t lo = p0 + int64_t(blockIdx.x) * R, hi = min(n, lo + R);
    // the workgroup's rows do not depend on the pivot: their positions and
    // entries are loaded first, beside the candidates (up to kStepPre rows
    // per lane; more rows, as at n above 8 kStepPre kStepGroups, are
    // loaded as they are reached)
    int32_t pp[kStepPre];
    double2 aj[kStepPre], ac[kStepPre];
#pragma unroll
    for (int q = 0; q < kStepPre; ++q) {
        const int64_t i = lo + 8 * q + r;
        const bool live = i < hi;
        pp[q] = live ? pos_in[i] : -1;
        aj[q] = live && cl == 0 ? A[i * n + j] : make_double2(0.0, 0.0);
        ac[q] = live && cl > 0 && j + cl < p1 ? A[i * n + j + cl] : make_double2(0.0, 0.0);
    }
    Cand c0 = t < ncin ? cin[t] : Cand{-1.0, INT32_MAX, -1};
    const Cand pv = cand_reduce(c0.v, c0.pos, c0.row, sc);
    const bool ok = pv.v > 0.0 && pv.v <= DBL_MAX;
    const int64_t pr = pv.row;
    if (blockIdx.x == 0 && t == 0) {
        piv[j] = pv.pos;
        if (!ok && info[0] == 0) info[0] = int32_t(j + 1);
    }
    const double2 u = j + cl < p1 ? A[pr * n + j + cl] : make_double2(0.0, 0.0);
    const double2 piv_v = A[pr * n + j];
    double bv = -1.0;
    int32_t bpos = INT32_MAX, brow = -1;
    for (int64_t i0 = lo, q = 0; i0 < hi; i0 += 8, ++q) {
        const int64_t i = i0 + r;
        const bool live = i < hi;
        int32_t p;
        double2 a0, a1;
        if (q < kStepPre) {
            // (q is uniform: the loop runs alike in every lane)
            p = pp[0];
            a0 = aj[0];
            a1 = ac[0];
#pragma unroll
            for (int k = 1; k < kStepPre; ++k)
                if (q == k) {
                    p = pp[k];
                    a0 = aj[k];
                    a1 = ac[k];
                }
        } else {
            p = live ? pos_in[i] : -1;
            a0 = live && cl == 0 ? A[i * n + j] : make_double2(0.0, 0.0);
            a1 = live && cl > 0 && j + cl < p1 ? A[i * n + j + cl] : make_double2(0.0, 0.0);
        }
        const bool upd = live && p >= j && i != pr;
        const int32_t np = i == pr ? int32_t(j) : (p == j ? pv.pos : p);
        if (live && cl == 0) pos_out[i] = np;
        // the multiplier, formed by lane 0 of the row's 32 and shared in the
        // wave (rows never straddle a wave)
        double2 l = make_double2(0.0, 0.0);
        if (upd && cl == 0) l = cdiv(a0, piv_v);
        l.x = __shfl(l.x, (t & 63) & ~31, 64);
        l.y = __shfl(l.y, (t & 63) & ~31, 64);
        if (!upd) continue;
        if (cl == 0) {
            A[i * n + j] = l;
        } else if (j + cl < p1) {
            const double2 v = cfma(make_double2(-l.x, -l.y), u, a1);
            A[i * n + j + cl] = v;
            if (cl == 1) {
                double m = fabs(v.x) + fabs(v.y);
                if (!(m <= DBL_MAX)) m = __builtin_inf();
                if (cand_before(m, np, bv, bpos)) {
                    bv = m;
                    bpos = np;
                    brow = int32_t(i);
                }
            }
        }
    }
    if (j + 1 >= p1) return;
    const Cand b = cand_reduce(bv, bpos, brow, sc2);
    if (t == 0) cout[blockIdx.x] = b;
}

// The panel's interchanges, rows j and piv[j] for j = p0 .. p1 - 1 in order,
// over every column of the factors (thread c < n: column c) and every
// right-hand side (thread n + k: right-hand side k).
__global__ __launch_bounds__(256) void gepp_swap_kernel(int64_t n, int64_t p0, int64_t p1,
                                                        double2 *__restrict__ A, int64_t nrhs,
                                                        double2 *__restrict__ X,
                                                        const int32_t *__restrict__ piv)
{
    const int64_t c = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (c < n) {
        for (int64_t j = p0; j < p1; ++j) {
            const int64_t p = piv[j];
            if (p == j) continue;
            const double2 a = A[j * n + c];
            A[j * n + c] = A[p * n + c];
            A[p * n + c] = a;
        }
    } else if (c - n < nrhs) {
        double2 *x = X + (c - n) * n;
        for (int64_t j = p0; j < p1; ++j) {
            const int64_t p = piv[j];
            if (p == j) continue;
            const double2 a = x[j];
            x[j] = x[p];
            x[p] = a;
        }
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
    // pivots, the info word, two candidate sets, two position arrays
    return 3 * align256(sizeof(int32_t) * size_t(n)) + 256 + 2 * align256(sizeof(Cand) * kStepGroups);
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
    const size_t iv = align256(sizeof(int32_t) * size_t(n)), cs = align256(sizeof(Cand) * kStepGroups);
    auto *piv = reinterpret_cast<int32_t *>(p);
    auto *dinfo = reinterpret_cast<int32_t *>(p + iv);
    Cand *cand[2] = {reinterpret_cast<Cand *>(p + iv + 256), reinterpret_cast<Cand *>(p + iv + 256 + cs)};
    int32_t *pos[2] = {reinterpret_cast<int32_t *>(p + iv + 256 + 2 * cs),
                       reinterpret_cast<int32_t *>(p + 2 * iv + 256 + 2 * cs)};
    auto *Xc = reinterpret_cast<double2 *>(X);
    if (X != B)
        MS_HIP(hipMemcpyAsync(X, B, sizeof(double2) * size_t(n) * size_t(nrhs), hipMemcpyDeviceToDevice, s));

    for (int64_t p0 = 0; p0 < n; p0 += kGW) {
        const int w = int(std::min<int64_t>(kGW, n - p0));
        const int64_t p1 = p0 + w;
        // the panel's rows [p0, n) split over G workgroups of R rows
        const int64_t rows = n - p0;
        const int64_t G = std::min<int64_t>(kStepGroups, (rows + 7) / 8);
        const int64_t R = (rows + G - 1) / G;
        hipLaunchKernelGGL(gepp_cand_kernel, dim3(unsigned(G)), dim3(kStepThreads), 0, s, n, p0, R, A, pos[0],
                           cand[0], dinfo);
        for (int64_t j = p0; j < p1; ++j) {
            const int b = int((j - p0) & 1);
            hipLaunchKernelGGL(gepp_step_kernel, dim3(unsigned(G)), dim3(kStepThreads), 0, s, n, j, p0, p1, R, A,
                               pos[b], pos[b ^ 1], cand[b], int(G), cand[b ^ 1], piv, dinfo);
        }
        hipLaunchKernelGGL(gepp_swap_kernel, dim3(grid_of(n + nrhs, 256)), dim3(256), 0, s, n, p0, p1, A, nrhs,
                           Xc, piv);
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
