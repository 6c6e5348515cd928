// Reduced-order frequency sweep (page "Solving Dense Matrices Fast in the
// Browser", section "Fewer frequency points: adaptive frequency sampling").
//
// Exact solves at a few frequencies give a real orthonormal basis V (the real
// and imaginary parts of the solutions).  On it, Z(w) = jwL - jPsi/w +
// Zs(w)G reduces to the q x q symmetric Z_r(w) = jw V^T L V - j V^T Psi V / w
// + Zs V^T G V, solved at every candidate frequency; the residual
// ||Z(w) V y - b|| of each candidate picks the next exact solve, until every
// candidate is below the tolerance.
//
// On the device: the exact solves (msolve_sweep), the products L V, Psi V
// and G V (afs_project_kernel: L and Psi streamed once per batch of new
// basis vectors), every inner product the reduced systems and the residuals
// need (afs_gram_kernel) and the answers x = V y (afs_reconstruct_kernel).
// On the host: the orthonormalisation of each new solution against the
// basis (q x n work per vector) and the q x q systems (one per candidate,
// spread over host threads).
//
// The residual needs no product with Z: with A = L V, P = Psi V, Q = G V and
// M = jw A - j P / w + Zs Q (so that Z V = M),
//   ||M y - b||^2 = y^H (M^H M) y - 2 Re(y^H M^H b) + ||b||^2,
// and M^H M, M^H b are sums of the Gram blocks A^T A, A^T P, ..., A^T b with
// scalar weights.
#include <algorithm>
#include <cmath>
#include <complex>
#include <thread>
#include <vector>

#include "common.hpp"

namespace msolve {
namespace {

constexpr int kProjRows = 2;     // rows of L and Psi per wave
constexpr int kProjCols = 8;     // basis vectors per launch
constexpr int kGramTile = 16;
constexpr int kGramChunk = 64;
constexpr double kDropTol = 1e-10;

// For rows r of L and Psi: W[rowA + c][r] = (L v_c)_r, W[rowP + c][r] =
// (Psi v_c)_r, W[rowQ + c][r] = g_r (v_c)_r, with v_c = W[v0 + c] (c < nc).
// One wave per kProjRows rows; lanes stride the columns (coalesced rows of
// L and Psi), the nc basis values of a column are loaded once for the rows.
__global__ __launch_bounds__(256) void afs_project_kernel(int64_t n, const double *L, const double *Psi,
                                                          const double *g, double *W, int64_t v0, int nc,
                                                          int64_t rowA, int64_t rowP, int64_t rowQ)
{
    const int lane = threadIdx.x & 63;
    const int64_t r0 = (int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6)) * kProjRows;
    if (r0 >= n) return;
    double a[kProjRows][kProjCols], p[kProjRows][kProjCols];
#pragma unroll
    for (int i = 0; i < kProjRows; ++i)
#pragma unroll
        for (int c = 0; c < kProjCols; ++c) {
            a[i][c] = 0.0;
            p[i][c] = 0.0;
        }
    const double *V = W + size_t(v0) * size_t(n);
    for (int64_t j = lane; j < n; j += 64) {
        double v[kProjCols];
#pragma unroll
        for (int c = 0; c < kProjCols; ++c) v[c] = c < nc ? V[size_t(c) * size_t(n) + size_t(j)] : 0.0;
#pragma unroll
        for (int i = 0; i < kProjRows; ++i) {
            const int64_t r = min<int64_t>(r0 + i, n - 1);
            const double l = L[size_t(r) * size_t(n) + size_t(j)];
            const double s = Psi[size_t(r) * size_t(n) + size_t(j)];
#pragma unroll
            for (int c = 0; c < kProjCols; ++c) {
                a[i][c] = fma(l, v[c], a[i][c]);
                p[i][c] = fma(s, v[c], p[i][c]);
            }
        }
    }
    // wave sums, in a fixed order
#pragma unroll
    for (int i = 0; i < kProjRows; ++i)
#pragma unroll
        for (int c = 0; c < kProjCols; ++c)
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) {
                a[i][c] += __shfl_xor(a[i][c], off);
                p[i][c] += __shfl_xor(p[i][c], off);
            }
    if (lane == 0) {
#pragma unroll
        for (int i = 0; i < kProjRows; ++i) {
            const int64_t r = r0 + i;
            if (r >= n) break;
#pragma unroll
            for (int c = 0; c < kProjCols; ++c) {
                if (c >= nc) break;
                W[size_t(rowA + c) * size_t(n) + size_t(r)] = a[i][c];
                W[size_t(rowP + c) * size_t(n) + size_t(r)] = p[i][c];
                W[size_t(rowQ + c) * size_t(n) + size_t(r)] = g[r] * V[size_t(c) * size_t(n) + size_t(r)];
            }
        }
    }
}

// Partial Gram sums: part[z][a][b] = sum over k in slice z of W[idx[a]][k]
// W[idx[b]][k] for the tile pair (blockIdx.x, blockIdx.y) with a <= b
// tiles (the lower tiles are left out).  Slices split [0, n) evenly.
__global__ __launch_bounds__(kGramTile *kGramTile) void afs_gram_kernel(int64_t n, const double *W,
                                                                         const int32_t *idx, int m,
                                                                         int slices, double *part)
{
    if (blockIdx.x > blockIdx.y) return;
    __shared__ double Ra[kGramTile][kGramChunk + 1];
    __shared__ double Rb[kGramTile][kGramChunk + 1];
    const int ta = threadIdx.x / kGramTile, tb = threadIdx.x % kGramTile;
    const int a0 = blockIdx.x * kGramTile, b0 = blockIdx.y * kGramTile;
    const int64_t per = (n + slices - 1) / slices;
    const int64_t k0 = int64_t(blockIdx.z) * per, k1 = min<int64_t>(n, k0 + per);
    double acc = 0.0;
    for (int64_t kc = k0; kc < k1; kc += kGramChunk) {
        for (int e = threadIdx.x; e < kGramTile * kGramChunk; e += kGramTile * kGramTile) {
            const int i = e / kGramChunk, k = e % kGramChunk;
            const bool kin = kc + k < k1;
            Ra[i][k] = kin && a0 + i < m ? W[size_t(idx[a0 + i]) * size_t(n) + size_t(kc + k)] : 0.0;
            Rb[i][k] = kin && b0 + i < m ? W[size_t(idx[b0 + i]) * size_t(n) + size_t(kc + k)] : 0.0;
        }
        __syncthreads();
#pragma unroll 8
        for (int k = 0; k < kGramChunk; ++k) acc = fma(Ra[ta][k], Rb[tb][k], acc);
        __syncthreads();
    }
    const int a = a0 + ta, b = b0 + tb;
    if (a < m && b < m) part[(size_t(blockIdx.z) * size_t(m) + size_t(a)) * size_t(m) + size_t(b)] = acc;
}

// G[a][b] = G[b][a] = sum of the slices in order (a <= b)
__global__ __launch_bounds__(256) void afs_gram_sum_kernel(int m, int slices, const double *part, double *G)
{
    const int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (e >= int64_t(m) * m) return;
    const int a = int(e / m), b = int(e % m);
    if (a > b) return;
    double s = 0.0;
    for (int z = 0; z < slices; ++z) s += part[(size_t(z) * size_t(m) + size_t(a)) * size_t(m) + size_t(b)];
    G[size_t(a) * size_t(m) + size_t(b)] = s;
    G[size_t(b) * size_t(m) + size_t(a)] = s;
}

// X[s][i] = sum_c V[c][i] y[s][c] (complex y, s = frequency * nrhs + rhs)
__global__ __launch_bounds__(256) void afs_reconstruct_kernel(int64_t n, int q, const double *V,
                                                              const double *Y, int64_t ystride, double *X)
{
    extern __shared__ double ys[];         // 2 q doubles
    const int64_t s = blockIdx.y;
    for (int c = threadIdx.x; c < 2 * q; c += 256) ys[c] = Y[size_t(s) * size_t(ystride) + size_t(c)];
    __syncthreads();
    const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (i >= n) return;
    double re = 0.0, im = 0.0;
    for (int c = 0; c < q; ++c) {
        const double v = V[size_t(c) * size_t(n) + size_t(i)];
        re = fma(v, ys[2 * c], re);
        im = fma(v, ys[2 * c + 1], im);
    }
    X[(size_t(s) * size_t(n) + size_t(i)) * 2] = re;
    X[(size_t(s) * size_t(n) + size_t(i)) * 2 + 1] = im;
}

struct AfsLayout {
    int64_t qmax, mmax, slices, nexact_batch;
    size_t sweep, xe, w, idx, part, g, y, total;
};

AfsLayout afs_layout(int64_t n, int64_t nrhs, int64_t nfreq, int64_t max_exact)
{
    AfsLayout l;
    l.nexact_batch = std::min<int64_t>(2, nfreq);
    l.qmax = 2 * nrhs * max_exact;
    l.mmax = 4 * l.qmax + 2 * nrhs;
    // K slices of the Gram sums: up to 16, with at most 2^22 partial entries
    l.slices = std::max<int64_t>(1, std::min<int64_t>(16, (int64_t(1) << 22) / (l.mmax * l.mmax)));
    size_t off = 0;
    l.sweep = off; off += align256(msolve_sweep_workspace_bytes(n, nrhs, l.nexact_batch));
    l.xe = off;    off += align256(size_t(16) * size_t(l.nexact_batch * nrhs) * size_t(n));
    l.w = off;     off += align256(sizeof(double) * size_t(l.mmax) * size_t(n));
    l.idx = off;   off += align256(sizeof(int32_t) * size_t(l.mmax));
    l.part = off;  off += align256(sizeof(double) * size_t(l.slices) * size_t(l.mmax * l.mmax));
    l.g = off;     off += align256(sizeof(double) * size_t(l.mmax * l.mmax));
    l.y = off;     off += align256(size_t(16) * size_t(nfreq * nrhs) * size_t(l.qmax));
    l.total = off;
    return l;
}

using cplx = std::complex<double>;

// Z y = b for nb right-hand sides (rows of B, overwritten by y) with the
// q x q matrix Z (overwritten): Gaussian elimination with partial pivoting
// by modulus, complex128.  Returns false on an exactly zero pivot.
bool small_solve(int64_t q, int64_t nb, cplx *Z, cplx *B)
{
    const size_t uq = size_t(q);
    for (int64_t k = 0; k < q; ++k) {
        int64_t p = k;
        for (int64_t i = k + 1; i < q; ++i)
            if (std::abs(Z[size_t(i) * uq + size_t(k)]) > std::abs(Z[size_t(p) * uq + size_t(k)])) p = i;
        if (Z[size_t(p) * uq + size_t(k)] == cplx(0.0, 0.0)) return false;
        if (p != k) {
            for (int64_t j = 0; j < q; ++j) std::swap(Z[size_t(k) * uq + size_t(j)], Z[size_t(p) * uq + size_t(j)]);
            for (int64_t r = 0; r < nb; ++r) std::swap(B[size_t(r) * uq + size_t(k)], B[size_t(r) * uq + size_t(p)]);
        }
        const cplx inv = 1.0 / Z[size_t(k) * uq + size_t(k)];
        for (int64_t i = k + 1; i < q; ++i) {
            const cplx l = Z[size_t(i) * uq + size_t(k)] * inv;
            if (l == cplx(0.0, 0.0)) continue;
            for (int64_t j = k + 1; j < q; ++j) Z[size_t(i) * uq + size_t(j)] -= l * Z[size_t(k) * uq + size_t(j)];
            for (int64_t r = 0; r < nb; ++r) B[size_t(r) * uq + size_t(i)] -= l * B[size_t(r) * uq + size_t(k)];
        }
    }
    for (int64_t r = 0; r < nb; ++r) {
        cplx *y = B + size_t(r) * uq;
        for (int64_t i = q - 1; i >= 0; --i) {
            cplx sacc = y[i];
            for (int64_t j = i + 1; j < q; ++j) sacc -= Z[size_t(i) * uq + size_t(j)] * y[j];
            y[i] = sacc / Z[size_t(i) * uq + size_t(i)];
        }
    }
    return true;
}

}  // namespace
}  // namespace msolve

using namespace msolve;

extern "C" size_t msolve_afs_workspace_bytes(int64_t n, int64_t nrhs, int64_t nfreq, int32_t max_exact)
{
    if (n < 1 || nrhs < 1 || nfreq < 1 || max_exact < 1) return 0;
    return afs_layout(n, nrhs, nfreq, std::min<int64_t>(max_exact, nfreq)).total;
}

extern "C" int msolve_afs(int64_t n, int64_t nfreq, const double *omega, const double *zs, const double *L,
                          const double *Psi, const double *g, int64_t nrhs, const double *B, double *X,
                          double tol, int32_t max_exact, double solve_tol, int32_t solve_max_iter,
                          int32_t *exact, int32_t *n_exact, double *estimate, int32_t *q_out, void *work,
                          size_t work_bytes, void *stream)
{
    if (n < 1 || nrhs < 1 || nfreq < 0 || max_exact < 1) return fail(MSOLVE_E_ARG, "msolve_afs: bad sizes");
    if (!omega || !zs || !L || !Psi || !g || !B || !X || !exact || !n_exact || !estimate || !q_out || !work)
        return fail(MSOLVE_E_ARG, "msolve_afs: null pointer");
    if (!(tol >= 0.0) || !(solve_tol >= 0.0) || solve_max_iter < 0)
        return fail(MSOLVE_E_ARG, "msolve_afs: tol, solve_tol >= 0 and solve_max_iter >= 0 required");
    for (int64_t f = 0; f < nfreq; ++f)
        if (!std::isfinite(omega[f]) || omega[f] == 0.0)
            return fail(MSOLVE_E_ARG, "msolve_afs: every omega must be finite and nonzero");
    if (nfreq * nrhs > 65535) return fail(MSOLVE_E_ARG, "msolve_afs: nfreq * nrhs must be <= 65535");
    *n_exact = 0;
    *q_out = 0;
    if (nfreq == 0) return MSOLVE_OK;
    const int64_t cap = std::min<int64_t>(max_exact, nfreq);
    if (work_bytes < msolve_afs_workspace_bytes(n, nrhs, nfreq, int32_t(cap)))
        return fail(MSOLVE_E_WORKSPACE, "msolve_afs: workspace too small");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const AfsLayout lay = afs_layout(n, nrhs, nfreq, cap);
    char *w = static_cast<char *>(work);
    double *Xe = reinterpret_cast<double *>(w + lay.xe);
    double *Wd = reinterpret_cast<double *>(w + lay.w);
    int32_t *idx_d = reinterpret_cast<int32_t *>(w + lay.idx);
    double *part = reinterpret_cast<double *>(w + lay.part);
    double *Gd = reinterpret_cast<double *>(w + lay.g);
    double *Yd = reinterpret_cast<double *>(w + lay.y);
    const size_t un = size_t(n);
    const int64_t qmax = lay.qmax;
    // rows of W: V at [0, qmax), L V at [qmax, 2 qmax), Psi V at [2 qmax, 3
    // qmax), G V at [3 qmax, 4 qmax), then Re b and Im b of each right-hand side
    const int64_t rowA = qmax, rowP = 2 * qmax, rowQ = 3 * qmax, rowB = 4 * qmax;

    // right-hand sides: their real and imaginary parts as rows of W, and norms
    std::vector<double> Bh(size_t(2 * nrhs) * un), parts(size_t(2 * nrhs) * un);
    MS_HIP(hipMemcpyAsync(Bh.data(), B, Bh.size() * sizeof(double), hipMemcpyDeviceToHost, s));
    MS_HIP(hipStreamSynchronize(s));
    std::vector<double> bnorm2(size_t(nrhs), 0.0);
    for (int64_t k = 0; k < nrhs; ++k)
        for (size_t i = 0; i < un; ++i) {
            const double re = Bh[(size_t(k) * un + i) * 2], im = Bh[(size_t(k) * un + i) * 2 + 1];
            parts[size_t(k) * un + i] = re;
            parts[size_t(nrhs + k) * un + i] = im;
            bnorm2[size_t(k)] += re * re + im * im;
        }
    for (int64_t k = 0; k < nrhs; ++k)
        if (!(bnorm2[size_t(k)] > 0.0) || !std::isfinite(bnorm2[size_t(k)]))
            return fail(MSOLVE_E_ARG, "msolve_afs: every right-hand side must be nonzero and finite");
    MS_HIP(hipMemcpyAsync(Wd + size_t(rowB) * un, parts.data(), parts.size() * sizeof(double),
                          hipMemcpyHostToDevice, s));

    std::vector<double> Vh;                // host copy of the basis rows
    int64_t q = 0;
    std::vector<int32_t> chosen;
    chosen.push_back(0);
    if (nfreq > 1 && cap > 1) chosen.push_back(int32_t(nfreq - 1));
    std::vector<int32_t> fresh = chosen;
    std::vector<double> est(size_t(nfreq), 0.0);
    std::vector<cplx> Y(size_t(nfreq * nrhs) * size_t(qmax));
    std::vector<double> xh(size_t(2 * lay.nexact_batch * nrhs) * un), u(un);
    std::vector<msolve_freq_info> finfo(size_t(lay.nexact_batch));

    while (true) {
        // 1. exact solves of the new frequencies, then their real and
        //    imaginary parts join the basis (two passes of modified
        //    Gram-Schmidt; a part with less than kDropTol of its norm left
        //    adds nothing)
        const int64_t k = int64_t(fresh.size());
        std::vector<double> om(static_cast<size_t>(k)), zz(static_cast<size_t>(2 * k));
        for (int64_t i = 0; i < k; ++i) {
            om[size_t(i)] = omega[fresh[size_t(i)]];
            zz[size_t(2 * i)] = zs[2 * fresh[size_t(i)]];
            zz[size_t(2 * i + 1)] = zs[2 * fresh[size_t(i)] + 1];
        }
        MS_TRY(msolve_sweep(n, k, om.data(), zz.data(), L, Psi, g, nrhs, B, Xe, solve_tol, solve_max_iter,
                            w + lay.sweep, lay.xe - lay.sweep, finfo.data(), nullptr, stream));
        for (int64_t i = 0; i < k; ++i)
            if (finfo[size_t(i)].status != 0)
                return fail(finfo[size_t(i)].status, "msolve_afs: an exact solve failed");
        MS_HIP(hipMemcpyAsync(xh.data(), Xe, size_t(2 * k * nrhs) * un * sizeof(double), hipMemcpyDeviceToHost, s));
        MS_HIP(hipStreamSynchronize(s));
        const int64_t q_old = q;
        for (int64_t sidx = 0; sidx < k * nrhs; ++sidx)
            for (int part_i = 0; part_i < 2; ++part_i) {
                double n0 = 0.0;
                for (size_t i = 0; i < un; ++i) {
                    u[i] = xh[(size_t(sidx) * un + i) * 2 + size_t(part_i)];
                    n0 += u[i] * u[i];
                }
                n0 = std::sqrt(n0);
                if (n0 == 0.0) continue;
                for (int pass = 0; pass < 2; ++pass)
                    for (int64_t c = 0; c < q; ++c) {
                        const double *v = Vh.data() + size_t(c) * un;
                        double d = 0.0;
                        for (size_t i = 0; i < un; ++i) d += v[i] * u[i];
                        for (size_t i = 0; i < un; ++i) u[i] -= d * v[i];
                    }
                double nu = 0.0;
                for (size_t i = 0; i < un; ++i) nu += u[i] * u[i];
                nu = std::sqrt(nu);
                if (!(nu > kDropTol * n0)) continue;
                if (q >= qmax) return fail(MSOLVE_E_ARG, "msolve_afs: basis larger than its workspace");
                for (size_t i = 0; i < un; ++i) Vh.push_back(u[i] / nu);
                ++q;
            }
        // 2. the new basis rows go to the device; L V, Psi V and G V for them
        if (q > q_old) {
            MS_HIP(hipMemcpyAsync(Wd + size_t(q_old) * un, Vh.data() + size_t(q_old) * un,
                                  size_t(q - q_old) * un * sizeof(double), hipMemcpyHostToDevice, s));
            for (int64_t c0 = q_old; c0 < q; c0 += kProjCols) {
                const int nc = int(std::min<int64_t>(kProjCols, q - c0));
                ProfScope prof(MSOLVE_K_AFS_PROJECT, s, 16.0 * double(n) * double(n));
                const int64_t waves = (n + kProjRows - 1) / kProjRows;
                hipLaunchKernelGGL(afs_project_kernel, dim3(unsigned((waves + 3) / 4)), dim3(256), 0, s, n, L,
                                   Psi, g, Wd, c0, nc, rowA + c0, rowP + c0, rowQ + c0);
                MS_HIP(hipGetLastError());
            }
        }
        // 3. every inner product among V, L V, Psi V, G V, Re b, Im b
        const int64_t m = 4 * q + 2 * nrhs;
        std::vector<int32_t> idx(static_cast<size_t>(m));
        for (int64_t c = 0; c < q; ++c) {
            idx[size_t(c)] = int32_t(c);
            idx[size_t(q + c)] = int32_t(rowA + c);
            idx[size_t(2 * q + c)] = int32_t(rowP + c);
            idx[size_t(3 * q + c)] = int32_t(rowQ + c);
        }
        for (int64_t r = 0; r < 2 * nrhs; ++r) idx[size_t(4 * q + r)] = int32_t(rowB + r);
        MS_HIP(hipMemcpyAsync(idx_d, idx.data(), idx.size() * sizeof(int32_t), hipMemcpyHostToDevice, s));
        const int slices = int(std::max<int64_t>(1, std::min<int64_t>(lay.slices, (n + kGramChunk - 1) / kGramChunk)));
        const unsigned tiles = unsigned((m + kGramTile - 1) / kGramTile);
        hipLaunchKernelGGL(afs_gram_kernel, dim3(tiles, tiles, unsigned(slices)), dim3(kGramTile * kGramTile), 0,
                           s, n, Wd, idx_d, int(m), slices, part);
        MS_HIP(hipGetLastError());
        hipLaunchKernelGGL(afs_gram_sum_kernel, dim3(unsigned((m * m + 255) / 256)), dim3(256), 0, s, int(m),
                           slices, part, Gd);
        MS_HIP(hipGetLastError());
        std::vector<double> G(static_cast<size_t>(m * m));
        MS_HIP(hipMemcpyAsync(G.data(), Gd, G.size() * sizeof(double), hipMemcpyDeviceToHost, s));
        MS_HIP(hipStreamSynchronize(s));
        auto gm = [&](int64_t a, int64_t b) { return G[size_t(a) * size_t(m) + size_t(b)]; };

        // 4. at every candidate: Z_r y = V^T b, and the residual from the
        //    Gram blocks (blocks a = 1, 2, 3: L V, Psi V, G V).  Candidates
        //    are independent: host threads take every T-th one.
        const size_t uq = size_t(q);
        auto evaluate = [&](int64_t f0, int64_t step) -> int {
            std::vector<cplx> Zr(uq * uq), br(size_t(nrhs) * uq), yk(size_t(nrhs) * uq), MM(uq * uq), t(uq), v(uq);
            for (int64_t f = f0; f < nfreq; f += step) {
                const double wf = omega[f];
                const cplx c[3] = {cplx(0.0, wf), cplx(0.0, -1.0 / wf), cplx(zs[2 * f], zs[2 * f + 1])};
                for (int64_t i = 0; i < q; ++i)
                    for (int64_t j = 0; j < q; ++j)
                        Zr[size_t(i) * uq + size_t(j)] =
                            c[0] * gm(i, q + j) + c[1] * gm(i, 2 * q + j) + c[2] * gm(i, 3 * q + j);
                for (int64_t kk = 0; kk < nrhs; ++kk)
                    for (int64_t i = 0; i < q; ++i)
                        br[size_t(kk) * uq + size_t(i)] = cplx(gm(i, 4 * q + kk), gm(i, 4 * q + nrhs + kk));
                yk = br;
                if (!small_solve(q, nrhs, Zr.data(), yk.data())) return MSOLVE_E_FALLBACK;
                // M^H M (Hermitian), with the weights conj(c_a) c_b
                cplx wgt[3][3];
                for (int a = 0; a < 3; ++a)
                    for (int b = 0; b < 3; ++b) wgt[a][b] = std::conj(c[a]) * c[b];
                for (int64_t i = 0; i < q; ++i)
                    for (int64_t j = 0; j < q; ++j) {
                        cplx sacc = 0.0;
                        for (int a = 0; a < 3; ++a)
                            for (int b = 0; b < 3; ++b) sacc += wgt[a][b] * gm((a + 1) * q + i, (b + 1) * q + j);
                        MM[size_t(i) * uq + size_t(j)] = sacc;
                    }
                double worst = 0.0;
                for (int64_t kk = 0; kk < nrhs; ++kk) {
                    const cplx *y = yk.data() + size_t(kk) * uq;
                    for (int64_t i = 0; i < q; ++i) {
                        cplx sacc = 0.0;
                        for (int a = 0; a < 3; ++a)
                            sacc += std::conj(c[a]) *
                                    cplx(gm((a + 1) * q + i, 4 * q + kk), gm((a + 1) * q + i, 4 * q + nrhs + kk));
                        t[size_t(i)] = sacc;
                        cplx vacc = 0.0;
                        for (int64_t j = 0; j < q; ++j) vacc += MM[size_t(i) * uq + size_t(j)] * y[j];
                        v[size_t(i)] = vacc;
                    }
                    cplx yMy = 0.0, yt = 0.0;
                    for (int64_t i = 0; i < q; ++i) {
                        yMy += std::conj(y[i]) * v[size_t(i)];
                        yt += std::conj(y[i]) * t[size_t(i)];
                    }
                    const double r2 = yMy.real() - 2.0 * yt.real() + bnorm2[size_t(kk)];
                    worst = std::max(worst, std::sqrt(std::max(r2, 0.0) / bnorm2[size_t(kk)]));
                    for (int64_t i = 0; i < q; ++i) Y[(size_t(f * nrhs + kk)) * size_t(qmax) + size_t(i)] = y[i];
                }
                est[size_t(f)] = worst;
            }
            return MSOLVE_OK;
        };
        const int64_t hw = std::max<int64_t>(1, int64_t(std::thread::hardware_concurrency()));
        const int64_t nthr = std::max<int64_t>(1, std::min<int64_t>(std::min<int64_t>(hw, 16), nfreq / 16));
        std::vector<int> sts(static_cast<size_t>(nthr), MSOLVE_OK);
        {
            std::vector<std::thread> pool;
            for (int64_t t0 = 1; t0 < nthr; ++t0)
                pool.emplace_back([&, t0] { sts[size_t(t0)] = evaluate(t0, nthr); });
            sts[0] = evaluate(0, nthr);
            for (auto &th : pool) th.join();
        }
        for (int st : sts)
            if (st != MSOLVE_OK) return fail(st, "msolve_afs: singular reduced system");
        // 5. the next exact solve: the largest estimate among the others
        if (int64_t(chosen.size()) >= cap) break;
        int64_t best = -1;
        for (int64_t f = 0; f < nfreq; ++f) {
            if (std::find(chosen.begin(), chosen.end(), int32_t(f)) != chosen.end()) continue;
            if (best < 0 || est[size_t(f)] > est[size_t(best)]) best = f;
        }
        if (best < 0 || !(est[size_t(best)] > tol)) break;
        chosen.push_back(int32_t(best));
        fresh.assign(1, int32_t(best));
    }

    // x = V y at every candidate
    MS_HIP(hipMemcpyAsync(Yd, Y.data(), Y.size() * sizeof(cplx), hipMemcpyHostToDevice, s));
    hipLaunchKernelGGL(afs_reconstruct_kernel, dim3(unsigned((n + 255) / 256), unsigned(nfreq * nrhs)), dim3(256),
                       size_t(16) * size_t(std::max<int64_t>(q, 1)), s, n, int(q), Wd, Yd, 2 * qmax, X);
    MS_HIP(hipGetLastError());
    MS_HIP(hipStreamSynchronize(s));
    for (size_t i = 0; i < chosen.size(); ++i) exact[i] = chosen[i];
    *n_exact = int32_t(chosen.size());
    for (int64_t f = 0; f < nfreq; ++f) estimate[f] = est[size_t(f)];
    *q_out = int32_t(q);
    return MSOLVE_OK;
}
