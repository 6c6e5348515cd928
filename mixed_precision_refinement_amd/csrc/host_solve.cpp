// Host fallback: complex128 LU with partial pivoting and substitution.
//
// The section "Double-precision answers from a GPU without double precision"
// of the page "Solving Dense Matrices Fast in the Browser" sends a frequency
// whose refinement does not converge to a direct solve on the CPU; the
// section "Measure first: the ceiling of JavaScript" describes that solver as
// falling back to LU with partial pivoting.  This is product code: a
// right-looking factorisation in column panels of kPanel with the trailing
// update split over std::thread workers by rows.  It is deliberately not the
// test oracle's code.
#include <algorithm>
#include <cmath>
#include <complex>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

#include "common.hpp"

namespace msolve {
namespace {

using cd = std::complex<double>;
constexpr int64_t kPanel = 32;

// threads for `rows` rows of `width` complex updates each: one per 2^16
// updates, at most the hardware threads (capped at 64)
unsigned worker_count(int64_t rows, int64_t width)
{
    unsigned hw = std::max(1u, std::thread::hardware_concurrency());
    hw = std::min(hw, 64u);
    const int64_t by_work = std::max<int64_t>(1, rows * width / 65536);
    return unsigned(std::min<int64_t>(hw, by_work));
}

template <class F>
void parallel_rows(int64_t lo, int64_t hi, int64_t width, F &&body)
{
    const int64_t rows = hi - lo;
    if (rows <= 0) return;
    const unsigned nw = worker_count(rows, width);
    if (nw <= 1) {
        body(lo, hi);
        return;
    }
    std::vector<std::thread> pool;
    pool.reserve(nw);
    const int64_t chunk = (rows + nw - 1) / nw;
    for (unsigned w = 0; w < nw; ++w) {
        const int64_t a = lo + int64_t(w) * chunk, b = std::min(hi, a + chunk);
        if (a >= b) break;
        pool.emplace_back([&body, a, b] { body(a, b); });
    }
    for (auto &t : pool) t.join();
}

}  // namespace

int host_gepp_solve(int64_t n, int64_t nrhs, const double *Zin, const double *Bin, double *Xout)
{
    std::vector<cd> a(size_t(n) * size_t(n));
    std::memcpy(a.data(), Zin, sizeof(cd) * a.size());
    std::vector<int64_t> perm(n);
    for (int64_t i = 0; i < n; ++i) perm[size_t(i)] = i;
    auto at = [&](int64_t i, int64_t j) -> cd & { return a[size_t(i) * size_t(n) + size_t(j)]; };

    for (int64_t p0 = 0; p0 < n; p0 += kPanel) {
        const int64_t p1 = std::min(n, p0 + kPanel);
        // unblocked factorisation of the column panel [p0, p1), rows p0..n
        for (int64_t k = p0; k < p1; ++k) {
            int64_t piv = k;
            double best = std::abs(at(k, k));
            for (int64_t i = k + 1; i < n; ++i) {
                const double m = std::abs(at(i, k));
                if (m > best) { best = m; piv = i; }
            }
            if (best == 0.0 || !std::isfinite(best)) return MSOLVE_E_FALLBACK;
            if (piv != k) {
                std::swap_ranges(&at(k, 0), &at(k, 0) + n, &at(piv, 0));
                std::swap(perm[size_t(k)], perm[size_t(piv)]);
            }
            const cd inv = 1.0 / at(k, k);
            parallel_rows(k + 1, n, p1 - k, [&](int64_t lo, int64_t hi) {
                for (int64_t i = lo; i < hi; ++i) {
                    const cd l = at(i, k) * inv;
                    at(i, k) = l;
                    for (int64_t j = k + 1; j < p1; ++j) at(i, j) -= l * at(k, j);
                }
            });
        }
        if (p1 >= n) break;
        // U12 = L11^-1 A12 (rows p0..p1, columns p1..n)
        for (int64_t k = p0; k < p1; ++k)
            for (int64_t i = k + 1; i < p1; ++i) {
                const cd l = at(i, k);
                for (int64_t j = p1; j < n; ++j) at(i, j) -= l * at(k, j);
            }
        // A22 -= L21 U12
        parallel_rows(p1, n, (n - p1) * (p1 - p0), [&](int64_t lo, int64_t hi) {
            for (int64_t i = lo; i < hi; ++i) {
                cd *ai = &at(i, 0);
                for (int64_t k = p0; k < p1; ++k) {
                    const cd l = ai[k];
                    const cd *uk = &at(k, 0);
                    for (int64_t j = p1; j < n; ++j) ai[j] -= l * uk[j];
                }
            }
        });
    }

    const cd *B = reinterpret_cast<const cd *>(Bin);
    cd *X = reinterpret_cast<cd *>(Xout);
    std::vector<cd> v(n);
    for (int64_t r = 0; r < nrhs; ++r) {
        for (int64_t i = 0; i < n; ++i) v[size_t(i)] = B[size_t(r) * size_t(n) + size_t(perm[size_t(i)])];
        for (int64_t i = 0; i < n; ++i) {
            cd s = v[size_t(i)];
            for (int64_t j = 0; j < i; ++j) s -= at(i, j) * v[size_t(j)];
            v[size_t(i)] = s;
        }
        for (int64_t i = n - 1; i >= 0; --i) {
            cd s = v[size_t(i)];
            for (int64_t j = i + 1; j < n; ++j) s -= at(i, j) * v[size_t(j)];
            v[size_t(i)] = s / at(i, i);
        }
        std::memcpy(X + size_t(r) * size_t(n), v.data(), sizeof(cd) * size_t(n));
    }
    return MSOLVE_OK;
}

}  // namespace msolve

extern "C" int msolve_host_solve_c128(int64_t n, int64_t nrhs, const double *Z, const double *B,
                                      double *X)
{
    using namespace msolve;
    if (n < 1 || nrhs < 1) return fail(MSOLVE_E_ARG, "msolve_host_solve_c128: n and nrhs must be >= 1");
    if (!Z || !B || !X) return fail(MSOLVE_E_ARG, "msolve_host_solve_c128: null pointer");
    const int st = host_gepp_solve(n, nrhs, Z, B, X);
    if (st != MSOLVE_OK) return fail(st, "msolve_host_solve_c128: matrix is singular (zero pivot)");
    return MSOLVE_OK;
}
