/*
 * CPU oracle for repeated solves of Z(w) x = b -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * load this code.  It shares no source, header, helper or table with the GPU
 * library and never calls it.  Everything is plain float64 / complex128
 * arithmetic written out from the definitions, deliberately slow and simple:
 * no blocking, no reordering beyond what each definition states.
 *
 * Complex numbers are stored interleaved (re, im) in row-major order; a
 * complex matrix of order n is 2*n*n doubles.  Right-hand sides and
 * solutions are stored as rows (nrhs x n).
 *
 * Sources (the page "Solving Dense Matrices Fast in the Browser -- Adaptive
 * Frequency Sampling and Mixed Precision on WebGPU"):
 *   - the model equation Z(w) = jwL - jPsi/w + Zs(w)G, section "Fewer
 *     frequency points: adaptive frequency sampling";
 *   - the direct solve that the refined answer must agree with (LU with
 *     partial pivoting on the CPU), sections "Measure first: the ceiling of
 *     JavaScript" and "Double-precision answers from a GPU without double
 *     precision";
 *   - the residual r = b - Z x in double precision, step 3 of the
 *     refinement list in that same section.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared (see build.py).
 * Contraction is off so that every product and sum is rounded on its own,
 * in the order written.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define RE(p, k) ((p)[2 * (size_t)(k)])
#define IM(p, k) ((p)[2 * (size_t)(k) + 1])

/* ------------------------------------------------------------------ */
/* threads                                                             */
/* ------------------------------------------------------------------ */

void orc_set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int orc_get_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------ */
/* complex scalar helpers (textbook definitions)                       */
/* ------------------------------------------------------------------ */

/* Smith's algorithm (R. L. Smith, CACM 5(8), 1962) for (a + jb) / (c + jd). */
static void smith_div(double a, double b, double c, double d, double *er, double *ei)
{
    if (fabs(c) >= fabs(d)) {
        double r = d / c;
        double den = c + d * r;
        *er = (a + b * r) / den;
        *ei = (b - a * r) / den;
    } else {
        double r = c / d;
        double den = c * r + d;
        *er = (a * r + b) / den;
        *ei = (b * r - a) / den;
    }
}

/* ------------------------------------------------------------------ */
/* O2: assembly of Z(w) from L, Psi and g                              */
/* ------------------------------------------------------------------ */

/*
 * Z(w) = j w L - j Psi / w + Zs(w) G, with G = diag(g) and Zs = zr + j zi.
 * L and Psi are real, so off the diagonal Z is purely imaginary:
 *     Im Z_ij = w * L_ij - Psi_ij / w,  Re Z_ij = 0;
 * on the diagonal the G term adds  zr * g_i  to the real part and
 * zi * g_i  to the imaginary part.  Operation order is fixed as written,
 * each operation rounded on its own (IEEE division, no fused multiply-add).
 */
void orc_assemble(int64_t n, double w, double zr, double zi,
                  const double *L, const double *Psi, const double *g, double *Z)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        for (int64_t j = 0; j < n; ++j) {
            size_t k = (size_t)i * (size_t)n + (size_t)j;
            double wl = w * L[k];
            double pw = Psi[k] / w;
            double im = wl - pw;
            double re = 0.0;
            if (i == j) {
                double gi = g[i];
                im = im + zi * gi;
                re = zr * gi;
            }
            RE(Z, k) = re;
            IM(Z, k) = im;
        }
    }
}

/* ------------------------------------------------------------------ */
/* O3 + O4: LU with partial pivoting and the two substitutions         */
/* ------------------------------------------------------------------ */

/*
 * Solves Z X^T = B^T for nrhs right-hand sides (rows of B) by Gaussian
 * elimination with partial pivoting in complex128.
 *   step k: the pivot row is the first i >= k with the largest |a_ik|
 *   (|.| = hypot); swap rows k and p (in A and in every right-hand side);
 *   if the pivot is exactly zero the matrix is singular; divide the column
 *   below the pivot by it; subtract l_ik * (row k) from every row i > k.
 * Then forward substitution with the unit lower factor and back
 * substitution with the upper factor.
 * A (2*n*n doubles) is overwritten with the factors; B is not modified.
 * Returns 0, or k+1 if the pivot of step k was zero.
 */
int orc_gepp_solve(int64_t n, int64_t nrhs, double *A, const double *B, double *X)
{
    double *y = (double *)malloc(sizeof(double) * 2 * (size_t)n * (size_t)(nrhs > 0 ? nrhs : 1));
    if (!y) return -1;
    memcpy(y, B, sizeof(double) * 2 * (size_t)n * (size_t)nrhs);

    for (int64_t k = 0; k < n; ++k) {
        /* pivot search: first index of the largest modulus */
        int64_t p = k;
        double best = -1.0;
        for (int64_t i = k; i < n; ++i) {
            size_t ik = (size_t)i * n + k;
            double m = hypot(RE(A, ik), IM(A, ik));
            if (m > best) { best = m; p = i; }
        }
        if (p != k) {
            for (int64_t j = 0; j < n; ++j) {
                size_t a = (size_t)k * n + j, b = (size_t)p * n + j;
                double tr = RE(A, a), ti = IM(A, a);
                RE(A, a) = RE(A, b); IM(A, a) = IM(A, b);
                RE(A, b) = tr;       IM(A, b) = ti;
            }
            for (int64_t r = 0; r < nrhs; ++r) {
                size_t a = (size_t)r * n + k, b = (size_t)r * n + p;
                double tr = RE(y, a), ti = IM(y, a);
                RE(y, a) = RE(y, b); IM(y, a) = IM(y, b);
                RE(y, b) = tr;       IM(y, b) = ti;
            }
        }
        size_t kk = (size_t)k * n + k;
        double pr = RE(A, kk), pi = IM(A, kk);
        if (pr == 0.0 && pi == 0.0) { free(y); return (int)(k + 1); }

        /* multipliers l_ik = a_ik / a_kk, then the rank-one update */
        #pragma omp parallel for schedule(static)
        for (int64_t i = k + 1; i < n; ++i) {
            size_t ik = (size_t)i * n + k;
            double lr, li;
            smith_div(RE(A, ik), IM(A, ik), pr, pi, &lr, &li);
            RE(A, ik) = lr; IM(A, ik) = li;
            double *ai = A + 2 * (size_t)i * n;
            const double *ak = A + 2 * (size_t)k * n;
            for (int64_t j = k + 1; j < n; ++j) {
                double ur = ak[2 * j], ui = ak[2 * j + 1];
                double mr = lr * ur - li * ui;
                double mi = lr * ui + li * ur;
                ai[2 * j] = ai[2 * j] - mr;
                ai[2 * j + 1] = ai[2 * j + 1] - mi;
            }
        }
    }

    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nrhs; ++r) {
        double *v = y + 2 * (size_t)r * n;
        /* forward: L v = P b, unit diagonal */
        for (int64_t i = 0; i < n; ++i) {
            double sr = v[2 * i], si = v[2 * i + 1];
            const double *ai = A + 2 * (size_t)i * n;
            for (int64_t j = 0; j < i; ++j) {
                double ar = ai[2 * j], aim = ai[2 * j + 1];
                double vr = v[2 * j], vi = v[2 * j + 1];
                sr = sr - (ar * vr - aim * vi);
                si = si - (ar * vi + aim * vr);
            }
            v[2 * i] = sr; v[2 * i + 1] = si;
        }
        /* back: U x = v */
        for (int64_t i = n - 1; i >= 0; --i) {
            double sr = v[2 * i], si = v[2 * i + 1];
            const double *ai = A + 2 * (size_t)i * n;
            for (int64_t j = i + 1; j < n; ++j) {
                double ar = ai[2 * j], aim = ai[2 * j + 1];
                double vr = v[2 * j], vi = v[2 * j + 1];
                sr = sr - (ar * vr - aim * vi);
                si = si - (ar * vi + aim * vr);
            }
            double xr, xi;
            smith_div(sr, si, ai[2 * i], ai[2 * i + 1], &xr, &xi);
            v[2 * i] = xr; v[2 * i + 1] = xi;
        }
    }
    memcpy(X, y, sizeof(double) * 2 * (size_t)n * (size_t)nrhs);
    free(y);
    return 0;
}

/* ------------------------------------------------------------------ */
/* LU without pivoting: what step 1 of the refinement list factorises  */
/* ------------------------------------------------------------------ */

/*
 * Doolittle elimination without row exchanges, in complex128, in place:
 * on return the strict lower triangle of A holds the unit lower factor L
 * and the upper triangle holds U, with A = L U.  Returns 0, or k+1 if the
 * pivot of step k was exactly zero (A is then partially factorised).
 */
int orc_lu_nopivot(int64_t n, double *A)
{
    for (int64_t k = 0; k < n; ++k) {
        size_t kk = (size_t)k * n + k;
        double pr = RE(A, kk), pi = IM(A, kk);
        if (pr == 0.0 && pi == 0.0) return (int)(k + 1);
        #pragma omp parallel for schedule(static)
        for (int64_t i = k + 1; i < n; ++i) {
            size_t ik = (size_t)i * n + k;
            double lr, li;
            smith_div(RE(A, ik), IM(A, ik), pr, pi, &lr, &li);
            RE(A, ik) = lr; IM(A, ik) = li;
            double *ai = A + 2 * (size_t)i * n;
            const double *ak = A + 2 * (size_t)k * n;
            for (int64_t j = k + 1; j < n; ++j) {
                double ur = ak[2 * j], ui = ak[2 * j + 1];
                ai[2 * j] = ai[2 * j] - (lr * ur - li * ui);
                ai[2 * j + 1] = ai[2 * j + 1] - (lr * ui + li * ur);
            }
        }
    }
    return 0;
}

/*
 * Given packed factors L\U (unit lower L strictly below the diagonal, U on
 * and above it), solve L U x = b for each row of B by forward then back
 * substitution, in complex128.  Steps 2 and 4 of the refinement list apply
 * exactly this solve with the single-precision factors.
 */
void orc_lu_solve(int64_t n, int64_t nrhs, const double *LU, const double *B, double *X)
{
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nrhs; ++r) {
        double *v = X + 2 * (size_t)r * n;
        memcpy(v, B + 2 * (size_t)r * n, sizeof(double) * 2 * (size_t)n);
        for (int64_t i = 0; i < n; ++i) {
            double sr = v[2 * i], si = v[2 * i + 1];
            const double *ai = LU + 2 * (size_t)i * n;
            for (int64_t j = 0; j < i; ++j) {
                sr = sr - (ai[2 * j] * v[2 * j] - ai[2 * j + 1] * v[2 * j + 1]);
                si = si - (ai[2 * j] * v[2 * j + 1] + ai[2 * j + 1] * v[2 * j]);
            }
            v[2 * i] = sr; v[2 * i + 1] = si;
        }
        for (int64_t i = n - 1; i >= 0; --i) {
            double sr = v[2 * i], si = v[2 * i + 1];
            const double *ai = LU + 2 * (size_t)i * n;
            for (int64_t j = i + 1; j < n; ++j) {
                sr = sr - (ai[2 * j] * v[2 * j] - ai[2 * j + 1] * v[2 * j + 1]);
                si = si - (ai[2 * j] * v[2 * j + 1] + ai[2 * j + 1] * v[2 * j]);
            }
            double xr, xi;
            smith_div(sr, si, ai[2 * i], ai[2 * i + 1], &xr, &xi);
            v[2 * i] = xr; v[2 * i + 1] = xi;
        }
    }
}

/* ------------------------------------------------------------------ */
/* residual r = b - Z x, compensated (Ogita, Rump, Oishi 2005, Dot2)   */
/* ------------------------------------------------------------------ */

/* error-free transformations (Knuth's TwoSum; TwoProduct via fma) */
static void two_sum(double a, double b, double *s, double *e)
{
    double x = a + b;
    double z = x - a;
    *e = (a - (x - z)) + (b - z);
    *s = x;
}

static void two_prod(double a, double b, double *p, double *e)
{
    double x = a * b;
    *e = fma(a, b, -x);
    *p = x;
}

/* accumulate a*b into the compensated pair (s, c) */
static void dot2_acc(double *s, double *c, double a, double b)
{
    double p, ep, t, es;
    two_prod(a, b, &p, &ep);
    two_sum(*s, p, &t, &es);
    *s = t;
    *c = *c + (ep + es);
}

/*
 * R = B - Z X for each row of X / B, every component evaluated as if in
 * twice the working precision and rounded once at the end (Dot2).
 *   Re r_i = Re b_i - sum_j (Re z_ij Re x_j - Im z_ij Im x_j)
 *   Im r_i = Im b_i - sum_j (Re z_ij Im x_j + Im z_ij Re x_j)
 */
void orc_residual(int64_t n, int64_t nrhs, const double *Z, const double *X,
                  const double *B, double *R)
{
    #pragma omp parallel for schedule(static) collapse(2)
    for (int64_t r = 0; r < nrhs; ++r) {
        for (int64_t i = 0; i < n; ++i) {
            const double *zi = Z + 2 * (size_t)i * n;
            const double *x = X + 2 * (size_t)r * n;
            double sr = RE(B, (size_t)r * n + i), cr = 0.0;
            double si = IM(B, (size_t)r * n + i), ci = 0.0;
            for (int64_t j = 0; j < n; ++j) {
                double a = zi[2 * j], b = zi[2 * j + 1];
                double xr = x[2 * j], xi = x[2 * j + 1];
                dot2_acc(&sr, &cr, -a, xr);
                dot2_acc(&sr, &cr, b, xi);
                dot2_acc(&si, &ci, -a, xi);
                dot2_acc(&si, &ci, -b, xr);
            }
            RE(R, (size_t)r * n + i) = sr + cr;
            IM(R, (size_t)r * n + i) = si + ci;
        }
    }
}

/* ------------------------------------------------------------------ */
/* norms                                                               */
/* ------------------------------------------------------------------ */

/* ||Z||_inf = max_i sum_j |z_ij|, |.| = hypot */
double orc_norm_inf_mat(int64_t n, const double *Z)
{
    double best = 0.0;
    #pragma omp parallel for schedule(static) reduction(max : best)
    for (int64_t i = 0; i < n; ++i) {
        double s = 0.0;
        for (int64_t j = 0; j < n; ++j) {
            size_t k = (size_t)i * n + j;
            s = s + hypot(RE(Z, k), IM(Z, k));
        }
        if (s > best) best = s;
    }
    return best;
}

/* ||v||_inf = max_i |v_i| for a complex vector of length n */
double orc_norm_inf_vec(int64_t n, const double *v)
{
    double best = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double m = hypot(RE(v, i), IM(v, i));
        if (m > best) best = m;
    }
    return best;
}
