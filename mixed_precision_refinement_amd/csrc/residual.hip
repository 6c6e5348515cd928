// Residual r = b - Z x in double precision (step 3 of the refinement list in
// the section "Double-precision answers from a GPU without double precision"
// of the page "Solving Dense Matrices Fast in the Browser").  The page had to
// emulate double precision with pairs of floats; gfx950 has native FP64, so
// this is a plain complex128 matrix-vector product for up to four right-hand
// sides that streams Z once.
//
// Memory bound: 16 n^2 bytes of Z + 48 n nrhs bytes of vectors per call.
// One wave64 per row (four rows per workgroup); lanes stride the row so each
// load instruction covers 1 KiB of contiguous Z.  The sums are reduced across
// the wave in a fixed order, so results are bitwise reproducible.  The
// infinity norms of r and x are folded in with integer atomic max on the bit
// patterns of non-negative doubles (order-independent, hence deterministic).
//
// Also the small vector kernels of the refinement loop (fills, norms).
#include <algorithm>
#include <cmath>

#include "common.hpp"

namespace msolve {
namespace {

constexpr int kMaxRhs = 4;

__device__ inline double wave_sum(double v)
{
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

__device__ inline double wave_max(double v)
{
    for (int off = 32; off > 0; off >>= 1) v = fmax(v, __shfl_xor(v, off, 64));
    return v;
}

__device__ inline void atomic_max_nonneg(uint64_t *slot, double v)
{
    // non-negative doubles (and +NaN, which sorts above +inf) order like
    // their unsigned bit patterns
    atomicMax(reinterpret_cast<unsigned long long *>(slot),
              static_cast<unsigned long long>(__double_as_longlong(v)));
}

__device__ inline double cabs(double re, double im) { return hypot(re, im); }

// A load of matrix data that is read once per launch, marked nontemporal so
// that it does not displace the vectors every workgroup re-reads from L2
// (measured at n = 8000: 5.4 -> 5.8 TB/s).
__device__ inline double2 ld_stream(const double2 *p)
{
    typedef double d2v __attribute__((ext_vector_type(2)));
    const d2v v = __builtin_nontemporal_load(reinterpret_cast<const d2v *>(p));
    return make_double2(v.x, v.y);
}

// Operands of a batch of residuals: system f (blockIdx.y) uses Z + f sZ,
// B + f sB, X + f sX, R + f sR (doubles) and the norm slots at + f sN;
// systems whose `active` entry is 0 are skipped.
struct ResidualArgs {
    int64_t n;
    const double *Z, *B, *X;
    double *R;
    uint64_t *rnorm, *xnorm;
    int64_t sZ, sB, sX, sR, sN;
    const uint32_t *active;
};

// One workgroup per RR consecutive rows; its four waves split the columns
// into four contiguous ranges (more waves in flight for small n), each lane
// loads x_j once for all RR rows, and the four partial sums are added in
// LDS in a fixed order.
template <int NR, int RR>
__global__ __launch_bounds__(256) void residual_kernel(ResidualArgs ra)
{
    __shared__ double2 part[4][RR][NR];
    const int64_t f = blockIdx.y;
    if (ra.active && ra.active[f] == 0) return;
    const int64_t n = ra.n;
    const double *__restrict__ Z = ra.Z + size_t(f) * size_t(ra.sZ);
    const double *__restrict__ B = ra.B + size_t(f) * size_t(ra.sB);
    const double *__restrict__ X = ra.X + size_t(f) * size_t(ra.sX);
    double *__restrict__ R = ra.R + size_t(f) * size_t(ra.sR);
    uint64_t *rnorm = ra.rnorm ? ra.rnorm + size_t(f) * size_t(ra.sN) : nullptr;
    uint64_t *xnorm = ra.xnorm ? ra.xnorm + size_t(f) * size_t(ra.sN) : nullptr;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t i0 = int64_t(blockIdx.x) * RR;
    const int64_t span = ((n + 255) / 256) * 64;          // columns per wave, multiple of 64
    const int64_t j0 = wave * span, j1 = min<int64_t>(n, j0 + span);
    const double2 *xv = reinterpret_cast<const double2 *>(X);
    const double2 *zr[RR];
#pragma unroll
    for (int r = 0; r < RR; ++r)
        zr[r] = reinterpret_cast<const double2 *>(Z) + size_t(min<int64_t>(i0 + r, n - 1)) * size_t(n);
    double sr[RR][NR], si[RR][NR];
#pragma unroll
    for (int r = 0; r < RR; ++r)
#pragma unroll
        for (int k = 0; k < NR; ++k) { sr[r][k] = 0.0; si[r][k] = 0.0; }
#pragma unroll 4
    for (int64_t j = j0 + lane; j < j1; j += 64) {
        double2 x[NR];
#pragma unroll
        for (int k = 0; k < NR; ++k) x[k] = xv[size_t(k) * size_t(n) + size_t(j)];
#pragma unroll
        for (int r = 0; r < RR; ++r) {
            const double2 z = ld_stream(zr[r] + j);
#pragma unroll
            for (int k = 0; k < NR; ++k) {
                sr[r][k] = fma(z.x, x[k].x, sr[r][k]);
                sr[r][k] = fma(-z.y, x[k].y, sr[r][k]);
                si[r][k] = fma(z.x, x[k].y, si[r][k]);
                si[r][k] = fma(z.y, x[k].x, si[r][k]);
            }
        }
    }
#pragma unroll
    for (int r = 0; r < RR; ++r)
#pragma unroll
        for (int k = 0; k < NR; ++k) {
            const double a = wave_sum(sr[r][k]);
            const double c = wave_sum(si[r][k]);
            if (lane == 0) part[wave][r][k] = make_double2(a, c);
        }
    __syncthreads();
    if (threadIdx.x < RR * NR) {
        const int r = threadIdx.x / NR, k = threadIdx.x % NR;
        const int64_t i = i0 + r;
        if (i < n) {
            const double a = ((part[0][r][k].x + part[1][r][k].x) + part[2][r][k].x) + part[3][r][k].x;
            const double c = ((part[0][r][k].y + part[1][r][k].y) + part[2][r][k].y) + part[3][r][k].y;
            const double2 b = reinterpret_cast<const double2 *>(B)[size_t(k) * size_t(n) + size_t(i)];
            const double rr = b.x - a, ri = b.y - c;
            reinterpret_cast<double2 *>(R)[size_t(k) * size_t(n) + size_t(i)] = make_double2(rr, ri);
            if (rnorm) atomic_max_nonneg(rnorm + k, cabs(rr, ri));
        }
    }
    // ||x_k||_inf, by the first workgroup only, in a loop of its own
    if (blockIdx.x == 0 && xnorm != nullptr && wave < NR) {
        const int k = wave;
        double xm = 0.0;
        for (int64_t j = lane; j < n; j += 64) {
            const double2 x = xv[size_t(k) * size_t(n) + size_t(j)];
            xm = fmax(xm, cabs(x.x, x.y));
        }
        xm = wave_max(xm);
        if (lane == 0) atomic_max_nonneg(xnorm + k, xm);
    }
}

// The same residual with Z(w_f) formed on the fly from the model instead of
// read from a stored complex128 matrix: entry (i, j) is, rounded operation
// by operation as in the assembly kernel,
//   Re = (i == j) ? zr_f g_i : 0,   Im = w_f L_ij - Psi_ij / w_f (+ zi_f g_i if i == j),
// so Z is bit-identical to the assembled one, and every per-row sum follows
// residual_kernel's order exactly (same column split, same reductions).
// A workgroup covers RR rows and FC frequencies, so each element of L and
// Psi it loads serves all of them.  The workgroups of one block of rows (one
// per group of FC frequencies) go to the same XCD one after another: the
// first brings the rows of L and Psi into that XCD's L2 and the others read
// them there, so per pass L and Psi come from memory about once.
struct ModelResidualArgs {
    int64_t n, nf;
    int row_blocks, groups;   // ceil(n / RR), ceil(nf / FC)
    const double *L, *Psi, *g;
    double w[kMaxBatch], zr[kMaxBatch], zi[kMaxBatch];
    // 1 / w rounded to nearest, and whether every w lies in [2^-64, 2^64]
    // (the range in which psi / w may be formed from it, see psi_over_w)
    double winv[kMaxBatch];
    int div_by_inv;
    const double *B, *X;
    double *R;
    uint64_t *rnorm, *xnorm;
    int64_t sB, sX, sR, sN;
    const uint32_t *active;
};

template <int NR, int RR, int FC>
__global__ __launch_bounds__(256) void residual_model_kernel(ModelResidualArgs ra)
{
#pragma clang fp contract(off)
    __shared__ double2 part[4][FC][RR][NR];
    const int64_t n = ra.n;
    // workgroups are dealt to the 8 XCDs round-robin: the t-th workgroup of
    // an XCD takes group t % groups of that XCD's block of rows t / groups
    const int lin = int(blockIdx.x), t = lin / 8;
    const int by = t % ra.groups, bx = (t / ra.groups) * 8 + lin % 8;
    if (bx >= ra.row_blocks) return;
    const int f0 = by * FC;
    const int nc = int(min<int64_t>(FC, ra.nf - f0));
    bool live[FC];
    bool any = false;
#pragma unroll
    for (int c = 0; c < FC; ++c) {
        live[c] = c < nc && (!ra.active || ra.active[f0 + c] != 0);
        any = any || live[c];
    }
    if (!any) return;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t i0 = int64_t(bx) * RR;
    const int64_t span = ((n + 255) / 256) * 64;          // columns per wave, multiple of 64
    const int64_t j0 = wave * span, j1 = min<int64_t>(n, j0 + span);
    double w[FC], zr[FC], zi[FC], wi[FC];
    const bool by_inv = ra.div_by_inv != 0;
    const double2 *xv[FC];
#pragma unroll
    for (int c = 0; c < FC; ++c) {
        const int fc = f0 + (c < nc ? c : 0);
        w[c] = ra.w[fc];
        wi[c] = ra.winv[fc];
        zr[c] = ra.zr[fc];
        zi[c] = ra.zi[fc];
        xv[c] = reinterpret_cast<const double2 *>(ra.X + size_t(fc) * size_t(ra.sX));
    }
    int64_t rows[RR];
    double gi[RR];
    const double *lr[RR], *pr[RR];
#pragma unroll
    for (int r = 0; r < RR; ++r) {
        rows[r] = min<int64_t>(i0 + r, n - 1);
        gi[r] = ra.g[rows[r]];
        lr[r] = ra.L + size_t(rows[r]) * size_t(n);
        pr[r] = ra.Psi + size_t(rows[r]) * size_t(n);
    }
    double sr[FC][RR][NR], si[FC][RR][NR];
#pragma unroll
    for (int c = 0; c < FC; ++c)
#pragma unroll
        for (int r = 0; r < RR; ++r)
#pragma unroll
            for (int k = 0; k < NR; ++k) { sr[c][r][k] = 0.0; si[c][r][k] = 0.0; }
    // Column j of the wave's span goes to lane (j - j0) % 64, every lane
    // adding its columns in increasing order (the order of residual_kernel).
    // The loads are software-pipelined: those of a lane's next column are
    // issued before the arithmetic of the current one, and every frequency's
    // x is loaded without a branch (a converged frequency's sums are
    // discarded), so no load waits behind another's use.
    struct Col {
        double l[RR], p[RR];
        double2 x[FC][NR];
    };
    auto load = [&](Col &cl, int64_t j) {
#pragma unroll
        for (int r = 0; r < RR; ++r) {
            cl.l[r] = lr[r][j];
            cl.p[r] = pr[r][j];
        }
#pragma unroll
        for (int c = 0; c < FC; ++c)
#pragma unroll
            for (int k = 0; k < NR; ++k) cl.x[c][k] = xv[c][size_t(k) * size_t(n) + size_t(j)];
    };
    auto add = [&](const Col &cl, int64_t j) {
#pragma unroll
        for (int c = 0; c < FC; ++c)
#pragma unroll
            for (int r = 0; r < RR; ++r) {
                const double wl = w[c] * cl.l[r];
                const double pw = psi_over_w(cl.p[r], w[c], wi[c], by_inv);
                double im = wl - pw;
                double re = 0.0;
                if (j == rows[r]) {
                    im = im + zi[c] * gi[r];
                    re = zr[c] * gi[r];
                }
#pragma unroll
                for (int k = 0; k < NR; ++k) {
                    sr[c][r][k] = fma(re, cl.x[c][k].x, sr[c][r][k]);
                    sr[c][r][k] = fma(-im, cl.x[c][k].y, sr[c][r][k]);
                    si[c][r][k] = fma(re, cl.x[c][k].y, si[c][r][k]);
                    si[c][r][k] = fma(im, cl.x[c][k].x, si[c][r][k]);
                }
            }
    };
    const int64_t cnt = max<int64_t>(j1 - j0, 0);      // uniform
    const int64_t full = cnt / 64;                      // columns for every lane
    Col ca, cb;
    if (full > 0) load(ca, j0 + lane);
    for (int64_t t = 0; t < full; t += 2) {
        const int64_t ja = j0 + lane + 64 * t;
        if (t + 1 < full) load(cb, ja + 64);
        // (the scheduler would otherwise move the loads down to their use)
        __builtin_amdgcn_sched_barrier(0);
        add(ca, ja);
        if (t + 1 < full) {
            if (t + 2 < full) load(ca, ja + 128);
            __builtin_amdgcn_sched_barrier(0);
            add(cb, ja + 64);
        }
    }
    if (lane < cnt - 64 * full) {
        const int64_t j = j0 + lane + 64 * full;
        load(ca, j);
        add(ca, j);
    }
#pragma unroll
    for (int c = 0; c < FC; ++c)
#pragma unroll
        for (int r = 0; r < RR; ++r)
#pragma unroll
            for (int k = 0; k < NR; ++k) {
                const double a = wave_sum(sr[c][r][k]);
                const double b = wave_sum(si[c][r][k]);
                if (lane == 0) part[wave][c][r][k] = make_double2(a, b);
            }
    __syncthreads();
    for (int e = threadIdx.x; e < FC * RR * NR; e += 256) {
        const int c = e / (RR * NR), r = (e / NR) % RR, k = e % NR;
        const int64_t i = i0 + r;
        if (!live[c] || i >= n) continue;
        const int64_t fc = f0 + c;
        const double a = ((part[0][c][r][k].x + part[1][c][r][k].x) + part[2][c][r][k].x) + part[3][c][r][k].x;
        const double b = ((part[0][c][r][k].y + part[1][c][r][k].y) + part[2][c][r][k].y) + part[3][c][r][k].y;
        const double2 bv = reinterpret_cast<const double2 *>(ra.B + size_t(fc) * size_t(ra.sB))[size_t(k) * size_t(n) + size_t(i)];
        const double rr = bv.x - a, ri = bv.y - b;
        reinterpret_cast<double2 *>(ra.R + size_t(fc) * size_t(ra.sR))[size_t(k) * size_t(n) + size_t(i)] = make_double2(rr, ri);
        if (ra.rnorm) atomic_max_nonneg(ra.rnorm + size_t(fc) * size_t(ra.sN) + k, cabs(rr, ri));
    }
    // ||x_k||_inf of each frequency, by the first workgroup of the group
    if (bx == 0 && ra.xnorm != nullptr) {
        for (int e = wave; e < FC * NR; e += 4) {
            const int c = e / NR, k = e % NR;
            if (!live[c]) continue;
            double xm = 0.0;
            for (int64_t j = lane; j < n; j += 64) {
                const double2 x = xv[c][size_t(k) * size_t(n) + size_t(j)];
                xm = fmax(xm, cabs(x.x, x.y));
            }
            xm = wave_max(xm);
            if (lane == 0) atomic_max_nonneg(ra.xnorm + size_t(f0 + c) * size_t(ra.sN) + k, xm);
        }
    }
}

__global__ void fill_u32_kernel(uint32_t *p, size_t count, uint32_t v)
{
    const size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < count) p[i] = v;
}

__global__ void fill_f64_kernel(double *p, size_t count, double v)
{
    const size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < count) p[i] = v;
}

// blockIdx.y selects the system (p + y stride)
__global__ void fill_f64_batch_kernel(double *p, size_t count, int64_t stride, double v)
{
    const size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < count) p[size_t(blockIdx.y) * size_t(stride) + i] = v;
}

// max_i |B[k][i]| for each row k (one workgroup per row) of system
// blockIdx.y (B + f sB, out + f sOut)
__global__ __launch_bounds__(256) void vec_norms_kernel(int64_t n, const double *B, int64_t sB,
                                                        uint64_t *out, int64_t sOut)
{
    const int64_t k = blockIdx.x;
    B += size_t(blockIdx.y) * size_t(sB);
    out += size_t(blockIdx.y) * size_t(sOut);
    const double2 *b = reinterpret_cast<const double2 *>(B) + size_t(k) * size_t(n);
    double m = 0.0;
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) m = fmax(m, cabs(b[i].x, b[i].y));
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0) atomic_max_nonneg(out + k, m);
}

// max_i v[i] of system blockIdx.y (v + f sv, out + f sOut)
__global__ __launch_bounds__(256) void max_reduce_kernel(int64_t n, const double *v, int64_t sv,
                                                         uint64_t *out, int64_t sOut)
{
    v += size_t(blockIdx.y) * size_t(sv);
    out += size_t(blockIdx.y) * size_t(sOut);
    double m = 0.0;
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += int64_t(gridDim.x) * blockDim.x)
        m = fmax(m, v[i]);
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0) atomic_max_nonneg(out, m);
}

// sum_j |Z_ij| for each row (one wave per row)
__global__ __launch_bounds__(256) void row_abs_sums_kernel(int64_t n, const double *Z, double *out)
{
    const int lane = threadIdx.x & 63;
    const int64_t i = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (i >= n) return;
    const double2 *zr = reinterpret_cast<const double2 *>(Z) + size_t(i) * size_t(n);
    double s = 0.0;
    for (int64_t j = lane; j < n; j += 64) s += cabs(zr[j].x, zr[j].y);
    s = wave_sum(s);
    if (lane == 0) out[i] = s;
}

__global__ void copy_c64_rows_kernel(int64_t n, int64_t nrhs, const float *src, int64_t ld_src,
                                     float *dst, int64_t ld_dst)
{
    const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (idx >= n * nrhs) return;
    const int64_t k = idx / n, i = idx % n;
    reinterpret_cast<float2 *>(dst)[size_t(k) * size_t(ld_dst) + size_t(i)] =
        reinterpret_cast<const float2 *>(src)[size_t(k) * size_t(ld_src) + size_t(i)];
}

inline unsigned grid_for(size_t count, unsigned block)
{
    return unsigned((count + block - 1) / block);
}

}  // namespace

template <int RR>
void launch_residual_rr(int nr, dim3 grid, hipStream_t s, const ResidualArgs &ra)
{
    switch (nr) {
    case 1: hipLaunchKernelGGL((residual_kernel<1, RR>), grid, dim3(256), 0, s, ra); break;
    case 2: hipLaunchKernelGGL((residual_kernel<2, RR>), grid, dim3(256), 0, s, ra); break;
    case 3: hipLaunchKernelGGL((residual_kernel<3, RR>), grid, dim3(256), 0, s, ra); break;
    default: hipLaunchKernelGGL((residual_kernel<4, RR>), grid, dim3(256), 0, s, ra); break;
    }
}

int launch_residual(int64_t n, int64_t nrhs, const ResidualBatch &rb, const double *Z,
                    const double *B, const double *X, double *R, uint64_t *rnorm_bits,
                    uint64_t *xnorm_bits, hipStream_t s)
{
    // rows per workgroup: enough workgroups to fill 256 CUs, x reused across rows
    const int rr = n >= 8192 ? 4 : ((n >= 4096 || n * rb.nf >= 8192) ? 2 : 1);
    const dim3 grid(unsigned((n + rr - 1) / rr), unsigned(rb.nf));
    for (int64_t k0 = 0; k0 < nrhs; k0 += kMaxRhs) {
        const int nr = int(std::min<int64_t>(kMaxRhs, nrhs - k0));
        const size_t off = size_t(k0) * size_t(n) * 2;
        ResidualArgs ra;
        ra.n = n;
        ra.Z = Z; ra.B = B + off; ra.X = X + off; ra.R = R + off;
        ra.rnorm = rnorm_bits ? rnorm_bits + k0 : nullptr;
        ra.xnorm = xnorm_bits ? xnorm_bits + k0 : nullptr;
        ra.sZ = rb.sZ; ra.sB = rb.sB; ra.sX = rb.sX; ra.sR = rb.sR; ra.sN = rb.sN;
        ra.active = rb.active;
        const double bytes = (16.0 * double(n) * double(n) + 48.0 * double(n) * nr) * double(rb.nf);
        ProfScope prof(MSOLVE_K_RESIDUAL, s, bytes);
        if (rr == 4)
            launch_residual_rr<4>(nr, grid, s, ra);
        else if (rr == 2)
            launch_residual_rr<2>(nr, grid, s, ra);
        else
            launch_residual_rr<1>(nr, grid, s, ra);
        MS_HIP(hipGetLastError());
    }
    return MSOLVE_OK;
}

template <int RR, int FC>
void launch_residual_model_rr(int nr, dim3 grid, hipStream_t s, const ModelResidualArgs &ra)
{
    switch (nr) {
    case 1: hipLaunchKernelGGL((residual_model_kernel<1, RR, FC>), grid, dim3(256), 0, s, ra); break;
    case 2: hipLaunchKernelGGL((residual_model_kernel<2, RR, FC>), grid, dim3(256), 0, s, ra); break;
    case 3: hipLaunchKernelGGL((residual_model_kernel<3, RR, FC>), grid, dim3(256), 0, s, ra); break;
    default: hipLaunchKernelGGL((residual_model_kernel<4, RR, FC>), grid, dim3(256), 0, s, ra); break;
    }
}

int launch_residual_model(int64_t n, int64_t nrhs, const ZModel &zm, const ResidualBatch &rb,
                          const double *B, const double *X, double *R, uint64_t *rnorm_bits,
                          uint64_t *xnorm_bits, hipStream_t s)
{
    if (rb.nf < 1 || rb.nf > kMaxBatch) return fail(MSOLVE_E_ARG, "residual: 1 to 32 frequencies per launch");
    // two rows and two frequencies per workgroup: with the rows of L and Psi
    // shared through L2, more of either only cost registers (measured: three
    // or four frequencies 25-35% slower at n = 2157, four rows 15% slower at
    // n = 16384 with four right-hand sides)
    constexpr int rr = 2, fc = 2;
    for (int64_t k0 = 0; k0 < nrhs; k0 += kMaxRhs) {
        const int nr = int(std::min<int64_t>(kMaxRhs, nrhs - k0));
        const int row_blocks = int((n + rr - 1) / rr), groups = int((rb.nf + fc - 1) / fc);
        const dim3 grid(unsigned((row_blocks + 7) / 8 * 8 * groups));
        const size_t off = size_t(k0) * size_t(n) * 2;
        ModelResidualArgs ra;
        ra.n = n;
        ra.nf = rb.nf;
        ra.row_blocks = row_blocks;
        ra.groups = groups;
        ra.L = zm.L; ra.Psi = zm.Psi; ra.g = zm.g;
        ra.div_by_inv = 1;
        for (int64_t f = 0; f < kMaxBatch; ++f) {
            ra.w[f] = f < rb.nf ? zm.w[f] : 1.0;
            ra.zr[f] = f < rb.nf ? zm.zr[f] : 0.0;
            ra.zi[f] = f < rb.nf ? zm.zi[f] : 0.0;
            ra.winv[f] = 1.0 / ra.w[f];
            const double aw = std::fabs(ra.w[f]);
            if (!(aw >= 0x1p-64 && aw <= 0x1p64)) ra.div_by_inv = 0;
        }
        ra.B = B + off; ra.X = X + off; ra.R = R + off;
        ra.rnorm = rnorm_bits ? rnorm_bits + k0 : nullptr;
        ra.xnorm = xnorm_bits ? xnorm_bits + k0 : nullptr;
        ra.sB = rb.sB; ra.sX = rb.sX; ra.sR = rb.sR; ra.sN = rb.sN;
        ra.active = rb.active;
        const double bytes = 16.0 * double(n) * double(n) + 48.0 * double(n) * nr * double(rb.nf);
        ProfScope prof(MSOLVE_K_RESIDUAL, s, bytes);
        launch_residual_model_rr<rr, fc>(nr, grid, s, ra);
        MS_HIP(hipGetLastError());
    }
    return MSOLVE_OK;
}

int launch_fill_u32(uint32_t *p, size_t count, uint32_t v, hipStream_t s)
{
    if (count == 0) return MSOLVE_OK;
    hipLaunchKernelGGL(fill_u32_kernel, dim3(grid_for(count, 256)), dim3(256), 0, s, p, count, v);
    MS_HIP(hipGetLastError());
    return MSOLVE_OK;
}

int launch_fill_f64(double *p, size_t count, double v, hipStream_t s)
{
    if (count == 0) return MSOLVE_OK;
    hipLaunchKernelGGL(fill_f64_kernel, dim3(grid_for(count, 256)), dim3(256), 0, s, p, count, v);
    MS_HIP(hipGetLastError());
    return MSOLVE_OK;
}

int launch_fill_f64_batch(double *p, size_t count, int64_t stride, int64_t nsys, double v,
                          hipStream_t s)
{
    if (count == 0 || nsys < 1) return MSOLVE_OK;
    hipLaunchKernelGGL(fill_f64_batch_kernel, dim3(grid_for(count, 256), unsigned(nsys)), dim3(256), 0,
                       s, p, count, stride, v);
    MS_HIP(hipGetLastError());
    return MSOLVE_OK;
}

int launch_copy_c64_rows(int64_t n, int64_t nrhs, const float *src, int64_t ld_src, float *dst,
                         int64_t ld_dst, hipStream_t s)
{
    const size_t count = size_t(n) * size_t(nrhs);
    if (count == 0) return MSOLVE_OK;
    hipLaunchKernelGGL(copy_c64_rows_kernel, dim3(grid_for(count, 256)), dim3(256), 0, s, n, nrhs,
                       src, ld_src, dst, ld_dst);
    MS_HIP(hipGetLastError());
    return MSOLVE_OK;
}

int launch_vec_norms(int64_t n, int64_t nrhs, int64_t nf, const double *B, int64_t sB,
                     uint64_t *out_bits, int64_t sOut, hipStream_t s)
{
    hipLaunchKernelGGL(vec_norms_kernel, dim3(unsigned(nrhs), unsigned(nf)), dim3(256), 0, s, n, B,
                       sB, out_bits, sOut);
    MS_HIP(hipGetLastError());
    return MSOLVE_OK;
}

int launch_max_reduce(int64_t n, int64_t nf, const double *v, int64_t sv, uint64_t *out_bits,
                      int64_t sOut, hipStream_t s)
{
    const unsigned blocks = unsigned(std::min<int64_t>(256, (n + 255) / 256));
    hipLaunchKernelGGL(max_reduce_kernel, dim3(blocks, unsigned(nf)), dim3(256), 0, s, n, v, sv,
                       out_bits, sOut);
    MS_HIP(hipGetLastError());
    return MSOLVE_OK;
}

int launch_row_abs_sums(int64_t n, const double *Z128, double *out, hipStream_t s)
{
    hipLaunchKernelGGL(row_abs_sums_kernel, dim3(unsigned((n + 3) / 4)), dim3(256), 0, s, n, Z128,
                       out);
    MS_HIP(hipGetLastError());
    return MSOLVE_OK;
}

}  // namespace msolve

extern "C" int msolve_residual_c128(int64_t n, int64_t nrhs, const double *Z128, const double *B,
                                    const double *X, double *R, double *norms, void *stream)
{
    using namespace msolve;
    if (n < 1 || nrhs < 1) return fail(MSOLVE_E_ARG, "msolve_residual_c128: n and nrhs must be >= 1");
    if (!Z128 || !B || !X || !R) return fail(MSOLVE_E_ARG, "msolve_residual_c128: null pointer");
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint64_t *bits = reinterpret_cast<uint64_t *>(norms);
    if (norms) MS_TRY(launch_fill_u32(reinterpret_cast<uint32_t *>(norms), size_t(4 * nrhs), 0u, s));
    return launch_residual(n, nrhs, ResidualBatch{}, Z128, B, X, R, bits, bits ? bits + nrhs : nullptr, s);
}
