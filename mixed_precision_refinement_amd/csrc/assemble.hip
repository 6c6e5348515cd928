// Assembly of Z(w) = j w L - j Psi / w + Zs(w) G on the GPU.
//
// Model equation of the page "Solving Dense Matrices Fast in the Browser --
// Adaptive Frequency Sampling and Mixed Precision on WebGPU", section "Fewer
// frequency points: adaptive frequency sampling": L, Psi and G do not depend
// on frequency, so each frequency only re-combines them.  The kernel streams
// L and Psi once and writes Z in complex128 (for the double-precision
// residual), its round-to-nearest complex64 copy (for the single-precision
// factorisation) and the row sums of |Z| (for the backward-error test).
//
// Memory bound: per frequency 24 n^2 bytes written (+ 8 n of row sums), or
// only the lower triangle's half of them when the matrix is complex symmetric
// and only that triangle is wanted; L and Psi (16 n^2 bytes) are read about
// once per batch.
// One wave64 per row; lanes stride the row so every load and store
// instruction of a wave touches one contiguous span.
#include <cmath>

#include "common.hpp"

namespace msolve {
namespace {

constexpr int kRowsPerBlock = 4;   // one wave per row, four waves per block
constexpr int kFreqPerPass = 4;    // frequencies written per read of L and Psi

__device__ inline double wave_sum(double v)
{
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

struct AssembleArgs {
    int64_t n, nf;
    int blocks, passes;       // ceil(n / 4) blocks of rows, ceil(nf / 4) groups of frequencies
    double w[kMaxBatch], zr[kMaxBatch], zi[kMaxBatch];
    double winv[kMaxBatch];   // 1 / w rounded to nearest (see psi_over_w)
    int div_by_inv;           // every w in [2^-64, 2^64]
    const double *L, *Psi, *g;
    double *Z128;
    int64_t sZ128;
    float *Z64;
    int64_t sZ64;
    double *zrowabs;
    int64_t sRow;
    // the strict upper triangle of Z128 and Z64 is left unwritten when
    // `lower` is set, or when `sym_flag` is not NULL and *sym_flag == 0 (the
    // symmetry check's word, read on the device: no difference found)
    int lower;
    const uint32_t *sym_flag;
};

// A workgroup writes four rows for four frequencies f0 .. f0 + 3, so each
// element of L and Psi it loads serves all four.  The workgroups of one
// block of rows (one per group of four frequencies) are dealt to the same XCD
// one after another: the first brings the rows of L and Psi into that XCD's
// L2 and the others read them there, so L and Psi come from memory about once.
__global__ __launch_bounds__(256) void assemble_kernel(AssembleArgs a)
{
    // Every operation below is rounded on its own, in the written order.
#pragma clang fp contract(off)
    const int lane = threadIdx.x & 63;
    const int64_t n = a.n;
    // workgroups are dealt to the 8 XCDs round-robin: the t-th workgroup of
    // an XCD takes group t % passes of that XCD's block of rows t / passes
    const int lin = int(blockIdx.x), t = lin / 8;
    const int by = t % a.passes, bx = (t / a.passes) * 8 + lin % 8;
    const int64_t i = int64_t(bx) * kRowsPerBlock + (threadIdx.x >> 6);
    if (bx >= a.blocks || i >= n) return;
    const bool lower = a.lower != 0 || (a.sym_flag != nullptr && *a.sym_flag == 0u);
    const int f0 = by * kFreqPerPass;
    const int nc = int(min<int64_t>(kFreqPerPass, a.nf - f0));
    double w[kFreqPerPass], zr[kFreqPerPass], zi[kFreqPerPass], wi[kFreqPerPass], acc[kFreqPerPass];
    const bool by_inv = a.div_by_inv != 0;
#pragma unroll
    for (int c = 0; c < kFreqPerPass; ++c) {
        const int f = f0 + (c < nc ? c : 0);
        w[c] = a.w[f];
        wi[c] = a.winv[f];
        zr[c] = a.zr[f];
        zi[c] = a.zi[f];
        acc[c] = 0.0;
    }
    const size_t row = size_t(i) * size_t(n);
    const double gi = a.g[i];
    for (int64_t j = lane; j < n; j += 64) {
        const size_t k = row + size_t(j);
        const double l = a.L[k], p = a.Psi[k];
#pragma unroll
        for (int c = 0; c < kFreqPerPass; ++c) {
            if (c >= nc) break;
            const size_t f = size_t(f0 + c);
            const double wl = w[c] * l;
            const double pw = psi_over_w(p, w[c], wi[c], by_inv);
            double im = wl - pw;
            double re = 0.0;
            double mag;
            if (j == i) {
                im = im + zi[c] * gi;
                re = zr[c] * gi;
                mag = hypot(re, im);
            } else {
                mag = fabs(im);
            }
            if (!lower || j <= i) {
                if (a.Z128) reinterpret_cast<double2 *>(a.Z128 + f * size_t(a.sZ128))[k] = make_double2(re, im);
                if (a.Z64) reinterpret_cast<float2 *>(a.Z64 + f * size_t(a.sZ64))[k] = make_float2(float(re), float(im));
            }
            acc[c] += mag;
        }
    }
    if (a.zrowabs) {
#pragma unroll
        for (int c = 0; c < kFreqPerPass; ++c) {
            if (c >= nc) break;
            const double v = wave_sum(acc[c]);
            if (lane == 0) a.zrowabs[size_t(f0 + c) * size_t(a.sRow) + size_t(i)] = v;
        }
    }
}

// *flag |= 1 when L or Psi is not exactly symmetric (a pair i > j with
// L_ij != L_ji or Psi_ij != Psi_ji; a NaN counts as a difference).  The
// workgroup at (ti, tj), tj <= ti, stages the 32 x 32 tile (tj, ti) in LDS
// and compares tile (ti, tj) with its transpose, both read along rows.
constexpr int kSymTile = 32;
__global__ __launch_bounds__(256) void sym_check_kernel(int64_t n, const double *L, const double *Psi,
                                                        uint32_t *flag)
{
    __shared__ double t[kSymTile][kSymTile + 1];
    const int64_t ti = blockIdx.x, tj = blockIdx.y;
    if (tj > ti) return;
    bool diff = false;
    for (int m = 0; m < 2; ++m) {
        const double *M = m ? Psi : L;
        for (int e = threadIdx.x; e < kSymTile * kSymTile; e += 256) {
            const int r = e / kSymTile, c = e % kSymTile;
            const int64_t gr = tj * kSymTile + r, gc = ti * kSymTile + c;
            t[r][c] = (gr < n && gc < n) ? M[size_t(gr) * size_t(n) + size_t(gc)] : 0.0;
        }
        __syncthreads();
        for (int e = threadIdx.x; e < kSymTile * kSymTile; e += 256) {
            const int r = e / kSymTile, c = e % kSymTile;
            const int64_t gr = ti * kSymTile + r, gc = tj * kSymTile + c;
            if (gr < n && gc < n && !(M[size_t(gr) * size_t(n) + size_t(gc)] == t[c][r])) diff = true;
        }
        __syncthreads();
    }
    if (diff) atomicOr(flag, 1u);
}

}  // namespace

int launch_sym_check(int64_t n, const double *L, const double *Psi, uint32_t *flag, hipStream_t s)
{
    const int64_t nt = (n + kSymTile - 1) / kSymTile;
    hipLaunchKernelGGL(sym_check_kernel, dim3(unsigned(nt), unsigned(nt)), dim3(256), 0, s, n, L, Psi, flag);
    MS_HIP(hipGetLastError());
    return MSOLVE_OK;
}

int launch_assemble(int64_t n, int64_t nf, const double *w, const double *zr, const double *zi,
                    const double *L, const double *Psi, const double *g, double *Z128,
                    int64_t sZ128, float *Z64, int64_t sZ64, double *zrowabs, int64_t sRow,
                    hipStream_t s, bool lower, const uint32_t *sym_flag)
{
    if (nf < 1 || nf > kMaxBatch) return fail(MSOLVE_E_ARG, "assemble: 1 to 32 frequencies per launch");
    AssembleArgs a;
    a.n = n;
    a.nf = nf;
    a.div_by_inv = 1;
    for (int64_t f = 0; f < kMaxBatch; ++f) {
        a.w[f] = f < nf ? w[f] : 1.0;
        a.zr[f] = f < nf ? zr[f] : 0.0;
        a.zi[f] = f < nf ? zi[f] : 0.0;
        a.winv[f] = 1.0 / a.w[f];
        const double aw = std::fabs(a.w[f]);
        if (!(aw >= 0x1p-64 && aw <= 0x1p64)) a.div_by_inv = 0;
    }
    a.L = L; a.Psi = Psi; a.g = g;
    a.Z128 = Z128; a.sZ128 = sZ128;
    a.Z64 = Z64; a.sZ64 = sZ64;
    a.zrowabs = zrowabs; a.sRow = sRow;
    a.lower = lower ? 1 : 0;
    a.sym_flag = sym_flag;
    const int64_t blocks = (n + kRowsPerBlock - 1) / kRowsPerBlock;
    const int64_t passes = (nf + kFreqPerPass - 1) / kFreqPerPass;
    a.blocks = int(blocks);
    a.passes = int(passes);
    const double nn = double(n) * double(n);
    // (with sym_flag the caller scales this record once it knows the flag)
    const double zel = lower ? 0.5 * double(n) * double(n + 1) : nn;   // elements of Z written
    const double bytes = 16.0 * nn +
                         ((Z128 ? 16.0 : 0.0) * zel + (Z64 ? 8.0 : 0.0) * zel + 8.0 * double(n)) * double(nf) +
                         8.0 * double(n);
    ProfScope prof(MSOLVE_K_ASSEMBLE, s, bytes);
    hipLaunchKernelGGL(assemble_kernel, dim3(unsigned((blocks + 7) / 8 * 8 * passes)), dim3(256), 0, s, a);
    MS_HIP(hipGetLastError());
    return MSOLVE_OK;
}

}  // namespace msolve

extern "C" int msolve_assemble(int64_t n, double omega, double zs_re, double zs_im,
                               const double *L, const double *Psi, const double *g,
                               double *Z128, float *Z64, double *zrowabs, void *stream)
{
    using namespace msolve;
    if (n < 1) return fail(MSOLVE_E_ARG, "msolve_assemble: n must be >= 1");
    if (!(omega == omega) || omega == 0.0 || omega - omega != 0.0)
        return fail(MSOLVE_E_ARG, "msolve_assemble: omega must be finite and nonzero");
    if (!L || !Psi || !g) return fail(MSOLVE_E_ARG, "msolve_assemble: null input pointer");
    if (!Z128 && !Z64 && !zrowabs)
        return fail(MSOLVE_E_ARG, "msolve_assemble: all outputs are NULL");
    return launch_assemble(n, 1, &omega, &zs_re, &zs_im, L, Psi, g, Z128, 0, Z64, 0, zrowabs, 0,
                           static_cast<hipStream_t>(stream));
}
