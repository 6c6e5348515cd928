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
// Memory bound: 16 n^2 bytes read, 24 n^2 bytes written (+ 8 n for g and the
// row sums).  One wave64 per row; lanes stride the row so every load and
// store instruction of a wave touches one contiguous span.
#include "common.hpp"

namespace msolve {
namespace {

constexpr int kRowsPerBlock = 4;   // one wave per row, four waves per block

__device__ inline double wave_sum(double v)
{
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

__global__ __launch_bounds__(256) void assemble_kernel(
    int64_t n, double w, double zr, double zi, const double *__restrict__ L,
    const double *__restrict__ Psi, const double *__restrict__ g,
    double *__restrict__ Z128, float *__restrict__ Z64, double *__restrict__ zrowabs)
{
    // Every operation below is rounded on its own, in the written order.
#pragma clang fp contract(off)
    const int lane = threadIdx.x & 63;
    const int64_t i = int64_t(blockIdx.x) * kRowsPerBlock + (threadIdx.x >> 6);
    if (i >= n) return;
    const size_t row = size_t(i) * size_t(n);
    const double gi = g[i];
    double acc = 0.0;
    for (int64_t j = lane; j < n; j += 64) {
        const size_t k = row + size_t(j);
        const double wl = w * L[k];
        const double pw = Psi[k] / w;
        double im = wl - pw;
        double re = 0.0;
        double mag;
        if (j == i) {
            im = im + zi * gi;
            re = zr * gi;
            mag = hypot(re, im);
        } else {
            mag = fabs(im);
        }
        if (Z128) reinterpret_cast<double2 *>(Z128)[k] = make_double2(re, im);
        if (Z64) reinterpret_cast<float2 *>(Z64)[k] = make_float2(float(re), float(im));
        acc += mag;
    }
    if (zrowabs) {
        acc = wave_sum(acc);
        if (lane == 0) zrowabs[i] = acc;
    }
}

}  // namespace

int launch_assemble(int64_t n, double w, double zr, double zi, const double *L,
                    const double *Psi, const double *g, double *Z128, float *Z64,
                    double *zrowabs, hipStream_t s)
{
    const int64_t blocks = (n + kRowsPerBlock - 1) / kRowsPerBlock;
    const double bytes = 16.0 * double(n) * double(n) + (Z128 ? 16.0 : 0.0) * double(n) * double(n) +
                         (Z64 ? 8.0 : 0.0) * double(n) * double(n) + 16.0 * double(n);
    ProfScope prof(MSOLVE_K_ASSEMBLE, s, bytes);
    hipLaunchKernelGGL(assemble_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, n, w, zr, zi,
                       L, Psi, g, Z128, Z64, zrowabs);
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
    return launch_assemble(n, omega, zs_re, zs_im, L, Psi, g, Z128, Z64, zrowabs,
                           static_cast<hipStream_t>(stream));
}
