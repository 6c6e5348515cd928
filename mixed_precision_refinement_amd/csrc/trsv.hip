// Triangular solves with the single-precision factors (steps 2 and 4 of the
// refinement list in the section "Double-precision answers from a GPU
// without double precision" of the page "Solving Dense Matrices Fast in the
// Browser": solve with the factorisation for x, then for each correction).
//
// Forward:  L y = fl32(r)     y_b = Linv_b (r_b - sum_{j<b} L_bj y_j)
// Back:     U d = y           d_b = Uinv_b (y_b - sum_{j>b} U_bj d_j)
// with Linv_b, Uinv_b the inverted diagonal blocks left by the factorisation.
//
// One persistent launch per direction: workgroup t takes block b in
// dependency order from an atomic ticket (so every block it waits for is
// already running), streams its block row of L (or U) against each finished
// block of the solution as soon as that block's ready flag carries this
// launch's epoch, and publishes its own block with a release store.  Every
// wait is bounded: on time-out the kernel raises a shared error word, every
// other wait sees it and gives up, and the host reports MSOLVE_E_DEVICE.
#include "common.hpp"

namespace msolve {
namespace {

constexpr int kTrsvThreads = 256;   // 64 rows x 4 quarter-row lanes
constexpr int kMaxRhs = 4;          // right-hand sides per launch
constexpr uint32_t kSpinLimit = 1u << 22;

__device__ inline bool wait_flag(const uint32_t *flag, uint32_t epoch, uint64_t *err)
{
    uint32_t spins = 0;
    while (__hip_atomic_load(flag, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) != epoch) {
        if (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) return false;
        if (++spins > kSpinLimit) {
            __hip_atomic_fetch_or(err, uint64_t(1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return false;
        }
        __builtin_amdgcn_s_sleep(2);
    }
    return true;
}

// acc[k] -= M[row][c0 .. c0+16) . v[k][q*16 .. q*16+16) for the calling lane's
// quarter q; cols beyond `cmax` (relative) are skipped.
__device__ inline void block_row_dot(const float2 *mrow, int q, int cmax, int nr,
                                     const float2 (*v)[kNB], float2 acc[kMaxRhs], bool valid)
{
    if (!valid) return;
#pragma unroll 4
    for (int c = 0; c < 16; ++c) {
        const int cc = q * 16 + c;
        if (cc >= cmax) break;
        const float2 m = mrow[cc];
#pragma unroll
        for (int k = 0; k < kMaxRhs; ++k) {
            if (k >= nr) break;
            const float2 y = v[k][cc];
            acc[k].x -= m.x * y.x - m.y * y.y;
            acc[k].y -= m.x * y.y + m.y * y.x;
        }
    }
}

__device__ inline float2 quarter_sum(float2 v)
{
    v.x += __shfl_xor(v.x, 1, 64);
    v.y += __shfl_xor(v.y, 1, 64);
    v.x += __shfl_xor(v.x, 2, 64);
    v.y += __shfl_xor(v.y, 2, 64);
    return v;
}

// y (nr x npad, complex64) = L^-1 fl32(r) for right-hand sides [0, nr)
__global__ __launch_bounds__(kTrsvThreads) void trsv_fwd_kernel(
    int64_t n, int64_t npad, int nr, const float *LU, const float *Dinv, const double *r128,
    const float *r64, float *Y, uint32_t *flags, uint32_t *counter, uint32_t epoch,
    uint64_t *err)
{
    __shared__ int sb, sok;
    __shared__ float2 vin[kMaxRhs][kNB];
    const int64_t nblk = (n + kNB - 1) / kNB;
    const int tid = threadIdx.x;
    if (tid == 0) {
        const uint32_t b = atomicAdd(counter, 1u);
        sb = b < uint32_t(nblk) ? int(b) : -1;
        if (int64_t(b) == nblk - 1) atomicExch(counter, 0u);   // every ticket is taken
    }
    __syncthreads();
    // a ticket outside [0, nblk) means the counter was not reset: refuse
    if (sb < 0 || int64_t(sb) >= nblk) {
        if (tid == 0) __hip_atomic_fetch_or(err, uint64_t(2), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    const int64_t b = sb;
    const int64_t r0 = b * kNB;
    const int i = tid >> 2, q = tid & 3;
    const bool valid = (r0 + i) < n;
    const float2 *L = reinterpret_cast<const float2 *>(LU);
    float2 *Yc = reinterpret_cast<float2 *>(Y);

    float2 acc[kMaxRhs];
#pragma unroll
    for (int k = 0; k < kMaxRhs; ++k) {
        acc[k] = make_float2(0.0f, 0.0f);
        if (k < nr && q == 0 && valid) {
            const size_t idx = size_t(k) * size_t(n) + size_t(r0 + i);
            if (r128) {
                const double2 v = reinterpret_cast<const double2 *>(r128)[idx];
                acc[k] = make_float2(float(v.x), float(v.y));
            } else {
                acc[k] = reinterpret_cast<const float2 *>(r64)[idx];
            }
        }
    }

    bool ok = true;
    for (int64_t j = 0; j < b && ok; ++j) {
        if (tid == 0) sok = wait_flag(flags + j, epoch, err) ? 1 : 0;
        __syncthreads();
        ok = sok != 0;
        if (!ok) break;
        (void)__hip_atomic_load(flags + j, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
        if (tid < nr * kNB) {
            const int k = tid / kNB, c = tid % kNB;
            vin[k][c] = Yc[size_t(k) * size_t(npad) + size_t(j * kNB + c)];
        }
        __syncthreads();
        block_row_dot(L + size_t(r0 + i) * size_t(n) + size_t(j * kNB), q, kNB, nr, vin, acc,
                      valid);
        __syncthreads();
    }

    // y_b = Linv_b acc
#pragma unroll
    for (int k = 0; k < kMaxRhs; ++k) acc[k] = quarter_sum(acc[k]);
    if (q == 0) {
#pragma unroll
        for (int k = 0; k < kMaxRhs; ++k)
            if (k < nr) vin[k][i] = acc[k];
    }
    __syncthreads();
    const float2 *Linv = reinterpret_cast<const float2 *>(Dinv) + size_t(b) * 2 * kNB * kNB;
    float2 y[kMaxRhs];
#pragma unroll
    for (int k = 0; k < kMaxRhs; ++k) y[k] = make_float2(0.0f, 0.0f);
    // y = Linv * v  ==  0 - (-Linv) v: reuse the subtracting dot with a sign flip
    block_row_dot(Linv + size_t(i) * kNB, q, kNB, nr, vin, y, true);
#pragma unroll
    for (int k = 0; k < kMaxRhs; ++k) {
        y[k] = quarter_sum(y[k]);
        if (k < nr && q == 0)
            Yc[size_t(k) * size_t(npad) + size_t(r0 + i)] = make_float2(-y[k].x, -y[k].y);
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) __hip_atomic_store(flags + b, epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// d = U^-1 y; X128 += d (when X128 is not NULL)
__global__ __launch_bounds__(kTrsvThreads) void trsv_bwd_kernel(
    int64_t n, int64_t npad, int nr, const float *LU, const float *Dinv, const float *Y,
    float *D, double *X128, uint32_t *flags, uint32_t *counter, uint32_t epoch, uint64_t *err)
{
    __shared__ int sb, sok;
    __shared__ float2 vin[kMaxRhs][kNB];
    const int64_t nblk = (n + kNB - 1) / kNB;
    const int tid = threadIdx.x;
    if (tid == 0) {
        const uint32_t t = atomicAdd(counter, 1u);
        sb = t < uint32_t(nblk) ? int(nblk - 1 - int64_t(t)) : -1;
        if (int64_t(t) == nblk - 1) atomicExch(counter, 0u);
    }
    __syncthreads();
    if (sb < 0 || int64_t(sb) >= nblk) {
        if (tid == 0) __hip_atomic_fetch_or(err, uint64_t(2), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    const int64_t b = sb;
    const int64_t r0 = b * kNB;
    const int i = tid >> 2, q = tid & 3;
    const bool valid = (r0 + i) < n;
    const float2 *U = reinterpret_cast<const float2 *>(LU);
    const float2 *Yc = reinterpret_cast<const float2 *>(Y);
    float2 *Dc = reinterpret_cast<float2 *>(D);

    float2 acc[kMaxRhs];
#pragma unroll
    for (int k = 0; k < kMaxRhs; ++k) {
        acc[k] = make_float2(0.0f, 0.0f);
        if (k < nr && q == 0) acc[k] = Yc[size_t(k) * size_t(npad) + size_t(r0 + i)];
    }

    bool ok = true;
    for (int64_t j = nblk - 1; j > b && ok; --j) {
        if (tid == 0) sok = wait_flag(flags + j, epoch, err) ? 1 : 0;
        __syncthreads();
        ok = sok != 0;
        if (!ok) break;
        (void)__hip_atomic_load(flags + j, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
        if (tid < nr * kNB) {
            const int k = tid / kNB, c = tid % kNB;
            vin[k][c] = Dc[size_t(k) * size_t(npad) + size_t(j * kNB + c)];
        }
        __syncthreads();
        const int cmax = int(min<int64_t>(kNB, n - j * kNB));
        block_row_dot(U + size_t(r0 + i) * size_t(n) + size_t(j * kNB), q, cmax, nr, vin, acc,
                      valid);
        __syncthreads();
    }

#pragma unroll
    for (int k = 0; k < kMaxRhs; ++k) acc[k] = quarter_sum(acc[k]);
    if (q == 0) {
#pragma unroll
        for (int k = 0; k < kMaxRhs; ++k)
            if (k < nr) vin[k][i] = acc[k];
    }
    __syncthreads();
    const float2 *Uinv = reinterpret_cast<const float2 *>(Dinv) + size_t(b) * 2 * kNB * kNB +
                         size_t(kNB) * kNB;
    float2 d[kMaxRhs];
#pragma unroll
    for (int k = 0; k < kMaxRhs; ++k) d[k] = make_float2(0.0f, 0.0f);
    block_row_dot(Uinv + size_t(i) * kNB, q, kNB, nr, vin, d, true);
#pragma unroll
    for (int k = 0; k < kMaxRhs; ++k) {
        d[k] = quarter_sum(d[k]);
        if (k < nr && q == 0) {
            const float2 v = make_float2(-d[k].x, -d[k].y);
            Dc[size_t(k) * size_t(npad) + size_t(r0 + i)] = v;
            if (X128 && valid) {
                double2 *xp = reinterpret_cast<double2 *>(X128) + size_t(k) * size_t(n) +
                              size_t(r0 + i);
                double2 xv = *xp;
                xv.x += double(v.x);
                xv.y += double(v.y);
                *xp = xv;
            }
        }
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) __hip_atomic_store(flags + b, epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

int launch_trsv_fwd(int64_t n, int64_t nrhs, const float *LU, const float *Dinv,
                    const double *r128, const float *r64, float *y, uint32_t *flags,
                    uint32_t *counter, uint32_t epoch, uint64_t *err, hipStream_t s)
{
    const int64_t nblk = nblocks(n);
    const int64_t npad = nblk * kNB;
    if (nrhs > kMaxRhs) return fail(MSOLVE_E_ARG, "trsv: at most 4 right-hand sides per launch");
    ProfScope prof(MSOLVE_K_TRSV_FWD, s, 4.0 * double(n) * double(n) + 8.0 * double(n) * double(nrhs));
    hipLaunchKernelGGL(trsv_fwd_kernel, dim3(unsigned(nblk)), dim3(kTrsvThreads), 0, s, n, npad,
                       int(nrhs), LU, Dinv, r128, r64, y, flags, counter, epoch, err);
    MS_HIP(hipGetLastError());
    return MSOLVE_OK;
}

int launch_trsv_bwd(int64_t n, int64_t nrhs, const float *LU, const float *Dinv,
                    const float *y, float *d, double *X128, uint32_t *flags,
                    uint32_t *counter, uint32_t epoch, uint64_t *err, hipStream_t s)
{
    const int64_t nblk = nblocks(n);
    const int64_t npad = nblk * kNB;
    if (nrhs > kMaxRhs) return fail(MSOLVE_E_ARG, "trsv: at most 4 right-hand sides per launch");
    ProfScope prof(MSOLVE_K_TRSV_BWD, s, 4.0 * double(n) * double(n) + 8.0 * double(n) * double(nrhs));
    hipLaunchKernelGGL(trsv_bwd_kernel, dim3(unsigned(nblk)), dim3(kTrsvThreads), 0, s, n, npad,
                       int(nrhs), LU, Dinv, y, d, X128, flags, counter, epoch, err);
    MS_HIP(hipGetLastError());
    return MSOLVE_OK;
}

}  // namespace msolve
