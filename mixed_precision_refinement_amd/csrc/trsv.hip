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
// already running).  Each of its four waves owns 16 rows of the block and
// walks the finished blocks of the solution on its own: one wave-wide load
// polls up to 64 ready counters, and every block found finished is consumed
// without further synchronisation (four lanes per row, 16 columns each).
// The diagonal block is applied from its inverse after one workgroup
// barrier; each wave then writes its rows and bumps the block's counter with
// a release increment (counters reach waves x epoch when a block is done).
// Every wait is bounded: on time-out the kernel raises a shared error word,
// every other wait sees it and gives up, and the host reports
// MSOLVE_E_DEVICE.
#include "common.hpp"

namespace msolve {
namespace {

constexpr int kTrsvThreads = 256;   // 4 waves x 16 rows x 4 quarter-row lanes
constexpr int kWaves = kTrsvThreads / 64;
constexpr int kMaxRhs = 4;          // right-hand sides per launch
constexpr uint32_t kSpinLimit = 1u << 22;

__device__ inline float2 quarter_sum(float2 v)
{
    v.x += __shfl_xor(v.x, 1, 64);
    v.y += __shfl_xor(v.y, 1, 64);
    v.x += __shfl_xor(v.x, 2, 64);
    v.y += __shfl_xor(v.y, 2, 64);
    return v;
}

// Wave-wide poll of up to 64 ready counters: returns how many consecutive
// blocks, starting at `j` and stepping by `dir`, have all kWaves writers done
// (counter >= target), at most `avail`.  Every lane's load is an acquire, so
// the blocks it reports are visible to the whole wave.
__device__ inline int poll_ready(const uint32_t *flags, int64_t j, int dir, int avail,
                                 uint32_t target)
{
    const int lane = threadIdx.x & 63;
    // every lane performs an acquire (lanes past `avail` re-read the last
    // flag), so each lane's later loads are ordered after it
    const int t = min(lane, avail - 1);
    const uint32_t v = __hip_atomic_load(flags + (j + dir * t), __ATOMIC_ACQUIRE,
                                         __HIP_MEMORY_SCOPE_AGENT);
    const bool ok = lane >= avail || v >= target;
    const uint64_t ready = __ballot(ok);
    const int cnt = (~ready == 0) ? 64 : __builtin_ctzll(~ready);
    return min(cnt, avail);
}

// acc[k] -= M[row][c .. c+16) . v[k][c .. c+16) for the calling lane's
// 16 columns; columns at or beyond `cmax` count as zero.  All loads are
// issued before any arithmetic (clamped addresses, masked values), so a
// block costs one memory round trip.
template <int NR>
__device__ inline void quarter_dot(const float2 *mrow, const float2 *v, int64_t vstride, int cmax,
                                   float2 acc[NR])
{
    float2 mv[16], yv[NR][16];
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        const int cc = c < cmax ? c : 0;
        mv[c] = mrow[cc];
#pragma unroll
        for (int k = 0; k < NR; ++k) yv[k][c] = v[size_t(k) * size_t(vstride) + cc];
    }
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        const float2 m = c < cmax ? mv[c] : make_float2(0.0f, 0.0f);
#pragma unroll
        for (int k = 0; k < NR; ++k) {
            acc[k].x -= m.x * yv[k][c].x - m.y * yv[k][c].y;
            acc[k].y -= m.x * yv[k][c].y + m.y * yv[k][c].x;
        }
    }
}

// FWD: y = L^-1 fl32(r).  BWD: d = U^-1 y and X128 += d.
// src128/src64: right-hand side (FWD: r as complex128 or complex64 rows of
// n; BWD: y as complex64 rows of npad).  out: complex64 rows of npad.
template <bool FWD, int NR>
__global__ __launch_bounds__(kTrsvThreads) void trsv_kernel(
    int64_t n, int64_t npad, const float *LU, const float *Dinv, const double *src128,
    const float *src64, float *out, double *X128, uint32_t *flags, uint32_t *counter,
    uint32_t epoch, uint64_t *err)
{
    __shared__ int sb;
    __shared__ float2 vin[kMaxRhs][kNB];
    const int64_t nblk = (n + kNB - 1) / kNB;
    const int tid = threadIdx.x;
    if (tid == 0) {
        const uint32_t t = atomicAdd(counter, 1u);
        sb = t < uint32_t(nblk) ? (FWD ? int(t) : int(nblk - 1 - int64_t(t))) : -1;
        if (int64_t(t) == nblk - 1) atomicExch(counter, 0u);   // every ticket is taken
    }
    __syncthreads();
    // a ticket outside [0, nblk) means the counter was not reset: refuse
    if (sb < 0) {
        if (tid == 0) __hip_atomic_fetch_or(err, uint64_t(2), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    const int64_t b = sb;
    const int64_t r0 = b * kNB;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int i = wave * 16 + (lane >> 2);   // row within the block
    const int q = lane & 3;
    const bool valid = (r0 + i) < n;
    const float2 *F = reinterpret_cast<const float2 *>(LU);
    float2 *O = reinterpret_cast<float2 *>(out);
    const uint32_t target = uint32_t(kWaves) * epoch;

    float2 acc[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) {
        acc[k] = make_float2(0.0f, 0.0f);
        if (q == 0 && valid) {
            if (FWD) {
                const size_t idx = size_t(k) * size_t(n) + size_t(r0 + i);
                if (src128) {
                    const double2 v = reinterpret_cast<const double2 *>(src128)[idx];
                    acc[k] = make_float2(float(v.x), float(v.y));
                } else {
                    acc[k] = reinterpret_cast<const float2 *>(src64)[idx];
                }
            } else {
                acc[k] = reinterpret_cast<const float2 *>(src64)[size_t(k) * size_t(npad) + size_t(r0 + i)];
            }
        }
    }

    // off-diagonal blocks, in dependency order, batch by batch as they finish
    const int dir = FWD ? 1 : -1;
    int64_t j = FWD ? 0 : nblk - 1;
    int64_t left = FWD ? b : (nblk - 1 - b);
    const float2 *frow = F + size_t(r0 + i) * size_t(n) + size_t(q * 16);
    uint32_t spins = 0;
    while (left > 0) {
        const int avail = int(min<int64_t>(left, 64));
        const int ready = poll_ready(flags, j, dir, avail, target);
        if (ready == 0) {
            if (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) break;
            if (++spins > kSpinLimit) {
                if (lane == 0)
                    __hip_atomic_fetch_or(err, uint64_t(1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
            continue;
        }
        for (int t = 0; t < ready; ++t, j += dir) {
            const int cmax = int(min<int64_t>(16, n - (j * kNB + q * 16)));
            if (valid && cmax > 0)
                quarter_dot<NR>(frow + size_t(j * kNB), O + size_t(j * kNB + q * 16), npad, cmax, acc);
        }
        left -= ready;
    }

    // diagonal block: out_b = Dinv_b acc
#pragma unroll
    for (int k = 0; k < NR; ++k) acc[k] = quarter_sum(acc[k]);
    if (q == 0) {
#pragma unroll
        for (int k = 0; k < NR; ++k) vin[k][i] = acc[k];
    }
    __syncthreads();
    const float2 *D = reinterpret_cast<const float2 *>(Dinv) + size_t(b) * 2 * kNB * kNB +
                      (FWD ? 0 : size_t(kNB) * kNB);
    float2 o[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) o[k] = make_float2(0.0f, 0.0f);
    quarter_dot<NR>(D + size_t(i) * kNB + q * 16, &vin[0][q * 16], kNB, 16, o);   // o = -D v
#pragma unroll
    for (int k = 0; k < NR; ++k) {
        o[k] = quarter_sum(o[k]);
        if (q == 0) {
            const float2 v = make_float2(-o[k].x, -o[k].y);
            O[size_t(k) * size_t(npad) + size_t(r0 + i)] = v;
            if (!FWD && X128 && valid) {
                double2 *xp = reinterpret_cast<double2 *>(X128) + size_t(k) * size_t(n) + size_t(r0 + i);
                double2 xv = *xp;
                xv.x += double(v.x);
                xv.y += double(v.y);
                *xp = xv;
            }
        }
    }
    // publish this wave's 16 rows: kWaves increments per block and launch
    __threadfence();
    if (lane == 0)
        __hip_atomic_fetch_add(flags + b, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
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
    switch (nrhs) {
#define MS_FWD(NRV) case NRV: hipLaunchKernelGGL((trsv_kernel<true, NRV>), dim3(unsigned(nblk)), \
        dim3(kTrsvThreads), 0, s, n, npad, LU, Dinv, r128, r64, y, nullptr, flags, counter, epoch, err); break;
    MS_FWD(1) MS_FWD(2) MS_FWD(3) MS_FWD(4)
#undef MS_FWD
    default: return fail(MSOLVE_E_ARG, "trsv: bad right-hand side count");
    }
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
    switch (nrhs) {
#define MS_BWD(NRV) case NRV: hipLaunchKernelGGL((trsv_kernel<false, NRV>), dim3(unsigned(nblk)), \
        dim3(kTrsvThreads), 0, s, n, npad, LU, Dinv, nullptr, y, d, X128, flags, counter, epoch, err); break;
    MS_BWD(1) MS_BWD(2) MS_BWD(3) MS_BWD(4)
#undef MS_BWD
    default: return fail(MSOLVE_E_ARG, "trsv: bad right-hand side count");
    }
    MS_HIP(hipGetLastError());
    return MSOLVE_OK;
}

}  // namespace msolve
