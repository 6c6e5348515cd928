// Triangular solves with the single-precision factors (steps 2 and 4 of the
// refinement list in the section "Double-precision answers from a GPU
// without double precision" of the page "Solving Dense Matrices Fast in the
// Browser": solve with the factorisation for x, then for each correction).
//
// Forward:  L y = fl32(r)     y_b = Linv_b (r_b - sum_{j<b} L_bj y_j)
// Back:     U d = y           d_b = Uinv_b (y_b - sum_{j>b} U_bj d_j)
// with Linv_b, Uinv_b the inverses of the diagonal blocks (here of 128 rows)
// that the factorisation leaves.
//
// One persistent launch per direction for a batch of systems.  The rows go
// in 128-row blocks (pairs of the factorisation's 64-row blocks), whose
// inverses the factorisation provides: the inverses of the two diagonal
// blocks and the coupling block of each pair.  A workgroup takes a
// (system, pair) from an atomic ticket in dependency order (so every block
// it waits for is already running).  Each of its eight waves owns 16 rows
// and walks the finished pairs of the solution on its own: one wave-wide
// load polls up to 64 ready counters, and every pair found finished is
// consumed without further synchronisation (four lanes per row, 16 columns
// of each 64-column block, interleaved in pairs so that a row's lanes read
// contiguous memory).  The pair's own 128 x 128 triangle is then applied
// from its inverse after one workgroup barrier; each wave writes its rows
// and bumps the pair's counter after a release fence (counters reach
// waves x epoch when a pair is done).  Every wait is bounded: on time-out
// the kernel raises a shared error word, every other wait sees it and gives
// up, and the host reports MSOLVE_E_DEVICE.
#include "common.hpp"

namespace msolve {
namespace {

constexpr int kSub = 2;                    // 64-row blocks per workgroup
constexpr int kTrsvThreads = 256 * kSub;   // 4 waves x 16 rows x 4 quarter-row lanes per block
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
// (counter >= target), at most `avail`.  The counters are read with relaxed
// loads; only a poll that finds work is followed by one agent-scope acquire
// fence, executed by the whole wave, which orders the wave's later loads of
// the reported blocks after the producers' release fences.  (An acquire on
// every poll would invalidate the cache on every spin of every waiting wave,
// which costs several microseconds per hand-off once many waves wait.)
__device__ inline int poll_ready(const uint32_t *flags, int64_t j, int dir, int avail,
                                 uint32_t target)
{
    const int lane = threadIdx.x & 63;
    const int t = min(lane, avail - 1);
    const uint32_t v = __hip_atomic_load(flags + (j + dir * t), __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    const bool ok = lane >= avail || v >= target;
    const uint64_t ready = __ballot(ok);
    const int cnt = min((~ready == 0) ? 64 : __builtin_ctzll(~ready), avail);
    if (cnt > 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    return cnt;
}

// Two consecutive complex64 values, read with one 16-byte load; 8-byte
// alignment is all that a matrix row of odd length guarantees.
struct __attribute__((aligned(8))) cpair {
    float2 a, b;
};

__device__ inline void cfms_acc(float2 &acc, float2 m, float2 y)
{
    acc.x -= m.x * y.x - m.y * y.y;
    acc.y -= m.x * y.y + m.y * y.x;
}

// acc[k] -= M[row][0 .. 64) . v[k][0 .. 64) over the calling lane's share of
// a 64-column block: lane q of a row takes the column pairs 8c + 2q, 8c + 2q
// + 1 (c = 0..7), so the four lanes of a row read 64 contiguous bytes per
// load and one wave-wide load touches 16 matrix lines and a single line of
// v.  Columns at or beyond `cmax` count as zero (only the last block of the
// matrix is ragged; it clamps its addresses and masks the values).  All
// loads are issued before the arithmetic: a block costs one round trip (two
// for three or four right-hand sides).
template <int NR>
__device__ inline void block_dot(const float2 *mrow, const float2 *v, int64_t vstride, int cmax,
                                 int q, float2 acc[NR])
{
    if (cmax >= kNB) {
        // three or four right-hand sides: two halves, to stay in registers
        constexpr int CH = NR <= 2 ? 8 : 4;
#pragma unroll
        for (int c0 = 0; c0 < 8; c0 += CH) {
            cpair mv[CH], yv[NR][CH];
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                mv[c] = *reinterpret_cast<const cpair *>(mrow + 8 * (c0 + c) + 2 * q);
#pragma unroll
                for (int k = 0; k < NR; ++k)
                    yv[k][c] = *reinterpret_cast<const cpair *>(v + size_t(k) * size_t(vstride) + 8 * (c0 + c) + 2 * q);
            }
#pragma unroll
            for (int c = 0; c < CH; ++c) {
#pragma unroll
                for (int k = 0; k < NR; ++k) {
                    cfms_acc(acc[k], mv[c].a, yv[k][c].a);
                    cfms_acc(acc[k], mv[c].b, yv[k][c].b);
                }
            }
        }
    } else {
        float2 mv[16], yv[NR][16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int col = 8 * (e >> 1) + 2 * q + (e & 1);
            const int cc = col < cmax ? col : 0;
            mv[e] = mrow[cc];
#pragma unroll
            for (int k = 0; k < NR; ++k) yv[k][e] = v[size_t(k) * size_t(vstride) + cc];
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int col = 8 * (e >> 1) + 2 * q + (e & 1);
            const float2 m = col < cmax ? mv[e] : make_float2(0.0f, 0.0f);
#pragma unroll
            for (int k = 0; k < NR; ++k) cfms_acc(acc[k], m, yv[k][e]);
        }
    }
}

// FWD: y = L^-1 fl32(r).  BWD: d = U^-1 y and X128 += d.
// src128/src64: right-hand side (FWD: r as complex128 or complex64 rows of
// n; BWD: y as complex64 rows of npad).  out: complex64 rows of npad.
// A launch solves a batch of nf independent systems: ticket t takes block
// t / nf of system t % nf, so a workgroup only waits for blocks of its own
// system with smaller tickets.
struct TrsvArgs {
    int64_t n, npad, nf;
    const float *LU, *Dinv;
    const double *src128;
    const float *src64;
    float *out;
    double *X128;
    int64_t sLU, sD, sSrc, sOut, sX;   // strides between systems
    const uint32_t *active;            // nullable: systems with a 0 entry are skipped
    uint32_t *flags;                   // one ready counter per super-block and system
    uint32_t *counter;
    uint32_t epoch;
    uint64_t *err;
};

// Loads row `mrow` of a 64-column block into the calling lane's column
// pairs (8c + 2q, 8c + 2q + 1), zero beyond `cmax` columns.
__device__ inline void load_block_row(const float2 *mrow, int cmax, int q, cpair m[8])
{
    if (cmax >= kNB) {
#pragma unroll
        for (int c = 0; c < 8; ++c) m[c] = *reinterpret_cast<const cpair *>(mrow + 8 * c + 2 * q);
    } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int c0 = 8 * c + 2 * q;
            m[c].a = c0 < cmax ? mrow[c0] : make_float2(0.0f, 0.0f);
            m[c].b = c0 + 1 < cmax ? mrow[c0 + 1] : make_float2(0.0f, 0.0f);
        }
    }
}

// acc[k] -= m . v[k] over the lane's column pairs of one block (v in LDS,
// rows of kNB complex, one per right-hand side)
template <int NR>
__device__ inline void apply_block_row(const cpair m[8], const float2 (*v)[kNB], int q, float2 acc[NR])
{
#pragma unroll
    for (int c = 0; c < 8; ++c) {
#pragma unroll
        for (int k = 0; k < NR; ++k) {
            const cpair y = *reinterpret_cast<const cpair *>(&v[k][8 * c + 2 * q]);
            cfms_acc(acc[k], m[c].a, y.a);
            cfms_acc(acc[k], m[c].b, y.b);
        }
    }
}

// A workgroup solves a pair of consecutive 64-row blocks (waves 0-3: the
// first block, 4-7: the second) as one 128-row block.  The finished pairs
// are consumed as they appear; then the pair's own 128 x 128 triangle is
// applied from its inverse in one step: each row takes the row of its own
// block's inverse and, where the inverse couples the two blocks (the second
// block of the forward solve, the first of the back solve), the row of the
// coupling block (from the factorisation's Dinv), both against the reduced
// right-hand sides of the pair.  Every needed inverse row is loaded before
// the wait.  One hand-off per 128 rows.
template <bool FWD, int NR>
__global__ __launch_bounds__(kTrsvThreads) void trsv_kernel(TrsvArgs a)
{
    static_assert(kSub == 2, "pairs of blocks");
    __shared__ int sb;
    __shared__ __align__(16) float2 vin[kSub][kMaxRhs][kNB];    // reduced right-hand sides
    const int64_t n = a.n, npad = a.npad;
    const int64_t nblk = (n + kNB - 1) / kNB;
    const int64_t nsb = (nblk + kSub - 1) / kSub;
    const int64_t total = nsb * a.nf;
    const int tid = threadIdx.x;
    if (tid == 0) {
        const uint32_t t = atomicAdd(a.counter, 1u);
        sb = t < uint32_t(total) ? int(t) : -1;
        if (int64_t(t) == total - 1) atomicExch(a.counter, 0u);   // every ticket is taken
    }
    __syncthreads();
    // a ticket outside [0, total) means the counter was not reset: refuse
    if (sb < 0) {
        if (tid == 0) __hip_atomic_fetch_or(a.err, uint64_t(2), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    const int64_t f = sb % a.nf;
    const int64_t st = sb / a.nf;
    if (a.active && a.active[f] == 0) return;
    const int64_t S = FWD ? st : nsb - 1 - st;                  // pair
    const float *LU = a.LU + size_t(f) * size_t(a.sLU);
    const float *Dinv = a.Dinv + size_t(f) * size_t(a.sD);
    const double *src128 = a.src128 ? a.src128 + size_t(f) * size_t(a.sSrc) : nullptr;
    const float *src64 = a.src64 ? a.src64 + size_t(f) * size_t(a.sSrc) : nullptr;
    float *out = a.out + size_t(f) * size_t(a.sOut);
    double *X128 = a.X128 ? a.X128 + size_t(f) * size_t(a.sX) : nullptr;
    uint32_t *flags = a.flags + size_t(f) * size_t(nsb);
    uint64_t *err = a.err;
    const uint32_t epoch = a.epoch;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = wave / 4;                                  // block of the pair
    const int i = (wave % 4) * 16 + (lane >> 2);                // row within the block
    const int q = lane & 3;
    const int64_t b = S * kSub + half;                          // this wave's block
    const bool bvalid = b < nblk;                               // uniform
    const int64_t r0 = b * kNB;
    const bool valid = bvalid && (r0 + i) < n;
    const bool paired = S * kSub + 1 < nblk;                    // uniform
    const bool coupled = paired && (FWD ? half == 1 : half == 0);
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

    // this row of the pair's inverse, loaded while the blocks it depends on
    // are still being solved: the own block's inverse row and the coupling
    // row (forward: X = -Li1 L10 Li0 in front of Li1; back: Y = -Ui0 U01 Ui1
    // behind Ui0)
    const float2 *Dc = reinterpret_cast<const float2 *>(Dinv);
    cpair d_own[8], d_cpl[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        d_own[c].a = d_own[c].b = make_float2(0.0f, 0.0f);
        d_cpl[c].a = d_cpl[c].b = make_float2(0.0f, 0.0f);
    }
    if (bvalid)
        load_block_row(Dc + size_t(b) * 2 * kNB * kNB + (FWD ? 0 : size_t(kNB) * kNB) + size_t(i) * kNB,
                       kNB, q, d_own);
    if (coupled)
        load_block_row(Dc + (size_t(nblk) + size_t(S)) * 2 * kNB * kNB + (FWD ? 0 : size_t(kNB) * kNB) +
                           size_t(i) * kNB, kNB, q, d_cpl);

    // finished pairs, in dependency order, batch by batch as they finish
    const int dir = FWD ? 1 : -1;
    int64_t J = FWD ? 0 : nsb - 1;
    int64_t left = FWD ? S : (nsb - 1 - S);
    const float2 *frow = F + size_t(valid ? r0 + i : 0) * size_t(n);
    uint32_t spins = 0;
    while (left > 0) {
        const int avail = int(min<int64_t>(left, 64));
        const int ready = poll_ready(flags, J, dir, avail, target);
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
        if (valid) {
            for (int t = 0; t < ready; ++t, J += dir) {
#pragma unroll
                for (int s2 = 0; s2 < kSub; ++s2) {
                    const int64_t bj = J * kSub + s2;
                    if (bj < nblk) {
                        const int cmax = int(min<int64_t>(kNB, n - bj * kNB));
                        block_dot<NR>(frow + size_t(bj * kNB), O + size_t(bj * kNB), npad, cmax, q, acc);
                    }
                }
            }
        } else {
            J += dir * ready;
        }
        left -= ready;
    }

    // the pair's 128-row block: out = (inverse row) . (reduced right-hand sides)
#pragma unroll
    for (int k = 0; k < NR; ++k) {
        const float2 v = quarter_sum(acc[k]);
        if (q == 0) vin[half][k][i] = v;
    }
    __syncthreads();
    float2 o[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) o[k] = make_float2(0.0f, 0.0f);
    if (bvalid) {
        apply_block_row<NR>(d_own, vin[half], q, o);            // o = -(own inverse row) v
        if (coupled) apply_block_row<NR>(d_cpl, vin[1 - half], q, o);
#pragma unroll
        for (int k = 0; k < NR; ++k) {
            o[k] = quarter_sum(o[k]);
            o[k] = make_float2(-o[k].x, -o[k].y);
            if (q == 0) O[size_t(k) * size_t(npad) + size_t(r0 + i)] = o[k];
        }
    }

    // publish this wave's rows: kWaves increments per pair and launch
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    if (lane == 0)
        __hip_atomic_fetch_add(flags + S, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // the complex128 solution update is read by later launches only
    if (!FWD && X128 && valid && q == 0) {
#pragma unroll
        for (int k = 0; k < NR; ++k) {
            double2 *xp = reinterpret_cast<double2 *>(X128) + size_t(k) * size_t(n) + size_t(r0 + i);
            double2 xv = *xp;
            xv.x += double(o[k].x);
            xv.y += double(o[k].y);
            *xp = xv;
        }
    }
}

}  // namespace

namespace {

int launch_trsv(bool fwd, int64_t n, int64_t nrhs, const TrsvBatch &tb, const float *LU,
                const float *Dinv, const double *src128, const float *src64, float *out,
                double *X128, uint32_t *flags, uint32_t *counter, uint32_t epoch, uint64_t *err,
                hipStream_t s)
{
    const int64_t nblk = nblocks(n);
    const int64_t nsb = (nblk + kSub - 1) / kSub;
    if (nrhs < 1 || nrhs > kMaxRhs) return fail(MSOLVE_E_ARG, "trsv: 1 to 4 right-hand sides per launch");
    TrsvArgs a;
    a.n = n; a.npad = nblk * kNB; a.nf = tb.nf;
    a.LU = LU; a.Dinv = Dinv; a.src128 = src128; a.src64 = src64; a.out = out; a.X128 = X128;
    a.sLU = tb.sLU; a.sD = tb.sD; a.sSrc = tb.sSrc; a.sOut = tb.sOut; a.sX = tb.sX;
    a.active = tb.active;
    a.flags = flags; a.counter = counter; a.epoch = epoch; a.err = err;
    const unsigned grid = unsigned(nsb * tb.nf);
    ProfScope prof(fwd ? MSOLVE_K_TRSV_FWD : MSOLVE_K_TRSV_BWD, s,
                   (4.0 * double(n) * double(n) + 8.0 * double(n) * double(nrhs)) * double(tb.nf));
#define MS_TRSV(NRV)                                                                          \
    case NRV:                                                                                 \
        if (fwd) hipLaunchKernelGGL((trsv_kernel<true, NRV>), dim3(grid), dim3(kTrsvThreads), 0, s, a); \
        else hipLaunchKernelGGL((trsv_kernel<false, NRV>), dim3(grid), dim3(kTrsvThreads), 0, s, a);   \
        break;
    switch (nrhs) {
        MS_TRSV(1) MS_TRSV(2) MS_TRSV(3) MS_TRSV(4)
    }
#undef MS_TRSV
    MS_HIP(hipGetLastError());
    return MSOLVE_OK;
}

}  // namespace

int launch_trsv_fwd(int64_t n, int64_t nrhs, const TrsvBatch &tb, const float *LU,
                    const float *Dinv, const double *r128, const float *r64, float *y,
                    uint32_t *flags, uint32_t *counter, uint32_t epoch, uint64_t *err,
                    hipStream_t s)
{
    return launch_trsv(true, n, nrhs, tb, LU, Dinv, r128, r64, y, nullptr, flags, counter, epoch,
                       err, s);
}

int launch_trsv_bwd(int64_t n, int64_t nrhs, const TrsvBatch &tb, const float *LU,
                    const float *Dinv, const float *y, float *d, double *X128, uint32_t *flags,
                    uint32_t *counter, uint32_t epoch, uint64_t *err, hipStream_t s)
{
    return launch_trsv(false, n, nrhs, tb, LU, Dinv, nullptr, y, d, X128, flags, counter, epoch,
                       err, s);
}

}  // namespace msolve
