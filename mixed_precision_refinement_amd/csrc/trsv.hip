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
// blocks and the coupling block of each pair.  A workgroup of 16 waves takes
// a (system, pair) from an atomic ticket in dependency order (so every block
// it waits for is already running).  Each wave owns 8 rows, eight lanes per
// row.  One wave polls the ready counters of the finished pairs and copies
// their values into LDS; a workgroup barrier hands them to every wave.  The
// matrix rows of the next pair are loaded into registers before the wait,
// and the pair's inverse blocks into LDS when the workgroup starts, so a
// hand-off costs one load of the finished solution values.  The pair's own
// 128 x 128 triangle is then applied from its inverse after one more
// workgroup barrier; the waves write their rows, and after a barrier one
// release fence and one increment of the pair's counter publish them
// (counters reach the launch's epoch when a pair is done).  Every wait is
// bounded: on time-out the kernel raises a shared error word, every other
// wait sees it and gives up, and the host reports MSOLVE_E_DEVICE.
#include "common.hpp"

namespace msolve {
namespace {

constexpr int kSub = 2;                   // 64-row blocks per workgroup
constexpr int kLanesPerRow = 8;
constexpr int kTrsvThreads = kSub * kNB * kLanesPerRow;   // 1024
constexpr int kWaves = kTrsvThreads / 64;                 // 16
constexpr int kRowsPerWave = 64 / kLanesPerRow;           // 8
constexpr int kCp = kNB / (2 * kLanesPerRow);             // column pairs per lane and block: 4
constexpr int kMaxRhs = 4;                // right-hand sides per launch
constexpr uint32_t kSpinLimit = 1u << 22;
constexpr int kRound = 4;                 // finished pairs staged per round

// sum over the eight lanes of a row
__device__ inline float2 row_sum(float2 v)
{
#pragma unroll
    for (int m = 1; m < kLanesPerRow; m <<= 1) {
        v.x += __shfl_xor(v.x, m, 64);
        v.y += __shfl_xor(v.y, m, 64);
    }
    return v;
}

// Wave-wide poll of up to 64 ready counters: returns how many consecutive
// blocks, starting at `j` and stepping by `dir`, are done (counter >=
// target), at most `avail`.  The counters are read with relaxed
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

// The lane's column pairs of a 64-column block: lane q of a row takes
// columns 16c + 2q and 16c + 2q + 1 (c = 0..3), so the eight lanes of a row
// read 128 contiguous bytes per load.  Columns at or beyond `cmax` count as
// zero (only the last block of the matrix is ragged; it clamps its
// addresses and masks the values).
__device__ inline void load_cols(const float2 *src, int cmax, int q, cpair v[kCp])
{
    if (cmax >= kNB) {
#pragma unroll
        for (int c = 0; c < kCp; ++c) v[c] = *reinterpret_cast<const cpair *>(src + 16 * c + 2 * q);
    } else {
#pragma unroll
        for (int c = 0; c < kCp; ++c) {
            const int c0 = 16 * c + 2 * q;
            const float2 a = src[c0 < cmax ? c0 : 0], b = src[c0 + 1 < cmax ? c0 + 1 : 0];
            v[c].a = c0 < cmax ? a : make_float2(0.0f, 0.0f);
            v[c].b = c0 + 1 < cmax ? b : make_float2(0.0f, 0.0f);
        }
    }
}

// FWD: y = L^-1 fl32(r).  BWD: d = U^-1 y and X128 += d.
// src128/src64: right-hand side (FWD: r as complex128 or complex64 rows of
// n; BWD: y as complex64 rows of npad).  out: complex64 rows of npad.
// A launch solves a batch of nf independent systems: ticket t takes pair
// t / nf of system t % nf, so a workgroup only waits for pairs of its own
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
    uint32_t *flags;                   // one ready counter per pair and system
    uint32_t *counter;
    uint32_t epoch;
    uint64_t *err;
};

// A workgroup solves a pair of consecutive 64-row blocks (waves 0-7: the
// first block, 8-15: the second) as one 128-row block.  The finished pairs
// are consumed as they appear; then the pair's own 128 x 128 triangle is
// applied from its inverse in one step: each row takes the row of its own
// block's inverse and, where the inverse couples the two blocks (the second
// block of the forward solve, the first of the back solve), the row of the
// coupling block, both against the reduced right-hand sides of the pair.
// One hand-off per 128 rows.
template <bool FWD, int NR>
__global__ __launch_bounds__(kTrsvThreads) void trsv_kernel(TrsvArgs a)
{
    static_assert(kSub == 2, "pairs of blocks");
    __shared__ int sb;
    __shared__ __align__(16) float2 inv[3][kNB][kNB];              // own inverses of the two blocks, coupling
    __shared__ __align__(16) float2 ys[2][kRound][kMaxRhs][kSub * kNB];   // finished pairs, two rounds
    __shared__ int round_cnt[2];
    __shared__ __align__(16) float2 vin[kSub][kMaxRhs][kNB];       // reduced right-hand sides
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
    const int half = wave / (kWaves / 2);                       // block of the pair
    const int i = (wave % (kWaves / 2)) * kRowsPerWave + lane / kLanesPerRow;   // row within the block
    const int q = lane % kLanesPerRow;
    const int64_t b = S * kSub + half;                          // this wave's block
    const bool bvalid = b < nblk;                               // uniform
    const int64_t r0 = b * kNB;
    const bool valid = bvalid && (r0 + i) < n;
    const bool paired = S * kSub + 1 < nblk;                    // uniform
    const bool coupled = paired && (FWD ? half == 1 : half == 0);
    const float2 *F = reinterpret_cast<const float2 *>(LU);
    float2 *O = reinterpret_cast<float2 *>(out);
    const uint32_t target = epoch;

    // the pair's inverse blocks into LDS (read after the barrier that
    // precedes the triangle step): the two diagonal blocks' inverses and the
    // coupling block (forward: X = -Li1 L10 Li0 below Li0; back:
    // Y = -Ui0 U01 Ui1 beside Ui1)
    {
        const float4 *Dq = reinterpret_cast<const float4 *>(Dinv);
        float4 *Iq = reinterpret_cast<float4 *>(&inv[0][0][0]);
        constexpr int Q = kNB * kNB / 2;                        // float4 per block
        const size_t up = FWD ? 0 : size_t(Q);
        const size_t src0 = size_t(S * kSub) * 2 * Q + up;
        const size_t src1 = size_t(S * kSub + 1) * 2 * Q + up;
        const size_t srcc = (size_t(nblk) + size_t(S)) * 2 * Q + up;
        for (int e = tid; e < 3 * Q; e += kTrsvThreads) {
            const int blk = e / Q, o = e % Q;
            const bool have = blk == 0 || paired;
            Iq[e] = have ? Dq[(blk == 0 ? src0 : blk == 1 ? src1 : srcc) + size_t(o)]
                         : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
    }

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

    // finished pairs, in dependency order, one after another as they finish;
    // the matrix values of the pair waited for are already in registers
    const int dir = FWD ? 1 : -1;
    int64_t J = FWD ? 0 : nsb - 1;
    int64_t left = FWD ? S : (nsb - 1 - S);
    const float2 *frow = F + size_t(valid ? r0 + i : 0) * size_t(n);
    cpair m[kSub][kCp];
    auto fetch = [&](int64_t Jp) {
#pragma unroll
        for (int s2 = 0; s2 < kSub; ++s2) {
            const int64_t bj = Jp * kSub + s2;
            const int cmax = bj < nblk ? int(min<int64_t>(kNB, n - bj * kNB)) : 0;
            load_cols(frow + size_t(bj < nblk ? bj * kNB : 0), cmax, q, m[s2]);
        }
    };
    if (valid && left > 0) fetch(J);
    // Rounds: wave 0 alone polls the ready counters (one poller per
    // workgroup keeps the polling traffic low), acquires, and copies the
    // values of up to kRound newly finished pairs into LDS (columns at and
    // beyond n as zero); one barrier hands them to every wave.  The two LDS
    // buffers alternate, so wave 0 fills the next round while the others
    // still read this one; the barrier of the next round orders the reuse.
    uint32_t spins = 0;
    int rb = 0;
    while (left > 0) {
        if (wave == 0) {
            int cnt = 0;
            while (true) {
                cnt = poll_ready(flags, J, dir, int(min<int64_t>(left, kRound)), target);
                if (cnt > 0) break;
                if (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) {
                    cnt = -1;
                    break;
                }
                if (++spins > kSpinLimit) {
                    if (lane == 0)
                        __hip_atomic_fetch_or(err, uint64_t(1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    cnt = -1;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
            for (int t = 0; t < cnt; ++t) {
                const int64_t c0 = (J + dir * t) * kSub * kNB + 2 * lane;
#pragma unroll
                for (int k = 0; k < NR; ++k) {
                    const float2 *src = O + size_t(k) * size_t(npad) + size_t(c0);
                    float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                    if (c0 + 1 < n) {
                        v = *reinterpret_cast<const float4 *>(src);
                    } else if (c0 < n) {
                        const float2 u = src[0];
                        v = make_float4(u.x, u.y, 0.0f, 0.0f);
                    }
                    *reinterpret_cast<float4 *>(&ys[rb][t][k][2 * lane]) = v;
                }
            }
            if (lane == 0) round_cnt[rb] = cnt;
        }
        __syncthreads();
        const int cnt = round_cnt[rb];
        if (cnt < 0) break;
        for (int t = 0; t < cnt; ++t) {
            if (valid) {
                if (t > 0) fetch(J);
#pragma unroll
                for (int s2 = 0; s2 < kSub; ++s2) {
#pragma unroll
                    for (int k = 0; k < NR; ++k) {
#pragma unroll
                        for (int c = 0; c < kCp; ++c) {
                            const cpair y = *reinterpret_cast<const cpair *>(&ys[rb][t][k][s2 * kNB + 16 * c + 2 * q]);
                            cfms_acc(acc[k], m[s2][c].a, y.a);
                            cfms_acc(acc[k], m[s2][c].b, y.b);
                        }
                    }
                }
            }
            J += dir;
            --left;
        }
        // the matrix values of the next pair, loaded while waiting for it
        if (valid && left > 0) fetch(J);
        rb ^= 1;
    }

    // the pair's 128-row block: out = (inverse row) . (reduced right-hand sides)
#pragma unroll
    for (int k = 0; k < NR; ++k) {
        const float2 v = row_sum(acc[k]);
        if (q == 0) vin[half][k][i] = v;
    }
    __syncthreads();
    float2 o[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) o[k] = make_float2(0.0f, 0.0f);
    if (bvalid) {
        // o -= (own inverse row) v, then -= (coupling row) v of the other block
#pragma unroll
        for (int part = 0; part < 2; ++part) {
            if (part == 1 && !coupled) break;
            const float2 *irow = &inv[part == 0 ? half : 2][i][0];
            const int vb = part == 0 ? half : 1 - half;
#pragma unroll
            for (int c = 0; c < kCp; ++c) {
                const cpair mv = *reinterpret_cast<const cpair *>(irow + 16 * c + 2 * q);
#pragma unroll
                for (int k = 0; k < NR; ++k) {
                    const cpair y = *reinterpret_cast<const cpair *>(&vin[vb][k][16 * c + 2 * q]);
                    cfms_acc(o[k], mv.a, y.a);
                    cfms_acc(o[k], mv.b, y.b);
                }
            }
        }
#pragma unroll
        for (int k = 0; k < NR; ++k) {
            o[k] = row_sum(o[k]);
            o[k] = make_float2(-o[k].x, -o[k].y);
            if (q == 0) O[size_t(k) * size_t(npad) + size_t(r0 + i)] = o[k];
        }
    }

    // publish the pair: after a barrier (every wave's rows are written), one
    // release fence and one increment per pair and launch
    __syncthreads();
    if (wave == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        if (lane == 0) __hip_atomic_fetch_add(flags + S, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
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
