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
// row.  The hand-off between workgroups is the solution values themselves:
// the output starts out "pending" (a bit pattern that no written value has),
// one wave polls the values of the next finished pairs until none is pending
// and copies them into LDS, and a workgroup barrier hands them to every wave.
// Values are written and polled with device-scope atomic stores and loads,
// so no fence, flag or counter is needed per hand-off.  The matrix rows of
// the next pair are loaded into registers before the wait, and the pair's
// inverse blocks into LDS when the workgroup starts.  The pair's own 128 x
// 128 triangle is then applied from its inverse after one more workgroup
// barrier.  Each launch also sets its rows of the other direction's output
// back to pending (the forward solve those of the back solve's output, the
// back solve those of its input, once read), so the buffers are ready for the
// next pass; the caller fills both with the pending pattern before the first.
// Every wait is bounded: on time-out the kernel raises a shared error word,
// every other wait sees it and gives up, and the host reports
// MSOLVE_E_DEVICE.
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
// A solution value not yet written: both floats kTrsvPendingWord (a NaN
// pattern that no written value has: outputs are written with NaN made
// canonical).
constexpr uint64_t kPending = (uint64_t(kTrsvPendingWord) << 32) | kTrsvPendingWord;

__device__ inline uint64_t c64_bits(float2 v)
{
    const float re = v.x != v.x ? __builtin_nanf("") : v.x;
    const float im = v.y != v.y ? __builtin_nanf("") : v.y;
    return uint64_t(__float_as_uint(re)) | (uint64_t(__float_as_uint(im)) << 32);
}
__device__ inline float2 c64_from_bits(uint64_t b)
{
    return make_float2(__uint_as_float(uint32_t(b)), __uint_as_float(uint32_t(b >> 32)));
}

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
    float *reset;                      // FWD: the back solve's output, BWD: src64 (rows set to pending)
    int64_t sReset;
    uint32_t *counter;
    uint64_t *err;
    uint64_t *dnorm;                   // nullable (back solve with X128): ||d_k|| bits at + f sN + k
    int64_t sN;
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
    float *reset = a.reset + size_t(f) * size_t(a.sReset);
    uint64_t *err = a.err;
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
    // the rows this workgroup owns in the other solve's output are pending
    // again (the forward solve resets the back solve's output, the back
    // solve the input it has just read), ready for the next launch
    if (q == 0 && bvalid) {
#pragma unroll
        for (int k = 0; k < NR; ++k)
            reinterpret_cast<uint64_t *>(reset)[size_t(k) * size_t(npad) + size_t(r0 + i)] = kPending;
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
    // Rounds: wave 0 alone polls the values of the next finished pairs
    // (relaxed device-scope loads; a pair is finished when none of its values
    // is pending) and copies up to kRound finished pairs into LDS; one
    // barrier hands them to every wave.  No fence is needed: the values are
    // the only data handed over, each written by one atomic store.
    // The two LDS buffers alternate, so wave 0 fills the next round while
    // the others still read this one; the barrier of the next round orders
    // the reuse.
    const uint64_t *O64 = reinterpret_cast<const uint64_t *>(out);
    uint32_t spins = 0;
    int rb = 0;
    while (left > 0) {
        if (wave == 0) {
            int cnt = 0;
            const int most = int(min<int64_t>(left, kRound));
            while (true) {
                // the values of every pair still wanted, loaded together;
                // lane l holds columns 2l and 2l + 1 of each
                const int want = most - cnt;
                uint64_t w[kRound][NR][2];
#pragma unroll
                for (int t = 0; t < kRound; ++t) {
                    const int64_t c0 = (J + dir * (cnt + t)) * kSub * kNB + 2 * lane;
#pragma unroll
                    for (int k = 0; k < NR; ++k) {
                        const uint64_t *src = O64 + size_t(k) * size_t(npad) + size_t(c0);
#pragma unroll
                        for (int e = 0; e < 2; ++e)
                            w[t][k][e] = t < want && c0 + e < n
                                             ? __hip_atomic_load(src + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                             : uint64_t(0);
                    }
                }
                // the leading finished pairs go to LDS (columns at and
                // beyond n as zero)
                int got = 0;
#pragma unroll
                for (int t = 0; t < kRound; ++t) {
                    bool pend = false;
#pragma unroll
                    for (int k = 0; k < NR; ++k) pend = pend || w[t][k][0] == kPending || w[t][k][1] == kPending;
                    if (got < t || t >= want || __ballot(pend) != 0) continue;
#pragma unroll
                    for (int k = 0; k < NR; ++k) {
                        const float2 u0 = c64_from_bits(w[t][k][0]), u1 = c64_from_bits(w[t][k][1]);
                        *reinterpret_cast<float4 *>(&ys[rb][cnt + t][k][2 * lane]) =
                            make_float4(u0.x, u0.y, u1.x, u1.y);
                    }
                    got = t + 1;
                }
                cnt += got;
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
            if (q == 0)
                __hip_atomic_store(reinterpret_cast<uint64_t *>(O) + size_t(k) * size_t(npad) + size_t(r0 + i),
                                   c64_bits(o[k]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
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
    // ||d||_inf of the update: a wave maximum of the moduli, then one
    // atomic maximum on the bits (non-negative doubles order like their
    // unsigned bit patterns, so the result does not depend on the order)
    if (!FWD && X128 && a.dnorm && bvalid) {
        uint64_t *dn = a.dnorm + size_t(f) * size_t(a.sN);
#pragma unroll
        for (int k = 0; k < NR; ++k) {
            double m = (valid && q == 0) ? hypot(double(o[k].x), double(o[k].y)) : 0.0;
            for (int off = 32; off > 0; off >>= 1) m = fmax(m, __shfl_xor(m, off, 64));
            if (lane == 0)
                atomicMax(reinterpret_cast<unsigned long long *>(dn + k),
                          static_cast<unsigned long long>(__double_as_longlong(m)));
        }
    }
}

}  // namespace

namespace {

int launch_trsv(bool fwd, int64_t n, int64_t nrhs, const TrsvBatch &tb, const float *LU,
                const float *Dinv, const double *src128, const float *src64, float *out,
                double *X128, float *reset, int64_t sReset, uint32_t *counter, uint64_t *err,
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
    a.reset = reset; a.sReset = sReset; a.counter = counter; a.err = err;
    a.dnorm = fwd ? nullptr : tb.dnorm; a.sN = tb.sN;
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
                    const float *Dinv, const double *r128, const float *r64, float *y, float *d,
                    uint32_t *counter, uint64_t *err, hipStream_t s)
{
    return launch_trsv(true, n, nrhs, tb, LU, Dinv, r128, r64, y, nullptr, d, tb.sOut, counter, err, s);
}

int launch_trsv_bwd(int64_t n, int64_t nrhs, const TrsvBatch &tb, const float *LU,
                    const float *Dinv, float *y, float *d, double *X128, uint32_t *counter,
                    uint64_t *err, hipStream_t s)
{
    return launch_trsv(false, n, nrhs, tb, LU, Dinv, nullptr, y, d, X128, y, tb.sSrc, counter, err, s);
}

}  // namespace msolve
