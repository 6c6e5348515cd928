// Unpivoted right-looking blocked LU of a complex64 matrix (step 1 of the
// refinement list in the section "Double-precision answers from a GPU
// without double precision" of the page "Solving Dense Matrices Fast in the
// Browser"; the page notes that this factorisation does not pivot).
//
// Per block column k (block size kNB):
//   1. lu_diag_kernel: one workgroup factors the kNB x kNB diagonal block in
//      registers and, in the same elimination loop, builds the inverses of
//      its unit-lower and upper factors (Dinv);
//   2. cgemm_kernel (batched, overwrite): U12 = L11^-1 A12 and
//      L21 = A21 U11^-1 -- the two triangular solves of the step, done as
//      products with the inverted diagonal blocks;
//   3. cgemm_kernel (subtract): A22 -= L21 U12, the trailing update and the
//      one dense contraction, on FP32 matrix cores -- applied for a group of
//      block columns at a time (K = G kNB), see launch_factor.
//
// The complex product is built from real v_mfma_f32_32x32x2f32 operations
// with separate accumulators for the real and the imaginary part:
//   Cr += Ar Br - Ai Bi,   Ci += Ar Bi + Ai Br   (4 real MFMAs, 8 flop per
// complex multiply-add).  The two K slots of each MFMA carry the two halves
// of the current K chunk, so both operands are read in their natural
// interleaved complex layout and no repacking pass is needed.
#include <algorithm>
#include <mutex>
#include <vector>

#include "common.hpp"

namespace msolve {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));

// ------------------------------------------------------------ complex

__device__ inline float2 cmul(float2 a, float2 b)
{
    return make_float2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}

// a - b c
__device__ inline float2 cfms(float2 a, float2 b, float2 c)
{
    return make_float2(a.x - (b.x * c.x - b.y * c.y), a.y - (b.x * c.y + b.y * c.x));
}

// 1 / p with scaling by max(|re|, |im|); flags a zero or non-finite pivot.
__device__ inline float2 cinv_checked(float2 p, bool *bad)
{
    const float s = fmaxf(fabsf(p.x), fabsf(p.y));
    if (!(s > 0.0f) || !isfinite(p.x) || !isfinite(p.y)) {
        *bad = true;
        return make_float2(__builtin_nanf(""), __builtin_nanf(""));
    }
    *bad = false;
    const float ar = p.x / s, ai = p.y / s;
    const float d = (ar * ar + ai * ai) * s;
    return make_float2(ar / d, -ai / d);
}

// ------------------------------------------------- diagonal block kernel

// A workgroup of kDiagWaves waves factors the NB x NB diagonal block
// (NB = 64 = wave width).  Lanes are columns; wave w owns the G = NB / 16 = 4
// consecutive rows 4w .. 4w + 3, one complex register per row.
//
// Row register T[r] packs two matrices in complementary lanes.  Before
// pivot j is applied, lanes c >= j hold the current (partially eliminated)
// row of A and lanes c < j hold row r of X = L^-1.  Pivot row j is used
// scaled by the reciprocal of its pivot, P_j = T[j] / u_jj, with lane j
// carrying 1 / u_jj itself, and applied to a later row r with a_rj = T[r][j]
// as
//     T[r][j] = 0,  T[r] -= a_rj P_j
// which eliminates the trailing row (lanes c > j: a_rc -= l_r u_jc with
// l_r = a_rj / u_jj), applies the column sweep X[r][:] -= l_r X[j][:] to the
// inverse (lanes c < j), and leaves x_rj = -l_r in lane j, which is also
// copied into lane j of the row's register of L.  The inverse of U comes
// from W = (U^T)^-1, swept the same way: W[r] -= (u_jr / u_jj) W[j] with the
// unscaled row W[j], which is divided by u_jj once it is final.
//
// The elimination runs in 16 super-steps of G pivots.  In super-step s wave
// s, whose rows have received every earlier pivot, eliminates among its own
// rows (pivot values move by readlane, no barrier) and publishes the G
// scaled pivot rows (and unscaled rows of W) in LDS; after one barrier every
// later wave applies the G pivots to its rows.  Buffers alternate between
// super-steps, so each super-step costs one barrier.
//
// Parts (what one workgroup keeps besides T, and what it stores):
//   kPartSym: a complex-symmetric block, read from its lower triangle.  Its
//     factors are stored as L D L^T: the upper triangle holds U = D L^T
//     (u_rc = d_r l_cr, each product rounded on its own, as the panel step
//     forms U's block rows), and U^-1 = (L^T)^-1 D^-1 = X^T D^-1 comes from
//     X = L^-1, so W is not swept.  Every stored factor of the symmetric
//     factorisation is then that of one L D L^T.
//   kPartLX and kPartUW: a general block, factorised by two workgroups that
//     run the same elimination of T with the same operations (every complex
//     product is written out with explicit fused multiply-adds, so the two
//     round alike and hold bit-identical rows of U).  kPartLX keeps L and
//     stores L\U and X = L^-1; kPartUW sweeps W and stores U^-1 = W^T.
//     Split this way each workgroup needs about half the registers of one
//     that sweeps both inverses, so the diagonal steps fit on a CU beside
//     the bulk product's workgroups, and the stored factors are still those
//     of one elimination.
constexpr int kDiagWaves = 16;
constexpr int kPartSym = 0, kPartLX = 1, kPartUW = 2;
// super-steps held at once in a general block's ring of pivot rows
constexpr int kDiagRing = 8;

__device__ inline float readlane_f(float v, int lane)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Plain two-float complex for the diagonal kernel: unlike float2 (a union
// type) it is always kept in registers when captured by reference.
struct cf {
    float x, y;
};
__device__ inline cf cfm(float x, float y) { return cf{x, y}; }
// a b: one rounded product and one fused multiply-add per component.
// FIXED: the fused product named here, so both workgroups of a general
// block round alike; otherwise the compiler picks which product it fuses
// (the symmetric part, where no second workgroup has to agree; on the
// near-resonance sweeps that rounding needed fewer LU retries).
template <bool FIXED = true>
__device__ inline cf cf_mul(cf a, cf b)
{
    if (FIXED) return cf{__builtin_fmaf(a.x, b.x, -(a.y * b.y)), __builtin_fmaf(a.x, b.y, a.y * b.x)};
    return cf{a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x};
}
// a - b c, two fused multiply-adds per component
__device__ inline cf cf_fms(cf a, cf b, cf c)
{
    return cf{__builtin_fmaf(-b.x, c.x, __builtin_fmaf(b.y, c.y, a.x)),
              __builtin_fmaf(-b.x, c.y, __builtin_fmaf(-b.y, c.x, a.y))};
}
// 1 / p from two hardware reciprocals (about 1 ulp each; the factors only
// need single-precision accuracy), scaled by max(|re|, |im|) against
// overflow; flags a zero or non-finite pivot.
template <bool FIXED = true>
__device__ inline cf cf_inv(cf p, bool *bad)
{
    const float s = fmaxf(fabsf(p.x), fabsf(p.y));
    *bad = !(s > 0.0f) || !isfinite(p.x) || !isfinite(p.y);
    const float rs = __builtin_amdgcn_rcpf(s);
    const float ar = p.x * rs, ai = p.y * rs;
    const float rd = __builtin_amdgcn_rcpf(FIXED ? __builtin_fmaf(ar, ar, ai * ai) : ar * ar + ai * ai) * rs;
    return *bad ? cf{__builtin_nanf(""), __builtin_nanf("")} : cf{ar * rd, -ai * rd};
}

// d c with every product and sum rounded on its own
__device__ inline cf cf_mul_rn(cf d, cf c)
{
#pragma clang fp contract(off)
    return cfm(d.x * c.x - d.y * c.y, d.x * c.y + d.y * c.x);
}

struct DiagShared {
    int bad_step;
    uint32_t ready[kDiagWaves];                  // wave s has published its pivot rows
    uint32_t consumed[kDiagRing];                // general block: waves that have applied a ring slot
};
// A general block's ring: slot t holds the four scaled pivot rows of a
// super-step (P_j = T[j] / u_jj, lane j: 1 / u_jj) and, for kPartUW, the four
// rows of W before their division by u_jj.
struct DiagRingSlot {
    cf p[4][64];
    cf w[4][64];
};

// One part of the factorisation of the diagonal block at (k0, k0) of the
// matrix at A (see the parts above).  Lt: kPartSym's LDS for L and the pivots.
// flag (kPartLX, kPartUW): the matrix's hand-off word between the two
// workgroups of a general block, raised to `step` by kPartUW once it has read
// the block, which kPartLX then overwrites (a kPartUW workgroup that starts
// late must still find the block unfactorised).
constexpr uint32_t kDiagSpinLimit = 1u << 22;

template <int NB, int PART>
__device__ __forceinline__ void diag_block(int64_t n, int64_t k0, float *A, float *Dinv_blk,
                                           int32_t *d_info, DiagShared &sh, cf (*Lt)[NB + 1],
                                           DiagRingSlot *ring, uint32_t *flag, uint32_t step)
{
    constexpr int G = NB / kDiagWaves;
    static_assert(NB == 64 && G == 4, "one lane per column, four rows per wave");
    constexpr bool KEEP_L = PART != kPartUW;   // the register of L
    constexpr bool SWEEP_W = PART == kPartUW;
    constexpr bool PAIR = PART != kPartSym;   // two workgroups that must round alike
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int nv = int(min<int64_t>(NB, n - k0));
    const int rb = w * G;                 // the wave's first row
    cf *Ac = reinterpret_cast<cf *>(A);

    cf T[G], W[G], Lr[G];                 // Lr: row r of L, multipliers in lanes < r
    cf Dr[G];                             // kPartSym: 1 / u_rr of the wave's rows
#pragma unroll
    for (int m = 0; m < G; ++m) {
        Lr[m] = cfm(0.0f, 0.0f);
        const int r = rb + m;
        T[m] = cfm(r == lane ? 1.0f : 0.0f, 0.0f);
        // (a symmetric block is read from its lower triangle only: the entry
        // right of the diagonal from its mirror below it)
        const bool up = PART == kPartSym && lane > r;
        const int rr = up ? lane : r, cc = up ? r : lane;
        if (r < nv && lane < nv) T[m] = Ac[size_t(k0 + rr) * size_t(n) + size_t(k0 + cc)];
        W[m] = cfm(r == lane ? 1.0f : 0.0f, 0.0f);
    }
    if (PART == kPartUW) {
        // every wave's loads of the block have returned before the hand-off
        // word is raised, so the other workgroup may then overwrite it
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (threadIdx.x == 0) __hip_atomic_store(flag, step, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // apply scaled pivot row pj (row j) to the wave's row m; no branches,
    // so the updates of the wave's rows interleave
    auto apply = [&](int m, int j, cf pj, cf ujr, cf wj) {
        const cf arj = cfm(readlane_f(T[m].x, j), readlane_f(T[m].y, j));
        const bool at_j = lane == j;
        T[m] = cf_fms(at_j ? cfm(0.0f, 0.0f) : T[m], arj, pj);
        if (KEEP_L) Lr[m] = at_j ? cfm(-T[m].x, -T[m].y) : Lr[m];
        if (SWEEP_W) W[m] = cf_fms(W[m], ujr, wj);
    };

    int my_bad = 0;                       // first bad pivot of the wave's rows
    if (threadIdx.x == 0) sh.bad_step = NB + 1;
    if constexpr (PART == kPartSym) {
        // Symmetric block: no barrier per super-step.  Every scaled pivot row
        // stays in LDS (in the space of Lt, which the write-back uses later),
        // and wave s raises its word of sh.ready once its four rows are there.
        // Wave w applies the pivots of waves 0 .. w-1 in order, each wave's as
        // soon as they are published, then eliminates among its own rows and
        // publishes them.  The chain from pivot to pivot no longer waits for
        // the slowest wave's updates; the operations and their order are
        // those of the super-steps.  (Each wait is bounded: on a time-out the
        // block's first pivot is reported bad, so the factors are not used.
        // Publishing each pivot row on its own needs two more registers,
        // which leaves no room beside two bulk workgroups: slower.)
        cf (*pall)[NB + 1] = Lt;
        if (threadIdx.x < kDiagWaves) sh.ready[threadIdx.x] = 0u;
        __syncthreads();
#pragma unroll 1
        for (int s = 0; s < w; ++s) {
            uint32_t spins = 0;
            while (__builtin_amdgcn_readfirstlane(
                       __hip_atomic_load(&sh.ready[s], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP)) == 0u) {
                if (++spins > kDiagSpinLimit) {
                    my_bad = 1;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
#pragma unroll
            for (int m = 0; m < G; ++m) {
                const int j = s * G + m;
                const cf pj = pall[j][lane];
#pragma unroll
                for (int m2 = 0; m2 < G; ++m2) apply(m2, j, pj, cfm(0.0f, 0.0f), cfm(0.0f, 0.0f));
            }
        }
#pragma unroll
        for (int m = 0; m < G; ++m) {
            const int j = rb + m;
            const cf pv = cfm(readlane_f(T[m].x, j), readlane_f(T[m].y, j));
            bool bad;
            const cf inv = cf_inv<PAIR>(pv, &bad);
            my_bad = (bad && my_bad == 0) ? j + 1 : my_bad;
            const cf pm = lane == j ? inv : cf_mul<PAIR>(inv, T[m]);
            pall[j][lane] = pm;
#pragma unroll
            for (int m2 = m + 1; m2 < G; ++m2) apply(m2, j, pm, cfm(0.0f, 0.0f), cfm(0.0f, 0.0f));
            Dr[m] = inv;
        }
        if (lane == 0) __hip_atomic_store(&sh.ready[w], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        // every wave has read the pivot rows before Lt is written
        __syncthreads();
    } else {
        // General block: no barrier per super-step either.  The scaled pivot
        // rows (and kPartUW's rows of W) go through a ring of kDiagRing
        // super-steps in LDS (the whole block's would not fit beside two
        // bulk workgroups): wave s raises its ready word once its rows are in
        // slot s mod kDiagRing, every later wave counts itself in the slot's
        // consumed word once it has applied them, and wave s + kDiagRing
        // writes the slot again only when all of them have.  A wave waits
        // only for earlier waves' rows or for waves that need nothing from
        // it, so every wait ends; each is bounded all the same (a time-out
        // reports the block's first pivot as bad).  The operations on each
        // row and their order are those of the super-steps, so both
        // workgroups of the block still round alike.
        if (threadIdx.x < kDiagWaves) sh.ready[threadIdx.x] = 0u;
        if (threadIdx.x < kDiagRing) sh.consumed[threadIdx.x] = 0u;
        __syncthreads();
#pragma unroll 1
        for (int s = 0; s < w; ++s) {
            uint32_t spins = 0;
            while (__builtin_amdgcn_readfirstlane(
                       __hip_atomic_load(&sh.ready[s], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP)) == 0u) {
                if (++spins > kDiagSpinLimit) {
                    my_bad = 1;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
            const DiagRingSlot &sl = ring[s % kDiagRing];
            // (rolled: unrolled, the loads of all four rows are issued
            // first and the step no longer fits its register budget)
#pragma unroll 1
            for (int m = 0; m < G; ++m) {
                const int j = s * G + m;
                const cf pj = sl.p[m][lane];
                const cf wj = SWEEP_W ? sl.w[m][lane] : cfm(0.0f, 0.0f);
                cf u[G];
#pragma unroll
                for (int m2 = 0; m2 < G; ++m2) u[m2] = SWEEP_W ? sl.p[m][rb + m2] : cfm(0.0f, 0.0f);
#pragma unroll
                for (int m2 = 0; m2 < G; ++m2) apply(m2, j, pj, u[m2], wj);
            }
            if (lane == 0)
                __hip_atomic_fetch_add(&sh.consumed[s % kDiagRing], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        // the wave's own slot, once the waves after super-step w - kDiagRing
        // have applied what it held
        DiagRingSlot &own = ring[w % kDiagRing];
        if (w >= kDiagRing) {
            const uint32_t readers = uint32_t(kDiagWaves - 1 - (w - kDiagRing));
            uint32_t spins = 0;
            while (__builtin_amdgcn_readfirstlane(__hip_atomic_load(&sh.consumed[w % kDiagRing], __ATOMIC_ACQUIRE,
                                                                    __HIP_MEMORY_SCOPE_WORKGROUP)) < readers) {
                if (++spins > kDiagSpinLimit) {
                    my_bad = 1;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
            // (this super-step's readers count only after its ready word)
            if (lane == 0)
                __hip_atomic_store(&sh.consumed[w % kDiagRing], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        // the wave's rows are next: eliminate among them and publish
#pragma unroll
        for (int m = 0; m < G; ++m) {
            const int j = rb + m;
            const cf pv = cfm(readlane_f(T[m].x, j), readlane_f(T[m].y, j));
            bool bad;
            const cf inv = cf_inv<PAIR>(pv, &bad);
            my_bad = (bad && my_bad == 0) ? j + 1 : my_bad;
            const cf pm = lane == j ? inv : cf_mul<PAIR>(inv, T[m]);
            own.p[m][lane] = pm;
            if (SWEEP_W) own.w[m][lane] = W[m];
#pragma unroll
            for (int m2 = m + 1; m2 < G; ++m2) {
                const cf ujr = SWEEP_W ? cfm(readlane_f(pm.x, rb + m2), readlane_f(pm.y, rb + m2))
                                       : cfm(0.0f, 0.0f);
                apply(m2, j, pm, ujr, W[m]);
            }
            Dr[m] = inv;
            if (SWEEP_W) W[m] = cf_mul(W[m], inv);
        }
        if (lane == 0) __hip_atomic_store(&sh.ready[w], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        __syncthreads();
    }

    if (PART == kPartLX) {
        // the block may be overwritten once the kPartUW workgroup has read
        // it (a bounded wait; on a time-out the block's first pivot is
        // reported bad, so the factors are not used)
        if (threadIdx.x == 0) {
            uint32_t spins = 0;
            while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < step) {
                if (++spins > kDiagSpinLimit) {
                    sh.bad_step = 1;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
        }
        __syncthreads();
    }

    // write back: L\U into A (valid part), L^-1 and U^-1 into Dinv
    cf *Linv = reinterpret_cast<cf *>(Dinv_blk);
    cf *Uinv = Linv + NB * NB;
    if (PART == kPartSym) {
        // L and the pivots through LDS, then U = D L^T and U^-1 = X^T D^-1
        // (column r of U^-1: x_ri / d_r for i < r, 1 / d_r on the diagonal)
#pragma unroll
        for (int m = 0; m < G; ++m) {
            const int r = rb + m;
            Lt[r][lane] = lane < r ? Lr[m] : (lane == r ? T[m] : cfm(0.0f, 0.0f));
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < G; ++m) {
            const int r = rb + m;
            const cf d = cfm(readlane_f(T[m].x, r), readlane_f(T[m].y, r));
            const cf u = lane < r ? Lr[m] : (lane == r ? T[m] : cf_mul_rn(d, Lt[lane][r]));
            if (r < nv && lane < nv) Ac[size_t(k0 + r) * size_t(n) + size_t(k0 + lane)] = u;
            Linv[r * NB + lane] = lane < r ? T[m] : cfm(lane == r ? 1.0f : 0.0f, 0.0f);
            Uinv[lane * NB + r] = lane < r ? cf_mul<false>(T[m], Dr[m]) : (lane == r ? Dr[m] : cfm(0.0f, 0.0f));
        }
    } else if (PART == kPartLX) {
#pragma unroll
        for (int m = 0; m < G; ++m) {
            const int r = rb + m;
            if (r < nv && lane < nv) Ac[size_t(k0 + r) * size_t(n) + size_t(k0 + lane)] = lane < r ? Lr[m] : T[m];
            Linv[r * NB + lane] = lane < r ? T[m] : cfm(lane == r ? 1.0f : 0.0f, 0.0f);
        }
    } else {
#pragma unroll
        for (int m = 0; m < G; ++m) {
            const int r = rb + m;
            Uinv[lane * NB + r] = lane <= r ? W[m] : cfm(0.0f, 0.0f);
        }
    }
    if (lane == 0 && my_bad != 0) atomicMin(&sh.bad_step, my_bad);
    __syncthreads();
    if (threadIdx.x == 0 && sh.bad_step <= nv) {
        if (atomicCAS(d_info, 0, int32_t(k0 + sh.bad_step)) != 0) { /* an earlier pivot is kept */ }
    }
}

// Diagonal step of a batch of nf matrices (matrix f: A + f sA, Dinv_blk +
// f sD, d_info + f, flags + f).  SYM: one kPartSym workgroup per matrix (grid
// nf).  Otherwise two workgroups per matrix (grid 2 nf): blockIdx.x < nf
// runs kPartUW for matrix blockIdx.x (dispatched first), the others kPartLX
// for matrix blockIdx.x - nf.  Both report a bad pivot, to the same word.
// step: the hand-off value of this diagonal step (its block index + 1; the
// flags are zero at the start of a factorisation).
template <int NB, bool SYM>
__global__ __launch_bounds__(kDiagWaves * 64) void lu_diag_kernel(
    int64_t n, int64_t k0, float *A, int64_t sA, float *Dinv_blk, int64_t sD, int32_t *d_info,
    uint32_t *flags, uint32_t step)
{
    // a step of the serial chain: its waves go first on SIMDs shared with
    // the bulk product
    __builtin_amdgcn_s_setprio(3);
    __shared__ DiagShared sh;
    __shared__ cf Lt[SYM ? NB : 1][NB + 1];
    __shared__ DiagRingSlot ring[SYM ? 1 : kDiagRing];
    const unsigned nf = SYM ? gridDim.x : gridDim.x / 2;
    const unsigned f = blockIdx.x % nf;
    A += size_t(f) * size_t(sA);
    Dinv_blk += size_t(f) * size_t(sD);
    d_info += f;
    if (SYM)
        diag_block<NB, kPartSym>(n, k0, A, Dinv_blk, d_info, sh, Lt, ring, nullptr, 0);
    else if (blockIdx.x < nf)
        diag_block<NB, kPartUW>(n, k0, A, Dinv_blk, d_info, sh, Lt, ring, flags + f, step);
    else
        diag_block<NB, kPartLX>(n, k0, A, Dinv_blk, d_info, sh, Lt, ring, flags + f, step);
}

// --------------------------------------------- coupling of block pairs

// For the pair of diagonal blocks (2t, 2t+1) of matrix f (t = t0 +
// blockIdx.x, blockIdx.y = f): the lower-left block of the inverse of the pair's
// unit-lower 128 x 128 part, X = -Li1 M Li0 with M = L[2t+1][2t]
// (kind 0), and the upper-right block of the inverse of its upper
// part, Y = -Ui0 N Ui1 with N = U[2t][2t+1] (kind 1); Li, Ui are
// the blocks' inverses already in Dinv.  With them the triangular solves
// apply a 128-row block's inverse in one step.  Rows (kind 0) or columns
// (kind 1) of M, N beyond n are zero.  blockIdx.z = 4 kind + q: the
// workgroup computes the 16 columns 16q .. 16q + 15 of the result, first
// T = M Li0 (kind 0) or N Ui1 (kind 1) on those columns, then the product
// with the left factor, both factors of each product staged in LDS.
__global__ __launch_bounds__(256) void coupling_kernel(int64_t n, int64_t t0, const float *A,
                                                       int64_t sA, float *Dinv, int64_t sD)
{
    constexpr int NB = kNB, QC = NB / 4;   // a quarter of the columns per workgroup
    __shared__ float2 P[NB][NB + 1];       // left factor of the current product
    __shared__ float2 R[NB][QC + 1];       // the quarter of the right factor
    const int64_t t = t0 + blockIdx.x;
    const int kind = blockIdx.z >> 2, cq = int(blockIdx.z & 3) * QC;
    const float2 *Ac = reinterpret_cast<const float2 *>(A + size_t(blockIdx.y) * size_t(sA));
    float2 *D = reinterpret_cast<float2 *>(Dinv + size_t(blockIdx.y) * size_t(sD));
    const int64_t nblk = (n + NB - 1) / NB;
    const int64_t b0 = 2 * t, b1 = 2 * t + 1;
    // inverse blocks: block b's unit-lower inverse at b * 2 NB^2, upper at + NB^2
    const float2 *Li0 = D + size_t(b0) * 2 * NB * NB, *Li1 = D + size_t(b1) * 2 * NB * NB;
    const float2 *Ui0 = Li0 + NB * NB, *Ui1 = Li1 + NB * NB;
    float2 *out = D + (size_t(nblk) + size_t(t)) * 2 * NB * NB + (kind ? NB * NB : 0);
    const float2 *right = kind ? Ui1 : Li0;    // T = (M or N) right
    const float2 *left = kind ? Ui0 : Li1;     // out = -left T
    // M = L[b1][b0] (rows beyond n are zero) or N = U[b0][b1] (columns
    // beyond n are zero), staged with the quarter of the right factor
    const int64_t grow0 = kind ? b0 * NB : b1 * NB;
    const int64_t gcol0 = kind ? b1 * NB : b0 * NB;
    for (int e = threadIdx.x; e < NB * NB; e += 256) {
        const int r = e / NB, c = e % NB;
        const bool in = grow0 + r < n && gcol0 + c < n;
        P[r][c] = in ? Ac[size_t(grow0 + r) * size_t(n) + size_t(gcol0 + c)] : make_float2(0.0f, 0.0f);
    }
    for (int e = threadIdx.x; e < NB * QC; e += 256) R[e / QC][e % QC] = right[(e / QC) * NB + cq + e % QC];
    __syncthreads();
    // thread: row i, columns c .. c + 3 of the quarter
    const int i = threadIdx.x / 4, c = (threadIdx.x % 4) * 4;
    float2 tv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) tv[j] = make_float2(0.0f, 0.0f);
    for (int k = 0; k < NB; ++k) {
        const float2 m = P[i][k];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float2 r = R[k][c + j];
            tv[j].x = __builtin_fmaf(m.x, r.x, __builtin_fmaf(-m.y, r.y, tv[j].x));
            tv[j].y = __builtin_fmaf(m.x, r.y, __builtin_fmaf(m.y, r.x, tv[j].y));
        }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) R[i][c + j] = tv[j];
    for (int e = threadIdx.x; e < NB * NB; e += 256) P[e / NB][e % NB] = left[e];
    __syncthreads();
    float2 ov[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) ov[j] = make_float2(0.0f, 0.0f);
    for (int k = 0; k < NB; ++k) {
        const float2 l = P[i][k];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float2 r = R[k][c + j];
            ov[j].x = __builtin_fmaf(-l.x, r.x, __builtin_fmaf(l.y, r.y, ov[j].x));
            ov[j].y = __builtin_fmaf(-l.x, r.y, __builtin_fmaf(-l.y, r.x, ov[j].y));
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) out[size_t(i) * NB + cq + c + j] = ov[j];
}

// ----------------------------------------------------------- cgemm kernel

struct GemmProblem {
    int64_t M, N, K;          // complex dimensions, K % KC == 0
    const float *A;           // M x K, row stride lda (complex elements)
    const float *B;           // K x N, row stride ldb
    float *C;                 // M x N, row stride ldc (may alias A or B, see below)
    int64_t lda, ldb, ldc;
    int64_t nb;               // independent products of this shape (a batch)
    int64_t sA, sB, sC;       // strides between the batch's operands (floats)
    int64_t tiles_n;          // column tiles
    int64_t tiles;            // tiles of one product
    int64_t lower;            // 1: square product, only the tiles that hold entries on
                              // or below the diagonal of C (the only problem of its launch)
    // kernels with TOUT: also T[c][r] = d_c C[r][c] (T row stride ldt, d_c at
    // Dg + c ldd complex elements; batch strides sC as C's)
    float *T;
    const float *Dg;
    int64_t ldt, ldd;
};

struct GemmBatch {
    GemmProblem p[2];
    int count;
    // single general product (count 1, not lower): > 0 walks the tiles in
    // strips of this many tile rows, column after column within a strip
    int group_rows = 0;
    // 1: the launch is a step of the factorisation's serial chain (panel or
    // L-region update), whose waves get a raised issue priority over those
    // of the bulk product running beside it
    int prio = 0;
    // > 0: each workgroup reserves this many bytes of LDS in all (static
    // arrays plus dynamic padding), which bounds how many share a CU; only
    // for launches of at most lds_tiles_max tiles
    int lds_bytes = 0;
    int64_t lds_tiles_max = 0;
};

__device__ inline floatx16 mfma32(float a, float b, floatx16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// C (=|-=) A B for complex64 matrices.  Workgroup tile BM x BN complex,
// WM x WN waves, each wave TM x TN sub-tiles of 32 x 32 complex.  K is
// walked in chunks of KC complex, staged through LDS (double-buffered) with
// row-contiguous global loads.  C may alias A when one tile spans all N
// columns (BN >= N), or alias B when one tile spans all M rows (BM >= M):
// every global read of the aliased operand by a workgroup precedes its
// epilogue, and no other workgroup reads that band.
// d c with every product and sum rounded on its own
__device__ inline float2 cmul_rn(float2 d, float2 c)
{
#pragma clang fp contract(off)
    return make_float2(d.x * c.x - d.y * c.y, d.x * c.y + d.y * c.x);
}

template <int WM, int WN, int TM, int TN, int KC, bool SUBTRACT, bool TOUT = false>
__global__ __launch_bounds__(WM *WN * 64, 2) void cgemm_kernel(GemmBatch batch)
{
    constexpr int THREADS = WM * WN * 64;
    constexpr int BM = WM * TM * 32;
    constexpr int BN = WN * TN * 32;
    constexpr int APAD = 2, BPAD = 2;
    constexpr int ALD = KC + APAD;       // LDS row stride of A (complex)
    constexpr int BLD = BN + BPAD;       // LDS row stride of B (complex)
    constexpr int HALF = KC / 2;
    constexpr int A_TOTAL = BM * KC / 2;              // 2-complex pieces per chunk
    constexpr int B_TOTAL = KC * BN / 2;
    constexpr int A_PIECES = (A_TOTAL + THREADS - 1) / THREADS;   // per thread
    constexpr int B_PIECES = (B_TOTAL + THREADS - 1) / THREADS;
    static_assert(KC % 2 == 0 && BN % 2 == 0, "pieces are pairs of complex numbers");

    // A and B chunks, double-buffered; the TOUT epilogue reuses the space
    __shared__ float2 lds[2 * BM * ALD + 2 * KC * BLD];
    float2 (*As)[BM * ALD] = reinterpret_cast<float2 (*)[BM * ALD]>(lds);
    float2 (*Bs)[KC * BLD] = reinterpret_cast<float2 (*)[KC * BLD]>(lds + 2 * BM * ALD);
    if (batch.prio) __builtin_amdgcn_s_setprio(3);

    int64_t t = blockIdx.x;
    int pi = 0;
    if (batch.count > 1) {
        const int64_t t0 = batch.p[0].tiles * batch.p[0].nb;
        if (t >= t0) {
            t -= t0;
            pi = 1;
        }
    } else {
        // workgroups are dealt to the 8 XCDs round-robin: give each XCD a
        // contiguous band of tiles (row-major, product after product), so
        // tiles that share rows of A and columns of B share that XCD's L2
        const int64_t total = batch.p[0].tiles * batch.p[0].nb;
        const int64_t per = (total + 7) / 8;
        t = (t % 8) * per + t / 8;
        if (t >= total) return;
    }
    const GemmProblem P = batch.p[pi];
    const int64_t f = t / P.tiles;
    t -= f * P.tiles;
    int64_t m0, n0;
    if (P.lower) {
        // Lower-triangle tiles: with R = BN / BM, the band of rows a (rows
        // a BN .. a BN + BN - 1) needs the column tiles 0 .. a (column tile
        // a holds the band's diagonal), R (a + 1) tiles in all: tile u of the
        // band is row tile R a + u / (a + 1), column tile u % (a + 1).  Tile
        // t lies in the band a with R a (a + 1) / 2 <= t < R (a + 1) (a + 2) / 2.
        // (Tiles with BN % BM != 0 are refused for lower products by the launcher.)
        constexpr int64_t R = BN % BM == 0 ? BN / BM : 1;
        int64_t a = int64_t((sqrt(1.0 + 8.0 * double(t) / double(R)) - 1.0) * 0.5);
        while (R * (a + 1) * (a + 2) / 2 <= t) ++a;
        while (a > 0 && R * a * (a + 1) / 2 > t) --a;
        const int64_t u = t - R * a * (a + 1) / 2;
        m0 = (R * a + u / (a + 1)) * BM;
        n0 = (u % (a + 1)) * BN;
        if (m0 >= P.M) return;              // the last band of rows may end early
    } else if (batch.group_rows > 0) {
        // strips of group_rows tile rows, walked column by column, so that
        // the tiles in flight on one XCD share few rows of A and few
        // columns of B (which then stay in that XCD's L2)
        const int64_t tiles_m = P.tiles / P.tiles_n;
        const int64_t strip = t / (int64_t(batch.group_rows) * P.tiles_n);
        const int64_t gr = min<int64_t>(batch.group_rows, tiles_m - strip * batch.group_rows);
        const int64_t j = t - strip * int64_t(batch.group_rows) * P.tiles_n;
        m0 = (strip * batch.group_rows + j % gr) * BM;
        n0 = (j / gr) * BN;
    } else {
        m0 = (t / P.tiles_n) * BM;
        n0 = (t % P.tiles_n) * BN;
    }
    const float2 *Ag = reinterpret_cast<const float2 *>(P.A + size_t(f) * size_t(P.sA));
    const float2 *Bg = reinterpret_cast<const float2 *>(P.B + size_t(f) * size_t(P.sB));
    float2 *Cg = reinterpret_cast<float2 *>(P.C + size_t(f) * size_t(P.sC));

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int l32 = lane & 31, h = lane >> 5;

    // Lane (l32, h) of sub-tile (a, b) holds rows a*32 + (r/4)*8 + h*4 + r%4,
    // column b*32 + l32 of the wave's block.
    const int64_t wrow0 = m0 + wm * TM * 32 + h * 4;
    const int64_t wcol0 = n0 + wn * TN * 32 + l32;
    const int64_t rows_left = P.M - wrow0;          // valid when a*32 + (r/4)*8 + r%4 < rows_left
    const int64_t cols_left = P.N - wcol0;          // valid when b*32 < cols_left
    const bool interior = (m0 + BM <= P.M) && (n0 + BN <= P.N);   // uniform
    float2 *cbase = Cg + size_t(min<int64_t>(wrow0, P.M - 1)) * size_t(P.ldc) +
                    size_t(min<int64_t>(wcol0, P.N - 1));
    // The accumulators start at zero and collect (-A) B when subtracting;
    // C then goes into registers of its own and is added in the epilogue.
    floatx16 cr[TM][TN], ci[TM][TN];
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                cr[a][b][r] = 0.0f;
                ci[a][b][r] = 0.0f;
            }

    // Every global load below is unconditional: rows and columns outside
    // the operands are clamped to their last row and column.  Such values
    // only reach accumulator entries outside C, which the epilogue does not
    // store.  (A load under a branch can make the compiler wait for it
    // before the next load is issued.)
    // C addresses: the tile's corner (uniform) plus this lane's 32-bit offset
    float2 cv[SUBTRACT ? TM : 1][SUBTRACT ? TN : 1][SUBTRACT ? 16 : 1];
    const float2 *ctile = Cg + size_t(m0) * size_t(P.ldc) + size_t(n0);
    const int lrow = wm * TM * 32 + h * 4, lcol = wn * TN * 32 + l32;
    auto load_c = [&]() {
        if constexpr (SUBTRACT) {
            const uint32_t ldc = uint32_t(P.ldc);
            const int rmax = int(min<int64_t>(BM, P.M - m0)) - 1, cmax = int(min<int64_t>(BN, P.N - n0)) - 1;
#pragma unroll
            for (int a = 0; a < TM; ++a)
#pragma unroll
                for (int b = 0; b < TN; ++b)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int lr = a * 32 + (r >> 2) * 8 + (r & 3);
                        if (interior) {
                            const float2 *crow = ctile + size_t(lr) * size_t(P.ldc) + size_t(b * 32);
                            cv[a][b][r] = crow[uint32_t(lrow) * ldc + uint32_t(lcol)];
                        } else {
                            const uint32_t row = uint32_t(min(lrow + lr, rmax));
                            const uint32_t col = uint32_t(min(lcol + b * 32, cmax));
                            cv[a][b][r] = ctile[row * ldc + col];
                        }
                    }
        }
    };

    // Each thread's sources in the chunk loads: a pair of complex numbers
    // of a row of A, and two of a row of B (adjacent columns; at the edge
    // both may be the last column).
    float2 ra[A_PIECES][2], rb[B_PIECES][2];
    const float2 *asrc[A_PIECES], *bsrc[B_PIECES];
    int bnext[B_PIECES];
#pragma unroll
    for (int i = 0; i < A_PIECES; ++i) {
        const int e = tid + THREADS * i;
        const int row = e / (KC / 2), kp = e % (KC / 2);
        asrc[i] = Ag + size_t(min<int64_t>(m0 + row, P.M - 1)) * size_t(P.lda) + size_t(2 * kp);
    }
#pragma unroll
    for (int i = 0; i < B_PIECES; ++i) {
        const int e = tid + THREADS * i;
        const int kr = e / (BN / 2) % KC, np = e % (BN / 2);
        const int64_t c0 = min<int64_t>(n0 + 2 * np, P.N - 1), c1 = min<int64_t>(n0 + 2 * np + 1, P.N - 1);
        bsrc[i] = Bg + size_t(kr) * size_t(P.ldb) + size_t(c0);
        bnext[i] = int(c1 - c0);
    }
    auto load_chunk = [&](int64_t k) {
#pragma unroll
        for (int i = 0; i < A_PIECES; ++i) {
            const int e = tid + THREADS * i;
            if (A_TOTAL % THREADS != 0 && e >= A_TOTAL) break;
            ra[i][0] = asrc[i][k];
            ra[i][1] = asrc[i][k + 1];
        }
#pragma unroll
        for (int i = 0; i < B_PIECES; ++i) {
            const int e = tid + THREADS * i;
            if (B_TOTAL % THREADS != 0 && e >= B_TOTAL) break;
            const float2 *q = bsrc[i] + size_t(k) * size_t(P.ldb);
            rb[i][0] = q[0];
            rb[i][1] = q[bnext[i]];
        }
    };
    auto store_chunk = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_PIECES; ++i) {
            const int e = tid + THREADS * i;
            if (A_TOTAL % THREADS != 0 && e >= A_TOTAL) break;
            const int row = e / (KC / 2), kp = e % (KC / 2);
            As[buf][row * ALD + 2 * kp] = ra[i][0];
            As[buf][row * ALD + 2 * kp + 1] = ra[i][1];
        }
#pragma unroll
        for (int i = 0; i < B_PIECES; ++i) {
            const int e = tid + THREADS * i;
            if (B_TOTAL % THREADS != 0 && e >= B_TOTAL) break;
            const int kr = e / (BN / 2), np = e % (BN / 2);
            Bs[buf][kr * BLD + 2 * np] = rb[i][0];
            Bs[buf][kr * BLD + 2 * np + 1] = rb[i][1];
        }
    };
    auto compute = [&](int buf) {
        const float2 *as = As[buf] + (wm * TM * 32 + l32) * ALD + h * HALF;
        const float2 *bs = Bs[buf] + (h * HALF) * BLD + wn * TN * 32 + l32;
#pragma unroll
        for (int s = 0; s < HALF; ++s) {
            float2 av[TM], bv[TN];
#pragma unroll
            for (int a = 0; a < TM; ++a) av[a] = as[a * 32 * ALD + s];
#pragma unroll
            for (int b = 0; b < TN; ++b) bv[b] = bs[s * BLD + b * 32];
            // C += A B:  Cr += ar br + (-ai) bi,  Ci += ar bi + ai br
            // C -= A B:  Cr += (-ar) br + ai bi,  Ci += (-ar) bi + (-ai) br
            float p[TM], q[TM], u[TM];
#pragma unroll
            for (int a = 0; a < TM; ++a) {
                p[a] = SUBTRACT ? -av[a].x : av[a].x;
                q[a] = SUBTRACT ? av[a].y : -av[a].y;
                u[a] = SUBTRACT ? -av[a].y : av[a].y;
            }
#pragma unroll
            for (int a = 0; a < TM; ++a) {
#pragma unroll
                for (int b = 0; b < TN; ++b) {
                    cr[a][b] = mfma32(p[a], bv[b].x, cr[a][b]);
                    cr[a][b] = mfma32(q[a], bv[b].y, cr[a][b]);
                    ci[a][b] = mfma32(p[a], bv[b].y, ci[a][b]);
                    ci[a][b] = mfma32(u[a], bv[b].x, ci[a][b]);
                }
            }
        }
    };

    // K chunks: the loads of chunk kc + 1 are in flight during the products
    // of chunk kc (LDS double-buffered).  C is loaded after the last chunk:
    // held in registers during the K loop it would leave no room for the
    // serial chain's diagonal step beside two bulk workgroups on a CU.
    const int64_t nk = P.K / KC;
    load_chunk(0);
    store_chunk(0);
    __syncthreads();
    int64_t kc = 0;
    for (; kc + 1 < nk; ++kc) {
        load_chunk((kc + 1) * KC);
        // the loads go out before the products (the scheduler would
        // otherwise sink them between the MFMAs, shortening their cover)
        __builtin_amdgcn_sched_barrier(0);
        compute(int(kc & 1));
        store_chunk(int((kc + 1) & 1));
        __syncthreads();
    }
    compute(int(kc & 1));
    load_c();

        // epilogue: C + the accumulated (-A) B when subtracting, then store
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int lr = a * 32 + (r >> 2) * 8 + (r & 3);
                if (interior || (lr < rows_left && b * 32 < cols_left)) {
                    float2 o = make_float2(cr[a][b][r], ci[a][b][r]);
                    if constexpr (SUBTRACT) o = make_float2(cv[a][b][r].x + o.x, cv[a][b][r].y + o.y);
                    cbase[size_t(lr) * size_t(P.ldc) + size_t(b * 32)] = o;
                }
            }
    if constexpr (TOUT) {
        // the scaled transpose of the tile, staged in LDS (in the space of
        // the A and B chunks, CW columns at a time) so that the rows of T are
        // written contiguously
        constexpr int CW = 32;
        static_assert(BN % CW == 0 && CW * (BM + 1) <= 2 * BM * ALD + 2 * KC * BLD, "transpose fits");
        __shared__ float2 ds[BN];
        float2 (*Ts)[BM + 1] = reinterpret_cast<float2 (*)[BM + 1]>(lds);
        float2 *Tg = reinterpret_cast<float2 *>(P.T + size_t(f) * size_t(P.sC));
        const float2 *Dgc = reinterpret_cast<const float2 *>(P.Dg + size_t(f) * size_t(P.sC));
        for (int c = tid; c < BN; c += THREADS)
            ds[c] = n0 + c < P.N ? Dgc[size_t(n0 + c) * size_t(P.ldd)] : make_float2(0.0f, 0.0f);
        __syncthreads();
        for (int c0 = 0; c0 < BN; c0 += CW) {
#pragma unroll
            for (int a = 0; a < TM; ++a)
#pragma unroll
                for (int b = 0; b < TN; ++b) {
                    const int col = wn * TN * 32 + l32 + b * 32;
                    if (col < c0 || col >= c0 + CW) continue;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row = wm * TM * 32 + h * 4 + a * 32 + (r >> 2) * 8 + (r & 3);
                        Ts[col - c0][row] = cmul_rn(ds[col], make_float2(cr[a][b][r], ci[a][b][r]));
                    }
                }
            __syncthreads();
            for (int e = tid; e < CW * BM; e += THREADS) {
                const int c = e / BM, rr = e % BM;
                if (n0 + c0 + c < P.N && m0 + rr < P.M)
                    Tg[size_t(n0 + c0 + c) * size_t(P.ldt) + size_t(m0 + rr)] = Ts[c][rr];
            }
            __syncthreads();
        }
    }
}

template <int WM, int WN, int TM, int TN, int KC, bool SUBTRACT, bool TOUT = false>
int launch_cgemm(GemmBatch batch, int kernel_id, hipStream_t s)
{
    constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
    double flops = 0.0;
    int64_t total = 0;
    for (int i = 0; i < batch.count; ++i) {
        GemmProblem &P = batch.p[i];
        if (P.K % KC != 0) return fail(MSOLVE_E_ARG, "cgemm: K must be a multiple of the chunk");
        P.tiles_n = (P.N + BN - 1) / BN;
        if (P.lower) {
            if (batch.count != 1 || P.M != P.N || BN % BM != 0)
                return fail(MSOLVE_E_ARG, "cgemm: lower needs one square product and whole row tiles per band");
            P.tiles = (BN / BM) * P.tiles_n * (P.tiles_n + 1) / 2;
            // the entries on and below the diagonal
            flops += 8.0 * double(P.M) * double(P.M + 1) / 2.0 * double(P.K) * double(P.nb);
        } else {
            P.tiles = ((P.M + BM - 1) / BM) * P.tiles_n;
            flops += 8.0 * double(P.M) * double(P.N) * double(P.K) * double(P.nb);
        }
        total += P.tiles * P.nb;
    }
    if (total == 0) return MSOLVE_OK;
    if (batch.count == 1) total = (total + 7) / 8 * 8;   // XCD swizzle covers 8 * ceil(T / 8)
    // the kernel's static LDS (A and B chunks, double-buffered)
    constexpr size_t kStatic = sizeof(float2) * 2 * (size_t(BM) * (KC + 2) + size_t(KC) * (BN + 2));
    const size_t dyn = !TOUT && total <= batch.lds_tiles_max && size_t(batch.lds_bytes) > kStatic
                           ? size_t(batch.lds_bytes) - kStatic
                           : 0;
    ProfScope prof(kernel_id, s, flops);
    hipLaunchKernelGGL((cgemm_kernel<WM, WN, TM, TN, KC, SUBTRACT, TOUT>), dim3(unsigned(total)),
                       dim3(WM * WN * 64), dyn, s, batch);
    MS_HIP(hipGetLastError());
    return MSOLVE_OK;
}

// a batch of nb products with operand strides sA, sB, sC (floats)
GemmProblem make_problem(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                         const float *B, int64_t ldb, float *C, int64_t ldc, int64_t nb,
                         int64_t sA, int64_t sB, int64_t sC)
{
    GemmProblem p;
    p.M = M; p.N = N; p.K = K;
    p.A = A; p.B = B; p.C = C;
    p.lda = lda; p.ldb = ldb; p.ldc = ldc;
    p.nb = nb; p.sA = sA; p.sB = sB; p.sC = sC;
    p.tiles_n = 0; p.tiles = 0;
    p.lower = 0;
    p.T = nullptr; p.Dg = nullptr; p.ldt = 0; p.ldd = 0;
    return p;
}

}  // namespace

namespace {

// tile configurations (chosen by timing the kernel alone on MI355X):
// skinny and small products use 64 x 64 tiles, the bulk trailing update
// 64 x 128 tiles with eight waves; both walk K in chunks of 8.
#define MS_SMALL_SUB 2, 2, 1, 1, 8, true
#define MS_SMALL_SET 2, 2, 1, 1, 8, false
#define MS_SMALL_SET_T 2, 2, 1, 1, 8, false, true
#define MS_BULK_SUB 2, 4, 1, 1, 8, true
// The trailing (bulk) update runs beside the serial chain of the next
// group (diagonal steps, panels, L-region updates).  When bulk workgroups
// fill a CU, a chain workgroup only starts where several of them have left
// the same CU, and the chain, not the bulk product, then sets the pace.
// Each bulk workgroup therefore reserves 54 KB of LDS: three do not fit in a
// CU's 160 KB, and beside two there remain 52 KB for a chain workgroup.
// (The 64 x 128 bulk kernel's registers allow two per CU anyway; the cap
// binds the 64 x 64 kernel of the smaller bulk products.)  Large bulk
// products (more tiles than kBulkCapTiles) outlast the chain and are not
// capped.
constexpr int kBulkLdsBytes = 55296;
constexpr int64_t kBulkCapTiles = 16384;

// The factorisation of a batch: nf matrices of order n at A + f sA (floats),
// their Dinv at Dinv + f sD and pivot reports at d_info + f.  Every launch
// below covers the whole batch.
struct FactorBatch {
    int64_t n, nf;
    float *A;
    int64_t sA;
    float *Dinv;
    int64_t sD;
    int32_t *d_info;
    // complex-symmetric matrices (A^T = A): the trailing updates touch only
    // the entries on and below the diagonal, and each block row of U is
    // formed as D L^T from its block column of L
    bool sym;
    // nf hand-off words of the general diagonal steps (zeroed at the start)
    uint32_t *flags;
};

float *blk(float *A, int64_t n, int64_t r, int64_t c) { return A + 2 * (size_t(r) * size_t(n) + size_t(c)); }

int launch_diag(const FactorBatch &fb, int64_t kb, hipStream_t s)
{
    // LU (8/3 NB^3 real flops) and the two triangular inverses (4/3 NB^3 each)
    const double flops = 16.0 / 3.0 * double(kNB) * double(kNB) * double(kNB) * double(fb.nf);
    ProfScope prof(MSOLVE_K_LU_DIAG, s, flops);
    float *Dinv_blk = fb.Dinv + size_t(kb) * 2 * 2 * kNB * kNB;
    if (fb.sym)
        hipLaunchKernelGGL((lu_diag_kernel<kNB, true>), dim3(unsigned(fb.nf)), dim3(kDiagWaves * 64), 0, s, fb.n,
                           kb * kNB, fb.A, fb.sA, Dinv_blk, fb.sD, fb.d_info, nullptr, 0u);
    else
        hipLaunchKernelGGL((lu_diag_kernel<kNB, false>), dim3(unsigned(2 * fb.nf)), dim3(kDiagWaves * 64), 0, s,
                           fb.n, kb * kNB, fb.A, fb.sA, Dinv_blk, fb.sD, fb.d_info, fb.flags, uint32_t(kb + 1));
    MS_HIP(hipGetLastError());
    return MSOLVE_OK;
}

// U12 = L11^-1 A12 over the columns right of block kb and L21 = A21 U11^-1
// over the rows below it (in place; one batched launch)
int launch_panel(const FactorBatch &fb, int64_t kb, hipStream_t s)
{
    const int64_t n = fb.n, nb = kNB, k0 = kb * nb, rest = n - k0 - nb;
    const float *Linv = fb.Dinv + size_t(kb) * 2 * 2 * nb * nb;
    const float *Uinv = Linv + 2 * nb * nb;
    float *A12 = blk(fb.A, n, k0, k0 + nb);
    float *A21 = blk(fb.A, n, k0 + nb, k0);
    if (fb.sym) {
        // L21 = A21 U11^-1, and from each tile of it the block row of U:
        // U[k0 + c][k0 + nb + r] = u_cc L21[r][c].  (Page "Solving Dense
        // Matrices Fast in the Browser", section "Measure first: the ceiling
        // of JavaScript": Z equals its transpose, and a factorisation that
        // uses this does half the work of LU.  With A = L U and A^T = A,
        // U = D L^T for D = diag(U), so the block row of U needs no product
        // of its own, and the trailing updates need only the entries on and
        // below the diagonal.)
        GemmBatch col;
        col.count = 1;
        col.prio = 1;
        col.p[0] = make_problem(rest, nb, nb, A21, n, Uinv, nb, A21, n, fb.nf, fb.sA, fb.sD, fb.sA);
        col.p[0].T = A12;
        col.p[0].ldt = n;
        col.p[0].Dg = blk(fb.A, n, k0, k0);
        col.p[0].ldd = n + 1;
        return launch_cgemm<MS_SMALL_SET_T>(col, MSOLVE_K_LU_PANEL, s);
    }
    GemmBatch panel;
    panel.count = 2;
    panel.prio = 1;
    // C aliases B (BM = nb spans all rows) and C aliases A (BN = nb spans all columns)
    panel.p[0] = make_problem(nb, rest, nb, Linv, nb, A12, n, A12, n, fb.nf, fb.sD, fb.sA, fb.sA);
    panel.p[1] = make_problem(rest, nb, nb, A21, n, Uinv, nb, A21, n, fb.nf, fb.sA, fb.sD, fb.sA);
    return launch_cgemm<MS_SMALL_SET>(panel, MSOLVE_K_LU_PANEL, s);
}

// Update of the L-shaped region at q0 of width w -- columns [q0, q0+w) for
// rows >= q0 and rows [q0, q0+w) for columns >= q0+w -- with the panels of
// the K columns starting at c0 (c0 + K <= q0).
int update_lregion(const FactorBatch &fb, int64_t c0, int64_t K, int64_t q0, int64_t w, hipStream_t s)
{
    const int64_t n = fb.n, right = n - q0 - w;
    float *A = fb.A;
    GemmBatch g;
    g.prio = 1;
    // (symmetric: the rows of the region right of it are formed by the
    // panel steps from the columns, so only the columns are updated)
    g.count = right > 0 && !fb.sym ? 2 : 1;
    g.p[0] = make_problem(n - q0, w, K, blk(A, n, q0, c0), n, blk(A, n, c0, q0), n,
                          blk(A, n, q0, q0), n, fb.nf, fb.sA, fb.sA, fb.sA);
    if (right > 0)
        g.p[1] = make_problem(w, right, K, blk(A, n, q0, c0), n, blk(A, n, c0, q0 + w), n,
                              blk(A, n, q0, q0 + w), n, fb.nf, fb.sA, fb.sA, fb.sA);
    return launch_cgemm<MS_SMALL_SUB>(g, MSOLVE_K_LU_UPDATE, s);
}

// trailing update A[r0:, r0:] -= A[r0:, c0:c0+K] A[c0:c0+K, r0:]
int update_bulk(const FactorBatch &fb, int64_t c0, int64_t K, int64_t r0, hipStream_t s)
{
    const int64_t n = fb.n, m = n - r0;
    float *A = fb.A;
    GemmBatch upd;
    upd.count = 1;
    upd.p[0] = make_problem(m, m, K, blk(A, n, r0, c0), n, blk(A, n, c0, r0), n, blk(A, n, r0, r0),
                            n, fb.nf, fb.sA, fb.sA, fb.sA);
    upd.p[0].lower = fb.sym ? 1 : 0;
    upd.group_rows = 8;
    upd.lds_bytes = kBulkLdsBytes;
    upd.lds_tiles_max = kBulkCapTiles;
    if (m >= 1024) return launch_cgemm<MS_BULK_SUB>(upd, MSOLVE_K_LU_BULK, s);
    return launch_cgemm<MS_SMALL_SUB>(upd, MSOLVE_K_LU_UPDATE, s);
}

// Factorise the group of up to G blocks starting at block kb, assuming its
// L-shaped region already holds every update from blocks before kb.  Inside
// the group the blocks go left-looking: block j's row and column first
// receive the updates of blocks kb..j-1, then its diagonal and panel steps
// run.  The trailing matrix beyond the group is not touched.  *covered is
// the number of blocks factorised.
int factor_group(const FactorBatch &fb, int64_t kb, int G, hipStream_t s, int *covered)
{
    const int64_t n = fb.n, nb = kNB, nblk = nblocks(n);
    *covered = 0;
    for (int64_t j = kb; j < kb + G && j < nblk; ++j) {
        const int64_t q0 = j * nb;
        if (j > kb) MS_TRY(update_lregion(fb, kb * nb, q0 - kb * nb, q0, std::min<int64_t>(nb, n - q0), s));
        MS_TRY(launch_diag(fb, j, s));
        *covered += 1;
        if (n - q0 - nb <= 0) break;
        MS_TRY(launch_panel(fb, j, s));
    }
    return MSOLVE_OK;
}

}  // namespace

// Blocks are taken in groups of G (8, 4 or 2 by size, see below); each
// group's bulk trailing update is one product with K = G nb, which divides
// the passes over the trailing matrix by G.
//
// sla (nullable): a second stream for look-ahead.  With it, while the main
// stream applies group g's update to the trailing matrix beyond group g+1,
// the second stream brings group g+1's rows and columns up to date and
// factorises group g+1, so the serial diagonal and panel steps overlap the
// bulk product.  The writes of the two streams are disjoint.
// The look-ahead stream of the current device: created on first use and
// kept for the life of the process (one per device).
namespace {
// a non-blocking stream per device and purpose, created on first use and
// kept for the life of the process
int cached_stream(int slot, hipStream_t *out)
{
    struct Entry {
        int dev, slot;
        hipStream_t s;
    };
    static std::mutex mu;
    static std::vector<Entry> cache;
    int dev = 0;
    MS_HIP(hipGetDevice(&dev));
    std::lock_guard<std::mutex> g(mu);
    for (const Entry &e : cache)
        if (e.dev == dev && e.slot == slot) {
            *out = e.s;
            return MSOLVE_OK;
        }
    hipStream_t st = nullptr;
    MS_HIP(hipStreamCreateWithFlags(&st, hipStreamNonBlocking));
    cache.push_back(Entry{dev, slot, st});
    *out = st;
    return MSOLVE_OK;
}
}  // namespace

int lookahead_stream(hipStream_t *out) { return cached_stream(0, out); }
int poll_stream(hipStream_t *out) { return cached_stream(1, out); }
int front_stream(hipStream_t *out) { return cached_stream(2, out); }

// the coupling blocks of the pairs t0 .. t1 - 1 (pairs of blocks that are
// both factorised)
int launch_couplings(int64_t n, int64_t nf, const float *A, int64_t sA, float *Dinv, int64_t sD,
                     int64_t t0, int64_t t1, hipStream_t s)
{
    if (t1 <= t0) return MSOLVE_OK;
    hipLaunchKernelGGL(coupling_kernel, dim3(unsigned(t1 - t0), unsigned(nf), 8), dim3(256), 0, s, n,
                       t0, A, sA, Dinv, sD);
    MS_HIP(hipGetLastError());
    return MSOLVE_OK;
}

int factor_blocks(int64_t n, int64_t nf, float *A, int64_t sA, float *Dinv, int64_t sD,
                  int32_t *d_info, bool sym, uint32_t *flags, hipStream_t s, hipStream_t sla);

int launch_factor(int64_t n, int64_t nf, float *A, int64_t sA, float *Dinv, int64_t sD,
                  int32_t *d_info, bool sym, uint32_t *flags, hipStream_t s, hipStream_t sla)
{
    return factor_blocks(n, nf, A, sA, Dinv, sD, d_info, sym, flags, s, sla);
}

int factor_blocks(int64_t n, int64_t nf, float *A, int64_t sA, float *Dinv, int64_t sD,
                  int32_t *d_info, bool sym, uint32_t *flags, hipStream_t s, hipStream_t sla)
{
    MS_TRY(launch_fill_u32(reinterpret_cast<uint32_t *>(d_info), size_t(nf), 0u, s));
    if (!sym) MS_TRY(launch_fill_u32(flags, size_t(nf), 0u, s));
    const FactorBatch fb{n, nf, A, sA, Dinv, sD, d_info, sym, flags};
    const int64_t nb = kNB;
    const int64_t nblk = nblocks(n);
    // blocks per group (K of the bulk products = G nb): 8 from order 12288,
    // where the bulk products set the pace (half the passes over the
    // trailing matrix); 4 once the trailing matrices are large (order 4096,
    // or a batch of four or more), else 2
    const int G = n >= 12288 ? 8 : ((n >= 4096 || nf >= 4) ? 4 : 2);
    // the coupling blocks of every pair within the first `blocks` blocks
    // not yet coupled (groups start at even blocks, so pairs never straddle
    // two groups)
    int64_t coupled = 0;
    auto couple = [&](int64_t blocks, hipStream_t st) -> int {
        const int64_t t1 = blocks / 2;
        MS_TRY(launch_couplings(n, nf, A, sA, Dinv, sD, coupled, t1, st));
        coupled = std::max(coupled, t1);
        return MSOLVE_OK;
    };
    if (!sla || nblk < 3 * G) {
        int64_t kb = 0;
        while (kb < nblk) {
            int covered = 0;
            MS_TRY(factor_group(fb, kb, G, s, &covered));
            MS_TRY(couple(kb + covered, s));
            const int64_t r0 = (kb + covered) * nb;
            if (r0 < n) MS_TRY(update_bulk(fb, kb * nb, covered * nb, r0, s));
            kb += covered;
        }
        return MSOLVE_OK;
    }

    // While s applies group g's update to the trailing matrix beyond group
    // g+1, the look-ahead stream brings group g+1's rows and columns up to
    // date and factorises group g+1, so the serial steps overlap the bulk
    // product.  The writes of the two streams are disjoint.
    hipStream_t sb = s;
    hipEvent_t ev[2] = {nullptr, nullptr};
    const bool lreg_first = nf >= 4 && n <= 4096;
    auto body = [&]() -> int {
        for (auto &e : ev) MS_HIP(hipEventCreateWithFlags(&e, hipEventDisableTiming));
        hipEvent_t ev_rest = ev[0], ev_grp = ev[1];
        // the look-ahead stream starts after everything queued on s so far
        MS_HIP(hipEventRecord(ev_rest, s));
        MS_HIP(hipStreamWaitEvent(sla, ev_rest, 0));
        // ev_grp marks a factorised group: its panels are final, which is all
        // that its bulk update needs.  The bulk update of group g (beyond
        // group g+1) and the L-region update of group g+1 write disjoint
        // parts of the matrix and only read group g's panels, so they run
        // side by side; group g+1's L-region must follow the bulk update of
        // group g-1, which wrote it.
        int covered = 0;
        int64_t kb = 0;
        MS_TRY(factor_group(fb, kb, G, sla, &covered));
        MS_HIP(hipEventRecord(ev_grp, sla));
        while (true) {
            const int64_t c0 = kb * nb, K = covered * nb;
            const int64_t q0 = c0 + K;                      // next group starts here
            if (q0 >= n) break;
            const int64_t w = std::min<int64_t>(G * nb, n - q0);
            // bulk stream: the trailing matrix beyond the next group
            const int64_t r0 = q0 + w;
            const int64_t kn = q0 / nb;
            // look-ahead stream: next group's rows/columns with this group's
            // panels.  The chain's workgroups (diagonal steps of 44-46
            // registers and 16 waves, panels, L-region updates) find room
            // beside two bulk workgroups on every CU (see kBulkLdsBytes) and,
            // with their raised priority, run there at close to their own
            // speed, so the chain needs no head start.
            MS_TRY(update_lregion(fb, c0, K, q0, w, sla));
            // batches of moderate order: the bulk update starts after this
            // L-region update, which then has the GPU to itself instead of
            // sharing it with the bulk product (the chain sets the pace there)
            if (lreg_first) MS_HIP(hipEventRecord(ev_grp, sla));
            // bulk stream: the trailing matrix beyond the next group, then
            // this group's couplings
            MS_HIP(hipStreamWaitEvent(sb, ev_grp, 0));
            if (r0 < n) MS_TRY(update_bulk(fb, c0, K, r0, sb));
            MS_TRY(couple(kb + covered, sb));
            // look-ahead stream: the next group
            MS_TRY(factor_group(fb, kn, G, sla, &covered));
            MS_HIP(hipEventRecord(ev_grp, sla));
            // the L-region update after next must follow this bulk update
            MS_HIP(hipEventRecord(ev_rest, sb));
            MS_HIP(hipStreamWaitEvent(sla, ev_rest, 0));
            kb = kn;
        }
        // join: s continues after everything on the look-ahead stream
        MS_HIP(hipEventRecord(ev_grp, sla));
        MS_HIP(hipStreamWaitEvent(s, ev_grp, 0));
        return couple(nblk, s);
    };
    const int st = body();
    for (auto &e : ev)
        if (e) (void)hipEventDestroy(e);
    return st;
}

}  // namespace msolve

namespace msolve {
namespace {
int factor_entry(const char *name, bool sym, int64_t n, float *A, float *Dinv, int32_t *d_info,
                 void *work, size_t work_bytes, void *stream)
{
    if (n < 1) return fail(MSOLVE_E_ARG, std::string(name) + ": n must be >= 1");
    if (!A || !Dinv || !d_info) return fail(MSOLVE_E_ARG, std::string(name) + ": null pointer");
    if (work_bytes < msolve_factor_workspace_bytes(n))
        return fail(MSOLVE_E_WORKSPACE, std::string(name) + ": workspace too small");
    if (!work) return fail(MSOLVE_E_ARG, std::string(name) + ": null workspace");
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint32_t *flags = static_cast<uint32_t *>(work);
    if (nblocks(n) < 12) return launch_factor(n, 1, A, 0, Dinv, 0, d_info, sym, flags, s, nullptr);
    hipStream_t sla = nullptr;
    MS_TRY(lookahead_stream(&sla));
    return launch_factor(n, 1, A, 0, Dinv, 0, d_info, sym, flags, s, sla);
}
}  // namespace
}  // namespace msolve

extern "C" int msolve_factor_c64(int64_t n, float *A, float *Dinv, int32_t *d_info, void *work,
                                 size_t work_bytes, void *stream)
{
    return msolve::factor_entry("msolve_factor_c64", false, n, A, Dinv, d_info, work, work_bytes, stream);
}

extern "C" int msolve_factor_c64_sym(int64_t n, float *A, float *Dinv, int32_t *d_info, void *work,
                                     size_t work_bytes, void *stream)
{
    return msolve::factor_entry("msolve_factor_c64_sym", true, n, A, Dinv, d_info, work, work_bytes,
                                stream);
}

extern "C" int msolve_factor_c64_batch(int64_t n, int64_t nf, float *A, int64_t stride_A, float *Dinv,
                                       int64_t stride_D, int32_t *d_info, int32_t sym, void *work,
                                       size_t work_bytes, void *stream)
{
    using namespace msolve;
    if (n < 1 || nf < 1 || nf > 65535) return fail(MSOLVE_E_ARG, "msolve_factor_c64_batch: bad sizes");
    if (!A || !Dinv || !d_info) return fail(MSOLVE_E_ARG, "msolve_factor_c64_batch: null pointer");
    if (stride_A < 2 * n * n || stride_D < int64_t(msolve_dinv_floats(n)))
        return fail(MSOLVE_E_ARG, "msolve_factor_c64_batch: strides smaller than one matrix");
    if (!work) return fail(MSOLVE_E_ARG, "msolve_factor_c64_batch: null workspace");
    if (work_bytes < msolve_factor_batch_workspace_bytes(n, nf))
        return fail(MSOLVE_E_WORKSPACE, "msolve_factor_c64_batch: workspace too small");
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipStream_t sla = nullptr;
    if (nblocks(n) >= 12) MS_TRY(lookahead_stream(&sla));
    return launch_factor(n, nf, A, stride_A, Dinv, stride_D, d_info, sym != 0, static_cast<uint32_t *>(work), s,
                         sla);
}
