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
//      one dense contraction, on FP32 matrix cores.
//
// The complex product is built from real v_mfma_f32_32x32x2f32 operations
// with separate accumulators for the real and the imaginary part:
//   Cr += Ar Br - Ai Bi,   Ci += Ar Bi + Ai Br   (4 real MFMAs, 8 flop per
// complex multiply-add).  The two K slots of each MFMA carry the two halves
// of the current K chunk, so both operands are read in their natural
// interleaved complex layout and no repacking pass is needed.
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

// Thread (ti, tj) of an R x R grid owns rows ti + R*a and columns tj + R*b
// (a, b = 0..3) of the NB x NB block: a cyclic layout, so the shrinking
// active region stays spread over all threads.  Step j needs row j and
// column j of the current matrix plus 1 / pivot; their owners publish them
// in LDS (double-buffered by step parity), so each step costs one barrier.
//
// Alongside the elimination the kernel builds, by column sweeps that use the
// same published rows and columns:
//   X = L^-1:        X = I; at step j, X[r][:] -= L[r][j] X[j][:]  (r > j)
//   W = (U^T)^-1:    W = I; at step j, W[j][:] /= U[j][j], then
//                    W[r][:] -= U[j][r] W[j][:]  (r > j)
// so that U^-1 = W^T.
template <int NB>
__global__ __launch_bounds__((NB / 4) * (NB / 4)) void lu_diag_kernel(
    int64_t n, int64_t k0, float *A, float *Dinv_blk, int32_t *d_info)
{
    constexpr int R = NB / 4;
    const int ti = threadIdx.x / R, tj = threadIdx.x % R;
    const int nv = int(min<int64_t>(NB, n - k0));
    float2 *Ac = reinterpret_cast<float2 *>(A);

    __shared__ float2 urow[2][NB], lcol[2][NB], xrow[2][NB], wrow[2][NB];
    __shared__ float2 pinv[2];
    __shared__ int bad_step;

    float2 a[4][4], x[4][4], wv[4][4];
#pragma unroll
    for (int ia = 0; ia < 4; ++ia) {
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) {
            const int r = ti + R * ia, c = tj + R * ib;
            const float2 one = make_float2(r == c ? 1.0f : 0.0f, 0.0f);
            if (r < nv && c < nv)
                a[ia][ib] = Ac[size_t(k0 + r) * size_t(n) + size_t(k0 + c)];
            else
                a[ia][ib] = one;
            x[ia][ib] = one;
            wv[ia][ib] = one;
        }
    }
    if (threadIdx.x == 0) {
        // thread 0 owns element (0, 0)
        bool bad;
        pinv[0] = cinv_checked(a[0][0], &bad);
        bad_step = bad ? 1 : 0;
    }
    // publish step 0
    if (ti == 0) {
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) {
            const int c = tj + R * ib;
            urow[0][c] = a[0][ib];
            xrow[0][c] = x[0][ib];
            wrow[0][c] = wv[0][ib];
        }
    }
    if (tj == 0) {
#pragma unroll
        for (int ia = 0; ia < 4; ++ia) lcol[0][ti + R * ia] = a[ia][0];
    }
    __syncthreads();

    for (int j = 0; j < NB; ++j) {
        const int p = j & 1, q = p ^ 1;
        const float2 inv = pinv[p];
        float2 l[4], ur[4], uc[4], xr[4], wr[4];
#pragma unroll
        for (int ia = 0; ia < 4; ++ia) {
            const int r = ti + R * ia;
            l[ia] = (r > j) ? cmul(lcol[p][r], inv) : make_float2(0.0f, 0.0f);
            ur[ia] = urow[p][r];
        }
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) {
            const int c = tj + R * ib;
            uc[ib] = urow[p][c];
            xr[ib] = xrow[p][c];
            wr[ib] = cmul(wrow[p][c], inv);
        }
#pragma unroll
        for (int ia = 0; ia < 4; ++ia) {
            const int r = ti + R * ia;
#pragma unroll
            for (int ib = 0; ib < 4; ++ib) {
                const int c = tj + R * ib;
                if (r > j) {
                    if (c > j) {
                        a[ia][ib] = cfms(a[ia][ib], l[ia], uc[ib]);
                    } else {
                        if (c == j) a[ia][ib] = l[ia];          // column j of L
                        x[ia][ib] = cfms(x[ia][ib], l[ia], xr[ib]);
                        wv[ia][ib] = cfms(wv[ia][ib], ur[ia], wr[ib]);
                    }
                } else if (r == j && c <= j) {
                    wv[ia][ib] = wr[ib];                        // row j of W is final
                }
            }
        }
        if (j + 1 < NB) {
            const int jj = j + 1;
#pragma unroll
            for (int ia = 0; ia < 4; ++ia) {
                if (ti + R * ia != jj) continue;
#pragma unroll
                for (int ib = 0; ib < 4; ++ib) {
                    const int c = tj + R * ib;
                    if (c >= jj) urow[q][c] = a[ia][ib];
                    if (c <= jj) {
                        xrow[q][c] = x[ia][ib];
                        wrow[q][c] = wv[ia][ib];
                    }
                    if (c == jj) {
                        bool bad;
                        pinv[q] = cinv_checked(a[ia][ib], &bad);
                        if (bad && bad_step == 0) bad_step = jj + 1;
                    }
                }
            }
#pragma unroll
            for (int ib = 0; ib < 4; ++ib) {
                if (tj + R * ib != jj) continue;
#pragma unroll
                for (int ia = 0; ia < 4; ++ia) {
                    const int r = ti + R * ia;
                    if (r > jj) lcol[q][r] = a[ia][ib];
                }
            }
        }
        __syncthreads();
    }

    // write back: L\U into A (valid part), L^-1 and U^-1 = W^T into Dinv
    float2 *Linv = reinterpret_cast<float2 *>(Dinv_blk);
    float2 *Uinv = Linv + NB * NB;
#pragma unroll
    for (int ia = 0; ia < 4; ++ia) {
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) {
            const int r = ti + R * ia, c = tj + R * ib;
            if (r < nv && c < nv) Ac[size_t(k0 + r) * size_t(n) + size_t(k0 + c)] = a[ia][ib];
            Linv[r * NB + c] = x[ia][ib];
            Uinv[c * NB + r] = wv[ia][ib];
        }
    }
    if (threadIdx.x == 0 && bad_step != 0 && bad_step <= nv) {
        if (atomicCAS(d_info, 0, int32_t(k0 + bad_step)) != 0) { /* earlier pivot kept */ }
    }
}

// ----------------------------------------------------------- cgemm kernel

struct GemmProblem {
    int64_t M, N, K;          // complex dimensions, K % KC == 0
    const float *A;           // M x K, row stride lda (complex elements)
    const float *B;           // K x N, row stride ldb
    float *C;                 // M x N, row stride ldc (may alias A or B, see below)
    int64_t lda, ldb, ldc;
    int64_t tiles_n;          // column tiles
    int64_t tiles;            // total tiles
};

struct GemmBatch {
    GemmProblem p[2];
    int count;
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
template <int WM, int WN, int TM, int TN, int KC, bool SUBTRACT>
__global__ __launch_bounds__(WM *WN * 64) void cgemm_kernel(GemmBatch batch)
{
    constexpr int THREADS = WM * WN * 64;
    constexpr int BM = WM * TM * 32;
    constexpr int BN = WN * TN * 32;
    constexpr int APAD = 2, BPAD = 2;
    constexpr int ALD = KC + APAD;       // LDS row stride of A (complex)
    constexpr int BLD = BN + BPAD;       // LDS row stride of B (complex)
    constexpr int HALF = KC / 2;
    constexpr int A_PIECES = BM * KC / 2 / THREADS;   // 2-complex pieces per thread
    constexpr int B_PIECES = KC * BN / 2 / THREADS;
    static_assert(A_PIECES * THREADS * 2 == BM * KC, "A chunk must split evenly");
    static_assert(B_PIECES * THREADS * 2 == KC * BN, "B chunk must split evenly");

    __shared__ float2 As[2][BM * ALD];
    __shared__ float2 Bs[2][KC * BLD];

    int64_t t = blockIdx.x;
    int pi = 0;
    if (batch.count > 1 && t >= batch.p[0].tiles) {
        t -= batch.p[0].tiles;
        pi = 1;
    }
    const GemmProblem P = batch.p[pi];
    const int64_t m0 = (t / P.tiles_n) * BM;
    const int64_t n0 = (t % P.tiles_n) * BN;
    const float2 *Ag = reinterpret_cast<const float2 *>(P.A);
    const float2 *Bg = reinterpret_cast<const float2 *>(P.B);
    float2 *Cg = reinterpret_cast<float2 *>(P.C);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int l32 = lane & 31, h = lane >> 5;

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

    float2 ra[A_PIECES][2], rb[B_PIECES][2];
    auto load_chunk = [&](int64_t k) {
#pragma unroll
        for (int i = 0; i < A_PIECES; ++i) {
            const int e = tid + THREADS * i;
            const int row = e / (KC / 2), kp = e % (KC / 2);
            const int64_t gm = m0 + row;
            if (gm < P.M) {
                const float2 *src = Ag + size_t(gm) * size_t(P.lda) + size_t(k + 2 * kp);
                ra[i][0] = src[0];
                ra[i][1] = src[1];
            } else {
                ra[i][0] = make_float2(0.0f, 0.0f);
                ra[i][1] = make_float2(0.0f, 0.0f);
            }
        }
#pragma unroll
        for (int i = 0; i < B_PIECES; ++i) {
            const int e = tid + THREADS * i;
            const int kr = e / (BN / 2), np = e % (BN / 2);
            const int64_t gn = n0 + 2 * np;
            const float2 *src = Bg + size_t(k + kr) * size_t(P.ldb) + size_t(gn);
            rb[i][0] = (gn < P.N) ? src[0] : make_float2(0.0f, 0.0f);
            rb[i][1] = (gn + 1 < P.N) ? src[1] : make_float2(0.0f, 0.0f);
        }
    };
    auto store_chunk = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_PIECES; ++i) {
            const int e = tid + THREADS * i;
            const int row = e / (KC / 2), kp = e % (KC / 2);
            As[buf][row * ALD + 2 * kp] = ra[i][0];
            As[buf][row * ALD + 2 * kp + 1] = ra[i][1];
        }
#pragma unroll
        for (int i = 0; i < B_PIECES; ++i) {
            const int e = tid + THREADS * i;
            const int kr = e / (BN / 2), np = e % (BN / 2);
            Bs[buf][kr * BLD + 2 * np] = rb[i][0];
            Bs[buf][kr * BLD + 2 * np + 1] = rb[i][1];
        }
    };

    const int64_t nk = P.K / KC;
    load_chunk(0);
    store_chunk(0);
    __syncthreads();
    for (int64_t kc = 0; kc < nk; ++kc) {
        const int buf = int(kc & 1);
        if (kc + 1 < nk) load_chunk((kc + 1) * KC);
        const float2 *as = As[buf] + (wm * TM * 32 + l32) * ALD + h * HALF;
        const float2 *bs = Bs[buf] + (h * HALF) * BLD + wn * TN * 32 + l32;
#pragma unroll
        for (int s = 0; s < HALF; ++s) {
            float2 av[TM], bv[TN];
#pragma unroll
            for (int a = 0; a < TM; ++a) av[a] = as[a * 32 * ALD + s];
#pragma unroll
            for (int b = 0; b < TN; ++b) bv[b] = bs[s * BLD + b * 32];
#pragma unroll
            for (int a = 0; a < TM; ++a) {
#pragma unroll
                for (int b = 0; b < TN; ++b) {
                    cr[a][b] = mfma32(av[a].x, bv[b].x, cr[a][b]);
                    cr[a][b] = mfma32(av[a].y, -bv[b].y, cr[a][b]);
                    ci[a][b] = mfma32(av[a].x, bv[b].y, ci[a][b]);
                    ci[a][b] = mfma32(av[a].y, bv[b].x, ci[a][b]);
                }
            }
        }
        if (kc + 1 < nk) store_chunk(buf ^ 1);
        __syncthreads();
    }

    // epilogue: lane holds rows (r/4)*8 + h*4 + r%4 of column l32 of each sub-tile
#pragma unroll
    for (int a = 0; a < TM; ++a) {
#pragma unroll
        for (int b = 0; b < TN; ++b) {
            const int64_t col = n0 + wn * TN * 32 + b * 32 + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = m0 + wm * TM * 32 + a * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
                if (row < P.M && col < P.N) {
                    float2 *cp = Cg + size_t(row) * size_t(P.ldc) + size_t(col);
                    if (SUBTRACT) {
                        const float2 v = *cp;
                        *cp = make_float2(v.x - cr[a][b][r], v.y - ci[a][b][r]);
                    } else {
                        *cp = make_float2(cr[a][b][r], ci[a][b][r]);
                    }
                }
            }
        }
    }
}

template <int WM, int WN, int TM, int TN, int KC, bool SUBTRACT>
int launch_cgemm(GemmBatch batch, int kernel_id, hipStream_t s)
{
    constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
    double flops = 0.0;
    int64_t total = 0;
    for (int i = 0; i < batch.count; ++i) {
        GemmProblem &P = batch.p[i];
        if (P.K % KC != 0) return fail(MSOLVE_E_ARG, "cgemm: K must be a multiple of the chunk");
        P.tiles_n = (P.N + BN - 1) / BN;
        P.tiles = ((P.M + BM - 1) / BM) * P.tiles_n;
        total += P.tiles;
        flops += 8.0 * double(P.M) * double(P.N) * double(P.K);
    }
    if (total == 0) return MSOLVE_OK;
    ProfScope prof(kernel_id, s, flops);
    hipLaunchKernelGGL((cgemm_kernel<WM, WN, TM, TN, KC, SUBTRACT>), dim3(unsigned(total)),
                       dim3(WM * WN * 64), 0, s, batch);
    MS_HIP(hipGetLastError());
    return MSOLVE_OK;
}

GemmProblem make_problem(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                         const float *B, int64_t ldb, float *C, int64_t ldc)
{
    GemmProblem p;
    p.M = M; p.N = N; p.K = K;
    p.A = A; p.B = B; p.C = C;
    p.lda = lda; p.ldb = ldb; p.ldc = ldc;
    p.tiles_n = 0; p.tiles = 0;
    return p;
}

}  // namespace

int launch_factor(int64_t n, float *A, float *Dinv, int32_t *d_info, hipStream_t s)
{
    MS_TRY(launch_fill_u32(reinterpret_cast<uint32_t *>(d_info), 1, 0u, s));
    const int64_t nb = kNB;
    const int64_t nblk = nblocks(n);
    for (int64_t kb = 0; kb < nblk; ++kb) {
        const int64_t k0 = kb * nb;
        float *dblk = Dinv + size_t(kb) * 2 * 2 * nb * nb;
        {
            const double flops = 8.0 * double(nb) * double(nb) * double(nb);  // LU + two inverses
            ProfScope prof(MSOLVE_K_LU_DIAG, s, flops);
            hipLaunchKernelGGL((lu_diag_kernel<kNB>), dim3(1), dim3((kNB / 4) * (kNB / 4)), 0, s, n,
                               k0, A, dblk, d_info);
            MS_HIP(hipGetLastError());
        }
        const int64_t rest = n - k0 - nb;
        if (rest <= 0) continue;
        const float *Linv = dblk;
        const float *Uinv = dblk + 2 * nb * nb;
        float *A12 = A + 2 * (size_t(k0) * size_t(n) + size_t(k0 + nb));
        float *A21 = A + 2 * (size_t(k0 + nb) * size_t(n) + size_t(k0));
        float *A22 = A + 2 * (size_t(k0 + nb) * size_t(n) + size_t(k0 + nb));
        // panel: U12 = L11^-1 A12 (C aliases B; BM = nb spans all rows) and
        //        L21 = A21 U11^-1 (C aliases A; BN = nb spans all columns)
        GemmBatch panel;
        panel.count = 2;
        panel.p[0] = make_problem(nb, rest, nb, Linv, nb, A12, n, A12, n);
        panel.p[1] = make_problem(rest, nb, nb, A21, n, Uinv, nb, A21, n);
        MS_TRY((launch_cgemm<2, 2, 1, 1, 16, false>(panel, MSOLVE_K_LU_PANEL, s)));
        GemmBatch upd;
        upd.count = 1;
        upd.p[0] = make_problem(rest, rest, nb, A21, n, A12, n, A22, n);
        const int64_t big_tiles = ((rest + 127) / 128) * ((rest + 127) / 128);
        if (big_tiles >= 512) {
            MS_TRY((launch_cgemm<2, 2, 2, 2, 16, true>(upd, MSOLVE_K_LU_UPDATE, s)));
        } else {
            MS_TRY((launch_cgemm<2, 2, 1, 1, 16, true>(upd, MSOLVE_K_LU_UPDATE, s)));
        }
    }
    return MSOLVE_OK;
}

}  // namespace msolve

extern "C" int msolve_factor_c64(int64_t n, float *A, float *Dinv, int32_t *d_info, void *work,
                                 size_t work_bytes, void *stream)
{
    using namespace msolve;
    if (n < 1) return fail(MSOLVE_E_ARG, "msolve_factor_c64: n must be >= 1");
    if (!A || !Dinv || !d_info) return fail(MSOLVE_E_ARG, "msolve_factor_c64: null pointer");
    if (work_bytes < msolve_factor_workspace_bytes(n))
        return fail(MSOLVE_E_WORKSPACE, "msolve_factor_c64: workspace too small");
    (void)work;
    return launch_factor(n, A, Dinv, d_info, static_cast<hipStream_t>(stream));
}
