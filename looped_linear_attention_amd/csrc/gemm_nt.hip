// gemm_nt.hip -- the plain products of the loop backward on bf16 MFMA, and
// the tiled transposes that give them K-contiguous operands (gfx950).
//
// LT2: Linear-Time Looped Transformers, Appendix C: every looped model is
// trained with bf16 mixed precision, so the gradients flow back through the
// weight-tied projection of each loop (Section 2, "Looped Transformer (LT)"
// and "LT2" paragraphs).  Per loop that is three products of the same shape
// class: the raw projections recomputed from the loop's input, the input
// gradient dY W and the weight gradient x^T dY.
//
// k_gemm_nt:  C[m][n] (op)= sum_k A[m][k] B[n][k], A and B K-contiguous rows.
// An operand is bf16 (used as is), fp32 split on the way into LDS as
// x ~ hi + lo (both bf16, about 16 significant bits; the products hi.hi +
// hi.lo + lo.hi when both are split, two when one is), or fp32 rounded to
// bf16 (the bf16 operand the forward used).  Accumulation is fp32 in the
// MFMA; the k order is fixed, so results are deterministic.
// Tile 128 x 128 x 32, four waves of 64 x 64 (2 x 2 MFMA 32x32x16 tiles).
// One LDS stage; the next k-step's operands are loaded into registers while
// the current one is multiplied.
#include "gdn_device.h"
#include "gdn_kernels.h"
#include "gemm_epi.h"

namespace gdn {

namespace {

constexpr int TM = 128, TN = 128, TK = 32;
constexpr int LDK = TK + 8;          // LDS row stride in bf16 elements (80 bytes)
constexpr int PLANE = TM * LDK;      // elements of one operand plane

// Registers that carry one operand's part of a k-step from global memory.
template <int MODE> struct Stage;
template <> struct Stage<OPND_BF16> { uint4 v[2]; };
template <> struct Stage<OPND_F32_SPLIT> { float4 v[4]; };
template <> struct Stage<OPND_F32_ROUND> { float4 v[4]; };

// Element type of an operand in memory (a plain trait, so that kernel
// signatures name no enumerator).
template <int MODE> struct ElemOf { using type = float; };
template <> struct ElemOf<0> { using type = bf16; };
template <int MODE> using Elem = typename ElemOf<MODE>::type;
static_assert(OPND_BF16 == 0, "ElemOf<0> is the bf16 operand");

// Thread t's pieces of a 128-row x 32-column tile: bf16 in 16-byte chunks of 8
// (row c / 4, column 8 (c % 4)), fp32 in chunks of 4 (row c / 8, column
// 4 (c % 8)), c = t + 256 i.  Rows past `rows` and columns past K read zeros
// (K is a multiple of 8).
template <int MODE>
__device__ __forceinline__ void stage_load(Stage<MODE> &st, const Elem<MODE> *X, int64_t ld, int r0, int rows,
                                           int k0, int K, int t) {
    if constexpr (MODE == OPND_BF16) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int c = t + 256 * i, r = c >> 2, kc = (c & 3) * 8;
            const bool ok = r0 + r < rows && k0 + kc < K;
            st.v[i] = ok ? *reinterpret_cast<const uint4 *>(X + (int64_t)(r0 + r) * ld + k0 + kc) : uint4{0, 0, 0, 0};
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = t + 256 * i, r = c >> 3, kc = (c & 7) * 4;
            const bool ok = r0 + r < rows && k0 + kc < K;
            st.v[i] = ok ? *reinterpret_cast<const float4 *>(X + (int64_t)(r0 + r) * ld + k0 + kc)
                         : float4{0.f, 0.f, 0.f, 0.f};
        }
    }
}

template <int MODE>
__device__ __forceinline__ void stage_store(const Stage<MODE> &st, bf16 *hi, bf16 *lo, int t) {
    if constexpr (MODE == OPND_BF16) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int c = t + 256 * i, r = c >> 2, kc = (c & 3) * 8;
            *reinterpret_cast<uint4 *>(hi + r * LDK + kc) = st.v[i];
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = t + 256 * i, r = c >> 3, kc = (c & 7) * 4;
            const float x[4] = {st.v[i].x, st.v[i].y, st.v[i].z, st.v[i].w};
            bf16 h[4], l[4];
            if constexpr (MODE == OPND_F32_SPLIT) {
                split_bf16<4>(x, h, l);
                *reinterpret_cast<bf16x4 *>(lo + r * LDK + kc) = pack4(l);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) h[j] = (bf16)x[j];
            }
            *reinterpret_cast<bf16x4 *>(hi + r * LDK + kc) = pack4(h);
        }
    }
}

template <int MA, int MB, int EPI, typename TOut>
__global__ __launch_bounds__(256) void k_gemm_nt(const Elem<MA> *__restrict__ A, int64_t lda,
                                                 const Elem<MB> *__restrict__ B, int64_t ldb, int M, int N, int K,
                                                 TOut *C, int64_t ldc, const float *__restrict__ rho,
                                                 const float *D1, int64_t ldd1, const float *D2, int64_t ldd2) {
    constexpr bool SA = MA == OPND_F32_SPLIT, SB = MB == OPND_F32_SPLIT;
    __shared__ bf16 lds[(2 + SA + SB) * PLANE];
    bf16 *Ah = lds, *Bh = lds + PLANE;
    bf16 *Al = lds + 2 * PLANE, *Bl = lds + (2 + SA) * PLANE;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int n0 = blockIdx.x * TN, m0 = blockIdx.y * TM;
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    Stage<MA> sa;
    Stage<MB> sb;
    stage_load<MA>(sa, A, lda, m0, M, 0, K, t);
    stage_load<MB>(sb, B, ldb, n0, N, 0, K, t);
    for (int k0 = 0; k0 < K; k0 += TK) {
        stage_store<MA>(sa, Ah, Al, t);
        stage_store<MB>(sb, Bh, Bl, t);
        __syncthreads();
        if (k0 + TK < K) {
            stage_load<MA>(sa, A, lda, m0, M, k0 + TK, K, t);
            stage_load<MB>(sb, B, ldb, n0, N, k0 + TK, K, t);
        }
#pragma unroll
        for (int kk = 0; kk < TK; kk += 16) {
            const int kc = kk + 8 * (lane >> 5);
            bf16x8 ah[2], bh[2], al[2], bl[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int ra = (wm + 32 * i + (lane & 31)) * LDK + kc, rb = (wn + 32 * i + (lane & 31)) * LDK + kc;
                ah[i] = *reinterpret_cast<const bf16x8 *>(Ah + ra);
                bh[i] = *reinterpret_cast<const bf16x8 *>(Bh + rb);
                if constexpr (SA) al[i] = *reinterpret_cast<const bf16x8 *>(Al + ra);
                if constexpr (SB) bl[i] = *reinterpret_cast<const bf16x8 *>(Bl + rb);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    acc[i][j] = mfma32x32x16(ah[i], bh[j], acc[i][j]);
                    if constexpr (SA) acc[i][j] = mfma32x32x16(al[i], bh[j], acc[i][j]);
                    if constexpr (SB) acc[i][j] = mfma32x32x16(ah[i], bl[j], acc[i][j]);
                }
        }
        __syncthreads();
    }

    // acc[i][j][e] is C[wm + 32 i + 8 (e / 4) + 4 (lane / 32) + e % 4][wn + 32 j + lane % 32]
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int m = m0 + wm + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
            if (m >= M) continue;
            if constexpr (EPI == EPI_SWIGLU) {
                // packed rows 64 g + r and 64 g + 32 + r are column r of W1 and W3 in group g
                const int f = (n0 + wn) / 2 + (lane & 31);
                if (f < N / 2) C[(int64_t)m * ldc + f] = from_f32<TOut>(swiglu(acc[i][0][e], acc[i][1][e]));
            } else {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int n = n0 + wn + 32 * j + (lane & 31);
                    if (n < N) epi_apply<EPI, TOut>(acc[i][j][e], m, n, C, ldc, rho, D1, ldd1, D2, ldd2);
                }
            }
        }
}

// out[c][r] = in[r][c] for r < R (converted), 0 for R <= r < Rp; 64 x 64 tiles
// through LDS so that both sides move whole rows.
template <typename TI, typename TO>
__global__ __launch_bounds__(256) void k_transpose(const TI *__restrict__ in, int64_t ldi, int R, int Cc,
                                                   TO *__restrict__ out, int64_t ldo, int Rp) {
    __shared__ float tile[64][65];
    const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64, tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int r = r0 + ty + 4 * i, c = c0 + tx;
        tile[ty + 4 * i][tx] = (r < R && c < Cc) ? to_f32(in[(int64_t)r * ldi + c]) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int c = c0 + ty + 4 * i, r = r0 + tx;
        if (c < Cc && r < Rp) out[(int64_t)c * ldo + r] = from_f32<TO>(tile[tx][ty + 4 * i]);
    }
}

// Both at once from one read of in [R][ldi]: hi/lo [R][ldh] as they are (rows
// r < R) and hiT/loT [Cc][ldo] transposed (r < Rp, zero past R).
__global__ __launch_bounds__(256) void k_split_both(const float *__restrict__ in, int64_t ldi, int R, int Cc,
                                                    bf16 *__restrict__ hi, bf16 *__restrict__ lo, int64_t ldh,
                                                    bf16 *__restrict__ hiT, bf16 *__restrict__ loT, int64_t ldo,
                                                    int Rp) {
    __shared__ float tile[64][65];
    const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64, tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int r = r0 + ty + 4 * i, c = c0 + tx;
        const bool ok = r < R && c < Cc;
        const float x[2] = {ok ? in[(int64_t)r * ldi + c] : 0.f, 0.f};
        tile[ty + 4 * i][tx] = x[0];
        if (ok) {
            bf16 h[2], l[2];
            split_bf16<2>(x, h, l);
            hi[(int64_t)r * ldh + c] = h[0];
            lo[(int64_t)r * ldh + c] = l[0];
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int c = c0 + ty + 4 * i, r = r0 + tx;
        if (c < Cc && r < Rp) {
            const float x[2] = {tile[tx][ty + 4 * i], 0.f};
            bf16 h[2], l[2];
            split_bf16<2>(x, h, l);
            hiT[(int64_t)c * ldo + r] = h[0];
            loT[(int64_t)c * ldo + r] = l[0];
        }
    }
}

template <int MA, int MB, int EPI, typename TOut>
void gemm_launch(const void *A, int64_t lda, const void *B, int64_t ldb, int M, int N, int K, void *C, int64_t ldc,
                 const float *rho, const float *D1, int64_t ldd1, const float *D2, int64_t ldd2, hipStream_t s) {
    const dim3 grid((N + TN - 1) / TN, (M + TM - 1) / TM);
    launch_kernel(k_gemm_nt<MA, MB, EPI, TOut>, grid, dim3(256), 0, s, (const Elem<MA> *)A, lda, (const Elem<MB> *)B,
                  ldb, M, N, K, (TOut *)C, ldc, rho, D1, ldd1, D2, ldd2);
}

template <int MA, int MB>
hipError_t gemm_modes(int epi, bool out_f32, const void *A, int64_t lda, const void *B, int64_t ldb, int M, int N,
                      int K, void *C, int64_t ldc, const float *rho, const float *D1, int64_t ldd1, const float *D2,
                      int64_t ldd2, hipStream_t s) {
#define GL(E)                                                                                               \
    do {                                                                                                    \
        if (out_f32) gemm_launch<MA, MB, E, float>(A, lda, B, ldb, M, N, K, C, ldc, rho, D1, ldd1, D2, ldd2, s); \
        else gemm_launch<MA, MB, E, bf16>(A, lda, B, ldb, M, N, K, C, ldc, rho, D1, ldd1, D2, ldd2, s);          \
    } while (0)
    switch (epi) {
        case EPI_STORE: GL(EPI_STORE); break;
        case EPI_ACCUM:
            if (!out_f32) return hipErrorInvalidValue;
            gemm_launch<MA, MB, EPI_ACCUM, float>(A, lda, B, ldb, M, N, K, C, ldc, rho, D1, ldd1, D2, ldd2, s);
            break;
        case EPI_RESID: GL(EPI_RESID); break;
        case EPI_ADD: GL(EPI_ADD); break;
        case EPI_ADD_RESID: GL(EPI_ADD_RESID); break;
        case EPI_GATE: GL(EPI_GATE); break;
        case EPI_SWIGLU: GL(EPI_SWIGLU); break;
        default: return hipErrorInvalidValue;
    }
#undef GL
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_nt_ex(int mode_a, int mode_b, int epi, bool out_f32, const void *A, int64_t lda, const void *B,
                             int64_t ldb, int M, int N, int K, void *C, int64_t ldc, const float *rho,
                             const float *D1, int64_t ldd1, const float *D2, int64_t ldd2, hipStream_t s) {
    if (M <= 0 || N <= 0 || K <= 0 || K % 8 || lda % 8 || ldb % 8 || (M + TM - 1) / TM > 65535)
        return hipErrorInvalidValue;
    const bool need_d1 = epi == EPI_RESID || epi == EPI_ADD || epi == EPI_ADD_RESID || epi == EPI_GATE;
    if ((need_d1 && !D1) || ((epi == EPI_RESID || epi == EPI_ADD_RESID) && !rho) || (epi == EPI_ADD_RESID && !D2))
        return hipErrorInvalidValue;
    if (epi == EPI_SWIGLU && N % 64) return hipErrorInvalidValue;
    if (mode_a == OPND_F32_SPLIT && mode_b == OPND_F32_SPLIT)
        return gemm_modes<OPND_F32_SPLIT, OPND_F32_SPLIT>(epi, out_f32, A, lda, B, ldb, M, N, K, C, ldc, rho, D1,
                                                          ldd1, D2, ldd2, s);
    if (mode_a == OPND_BF16 && mode_b == OPND_BF16)
        return gemm_modes<OPND_BF16, OPND_BF16>(epi, out_f32, A, lda, B, ldb, M, N, K, C, ldc, rho, D1, ldd1, D2,
                                                ldd2, s);
    return hipErrorInvalidValue;
}

hipError_t launch_gemm_nt(int mode_a, int mode_b, int epi, const void *A, int64_t lda, const void *B, int64_t ldb,
                          int M, int N, int K, float *C, int64_t ldc, const float *rho, const float *Dsrc,
                          int64_t ldd, hipStream_t s) {
    return launch_gemm_nt_ex(mode_a, mode_b, epi, true, A, lda, B, ldb, M, N, K, C, ldc, rho, Dsrc, ldd, nullptr, 0,
                             s);
}

hipError_t launch_split_both(const float *in, int64_t ldi, int R, int Cc, bf16 *hi, bf16 *lo, int64_t ldh, bf16 *hiT,
                             bf16 *loT, int64_t ldo, int Rp, hipStream_t s) {
    if (R < 0 || Cc <= 0 || Rp < R || (Rp + 63) / 64 > 65535) return hipErrorInvalidValue;
    if (Rp == 0) return hipSuccess;
    launch_kernel(k_split_both, dim3((Cc + 63) / 64, (Rp + 63) / 64), dim3(256), 0, s, in, ldi, R, Cc, hi, lo, ldh,
                  hiT, loT, ldo, Rp);
    return hipGetLastError();
}

hipError_t launch_transpose(bool in_f32, bool out_f32, const void *in, int64_t ldi, int R, int Cc, void *out,
                            int64_t ldo, int Rp, hipStream_t s) {
    if (R < 0 || Cc <= 0 || Rp < R || (Rp + 63) / 64 > 65535) return hipErrorInvalidValue;
    if (Rp == 0) return hipSuccess;
    const dim3 grid((Cc + 63) / 64, (Rp + 63) / 64);
    if (in_f32 && out_f32)
        launch_kernel(k_transpose<float, float>, grid, dim3(256), 0, s, (const float *)in, ldi, R, Cc, (float *)out, ldo, Rp);
    else if (in_f32)
        launch_kernel(k_transpose<float, bf16>, grid, dim3(256), 0, s, (const float *)in, ldi, R, Cc, (bf16 *)out, ldo, Rp);
    else if (!out_f32)
        launch_kernel(k_transpose<bf16, bf16>, grid, dim3(256), 0, s, (const bf16 *)in, ldi, R, Cc, (bf16 *)out, ldo, Rp);
    else
        launch_kernel(k_transpose<bf16, float>, grid, dim3(256), 0, s, (const bf16 *)in, ldi, R, Cc, (float *)out, ldo, Rp);
    return hipGetLastError();
}

}  // namespace gdn
