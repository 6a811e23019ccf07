// gemm_tile.hip -- bf16 MFMA products with fused epilogues on gfx950 for the
// token-by-feature GEMMs around the mixer: the products of the backward
// through the loops (LT2: Linear-Time Looped Transformers, Appendix C, bf16
// mixed-precision training) and those of the LT2 block (Section 2, "LT2"
// paragraph: the gated mixer output's projection and the FFN of each block).
//
// C[m][n] = epi(sum_k A[m][k] B[n][k]), A [M][lda] and B [N][ldb] bf16 with
// K-contiguous rows.  An fp32 operand enters as two bf16 planes (hi + lo,
// about 16 significant bits): the k-loop then runs over passes of the planes
// (hi.hi, lo.hi and/or hi.lo), all accumulated in fp32.
//
// Tile 384 (m) x 256 (n) x 64 (k), eight waves of 96 x 128 (3 x 4 MFMA
// 32x32x16 tiles, 192 fp32 accumulators per lane; each k-step reads 7
// fragments for 12 MFMAs).  Operands go global -> LDS with direct loads into
// two 80 KiB stages (the whole LDS): block i+1 lands while block i is
// multiplied, one wait and one barrier per 64 channels.  The LDS tile rows
// are XOR-swizzled in 16-byte chunks by row / 2 so that the fragment reads of
// 16 consecutive rows hit distinct bank groups.  A lane holds, for one
// feature column, 16 token rows per MFMA tile, so every epilogue store of a
// row of 32 features is one contiguous 128-byte (fp32) run.
#include "gdn_device.h"
#include "gdn_kernels.h"
#include "gemm_epi.h"

namespace gdn {

namespace {

constexpr int GM = 384, GN = 256, GK = 64;
constexpr int GSA = GM * GK, GSB = GN * GK, GSTAGE = GSA + GSB;   // bf16 elements
constexpr int G_LDS = 2 * GSTAGE * 2;                             // bytes, two stages
constexpr int GLOADS = (GSA + GSB) / 8 / 64 / 8;                  // direct loads per wave per block (10)
constexpr int GLOADS_A = GSA / 8 / 64 / 8;                        // of which A's (6)

__device__ __forceinline__ int gswz(int r, int ch) { return r * GK + ((ch ^ ((r >> 1) & 7)) << 3); }

// Per-lane byte offsets of the wave's direct loads, relative to the tile's
// first row: wave w's load i covers LDS chunks [(8 i' + w) 64, +64) of its
// operand tile (i' = i for A, i - 6 for B); LDS chunk p holds row p / 8 and
// logical chunk (p % 8) ^ ((row / 2) % 8).  Rows past the operand's end
// re-read its last row (their results are never stored).
struct TileSrc {
    unsigned off[GLOADS];
};
__device__ __forceinline__ TileSrc tile_src(int lane, int wave, int rows_a, int rows_b, int64_t lda, int64_t ldb) {
    TileSrc s;
#pragma unroll
    for (int i = 0; i < GLOADS; ++i) {
        const bool isa = i < GLOADS_A;
        const int p = (8 * (isa ? i : i - GLOADS_A) + wave) * 64 + lane;
        const int r = p >> 3, ch = (p & 7) ^ ((r >> 1) & 7);
        const int row = min(r, (isa ? rows_a : rows_b) - 1);
        s.off[i] = (unsigned)(((unsigned)row * (unsigned)(isa ? lda : ldb) + ch * 8) * 2u);
    }
    return s;
}

// The planes of pass p (p-th group of K / 64 blocks): 0 = (A hi, B hi),
// then (A lo, B hi) when A is split, then (A hi, B lo) when B is split.
struct Planes {
    const bf16 *a, *a2, *b, *b2;   // hi, lo planes (lo null when not split), tile origin applied
};
__device__ __forceinline__ void block_bases(const Planes &P, int pass, int kb, const bf16 *&ab, const bf16 *&bb) {
    const bool alo = pass == 1 && P.a2, blo = pass >= 1 && !(pass == 1 && P.a2);
    ab = (alo ? P.a2 : P.a) + kb * GK;
    bb = (blo ? P.b2 : P.b) + kb * GK;
}

template <int EPI, typename TOut>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_gemm_tile(
    const bf16 *__restrict__ A, const bf16 *__restrict__ A2, int64_t lda, const bf16 *__restrict__ B,
    const bf16 *__restrict__ B2, int64_t ldb, int M, int N, int K, int m_tiles, int n_tiles, int ksplit,
    int64_t cstride, TOut *__restrict__ C, int64_t ldc, const float *__restrict__ rho, const float *__restrict__ D1,
    int64_t ldd1, const float *__restrict__ D2, int64_t ldd2) {
    __shared__ __attribute__((aligned(16))) char smem[G_LDS];
    bf16 *stages = reinterpret_cast<bf16 *>(smem);
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = wave >> 1, wn = wave & 1;   // 4 x 2 waves of 96 tokens x 128 features
    // Workgroup ids go to the 8 XCDs round-robin; XCD x takes the tiles
    // x, x + 8, ... of the token-tile-major order, so one XCD's tiles share
    // token tiles (A rows) in its L2 as the features advance.
    // With ksplit > 1 the k-blocks (over all passes) are divided into ksplit
    // contiguous ranges; range z's partial sums go to C + z cstride.
    const int ntot = m_tiles * n_tiles;
    const int split = blockIdx.x / ntot, id = blockIdx.x % ntot;
    C += (int64_t)split * cstride;
    const int tix = (ntot % 8 == 0) ? (id % 8) * (ntot / 8) + id / 8 : id;
    const int m_tile = tix / n_tiles, n_tile = tix % n_tiles;
    const int m0 = m_tile * GM, n0 = n_tile * GN;

    const TileSrc src = tile_src(lane, wave, min(GM, M - m0), min(GN, N - n0), lda, ldb);
    Planes P{A + (int64_t)m0 * lda, A2 ? A2 + (int64_t)m0 * lda : nullptr, B + (int64_t)n0 * ldb,
             B2 ? B2 + (int64_t)n0 * ldb : nullptr};
    const int nkb = K / GK, npass = 1 + (A2 != nullptr) + (B2 != nullptr), nall = nkb * npass;
    const int blk0 = (int)((int64_t)nall * split / ksplit), nblk = (int)((int64_t)nall * (split + 1) / ksplit) - blk0;
    auto issue = [&](int blk, bf16 *stage) __attribute__((always_inline)) {
        const int b = blk0 + min(blk, nblk - 1);
        const bf16 *ab, *bb;
        block_bases(P, b / nkb, b % nkb, ab, bb);
        return [=](int i) __attribute__((always_inline)) {
            if (i < GLOADS_A) dma16_async_s(ab, src.off[i], stage + (8 * i + wave) * 64 * 8);
            else dma16_async_s(bb, src.off[i], stage + GSA + (8 * (i - GLOADS_A) + wave) * 64 * 8);
        };
    };

    {
        auto l0 = issue(0, stages);
#pragma unroll
        for (int i = 0; i < GLOADS; ++i) l0(i);
        auto l1 = issue(1, stages + GSTAGE);
#pragma unroll
        for (int i = 0; i < GLOADS; ++i) l1(i);
    }
    wait_vmcnt<GLOADS>();   // block 0 has landed; block 1 may be in flight

    f32x16 acc[3][4];
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    struct Fr {
        bf16x8 a[3], b[4];
    };
    auto read = [&](Fr &F, const bf16 *stage, int ks) __attribute__((always_inline)) {
        const int ch = 2 * ks + (lane >> 5);
#pragma unroll
        for (int i = 0; i < 3; ++i)
            F.a[i] = *reinterpret_cast<const bf16x8 *>(stage + gswz(wm * 96 + i * 32 + (lane & 31), ch));
#pragma unroll
        for (int j = 0; j < 4; ++j)
            F.b[j] = *reinterpret_cast<const bf16x8 *>(stage + GSA + gswz(wn * 128 + j * 32 + (lane & 31), ch));
    };
    // step it: wait for block it's loads, barrier (every wave is done with
    // block it - 1, whose stage takes block it + 1), four k-steps of 12 MFMAs
    // with block it + 1's ten direct loads spread between them
    auto kstep = [&](auto load_c, int it) __attribute__((always_inline)) {
        constexpr bool LOAD = decltype(load_c)::value;
        if constexpr (LOAD) wait_vmcnt<0>();
        lds_barrier();
        const bf16 *cur = stages + (it & 1) * GSTAGE;
        auto ld = issue(it + 1, stages + ((it + 1) & 1) * GSTAGE);
        Fr fr[2];
        read(fr[0], cur, 0);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (s < 3) read(fr[(s + 1) & 1], cur, s + 1);
#pragma unroll
            for (int j = 0; j < 12; ++j) {
                const int ti = j / 4, tj = j % 4, i = 12 * s + j;
                acc[ti][tj] = mfma32x32x16(fr[s & 1].a[ti], fr[s & 1].b[tj], acc[ti][tj]);
                if (LOAD && i % 4 == 1 && i / 4 < GLOADS) ld(i / 4);
            }
        }
    };
    kstep(std::false_type(), 0);
    for (int it = 1; it < nblk; ++it) kstep(std::true_type(), it);
    wait_vmcnt<0>();   // the repeated loads issued past the last block

    // acc[ti][tj][e]: token m0 + 96 wm + 32 ti + 8 (e / 4) + 4 (lane / 32) + e % 4,
    //                 feature n0 + 128 wn + 32 tj + lane % 32
    // Per 32 x 32 tile, the epilogue's operands are all loaded before any of
    // its results is stored, so the loads go out back to back.
    const int nb = n0 + wn * 128 + (lane & 31);
    constexpr bool NEED1 = EPI == EPI_RESID || EPI == EPI_ADD || EPI == EPI_ADD_RESID || EPI == EPI_GATE ||
                           EPI == EPI_ACCUM;
    constexpr bool NEED2 = EPI == EPI_ADD_RESID;
#pragma unroll
    for (int ti = 0; ti < 3; ++ti) {
        const int mb = m0 + wm * 96 + ti * 32 + 4 * (lane >> 5);
        if constexpr (EPI == EPI_SWIGLU) {
            // features 64 g + r and 64 g + 32 + r of the packed rows are column r of W1 and W3 in group g:
            // tiles (0, 1) and (2, 3) of the wave
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int m = mb + 8 * (e >> 2) + (e & 3);
                if (m >= M) continue;
#pragma unroll
                for (int pr = 0; pr < 2; ++pr) {
                    const int f = (n0 + wn * 128 + 64 * pr) / 2 + (lane & 31);
                    if (f < N / 2)
                        C[(int64_t)m * ldc + f] = from_f32<TOut>(swiglu(acc[ti][2 * pr][e], acc[ti][2 * pr + 1][e]));
                }
            }
        } else {
#pragma unroll
            for (int tj = 0; tj < 4; ++tj) {
                const int n = nb + 32 * tj;
                if (n >= N) continue;
                float d1[16], d2[16];
                if constexpr (NEED1) {
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int m = mb + 8 * (e >> 2) + (e & 3);
                        const bool ok = m < M;
                        if constexpr (EPI == EPI_ACCUM) d1[e] = ok ? to_f32(C[(int64_t)m * ldc + n]) : 0.f;
                        else d1[e] = ok ? D1[(int64_t)m * ldd1 + n] : 0.f;
                        if constexpr (NEED2) d2[e] = ok ? D2[(int64_t)m * ldd2 + n] : 0.f;
                    }
                }
                const float r = (EPI == EPI_RESID || EPI == EPI_ADD_RESID) ? rho[n] : 0.f;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int m = mb + 8 * (e >> 2) + (e & 3);
                    if (m >= M) continue;
                    const float x = acc[ti][tj][e];
                    float y;
                    if constexpr (EPI == EPI_STORE) y = x;
                    else if constexpr (EPI == EPI_ACCUM) y = d1[e] + x;
                    else if constexpr (EPI == EPI_RESID) y = x + r * d1[e];
                    else if constexpr (EPI == EPI_ADD) y = x + d1[e];
                    else if constexpr (EPI == EPI_ADD_RESID) y = x + d1[e] + r * d2[e];
                    else y = d1[e] / (1.f + expf(-x));   // EPI_GATE
                    C[(int64_t)m * ldc + n] = from_f32<TOut>(y);
                }
            }
        }
    }
}

template <int EPI, typename TOut>
void tile_launch(const bf16 *A, const bf16 *A2, int64_t lda, const bf16 *B, const bf16 *B2, int64_t ldb, int M,
                 int N, int K, int ksplit, int64_t cstride, TOut *C, int64_t ldc, const float *rho, const float *D1,
                 int64_t ldd1, const float *D2, int64_t ldd2, hipStream_t s) {
    const int mt = (M + GM - 1) / GM, nt = (N + GN - 1) / GN;
    launch_kernel(k_gemm_tile<EPI, TOut>, dim3(mt * nt * ksplit), dim3(512), 0, s, A, A2, lda, B, B2, ldb, M, N, K,
                  mt, nt, ksplit, cstride, C, ldc, rho, D1, ldd1, D2, ldd2);
}

}  // namespace

hipError_t launch_gemm_tile(int epi, bool out_f32, const bf16 *A, const bf16 *A2, int64_t lda, const bf16 *B,
                            const bf16 *B2, int64_t ldb, int M, int N, int K, void *C, int64_t ldc, const float *rho,
                            const float *D1, int64_t ldd1, const float *D2, int64_t ldd2, hipStream_t s, int ksplit,
                            int64_t cstride) {
    if (M <= 0 || N <= 0 || K <= 0 || K % GK || lda % 8 || ldb % 8 || lda < K || ldb < K) return hipErrorInvalidValue;
    if ((int64_t)GM * lda * 2 >= (int64_t(1) << 32) || (int64_t)GN * ldb * 2 >= (int64_t(1) << 32))
        return hipErrorInvalidValue;   // per-tile byte offsets are 32-bit
    const int npass = 1 + (A2 != nullptr) + (B2 != nullptr);
    if (ksplit < 1 || ksplit > (K / GK) * npass || (ksplit > 1 && epi != EPI_STORE && epi != EPI_ACCUM))
        return hipErrorInvalidValue;   // a split sum takes no epilogue but store or accumulate
    const int64_t tiles = (int64_t)((M + GM - 1) / GM) * ((N + GN - 1) / GN) * ksplit;
    if (tiles > INT32_MAX) return hipErrorInvalidValue;
    const bool need_d1 = epi == EPI_RESID || epi == EPI_ADD || epi == EPI_ADD_RESID || epi == EPI_GATE;
    if ((need_d1 && !D1) || ((epi == EPI_RESID || epi == EPI_ADD_RESID) && !rho) || (epi == EPI_ADD_RESID && !D2))
        return hipErrorInvalidValue;
    if (epi == EPI_SWIGLU && N % 64) return hipErrorInvalidValue;
#define TL(E)                                                                                                  \
    do {                                                                                                       \
        if (out_f32) tile_launch<E, float>(A, A2, lda, B, B2, ldb, M, N, K, ksplit, cstride, (float *)C, ldc, rho, D1, ldd1, D2, ldd2, s); \
        else tile_launch<E, bf16>(A, A2, lda, B, B2, ldb, M, N, K, ksplit, cstride, (bf16 *)C, ldc, rho, D1, ldd1, D2, ldd2, s);           \
    } while (0)
    switch (epi) {
        case EPI_STORE: TL(EPI_STORE); break;
        case EPI_ACCUM:
            if (!out_f32) return hipErrorInvalidValue;
            tile_launch<EPI_ACCUM, float>(A, A2, lda, B, B2, ldb, M, N, K, ksplit, cstride, (float *)C, ldc, rho, D1,
                                          ldd1, D2, ldd2, s);
            break;
        case EPI_RESID: TL(EPI_RESID); break;
        case EPI_ADD: TL(EPI_ADD); break;
        case EPI_ADD_RESID: TL(EPI_ADD_RESID); break;
        case EPI_GATE: TL(EPI_GATE); break;
        case EPI_SWIGLU: TL(EPI_SWIGLU); break;
        default: return hipErrorInvalidValue;
    }
#undef TL
    return hipGetLastError();
}

}  // namespace gdn
