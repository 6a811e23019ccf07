// proj_gemm.hip -- per-loop projection X . [Wq|Wk|Wv|wa|wb] with a fused
// per-head epilogue, for the looped gated-delta-rule mixer on gfx950.
//
// LT2: Linear-Time Looped Transformers, Section 2 "LT2" paragraph: q_t, k_t
// and v_t are projections of h_t; the weights are shared by all T loops
// (Section 2, "Looped Transformer (LT)" paragraph).  The epilogue applies the
// per-head L2 normalisation of q and k and the data-dependent gates (Fig. 6
// caption: gating plus the delta rule): alpha = alpha_lo + (1 - alpha_lo)
// sigmoid(-a), beta = sigmoid(b), a = x.wa, b = x.wb.
//
// bf16 path: 128x128x64 block tiles, 4 waves of 64x64 (2x2 MFMA 32x32x16
// tiles), double-buffered LDS with a 16-byte XOR swizzle, fp32 accumulation.
// The packed weight puts each head's q|k|v rows in whole 128-row tiles, so one
// output tile always holds complete head sections for the normalisation.
// fp32 path: a plain VALU tiled GEMM with the same epilogue.
#include <type_traits>

#include "gdn_device.h"
#include "gdn_kernels.h"

namespace gdn {

namespace {

constexpr int BN = 128;
constexpr int CS_LD = BN + 4;  // row stride (floats) of the fp32 epilogue tile in LDS

// ---------------------------------------------------------------------------
// weight packing: Wpack[n][c] with n = packed output column, c = input channel
// ---------------------------------------------------------------------------
template <typename T>
__global__ void k_pack(int d, int H, int D, const T *__restrict__ Wq, const T *__restrict__ Wk,
                       const T *__restrict__ Wv, const T *__restrict__ wa,
                       const T *__restrict__ wb, T *__restrict__ Wp, int64_t total) {
    int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= total) return;
    const int64_t n = idx / d;
    const int c = (int)(idx % d);
    const int64_t qkv = (int64_t)H * 3 * D, qkvp = qkv_rows_padded(H, D);
    float val = 0.f;
    if (n < qkv) {
        const int j = (int)(n / (3 * D)), w = (int)(n % (3 * D));
        const int kind = w / D, off = w % D;
        const T *src = kind == 0 ? Wq : (kind == 1 ? Wk : Wv);
        val = to_f32(src[(int64_t)c * H * D + (int64_t)j * D + off]);
    } else if (n >= qkvp) {
        const int g = (int)(n - qkvp);
        if (g < H) val = to_f32(wa[(int64_t)c * H + g]);
        else if (g < 2 * H) val = to_f32(wb[(int64_t)c * H + (g - H)]);
    }
    Wp[idx] = from_f32<T>(val);
}

// ---------------------------------------------------------------------------
// epilogue on an fp32 tile Cs[BMx128] of output columns [n0, n0+128)
// ---------------------------------------------------------------------------
template <int D, int BM, typename TOut>
__device__ __forceinline__ void proj_epilogue(const float *Cs, float *red, int m0, int n0, int M,
                                              int H, TOut *q, TOut *k, TOut *v, float *alpha,
                                              float *beta, float alpha_lo, float eps) {
    const int t = threadIdx.x;
    const int qkv_cols = H * 3 * D;
    if (n0 >= (int)qkv_rows_padded(H, D)) {  // gate tile: columns [0,H) are a, [H,2H) are b
        for (int idx = t; idx < BM * H; idx += 256) {
            const int r = idx / H, j = idx % H, m = m0 + r;
            if (m < M) {
                const float a = Cs[r * CS_LD + j], b = Cs[r * CS_LD + H + j];
                alpha[(int64_t)m * H + j] = alpha_lo + (1.f - alpha_lo) / (1.f + expf(a));
                beta[(int64_t)m * H + j] = 1.f / (1.f + expf(-b));
            }
        }
        return;
    }
    constexpr int TPR = 256 / BM;       // threads per row
    constexpr int CPT = BN / TPR;       // columns per thread (<= D: never straddles a section)
    constexpr int PPS = D / CPT;        // threads per head section
    const int r = t % BM, part = t / BM, c0 = part * CPT;
    const float *row = Cs + r * CS_LD + c0;
    float ss = 0.f;
#pragma unroll 8
    for (int c = 0; c < CPT; ++c) ss += row[c] * row[c];
    red[part * BM + r] = ss;
    __syncthreads();
    const int n = n0 + c0;
    const int j = n / (3 * D), kind = (n % (3 * D)) / D, off = n % D;
    const int first = (part / PPS) * PPS;
    float tot = 0.f;
#pragma unroll
    for (int p = 0; p < PPS; ++p) tot += red[(first + p) * BM + r];
    const float scale = (kind == 2) ? 1.f : 1.f / sqrtf(tot + eps);
    const int m = m0 + r;
    if (m >= M || n >= qkv_cols) return;  // tail rows and zero padding columns
    TOut *dst = (kind == 0 ? q : (kind == 1 ? k : v)) + ((int64_t)m * H + j) * D + off;
    if constexpr (std::is_same<TOut, bf16>::value) {
#pragma unroll
        for (int c = 0; c < CPT; c += 8) {
            bf16x8 pk;
#pragma unroll
            for (int i = 0; i < 8; ++i) pk[i] = (bf16)(row[c + i] * scale);
            *reinterpret_cast<bf16x8 *>(dst + c) = pk;
        }
    } else {
#pragma unroll
        for (int c = 0; c < CPT; c += 4) {
            float4 pk = make_float4(row[c] * scale, row[c + 1] * scale, row[c + 2] * scale,
                                    row[c + 3] * scale);
            *reinterpret_cast<float4 *>(dst + c) = pk;
        }
    }
}

// ---------------------------------------------------------------------------
// bf16 MFMA GEMM: C[m][n] = sum_c X[m][c] * Wp[n][c]
// ---------------------------------------------------------------------------
constexpr int BM_BF = 128, BK_BF = 64;
constexpr int TILE_ELEMS = BM_BF * BK_BF;  // bf16 elements per operand tile (both are 128 x 64)

// 16-byte chunk `ch` (0..7) of row `r` of a 128x64 bf16 tile, XOR-swizzled by row.
__device__ __forceinline__ int swz(int r, int ch) { return r * BK_BF + ((ch ^ (r & 7)) << 3); }

template <int D>
__global__ __launch_bounds__(256) void k_proj_bf16(const bf16 *__restrict__ x,
                                                   const bf16 *__restrict__ Wp, int M, int K, int H,
                                                   bf16 *q, bf16 *k, bf16 *v, float *alpha,
                                                   float *beta, float alpha_lo, float eps) {
    constexpr int LDS_MAIN = 2 * 2 * TILE_ELEMS * 2;      // A,B double-buffered, bytes
    constexpr int LDS_EPI = BM_BF * CS_LD * 4 + 2 * BM_BF * 4;
    constexpr int LDS_BYTES = LDS_MAIN > LDS_EPI ? LDS_MAIN : LDS_EPI;
    __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];
    bf16 *As = reinterpret_cast<bf16 *>(smem);
    bf16 *Bs = As + 2 * TILE_ELEMS;

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM_BF;
    const int wm = wave >> 1, wn = wave & 1;

    // global -> register staging: each thread moves 4 chunks of A and 4 of B per k-block
    uint4 ra[4], rb[4];
    auto gload = [&](int kb) {
        const int k0 = kb * BK_BF;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = t + 256 * i, r = c >> 3, ch = c & 7;
            const int m = m0 + r;
            if (m < M) ra[i] = *reinterpret_cast<const uint4 *>(x + (int64_t)m * K + k0 + ch * 8);
            else ra[i] = make_uint4(0, 0, 0, 0);
            rb[i] = *reinterpret_cast<const uint4 *>(Wp + (int64_t)(n0 + r) * K + k0 + ch * 8);
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = t + 256 * i, r = c >> 3, ch = c & 7;
            *reinterpret_cast<uint4 *>(As + buf * TILE_ELEMS + swz(r, ch)) = ra[i];
            *reinterpret_cast<uint4 *>(Bs + buf * TILE_ELEMS + swz(r, ch)) = rb[i];
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int nkb = K / BK_BF;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kb = 0; kb < nkb; ++kb) {
        const int buf = kb & 1;
        if (kb + 1 < nkb) gload(kb + 1);
        const bf16 *Ab = As + buf * TILE_ELEMS;
        const bf16 *Bb = Bs + buf * TILE_ELEMS;
#pragma unroll
        for (int s = 0; s < BK_BF / 16; ++s) {
            const int ch = 2 * s + (lane >> 5);
            bf16x8 af[2], bfr[2];
#pragma unroll
            for (int tm = 0; tm < 2; ++tm) {
                const int r = wm * 64 + tm * 32 + (lane & 31);
                af[tm] = *reinterpret_cast<const bf16x8 *>(Ab + swz(r, ch));
            }
#pragma unroll
            for (int tn = 0; tn < 2; ++tn) {
                const int r = wn * 64 + tn * 32 + (lane & 31);
                bfr[tn] = *reinterpret_cast<const bf16x8 *>(Bb + swz(r, ch));
            }
#pragma unroll
            for (int tm = 0; tm < 2; ++tm)
#pragma unroll
                for (int tn = 0; tn < 2; ++tn) acc[tm][tn] = mfma32x32x16(af[tm], bfr[tn], acc[tm][tn]);
        }
        if (kb + 1 < nkb) {
            sstore(buf ^ 1);
        }
        __syncthreads();
    }

    // accumulators -> fp32 tile in LDS (reuses the operand buffers)
    float *Cs = reinterpret_cast<float *>(smem);
    float *red = Cs + BM_BF * CS_LD;
#pragma unroll
    for (int tm = 0; tm < 2; ++tm)
#pragma unroll
        for (int tn = 0; tn < 2; ++tn)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int r = wm * 64 + tm * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                const int c = wn * 64 + tn * 32 + (lane & 31);
                Cs[r * CS_LD + c] = acc[tm][tn][e];
            }
    __syncthreads();
    proj_epilogue<D, BM_BF, bf16>(Cs, red, m0, n0, M, H, q, k, v, alpha, beta, alpha_lo, eps);
}

// ---------------------------------------------------------------------------
// fp32 VALU GEMM (small fp32 workloads), 64x128x16 tiles
// ---------------------------------------------------------------------------
constexpr int BM_F = 64, BK_F = 16;

template <int D>
__global__ __launch_bounds__(256) void k_proj_f32(const float *__restrict__ x,
                                                  const float *__restrict__ Wp, int M, int K, int H,
                                                  float *q, float *k, float *v, float *alpha,
                                                  float *beta, float alpha_lo, float eps) {
    constexpr int LDS_MAIN = (BM_F + BN) * (BK_F + 1) * 4;
    constexpr int LDS_EPI = BM_F * CS_LD * 4 + 4 * BM_F * 4;
    constexpr int LDS_BYTES = LDS_MAIN > LDS_EPI ? LDS_MAIN : LDS_EPI;
    __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];
    float *As = reinterpret_cast<float *>(smem);      // [BM_F][BK_F+1]
    float *Bs = As + BM_F * (BK_F + 1);                // [BN][BK_F+1]
    const int t = threadIdx.x;
    const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM_F;
    const int tr = t / 16, tc = t % 16;  // thread owns rows tr*4..+4, cols tc + 16*j (j<8)
    float acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;
    for (int k0 = 0; k0 < K; k0 += BK_F) {
        for (int idx = t; idx < BM_F * BK_F; idx += 256) {
            const int r = idx / BK_F, c = idx % BK_F, m = m0 + r;
            As[r * (BK_F + 1) + c] = (m < M && k0 + c < K) ? x[(int64_t)m * K + k0 + c] : 0.f;
        }
        for (int idx = t; idx < BN * BK_F; idx += 256) {
            const int r = idx / BK_F, c = idx % BK_F;
            Bs[r * (BK_F + 1) + c] = (k0 + c < K) ? Wp[(int64_t)(n0 + r) * K + k0 + c] : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < BK_F; ++kk) {
            float a[4], b[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[(tr * 4 + i) * (BK_F + 1) + kk];
#pragma unroll
            for (int j = 0; j < 8; ++j) b[j] = Bs[(tc + 16 * j) * (BK_F + 1) + kk];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
    float *Cs = reinterpret_cast<float *>(smem);
    float *red = Cs + BM_F * CS_LD;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) Cs[(tr * 4 + i) * CS_LD + tc + 16 * j] = acc[i][j];
    __syncthreads();
    proj_epilogue<D, BM_F, float>(Cs, red, m0, n0, M, H, q, k, v, alpha, beta, alpha_lo, eps);
}

}  // namespace

hipError_t launch_pack_weights(bool f32, int d, int H, int D, const void *Wq, const void *Wk,
                               const void *Wv, const void *wa, const void *wb, void *Wpack,
                               hipStream_t s) {
    const int64_t total = packed_rows(H, D) * d;
    const int threads = 256;
    const int64_t blocks = (total + threads - 1) / threads;
    if (f32)
        hipLaunchKernelGGL(k_pack<float>, dim3((unsigned)blocks), dim3(threads), 0, s, d, H, D,
                           (const float *)Wq, (const float *)Wk, (const float *)Wv,
                           (const float *)wa, (const float *)wb, (float *)Wpack, total);
    else
        hipLaunchKernelGGL(k_pack<bf16>, dim3((unsigned)blocks), dim3(threads), 0, s, d, H, D,
                           (const bf16 *)Wq, (const bf16 *)Wk, (const bf16 *)Wv, (const bf16 *)wa,
                           (const bf16 *)wb, (bf16 *)Wpack, total);
    return hipGetLastError();
}

hipError_t launch_project(bool f32, int M, int d, int H, int D, const void *x, const void *Wpack,
                          void *q, void *k, void *v, float *alpha, float *beta, float alpha_lo,
                          float eps, hipStream_t s) {
    const int ntiles = (int)(packed_rows(H, D) / BN);
    if (f32) {
        dim3 grid(ntiles, (M + BM_F - 1) / BM_F);
        if (D == 128)
            hipLaunchKernelGGL(k_proj_f32<128>, grid, dim3(256), 0, s, (const float *)x,
                               (const float *)Wpack, M, d, H, (float *)q, (float *)k, (float *)v,
                               alpha, beta, alpha_lo, eps);
        else
            hipLaunchKernelGGL(k_proj_f32<64>, grid, dim3(256), 0, s, (const float *)x,
                               (const float *)Wpack, M, d, H, (float *)q, (float *)k, (float *)v,
                               alpha, beta, alpha_lo, eps);
    } else {
        dim3 grid(ntiles, (M + BM_BF - 1) / BM_BF);
        if (D == 128)
            hipLaunchKernelGGL(k_proj_bf16<128>, grid, dim3(256), 0, s, (const bf16 *)x,
                               (const bf16 *)Wpack, M, d, H, (bf16 *)q, (bf16 *)k, (bf16 *)v,
                               alpha, beta, alpha_lo, eps);
        else
            hipLaunchKernelGGL(k_proj_bf16<64>, grid, dim3(256), 0, s, (const bf16 *)x,
                               (const bf16 *)Wpack, M, d, H, (bf16 *)q, (bf16 *)k, (bf16 *)v,
                               alpha, beta, alpha_lo, eps);
    }
    return hipGetLastError();
}

}  // namespace gdn
