// scan_chunk.hip -- chunkwise-parallel prefill of the gated delta rule on gfx950.
//
// Recurrence (LT2: Linear-Time Looped Transformers, Section 2 "LT2"
// paragraph and Appendix B.1; the update is the gated delta rule of the GDN
// reference the pages cite), per (sequence, head):
//     S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,  o_t = S_t^T q_t.
// With u_t = beta_t (v_t - alpha_t S_{t-1}^T k_t) this is S_t = alpha_t S_{t-1} + k_t u_t^T.
// Over one chunk of C = 64 tokens with start state S (rows r, i index tokens of
// the chunk; gamma_r = prod_{m<=r} alpha_m; Gam_ri = prod_{i<m<=r} alpha_m):
//     N   = diag(beta) strict_lower(Gam (.) K K^T),   T = (I + N)^{-1}
//     P   = lower_incl(Gam (.) Q K^T)
//     E   = V - diag(gamma) K S                        (chunk-local residual)
//     U   = T diag(beta) E
//     O   = diag(gamma) Q S + P U      = diag(gamma) Q S + M E,  M = P T diag(beta)
//     S'  = gamma_C S + K^T diag(gamma_C/gamma) U = gamma_C S + W E,
//           W = K^T diag(gamma_C/gamma) T diag(beta)   [D x C]
// (the UT/WY rewrite of the delta rule cited by the pages as "a fused
// chunkwise kernel"; every decay ratio is formed as a direct product of the
// alphas in between, so it cannot underflow into 0/0).
//
// k_scan_prep: fully parallel over (b, h, chunk): Gam, K K^T and Q K^T on bf16
//   MFMA, the unit-lower-triangular inverse T in fp32 (16x16 diagonal blocks by
//   forward substitution, then block rows), and W, M (each as a bf16 hi plane
//   followed by a bf16 lo plane, hi + lo ~= the fp32 value) and gamma to the
//   workspace.
// k_scan_carry: one workgroup per (b, h, 16 columns of S); the columns of S
//   never mix, so column slices are independent scans.  Each of the 4 waves
//   keeps D/4 rows of the fp32 state slice in registers, forms its share of
//   K.S and Q.S, reduce-scatters them by token tile through LDS, all-gathers
//   the E tiles, then updates its rows (S' = gamma_C S + W E) and writes O for
//   its 16 tokens.  The products use split-bf16 operands (x = hi + lo, ~16
//   significant bits) with fp32 accumulation; operands that are exact bf16
//   inputs are not split.  Chunk operands are loaded a chunk ahead of use.
#include <type_traits>

#include "gdn_device.h"
#include "gdn_kernels.h"

namespace gdn {

namespace {

constexpr int C = 64;       // tokens per chunk
constexpr int LDP = C + 1;  // padded row stride of the 64x64 fp32 LDS matrices

template <typename T> struct In;
template <> struct In<float> { static constexpr bool f32 = true; };
template <> struct In<bf16> { static constexpr bool f32 = false; };

// A chunk tile of K or Q in LDS: 64 token rows of D elements, no padding, the
// 16-byte chunks of row r permuted by an XOR with a row-dependent key, so that
// 16 consecutive rows reading the same logical chunk hit distinct bank groups.
// It arrives by direct loads of whole 1 KiB runs (tile_load).
template <int D, typename TIn> struct KTile {
    static constexpr int ES = (int)sizeof(TIn);
    static constexpr int ROWB = D * ES;                  // bytes of a token row
    static constexpr int NCH = ROWB / 16;                // 16-byte chunks per row
    static constexpr int SH = (ES == 4 && D == 128) ? 1 : 0;
    static constexpr int BYTES = C * ROWB;
    static constexpr int INS = BYTES / 1024;             // direct-load instructions per tile
    // physical 16-byte chunk of logical chunk c in row r
    __device__ static int phys(int r, int c) { return c ^ ((r << SH) & (NCH - 1)); }
};

// Direct loads of the tile of `src` ([tokens][H][D]) for head h and the 64
// tokens from row tok0 (rows past `last` re-read row `last`): instructions
// n = n0, n0 + step, ... of the tile.
template <int D, typename TIn>
__device__ __forceinline__ void tile_load(unsigned char *tile, const TIn *src, int64_t tok0, int last, int H, int h,
                                          int lane, int n0, int step) {
    using T = KTile<D, TIn>;
    constexpr int EPC = 16 / T::ES;
    for (int n = n0; n < T::INS; n += step) {
        const int p = n * 64 + lane;
        const int r = p / T::NCH, c = T::phys(r, p % T::NCH);
        dma16_async(src + ((tok0 + min(r, last)) * H + h) * D + c * EPC, tile + n * 1024);
    }
}

// 8 consecutive elements [k0, k0 + 8) of row r of a tile (k0 a multiple of 8), as floats
template <int D, typename TIn>
__device__ __forceinline__ void tile_frag8(const unsigned char *tile, int r, int k0, float (&f)[8]) {
    using T = KTile<D, TIn>;
    const unsigned char *row = tile + r * T::ROWB;
    if constexpr (T::ES == 2) {
        const bf16x8 v = *reinterpret_cast<const bf16x8 *>(row + T::phys(r, k0 / 8) * 16);
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = (float)v[i];
    } else {
        const float4 a = *reinterpret_cast<const float4 *>(row + T::phys(r, k0 / 4) * 16);
        const float4 b = *reinterpret_cast<const float4 *>(row + T::phys(r, k0 / 4 + 1) * 16);
        f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
        f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
    }
}
// the same 8 elements as raw bf16 (bf16 tiles)
template <int D>
__device__ __forceinline__ bf16x8 tile_bf8(const unsigned char *tile, int r, int k0) {
    using T = KTile<D, bf16>;
    return *reinterpret_cast<const bf16x8 *>(tile + r * T::ROWB + T::phys(r, k0 / 8) * 16);
}
// element (r, i) of a tile, as a float
template <int D, typename TIn>
__device__ __forceinline__ float tile_elem(const unsigned char *tile, int r, int i) {
    using T = KTile<D, TIn>;
    constexpr int EPC = 16 / T::ES;
    const TIn *e = reinterpret_cast<const TIn *>(tile + r * T::ROWB + T::phys(r, i / EPC) * 16) + i % EPC;
    return to_f32(*e);
}

// Fragment order of the per-chunk [R x 64] matrices W (R = D rows of S) and M
// (R = 64 output tokens) that the prep kernel writes and the carry reads.  Rows are
// split over the 4 waves (RW = R/4 each, NT = RW/16 tiles of 16); row
// RW w + 4 NT g + 4 tt + j (j < 4) is output row 4 g + j of the wave's tile tt
// (for M, and for W with D = 64, this is simply row 16 tt + 4 g + j).  The 64
// tokens form two 32-token k-steps s; lane l = lr + 16 lg of the wave holds
// output row lr and, in slot jj of its 8-element fragment, token
// 32 s + 4 lg + jj (jj < 4) or 32 s + 16 + 4 lg + (jj - 4) (jj >= 4).  Layout:
// [wave][tt][s][part: hi, lo][lane][8] bf16, so each wave reads its fragments
// with fully coalesced 16-byte loads.  The lo part sits 8 * 64 elements after
// the hi part.

// ---------------------------------------------------------------------------
// prep
// ---------------------------------------------------------------------------
// One workgroup (4 waves) per (b, h, chunk).  Decay products come from the
// chunk's log-cumsum lg_r = sum_{m<=r} log alpha_m, kept in fp64 so that
// Gam_ri = exp(lg_r - lg_i) loses nothing to cancellation (alpha is clamped
// above 0; a true zero gate gives a product below 1e-37 instead of 0).
// K K^T and K Q^T run on MFMA.  T = (I + N)^{-1} is formed from the 16x16
// diagonal blocks (forward substitution in registers) merged 16 -> 32 -> 64
// with the block rule [A 0; B C]^{-1} = [A^{-1} 0; -C^{-1} B A^{-1}  C^{-1}]
// (split-bf16 MFMA products).  W and M are computed transposed on MFMA so that
// each lane holds 8 consecutive fragment slots of the carry's layout and
// stores them with one 16-byte write per part.

// c += a.b on 16x16x32 bf16 MFMA, exact when both are bf16 values (EXACT),
// else with both operands split into bf16 hi + lo (3 passes).
template <bool EXACT>
__device__ __forceinline__ f32x4 mma8(const float (&a)[8], const float (&b)[8], f32x4 c) {
    __bf16 ah[8], al[8], bh[8], bl[8];
    split_bf16(a, ah, al);
    split_bf16(b, bh, bl);
    c = mfma16x16x32(pack8(ah), pack8(bh), c);
    if constexpr (!EXACT) {
        c = mfma16x16x32(pack8(ah), pack8(bl), c);
        c = mfma16x16x32(pack8(al), pack8(bh), c);
    }
    return c;
}
// c += a.b on 16x16x16 (k = 4 (l/16) + i), both fp32, split (3 passes)
__device__ __forceinline__ f32x4 mma4s(const float (&a)[4], const float (&b)[4], f32x4 c) {
    __bf16 ah[4], al[4], bh[4], bl[4];
    split_bf16(a, ah, al);
    split_bf16(b, bh, bl);
    c = mfma16x16x16(pack4(ah), pack4(bh), c);
    c = mfma16x16x16(pack4(ah), pack4(bl), c);
    return mfma16x16x16(pack4(al), pack4(bh), c);
}

// With BWO it also writes the chunk matrices that the backward pass takes (A,
// P, T, M^T fp32 row-major, the log-cumsum, gamma and c; A and P zero in the
// rows, M^T in the columns of tokens past the end; W^T as bf16 hi and lo
// planes; K^T and Q^T from the LDS tiles, zero past the end).
template <int D, typename TIn, bool GP, bool BWO>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void k_scan_prep(const TIn *__restrict__ q,
                                                   const TIn *__restrict__ k,
                                                   const float *__restrict__ alpha,
                                                   const float *__restrict__ beta,
                                                   const float *__restrict__ zp, int P, int Mtot,
                                                   float *__restrict__ alpha_out,
                                                   float *__restrict__ beta_out,
                                                   float alpha_lo, int L, int H,
                                                   int Nc, float *__restrict__ wsW,
                                                   float *__restrict__ wsM,
                                                   float *__restrict__ wsg, PrepBwd bo) {
    constexpr bool F32 = In<TIn>::f32;
    constexpr int LT = C + 4;                // row stride (floats) of the 64x64 N and T tiles
    constexpr int KS = D / 32;               // k-steps of the D contractions
    constexpr int RW = D / 4, NT = RW / 16;  // W rows per wave, 16-row tiles per wave
    using KT = KTile<D, TIn>;
    // LDS (35 KB with bf16 dk = 128, so four workgroups fit on a CU): one array
    // holds the Q tile until phase 2 has read it, then N, and T is formed in
    // place over N (each block of N is read, by the wave that overwrites it or
    // before a barrier, before T's block replaces it); the phase-5 exchange
    // lives in the strictly upper 16x16 blocks, which are zeroed after it.
    constexpr int TQ_FLOATS = C * LT > KT::BYTES / 4 ? C * LT : KT::BYTES / 4;
    __shared__ __attribute__((aligned(16))) unsigned char Ks[KT::BYTES];
    __shared__ __attribute__((aligned(16))) float TQs[TQ_FLOATS];
    unsigned char *const Qs = reinterpret_cast<unsigned char *>(TQs);
    float *const Ns = TQs;
    float *const Ts = TQs;
    // exchange slot of (wave w, lane): upper block (0,1), (0,2), (0,3) or (1,2) of N
    auto ys_slot = [&](int w, int ln) {
        const int bi = w < 3 ? 0 : 1, bj = w < 3 ? w + 1 : 2;
        return reinterpret_cast<f32x4 *>(Ns + (16 * bi + (ln >> 2)) * LT + 16 * bj + 4 * (ln & 3));
    };
    __shared__ double lgs[C];
    __shared__ float bes[C];

    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    // heads run fastest along x: with H a multiple of 8, head h runs on XCD
    // h mod 8, where the projection wrote its q and k and its carry runs
    const int h = blockIdx.x % H, chunk = blockIdx.x / H, b = blockIdx.y;
    const int c0 = chunk * C;
    const int64_t tok0 = (int64_t)b * L + c0;
    const int64_t cid = ((int64_t)b * H + h) * Nc + chunk;

    // (1) K and Q tiles into LDS by direct loads of whole 1 KiB runs (rows past
    // the end of the sequence re-read the last row: beta = 0 makes their rows
    // of T unit rows, so they meet only exact zeros in W, and the outputs of Q
    // rows past the end are never stored), gates, and the fp64 log-cumsum of
    // alpha.  Every global load is issued before the first wait.
    // Waves 1-3 issue the tile loads and wave 0 only the gate loads, so the
    // compiler's waits for the gates in wave 0 do not also wait for the tiles.
    const int last = L - 1 - c0;         // last valid row of the chunk
    if (wave > 0) {
        tile_load<D, TIn>(Ks, k, tok0, last, H, h, lane, wave - 1, 3);
        tile_load<D, TIn>(Qs, q, tok0, last, H, h, lane, wave - 1, 3);
    }
    float a_raw = 1.f, b_raw = 0.f;
    float za[GP ? 16 : 1], zb[GP ? 16 : 1];
    if (wave == 0) {
        if constexpr (GP) {
            // partial pre-activations of the gates (P <= 16 of them), summed below
            const float *src = zp + tok0 + min(lane, last);
#pragma unroll
            for (int p = 0; p < 16; ++p) {
                const int64_t row = (int64_t)min(p, P - 1) * 2 * H + h;
                za[p] = src[row * Mtot];
                zb[p] = src[(row + H) * Mtot];
            }
        } else {
            const int64_t gi = (tok0 + min(lane, last)) * H + h;
            a_raw = alpha[gi];
            b_raw = beta[gi];
        }
    }
    if (wave == 0) {
        if constexpr (GP) {
            float sa = 0.f, sb = 0.f;
#pragma unroll
            for (int p = 0; p < 16; ++p) {
                if (p < P) {
                    sa += za[p];
                    sb += zb[p];
                }
            }
            a_raw = alpha_lo + (1.f - alpha_lo) / (1.f + expf(sa));
            b_raw = 1.f / (1.f + expf(-sb));
            if (alpha_out && lane <= last) {
                const int64_t gi = (tok0 + lane) * H + h;
                alpha_out[gi] = a_raw;
                beta_out[gi] = b_raw;
            }
        }
        const bool ok = lane <= last;
        const float a = ok ? a_raw : 1.f;   // padded tokens: identity
        double x = log((double)fmaxf(a, 1e-37f));
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const double y = __shfl_up(x, off, 64);
            if (lane >= off) x += y;
        }
        lgs[lane] = x;
        bes[lane] = ok ? b_raw : 0.f;
        if constexpr (BWO) {
            const double xl = __shfl(x, 63, 64);
            bo.lg[cid * C + lane] = x;
            bo.gam[cid * C + lane] = (float)exp(x);
            bo.c[cid * C + lane] = (float)exp(xl - x);
        }
    }
    wait_vmcnt<0>();   // this wave's direct loads of the K and Q tiles landed
    __syncthreads();   // ... and the other waves'.
    if constexpr (BWO) {   // K^T, Q^T [D][64]: 8 consecutive tokens of one column per item
        for (int u = t; u < D * (C / 8); u += 256) {
            const int i = u / (C / 8), r0 = 8 * (u % (C / 8));
            float kv[8], qv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const bool ok = r0 + e <= last;
                kv[e] = ok ? tile_elem<D, TIn>(Ks, r0 + e, i) : 0.f;
                qv[e] = ok ? tile_elem<D, TIn>(Qs, r0 + e, i) : 0.f;
            }
            const int64_t o = (cid * D + i) * C + r0;
            __bf16 kh[8], kl[8], qh[8], ql[8];
            split_bf16(kv, kh, kl);
            split_bf16(qv, qh, ql);
            *reinterpret_cast<bf16x8 *>(bo.Kth + o) = pack8(kh);
            *reinterpret_cast<bf16x8 *>(bo.Qth + o) = pack8(qh);
            if constexpr (F32) {
                *reinterpret_cast<bf16x8 *>(bo.Ktl + o) = pack8(kl);
                *reinterpret_cast<bf16x8 *>(bo.Qtl + o) = pack8(ql);
            }
        }
    }

    // (2) N = diag(beta) strict_lower(Gam (.) K K^T) for this wave's 16 rows;
    // P^T tiles (m-tile mt, r-tile wave) = Gam (.) K Q^T, m <= r, in registers
    // Every LDS operand of the phase is read up front (one round trip).
    float pv[4][4];
    {
        const int r_a = 16 * wave + lr;
        f32x4 kk[4], kq[4];
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) kk[tn] = kq[tn] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (!F32) {
            bf16x8 ka[KS], qa[KS];
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                ka[s] = tile_bf8<D>(Ks, r_a, 32 * s + 8 * lg);
                qa[s] = tile_bf8<D>(Qs, r_a, 32 * s + 8 * lg);
            }
#pragma unroll
            for (int tn = 0; tn < 4; ++tn)
                if (tn <= wave) {
                    bf16x8 kb[KS];
#pragma unroll
                    for (int s = 0; s < KS; ++s) kb[s] = tile_bf8<D>(Ks, 16 * tn + lr, 32 * s + 8 * lg);
#pragma unroll
                    for (int s = 0; s < KS; ++s) {
                        kk[tn] = mfma16x16x32(ka[s], kb[s], kk[tn]);   // K_r . K_i   (rows r of this wave)
                        kq[tn] = mfma16x16x32(kb[s], qa[s], kq[tn]);   // K_m . Q_r   (rows m of tile tn)
                    }
                }
        } else {
#pragma unroll
            for (int tn = 0; tn < 4; ++tn)
                if (tn <= wave) {
#pragma unroll
                    for (int s = 0; s < KS; ++s) {
                        float a[8], bb[8], qv[8];
                        tile_frag8<D, TIn>(Ks, r_a, 32 * s + 8 * lg, a);
                        tile_frag8<D, TIn>(Ks, 16 * tn + lr, 32 * s + 8 * lg, bb);
                        tile_frag8<D, TIn>(Qs, r_a, 32 * s + 8 * lg, qv);
                        kk[tn] = mma8<false>(a, bb, kk[tn]);
                        kq[tn] = mma8<false>(bb, qv, kq[tn]);
                    }
                }
        }
        __syncthreads();   // every wave has read the Q tile, which N overwrites
        // decay factors: N[row][col] uses Gam(row, col), P[r][m] uses Gam(r, m)
        double lrow[4], lcol[4], lm[4][4];
        float brow[4];
        const double lr_a = lgs[r_a];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            lrow[j] = lgs[16 * wave + 4 * lg + j];
            brow[j] = bes[16 * wave + 4 * lg + j];
        }
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) {
            lcol[tn] = lgs[16 * tn + lr];
#pragma unroll
            for (int j = 0; j < 4; ++j) lm[tn][j] = lgs[16 * tn + 4 * lg + j];
        }
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * wave + 4 * lg + j, col = 16 * tn + lr;   // N[row][col]
                const float gn = __expf((float)(lrow[j] - lcol[tn]));
                const float nv = col < row ? brow[j] * gn * kk[tn][j] : 0.f;
                if (tn <= wave) Ns[row * LT + col] = nv;
                const int m = 16 * tn + 4 * lg + j;                               // P[r_a][m]
                const float gp = __expf((float)(lr_a - lm[tn][j]));
                pv[tn][j] = (tn <= wave && m <= r_a) ? gp * kq[tn][j] : 0.f;
                if constexpr (BWO)
                    bo.A[cid * C * C + row * C + col] = (tn <= wave && col < row && row <= last) ? gn * kk[tn][j] : 0.f;
            }
            if constexpr (BWO) {
                const bool ok = r_a <= last;
                *reinterpret_cast<f32x4 *>(bo.P + cid * C * C + r_a * C + 16 * tn + 4 * lg) =
                    f32x4{ok ? pv[tn][0] : 0.f, ok ? pv[tn][1] : 0.f, ok ? pv[tn][2] : 0.f, ok ? pv[tn][3] : 0.f};
            }
        }
    }
    __syncthreads();

    // (3) diagonal block `wave` of T by forward substitution: lane column c = lr
    {
        float tv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) tv[i] = (i == lr) ? 1.f : 0.f;
        const float *nb = Ns + (16 * wave) * LT + 16 * wave;
#pragma unroll
        for (int r = 1; r < 16; ++r) {
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < r; ++i) acc = fmaf(nb[r * LT + i], tv[i], acc);
            if (r > lr) tv[r] = -acc;
        }
        if (lg == 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) Ts[(16 * wave + r) * LT + 16 * wave + lr] = tv[r];
        }
    }
    __syncthreads();

    // 16x16 block helpers on MFMA 16x16x16 (k = 4 lg + i): A rows from a
    // row-major tile, B (k x col) from a row-major tile or a C-layout register
    auto a_rows = [&](const float *tile, int row0, int col0, float (&f)[4]) {
        const float4 v = *reinterpret_cast<const float4 *>(tile + (row0 + lr) * LT + col0 + 4 * lg);
        f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
    };
    auto b_cols = [&](const float *tile, int row0, int col0, float (&f)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = tile[(row0 + 4 * lg + i) * LT + col0 + lr];
    };
    // (4) T_{2i+1, 2i} = -T_{2i+1,2i+1} N_{2i+1,2i} T_{2i,2i}  (waves 0, 1)
    if (wave < 2) {
        const int bi = 2 * wave + 1, bj = 2 * wave;
        float a[4], bb[4];
        f32x4 y = {0.f, 0.f, 0.f, 0.f}, z = {0.f, 0.f, 0.f, 0.f};
        a_rows(Ns, 16 * bi, 16 * bj, a);
        b_cols(Ts, 16 * bj, 16 * bj, bb);
        y = mma4s(a, bb, y);
        a_rows(Ts, 16 * bi, 16 * bi, a);
        const float yb[4] = {y[0], y[1], y[2], y[3]};
        z = mma4s(a, yb, z);
#pragma unroll
        for (int j = 0; j < 4; ++j) Ts[(16 * bi + 4 * lg + j) * LT + 16 * bj + lr] = -z[j];
    }
    __syncthreads();
    // (5) rows 32..63, cols 0..31: -T_BB (N_BA T_AA) on 16x16 blocks (p, qq)
    const int p = wave >> 1, qq = wave & 1;
    {
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (kb < qq) continue;   // T_{kb, qq} = 0 above the diagonal
            float a[4], bb[4];
            a_rows(Ns, 16 * (2 + p), 16 * kb, a);
            b_cols(Ts, 16 * kb, 16 * qq, bb);
            y = mma4s(a, bb, y);
        }
        *ys_slot(wave, lane) = y;
    }
    __syncthreads();
    {
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (kb > p) continue;   // T_BB is block lower triangular
            float a[4];
            a_rows(Ts, 16 * (2 + p), 16 * (2 + kb), a);
            const f32x4 yv = *ys_slot(2 * kb + qq, lane);
            const float yb[4] = {yv[0], yv[1], yv[2], yv[3]};
            z = mma4s(a, yb, z);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) Ts[(16 * (2 + p) + 4 * lg + j) * LT + 16 * qq + lr] = -z[j];
    }
    __syncthreads();
    // the strictly upper 16x16 blocks of T are zero (they held the exchange)
    for (int idx = t; idx < 6 * 256; idx += 256) {
        const int blk = idx >> 8, e = idx & 255;
        const int bi = blk < 3 ? 0 : (blk < 5 ? 1 : 2);
        const int bj = blk < 3 ? blk + 1 : (blk < 5 ? blk - 1 : 3);
        Ts[(16 * bi + (e >> 4)) * LT + 16 * bj + (e & 15)] = 0.f;
    }
    __syncthreads();
    if constexpr (BWO) {   // T, row r = t / 4, 16 columns from 16 (t % 4)
        const int r = t >> 2, c16 = 16 * (t & 3);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            *reinterpret_cast<float4 *>(bo.T + cid * C * C + r * C + c16 + 4 * u) =
                *reinterpret_cast<const float4 *>(Ts + r * LT + c16 + 4 * u);
    }

    // (6) Tb^T fragments, A operand over k = token m (carry slot order):
    // Tb[m][c] = T[m][c] beta_c; the W variant also carries gamma_C / gamma_m
    bf16 *dW = reinterpret_cast<bf16 *>(wsW + cid * D * C);
    bf16 *dM = reinterpret_cast<bf16 *>(wsM + cid * C * C);
    const double lgC = lgs[C - 1];
    // gamma_C / gamma_m for the lane's 16 token slots m, and beta of its 4 columns
    float gw[2][8], bcs[4];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const int m = 32 * s + (jj < 4 ? 4 * lg + jj : 16 + 4 * lg + jj - 4);
            gw[s][jj] = __expf((float)(lgC - lgs[m]));
        }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) bcs[ct] = bes[16 * ct + lr];
    // K^T fragments of this wave's W rows (B operand of W^T, k = token m), each
    // scaled by gamma_C / gamma_m of its token
    float bk[NT][2][8];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
        const int i = RW * wave + 4 * NT * (lr >> 2) + 4 * tt + (lr & 3);
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const int m = 32 * s + (jj < 4 ? 4 * lg + jj : 16 + 4 * lg + jj - 4);
                bk[tt][s][jj] = tile_elem<D, TIn>(Ks, m, i) * gw[s][jj];
            }
    }
    // (7, 8) per output k-step s2 of the carry (c-tiles 2 s2, 2 s2 + 1) and per
    // c-tile h2 of it: the Tb fragments of the c-tile, then its half of the W^T
    // tiles (rows c, columns = this wave's S rows; lane column lr of tile tt is S
    // row RW wave + 4 NT (lr / 4) + 4 tt + lr % 4) and of the M^T tile (rows c,
    // columns = output tokens 16 wave + lr; B = P^T from registers, k-step s
    // covering the m-tiles 2s, 2s+1)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
        f32x4 aw_acc[NT][2], am_acc[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            const int ct = 2 * s2 + h2, c = 16 * ct + lr;
            float tb[2][8];
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    const int m = 32 * s + (jj < 4 ? 4 * lg + jj : 16 + 4 * lg + jj - 4);
                    tb[s][jj] = Ts[m * LT + c] * bcs[ct];
                }
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                aw_acc[tt][h2] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 2; ++s) aw_acc[tt][h2] = mma8<false>(tb[s], bk[tt][s], aw_acc[tt][h2]);
            }
            am_acc[h2] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                if (2 * s > wave) continue;   // P[r][m] = 0 for m > r
                const float bp[8] = {pv[2 * s][0], pv[2 * s][1], pv[2 * s][2], pv[2 * s][3],
                                     pv[2 * s + 1][0], pv[2 * s + 1][1], pv[2 * s + 1][2], pv[2 * s + 1][3]};
                am_acc[h2] = mma8<false>(tb[s], bp, am_acc[h2]);
            }
        }
        auto store_pair = [&](const f32x4 (&acc)[2], bf16 *dst) __attribute__((always_inline)) {
            float v[8] = {acc[0][0], acc[0][1], acc[0][2], acc[0][3], acc[1][0], acc[1][1], acc[1][2], acc[1][3]};
            __bf16 vh[8], vl[8];
            split_bf16(v, vh, vl);
            *reinterpret_cast<bf16x8 *>(dst) = pack8(vh);
            *reinterpret_cast<bf16x8 *>(dst + 8 * 64) = pack8(vl);
        };
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
            store_pair(aw_acc[tt], dW + ((((int64_t)(wave * NT + tt) * 2 + s2) * 2) * 64 + lane) * 8);
        store_pair(am_acc, dM + ((((int64_t)wave * 2 + s2) * 2) * 64 + lane) * 8);
        if constexpr (BWO) {
            // W^T[c][i] and M^T[c][r] at rows c = 16 (2 s2 + h2) + 4 lg + j of the accumulator tiles
            const int rr = 16 * wave + lr;
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int c = 16 * (2 * s2 + h2) + 4 * lg + j;
#pragma unroll
                    for (int tt = 0; tt < NT; ++tt) {
                        const int i = RW * wave + 4 * NT * (lr >> 2) + 4 * tt + (lr & 3);
                        const float x[2] = {aw_acc[tt][h2][j], 0.f};
                        __bf16 xh[2], xl[2];
                        split_bf16(x, xh, xl);
                        bo.Wth[(cid * C + c) * D + i] = xh[0];
                        bo.Wtl[(cid * C + c) * D + i] = xl[0];
                    }
                    bo.Mt[(cid * C + c) * C + rr] = rr <= last ? am_acc[h2][j] : 0.f;
                }
        }
    }
    // (9) gamma
    if (t < C) wsg[cid * C + t] = __expf((float)lgs[t]);
}

// ---------------------------------------------------------------------------
// carry: one kernel per loop, sequential over chunks
// ---------------------------------------------------------------------------
// One workgroup per (b, h, 16-column slice of S); the columns of S never mix,
// so column slices are independent scans.  Nine waves:
//   waves 0-3  the chain.  Wave w keeps RW = D/4 rows of the fp32 state slice in
//              registers.  Lane l = lr + 16 g holds column lr and, in tile tt of
//              its rows, the rows
//                  srow(w, g, tt, j) = RW w + 4 NT g + 4 tt + j,   j = 0..3,
//              so the KW rows a lane contributes to the K.S product are
//              contiguous (RW w + KW g .. + KW) and its K fragment is one
//              contiguous run of a token row.  Row order inside an MFMA output
//              tile is free, so the W fragments that update S (written by the
//              prep kernel) put S row srow(w, g, tt, j) at output row 4 g + j of
//              tile tt.  Per chunk: the chunk-start state S_c (split) into LDS,
//              the wave's partial K.S over its rows, reduce-scatter through LDS
//              (wave w owns tokens 16w..16w+15), E = V - diag(gamma) K S_c for its
//              tokens into LDS, then S' = gamma_C S + W E on its rows.
//   wave 4     the producer: issues every direct load of the workgroup's
//              shared operands into LDS: the chain's K tile, V slice, gamma (two
//              stages when they fit) and W fragments, and the output's Q tile, M
//              fragments and gamma.
//   waves 5-8  the output: wave 5 + o computes, for tokens 16 o .. 16 o + 15 of
//              chunk cc - 1 while the chain works on chunk cc,
//                  O = diag(gamma) Q S_c + M E
//              from Q, M, gamma, S_c and E in LDS and h_prev loaded a chunk ahead
//              into registers, and writes O itself or the loop residual
//              h = O + rho (.) h_prev (with a bf16 copy for the next loop's
//              projection).
// Every operand that all 16-column slices of a head share (K, W, Q, M: about 80
// KiB per chunk with bf16 inputs) arrives through direct global -> LDS loads of
// whole 1 KiB runs: they take the CU's vector-memory path about a third of the
// cycles per byte that 16-byte register loads of fragment-shaped pieces do, and
// that path bounds the chunk step.
// S_c and E never leave the CU.  The products use split-bf16 operands (x = hi
// + lo, ~16 significant bits) with fp32 accumulation; exact bf16 inputs are not
// split.
template <int D, typename TIn> struct CarryCfg {
    static constexpr int RW = D / 4;                     // state rows per wave
    static constexpr int NT = RW / 16;                   // 16-row tiles per wave
    static constexpr int KW = (D == 128) ? 8 : 4;        // k-width of the K.S / Q.S MFMA
    static constexpr int NSL = D / 16;                   // column slices of S
    static constexpr int ES = (int)sizeof(TIn);
    static constexpr int ROWB = D * ES;                  // bytes of a token row of K
    static constexpr int NCH = KTile<D, TIn>::NCH;       // 16-byte chunks per row
    static constexpr int SH = KTile<D, TIn>::SH;
    static constexpr int TILE = C * ROWB;                // bytes of a K chunk tile
    static constexpr int K_INS = TILE / 1024;            // direct-load instructions for K
    static constexpr int VROWB = 16 * ES;                // bytes of a token row of the V slice
    static constexpr int V_INS = C * VROWB / 1024;
    static constexpr int W_BYTES = D * C * 4;            // W hi and lo parts of one chunk
    static constexpr int W_INS = W_BYTES / 1024;
    static constexpr int VG_INS = V_INS + 1;             // V slice, gamma
    static constexpr int M_BYTES = C * C * 4;            // M hi and lo parts of one chunk
    static constexpr int M_INS = M_BYTES / 1024;
    static constexpr int QM_INS = K_INS + M_INS + 1;      // Q tile, M, gamma of the output
    // one chunk-start state slice as [wave][part: hi, lo][lane][KW] bf16
    static constexpr int SC_BYTES = 4 * 2 * 64 * KW * 2;
    // LDS besides the W / V / gamma stages: the K tile, the output's Q / M /
    // gamma, the K.S partials, E (two parities) and S_c (two parities)
    static constexpr int FIXED = TILE + TILE + M_BYTES + C * 4 + 16384 + 2 * 4096 + 2 * SC_BYTES;
    // stages of W, V, gamma: two when they fit
    static constexpr int STG = 2 * (W_BYTES + C * VROWB + C * 4) + FIXED <= 160 * 1024 ? 2 : 1;
    static_assert(STG * (W_BYTES + C * VROWB + C * 4) + FIXED <= 160 * 1024, "carry LDS");
};

// physical 16-byte chunk of logical chunk c in row r of a K tile
template <int D, typename TIn>
__device__ __forceinline__ int k_phys(int r, int c) {
    return KTile<D, TIn>::phys(r, c);
}

// Direct loads of chunk `cc` into LDS, all issued by the producer wave.
// state_produce_k: the K tile (16-byte chunks XOR-swizzled by row, K_INS
// instructions); state_produce_vg: the V slice of the workgroup's 16 columns
// and gamma (VG_INS); state_produce_w: the chunk's W fragments, a byte copy of
// their fragment-order block (W_INS).  Tokens past the end of the sequence re-read the
// last token: the prep kernel gives them beta = 0, which zeroes their columns
// of W, so any finite value is harmless.
// Per-lane byte offsets of the K and V direct loads within a chunk's first
// token row, computed once: full chunks then issue each load from a
// wave-uniform base with no per-load vector arithmetic.
template <int D, typename TIn> struct KvOffsets {
    unsigned k[CarryCfg<D, TIn>::K_INS], v[CarryCfg<D, TIn>::V_INS];
};
template <int D, typename TIn>
__device__ __forceinline__ KvOffsets<D, TIn> kv_offsets(int H, int lane) {
    using G = CarryCfg<D, TIn>;
    KvOffsets<D, TIn> o;
    const unsigned rs = (unsigned)(H * D * G::ES);   // bytes per token row of q/k/v
#pragma unroll
    for (int n = 0; n < G::K_INS; ++n) {
        const int p = n * 64 + lane;
        const int r = p / G::NCH, c = (p % G::NCH) ^ ((r << G::SH) & (G::NCH - 1));
        o.k[n] = r * rs + c * 16;
    }
    constexpr int LPR = G::VROWB / 16;   // lanes per V row
#pragma unroll
    for (int n = 0; n < G::V_INS; ++n) {
        const int p = n * 64 + lane;
        o.v[n] = (p / LPR) * rs + (p % LPR) * 16;
    }
    return o;
}
template <int D, typename TIn>
__device__ __forceinline__ void state_produce_k(unsigned ks, int cc, int L, int H, int h, int64_t tokb,
                                                const TIn *__restrict__ k, int lane, const KvOffsets<D, TIn> &off) {
    using G = CarryCfg<D, TIn>;
    constexpr int EPC = 16 / G::ES;   // elements per 16-byte chunk
    const int c0 = cc * C;
    if (c0 + C <= L) {
        const TIn *kb = k + ((tokb + c0) * H + h) * D;
#pragma unroll
        for (int n = 0; n < G::K_INS; ++n) dma16_async_s_at(kb, off.k[n], ks + n * 1024);
    } else {
#pragma unroll
        for (int n = 0; n < G::K_INS; ++n) {
            const int p = n * 64 + lane;
            const int r = p / G::NCH, c = (p % G::NCH) ^ ((r << G::SH) & (G::NCH - 1));
            const int tok = min(c0 + r, L - 1);
            dma16_async_at(k + ((tokb + tok) * H + h) * D + c * EPC, ks + n * 1024);
        }
    }
}
template <int D, typename TIn>
__device__ __forceinline__ void state_produce_vg(unsigned vs, unsigned gs, int cc, int L, int H, int h,
                                                 int64_t tokb, int col0, const TIn *__restrict__ v, const float *g,
                                                 int64_t cidb, int lane, const KvOffsets<D, TIn> &off) {
    using G = CarryCfg<D, TIn>;
    constexpr int EPC = 16 / G::ES;
    const int c0 = cc * C;
    if (c0 + C <= L) {
        const TIn *vb = v + ((tokb + c0) * H + h) * D + col0;
#pragma unroll
        for (int n = 0; n < G::V_INS; ++n) dma16_async_s_at(vb, off.v[n], vs + n * 1024);
    } else {
        constexpr int LPR = G::VROWB / 16;   // lanes per V row
#pragma unroll
        for (int n = 0; n < G::V_INS; ++n) {
            const int p = n * 64 + lane, r = p / LPR, qq = p % LPR;
            const int tok = min(c0 + r, L - 1);
            dma16_async_at(v + ((tokb + tok) * H + h) * D + col0 + qq * EPC, vs + n * 1024);
        }
    }
    // one instruction with 16 active lanes (64 floats)
    if (lane < C / 4) dma16_async_s_at(g + (cidb + cc) * C, lane * 16, gs);
}
// The output's operands of chunk cc: the Q tile (laid out as the K tile), the
// chunk's M fragments (a byte copy) and gamma (QM_INS instructions).
template <int D, typename TIn>
__device__ __forceinline__ void out_produce_qm(unsigned qs, unsigned ms, unsigned gs, int cc, int L, int H, int h,
                                               int64_t tokb, const TIn *__restrict__ q, const float *M,
                                               const float *g, int64_t cidb, int lane,
                                               const KvOffsets<D, TIn> &off) {
    using G = CarryCfg<D, TIn>;
    constexpr int EPC = 16 / G::ES;
    const int c0 = cc * C;
    if (c0 + C <= L) {
        const TIn *qb = q + ((tokb + c0) * H + h) * D;
#pragma unroll
        for (int n = 0; n < G::K_INS; ++n) dma16_async_s_at(qb, off.k[n], qs + n * 1024);
    } else {
#pragma unroll
        for (int n = 0; n < G::K_INS; ++n) {
            const int p = n * 64 + lane;
            const int r = p / G::NCH, c = (p % G::NCH) ^ ((r << G::SH) & (G::NCH - 1));
            const int tok = min(c0 + r, L - 1);
            dma16_async_at(q + ((tokb + tok) * H + h) * D + c * EPC, qs + n * 1024);
        }
    }
    const float *msrc = M + (cidb + cc) * C * C;
#pragma unroll
    for (int n = 0; n < G::M_INS; ++n) dma16_async_s_at(msrc + n * 256, lane * 16, ms + n * 1024);
    if (lane < C / 4) dma16_async_s_at(g + (cidb + cc) * C, lane * 16, gs);
}
template <int D, typename TIn>
__device__ __forceinline__ void state_produce_w(unsigned ws, int cc, const float *W, int64_t cidb, int lane) {
    using G = CarryCfg<D, TIn>;
    const float *wsrc = W + (cidb + cc) * D * C;
#pragma unroll
    for (int n = 0; n < G::W_INS; ++n) dma16_async_s_at(wsrc + n * 256, lane * 16, ws + n * 1024);
}

// K.S A fragment (token row r, this lane's KW state rows) from a K tile
template <int D, typename TIn>
__device__ __forceinline__ void k_frag(const unsigned char *tile, int r, int wave, int lg,
                                       TIn (&dst)[CarryCfg<D, TIn>::KW]) {
    using G = CarryCfg<D, TIn>;
    constexpr int BYTES = G::KW * G::ES;
    const int b0 = (G::RW * wave + G::KW * lg) * G::ES;
    const unsigned char *row = tile + r * G::ROWB;
    if constexpr (BYTES >= 16) {
#pragma unroll
        for (int part = 0; part < BYTES / 16; ++part) {
            const uint4 u = *reinterpret_cast<const uint4 *>(row + k_phys<D, TIn>(r, b0 / 16 + part) * 16);
            __builtin_memcpy(&dst[part * (16 / G::ES)], &u, 16);
        }
    } else {
        const uint2 u = *reinterpret_cast<const uint2 *>(row + k_phys<D, TIn>(r, b0 / 16) * 16 + b0 % 16);
        __builtin_memcpy(&dst[0], &u, 8);
    }
}

template <int KW>
__device__ __forceinline__ f32x4 mma_bf(const __bf16 (&a)[KW], const __bf16 (&b)[KW], f32x4 c);
template <>
__device__ __forceinline__ f32x4 mma_bf<8>(const __bf16 (&a)[8], const __bf16 (&b)[8], f32x4 c) {
    return mfma16x16x32(pack8(a), pack8(b), c);
}
template <>
__device__ __forceinline__ f32x4 mma_bf<4>(const __bf16 (&a)[4], const __bf16 (&b)[4], f32x4 c) {
    return mfma16x16x16(pack4(a), pack4(b), c);
}

// c += a.b, b given as bf16 hi/lo parts; a an exact bf16 fragment (2 passes)
template <int KW>
__device__ __forceinline__ f32x4 mma_a(const __bf16 (&a)[KW], const __bf16 (&bh)[KW],
                                       const __bf16 (&bl)[KW], f32x4 c) {
    c = mma_bf<KW>(a, bh, c);
    return mma_bf<KW>(a, bl, c);
}
// ... or an fp32 fragment, split here (3 passes)
template <int KW>
__device__ __forceinline__ f32x4 mma_a(const float (&a)[KW], const __bf16 (&bh)[KW],
                                       const __bf16 (&bl)[KW], f32x4 c) {
    __bf16 ah[KW], al[KW];
    split_bf16(a, ah, al);
    c = mma_bf<KW>(ah, bh, c);
    c = mma_bf<KW>(ah, bl, c);
    return mma_bf<KW>(al, bh, c);
}
// c += a.b with both operands as hi/lo parts (3 passes)
__device__ __forceinline__ f32x4 mma_hl(const bf16x8 &ah, const bf16x8 &al, const bf16x8 &bh,
                                        const bf16x8 &bl, f32x4 c) {
    c = mfma16x16x32(ah, bh, c);
    c = mfma16x16x32(ah, bl, c);
    return mfma16x16x32(al, bh, c);
}

// Barrier schedule per chunk cc (all nine waves take part in each):
//   B0  K, V, gamma and W of chunk cc have landed; the chain is done with chunk cc-1.
//       Chain: S_c into LDS, K.S partials.  Producer (two stages): V, gamma and
//       W of cc+1 into the other stages (their last reader, chunk cc-1, passed
//       B2 before).  Output: h_prev of chunk cc into registers.
//   B1  partials and S_c visible; the output operands of chunk cc-1 have
//       landed; the K tile is no longer read.  Chain: reduce, E into LDS, W
//       fragments.  Producer: the K tile of cc+1 (one stage), waited for with V,
//       gamma and W before B0.  Output: chunk cc-1 from Q, M, gamma, S_c and E of
//       cc-1 in LDS and h_prev in registers, stores.
//   B2  E visible; the output operands are no longer read.  Chain:
//       S = gamma_C S + W E.  Producer: the output operands of cc (one stage;
//       with one stage of everything, all loads of cc+1 as well).
// After the last chunk one more barrier (B3) makes the last output operands
// visible for the output waves' final step.  With two stages the producer's
// wait counts are the same every chunk: it issues one extra copy of chunk 0's
// output operands up front, and past the last chunk it re-reads the last chunk
// into the idle stages; it drains its loads before it exits.  S_c of chunk cc
// is rewritten at chunk cc+2 (after B0) and E at chunk cc+2 (after B1), after
// the output waves used them at cc+1.
constexpr int CARRY_THREADS = 576;
// Chunks ahead of the output step that the output waves' L2 prefetch touches.
// Where a loop's operands do not fit in the MALL (32k tokens: about 1.2 GB) the
// direct loads otherwise wait on HBM latency.
constexpr int PF_AHEAD = 3;

// h_prev at the lane's 4 (token, column) cells of one output step
enum CarryExtra : int { XM_NONE = 0, XM_STATES = 1, XM_HALT = 2 };

struct OutIn {
    float hp[4];
    int hf[4];   // halted flags of the rows (XM_HALT)
};

// XM: what the carry does besides the scan: XM_NONE, XM_STATES (store each
// chunk's start state for the backward pass) or XM_HALT (skip the outputs of
// halted rows); each is compiled in only where it is used.
template <int D, typename TIn, int RES, bool XN, int XM>
__global__ __launch_bounds__(CARRY_THREADS) void k_scan_carry(
    const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v, int L, int H, int Nc,
    const float *W, const float *__restrict__ M, const float *g, const float *s_init,
    float *s_final, float *__restrict__ o, const void *h_prev, const float *__restrict__ rho,
    float *h_out, bf16 *x_next, float *__restrict__ s_chunks, const int *__restrict__ halted) {
    using G = CarryCfg<D, TIn>;
    constexpr int NT = G::NT, RW = G::RW, KW = G::KW, STG = G::STG;
    // every stage is an object of its own, so the compiler can tell the buffers
    // a chunk reads from the ones the next chunk's direct loads write
    __shared__ __attribute__((aligned(16))) unsigned char k_s[G::TILE];
    __shared__ __attribute__((aligned(16))) unsigned char w0_s[G::W_BYTES], w1_s[STG == 2 ? G::W_BYTES : 16];
    __shared__ __attribute__((aligned(16))) unsigned char v0_s[C * G::VROWB], v1_s[STG == 2 ? C * G::VROWB : 16];
    __shared__ __attribute__((aligned(16))) float g0_s[C], g1_s[STG == 2 ? C : 4];
    __shared__ __attribute__((aligned(16))) f32x4 red[4][4][64];   // [source wave][token tile][lane]
    __shared__ __attribute__((aligned(16))) uint4 ex[2][4][64];    // [chunk parity][token tile][lane]: E hi | lo
    __shared__ __attribute__((aligned(16))) unsigned char sc_s[2][G::SC_BYTES];   // [chunk parity] S_c
    // the output step's Q tile (K-tile layout), M fragments and gamma
    __shared__ __attribute__((aligned(16))) unsigned char q_s[G::TILE], m_s[G::M_BYTES];
    __shared__ __attribute__((aligned(16))) float go_s[C];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    // heads run along x so that the D/16 column slices of one head, which read the
    // same K and W, get workgroup ids that are congruent mod 8 and share an XCD
    const int h = blockIdx.x, slice = blockIdx.y, b = blockIdx.z;
    const int col0 = slice * 16, col = col0 + lr;
    const int64_t tokb = (int64_t)b * L;
    const int64_t cidb = ((int64_t)b * H + h) * Nc;

    if (wave == 4) {
        // producer; two chunks per iteration so that the stages are compile-time choices
        const unsigned lk = lds_addr(k_s), lv[2] = {lds_addr(v0_s), lds_addr(v1_s)};
        const unsigned lgm[2] = {lds_addr(g0_s), lds_addr(g1_s)}, lw[2] = {lds_addr(w0_s), lds_addr(w1_s)};
        const unsigned lq = lds_addr(q_s), lm = lds_addr(m_s), lgo = lds_addr(go_s);
        const KvOffsets<D, TIn> off = kv_offsets<D, TIn>(H, lane);
        auto produce_qm = [&](int cc) __attribute__((always_inline)) {
            out_produce_qm<D, TIn>(lq, lm, lgo, cc, L, H, h, tokb, q, M, g, cidb, lane, off);
        };
        auto pstep = [&](auto stc, int cc) __attribute__((always_inline)) {
            constexpr int NX = STG == 2 ? 1 - decltype(stc)::value : 0;   // stage that receives chunk cc+1
            const int nx = min(cc + 1, Nc - 1);
            if constexpr (STG == 2) {
                wait_vmcnt<G::QM_INS>();    // V, gamma, W, K of cc landed (output operands of cc-1 in flight)
                lds_barrier();              // B0
                state_produce_vg<D, TIn>(lv[NX], lgm[NX], nx, L, H, h, tokb, col0, v, g, cidb, lane, off);
                state_produce_w<D, TIn>(lw[NX], nx, W, cidb, lane);
                wait_vmcnt<G::VG_INS + G::W_INS>();   // output operands of cc-1 landed (V, gamma, W of cc+1 in flight)
                lds_barrier();              // B1: the K tile of cc is no longer read
                state_produce_k<D, TIn>(lk, nx, L, H, h, tokb, k, lane, off);
                lds_barrier();              // B2
                produce_qm(cc);
            } else {
                wait_vmcnt<0>();            // every load of cc (and the output operands of cc-1) landed
                lds_barrier();              // B0
                lds_barrier();              // B1
                lds_barrier();              // B2: nothing loaded for chunk cc is read any more
                state_produce_vg<D, TIn>(lv[0], lgm[0], nx, L, H, h, tokb, col0, v, g, cidb, lane, off);
                state_produce_k<D, TIn>(lk, nx, L, H, h, tokb, k, lane, off);
                state_produce_w<D, TIn>(lw[0], nx, W, cidb, lane);
                produce_qm(cc);
            }
        };
        state_produce_vg<D, TIn>(lv[0], lgm[0], 0, L, H, h, tokb, col0, v, g, cidb, lane, off);
        state_produce_w<D, TIn>(lw[0], 0, W, cidb, lane);
        state_produce_k<D, TIn>(lk, 0, L, H, h, tokb, k, lane, off);
        if constexpr (STG == 2) produce_qm(0);   // (V, gamma, W of chunk 0 precede K here: the same order as later)   // keeps the wait counts uniform; rewritten after B2 of chunk 0
        for (int cc = 0; cc < Nc; cc += 2) {
            pstep(std::integral_constant<int, 0>(), cc);
            if (cc + 1 < Nc) pstep(std::integral_constant<int, 1>(), cc + 1);
        }
        wait_vmcnt<0>();   // the last output operands landed; no direct load may write LDS after the end
        lds_barrier();     // B3
        return;
    }

    if (wave >= 5) {
        // output waves: tokens 16 ot .. 16 ot + 15 of each chunk, this slice's columns
        const int ot = wave - 5;
        const int d = H * D;
        const float rho_c = RES ? rho[h * D + col] : 0.f;
        // h_prev of chunk cc into registers (rows past the end of the sequence
        // read the last row; their results are never stored)
        auto load_hp = [&](OutIn &in, int cc) __attribute__((always_inline)) {
            const int c0 = cc * C, last = L - 1 - c0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                in.hp[j] = 0.f;
                if constexpr (XM == XM_HALT) in.hf[j] = halted[tokb + c0 + min(16 * ot + 4 * lg + j, last)];
                if constexpr (RES != 0) {
                    const int64_t off = (tokb + c0 + min(16 * ot + 4 * lg + j, last)) * (int64_t)d + (int64_t)h * D + col;
                    if constexpr (RES == 2) in.hp[j] = (float)static_cast<const bf16 *>(h_prev)[off];
                    else in.hp[j] = static_cast<const float *>(h_prev)[off];
                }
            }
        };
        // output step of chunk cc: S_c and E from the LDS buffers of parity P,
        // Q, M and gamma from the output operand buffers
        auto compute = [&](auto pc, const OutIn &in, int cc) __attribute__((always_inline)) {
            constexpr int P = decltype(pc)::value;
            const int c0 = cc * C;
            const bf16 *scs = reinterpret_cast<const bf16 *>(sc_s[P]) + lane * KW;
            // four independent accumulator chains (Q S_c over k-steps {0,2} and
            // {1,3}, M E over the two k-steps), so the MFMAs overlap
            f32x4 qs2[2], me2[2];
            const bf16x8 *mf = reinterpret_cast<const bf16x8 *>(m_s) + lane;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                TIn qa[KW];
                k_frag<D, TIn>(q_s, 16 * ot + lr, ks, lg, qa);
                __bf16 sh[KW], sl[KW];
                __builtin_memcpy(sh, scs + (ks * 2 + 0) * 64 * KW, 2 * KW);
                __builtin_memcpy(sl, scs + (ks * 2 + 1) * 64 * KW, 2 * KW);
                if (ks < 2) qs2[ks] = f32x4{0.f, 0.f, 0.f, 0.f};
                qs2[ks & 1] = mma_a<KW>(qa, sh, sl, qs2[ks & 1]);
                if (ks < 2) {
                    const int s = ks;
                    const uint4 a4 = ex[P][2 * s][lane], c4 = ex[P][2 * s + 1][lane];
                    const uint4 hi = make_uint4(a4.x, a4.y, c4.x, c4.y), lo = make_uint4(a4.z, a4.w, c4.z, c4.w);
                    bf16x8 ebh, ebl;
                    __builtin_memcpy(&ebh, &hi, 16);
                    __builtin_memcpy(&ebl, &lo, 16);
                    me2[s] = mma_hl(mf[((ot * 2 + s) * 2 + 0) * 64], mf[((ot * 2 + s) * 2 + 1) * 64], ebh, ebl,
                                    f32x4{0.f, 0.f, 0.f, 0.f});
                }
            }
            const f32x4 qs = qs2[0] + qs2[1], me = me2[0] + me2[1];
            const f32x4 gv = *reinterpret_cast<const f32x4 *>(go_s + 16 * ot + 4 * lg);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * ot + 4 * lg + j;
                if (c0 + r >= L) continue;
                const float ov = gv[j] * qs[j] + me[j];
                const int64_t row = tokb + c0 + r;
                if constexpr (XM == XM_HALT)
                    if (in.hf[j] != 0) continue;   // a halted position keeps its state
                if constexpr (RES == 0) {
                    if (o) o[(row * H + h) * D + col] = ov;
                } else {
                    const float hv = ov + rho_c * in.hp[j];
                    const int64_t hi = row * d + (int64_t)h * D + col;
                    h_out[hi] = hv;
                    if constexpr (XN) x_next[hi] = (bf16)hv;
                }
            }
        };
        OutIn in0, in1;
        // one chunk per step, two per iteration so that the register set and the
        // LDS parity are compile-time choices
        // L2 prefetch, PF_AHEAD chunks ahead: one load touching each 128-byte line of
        // that chunk's K, Q, W, M, V, h_prev and gamma for this head, the lines dealt
        // over the head's slice workgroups (which share an XCD's L2).  The loaded word
        // is consumed two chunks later, long after it has arrived.
        unsigned pfv[2] = {0u, 0u};
        auto prefetch = [&](auto pc, int cc) __attribute__((always_inline)) {
            constexpr int P = decltype(pc)::value;
            constexpr int RL = G::ROWB / 128;
            constexpr int KL = C * RL, WL = G::W_BYTES / 128, ML = G::M_BYTES / 128;
            constexpr int HES = RES == 2 ? 2 : 4;
            constexpr int HRL = RES ? D * HES / 128 : 0, HL = C * HRL, GL = C * 4 / 128;
            constexpr int NL = 3 * KL + WL + ML + HL + GL;
            asm volatile("" ::"v"(pfv[P]));
            const int j = slice + G::NSL * (lane * 4 + ot);
            if (j < NL) {
                const int cp = min(cc + PF_AHEAD, Nc - 1), c0p = cp * C;
                const char *p;
                int jj = j;
                auto row_tok = [&](int r) { return tokb + min(c0p + r, L - 1); };
                if (jj < KL) {
                    p = reinterpret_cast<const char *>(k + (row_tok(jj / RL) * H + h) * D) + (jj % RL) * 128;
                } else if ((jj -= KL) < KL) {
                    p = reinterpret_cast<const char *>(q + (row_tok(jj / RL) * H + h) * D) + (jj % RL) * 128;
                } else if ((jj -= KL) < KL) {
                    p = reinterpret_cast<const char *>(v + (row_tok(jj / RL) * H + h) * D) + (jj % RL) * 128;
                } else if ((jj -= KL) < WL) {
                    p = reinterpret_cast<const char *>(W + (cidb + cp) * D * C) + jj * 128;
                } else if ((jj -= WL) < ML) {
                    p = reinterpret_cast<const char *>(M + (cidb + cp) * C * C) + jj * 128;
                } else if ((jj -= ML) < HL) {
                    p = reinterpret_cast<const char *>(h_prev) +
                        (row_tok(jj / HRL) * (int64_t)d + (int64_t)h * D) * HES + (jj % HRL) * 128;
                } else {
                    jj -= HL;
                    p = reinterpret_cast<const char *>(g + (cidb + cp) * C) + jj * 128;
                }
                pfv[P] = *reinterpret_cast<const unsigned *>(p);
            }
        };
        auto ostep = [&](auto pc, OutIn &cur, OutIn &prev, int cc) __attribute__((always_inline)) {
            constexpr int P = decltype(pc)::value;   // parity of chunk cc
            lds_barrier();   // B0
            load_hp(cur, cc);
            prefetch(pc, cc);
            lds_barrier();   // B1
            if (cc > 0) compute(std::integral_constant<int, 1 - P>(), prev, cc - 1);
            lds_barrier();   // B2
        };
        for (int cc = 0; cc < Nc; cc += 2) {
            ostep(std::integral_constant<int, 0>(), in0, in1, cc);
            if (cc + 1 < Nc) ostep(std::integral_constant<int, 1>(), in1, in0, cc + 1);
        }
        asm volatile("" ::"v"(pfv[0]), "v"(pfv[1]));
        lds_barrier();   // B3: the last chunk's output operands are visible
        // the last chunk: its S_c and E stay in LDS, nobody rewrites them
        if ((Nc - 1) & 1) compute(std::integral_constant<int, 1>(), in1, Nc - 1);
        else compute(std::integral_constant<int, 0>(), in0, Nc - 1);
        return;
    }

    // chain waves.  state slice: Sv[tt][j] = S[RW wave + 4 NT lg + 4 tt + j][col]
    float Sv[NT][4];
    const int64_t sbase = ((int64_t)b * H + h) * D * D;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            Sv[tt][j] = s_init ? s_init[sbase + (int64_t)(RW * wave + 4 * NT * lg + 4 * tt + j) * D + col] : 0.f;
    // Nothing loaded before the loop may be pending inside it: otherwise the
    // compiler's wait for these registers lands in the loop body.
    wait_vmcnt<0>();

    // One chunk step on LDS stage ST (= cc mod 2 with two stages).  Two steps per
    // loop iteration so that stage and parity are compile-time constants.
    int ccs = 0;   // chunk of the step
    auto step = [&](auto pc) __attribute__((always_inline)) {
        constexpr int P = decltype(pc)::value;
        constexpr int ST = STG == 2 ? P : 0;
        const unsigned char *k_cur = k_s;
        const unsigned char *v_cur = ST == 0 ? v0_s : v1_s;
        const float *g_cur = ST == 0 ? g0_s : g1_s;
        const bf16x8 *w_cur = reinterpret_cast<const bf16x8 *>(ST == 0 ? w0_s : w1_s) + wave * NT * 4 * 64 + lane;
        lds_barrier();   // (B0) chunk cc's loads have landed; chunk cc-1's stage is free
        if constexpr (XM == XM_STATES) {   // chunk-start states for the backward pass
            float *dst = s_chunks + (cidb + ccs) * D * D;
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                for (int j = 0; j < 4; ++j) dst[(int64_t)(RW * wave + 4 * NT * lg + 4 * tt + j) * D + col] = Sv[tt][j];
        }
        ++ccs;
        // chunk-start state as the B operand of K.S (and, in LDS, of Q.S for the output waves)
        __bf16 sh[KW], sl[KW];
        {
            float sf[KW];
#pragma unroll
            for (int i = 0; i < KW; ++i) sf[i] = Sv[i / 4][i % 4];
            split_bf16(sf, sh, sl);
            bf16 *dst = reinterpret_cast<bf16 *>(sc_s[P]) + (wave * 2 * 64 + lane) * KW;
            __builtin_memcpy(dst, sh, 2 * KW);
            __builtin_memcpy(dst + 64 * KW, sl, 2 * KW);
        }
        f32x4 ks[4];
#pragma unroll
        for (int tm = 0; tm < 4; ++tm) {
            TIn ak[KW];
            k_frag<D, TIn>(k_cur, 16 * tm + lr, wave, lg, ak);
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            ks[tm] = mma_a<KW>(ak, sh, sl, z);
        }
#pragma unroll
        for (int tm = 0; tm < 4; ++tm)
            if (tm != wave) red[wave][tm][lane] = ks[tm];
        lds_barrier();   // (B1) partials and S_c visible; W of chunk cc has landed
        f32x4 kt = ks[0];
#pragma unroll
        for (int tm = 1; tm < 4; ++tm)
            if (tm == wave) kt = ks[tm];
#pragma unroll
        for (int src = 0; src < 4; ++src)
            if (src != wave) kt += red[src][wave][lane];
        // W fragments of this wave's rows (read now, used after B2)
        bf16x8 wh[NT][2], wl[NT][2];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                wh[tt][s] = w_cur[((tt * 2 + s) * 2 + 0) * 64];
                wl[tt][s] = w_cur[((tt * 2 + s) * 2 + 1) * 64];
            }
        // E = V - diag(gamma) K S for tokens 16 wave + 4 lg + j
        float e[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 16 * wave + 4 * lg + j;
            float vv;
            if constexpr (G::ES == 2) vv = (float)reinterpret_cast<const bf16 *>(v_cur)[r * 16 + lr];
            else vv = reinterpret_cast<const float *>(v_cur)[r * 16 + lr];
            e[j] = vv - g_cur[r] * kt[j];
        }
        const float gC = g_cur[C - 1];   // read before B2: with one stage the producer refills it after B2
        {
            __bf16 eh[4], el[4];
            split_bf16(e, eh, el);
            uint4 u;
            __builtin_memcpy(&u.x, eh, 8);
            __builtin_memcpy(&u.z, el, 8);
            ex[P][wave][lane] = u;
        }
        lds_barrier();   // (B2) every E tile visible
        // E as the B operand: k-step s covers the token tiles 2s and 2s+1
        bf16x8 ebh[2], ebl[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const uint4 a4 = ex[P][2 * s][lane], c4 = ex[P][2 * s + 1][lane];
            uint4 hi = make_uint4(a4.x, a4.y, c4.x, c4.y), lo = make_uint4(a4.z, a4.w, c4.z, c4.w);
            __builtin_memcpy(&ebh[s], &hi, 16);
            __builtin_memcpy(&ebl[s], &lo, 16);
        }
        // S' = gamma_C S + W E (this wave's rows); one accumulator chain per
        // (row tile, k-step), so the MFMAs overlap
        f32x4 we[NT][2];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
                we[tt][s] = mma_hl(wh[tt][s], wl[tt][s], ebh[s], ebl[s], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int j = 0; j < 4; ++j) Sv[tt][j] = gC * Sv[tt][j] + (we[tt][0][j] + we[tt][1][j]);
    };
    for (int cc = 0; cc < Nc; cc += 2) {
        step(std::integral_constant<int, 0>());
        if (cc + 1 < Nc) step(std::integral_constant<int, 1>());
    }
    lds_barrier();   // B3 (the output waves' last step)
    if (s_final) {
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                s_final[sbase + (int64_t)(RW * wave + 4 * NT * lg + 4 * tt + j) * D + col] = Sv[tt][j];
    }
}

// ---------------------------------------------------------------------------
// carry on 32-column slices (bf16 inputs, dk = dv = 128)
// ---------------------------------------------------------------------------
// One workgroup per (b, h, 32-column slice of S): half as many workgroups as
// the 16-column carry, each bringing the chunk operands that all slices of a
// head share (K, W, Q, M: 80 KiB per chunk) into its CU once for twice the
// columns.  With 4 sequences of 16 heads this is 256 workgroups, one round on
// the chip.  Nine waves:
//   waves 0-3  the chain.  Wave w works on column tile ct = w / 2 (16 of the
//              slice's columns) and row half rh = w % 2 (rows 64 rh .. 64 rh + 63
//              of S).  Lane l = lr + 16 g keeps column 16 ct + lr and, in its
//              tile tt (0..3), the rows
//                  64 rh + 32 (tt / 2) + 8 g + 4 (tt % 2) + j,   j = 0..3,
//              which are the rows that wave 2 rh + tt / 2 of the 16-column
//              layout holds in its tile tt % 2: the prep's W fragments serve
//              unchanged (rows of wave rh are fragments 4 rh .. 4 rh + 3).  Per
//              chunk: S_c (split) into LDS, the partial K.S over its 64 rows for
//              all 64 tokens, a pairwise exchange with the other row half (row
//              half rh owns token tiles 2 rh and 2 rh + 1), E = V - diag(gamma) K S_c
//              for its tiles into LDS, then S' = gamma_C S + W E on its rows.
//   wave 4     the producer: every direct global -> LDS load of the workgroup.
//   waves 5-8  the output: wave 5 + o handles tokens 16 o .. 16 o + 15 of both
//              column tiles.  Q S_c of chunk cc in the window after B1 (S_c and
//              Q of cc in LDS), then M E of cc, O = diag(gamma) Q S_c + M E, the
//              loop residual and the stores in the window after B2 (E of cc in
//              LDS).
// Barrier schedule per chunk cc (all nine waves take part in each):
//   B0  K, V, gamma, W of cc have landed.  Chain: S_c into LDS, K.S partials.
//       Producer: V, gamma, W of cc+1 into the other stage, then M of cc.
//       Output: h_prev of cc into registers, L2 prefetch.
//   B1  partials and S_c visible; Q of cc has landed; the K tile is free.
//       Chain: exchange, W fragments, E into LDS.  Producer: K of cc+1.
//       Output: Q S_c.
//   B2  E visible; M of cc has landed; Q is free.  Chain: S update.  Producer:
//       Q of cc+1.  Output: M E, residual, stores.
// M of cc is read after B2(cc) and rewritten after B0(cc+1), E after B1(cc+1)
// and S_c after B0(cc+1), so each needs a single buffer; V, gamma and W have
// two stages.  The producer's wait counts are the same every chunk (past the
// last chunk it re-reads the last one into buffers nobody reads any more).

// Chunks ahead of the output step that the 32-column carry's L2 prefetch touches.
// This carry runs when the (sequence, head) pairs are many (at 4 x 16 of them each
// XCD holds eight slice groups), and lines fetched further ahead are then evicted
// from the XCD's L2 before use and fetched again.
constexpr int PFW_AHEAD = 1;

struct CarryW {
    static constexpr int D = 128;
    static constexpr int SW = 32;                    // columns of S per workgroup
    static constexpr int NSL = D / SW;               // slices per head
    static constexpr int ROWB = D * 2;               // bytes of a token row of K or Q
    static constexpr int TILE = C * ROWB;            // K or Q chunk tile (16 KiB)
    static constexpr int T_INS = TILE / 1024;        // direct loads per tile
    static constexpr int VROWB = SW * 2;             // bytes of a token row of the V slice
    static constexpr int V_INS = C * VROWB / 1024;
    static constexpr int W_BYTES = D * C * 4;        // W hi and lo parts of one chunk
    static constexpr int W_INS = W_BYTES / 1024;
    static constexpr int VGW_INS = V_INS + 1 + W_INS;
    static constexpr int M_BYTES = C * C * 4;        // M hi and lo parts of one chunk
    static constexpr int M_INS = M_BYTES / 1024;
    static_assert(VGW_INS + M_INS < 64, "the vector-memory counter holds 0..63");
};

template <int RES, bool XN, int XM>
__global__ __launch_bounds__(CARRY_THREADS) void k_scan_carry_w(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v, int L, int H, int Nc,
    const float *W, const float *__restrict__ M, const float *g, const float *s_init,
    float *s_final, float *__restrict__ o, const void *h_prev, const float *__restrict__ rho,
    float *h_out, bf16 *x_next, float *__restrict__ s_chunks, const int *__restrict__ halted) {
    using G = CarryW;
    using KT = KTile<128, bf16>;
    constexpr int D = G::D;
    __shared__ __attribute__((aligned(16))) unsigned char k_s[G::TILE], q_s[G::TILE], m_s[G::M_BYTES];
    __shared__ __attribute__((aligned(16))) unsigned char w0_s[G::W_BYTES], w1_s[G::W_BYTES];
    __shared__ __attribute__((aligned(16))) unsigned char v0_s[C * G::VROWB], v1_s[C * G::VROWB];
    __shared__ __attribute__((aligned(16))) float g0_s[C], g1_s[C];
    __shared__ __attribute__((aligned(16))) f32x4 red[4][2][64];   // [source wave][token tile of the partner][lane]
    __shared__ __attribute__((aligned(16))) uint4 ex[2][4][64];    // [column tile][token tile][lane]: E hi | lo
    __shared__ __attribute__((aligned(16))) uint4 sc[2][4][2][64]; // [column tile][k-step][hi, lo][lane]: S_c

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    // heads run along x, so the slices of one head get workgroup ids congruent
    // mod 8 and share an XCD's L2
    const int h = blockIdx.x, slice = blockIdx.y, b = blockIdx.z;
    const int col0 = slice * G::SW;
    const int64_t tokb = (int64_t)b * L;
    const int64_t cidb = ((int64_t)b * H + h) * Nc;

    if (wave == 4) {
        // ---- producer ----
        const unsigned lk = lds_addr(k_s), lq = lds_addr(q_s), lm = lds_addr(m_s);
        const unsigned lv[2] = {lds_addr(v0_s), lds_addr(v1_s)}, lgm[2] = {lds_addr(g0_s), lds_addr(g1_s)};
        const unsigned lw[2] = {lds_addr(w0_s), lds_addr(w1_s)};
        const unsigned rs = (unsigned)(H * D * 2);   // bytes per token row of q / k / v
        unsigned toff[G::T_INS], voff[G::V_INS];
#pragma unroll
        for (int n = 0; n < G::T_INS; ++n) {
            const int p = n * 64 + lane, r = p / KT::NCH;
            toff[n] = r * rs + KT::phys(r, p % KT::NCH) * 16;
        }
        constexpr int LPR = G::VROWB / 16;   // lanes per V row
#pragma unroll
        for (int n = 0; n < G::V_INS; ++n) {
            const int p = n * 64 + lane;
            voff[n] = (p / LPR) * rs + (p % LPR) * 16;
        }
        // K or Q tile of chunk cc (rows past the end re-read the last row)
        auto load_tile = [&](unsigned dst, const bf16 *src, int cc) __attribute__((always_inline)) {
            const int c0 = cc * C;
            if (c0 + C <= L) {
                const bf16 *base = src + ((tokb + c0) * H + h) * D;
#pragma unroll
                for (int n = 0; n < G::T_INS; ++n) dma16_async_s_at(base, toff[n], dst + n * 1024);
            } else {
#pragma unroll
                for (int n = 0; n < G::T_INS; ++n) {
                    const int p = n * 64 + lane, r = p / KT::NCH;
                    const int tok = min(c0 + r, L - 1);
                    dma16_async_at(src + ((tokb + tok) * H + h) * D + KT::phys(r, p % KT::NCH) * 8, dst + n * 1024);
                }
            }
        };
        // V slice, gamma and W of chunk cc into stage st
        auto load_vgw = [&](int st, int cc) __attribute__((always_inline)) {
            const int c0 = cc * C;
            if (c0 + C <= L) {
                const bf16 *vb = v + ((tokb + c0) * H + h) * D + col0;
#pragma unroll
                for (int n = 0; n < G::V_INS; ++n) dma16_async_s_at(vb, voff[n], lv[st] + n * 1024);
            } else {
#pragma unroll
                for (int n = 0; n < G::V_INS; ++n) {
                    const int p = n * 64 + lane;
                    const int tok = min(c0 + p / LPR, L - 1);
                    dma16_async_at(v + ((tokb + tok) * H + h) * D + col0 + (p % LPR) * 8, lv[st] + n * 1024);
                }
            }
            if (lane < C / 4) dma16_async_s_at(g + (cidb + cc) * C, lane * 16, lgm[st]);   // one instruction
            const float *wsrc = W + (cidb + cc) * D * C;
#pragma unroll
            for (int n = 0; n < G::W_INS; ++n) dma16_async_s_at(wsrc + n * 256, lane * 16, lw[st] + n * 1024);
        };
        auto load_m = [&](int cc) __attribute__((always_inline)) {
            const float *msrc = M + (cidb + cc) * C * C;
#pragma unroll
            for (int n = 0; n < G::M_INS; ++n) dma16_async_s_at(msrc + n * 256, lane * 16, lm + n * 1024);
        };
        auto pstep = [&](auto stc, int cc) __attribute__((always_inline)) {
            constexpr int ST = decltype(stc)::value;   // stage of chunk cc
            const int nx = min(cc + 1, Nc - 1);
            wait_vmcnt<G::T_INS>();                    // K, V, gamma, W of cc landed (Q of cc in flight)
            lds_barrier();                             // B0
            load_vgw(1 - ST, nx);
            load_m(cc);
            wait_vmcnt<G::VGW_INS + G::M_INS>();       // Q of cc landed
            lds_barrier();                             // B1
            load_tile(lk, k, nx);
            wait_vmcnt<G::T_INS>();                    // M of cc landed
            lds_barrier();                             // B2
            load_tile(lq, q, nx);
        };
        load_vgw(0, 0);
        load_tile(lk, k, 0);
        load_tile(lq, q, 0);
        for (int cc = 0; cc < Nc; cc += 2) {
            pstep(std::integral_constant<int, 0>(), cc);
            if (cc + 1 < Nc) pstep(std::integral_constant<int, 1>(), cc + 1);
        }
        wait_vmcnt<0>();   // no direct load may write LDS after the workgroup ends
        return;
    }

    if (wave < 4) {
        // ---- chain ----
        const int ct = wave >> 1, rh = wave & 1;
        const int col = col0 + 16 * ct + lr;
        const int64_t sbase = ((int64_t)b * H + h) * D * D;
        auto srow = [&](int tt, int j) { return 64 * rh + 32 * (tt >> 1) + 8 * lg + 4 * (tt & 1) + j; };
        float Sv[4][4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int j = 0; j < 4; ++j) Sv[tt][j] = s_init ? s_init[sbase + (int64_t)srow(tt, j) * D + col] : 0.f;
        // nothing loaded before the loop may be pending inside it
        wait_vmcnt<0>();
        const bf16x8 *wf0 = reinterpret_cast<const bf16x8 *>(w0_s) + rh * 16 * 64 + lane;
        const bf16x8 *wf1 = reinterpret_cast<const bf16x8 *>(w1_s) + rh * 16 * 64 + lane;
        int ccs = 0;   // chunk of the step
        auto step = [&](auto stc) __attribute__((always_inline)) {
            constexpr int ST = decltype(stc)::value;
            const bf16 *v_cur = reinterpret_cast<const bf16 *>(ST == 0 ? v0_s : v1_s);
            const float *g_cur = ST == 0 ? g0_s : g1_s;
            const bf16x8 *w_cur = ST == 0 ? wf0 : wf1;
            lds_barrier();   // B0
            if constexpr (XM == XM_STATES) {   // chunk-start states for the backward pass
                float *dst = s_chunks + (cidb + ccs) * D * D;
#pragma unroll
                for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                    for (int j = 0; j < 4; ++j) dst[(int64_t)srow(tt, j) * D + col] = Sv[tt][j];
            }
            ++ccs;
            // S_c as the B operand of K.S, local k-step kl = rows 64 rh + 32 kl ..; also into LDS for Q.S_c
            bf16x8 sh[2], sl[2];
#pragma unroll
            for (int kl = 0; kl < 2; ++kl) {
                const float sf[8] = {Sv[2 * kl][0], Sv[2 * kl][1], Sv[2 * kl][2], Sv[2 * kl][3],
                                     Sv[2 * kl + 1][0], Sv[2 * kl + 1][1], Sv[2 * kl + 1][2], Sv[2 * kl + 1][3]};
                __bf16 hh[8], ll[8];
                split_bf16(sf, hh, ll);
                sh[kl] = pack8(hh);
                sl[kl] = pack8(ll);
                __builtin_memcpy(&sc[ct][2 * rh + kl][0][lane], &sh[kl], 16);
                __builtin_memcpy(&sc[ct][2 * rh + kl][1][lane], &sl[kl], 16);
            }
            f32x4 ks[4];
#pragma unroll
            for (int tm = 0; tm < 4; ++tm) {
                ks[tm] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kl = 0; kl < 2; ++kl) {
                    const bf16x8 a = tile_bf8<D>(k_s, 16 * tm + lr, 64 * rh + 32 * kl + 8 * lg);
                    ks[tm] = mfma16x16x32(a, sh[kl], ks[tm]);
                    ks[tm] = mfma16x16x32(a, sl[kl], ks[tm]);
                }
            }
            // the partner owns the other row half's token tiles
            red[wave][0][lane] = rh ? ks[0] : ks[2];
            red[wave][1][lane] = rh ? ks[1] : ks[3];
            lds_barrier();   // B1
            f32x4 kt[2];
            kt[0] = (rh ? ks[2] : ks[0]) + red[wave ^ 1][0][lane];
            kt[1] = (rh ? ks[3] : ks[1]) + red[wave ^ 1][1][lane];
            // W fragments of this row half (read now, used after B2)
            bf16x8 wh[4][2], wl[4][2];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    wh[tt][s2] = w_cur[((tt * 2 + s2) * 2 + 0) * 64];
                    wl[tt][s2] = w_cur[((tt * 2 + s2) * 2 + 1) * 64];
                }
            // E = V - diag(gamma) K S_c for tokens 16 tm + 4 lg + j of the two owned tiles
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int tm = 2 * rh + i;
                float e[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 16 * tm + 4 * lg + j;
                    e[j] = (float)v_cur[r * G::SW + 16 * ct + lr] - g_cur[r] * kt[i][j];
                }
                __bf16 eh[4], el[4];
                split_bf16(e, eh, el);
                uint4 u;
                __builtin_memcpy(&u.x, eh, 8);
                __builtin_memcpy(&u.z, el, 8);
                ex[ct][tm][lane] = u;
            }
            const float gC = g_cur[C - 1];
            lds_barrier();   // B2
            // E of this column tile as the B operand: k-step s2 covers token tiles 2 s2, 2 s2 + 1
            bf16x8 ebh[2], ebl[2];
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const uint4 a4 = ex[ct][2 * s2][lane], c4 = ex[ct][2 * s2 + 1][lane];
                const uint4 hi = make_uint4(a4.x, a4.y, c4.x, c4.y), lo = make_uint4(a4.z, a4.w, c4.z, c4.w);
                __builtin_memcpy(&ebh[s2], &hi, 16);
                __builtin_memcpy(&ebl[s2], &lo, 16);
            }
            // S' = gamma_C S + W E: one accumulator chain per (row tile, k-step)
            f32x4 we[4][2];
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                for (int tt = 0; tt < 4; ++tt)
                    we[tt][s2] = mma_hl(wh[tt][s2], wl[tt][s2], ebh[s2], ebl[s2], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                for (int j = 0; j < 4; ++j) Sv[tt][j] = gC * Sv[tt][j] + (we[tt][0][j] + we[tt][1][j]);
        };
        for (int cc = 0; cc < Nc; cc += 2) {
            step(std::integral_constant<int, 0>());
            if (cc + 1 < Nc) step(std::integral_constant<int, 1>());
        }
        if (s_final) {
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                for (int j = 0; j < 4; ++j) s_final[sbase + (int64_t)srow(tt, j) * D + col] = Sv[tt][j];
        }
        return;
    }

    // ---- output (waves 5-8): tokens 16 ot .. 16 ot + 15, both column tiles ----
    const int ot = wave - 5;
    const int d = H * D;
    float rho_c[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) rho_c[ct] = RES ? rho[h * D + col0 + 16 * ct + lr] : 0.f;
    float hp[2][4];
    int hf[4];   // halted flags of the rows (XM_HALT)
    // h_prev of chunk cc and the rows' halted flags (rows past the end of the
    // sequence read the last row; never stored)
    auto load_hp = [&](int cc) __attribute__((always_inline)) {
        const int c0 = cc * C, last = L - 1 - c0;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if constexpr (XM == XM_HALT) hf[j] = halted[tokb + c0 + min(16 * ot + 4 * lg + j, last)];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                hp[ct][j] = 0.f;
                if constexpr (RES != 0) {
                    const int64_t off = (tokb + c0 + min(16 * ot + 4 * lg + j, last)) * (int64_t)d + (int64_t)h * D +
                                        col0 + 16 * ct + lr;
                    if constexpr (RES == 2) hp[ct][j] = (float)static_cast<const bf16 *>(h_prev)[off];
                    else hp[ct][j] = static_cast<const float *>(h_prev)[off];
                }
            }
    };
    // L2 prefetch, PFW_AHEAD chunks ahead: one load touching each 128-byte line of
    // that chunk's K, Q, V, W, M, h_prev and gamma for this head, the lines dealt
    // over the head's slice workgroups (which share an XCD's L2); the loaded word
    // is consumed two chunks later.
    unsigned pfv[2] = {0u, 0u};
    auto prefetch = [&](auto pc, int cc) __attribute__((always_inline)) {
        constexpr int P = decltype(pc)::value;
        constexpr int RL = G::ROWB / 128;
        constexpr int KL = C * RL, WL = G::W_BYTES / 128, ML = G::M_BYTES / 128;
        constexpr int HES = RES == 2 ? 2 : 4;
        constexpr int HRL = RES ? D * HES / 128 : 0, HL = C * HRL;
        constexpr int NL = 3 * KL + WL + ML + HL + 2;
        asm volatile("" ::"v"(pfv[P]));
        const int j = slice + G::NSL * (lane * 4 + ot);
        if (j < NL) {
            const int cp = min(cc + PFW_AHEAD, Nc - 1), c0p = cp * C;
            const char *p;
            int jj = j;
            auto row_tok = [&](int r) { return tokb + min(c0p + r, L - 1); };
            if (jj < KL) {
                p = reinterpret_cast<const char *>(k + (row_tok(jj / RL) * H + h) * D) + (jj % RL) * 128;
            } else if ((jj -= KL) < KL) {
                p = reinterpret_cast<const char *>(q + (row_tok(jj / RL) * H + h) * D) + (jj % RL) * 128;
            } else if ((jj -= KL) < KL) {
                p = reinterpret_cast<const char *>(v + (row_tok(jj / RL) * H + h) * D) + (jj % RL) * 128;
            } else if ((jj -= KL) < WL) {
                p = reinterpret_cast<const char *>(W + (cidb + cp) * D * C) + jj * 128;
            } else if ((jj -= WL) < ML) {
                p = reinterpret_cast<const char *>(M + (cidb + cp) * C * C) + jj * 128;
            } else if ((jj -= ML) < HL) {
                p = reinterpret_cast<const char *>(h_prev) +
                    (row_tok(jj / HRL) * (int64_t)d + (int64_t)h * D) * HES + (jj % HRL) * 128;
            } else {
                jj -= HL;
                p = reinterpret_cast<const char *>(g + (cidb + cp) * C) + jj * 128;
            }
            pfv[P] = *reinterpret_cast<const unsigned *>(p);
        }
    };
    const bf16x8 *mf = reinterpret_cast<const bf16x8 *>(m_s) + lane;
    auto ostep = [&](auto stc, int cc) __attribute__((always_inline)) {
        constexpr int ST = decltype(stc)::value;
        const float *g_cur = ST == 0 ? g0_s : g1_s;
        const int c0 = cc * C;
        lds_barrier();   // B0
        load_hp(cc);
        prefetch(stc, cc);
        lds_barrier();   // B1
        // Q S_c for both column tiles: two accumulator chains each (k-steps {0,2}, {1,3})
        f32x4 qa[2][2];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const bf16x8 a = tile_bf8<D>(q_s, 16 * ot + lr, 32 * ks + 8 * lg);
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                bf16x8 bh, bl;
                __builtin_memcpy(&bh, &sc[ct][ks][0][lane], 16);
                __builtin_memcpy(&bl, &sc[ct][ks][1][lane], 16);
                if (ks < 2) qa[ct][ks] = f32x4{0.f, 0.f, 0.f, 0.f};
                qa[ct][ks & 1] = mfma16x16x32(a, bh, qa[ct][ks & 1]);
                qa[ct][ks & 1] = mfma16x16x32(a, bl, qa[ct][ks & 1]);
            }
        }
        lds_barrier();   // B2
        f32x4 me[2][2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const bf16x8 mh = mf[((ot * 2 + s2) * 2 + 0) * 64], ml = mf[((ot * 2 + s2) * 2 + 1) * 64];
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                const uint4 a4 = ex[ct][2 * s2][lane], c4 = ex[ct][2 * s2 + 1][lane];
                const uint4 hi = make_uint4(a4.x, a4.y, c4.x, c4.y), lo = make_uint4(a4.z, a4.w, c4.z, c4.w);
                bf16x8 ebh, ebl;
                __builtin_memcpy(&ebh, &hi, 16);
                __builtin_memcpy(&ebl, &lo, 16);
                me[ct][s2] = mma_hl(mh, ml, ebh, ebl, f32x4{0.f, 0.f, 0.f, 0.f});
            }
        }
        const f32x4 gv = *reinterpret_cast<const f32x4 *>(g_cur + 16 * ot + 4 * lg);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            const f32x4 qs = qa[ct][0] + qa[ct][1], mev = me[ct][0] + me[ct][1];
            const int col = col0 + 16 * ct + lr;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * ot + 4 * lg + j;
                if (c0 + r >= L) continue;
                const float ov = gv[j] * qs[j] + mev[j];
                const int64_t row = tokb + c0 + r;
                if constexpr (XM == XM_HALT)
                    if (hf[j] != 0) continue;   // a halted position keeps its state
                if constexpr (RES == 0) {
                    if (o) o[(row * H + h) * D + col] = ov;
                } else {
                    const float hv = ov + rho_c[ct] * hp[ct][j];
                    const int64_t hi = row * d + (int64_t)h * D + col;
                    h_out[hi] = hv;
                    if constexpr (XN) x_next[hi] = (bf16)hv;
                }
            }
        }
    };
    for (int cc = 0; cc < Nc; cc += 2) {
        ostep(std::integral_constant<int, 0>(), cc);
        if (cc + 1 < Nc) ostep(std::integral_constant<int, 1>(), cc + 1);
    }
    asm volatile("" ::"v"(pfv[0]), "v"(pfv[1]));
}

}  // namespace

// Compute units of the current device (looked up once per device).
static int compute_units() {
    static int cus[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cus[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

hipError_t launch_scan_prep(bool f32, int B, int L, int H, int D, const void *q, const void *k,
                            GateSrc gs, ChunkWs ws, hipStream_t s) {
    const int Nc = (L + C - 1) / C;
    if ((int64_t)Nc * H > INT32_MAX) return hipErrorInvalidValue;
    dim3 grid((unsigned)(Nc * H), B);
    if (gs.zp && (f32 || gs.P < 1 || gs.P > 16)) return hipErrorInvalidValue;
#define PREP1(DD, TT, GP, BW)                                                                       \
    launch_kernel((k_scan_prep<DD, TT, GP, BW>), grid, dim3(256), 0, s, (const TT *)q, (const TT *)k, \
                  gs.alpha, gs.beta, gs.zp, gs.P, B * L, gs.alpha_out, gs.beta_out, gs.alpha_lo, L, H, Nc, \
                  ws.W, ws.M, ws.g, ws.bwd)
#define PREP(DD, TT, GP)                                                                            \
    do {                                                                                           \
        if (ws.bwd.T) PREP1(DD, TT, GP, true); else PREP1(DD, TT, GP, false);                        \
    } while (0)
    if (f32) {
        if (D == 128) PREP(128, float, false); else PREP(64, float, false);
    } else if (gs.zp) {
        if (D == 128) PREP(128, bf16, true); else PREP(64, bf16, true);
    } else {
        if (D == 128) PREP(128, bf16, false); else PREP(64, bf16, false);
    }
#undef PREP
#undef PREP1
    return hipGetLastError();
}

hipError_t launch_scan_carry(bool f32, int B, int L, int H, int D, const void *q, const void *k, const void *v,
                             ChunkWs ws, const float *s_init, float *s_final, CarryOut out, hipStream_t s) {
    const int Nc = (L + C - 1) / C;
    const int res = out.h_out == nullptr ? 0 : (out.h_prev_bf16 ? 2 : 1);
    const bool xn = out.h_out != nullptr && out.x_next != nullptr;
    // chunk-start states only in the scan form, halting only with the loop residual
    if ((out.s_chunks && (res != 0 || out.halted)) || (out.halted && res == 0)) return hipErrorInvalidValue;
    const int xm = out.s_chunks ? XM_STATES : (out.halted ? XM_HALT : XM_NONE);
    // 32-column slices when 16-column ones would need more than one round of
    // workgroups (one workgroup per CU: each holds most of the CU's LDS).  A
    // 32-column chunk step takes nearly twice as long, so with one round of
    // 16-column workgroups those are faster.
    if (!f32 && D == 128 && (int64_t)B * H * (D / 16) > compute_units()) {
        const dim3 gridw(H, D / CarryW::SW, B);
#define CARRYW(R, X, XM)                                                                           \
    launch_kernel((k_scan_carry_w<R, X, XM>), gridw, dim3(CARRY_THREADS), 0, s, (const bf16 *)q, (const bf16 *)k, \
                  (const bf16 *)v, L, H, Nc, (const float *)ws.W, (const float *)ws.M, (const float *)ws.g, \
                  s_init, s_final, out.o, out.h_prev, out.rho, out.h_out, out.x_next, out.s_chunks, out.halted)
#define CARRYW_H(R, X)                                                                             \
    do {                                                                                           \
        if (xm == XM_HALT) CARRYW(R, X, XM_HALT); else CARRYW(R, X, XM_NONE);                      \
    } while (0)
        if (res == 0) { if (xm == XM_STATES) CARRYW(0, false, XM_STATES); else CARRYW(0, false, XM_NONE); }
        else if (res == 1) { if (xn) CARRYW_H(1, true); else CARRYW_H(1, false); }
        else { if (xn) CARRYW_H(2, true); else CARRYW_H(2, false); }
#undef CARRYW_H
#undef CARRYW
        return hipGetLastError();
    }
    dim3 grid(H, D / 16, B);
#define CARRY(DD, T, R, X, XM)                                                                     \
    launch_kernel((k_scan_carry<DD, T, R, X, XM>), grid, dim3(CARRY_THREADS), 0, s, (const T *)q, (const T *)k, \
                  (const T *)v, L, H, Nc, (const float *)ws.W, (const float *)ws.M, (const float *)ws.g, \
                  s_init, s_final, out.o, out.h_prev, out.rho, out.h_out, out.x_next, out.s_chunks, out.halted)
#define CARRY_H(DD, T, R, X)                                                                       \
    do {                                                                                           \
        if (xm == XM_HALT) CARRY(DD, T, R, X, XM_HALT); else CARRY(DD, T, R, X, XM_NONE);          \
    } while (0)
#define CARRY_R(DD, T)                                                                             \
    do {                                                                                           \
        if (res == 0) { if (xm == XM_STATES) CARRY(DD, T, 0, false, XM_STATES); else CARRY(DD, T, 0, false, XM_NONE); } \
        else if (res == 1) { if (xn) CARRY_H(DD, T, 1, true); else CARRY_H(DD, T, 1, false); }     \
        else { if (xn) CARRY_H(DD, T, 2, true); else CARRY_H(DD, T, 2, false); }                   \
    } while (0)
    if (f32) {
        if (D == 128) CARRY_R(128, float); else CARRY_R(64, float);
    } else {
        if (D == 128) CARRY_R(128, bf16); else CARRY_R(64, bf16);
    }
#undef CARRY_R
#undef CARRY_H
#undef CARRY
    return hipGetLastError();
}

}  // namespace gdn
