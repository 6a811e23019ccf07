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

// Position of element (row, token c) of a per-chunk [R x 64] matrix (W: R = D
// rows of S; M: R = 64 output tokens) in the carry's fragment order.  Rows are
// split over the 4 waves (RW = R/4 each, NT = RW/16 tiles of 16); row
// RW w + 4 NT g + 4 tt + j (j < 4) is output row 4 g + j of the wave's tile tt
// (for M, and for W with D = 64, this is simply row 16 tt + 4 g + j).  The 64
// tokens form two 32-token k-steps s; lane l = lr + 16 lg of the wave holds
// output row lr and, in slot jj of its 8-element fragment, token
// 32 s + 4 lg + jj (jj < 4) or 32 s + 16 + 4 lg + (jj - 4) (jj >= 4).  Layout:
// [wave][tt][s][part: hi, lo][lane][8] bf16, so each wave reads its fragments
// with fully coalesced 16-byte loads.  The lo part sits 8 * 64 elements after
// the hi part.
template <int R>
__device__ __forceinline__ int64_t frag_index(int row, int c) {
    constexpr int RW = R / 4, NT = RW / 16;
    const int w = row / RW, rem = row % RW;
    const int g = rem / (4 * NT), tt = (rem % (4 * NT)) / 4, lr = 4 * g + rem % 4;
    const int s = c / 32, o = c % 32;
    const int lg = (o % 16) / 4, jj = (o % 4) + (o >= 16 ? 4 : 0);
    const int lane = lr + 16 * lg;
    return ((((int64_t)(w * NT + tt) * 2 + s) * 2) * 64 + lane) * 8 + jj;
}

// ---------------------------------------------------------------------------
// prep
// ---------------------------------------------------------------------------
template <int D, typename TIn>
__global__ __launch_bounds__(256) void k_scan_prep(const TIn *__restrict__ q,
                                                   const TIn *__restrict__ k,
                                                   const float *__restrict__ alpha,
                                                   const float *__restrict__ beta, int L, int H,
                                                   int Nc, float *__restrict__ wsW,
                                                   float *__restrict__ wsM,
                                                   float *__restrict__ wsg) {
    constexpr bool F32 = In<TIn>::f32;
    constexpr int PADK = F32 ? 4 : 8;
    constexpr int LDK = D + PADK;  // row stride (elements) of the K/Q tiles
    __shared__ __attribute__((aligned(16))) TIn Ks[C * LDK];
    __shared__ __attribute__((aligned(16))) TIn Qs[C * LDK];
    __shared__ float Gm[C * LDP];   // Gm[r][i] = prod_{i<m<=r} alpha_m  (i <= r)
    __shared__ float Ns[C * LDP];
    __shared__ float Ps[C * LDP];
    __shared__ float Ts[C * LDP];
    __shared__ float Xs[16 * 49];
    __shared__ float als[C], bes[C], gam[C];

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int c0 = chunk * C;
    const int64_t tok0 = (int64_t)b * L + c0;

    // (1) K, Q tiles (zero rows past the end of the sequence), alpha, beta
    constexpr int VEC = 16 / sizeof(TIn);        // elements per 16-byte load
    constexpr int CPR = D / VEC;                 // 16-byte chunks per row
    for (int idx = t; idx < C * CPR; idx += 256) {
        const int r = idx / CPR, ch = idx % CPR;
        uint4 kv = make_uint4(0, 0, 0, 0), qv = make_uint4(0, 0, 0, 0);
        if (c0 + r < L) {
            const int64_t off = ((tok0 + r) * H + h) * D + ch * VEC;
            kv = *reinterpret_cast<const uint4 *>(k + off);
            qv = *reinterpret_cast<const uint4 *>(q + off);
        }
        *reinterpret_cast<uint4 *>(Ks + r * LDK + ch * VEC) = kv;
        *reinterpret_cast<uint4 *>(Qs + r * LDK + ch * VEC) = qv;
    }
    if (t < C) {
        const bool ok = c0 + t < L;
        als[t] = ok ? alpha[(tok0 + t) * H + h] : 1.f;   // padded tokens: identity transition
        bes[t] = ok ? beta[(tok0 + t) * H + h] : 0.f;
    }
    __syncthreads();

    // (2) decay products
    if (t < C) {
        float p = 1.f;
        for (int i = t; i >= 0; --i) {
            Gm[t * LDP + i] = p;
            p *= als[i];
        }
        gam[t] = p;
    }
    __syncthreads();

    // (3) K K^T and Q K^T, lower block triangle; wave w owns rows [16w, 16w+16)
    {
        const int r_a = 16 * wave + (lane & 15);
        const int kq = 8 * (lane >> 4);
        for (int tn = 0; tn < 4; ++tn) {
            f32x4 kk = {0.f, 0.f, 0.f, 0.f}, qk = {0.f, 0.f, 0.f, 0.f};
            if (tn <= wave) {
                const int r_b = 16 * tn + (lane & 15);
#pragma unroll
                for (int ks = 0; ks < D / 32; ++ks) {
                    const int kc = 32 * ks + kq;
                    if constexpr (!F32) {
                        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(Ks + r_a * LDK + kc);
                        const bf16x8 aq = *reinterpret_cast<const bf16x8 *>(Qs + r_a * LDK + kc);
                        const bf16x8 bb = *reinterpret_cast<const bf16x8 *>(Ks + r_b * LDK + kc);
                        kk = mfma16x16x32(a, bb, kk);
                        qk = mfma16x16x32(aq, bb, qk);
                    } else {
                        float fa[8], fq[8], fb[8];
#pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            fa[i] = Ks[r_a * LDK + kc + i];
                            fq[i] = Qs[r_a * LDK + kc + i];
                            fb[i] = Ks[r_b * LDK + kc + i];
                        }
                        __bf16 ah[8], al[8], qh[8], ql[8], bh[8], bl[8];
                        split_bf16(fa, ah, al);
                        split_bf16(fq, qh, ql);
                        split_bf16(fb, bh, bl);
                        kk = mfma16x16x32(pack8(ah), pack8(bh), kk);
                        kk = mfma16x16x32(pack8(ah), pack8(bl), kk);
                        kk = mfma16x16x32(pack8(al), pack8(bh), kk);
                        qk = mfma16x16x32(pack8(qh), pack8(bh), qk);
                        qk = mfma16x16x32(pack8(qh), pack8(bl), qk);
                        qk = mfma16x16x32(pack8(ql), pack8(bh), qk);
                    }
                }
            }
            const int col = 16 * tn + (lane & 15);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * wave + 4 * (lane >> 4) + j;
                const float g = (col <= row) ? Gm[row * LDP + col] : 0.f;
                Ns[row * LDP + col] = (col < row) ? bes[row] * g * kk[j] : 0.f;
                Ps[row * LDP + col] = (col <= row) ? g * qk[j] : 0.f;
            }
        }
    }
    __syncthreads();

    // (4) T = (I + N)^{-1}: diagonal 16x16 blocks by forward substitution ...
    for (int idx = t; idx < C * C; idx += 256) {  // zero everything above the block diagonal
        const int r = idx / C, c = idx % C;
        if ((c >> 4) > (r >> 4)) Ts[r * LDP + c] = 0.f;
    }
    if (t < C) {
        const int blk = t >> 4, c = t & 15, base = 16 * blk, col = base + c;
        for (int r = 0; r < 16; ++r) {
            const int row = base + r;
            float val;
            if (r < c) val = 0.f;
            else if (r == c) val = 1.f;
            else {
                val = 0.f;
                for (int i = c; i < r; ++i) val -= Ns[row * LDP + base + i] * Ts[(base + i) * LDP + col];
            }
            Ts[row * LDP + col] = val;
        }
    }
    __syncthreads();
    // ... then block rows: T_ij = -T_ii sum_{m=j}^{i-1} N_im T_mj  (j < i)
    for (int bi = 1; bi < 4; ++bi) {
        for (int idx = t; idx < 256 * bi; idx += 256) {
            const int bj = idx >> 8, r = (idx >> 4) & 15, c = idx & 15;
            const int row = 16 * bi + r, col = 16 * bj + c;
            float acc = 0.f;
            for (int m = 16 * bj; m < 16 * bi; ++m) acc += Ns[row * LDP + m] * Ts[m * LDP + col];
            Xs[r * 49 + 16 * bj + c] = acc;
        }
        __syncthreads();
        for (int idx = t; idx < 256 * bi; idx += 256) {
            const int bj = idx >> 8, r = (idx >> 4) & 15, c = idx & 15;
            const int row = 16 * bi + r, col = 16 * bj + c;
            float acc = 0.f;
            for (int m = 0; m <= r; ++m) acc += Ts[row * LDP + 16 * bi + m] * Xs[m * 49 + 16 * bj + c];
            Ts[row * LDP + col] = -acc;
        }
        __syncthreads();
    }

    // (5) Tb = T diag(beta)
    for (int idx = t; idx < C * C; idx += 256) {
        const int r = idx / C, c = idx % C;
        Ts[r * LDP + c] *= bes[c];
    }
    __syncthreads();

    const int64_t cid = ((int64_t)b * H + h) * Nc + chunk;
    // (6) W[i][c] = sum_r K[r][i] * (gamma_C / gamma_r) * Tb[r][c]
    {
        constexpr int IPT = D / 4;
        const int c = t & 63, i0 = (t >> 6) * IPT;
        float acc[IPT];
#pragma unroll
        for (int ii = 0; ii < IPT; ++ii) acc[ii] = 0.f;
        for (int r = 0; r < C; ++r) {
            const float g = Gm[(C - 1) * LDP + r] * Ts[r * LDP + c];
#pragma unroll
            for (int ii = 0; ii < IPT; ++ii) acc[ii] = fmaf(to_f32(Ks[r * LDK + i0 + ii]), g, acc[ii]);
        }
        // W ~= Wh + Wl (bf16 hi/lo) stored in the carry's fragment order
        bf16 *dst = reinterpret_cast<bf16 *>(wsW + cid * D * C);
#pragma unroll
        for (int ii = 0; ii < IPT; ++ii) {
            const bf16 hi = (bf16)acc[ii];
            const int64_t at = frag_index<D>(i0 + ii, c);
            dst[at] = hi;
            dst[at + 8 * 64] = (bf16)(acc[ii] - (float)hi);
        }
    }
    // (7) M[r][c] = sum_m P[r][m] Tb[m][c]
    {
        const int c = t & 63, r0 = (t >> 6) * 16;
        float acc[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) acc[rr] = 0.f;
        for (int m = 0; m < C; ++m) {
            const float tb = Ts[m * LDP + c];
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) acc[rr] = fmaf(Ps[(r0 + rr) * LDP + m], tb, acc[rr]);
        }
        bf16 *dst = reinterpret_cast<bf16 *>(wsM + cid * C * C);
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const bf16 hi = (bf16)acc[rr];
            const int at = frag_index<C>(r0 + rr, c);   // M rows: 16 per wave, like a D = 64 W
            dst[at] = hi;
            dst[at + 8 * 64] = (bf16)(acc[rr] - (float)hi);
        }
    }
    // (8) gamma
    if (t < C) wsg[cid * C + t] = gam[t];
}

// ---------------------------------------------------------------------------
// carry
// ---------------------------------------------------------------------------
// One workgroup per (b, h, 16-column slice of S); wave w keeps RW = D/4 rows
// of the fp32 state slice in registers.  Lane l = lr + 16 g holds column lr
// and, in tile tt of its rows, the rows
//     srow(w, g, tt, j) = RW w + 4 NT g + 4 tt + j,   j = 0..3,
// so the KW rows a lane contributes to the K.S product are contiguous
// (RW w + KW g .. + KW) and its K fragment is one contiguous run of a token
// row.  Row order inside an MFMA output tile is free, so the W fragments that
// update S (written by the prep kernel) put S row srow(w, g, tt, j) at output
// row 4 g + j of tile tt.
//
// Per chunk the K and Q tiles, the V and h_prev slices and gamma are copied
// global -> LDS with direct loads (coalesced 16-byte rows, XOR-swizzled so the
// fragment reads are bank-conflict free), double-buffered where LDS allows, a
// chunk ahead of use; the per-wave W and M fragments come straight into
// registers, also a chunk ahead.  Exchange per chunk: each wave's partial K.S
// and Q.S of the three token tiles it does not own go through LDS (reduce-
// scatter; wave w owns tokens 16w..16w+15), then the E tile of each wave goes
// through LDS to all waves (all-gather), since W.E and M.E contract over all
// 64 tokens.
template <int D, typename TIn> struct CarryCfg {
    static constexpr int RW = D / 4;                     // state rows per wave
    static constexpr int NT = RW / 16;                   // 16-row tiles per wave
    static constexpr int KW = (D == 128) ? 8 : 4;        // k-width of the K.S MFMA
    static constexpr int ES = (int)sizeof(TIn);
    static constexpr int ROWB = D * ES;                  // bytes of a token row of K or Q
    static constexpr int NCH = ROWB / 16;                // 16-byte chunks per row
    static constexpr int SH = (ES == 4 && D == 128) ? 1 : 0;
    static constexpr int TILE = C * ROWB;                // bytes of a K or Q chunk tile
    static constexpr int KQ_STAGES = (4 * TILE <= 65536) ? 2 : 1;
    static constexpr int KQ_INS = 2 * TILE / 1024;       // direct-load instructions for K and Q
    static constexpr int VROWB = 16 * ES;                // bytes of a token row of the V slice
    static constexpr int V_INS = C * VROWB / 1024;
};

// physical 16-byte chunk of logical chunk c in row r of a K/Q tile
template <int D, typename TIn>
__device__ __forceinline__ int kq_phys(int r, int c) {
    using G = CarryCfg<D, TIn>;
    return c ^ ((r << G::SH) & (G::NCH - 1));
}

// Per-wave W and M fragments of one chunk (bf16 hi/lo, fragment order).
template <int D> struct WMFrags {
    static constexpr int NT = D / 64;
    bf16x8 wh[NT][2], wl[NT][2], mh[2], ml[2];
};

template <int D>
__device__ __forceinline__ void load_wm(WMFrags<D> &F, const float *W, const float *M, int64_t cid,
                                        int wave, int lane) {
    constexpr int NT = D / 64;
    const bf16x8 *Wf = reinterpret_cast<const bf16x8 *>(W + cid * D * C) + (int64_t)wave * NT * 4 * 64 + lane;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            F.wh[tt][s] = Wf[((tt * 2 + s) * 2 + 0) * 64];
            F.wl[tt][s] = Wf[((tt * 2 + s) * 2 + 1) * 64];
        }
    const bf16x8 *Mf = reinterpret_cast<const bf16x8 *>(M + cid * C * C) + (int64_t)wave * 4 * 64 + lane;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        F.mh[s] = Mf[(s * 2 + 0) * 64];
        F.ml[s] = Mf[(s * 2 + 1) * 64];
    }
}

// Issues this wave's share of the direct loads of chunk `cc`: K and Q tiles
// (into kq, when KQ is set), V slice and gamma (vs, gs) and, RES != 0, the
// h_prev slice (hs).  Tokens past the end of the sequence re-read the last
// token: the prep kernel gives them beta = 0, which zeroes their columns of W
// and M, and their outputs are never stored, so any finite value is harmless.
template <int D, typename TIn, int RES, bool KQ, bool REST>
__device__ __forceinline__ void carry_issue(unsigned char *__restrict__ kq, unsigned char *__restrict__ vs,
                                            float *__restrict__ gs, unsigned char *__restrict__ hs, int cc,
                                            int L, int H, int h, int64_t tokb, int col0,
                                            const TIn *__restrict__ q, const TIn *__restrict__ k,
                                            const TIn *__restrict__ v, const float *__restrict__ g,
                                            int64_t cidb, const void *__restrict__ h_prev, int wave,
                                            int lane) {
    using G = CarryCfg<D, TIn>;
    constexpr int EPC = 16 / G::ES;   // elements per 16-byte chunk
    const int c0 = cc * C;
    if constexpr (KQ) {
#pragma unroll
        for (int n = 0; n < G::KQ_INS / 4; ++n) {
            const int I = 4 * n + wave;
            const int tensor = I / (G::KQ_INS / 2);
            const int base = (I % (G::KQ_INS / 2)) * 64, p = base + lane;
            const int r = p / G::NCH, c = (p % G::NCH) ^ ((r << G::SH) & (G::NCH - 1));
            const int tok = min(c0 + r, L - 1);
            const TIn *src = (tensor ? q : k) + ((tokb + tok) * H + h) * D + c * EPC;
            dma16_async(src, kq + tensor * G::TILE + base * 16);
        }
    }
    if constexpr (REST) {
        constexpr int LPR = G::VROWB / 16;   // lanes per V row
        if (wave < G::V_INS) {
            const int p = wave * 64 + lane, r = p / LPR, qq = p % LPR;
            const int tok = min(c0 + r, L - 1);
            dma16_async(v + ((tokb + tok) * H + h) * D + col0 + qq * EPC, vs + wave * 1024);
        }
        if constexpr (RES != 0) {
            constexpr int HES = RES == 2 ? 2 : 4;
            constexpr int HLPR = 16 * HES / 16, H_INS = C * 16 * HES / 1024;
            if (wave < H_INS) {
                const int p = wave * 64 + lane, r = p / HLPR, qq = p % HLPR;
                const int tok = min(c0 + r, L - 1);
                const int64_t off = (tokb + tok) * (int64_t)H * D + (int64_t)h * D + col0 + qq * (16 / HES);
                dma16_async(static_cast<const unsigned char *>(h_prev) + off * HES, hs + wave * 1024);
            }
        }
        if (wave == 3 && lane < C / 4) dma16_async(g + (cidb + cc) * C + 4 * lane, gs);
    }
}

// K.S / Q.S A fragment (token row r, this lane's KW state rows) from a K/Q tile
template <int D, typename TIn>
__device__ __forceinline__ void kq_frag(const unsigned char *tile, int r, int wave, int lg,
                                        TIn (&dst)[CarryCfg<D, TIn>::KW]) {
    using G = CarryCfg<D, TIn>;
    constexpr int BYTES = G::KW * G::ES;
    const int b0 = (G::RW * wave + G::KW * lg) * G::ES;
    const unsigned char *row = tile + r * G::ROWB;
    if constexpr (BYTES >= 16) {
#pragma unroll
        for (int part = 0; part < BYTES / 16; ++part) {
            const uint4 u = *reinterpret_cast<const uint4 *>(row + kq_phys<D, TIn>(r, b0 / 16 + part) * 16);
            __builtin_memcpy(&dst[part * (16 / G::ES)], &u, 16);
        }
    } else {
        const uint2 u = *reinterpret_cast<const uint2 *>(row + kq_phys<D, TIn>(r, b0 / 16) * 16 + b0 % 16);
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

// number of global stores one lane issues per full chunk (the wait for the
// next chunk's direct loads lets exactly these stay in flight)
template <int RES, bool XN> struct CarryStores {
    static constexpr int N = RES == 0 ? 4 : (XN ? 8 : 4);
};

struct CarryLdsX {
    f32x4 red[4][4][2][64];   // [source wave][token tile][K.S | Q.S][lane]
    uint4 ex[4][64];          // [token tile][lane]: E hi (bf16x4) in .x .y, lo in .z .w
};

template <int D, typename TIn, int RES, bool XN, typename AfterB1>
__device__ __forceinline__ void carry_chunk(
    const WMFrags<D> &F, float (&Sv)[D / 64][4], int cc, int L, int H, int h, int64_t tokb, int col,
    float rho_c, const unsigned char *__restrict__ kq, const unsigned char *__restrict__ vs,
    const float *__restrict__ gs, const unsigned char *__restrict__ hs, CarryLdsX *__restrict__ Xp,
    float *o, float *h_out, bf16 *x_next, AfterB1 &&after_b1) {
    CarryLdsX &X = *Xp;
    using G = CarryCfg<D, TIn>;
    constexpr int NT = G::NT, KW = G::KW;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lr = lane & 15, lg = lane >> 4;

    // B operand of K.S / Q.S: this lane's KW contiguous state rows, hi/lo
    __bf16 sh[KW], sl[KW];
    {
        float sf[KW];
#pragma unroll
        for (int i = 0; i < KW; ++i) sf[i] = Sv[i / 4][i % 4];
        split_bf16(sf, sh, sl);
    }
    f32x4 ks[4], qs[4];
#pragma unroll
    for (int tm = 0; tm < 4; ++tm) {
        TIn ak[KW], aq[KW];
        kq_frag<D, TIn>(kq, 16 * tm + lr, wave, lg, ak);
        kq_frag<D, TIn>(kq + G::TILE, 16 * tm + lr, wave, lg, aq);
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        ks[tm] = mma_a<KW>(ak, sh, sl, z);
        qs[tm] = mma_a<KW>(aq, sh, sl, z);
    }
#pragma unroll
    for (int tm = 0; tm < 4; ++tm)
        if (tm != wave) {
            X.red[wave][tm][0][lane] = ks[tm];
            X.red[wave][tm][1][lane] = qs[tm];
        }
    lds_barrier();   // (B1) partials visible; every wave done reading this chunk's K and Q
    after_b1();      // single-buffered K/Q: the next chunk's tiles may now be loaded
    // own token tile: sum of the four partials (wave-uniform selects keep tiles in registers)
    f32x4 kt = ks[0], qt = qs[0];
#pragma unroll
    for (int tm = 1; tm < 4; ++tm)
        if (tm == wave) { kt = ks[tm]; qt = qs[tm]; }
#pragma unroll
    for (int src = 0; src < 4; ++src)
        if (src != wave) {
            const f32x4 a = X.red[src][wave][0][lane], b = X.red[src][wave][1][lane];
            kt += a;
            qt += b;
        }
    // E = V - diag(gamma) K S for tokens 16 wave + 4 lg + j
    float e[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 16 * wave + 4 * lg + j;
        float vv;
        if constexpr (G::ES == 2) vv = (float)reinterpret_cast<const bf16 *>(vs)[r * 16 + lr];
        else vv = reinterpret_cast<const float *>(vs)[r * 16 + lr];
        e[j] = vv - gs[r] * kt[j];
    }
    {
        __bf16 eh[4], el[4];
        split_bf16(e, eh, el);
        uint4 u;
        __builtin_memcpy(&u.x, eh, 8);
        __builtin_memcpy(&u.z, el, 8);
        X.ex[wave][lane] = u;
    }
    lds_barrier();   // (B2) every E tile visible
    // E as the B operand: k-step s covers the token tiles 2s and 2s+1
    bf16x8 ebh[2], ebl[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const uint4 a = X.ex[2 * s][lane], b = X.ex[2 * s + 1][lane];
        uint4 hi = make_uint4(a.x, a.y, b.x, b.y), lo = make_uint4(a.z, a.w, b.z, b.w);
        __builtin_memcpy(&ebh[s], &hi, 16);
        __builtin_memcpy(&ebl[s], &lo, 16);
    }
    const float gC = gs[C - 1];
    // S' = gamma_C S + W E (this wave's rows)
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
        f32x4 we = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 2; ++s) we = mma_hl(F.wh[tt][s], F.wl[tt][s], ebh[s], ebl[s], we);
#pragma unroll
        for (int j = 0; j < 4; ++j) Sv[tt][j] = gC * Sv[tt][j] + we[j];
    }
    // O = diag(gamma) Q S + M E for tokens 16 wave + 4 lg + j
    f32x4 me = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 2; ++s) me = mma_hl(F.mh[s], F.ml[s], ebh[s], ebl[s], me);
    // Outputs through buffer stores whose range ends at the last token of the
    // sequence: rows past it are dropped by the hardware, so every lane issues
    // exactly CarryStores::N stores per chunk, with no branch around them (the
    // wait for the next chunk's loads relies on that count).
    const int d = H * D;
    const int nvalid = min(C, L - cc * C);
    const int64_t row0 = tokb + (int64_t)cc * C;
    if constexpr (RES == 0) {
        const __amdgpu_buffer_rsrc_t ro = buffer_rsrc(o + row0 * d, nvalid * d * 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 16 * wave + 4 * lg + j;
            const float ov = gs[r] * qt[j] + me[j];
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, ov), ro, (r * d + h * D + col) * 4, 0, 0);
        }
    } else {
        const __amdgpu_buffer_rsrc_t rh = buffer_rsrc(h_out + row0 * d, nvalid * d * 4);
        __amdgpu_buffer_rsrc_t rx;
        if constexpr (XN) rx = buffer_rsrc(x_next + row0 * d, nvalid * d * 2);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 16 * wave + 4 * lg + j;
            const float ov = gs[r] * qt[j] + me[j];
            float hp;
            if constexpr (RES == 2) hp = (float)reinterpret_cast<const bf16 *>(hs)[r * 16 + lr];
            else hp = reinterpret_cast<const float *>(hs)[r * 16 + lr];
            const float hn = ov + rho_c * hp;
            const int e = r * d + h * D + col;
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, hn), rh, e * 4, 0, 0);
            if constexpr (XN)
                __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(short, (bf16)hn), rx, e * 2, 0, 0);
        }
    }
}

template <int D, typename TIn, int RES, bool XN>
__global__ __launch_bounds__(256) void k_scan_carry(
    const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v, int L, int H,
    int Nc, const float *W, const float *M, const float *__restrict__ g,
    const float *__restrict__ s_init, float *__restrict__ s_final, float *__restrict__ o,
    const void *h_prev, const float *__restrict__ rho, float *h_out, bf16 *x_next) {
    // (W and M are not __restrict__: their loads must stay ordered with the
    // wait_vmcnt fences, which a restrict pointer's loads may be moved across.)
    using G = CarryCfg<D, TIn>;
    constexpr int NT = G::NT, RW = G::RW;
    constexpr int HB = RES == 0 ? 16 : C * 16 * (RES == 2 ? 2 : 4);
    constexpr int NST = CarryStores<RES, XN>::N;
    // every stage is an object of its own, so the compiler can tell the buffers
    // a chunk reads from the ones the next chunk's direct loads write
    __shared__ __attribute__((aligned(16))) unsigned char kq0_s[2 * G::TILE];
    __shared__ __attribute__((aligned(16))) unsigned char kq1_s[G::KQ_STAGES == 2 ? 2 * G::TILE : 16];
    __shared__ __attribute__((aligned(16))) unsigned char v0_s[C * G::VROWB], v1_s[C * G::VROWB];
    __shared__ __attribute__((aligned(16))) unsigned char h0_s[HB], h1_s[HB];
    __shared__ __attribute__((aligned(16))) float g0_s[C], g1_s[C];
    __shared__ CarryLdsX X;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lg = lane >> 4;
    // heads run along x so that the D/16 column slices of one head, which read the
    // same K, Q, W and M, get workgroup ids that are congruent mod 8 and share an XCD
    const int h = blockIdx.x, slice = blockIdx.y, b = blockIdx.z;
    const int col0 = slice * 16, col = col0 + (lane & 15);
    const int64_t tokb = (int64_t)b * L;
    const int64_t cidb = ((int64_t)b * H + h) * Nc;
    const float rho_c = RES ? rho[h * D + col] : 0.f;

    // state slice: Sv[tt][j] = S[RW wave + 4 NT lg + 4 tt + j][col]
    float Sv[NT][4];
    const int64_t sbase = ((int64_t)b * H + h) * D * D;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            Sv[tt][j] = s_init ? s_init[sbase + (int64_t)(RW * wave + 4 * NT * lg + 4 * tt + j) * D + col] : 0.f;
    // Nothing loaded before the loop may be pending inside it: otherwise the
    // compiler's wait for these registers lands in the loop body (every chunk).
    wait_vmcnt<0>();

    WMFrags<D> fa, fb;
    carry_issue<D, TIn, RES, true, true>(kq0_s, v0_s, g0_s, h0_s, 0, L, H, h, tokb, col0, q, k, v, g, cidb,
                                         h_prev, wave, lane);
    load_wm<D>(fa, W, M, cidb, wave, lane);
    wait_vmcnt<0>();   // chunk 0's loads (the waits in the loop assume only stores are older)

    // One chunk step on LDS stage ST (= cc mod 2): wait for chunk cc's loads,
    // issue chunk cc+1's into the other stage, compute cc.  Two steps per loop
    // iteration so stages are compile-time constants and the W/M register sets
    // swap roles without copies.
    auto step = [&](auto stc, int cc, const WMFrags<D> &cur, WMFrags<D> &nxt) __attribute__((always_inline)) {
        constexpr int ST = decltype(stc)::value;
        unsigned char *kq_cur = (G::KQ_STAGES == 1 || ST == 0) ? kq0_s : kq1_s;
        unsigned char *kq_nxt = (G::KQ_STAGES == 1 || ST == 1) ? kq0_s : kq1_s;
        unsigned char *v_cur = ST == 0 ? v0_s : v1_s, *v_nxt = ST == 0 ? v1_s : v0_s;
        unsigned char *h_cur = ST == 0 ? h0_s : h1_s, *h_nxt = ST == 0 ? h1_s : h0_s;
        float *g_cur = ST == 0 ? g0_s : g1_s, *g_nxt = ST == 0 ? g1_s : g0_s;
        wait_vmcnt<NST>();   // only the previous chunk's stores may remain in flight
        lds_barrier();            // (B0) chunk cc's direct loads of every wave have landed
        const bool more = cc + 1 < Nc;
        if (more) {
            carry_issue<D, TIn, RES, G::KQ_STAGES == 2, true>(kq_nxt, v_nxt, g_nxt, h_nxt, cc + 1, L, H, h, tokb,
                                                            col0, q, k, v, g, cidb, h_prev, wave, lane);
            load_wm<D>(nxt, W, M, cidb + cc + 1, wave, lane);
        }
        carry_chunk<D, TIn, RES, XN>(cur, Sv, cc, L, H, h, tokb, col, rho_c, kq_cur, v_cur, g_cur, h_cur, &X, o,
                                     h_out, x_next, [&]() __attribute__((always_inline)) {
                                         if constexpr (G::KQ_STAGES == 1)
                                             if (more)
                                                 carry_issue<D, TIn, RES, true, false>(
                                                     kq0_s, v_nxt, g_nxt, h_nxt, cc + 1, L, H, h, tokb, col0,
                                                     q, k, v, g, cidb, h_prev, wave, lane);
                                     });
    };
    for (int cc = 0; cc < Nc; cc += 2) {
        step(std::integral_constant<int, 0>(), cc, fa, fb);
        if (cc + 1 < Nc) step(std::integral_constant<int, 1>(), cc + 1, fb, fa);
    }
    if (s_final) {
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                s_final[sbase + (int64_t)(RW * wave + 4 * NT * lg + 4 * tt + j) * D + col] = Sv[tt][j];
    }
}

}  // namespace

hipError_t launch_scan_prep(bool f32, int B, int L, int H, int D, const void *q, const void *k,
                            const float *alpha, const float *beta, ChunkWs ws, hipStream_t s) {
    const int Nc = (L + C - 1) / C;
    dim3 grid(Nc, H, B);
#define PREP(DD, T)                                                                                \
    launch_kernel((k_scan_prep<DD, T>), grid, dim3(256), 0, s, (const T *)q, (const T *)k,   \
                       alpha, beta, L, H, Nc, ws.W, ws.M, ws.g)
    if (f32) {
        if (D == 128) PREP(128, float); else PREP(64, float);
    } else {
        if (D == 128) PREP(128, bf16); else PREP(64, bf16);
    }
#undef PREP
    return hipGetLastError();
}

hipError_t launch_scan_carry(bool f32, int B, int L, int H, int D, const void *q, const void *k,
                             const void *v, ChunkWs ws, const float *s_init, float *s_final,
                             CarryOut out, hipStream_t s) {
    const int Nc = (L + C - 1) / C;
    dim3 grid(H, D / 16, B);
    const int res = out.h_out == nullptr ? 0 : (out.h_prev_bf16 ? 2 : 1);
    const bool xn = out.h_out != nullptr && out.x_next != nullptr;
#define CARRY(DD, T, R, X)                                                                         \
    launch_kernel((k_scan_carry<DD, T, R, X>), grid, dim3(256), 0, s, (const T *)q, (const T *)k,  \
                  (const T *)v, L, H, Nc, ws.W, ws.M, ws.g, s_init, s_final, out.o, out.h_prev,    \
                  out.rho, out.h_out, out.x_next)
#define CARRY_R(DD, T)                                                                             \
    do {                                                                                           \
        if (res == 0) CARRY(DD, T, 0, false);                                                      \
        else if (res == 1) { if (xn) CARRY(DD, T, 1, true); else CARRY(DD, T, 1, false); }         \
        else { if (xn) CARRY(DD, T, 2, true); else CARRY(DD, T, 2, false); }                       \
    } while (0)
    if (f32) {
        if (D == 128) CARRY_R(128, float); else CARRY_R(64, float);
    } else {
        if (D == 128) CARRY_R(128, bf16); else CARRY_R(64, bf16);
    }
#undef CARRY_R
#undef CARRY
    return hipGetLastError();
}

}  // namespace gdn
