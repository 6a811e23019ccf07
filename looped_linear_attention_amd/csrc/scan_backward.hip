// scan_backward.hip -- backward pass of the chunkwise gated-delta-rule scan on gfx950.
//
// The forward recurrence (LT2: Linear-Time Looped Transformers, Section 2
// "LT2" paragraph and Appendix B.1; the gated delta rule of the GDN reference
// the pages cite) is trained through (Appendix C: every looped model is
// trained with bf16 mixed precision at T = 4).  Per (sequence, head) and
// chunk of C = 64 tokens with start state S, end state S', gamma_r = prod of
// alpha up to r within the chunk, Gam_ri = gamma_r / gamma_i, c_r = gamma_C /
// gamma_r:
//     A  = strict_lower(Gam (.) K K^T),  T = (I + diag(beta) A)^{-1},  Tb = T diag(beta)
//     P  = lower_incl(Gam (.) Q K^T)
//     E  = V - diag(gamma) K S,          U = Tb E
//     O  = diag(gamma) Q S + P U,        S' = gamma_C S + (diag(c) K)^T U
// (the forward writes M = P Tb and W = (diag(c) K)^T Tb, so O = diag(gamma) Q S
// + M E and S' = gamma_C S + W E).  Given dO and dS' the backward is
//     dU = P^T dO + diag(c) K dS'
//     dE = Tb^T dU = M^T dO + W^T dS'                       (= dV)
//     dS = gamma_C dS' + Q^T diag(gamma) dO - K^T diag(gamma) dE
// chunk after chunk in reverse (k_bwd_carry: sequential over chunks, parallel
// over column slices of S, from the fp32 T, P, gamma, c that the forward's
// chunk preparation also writes when asked), and per chunk, in parallel
// (k_bwd_chunk):
//     dP  = lower_incl(dO U^T),  dTb = dU E^T,  dT = dTb diag(beta),
//     dN  = strict_lower(-T^T dT T^T),  dA = diag(beta) dN
//     dQ  = diag(gamma) dO S^T + (Gam (.) dP) K
//     dK  = (Gam (.) dP)^T Q + (Gam (.) dA) K + (Gam (.) dA)^T K
//           - diag(gamma) dE S^T + diag(c) U dS'^T
//     dbeta_m = sum_r dTb_rm T_rm + sum_i dN_mi A_mi
// and the decay gradient through the chunk's log-cumsum lg (gamma_r = e^{lg_r},
// Gam_ab = e^{lg_a - lg_b}, c_r = e^{lg_last - lg_r}, each depending on
// log alpha_m for m <= r, b < m <= a, r < m respectively; gamma_C on every m):
//     dlog alpha_m = sum_{r >= m} gamma_r dgamma_r + sum_{a >= m > b} (A (.) dA + P (.) dP)_ab
//                    + sum_{r < m} c_r dc_r + gamma_C dgamma_C,   dalpha_m = dlog alpha_m / alpha_m,
//     dgamma_r = sum_j dO_rj (Q S)_rj - dE_rj (K S)_rj,  dc_r = sum_j U_rj (K dS')_rj,
//     dgamma_C = sum S (.) dS'.
// Tokens past the end of a sequence are zero rows with alpha = 1, beta = 0,
// so they contribute nothing.  Products of the reverse carry and of the chunk
// kernel run on 16x16x32 MFMA with fp32 operands split into bf16 hi + lo
// (exact bf16 inputs are not split); the rest is fp32 VALU arithmetic.
#include "gdn_device.h"
#include "gdn_kernels.h"

namespace gdn {

namespace {

constexpr int C = 64;

// Per-chunk matrices of the backward, fp32: T, P, A [64][64] row-major, the
// log-cumsum lg [64] (fp64), gamma = e^lg and c = e^(lg_last - lg) [64]; and
// the operands of the reverse carry: W^T = diag(beta) T^T diag(c) K [64][D]
// as bf16 hi and lo planes, K^T and Q^T [D][64] as bf16 hi (and, for fp32
// inputs, lo) planes, M^T dO = diag(beta) T^T P^T dO [64][D] fp32, and
// M^T = diag(beta) T^T P^T [64][64] fp32.  The forward's chunk preparation
// writes all but M^T dO (k_bwd_ops).
struct BwdMats {
    float *T, *P, *A;
    double *lg;
    float *gam, *c;
    bf16 *Wth, *Wtl, *Kth, *Ktl, *Qth, *Qtl;
    float *MtdO, *Mt;
};
// bytes per chunk
__host__ __device__ constexpr size_t bwd_mats_per_chunk(int D) {
    return 4 * C * C * 4 + C * 8 + 2 * C * 4 + (size_t)6 * D * C * 2 + (size_t)C * D * 4;
}
// The regions of a BwdMats block for `chunks` chunks, each array for all chunks in turn.
BwdMats bwd_mats(float *base, int64_t chunks, int D) {
    BwdMats m;
    m.T = base;
    m.P = m.T + chunks * C * C;
    m.A = m.P + chunks * C * C;
    m.lg = reinterpret_cast<double *>(m.A + chunks * C * C);
    m.gam = reinterpret_cast<float *>(m.lg + chunks * C);
    m.c = m.gam + chunks * C;
    bf16 *b = reinterpret_cast<bf16 *>(m.c + chunks * C);
    const int64_t plane = chunks * C * D;
    m.Wth = b;
    m.Wtl = b + plane;
    m.Kth = b + 2 * plane;
    m.Ktl = b + 3 * plane;
    m.Qth = b + 4 * plane;
    m.Qtl = b + 5 * plane;
    m.MtdO = reinterpret_cast<float *>(b + 6 * plane);
    m.Mt = m.MtdO + chunks * C * D;
    return m;
}

// ---------------------------------------------------------------------------
// M^T dO: one workgroup (4 waves) per (b, h, chunk)
// ---------------------------------------------------------------------------
// (M^T dO)[m][i] = sum_r M^T[m][r] dO[r][i] on 16x16x32 MFMA, both operands
// fp32 split into bf16 hi + lo (3 passes).  dO is staged transposed ([i][r])
// in LDS as the two bf16 planes; wave w forms output rows 16 w .. 16 w + 15.
// Rows of dO past the end of the sequence are zero.
constexpr int BO_THREADS = 256;

template <int D>
__global__ __launch_bounds__(BO_THREADS) void k_bwd_ops(const float *__restrict__ d_o, int L, int H, int Nc,
                                                        BwdMats bm) {
    constexpr int TL = C + 8;   // row stride (bf16) of the transposed planes: 16-byte aligned rows
    __shared__ __attribute__((aligned(16))) bf16 dOh[D * TL], dOl[D * TL];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6, lr = lane & 15, lg = lane >> 4;
    const int h = blockIdx.x % H, chunk = blockIdx.x / H, b = blockIdx.y;
    const int c0 = chunk * C, nvalid = min(C, L - c0);
    const int64_t tok0 = (int64_t)b * L + c0;
    const int64_t cid = ((int64_t)b * H + h) * Nc + chunk;
    // token rows 2 rp, 2 rp + 1 and columns 4 q4 .. 4 q4 + 3 per item: one 4-byte LDS write per column and plane
    for (int n = t; n < (C / 2) * (D / 4); n += BO_THREADS) {
        const int rp = n / (D / 4), i4 = 4 * (n % (D / 4)), r = 2 * rp;
        float4 v0 = {0.f, 0.f, 0.f, 0.f}, v1 = {0.f, 0.f, 0.f, 0.f};
        if (r < nvalid) v0 = *reinterpret_cast<const float4 *>(d_o + ((tok0 + r) * H + h) * D + i4);
        if (r + 1 < nvalid) v1 = *reinterpret_cast<const float4 *>(d_o + ((tok0 + r + 1) * H + h) * D + i4);
        const float x[8] = {v0.x, v1.x, v0.y, v1.y, v0.z, v1.z, v0.w, v1.w};
        bf16 hh[8], ll[8];
        split_bf16<8>(x, hh, ll);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bf16 ph[2] = {hh[2 * e], hh[2 * e + 1]}, pl2[2] = {ll[2 * e], ll[2 * e + 1]};
            __builtin_memcpy(dOh + (i4 + e) * TL + r, ph, 4);
            __builtin_memcpy(dOl + (i4 + e) * TL + r, pl2, 4);
        }
    }
    // A fragments: M^T row 16 wave + lr, k = r = 32 s + 8 lg ..
    bf16x8 ah[2], al[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const float4 *src = reinterpret_cast<const float4 *>(bm.Mt + (cid * C + 16 * wave + lr) * C + 32 * s + 8 * lg);
        const float4 a = src[0], c = src[1];
        const float x[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
        bf16 hh[8], ll[8];
        split_bf16<8>(x, hh, ll);
        ah[s] = pack8(hh);
        al[s] = pack8(ll);
    }
    __syncthreads();
#pragma unroll 2
    for (int ct = 0; ct < D / 16; ++ct) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int o = (16 * ct + lr) * TL + 32 * s + 8 * lg;
            const bf16x8 bh = *reinterpret_cast<const bf16x8 *>(dOh + o), bl = *reinterpret_cast<const bf16x8 *>(dOl + o);
            acc = mfma16x16x32(ah[s], bh, acc);
            acc = mfma16x16x32(ah[s], bl, acc);
            acc = mfma16x16x32(al[s], bh, acc);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) bm.MtdO[(cid * C + 16 * wave + 4 * lg + j) * D + 16 * ct + lr] = acc[j];
    }
}

// ---------------------------------------------------------------------------
// reverse carry: one workgroup (4 waves) per (b, h, 16-column slice), chunks in reverse
// ---------------------------------------------------------------------------
// The slice's state gradient dS' [D][16] lives in registers in the 16x16x32
// MFMA output layout: wave w holds rows D/4 w .. D/4 (w+1) - 1, lane (lr, lg)
// = (lane % 16, lane / 16) the rows 16 rt + 4 lg + jj of its row tiles rt at
// column lr.  Per chunk:
//   1. dS' (split) into LDS as [column][row]; dS' out to ds_end.   barrier A
//   2. Y = W^T dS' (wave w: token rows 16 w ..; 3 passes), dE = M^T dO + Y
//      out to dv; -gamma (.) dE and gamma (.) dO (split) into LDS as
//      [column][token].                                            barrier B
//   3. dS = gamma_C dS' + Q^T (gamma dO) - K^T (gamma dE) on the wave's rows.
// The next chunk's operands (W^T, K^T, Q^T fragments, M^T dO, dO, gamma) are
// loaded into registers one chunk ahead.
constexpr int BC_THREADS = 256;

template <int D, bool SPLIT_KQ>
struct BwdCarryOps {
    static constexpr int RT = D / 64;   // 16-row tiles of dS' per wave
    static constexpr int KS = D / 32;   // k-steps of W^T dS'
    bf16x8 wh[KS], wl[KS];              // W^T rows 16 w + lr, k = 32 s + 8 lg ..
    bf16x8 kh[RT][2], qh[RT][2];        // K^T, Q^T rows of the wave, k = m = 32 s + 8 lg ..
    bf16x8 kl[SPLIT_KQ ? RT : 1][2], ql[SPLIT_KQ ? RT : 1][2];
    float mt[4], od[4], g[4];           // M^T dO, dO and gamma at token rows 16 w + 4 lg + jj, column lr
    float gC;
};

template <int D, bool SPLIT_KQ>
__device__ __forceinline__ void bwd_carry_load(BwdCarryOps<D, SPLIT_KQ> &o, const BwdMats &bm, const float *d_o,
                                               int64_t cid, int64_t tok0, int nvalid, int H, int h, int col0,
                                               int wave, int lr, int lg) {
    using G = BwdCarryOps<D, SPLIT_KQ>;
    const int mrow = 16 * wave + lr;
#pragma unroll
    for (int s = 0; s < G::KS; ++s) {
        const int64_t off = (cid * C + mrow) * D + 32 * s + 8 * lg;
        o.wh[s] = *reinterpret_cast<const bf16x8 *>(bm.Wth + off);
        o.wl[s] = *reinterpret_cast<const bf16x8 *>(bm.Wtl + off);
    }
#pragma unroll
    for (int rt = 0; rt < G::RT; ++rt)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int i = (D / 4) * wave + 16 * rt + lr;
            const int64_t off = (cid * D + i) * C + 32 * s + 8 * lg;
            o.kh[rt][s] = *reinterpret_cast<const bf16x8 *>(bm.Kth + off);
            o.qh[rt][s] = *reinterpret_cast<const bf16x8 *>(bm.Qth + off);
            if constexpr (SPLIT_KQ) {
                o.kl[rt][s] = *reinterpret_cast<const bf16x8 *>(bm.Ktl + off);
                o.ql[rt][s] = *reinterpret_cast<const bf16x8 *>(bm.Qtl + off);
            }
        }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        const int m = 16 * wave + 4 * lg + jj;
        o.mt[jj] = bm.MtdO[(cid * C + m) * D + col0 + lr];
        o.od[jj] = m < nvalid ? d_o[((tok0 + m) * H + h) * D + col0 + lr] : 0.f;
        o.g[jj] = bm.gam[cid * C + m];
    }
    o.gC = bm.gam[cid * C + C - 1];
}

template <int D, typename TIn>
__global__ __launch_bounds__(BC_THREADS) void k_bwd_carry(const float *__restrict__ d_o, BwdMats bm,
                                                          const float *__restrict__ d_sfinal, int L, int H, int Nc,
                                                          float *__restrict__ dv, float *__restrict__ ds_end,
                                                          float *__restrict__ ds_init) {
    constexpr bool SPLIT_KQ = sizeof(TIn) == 4;
    using G = BwdCarryOps<D, SPLIT_KQ>;
    constexpr int SLD = D + 8, MLD = C + 8;          // LDS row strides (bf16): 16-byte aligned rows
    __shared__ bf16 dSh[16 * SLD], dSl[16 * SLD];    // dS' as [column][row]
    __shared__ bf16 gEh[16 * MLD], gEl[16 * MLD];    // -gamma (.) dE as [column][token]
    __shared__ bf16 gOh[16 * MLD], gOl[16 * MLD];    // gamma (.) dO as [column][token]
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6, lr = lane & 15, lg = lane >> 4;
    const int h = blockIdx.x, slice = blockIdx.y, b = blockIdx.z;
    const int col0 = slice * 16;
    const int64_t tokb = (int64_t)b * L;
    const int64_t cidb = ((int64_t)b * H + h) * Nc;
    const int64_t sbase = ((int64_t)b * H + h) * D * D;
    const int rbase = (D / 4) * wave;

    f32x4 dS[G::RT];
#pragma unroll
    for (int rt = 0; rt < G::RT; ++rt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int i = rbase + 16 * rt + 4 * lg + jj;
            dS[rt][jj] = d_sfinal ? d_sfinal[sbase + (int64_t)i * D + col0 + lr] : 0.f;
        }

    G ops[2];
    auto load = [&](G &o, int c) {
        bwd_carry_load<D, SPLIT_KQ>(o, bm, d_o, cidb + c, tokb + (int64_t)c * C, min(C, L - c * C), H, h, col0,
                                    wave, lr, lg);
    };
    auto step = [&](const G &o, int c) {
        const int64_t cid = cidb + c;
        const int c0 = c * C, nvalid = min(C, L - c0);
        // 1. dS' into LDS (split, transposed) and out
#pragma unroll
        for (int rt = 0; rt < G::RT; ++rt) {
            const float v[4] = {dS[rt][0], dS[rt][1], dS[rt][2], dS[rt][3]};
            bf16 hi[4], lo[4];
            split_bf16<4>(v, hi, lo);
            const int i = rbase + 16 * rt + 4 * lg;
            *reinterpret_cast<bf16x4 *>(dSh + lr * SLD + i) = pack4(hi);
            *reinterpret_cast<bf16x4 *>(dSl + lr * SLD + i) = pack4(lo);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) ds_end[(cid * D + i + jj) * D + col0 + lr] = v[jj];
        }
        lds_barrier();
        // 2. Y = W^T dS' for token rows 16 wave .., dE = M^T dO + Y
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < G::KS; ++s) {
            const bf16x8 bh = *reinterpret_cast<const bf16x8 *>(dSh + lr * SLD + 32 * s + 8 * lg);
            const bf16x8 bl = *reinterpret_cast<const bf16x8 *>(dSl + lr * SLD + 32 * s + 8 * lg);
            y = mfma16x16x32(o.wh[s], bh, y);
            y = mfma16x16x32(o.wh[s], bl, y);
            y = mfma16x16x32(o.wl[s], bh, y);
        }
        {
            float ge[4], go[4];
            bf16 eh[4], el[4], oh[4], ol[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int m = 16 * wave + 4 * lg + jj;
                const float de = o.mt[jj] + y[jj];
                if (m < nvalid) dv[((tokb + c0 + m) * H + h) * D + col0 + lr] = de;
                ge[jj] = -o.g[jj] * de;
                go[jj] = o.g[jj] * o.od[jj];
            }
            split_bf16<4>(ge, eh, el);
            split_bf16<4>(go, oh, ol);
            const int m0 = 16 * wave + 4 * lg;
            *reinterpret_cast<bf16x4 *>(gEh + lr * MLD + m0) = pack4(eh);
            *reinterpret_cast<bf16x4 *>(gEl + lr * MLD + m0) = pack4(el);
            *reinterpret_cast<bf16x4 *>(gOh + lr * MLD + m0) = pack4(oh);
            *reinterpret_cast<bf16x4 *>(gOl + lr * MLD + m0) = pack4(ol);
        }
        lds_barrier();
        // 3. dS = gamma_C dS' + Q^T (gamma dO) - K^T (gamma dE)
#pragma unroll
        for (int rt = 0; rt < G::RT; ++rt) {
            f32x4 acc;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) acc[jj] = o.gC * dS[rt][jj];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int mo = lr * MLD + 32 * s + 8 * lg;
                const bf16x8 oh = *reinterpret_cast<const bf16x8 *>(gOh + mo);
                const bf16x8 ol = *reinterpret_cast<const bf16x8 *>(gOl + mo);
                const bf16x8 eh = *reinterpret_cast<const bf16x8 *>(gEh + mo);
                const bf16x8 el = *reinterpret_cast<const bf16x8 *>(gEl + mo);
                acc = mfma16x16x32(o.qh[rt][s], oh, acc);
                acc = mfma16x16x32(o.qh[rt][s], ol, acc);
                acc = mfma16x16x32(o.kh[rt][s], eh, acc);
                acc = mfma16x16x32(o.kh[rt][s], el, acc);
                if constexpr (SPLIT_KQ) {
                    acc = mfma16x16x32(o.ql[rt][s], oh, acc);
                    acc = mfma16x16x32(o.kl[rt][s], eh, acc);
                }
            }
            dS[rt] = acc;
        }
    };

    load(ops[0], Nc - 1);
    for (int c = Nc - 1; c >= 0; c -= 2) {
        if (c >= 1) load(ops[1], c - 1);
        step(ops[0], c);
        if (c >= 1) {
            if (c >= 2) load(ops[0], c - 2);
            step(ops[1], c - 1);
        }
    }
    if (ds_init) {
#pragma unroll
        for (int rt = 0; rt < G::RT; ++rt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                ds_init[sbase + (int64_t)(rbase + 16 * rt + 4 * lg + jj) * D + col0 + lr] = dS[rt][jj];
    }
}

// ---------------------------------------------------------------------------
// per-chunk gradients: one workgroup (8 waves) per (b, h, chunk), on MFMA
// ---------------------------------------------------------------------------
// The columns j of S, dS', dO, dE are walked in blocks of 32.  Per block, wave
// w (row group rg = w % 4: token rows 16 rg .., column half hc = w / 4):
//   A. stage S and dS' of the block transposed ([j][i]) and as they are
//      ([i][j]), and dO transposed ([j][r]), in LDS as bf16 hi/lo planes;
//   B. K S, Q S, K dS' and P^T dO for its 16 x 16 tile on 16x16x32 MFMA, formed
//      transposed (a lane holds four consecutive columns of one token, so the
//      [token][column] planes take 8-byte stores), then E = V - diag(gamma) K S,
//      dU = P^T dO + diag(c) K dS', its share of dgamma; E (beta-scaled,
//      transposed; and as is), dU into LDS;
//   C. U = T diag(beta) E for its tile (transposed likewise), its share of dc;
//      U and diag(c) U into LDS;
//   D. accumulate dP += dO U^T, dTb += dU E^T (two 16 x 16 tiles each) and
//      dQ += diag(gamma) dO S^T, dK += -diag(gamma) dE S^T + diag(c) U dS'^T
//      (four 16-row x 16-column tiles each) in registers; the staging of A
//      also sums S (.) dS' (each element once).
// fp32 operands enter the MFMA as bf16 hi + lo (3 passes; 2 where one side is
// an exact bf16 input).  After the blocks: dP and dTb into LDS (fp32), the
// 64 x 64 products Y = T^T dT and dN = -Y T^T on MFMA (3 passes), dA, dbeta, then dQ +=
// (Gam (.) dP) K and dK += (Gam (.) dP)^T Q + (Gam (.) dA + (Gam (.) dA)^T) K on
// MFMA with K^T and Q^T from the carry operands, and the decay gradient.
constexpr int BK_THREADS = 512;

// 8 consecutive fp32 values (16-byte aligned) as bf16 hi and lo parts
__device__ __forceinline__ void ld_split8(const float *p, bf16x8 &hi, bf16x8 &lo) {
    const float4 a = *reinterpret_cast<const float4 *>(p), b = *reinterpret_cast<const float4 *>(p + 4);
    const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    bf16 h[8], l[8];
    split_bf16<8>(x, h, l);
    hi = pack8(h);
    lo = pack8(l);
}
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8 &hi, bf16x8 &lo) {
    bf16 h[8], l[8];
    split_bf16<8>(x, h, l);
    hi = pack8(h);
    lo = pack8(l);
}
// c += a.b with both sides as hi/lo parts (3 passes), or a exact (2 passes)
__device__ __forceinline__ f32x4 mm3(const bf16x8 &ah, const bf16x8 &al, const bf16x8 &bh, const bf16x8 &bl,
                                     f32x4 c) {
    c = mfma16x16x32(ah, bh, c);
    c = mfma16x16x32(ah, bl, c);
    return mfma16x16x32(al, bh, c);
}
__device__ __forceinline__ f32x4 mm2(const bf16x8 &a, const bf16x8 &bh, const bf16x8 &bl, f32x4 c) {
    c = mfma16x16x32(a, bh, c);
    return mfma16x16x32(a, bl, c);
}
// ... or with b exact
__device__ __forceinline__ f32x4 mm2b(const bf16x8 &ah, const bf16x8 &al, const bf16x8 &b, f32x4 c) {
    c = mfma16x16x32(ah, b, c);
    return mfma16x16x32(al, b, c);
}
// A fragment of an input row (K, Q): exact bf16, or fp32 split
template <typename TIn>
__device__ __forceinline__ void in_frag(const TIn *p, bf16x8 &hi, bf16x8 &lo) {
    if constexpr (sizeof(TIn) == 2) {
        hi = *reinterpret_cast<const bf16x8 *>(p);
    } else {
        ld_split8(reinterpret_cast<const float *>(p), hi, lo);
    }
}

template <int D, typename TIn>
__global__ __launch_bounds__(BK_THREADS) void k_bwd_chunk(
    const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v, const float *__restrict__ alpha,
    const float *__restrict__ beta, const float *__restrict__ d_o, const float *__restrict__ dvin,
    const float *__restrict__ s_chunks, const float *__restrict__ ds_end, BwdMats bm, int L, int H, int Nc,
    float *__restrict__ dq, float *__restrict__ dk, float *__restrict__ dalpha, float *__restrict__ dbeta) {
    constexpr bool F32 = sizeof(TIn) == 4;
    constexpr int JB = 32, NB = D / JB, KSD = D / 32;
    constexpr int SL = D + 8, ML = C + 8, JL = JB + 8;   // LDS row strides (bf16)
    constexpr int QT = D / 32;                           // 16-column i tiles per wave in dQ, dK
    static_assert((D / 4) * (JB / 4) + (C / 4) * (JB / 4) <= BK_THREADS, "staging threads");
    // block phase: bf16 planes
    constexpr int O_PT = 0, O_ST = O_PT + 2 * C * ML, O_DST = O_ST + 2 * JB * SL, O_DOT = O_DST + 2 * JB * SL,
                  O_ET = O_DOT + 2 * JB * ML, O_EN = O_ET + 2 * JB * ML, O_UN = O_EN + 2 * C * JL,
                  O_CU = O_UN + 2 * C * JL, O_DU = O_CU + 2 * C * JL, O_SN = O_DU + 2 * C * JL,
                  O_DSN = O_SN + 2 * D * JL, BLK_ELEMS = O_DSN + 2 * D * JL;
    // final phase: fp32 [64][65] matrices over the same memory
    constexpr int FL = C + 1, MAT = C * FL, FIN_FLOATS = 6 * MAT + 10 * C;   // six matrices, then sum partials
    constexpr int LDS_BYTES = (BLK_ELEMS * 2 > FIN_FLOATS * 4) ? BLK_ELEMS * 2 : FIN_FLOATS * 4;
    __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];
    bf16 *pl = reinterpret_cast<bf16 *>(smem);
    float *fm = reinterpret_cast<float *>(smem);
    float *Ts = fm, *As = fm + MAT, *Ps = fm + 2 * MAT, *Gs = fm + 3 * MAT, *dPs = fm + 4 * MAT, *dXs = fm + 5 * MAT;
    float *part = fm + 6 * MAT, *part2 = part + 8 * C;   // [8][C] and [2][C] partial sums
    __shared__ double lgs[C];
    __shared__ float gam[C], cr[C], bes[C], als[C], dgam2[2][C], dcr2[2][C], dbn[C], dlg[C], dbp[C], sdd[8];

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6, lr = lane & 15, lg = lane >> 4;
    const int rg = wave & 3, hc = wave >> 2;
    const int h = blockIdx.x % H, chunk = blockIdx.x / H, b = blockIdx.y;
    const int c0 = chunk * C, nvalid = min(C, L - c0);
    const int64_t tok0 = (int64_t)b * L + c0;
    const int64_t cid = ((int64_t)b * H + h) * Nc + chunk;
    const int64_t rs = (int64_t)H * D;   // elements between consecutive tokens of q, k, v, dO, dE
    const TIn *kb = k + (tok0 * H + h) * D, *qb = q + (tok0 * H + h) * D, *vb = v + (tok0 * H + h) * D;
    const float *dob = d_o + (tok0 * H + h) * D, *deb = dvin + (tok0 * H + h) * D;
    const float *Sg = s_chunks + cid * D * D, *dSg = ds_end + cid * D * D;

    // P^T into LDS (split) and the chunk's scalars; P by 4 x 4 blocks (rows 4 r4 .., columns 4 m4 ..), so
    // that each transposed row piece is one 8-byte store
    if (t < (C / 4) * (C / 4)) {
        const int r4 = (t & 7) + 8 * ((t >> 6) & 1), m4 = ((t >> 3) & 7) + 8 * (t >> 7);
        float x[4][4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const float4 p4 = *reinterpret_cast<const float4 *>(bm.P + cid * C * C + (4 * r4 + rr) * C + 4 * m4);
            x[0][rr] = p4.x; x[1][rr] = p4.y; x[2][rr] = p4.z; x[3][rr] = p4.w;
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            bf16 hh[4], ll[4];
            split_bf16<4>(x[c], hh, ll);
            *reinterpret_cast<bf16x4 *>(pl + O_PT + (4 * m4 + c) * ML + 4 * r4) = pack4(hh);
            *reinterpret_cast<bf16x4 *>(pl + O_PT + C * ML + (4 * m4 + c) * ML + 4 * r4) = pack4(ll);
        }
    }
    if (t < C) {
        const bool ok = t < nvalid;
        const int64_t gi = (tok0 + (ok ? t : 0)) * H + h;
        als[t] = ok ? alpha[gi] : 1.f;
        bes[t] = ok ? beta[gi] : 0.f;
        lgs[t] = bm.lg[cid * C + t];
        gam[t] = bm.gam[cid * C + t];
        cr[t] = bm.c[cid * C + t];
    }
    __syncthreads();

    const int ra = 16 * rg + lr;                 // this lane's A row in the row-group products
    const bool ra_ok = ra < nvalid;
    f32x4 dPa[2], dTa[2], dQa[QT], dKa[QT];
#pragma unroll
    for (int x = 0; x < 2; ++x) dPa[x] = dTa[x] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int x = 0; x < QT; ++x) dQa[x] = dKa[x] = f32x4{0.f, 0.f, 0.f, 0.f};
    float dgacc = 0.f, dcacc = 0.f, sdacc = 0.f;   // this lane's token ra: its dgamma, dc shares
    const bf16x8 z8 = {};

    for (int jb = 0; jb < NB; ++jb) {
        const int j0 = jb * JB;
        // A. S, dS' as they are ([i][j]) and transposed ([j][i]), and dO transposed ([j][r]), split, by 4 x 4
        // blocks (rows 4 i4 .., columns 4 qd ..): every plane row piece is one 8-byte store
        if (t < (D / 4) * (JB / 4)) {
            const int i4 = (t & 7) + 8 * (t >> 6), qd = (t >> 3) & 7;
            float xs[4][4], xd[4][4];   // [column c][row rr]
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int64_t o = (int64_t)(4 * i4 + rr) * D + j0 + 4 * qd;
                const float4 sv = *reinterpret_cast<const float4 *>(Sg + o);
                const float4 dv = *reinterpret_cast<const float4 *>(dSg + o);
                const float sr[4] = {sv.x, sv.y, sv.z, sv.w}, dr[4] = {dv.x, dv.y, dv.z, dv.w};
                bf16 sh[4], sl[4], dh[4], dl[4];
                split_bf16<4>(sr, sh, sl);
                split_bf16<4>(dr, dh, dl);
                const int i = 4 * i4 + rr;
                *reinterpret_cast<bf16x4 *>(pl + O_SN + i * JL + 4 * qd) = pack4(sh);
                *reinterpret_cast<bf16x4 *>(pl + O_SN + D * JL + i * JL + 4 * qd) = pack4(sl);
                *reinterpret_cast<bf16x4 *>(pl + O_DSN + i * JL + 4 * qd) = pack4(dh);
                *reinterpret_cast<bf16x4 *>(pl + O_DSN + D * JL + i * JL + 4 * qd) = pack4(dl);
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    xs[c][rr] = sr[c];
                    xd[c][rr] = dr[c];
                    sdacc = fmaf(sr[c], dr[c], sdacc);
                }
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                bf16 sh[4], sl[4], dh[4], dl[4];
                split_bf16<4>(xs[c], sh, sl);
                split_bf16<4>(xd[c], dh, dl);
                const int j = 4 * qd + c;
                *reinterpret_cast<bf16x4 *>(pl + O_ST + j * SL + 4 * i4) = pack4(sh);
                *reinterpret_cast<bf16x4 *>(pl + O_ST + JB * SL + j * SL + 4 * i4) = pack4(sl);
                *reinterpret_cast<bf16x4 *>(pl + O_DST + j * SL + 4 * i4) = pack4(dh);
                *reinterpret_cast<bf16x4 *>(pl + O_DST + JB * SL + j * SL + 4 * i4) = pack4(dl);
            }
        } else if (t >= BK_THREADS - (C / 4) * (JB / 4)) {
            // dO of the block's columns, transposed, by 4 x 4 blocks (tokens 4 r4 .., columns 4 qd ..)
            const int u = t - (BK_THREADS - (C / 4) * (JB / 4));
            const int r4 = (u & 7) + 8 * (u >> 6), qd = (u >> 3) & 7;
            float xo[4][4];   // [column c][token rr]
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int r = 4 * r4 + rr;
                float4 ov = {0.f, 0.f, 0.f, 0.f};
                if (r < nvalid) ov = *reinterpret_cast<const float4 *>(dob + r * rs + j0 + 4 * qd);
                xo[0][rr] = ov.x; xo[1][rr] = ov.y; xo[2][rr] = ov.z; xo[3][rr] = ov.w;
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                bf16 oh[4], ol[4];
                split_bf16<4>(xo[c], oh, ol);
                *reinterpret_cast<bf16x4 *>(pl + O_DOT + (4 * qd + c) * ML + 4 * r4) = pack4(oh);
                *reinterpret_cast<bf16x4 *>(pl + O_DOT + JB * ML + (4 * qd + c) * ML + 4 * r4) = pack4(ol);
            }
        }
        __syncthreads();
        // B. tile (columns j0 + 16 hc .., tokens 16 rg ..), formed transposed so that a lane holds four
        // consecutive columns of one token: (K S)^T, (Q S)^T, (K dS')^T, (P^T dO)^T
        const int jl = 16 * hc + lr;   // this lane's A row (a column j) within the block
        f32x4 ks = {0.f, 0.f, 0.f, 0.f}, qs = ks, kd = ks, pd = ks;
#pragma unroll
        for (int s = 0; s < KSD; ++s) {
            const int kk = 32 * s + 8 * lg;
            bf16x8 kh = z8, kl = z8, qh = z8, ql = z8;
            if (ra_ok) {
                in_frag<TIn>(kb + ra * rs + kk, kh, kl);
                in_frag<TIn>(qb + ra * rs + kk, qh, ql);
            }
            const bf16x8 sh = *reinterpret_cast<const bf16x8 *>(pl + O_ST + jl * SL + kk);
            const bf16x8 sl = *reinterpret_cast<const bf16x8 *>(pl + O_ST + JB * SL + jl * SL + kk);
            const bf16x8 dh = *reinterpret_cast<const bf16x8 *>(pl + O_DST + jl * SL + kk);
            const bf16x8 dl = *reinterpret_cast<const bf16x8 *>(pl + O_DST + JB * SL + jl * SL + kk);
            ks = mm2b(sh, sl, kh, ks);
            qs = mm2b(sh, sl, qh, qs);
            kd = mm2b(dh, dl, kh, kd);
            if constexpr (F32) {
                ks = mfma16x16x32(sh, kl, ks);
                qs = mfma16x16x32(sh, ql, qs);
                kd = mfma16x16x32(dh, kl, kd);
            }
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int kk = 32 * s + 8 * lg;
            const bf16x8 ah = *reinterpret_cast<const bf16x8 *>(pl + O_DOT + jl * ML + kk);
            const bf16x8 al = *reinterpret_cast<const bf16x8 *>(pl + O_DOT + JB * ML + jl * ML + kk);
            const bf16x8 bh = *reinterpret_cast<const bf16x8 *>(pl + O_PT + ra * ML + kk);
            const bf16x8 bl = *reinterpret_cast<const bf16x8 *>(pl + O_PT + C * ML + ra * ML + kk);
            pd = mm3(ah, al, bh, bl, pd);
        }
        // element jj: column j = j0 + jq + jj (jq = 16 hc + 4 lg), token r = ra
        const int jq = 16 * hc + 4 * lg;
        {
            float vv[4] = {0.f, 0.f, 0.f, 0.f}, od[4] = {0.f, 0.f, 0.f, 0.f}, de[4] = {0.f, 0.f, 0.f, 0.f};
            if (ra_ok) {
                const float4 o4 = *reinterpret_cast<const float4 *>(dob + ra * rs + j0 + jq);
                const float4 e4 = *reinterpret_cast<const float4 *>(deb + ra * rs + j0 + jq);
                od[0] = o4.x; od[1] = o4.y; od[2] = o4.z; od[3] = o4.w;
                de[0] = e4.x; de[1] = e4.y; de[2] = e4.z; de[3] = e4.w;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) vv[jj] = to_f32(vb[ra * rs + j0 + jq + jj]);
            }
            const float gr = gam[ra], br = bes[ra], cg = cr[ra];
            float ev[4], bev[4], du[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                ev[jj] = vv[jj] - gr * ks[jj];
                bev[jj] = br * ev[jj];
                du[jj] = pd[jj] + cg * kd[jj];
                dgacc = fmaf(od[jj], qs[jj], fmaf(-de[jj], ks[jj], dgacc));
            }
            bf16 eh[4], el[4], nh[4], nl[4], uh[4], ul[4];
            split_bf16<4>(bev, eh, el);
            split_bf16<4>(ev, nh, nl);
            split_bf16<4>(du, uh, ul);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                pl[O_ET + (jq + jj) * ML + ra] = eh[jj];
                pl[O_ET + JB * ML + (jq + jj) * ML + ra] = el[jj];
            }
            *reinterpret_cast<bf16x4 *>(pl + O_EN + ra * JL + jq) = pack4(nh);
            *reinterpret_cast<bf16x4 *>(pl + O_EN + C * JL + ra * JL + jq) = pack4(nl);
            *reinterpret_cast<bf16x4 *>(pl + O_DU + ra * JL + jq) = pack4(uh);
            *reinterpret_cast<bf16x4 *>(pl + O_DU + C * JL + ra * JL + jq) = pack4(ul);
        }
        __syncthreads();
        // C. U^T = (diag(beta) E)^T T^T for the tile; dc; U and diag(c) U into LDS
        {
            f32x4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int kk = 32 * s + 8 * lg;
                bf16x8 bh, bl;
                ld_split8(bm.T + cid * C * C + ra * C + kk, bh, bl);
                const bf16x8 ah = *reinterpret_cast<const bf16x8 *>(pl + O_ET + jl * ML + kk);
                const bf16x8 al = *reinterpret_cast<const bf16x8 *>(pl + O_ET + JB * ML + jl * ML + kk);
                u = mm3(ah, al, bh, bl, u);
            }
            float uv[4], cu[4];
            const float cg = cr[ra];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                uv[jj] = u[jj];
                cu[jj] = cg * u[jj];
                dcacc = fmaf(u[jj], kd[jj], dcacc);
            }
            bf16 uh[4], ul[4], ch[4], cl[4];
            split_bf16<4>(uv, uh, ul);
            split_bf16<4>(cu, ch, cl);
            *reinterpret_cast<bf16x4 *>(pl + O_UN + ra * JL + jq) = pack4(uh);
            *reinterpret_cast<bf16x4 *>(pl + O_UN + C * JL + ra * JL + jq) = pack4(ul);
            *reinterpret_cast<bf16x4 *>(pl + O_CU + ra * JL + jq) = pack4(ch);
            *reinterpret_cast<bf16x4 *>(pl + O_CU + C * JL + ra * JL + jq) = pack4(cl);
        }
        __syncthreads();
        // D. accumulate (k = the block's 32 columns j: one MFMA k-step)
        {
            const int kk = 8 * lg;
            // A rows ra: gamma dO, -gamma dE (fp32, split), dU, diag(c) U (LDS)
            float od8[8] = {}, de8[8] = {};
            if (ra_ok) {
                const float4 o0 = *reinterpret_cast<const float4 *>(dob + ra * rs + j0 + kk);
                const float4 o1 = *reinterpret_cast<const float4 *>(dob + ra * rs + j0 + kk + 4);
                const float4 e0 = *reinterpret_cast<const float4 *>(deb + ra * rs + j0 + kk);
                const float4 e1 = *reinterpret_cast<const float4 *>(deb + ra * rs + j0 + kk + 4);
                const float og[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
                const float eg[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    od8[e] = og[e];
                    de8[e] = eg[e];
                }
            }
            bf16x8 oh, ol, goh, gol, geh, gel;
            split8(od8, oh, ol);
            {
                float go[8], ge[8];
                const float gr = gam[ra];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    go[e] = gr * od8[e];
                    ge[e] = -gr * de8[e];
                }
                split8(go, goh, gol);
                split8(ge, geh, gel);
            }
            const bf16x8 duh = *reinterpret_cast<const bf16x8 *>(pl + O_DU + ra * JL + kk);
            const bf16x8 dul = *reinterpret_cast<const bf16x8 *>(pl + O_DU + C * JL + ra * JL + kk);
            const bf16x8 cuh = *reinterpret_cast<const bf16x8 *>(pl + O_CU + ra * JL + kk);
            const bf16x8 cul = *reinterpret_cast<const bf16x8 *>(pl + O_CU + C * JL + ra * JL + kk);
            // dP += dO U^T, dTb += dU E^T: m tiles 2 hc, 2 hc + 1
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const int mrow = 16 * (2 * hc + x) + lr;
                const bf16x8 ubh = *reinterpret_cast<const bf16x8 *>(pl + O_UN + mrow * JL + kk);
                const bf16x8 ubl = *reinterpret_cast<const bf16x8 *>(pl + O_UN + C * JL + mrow * JL + kk);
                const bf16x8 ebh = *reinterpret_cast<const bf16x8 *>(pl + O_EN + mrow * JL + kk);
                const bf16x8 ebl = *reinterpret_cast<const bf16x8 *>(pl + O_EN + C * JL + mrow * JL + kk);
                dPa[x] = mm3(oh, ol, ubh, ubl, dPa[x]);
                dTa[x] = mm3(duh, dul, ebh, ebl, dTa[x]);
            }
            // dQ += (gamma dO) S^T, dK += (-gamma dE) S^T + (c U) dS'^T: i tiles QT hc ..
#pragma unroll
            for (int x = 0; x < QT; ++x) {
                const int irow = 16 * (QT * hc + x) + lr;
                const bf16x8 sh = *reinterpret_cast<const bf16x8 *>(pl + O_SN + irow * JL + kk);
                const bf16x8 sl = *reinterpret_cast<const bf16x8 *>(pl + O_SN + D * JL + irow * JL + kk);
                const bf16x8 dh = *reinterpret_cast<const bf16x8 *>(pl + O_DSN + irow * JL + kk);
                const bf16x8 dl = *reinterpret_cast<const bf16x8 *>(pl + O_DSN + D * JL + irow * JL + kk);
                dQa[x] = mm3(goh, gol, sh, sl, dQa[x]);
                dKa[x] = mm3(geh, gel, sh, sl, dKa[x]);
                dKa[x] = mm3(cuh, cul, dh, dl, dKa[x]);
            }
        }
        __syncthreads();   // the next block restages every plane
    }

    // per-token sums of this wave's dgamma and dc shares (the four lane groups lg hold token ra's columns)
    {
        float g = dgacc, cc = dcacc;
        g += __shfl_xor(g, 16, 64);
        cc += __shfl_xor(cc, 16, 64);
        g += __shfl_xor(g, 32, 64);
        cc += __shfl_xor(cc, 32, 64);
        if (lg == 0) {
            dgam2[hc][ra] = g;
            dcr2[hc][ra] = cc;
        }
    }
    {
        float v2 = sdacc;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) v2 += __shfl_xor(v2, off, 64);
        if (lane == 0) sdd[wave] = v2;
    }
    // dP (lower incl) and dTb into LDS fp32; T, A, P, Gam for the 64 x 64 steps
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int r = 16 * rg + 4 * lg + jj, m = 16 * (2 * hc + x) + lr;
            dPs[r * FL + m] = m <= r ? dPa[x][jj] : 0.f;
            dXs[r * FL + m] = dTa[x][jj];
        }
    for (int n = t; n < C * C; n += BK_THREADS) {
        const int r = n / C, m = n % C;
        Ts[r * FL + m] = bm.T[cid * C * C + n];
        As[r * FL + m] = bm.A[cid * C * C + n];
        Ps[r * FL + m] = bm.P[cid * C * C + n];
        Gs[r * FL + m] = m <= r ? (float)exp(lgs[r] - lgs[m]) : 0.f;
    }
    __syncthreads();
    // dbeta part 1 (from Tb = T diag(beta)): sum_r dTb_rm T_rm, over 8 row groups of 8
    {
        const int m = t & 63, g = t >> 6;
        float sp = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) sp = fmaf(dXs[(8 * g + e) * FL + m], Ts[(8 * g + e) * FL + m], sp);
        part[g * C + m] = sp;
    }
    // Y = T^T dT with dT = dTb diag(beta), on MFMA (3 passes).  Wave w: row tile w % 4 of Y,
    // column tiles 2 (w / 4) + {0, 1}; T is lower triangular, so its zeros bound the sums.
    const int yr = wave & 3, yc = 2 * (wave >> 2);
    f32x4 yacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int kk = 32 * s + 8 * lg;
        float a8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) a8[e] = Ts[(kk + e) * FL + 16 * yr + lr];
        bf16x8 ah, al;
        split8(a8, ah, al);
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            const int m = 16 * (yc + x) + lr;
            float b8[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) b8[e] = dXs[(kk + e) * FL + m] * bes[m];
            bf16x8 bh, bl;
            split8(b8, bh, bl);
            yacc[x] = mm3(ah, al, bh, bl, yacc[x]);
        }
    }
    __syncthreads();   // dTb read by every wave; Y replaces it
    if (t < C) {
        float sp = 0.f;
#pragma unroll
        for (int g = 0; g < 8; ++g) sp += part[g * C + t];
        dbp[t] = sp;
    }
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) dXs[(16 * yr + 4 * lg + jj) * FL + 16 * (yc + x) + lr] = yacc[x][jj];
    __syncthreads();
    // dN = -(Y T^T) strictly below the diagonal (T's zeros bound the sums), same tiles;
    // dA = diag(beta) dN; dbeta part 2: sum_i dN_ri A_ri
    f32x4 nacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int kk = 32 * s + 8 * lg;
        float a8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) a8[e] = dXs[(16 * yr + lr) * FL + kk + e];
        bf16x8 ah, al;
        split8(a8, ah, al);
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            const int i = 16 * (yc + x) + lr;
            float b8[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) b8[e] = Ts[i * FL + kk + e];
            bf16x8 bh, bl;
            split8(b8, bh, bl);
            nacc[x] = mm3(ah, al, bh, bl, nacc[x]);
        }
    }
    __syncthreads();   // Y read by every wave; dA replaces it
    {
        float p2[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int r = 16 * yr + 4 * lg + jj, i = 16 * (yc + x) + lr;
                const float dn = i < r ? -nacc[x][jj] : 0.f;
                dXs[r * FL + i] = bes[r] * dn;
                p2[jj] = fmaf(dn, As[r * FL + i], p2[jj]);
            }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) p2[jj] += __shfl_xor(p2[jj], off, 64);
            if (lr == 0) part2[(wave >> 2) * C + 16 * yr + 4 * lg + jj] = p2[jj];
        }
    }
    __syncthreads();
    if (t < C) dbn[t] = part2[t] + part2[C + t];
    // dQ += (Gam (.) dP) K;  dK += (Gam (.) dP)^T Q + (Gam (.) dA + (Gam (.) dA)^T) K   (k = m, 64)
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int kk = 32 * s + 8 * lg;
        float xp[8], xpt[8], xa[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int m = kk + e;
            xp[e] = Gs[ra * FL + m] * dPs[ra * FL + m];
            xpt[e] = Gs[m * FL + ra] * dPs[m * FL + ra];
            xa[e] = Gs[ra * FL + m] * dXs[ra * FL + m] + Gs[m * FL + ra] * dXs[m * FL + ra];
        }
        bf16x8 ph, pl8, pth, ptl, ah, al;
        split8(xp, ph, pl8);
        split8(xpt, pth, ptl);
        split8(xa, ah, al);
#pragma unroll
        for (int x = 0; x < QT; ++x) {
            const int irow = 16 * (QT * hc + x) + lr;
            const int64_t off = (cid * D + irow) * C + kk;
            const bf16x8 kth = *reinterpret_cast<const bf16x8 *>(bm.Kth + off);
            const bf16x8 qth = *reinterpret_cast<const bf16x8 *>(bm.Qth + off);
            dQa[x] = mm2b(ph, pl8, kth, dQa[x]);
            dKa[x] = mm2b(pth, ptl, qth, dKa[x]);
            dKa[x] = mm2b(ah, al, kth, dKa[x]);
            if constexpr (F32) {
                const bf16x8 ktl = *reinterpret_cast<const bf16x8 *>(bm.Ktl + off);
                const bf16x8 qtl = *reinterpret_cast<const bf16x8 *>(bm.Qtl + off);
                dQa[x] = mfma16x16x32(ph, ktl, dQa[x]);
                dKa[x] = mfma16x16x32(pth, qtl, dKa[x]);
                dKa[x] = mfma16x16x32(ah, ktl, dKa[x]);
            }
        }
    }
    // The decay gradient.  gamma_r depends on log alpha_m for m <= r, Gam_ab for b < m <= a, c_r for
    // r < m, gamma_C on all m, so
    //     dlog alpha_m = sum_{r >= m} gamma_r dgamma_r + sum_{a >= m > b} (A (.) dA + P (.) dP)_ab
    //                    + sum_{r < m} c_r dc_r + gamma_C dgamma_C,
    // each term a sum of the contributions that actually depend on alpha_m (no cancelling pairs).
    // The middle sum as prefix sums: R[a][m] = sum_{b < m} (A (.) dA + P (.) dP)_ab by rows (into the Gam
    // matrix's memory, read for the last time above), then sum_{a >= m} R[a][m] per m.
    __syncthreads();
    float *Rs = Gs;
    {
        // row a by 8 threads of 8 columns: the row's exclusive prefix sums of Z = A (.) dA + P (.) dP
        const int a = t >> 3, q = t & 7;
        float z[8], tot = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int m = 8 * q + e;
            z[e] = As[a * FL + m] * dXs[a * FL + m] + Ps[a * FL + m] * dPs[a * FL + m];
            tot += z[e];
        }
        float inc = tot;
#pragma unroll
        for (int off = 1; off < 8; off <<= 1) {
            const float y = __shfl_up(inc, off, 8);
            if (q >= off) inc += y;
        }
        float run = inc - tot;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            Rs[a * FL + 8 * q + e] = run;
            run += z[e];
        }
    }
    __syncthreads();
    {
        // sum_{a >= m} R[a][m] over 8 row groups of 8
        const int m = t & 63, g = t >> 6;
        float sp = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int a = 8 * g + e;
            if (a >= m) sp += Rs[a * FL + m];
        }
        part[g * C + m] = sp;
    }
    __syncthreads();
    if (t < C) {
        // wave 0, lane m: sum_{r >= m} gamma_r dgamma_r and sum_{r < m} c_r dc_r as scans over the lanes
        const int m = t;
        float s2 = 0.f;
#pragma unroll
        for (int g = 0; g < 8; ++g) s2 += part[g * C + m];
        float dgCt = 0.f;
        for (int w = 0; w < BK_THREADS / 64; ++w) dgCt += sdd[w];
        const float g1 = gam[m] * (dgam2[0][m] + dgam2[1][m]);
        const float c3 = cr[m] * (dcr2[0][m] + dcr2[1][m]);
        float s1 = g1, p3 = c3;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float yd = __shfl_down(s1, off, 64), yu = __shfl_up(p3, off, 64);
            if (m + off < 64) s1 += yd;
            if (m >= off) p3 += yu;
        }
        dlg[m] = s1 + s2 + (p3 - c3) + gam[C - 1] * dgCt;
    }
    __syncthreads();
    if (t < C && t < nvalid) {
        const int64_t gi = (tok0 + t) * H + h;
        dalpha[gi] = dlg[t] / als[t];
        dbeta[gi] = dbp[t] + dbn[t];
    }
    // dQ, dK: element jj of lane (lr, lg) in tile x is row r = 16 rg + 4 lg + jj, column i = 16 (QT hc + x) + lr
#pragma unroll
    for (int x = 0; x < QT; ++x)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int r = 16 * rg + 4 * lg + jj, i = 16 * (QT * hc + x) + lr;
            if (r < nvalid) {
                const int64_t o = ((tok0 + r) * H + h) * D + i;
                dq[o] = dQa[x][jj];
                dk[o] = dKa[x][jj];
            }
        }
}

}  // namespace

PrepBwd bwd_prep_out(float *mats, int64_t chunks, int D) {
    const BwdMats bm = bwd_mats(mats, chunks, D);
    return PrepBwd{bm.T, bm.P, bm.A, bm.lg, bm.gam, bm.c, bm.Wth, bm.Wtl, bm.Kth, bm.Ktl, bm.Qth, bm.Qtl, bm.Mt};
}

hipError_t launch_bwd_ops(int B, int L, int H, int D, const float *d_o, float *mats, hipStream_t s) {
    const int Nc = (L + C - 1) / C;
    const dim3 grid((unsigned)(Nc * H), B);
    const BwdMats bm = bwd_mats(mats, (int64_t)B * H * Nc, D);
    if (D == 128) launch_kernel(k_bwd_ops<128>, grid, dim3(BO_THREADS), 0, s, d_o, L, H, Nc, bm);
    else if (D == 64) launch_kernel(k_bwd_ops<64>, grid, dim3(BO_THREADS), 0, s, d_o, L, H, Nc, bm);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_bwd_carry(bool f32, int B, int L, int H, int D, const float *d_o, const float *d_sfinal,
                            float *mats, float *dv, float *ds_end, float *ds_init, hipStream_t s) {
    const int Nc = (L + C - 1) / C;
    const dim3 grid(H, D / 16, B);
    const BwdMats bm = bwd_mats(mats, (int64_t)B * H * Nc, D);
#define BC(DD, T)                                                                                    \
    launch_kernel((k_bwd_carry<DD, T>), grid, dim3(BC_THREADS), 0, s, d_o, bm, d_sfinal, L, H, Nc, dv, ds_end, ds_init)
    if (f32) {
        if (D == 64) BC(64, float); else return hipErrorInvalidValue;
    } else {
        if (D == 128) BC(128, bf16); else BC(64, bf16);
    }
#undef BC
    return hipGetLastError();
}

hipError_t launch_bwd_chunk(bool f32, int B, int L, int H, int D, const void *q, const void *k, const void *v,
                            const float *alpha, const float *beta, const float *d_o, const float *dv,
                            const float *s_chunks, const float *ds_end, float *mats, float *dq, float *dk,
                            float *dalpha, float *dbeta, hipStream_t s) {
    const int Nc = (L + C - 1) / C;
    const dim3 grid((unsigned)(Nc * H), B);
    const BwdMats bm = bwd_mats(mats, (int64_t)B * H * Nc, D);
#define BK(DD, T)                                                                                    \
    launch_kernel((k_bwd_chunk<DD, T>), grid, dim3(BK_THREADS), 0, s, (const T *)q, (const T *)k, (const T *)v, \
                  alpha, beta, d_o, dv, s_chunks, ds_end, bm, L, H, Nc, dq, dk, dalpha, dbeta)
    if (f32) {
        if (D == 64) BK(64, float); else return hipErrorInvalidValue;
    } else {
        if (D == 128) BK(128, bf16); else BK(64, bf16);
    }
#undef BK
    return hipGetLastError();
}

size_t bwd_mats_bytes(int64_t chunks, int D) { return (size_t)chunks * bwd_mats_per_chunk(D); }

}  // namespace gdn
