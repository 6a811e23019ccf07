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
// over column slices of S, from the fp32 T, P, gamma, c that k_bwd_prep forms
// per chunk), and per chunk, in parallel (k_bwd_chunk):
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
// so they contribute nothing.  Everything here is fp32 VALU arithmetic.
#include "gdn_device.h"
#include "gdn_kernels.h"

namespace gdn {

namespace {

constexpr int C = 64;

// Per-chunk matrices of the backward, fp32: T, P, A [64][64] row-major, the
// log-cumsum lg [64] (fp64), gamma = e^lg and c = e^(lg_last - lg) [64]; and
// the operands of the reverse carry: W^T = diag(beta) T^T diag(c) K [64][D]
// as bf16 hi and lo planes, K^T and Q^T [D][64] as bf16 hi (and, for fp32
// inputs, lo) planes, and M^T dO = diag(beta) T^T P^T dO [64][D] fp32.
struct BwdMats {
    float *T, *P, *A;
    double *lg;
    float *gam, *c;
    bf16 *Wth, *Wtl, *Kth, *Ktl, *Qth, *Qtl;
    float *MtdO;
};
// bytes per chunk
__host__ __device__ constexpr size_t bwd_mats_per_chunk(int D) {
    return 3 * C * C * 4 + C * 8 + 2 * C * 4 + (size_t)6 * D * C * 2 + (size_t)C * D * 4;
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
    return m;
}

// ---------------------------------------------------------------------------
// backward prep: one workgroup per (b, h, chunk)
// ---------------------------------------------------------------------------
constexpr int BP_THREADS = 256;

template <int D, typename TIn>
__global__ __launch_bounds__(BP_THREADS) void k_bwd_prep(const TIn *__restrict__ q, const TIn *__restrict__ k,
                                                         const float *__restrict__ alpha,
                                                         const float *__restrict__ beta, int L, int H, int Nc,
                                                         BwdMats bm) {
    __shared__ TIn Ks[C][D], Qs[C][D];
    __shared__ float As[C][C + 1], bes[C];
    __shared__ double lgs[C];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int h = blockIdx.x % H, chunk = blockIdx.x / H, b = blockIdx.y;
    const int c0 = chunk * C, nvalid = min(C, L - c0);
    const int64_t tok0 = (int64_t)b * L + c0;
    const int64_t cid = ((int64_t)b * H + h) * Nc + chunk;
    for (int n = t; n < C * D; n += BP_THREADS) {
        const int r = n / D, i = n % D;
        const bool ok = r < nvalid;
        const int64_t off = ((tok0 + (ok ? r : 0)) * H + h) * D + i;
        Ks[r][i] = ok ? k[off] : from_f32<TIn>(0.f);
        Qs[r][i] = ok ? q[off] : from_f32<TIn>(0.f);
    }
    if (wave == 0) {
        // log-cumsum of alpha in fp64 (tokens past the end: alpha = 1, beta = 0)
        const bool ok = lane < nvalid;
        const int64_t gi = (tok0 + (ok ? lane : 0)) * H + h;
        const float a = ok ? alpha[gi] : 1.f;
        bes[lane] = ok ? beta[gi] : 0.f;
        double x = log((double)fmaxf(a, 1e-37f));
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const double y = __shfl_up(x, off, 64);
            if (lane >= off) x += y;
        }
        lgs[lane] = x;
        const double last = __shfl(x, 63, 64);
        bm.lg[cid * C + lane] = x;
        bm.gam[cid * C + lane] = (float)exp(x);
        bm.c[cid * C + lane] = (float)exp(last - x);
    }
    __syncthreads();
    // A = strict_lower(Gam (.) K K^T), P = lower_incl(Gam (.) Q K^T)
    float *Ag = bm.A + cid * C * C, *Pg = bm.P + cid * C * C, *Tg = bm.T + cid * C * C;
    for (int n = t; n < C * C; n += BP_THREADS) {
        const int r = n / C, i = n % C;
        float kk = 0.f, qk = 0.f;
        if (i <= r) {
            for (int e = 0; e < D; ++e) {
                const float ki = to_f32(Ks[i][e]);
                kk = fmaf(to_f32(Ks[r][e]), ki, kk);
                qk = fmaf(to_f32(Qs[r][e]), ki, qk);
            }
        }
        const float gm = i <= r ? (float)exp(lgs[r] - lgs[i]) : 0.f;
        const float av = i < r ? gm * kk : 0.f;
        As[r][i] = av;
        Ag[n] = av;
        Pg[n] = i <= r ? gm * qk : 0.f;
    }
    __syncthreads();
    // T = (I + diag(beta) A)^{-1}: column cc by forward substitution
    if (t < C) {
        const int cc = t;
        float tcol[C];
#pragma unroll
        for (int r = 0; r < C; ++r) {
            float v = r == cc ? 1.f : 0.f;
            if (r > cc) {
                float s = 0.f;
#pragma unroll
                for (int i = 0; i < r; ++i)
                    if (i >= cc) s = fmaf(As[r][i], tcol[i], s);
                v = -bes[r] * s;
            }
            tcol[r] = v;
            Tg[r * C + cc] = v;
        }
    }
}

// ---------------------------------------------------------------------------
// carry operands: one workgroup per (b, h, chunk), in 32-column blocks
// ---------------------------------------------------------------------------
// W^T[m][i] = beta_m sum_{r >= m} T[r][m] c_r K[r][i], (P^T dO)[m][i] =
// sum_{r >= m} P[r][m] dO[r][i], M^T dO[m][i] = beta_m sum_{r >= m} T[r][m]
// (P^T dO)[r][i]; K^T and Q^T copied transposed.  Rows past the end of the
// sequence are zero (beta = 0 there).
constexpr int BO_THREADS = 256;

template <int D, typename TIn>
__global__ __launch_bounds__(BO_THREADS) void k_bwd_ops(const TIn *__restrict__ q, const TIn *__restrict__ k,
                                                        const float *__restrict__ beta, const float *__restrict__ d_o,
                                                        int L, int H, int Nc, BwdMats bm) {
    constexpr bool SPLIT_KQ = sizeof(TIn) == 4;
    __shared__ float Ts[C][C + 1], Ps[C][C + 1];
    __shared__ float Kc[C][33], Kr[C][33], Qr[C][33], dOb[C][33], PdO[C][33];
    __shared__ float bes[C];
    const int t = threadIdx.x;
    const int h = blockIdx.x % H, chunk = blockIdx.x / H, b = blockIdx.y;
    const int c0 = chunk * C, nvalid = min(C, L - c0);
    const int64_t tok0 = (int64_t)b * L + c0;
    const int64_t cid = ((int64_t)b * H + h) * Nc + chunk;
    for (int n = t; n < C * C; n += BO_THREADS) {
        Ts[n / C][n % C] = bm.T[cid * C * C + n];
        Ps[n / C][n % C] = bm.P[cid * C * C + n];
    }
    if (t < C) bes[t] = t < nvalid ? beta[(tok0 + t) * H + h] : 0.f;
    const int m = t >> 2, i8 = (t & 3) * 8;   // this thread's row and 8 columns of a block
    for (int cb = 0; cb < D; cb += 32) {
        __syncthreads();   // the previous block's readers are done
        for (int n = t; n < C * 32; n += BO_THREADS) {
            const int r = n >> 5, i = n & 31;
            const bool ok = r < nvalid;
            const int64_t off = ((tok0 + (ok ? r : 0)) * H + h) * D + cb + i;
            const float kv = ok ? to_f32(k[off]) : 0.f;
            Kr[r][i] = kv;
            Kc[r][i] = kv * bm.c[cid * C + r];
            Qr[r][i] = ok ? to_f32(q[off]) : 0.f;
            dOb[r][i] = ok ? d_o[off] : 0.f;
        }
        __syncthreads();
        float w[8] = {}, pd[8] = {};
        for (int r = m; r < C; ++r) {
            const float tr = Ts[r][m], pr = Ps[r][m];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                w[e] = fmaf(tr, Kc[r][i8 + e], w[e]);
                pd[e] = fmaf(pr, dOb[r][i8 + e], pd[e]);
            }
        }
        const float bm_ = bes[m];
        {
            float wv[8];
            bf16 hi[8], lo[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                wv[e] = bm_ * w[e];
                PdO[m][i8 + e] = pd[e];
            }
            split_bf16<8>(wv, hi, lo);
            const int64_t o = (cid * C + m) * D + cb + i8;
            *reinterpret_cast<bf16x8 *>(bm.Wth + o) = pack8(hi);
            *reinterpret_cast<bf16x8 *>(bm.Wtl + o) = pack8(lo);
        }
        // K^T, Q^T of the block: [i][m]
        for (int n = t; n < 32 * C; n += BO_THREADS) {
            const int i = n >> 6, r = n & 63;
            const int64_t o = (cid * D + cb + i) * C + r;
            if constexpr (SPLIT_KQ) {
                const float kv[2] = {Kr[r][i], Qr[r][i]};
                bf16 hi[2], lo[2];
                split_bf16<2>(kv, hi, lo);
                bm.Kth[o] = hi[0];
                bm.Ktl[o] = lo[0];
                bm.Qth[o] = hi[1];
                bm.Qtl[o] = lo[1];
            } else {
                bm.Kth[o] = (bf16)Kr[r][i];
                bm.Qth[o] = (bf16)Qr[r][i];
            }
        }
        __syncthreads();
        float mo[8] = {};
        for (int r = m; r < C; ++r) {
            const float tr = Ts[r][m];
#pragma unroll
            for (int e = 0; e < 8; ++e) mo[e] = fmaf(tr, PdO[r][i8 + e], mo[e]);
        }
        float4 *dst = reinterpret_cast<float4 *>(bm.MtdO + (cid * C + m) * D + cb + i8);
        dst[0] = float4{bm_ * mo[0], bm_ * mo[1], bm_ * mo[2], bm_ * mo[3]};
        dst[1] = float4{bm_ * mo[4], bm_ * mo[5], bm_ * mo[6], bm_ * mo[7]};
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
// per-chunk gradients: one workgroup per (b, h, chunk), all columns
// ---------------------------------------------------------------------------
constexpr int BK_THREADS = 512;

template <int D, typename TIn>
__global__ __launch_bounds__(BK_THREADS) void k_bwd_chunk(
    const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v, const float *__restrict__ alpha,
    const float *__restrict__ beta, const float *__restrict__ d_o, const float *__restrict__ dvin,
    const float *__restrict__ s_chunks, const float *__restrict__ ds_end, BwdMats bm, int L, int H, int Nc,
    float *__restrict__ dq, float *__restrict__ dk, float *__restrict__ dalpha, float *__restrict__ dbeta) {
    __shared__ TIn Ks[C][D], Qs[C][D];
    __shared__ float As[C][C + 1], Ps[C][C + 1], Ts[C][C + 1], Gs[C][C + 1];   // Gs: Gam (lower incl)
    // the column-block buffers (S and dS' blocks, then E, U, dO, dE, dU, K dS' of the block) while the
    // columns are walked; afterwards the same memory holds dP and the dT / dA matrix
    constexpr int BLK = 2 * D * 17 + 6 * C * 17, MAT = 2 * C * (C + 1);
    __shared__ float scratch[BLK > MAT ? BLK : MAT];
    float (*Sb)[17] = reinterpret_cast<float (*)[17]>(scratch);
    float (*dSb)[17] = reinterpret_cast<float (*)[17]>(scratch + D * 17);
    float (*Eb)[17] = reinterpret_cast<float (*)[17]>(scratch + 2 * D * 17);
    float (*Ub)[17] = Eb + C, (*dOb)[17] = Eb + 2 * C, (*dEb)[17] = Eb + 3 * C, (*dUb)[17] = Eb + 4 * C,
          (*KdSb)[17] = Eb + 5 * C;
    float (*dPs)[C + 1] = reinterpret_cast<float (*)[C + 1]>(scratch);
    float (*dXs)[C + 1] = reinterpret_cast<float (*)[C + 1]>(scratch + C * (C + 1));
    __shared__ double lgs[C];
    __shared__ float gam[C], cr[C], bes[C], als[C], dgam[C], dcr[C], dbn[C], dlg[C], red[BK_THREADS / 64];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int h = blockIdx.x % H, chunk = blockIdx.x / H, b = blockIdx.y;
    const int c0 = chunk * C, nvalid = min(C, L - c0);
    const int64_t tok0 = (int64_t)b * L + c0;
    const int64_t cid = ((int64_t)b * H + h) * Nc + chunk;

    // K, Q tiles (rows past the end are zero), gates, and the chunk matrices of the backward prep
    for (int n = t; n < C * D; n += BK_THREADS) {
        const int r = n / D, i = n % D;
        const bool ok = r < nvalid;
        const int64_t off = ((tok0 + (ok ? r : 0)) * H + h) * D + i;
        Ks[r][i] = ok ? k[off] : from_f32<TIn>(0.f);
        Qs[r][i] = ok ? q[off] : from_f32<TIn>(0.f);
    }
    for (int n = t; n < C * C; n += BK_THREADS) {
        const int r = n / C, i = n % C;
        As[r][i] = bm.A[cid * C * C + n];
        Ps[r][i] = bm.P[cid * C * C + n];
        Ts[r][i] = bm.T[cid * C * C + n];
    }
    if (t < C) {
        const bool ok = t < nvalid;
        const int64_t gi = (tok0 + (ok ? t : 0)) * H + h;
        als[t] = ok ? alpha[gi] : 1.f;
        bes[t] = ok ? beta[gi] : 0.f;
        lgs[t] = bm.lg[cid * C + t];
        gam[t] = bm.gam[cid * C + t];
        cr[t] = bm.c[cid * C + t];
        dgam[t] = 0.f;
        dcr[t] = 0.f;
    }
    __syncthreads();
    for (int n = t; n < C * C; n += BK_THREADS) {
        const int r = n / C, i = n % C;
        Gs[r][i] = i <= r ? (float)exp(lgs[r] - lgs[i]) : 0.f;
    }
    __syncthreads();

    // accumulators in registers: dQ, dK rows r = t / 8, columns i = t % 8 + 8 a;
    // dP, dTb rows r, columns m = t % 8 + 8 a
    constexpr int QA = D / 8;
    const int rr = t >> 3, cq = t & 7;
    float dQa[QA], dKa[QA], dPa[8], dTa[8];
#pragma unroll
    for (int a = 0; a < QA; ++a) dQa[a] = dKa[a] = 0.f;
#pragma unroll
    for (int a = 0; a < 8; ++a) dPa[a] = dTa[a] = 0.f;
    float dgC = 0.f;   // this thread's share of sum S (.) dS'

    for (int jb = 0; jb < D / 16; ++jb) {
        const int j0 = jb * 16;
        for (int n = t; n < D * 16; n += BK_THREADS) {
            const int i = n / 16, j = n % 16;
            const int64_t off = (cid * D + i) * D + j0 + j;
            Sb[i][j] = s_chunks[off];
            dSb[i][j] = ds_end[off];
        }
        for (int n = t; n < C * 16; n += BK_THREADS) {
            const int r = n / 16, j = n % 16;
            const bool ok = r < nvalid;
            const int64_t off = ((tok0 + (ok ? r : 0)) * H + h) * D + j0 + j;
            dOb[r][j] = ok ? d_o[off] : 0.f;
            dEb[r][j] = ok ? dvin[off] : 0.f;
            Eb[r][j] = ok ? to_f32(v[off]) : 0.f;   // V for now; E below
        }
        __syncthreads();
        // K S, Q S, K dS' (64 x 16): thread (r = t / 8, j = 2 (t % 8) + {0, 1})
        {
            const int r = rr;
            float dg = 0.f;
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int j = 2 * cq + jj;
                float ks = 0.f, qs = 0.f, kd = 0.f;
                for (int i = 0; i < D; ++i) {
                    const float kv = to_f32(Ks[r][i]), s = Sb[i][j];
                    ks = fmaf(kv, s, ks);
                    qs = fmaf(to_f32(Qs[r][i]), s, qs);
                    kd = fmaf(kv, dSb[i][j], kd);
                }
                const float e = Eb[r][j] - gam[r] * ks;
                dg += dOb[r][j] * qs - dEb[r][j] * ks;
                Eb[r][j] = e;
                KdSb[r][j] = kd;
            }
            // row sums over the 8 threads of row r (consecutive lanes)
#pragma unroll
            for (int off = 1; off < 8; off <<= 1) dg += __shfl_xor(dg, off, 64);
            if (cq == 0) dgam[r] += dg;
        }
        for (int n = t; n < D * 16; n += BK_THREADS) {
            const int i = n / 16, j = n % 16;
            dgC = fmaf(Sb[i][j], dSb[i][j], dgC);
        }
        __syncthreads();
        // U = T diag(beta) E; dU = P^T dO + diag(c) K dS'
        {
            const int r = rr;
            float dc = 0.f;
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int j = 2 * cq + jj;
                float u = 0.f, du = 0.f;
                for (int m = 0; m <= r; ++m) u = fmaf(Ts[r][m] * bes[m], Eb[m][j], u);
                for (int m = r; m < C; ++m) du = fmaf(Ps[m][r], dOb[m][j], du);
                du = fmaf(cr[r], KdSb[r][j], du);
                Ub[r][j] = u;
                dUb[r][j] = du;
                dc = fmaf(u, KdSb[r][j], dc);
            }
#pragma unroll
            for (int off = 1; off < 8; off <<= 1) dc += __shfl_xor(dc, off, 64);
            if (cq == 0) dcr[r] += dc;
        }
        __syncthreads();
        // accumulate dP = dO U^T (lower incl), dTb = dU E^T, dQ, dK
        {
            const int r = rr;
#pragma unroll
            for (int a = 0; a < 8; ++a) {
                const int m = cq + 8 * a;
                float p = 0.f, tb = 0.f;
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    p = fmaf(dOb[r][j], Ub[m][j], p);
                    tb = fmaf(dUb[r][j], Eb[m][j], tb);
                }
                dPa[a] += p;
                dTa[a] += tb;
            }
            const float gr = gam[r], crr = cr[r];
#pragma unroll
            for (int a = 0; a < QA; ++a) {
                const int i = cq + 8 * a;
                float aq = 0.f, ak = 0.f;
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    aq = fmaf(dOb[r][j], Sb[i][j], aq);
                    ak = fmaf(crr * Ub[r][j], dSb[i][j], fmaf(-gr * dEb[r][j], Sb[i][j], ak));
                }
                dQa[a] = fmaf(gr, aq, dQa[a]);
                dKa[a] += ak;
            }
        }
        __syncthreads();   // the next block restages the block buffers
    }

    // ---- the chunk-matrix gradients (dP, then dTb -> dT -> Y = T^T dT -> dA, in the freed block memory) ----
#pragma unroll
    for (int a = 0; a < 8; ++a) {
        const int m = cq + 8 * a;
        dPs[rr][m] = m <= rr ? dPa[a] : 0.f;
        dXs[rr][m] = dTa[a];   // dTb for now
    }
    // the thread-local share of sum S (.) dS' to one value
    {
        float v2 = dgC;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) v2 += __shfl_xor(v2, off, 64);
        if (lane == 0) red[wave] = v2;
    }
    __syncthreads();
    // dbeta part 1 (from Tb = T diag(beta)): sum_r dTb_rm T_rm; dT = dTb diag(beta) in place
    float dbm = 0.f;
    if (t < C) {
        const int m = t;
        for (int r = 0; r < C; ++r) dbm = fmaf(dXs[r][m], Ts[r][m], dbm);
    }
    __syncthreads();
    for (int n = t; n < C * C; n += BK_THREADS) {
        const int r = n / C, m = n % C;
        dXs[r][m] *= bes[m];
    }
    __syncthreads();
    // Y = T^T dT (row rr, columns m = t % 8 + 8 a, in registers), then dN = -Y T^T (strict lower)
    float Y[8];
#pragma unroll
    for (int a = 0; a < 8; ++a) {
        const int m = cq + 8 * a;
        float acc = 0.f;
        for (int r = rr; r < C; ++r) acc = fmaf(Ts[r][rr], dXs[r][m], acc);   // T_r,rr nonzero for r >= rr
        Y[a] = acc;
    }
    __syncthreads();
#pragma unroll
    for (int a = 0; a < 8; ++a) dXs[rr][cq + 8 * a] = Y[a];
    __syncthreads();
    // dN_ri = -sum_m Y_rm T_im (strict lower); dA = diag(beta) dN; dbeta part 2: sum_i dN_ri A_ri
    float dNr[8];
#pragma unroll
    for (int a = 0; a < 8; ++a) {
        const int i = cq + 8 * a;
        float acc = 0.f;
        if (i < rr) {
            for (int m = 0; m <= i; ++m) acc = fmaf(dXs[rr][m], Ts[i][m], acc);   // T_im is zero for m > i
        }
        dNr[a] = -acc;
    }
    __syncthreads();
    // dXs <- dA = diag(beta) dN (strict lower)
#pragma unroll
    for (int a = 0; a < 8; ++a) dXs[rr][cq + 8 * a] = bes[rr] * dNr[a];
    {
        float p2 = 0.f;
#pragma unroll
        for (int a = 0; a < 8; ++a) p2 = fmaf(dNr[a], As[rr][cq + 8 * a], p2);
#pragma unroll
        for (int off = 1; off < 8; off <<= 1) p2 += __shfl_xor(p2, off, 64);
        if (cq == 0) dbn[rr] = p2;   // dbeta of row rr through N = diag(beta) A
    }
    __syncthreads();
    // dQ += (Gam (.) dP) K;  dK += (Gam (.) dP)^T Q + (Gam (.) dA) K + (Gam (.) dA)^T K
    {
        const int r = rr;
#pragma unroll
        for (int a = 0; a < QA; ++a) {
            const int i = cq + 8 * a;
            float aq = 0.f, ak = 0.f;
            for (int m = 0; m < C; ++m) {
                const float gpr = Gs[r][m];   // Gam_rm (zero for m > r)
                const float gmr = Gs[m][r];   // Gam_mr (zero for r > m)
                const float km = to_f32(Ks[m][i]);
                aq = fmaf(gpr * dPs[r][m], km, aq);
                ak = fmaf(gmr * dPs[m][r], to_f32(Qs[m][i]), ak);
                ak = fmaf(gpr * dXs[r][m] + gmr * dXs[m][r], km, ak);
            }
            dQa[a] += aq;
            dKa[a] += ak;
        }
    }
    // The decay gradient.  gamma_r depends on log alpha_m for m <= r, Gam_ab for b < m <= a, c_r for
    // r < m, gamma_C on all m, so
    //     dlog alpha_m = sum_{r >= m} gamma_r dgamma_r + sum_{a >= m > b} (A (.) dA + P (.) dP)_ab
    //                    + sum_{r < m} c_r dc_r + gamma_C dgamma_C,
    // each term a sum of the contributions that actually depend on alpha_m (no cancelling pairs).
    if (t < C) {
        const int m = t;
        float dgCt = 0.f;
        for (int w = 0; w < BK_THREADS / 64; ++w) dgCt += red[w];
        float s1 = 0.f, s2 = 0.f, s3 = 0.f;
        for (int r = m; r < C; ++r) s1 = fmaf(gam[r], dgam[r], s1);
        for (int a = m; a < C; ++a)
            for (int b2 = 0; b2 < m; ++b2) s2 += As[a][b2] * dXs[a][b2] + Ps[a][b2] * dPs[a][b2];
        for (int r = 0; r < m; ++r) s3 = fmaf(cr[r], dcr[r], s3);
        dlg[m] = s1 + s2 + s3 + gam[C - 1] * dgCt;
    }
    __syncthreads();
    // outputs
    if (t < C) {
        const int m = t;
        if (m < nvalid) {
            const int64_t gi = (tok0 + m) * H + h;
            dalpha[gi] = dlg[m] / als[m];
            dbeta[gi] = dbm + dbn[m];
        }
    }
    if (rr < nvalid) {
        const int64_t base = ((tok0 + rr) * H + h) * D;
#pragma unroll
        for (int a = 0; a < QA; ++a) {
            dq[base + cq + 8 * a] = dQa[a];
            dk[base + cq + 8 * a] = dKa[a];
        }
    }
}

}  // namespace

hipError_t launch_bwd_prep(bool f32, int B, int L, int H, int D, const void *q, const void *k, const float *alpha,
                           const float *beta, float *mats, hipStream_t s) {
    const int Nc = (L + C - 1) / C;
    const dim3 grid((unsigned)(Nc * H), B);
    const BwdMats bm = bwd_mats(mats, (int64_t)B * H * Nc, D);
#define BP(DD, T) launch_kernel((k_bwd_prep<DD, T>), grid, dim3(BP_THREADS), 0, s, (const T *)q, (const T *)k, alpha, beta, L, H, Nc, bm)
    if (f32) {
        if (D == 64) BP(64, float); else return hipErrorInvalidValue;
    } else {
        if (D == 128) BP(128, bf16); else BP(64, bf16);
    }
#undef BP
    return hipGetLastError();
}

hipError_t launch_bwd_ops(bool f32, int B, int L, int H, int D, const void *q, const void *k, const float *beta,
                          const float *d_o, float *mats, hipStream_t s) {
    const int Nc = (L + C - 1) / C;
    const dim3 grid((unsigned)(Nc * H), B);
    const BwdMats bm = bwd_mats(mats, (int64_t)B * H * Nc, D);
#define BO(DD, T) launch_kernel((k_bwd_ops<DD, T>), grid, dim3(BO_THREADS), 0, s, (const T *)q, (const T *)k, beta, d_o, L, H, Nc, bm)
    if (f32) {
        if (D == 64) BO(64, float); else return hipErrorInvalidValue;
    } else {
        if (D == 128) BO(128, bf16); else BO(64, bf16);
    }
#undef BO
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
