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
// log-cumsum lg [64] (fp64), gamma = e^lg and c = e^(lg_last - lg) [64].
struct BwdMats {
    float *T, *P, *A;
    double *lg;
    float *gam, *c;
};
constexpr size_t BWD_MATS_PER_CHUNK = 3 * C * C * 4 + C * 8 + 2 * C * 4;   // bytes per chunk
// The regions of a BwdMats block for `chunks` chunks, each array for all chunks in turn.
BwdMats bwd_mats(float *base, int64_t chunks) {
    BwdMats m;
    m.T = base;
    m.P = m.T + chunks * C * C;
    m.A = m.P + chunks * C * C;
    m.lg = reinterpret_cast<double *>(m.A + chunks * C * C);
    m.gam = reinterpret_cast<float *>(m.lg + chunks * C);
    m.c = m.gam + chunks * C;
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
// reverse carry: one workgroup per (b, h, 16-column slice), chunks in reverse
// ---------------------------------------------------------------------------
constexpr int BC_THREADS = 256;

template <int D, typename TIn>
__global__ __launch_bounds__(BC_THREADS) void k_bwd_carry(
    const TIn *__restrict__ q, const TIn *__restrict__ k, const float *__restrict__ beta, const float *__restrict__ d_o,
    BwdMats bm, const float *__restrict__ d_sfinal, int L, int H, int Nc, float *__restrict__ dv,
    float *__restrict__ ds_end, float *__restrict__ ds_init) {
    __shared__ float Tf[C][C + 1], Pf[C][C + 1];
    __shared__ float Kf[C][D + 1], Qf[C][D + 1];
    __shared__ float dOs[C][17], dUs[C][17], dEs[C][17], dSs[D][17];
    __shared__ float gs[C], cs[C], bs[C];
    const int t = threadIdx.x;
    const int h = blockIdx.x, slice = blockIdx.y, b = blockIdx.z;
    const int col0 = slice * 16;
    const int64_t tokb = (int64_t)b * L;
    const int64_t cidb = ((int64_t)b * H + h) * Nc;
    const int64_t sbase = ((int64_t)b * H + h) * D * D;
    // this thread's state elements dS[i][j]: j = t % 16, i = t / 16 + 16 a
    constexpr int RA = D / 16;
    const int jc = t & 15, i0 = t >> 4;
    float dS[RA];
#pragma unroll
    for (int a = 0; a < RA; ++a) dS[a] = d_sfinal ? d_sfinal[sbase + (int64_t)(i0 + 16 * a) * D + col0 + jc] : 0.f;

    for (int c = Nc - 1; c >= 0; --c) {
        const int c0 = c * C, nvalid = min(C, L - c0);
        const int64_t cid = cidb + c;
        // stage the chunk: T, P, gamma, c, beta, K, Q, the dO slice; dS' (the current state) to LDS and out
        for (int n = t; n < C * C; n += BC_THREADS) {
            Tf[n / C][n % C] = bm.T[cid * C * C + n];
            Pf[n / C][n % C] = bm.P[cid * C * C + n];
        }
        for (int n = t; n < C * D; n += BC_THREADS) {
            const int r = n / D, i = n % D;
            const bool ok = r < nvalid;
            const int64_t off = ((tokb + c0 + (ok ? r : 0)) * H + h) * D + i;
            Kf[r][i] = ok ? to_f32(k[off]) : 0.f;
            Qf[r][i] = ok ? to_f32(q[off]) : 0.f;
        }
        for (int n = t; n < C * 16; n += BC_THREADS) {
            const int r = n / 16, j = n % 16;
            dOs[r][j] = r < nvalid ? d_o[((tokb + c0 + r) * H + h) * D + col0 + j] : 0.f;
        }
        if (t < C) {
            gs[t] = bm.gam[cid * C + t];
            cs[t] = bm.c[cid * C + t];
            bs[t] = t < nvalid ? beta[(tokb + c0 + t) * H + h] : 0.f;
        }
#pragma unroll
        for (int a = 0; a < RA; ++a) {
            const int i = i0 + 16 * a;
            dSs[i][jc] = dS[a];
            ds_end[(cid * D + i) * D + col0 + jc] = dS[a];
        }
        __syncthreads();
        // dU = P^T dO + diag(c) K dS'   (64 x 16)
        for (int n = t; n < C * 16; n += BC_THREADS) {
            const int m = n / 16, j = n % 16;
            float pd = 0.f, kd = 0.f;
            for (int r = m; r < C; ++r) pd = fmaf(Pf[r][m], dOs[r][j], pd);
            for (int i = 0; i < D; ++i) kd = fmaf(Kf[m][i], dSs[i][j], kd);
            dUs[m][j] = fmaf(cs[m], kd, pd);
        }
        __syncthreads();
        // dE = diag(beta) T^T dU   (= dV)
        for (int n = t; n < C * 16; n += BC_THREADS) {
            const int m = n / 16, j = n % 16;
            float acc = 0.f;
            for (int r = m; r < C; ++r) acc = fmaf(Tf[r][m], dUs[r][j], acc);
            acc *= bs[m];
            dEs[m][j] = acc;
            if (m < nvalid) dv[((tokb + c0 + m) * H + h) * D + col0 + j] = acc;
        }
        __syncthreads();
        // dS = gamma_C dS' + Q^T diag(gamma) dO - K^T diag(gamma) dE
        const float gC = gs[C - 1];
#pragma unroll
        for (int a = 0; a < RA; ++a) {
            const int i = i0 + 16 * a;
            float acc = 0.f;
            for (int r = 0; r < C; ++r) acc = fmaf(gs[r], Qf[r][i] * dOs[r][jc] - Kf[r][i] * dEs[r][jc], acc);
            dS[a] = gC * dS[a] + acc;
        }
        __syncthreads();   // the next chunk restages every buffer
    }
    if (ds_init) {
#pragma unroll
        for (int a = 0; a < RA; ++a) ds_init[sbase + (int64_t)(i0 + 16 * a) * D + col0 + jc] = dS[a];
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
    const BwdMats bm = bwd_mats(mats, (int64_t)B * H * Nc);
#define BP(DD, T) launch_kernel((k_bwd_prep<DD, T>), grid, dim3(BP_THREADS), 0, s, (const T *)q, (const T *)k, alpha, beta, L, H, Nc, bm)
    if (f32) {
        if (D == 64) BP(64, float); else return hipErrorInvalidValue;
    } else {
        if (D == 128) BP(128, bf16); else BP(64, bf16);
    }
#undef BP
    return hipGetLastError();
}

hipError_t launch_bwd_carry(bool f32, int B, int L, int H, int D, const void *q, const void *k, const float *beta,
                            const float *d_o, const float *d_sfinal, float *mats, float *dv, float *ds_end,
                            float *ds_init, hipStream_t s) {
    const int Nc = (L + C - 1) / C;
    const dim3 grid(H, D / 16, B);
    const BwdMats bm = bwd_mats(mats, (int64_t)B * H * Nc);
#define BC(DD, T)                                                                                    \
    launch_kernel((k_bwd_carry<DD, T>), grid, dim3(BC_THREADS), 0, s, (const T *)q, (const T *)k, beta, d_o, bm, \
                  d_sfinal, L, H, Nc, dv, ds_end, ds_init)
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
    const BwdMats bm = bwd_mats(mats, (int64_t)B * H * Nc);
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

size_t bwd_mats_bytes(int64_t chunks) { return (size_t)chunks * BWD_MATS_PER_CHUNK; }

}  // namespace gdn
