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
//   forward substitution, then block rows), and W, M, gamma to the workspace.
// k_scan_carry: one workgroup per (b, h, 16 columns of S); the columns of S
//   never mix, so column slices are independent scans.  Each of the 4 waves
//   keeps D/4 rows of the fp32 state slice in registers (MFMA accumulator
//   layout) and, per chunk, forms its share of K.S and Q.S, exchanges the
//   partial sums through LDS (one barrier per chunk, double-buffered), then
//   computes E, S' = gamma_C S + W E (its own rows) and O for 16 tokens.  The
//   products use split-bf16 operands (x = hi + lo, ~16 significant bits) with
//   fp32 accumulation; operands that are exact bf16 inputs are not split.
//   Next-chunk operands are prefetched into registers during the current chunk.
#include "gdn_device.h"
#include "gdn_kernels.h"

namespace gdn {

namespace {

constexpr int C = 64;       // tokens per chunk
constexpr int LDP = C + 1;  // padded row stride of the 64x64 fp32 LDS matrices

template <typename T> struct In;
template <> struct In<float> { static constexpr bool f32 = true; };
template <> struct In<bf16> { static constexpr bool f32 = false; };

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
        float *dst = wsW + cid * D * C;
#pragma unroll
        for (int ii = 0; ii < IPT; ++ii) dst[(int64_t)(i0 + ii) * C + c] = acc[ii];
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
        float *dst = wsM + cid * C * C;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) dst[(r0 + rr) * C + c] = acc[rr];
    }
    // (8) gamma
    if (t < C) wsg[cid * C + t] = gam[t];
}

// ---------------------------------------------------------------------------
// carry
// ---------------------------------------------------------------------------
// Operand fragments of one chunk for one wave, prefetched a chunk ahead.
template <int D, bool F32>
struct ChunkFrags {
    static constexpr int NT = D / 64;           // 16-row tiles of S per wave (D/4 rows)
    static constexpr int KW = (D == 128) ? 8 : 4;  // k-width of the K.S / Q.S MFMA
    float kf[4][KW], qf[4][KW];                 // K, Q rows (tokens 16tm + l%16), wave's S rows
    float wf[NT][2][8];                         // W rows (wave's S rows), permuted token slots
    float mf[2][8];                             // M rows (tokens 16w + l%16), permuted token slots
    float vv[4][4];                             // V in accumulator layout
    float gv[4][4];                             // gamma in accumulator layout
    float gC;
};

template <int D, typename TIn>
__device__ __forceinline__ void load_frags(ChunkFrags<D, In<TIn>::f32> &F, int chunk, int L, int H,
                                           int h, int64_t tokb, int col0, const TIn *q,
                                           const TIn *k, const TIn *v, const float *W,
                                           const float *M, const float *g, int64_t cidb) {
    constexpr int NT = D / 64, RW = D / 4;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int c0 = chunk * C;
    const int sr0 = wave * RW;
    // K, Q: token 16tm + lr; S-row slots sr0 + 4lg + {0..3} (and + 16 for D == 128)
#pragma unroll
    for (int tm = 0; tm < 4; ++tm) {
        const int tok = c0 + 16 * tm + lr;
        const bool ok = tok < L;
        const int64_t base = ((tokb + tok) * H + h) * D + sr0 + 4 * lg;
#pragma unroll
        for (int part = 0; part < F.KW / 4; ++part) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                F.kf[tm][4 * part + i] = ok ? to_f32(k[base + 16 * part + i]) : 0.f;
                F.qf[tm][4 * part + i] = ok ? to_f32(q[base + 16 * part + i]) : 0.f;
            }
        }
    }
    const int64_t cid = cidb + chunk;
    const float *Wc = W + cid * D * C;
    const float *Mc = M + cid * C * C;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
        const float *wr = Wc + (int64_t)(sr0 + 16 * tt + lr) * C;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const float4 a = *reinterpret_cast<const float4 *>(wr + 32 * s + 4 * lg);
            const float4 bq = *reinterpret_cast<const float4 *>(wr + 32 * s + 16 + 4 * lg);
            F.wf[tt][s][0] = a.x; F.wf[tt][s][1] = a.y; F.wf[tt][s][2] = a.z; F.wf[tt][s][3] = a.w;
            F.wf[tt][s][4] = bq.x; F.wf[tt][s][5] = bq.y; F.wf[tt][s][6] = bq.z; F.wf[tt][s][7] = bq.w;
        }
    }
    {
        const float *mr = Mc + (16 * wave + lr) * C;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const float4 a = *reinterpret_cast<const float4 *>(mr + 32 * s + 4 * lg);
            const float4 bq = *reinterpret_cast<const float4 *>(mr + 32 * s + 16 + 4 * lg);
            F.mf[s][0] = a.x; F.mf[s][1] = a.y; F.mf[s][2] = a.z; F.mf[s][3] = a.w;
            F.mf[s][4] = bq.x; F.mf[s][5] = bq.y; F.mf[s][6] = bq.z; F.mf[s][7] = bq.w;
        }
    }
    const float *gc = g + cid * C;
#pragma unroll
    for (int tm = 0; tm < 4; ++tm) {
        const float4 gg = *reinterpret_cast<const float4 *>(gc + 16 * tm + 4 * lg);
        F.gv[tm][0] = gg.x; F.gv[tm][1] = gg.y; F.gv[tm][2] = gg.z; F.gv[tm][3] = gg.w;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int tok = c0 + 16 * tm + 4 * lg + j;
            F.vv[tm][j] = (tok < L) ? to_f32(v[((tokb + tok) * H + h) * D + col0 + lr]) : 0.f;
        }
    }
    F.gC = gc[C - 1];
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

// c += a . b with a, b given in fp32; a_exact: a is already representable in bf16.
template <int KW, bool A_EXACT>
__device__ __forceinline__ f32x4 mma_split(const float (&a)[KW], const __bf16 (&bh)[KW],
                                           const __bf16 (&bl)[KW], f32x4 c) {
    __bf16 ah[KW], al[KW];
    split_bf16(a, ah, al);
    c = mma_bf<KW>(ah, bh, c);
    c = mma_bf<KW>(ah, bl, c);
    if constexpr (!A_EXACT) c = mma_bf<KW>(al, bh, c);
    return c;
}

template <int D, typename TIn, bool LOOP>
__global__ __launch_bounds__(256) void k_scan_carry(
    const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v, int L, int H,
    int Nc, const float *__restrict__ W, const float *__restrict__ M, const float *__restrict__ g,
    const float *__restrict__ s_init, float *__restrict__ s_final, float *__restrict__ o,
    const void *h_prev, int h_prev_bf16, const float *__restrict__ rho,
    float *h_out, bf16 *x_next) {
    constexpr bool F32 = In<TIn>::f32;
    constexpr int NT = D / 64, RW = D / 4;
    constexpr int KW = (D == 128) ? 8 : 4;
    __shared__ __attribute__((aligned(16))) f32x4 red[2][4][2][4][64];  // [buf][wave][KS|QS][tile][lane]

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int slice = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int col0 = slice * 16;
    const int col = col0 + lr;
    const int sr0 = wave * RW;
    const int64_t tokb = (int64_t)b * L;
    const int64_t cidb = ((int64_t)b * H + h) * Nc;
    const int d = H * D;

    // state slice: S[sr0 + 16tt + 4lg + j][col]
    float Sv[NT][4];
    const int64_t sbase = ((int64_t)b * H + h) * D * D;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            Sv[tt][j] = s_init ? s_init[sbase + (int64_t)(sr0 + 16 * tt + 4 * lg + j) * D + col] : 0.f;

    ChunkFrags<D, F32> cur, nxt;
    load_frags<D, TIn>(cur, 0, L, H, h, tokb, col0, q, k, v, W, M, g, cidb);

    for (int chunk = 0; chunk < Nc; ++chunk) {
        const int buf = chunk & 1;
        if (chunk + 1 < Nc) load_frags<D, TIn>(nxt, chunk + 1, L, H, h, tokb, col0, q, k, v, W, M, g, cidb);

        // split the state slice into the B operand of K.S / Q.S
        __bf16 sh[KW], sl[KW];
        {
            float sf[KW];
#pragma unroll
            for (int i = 0; i < KW; ++i) sf[i] = Sv[i / 4][i % 4];
            split_bf16(sf, sh, sl);
        }
        // partial K.S and Q.S over this wave's S rows
#pragma unroll
        for (int tm = 0; tm < 4; ++tm) {
            f32x4 ks = {0.f, 0.f, 0.f, 0.f}, qs = {0.f, 0.f, 0.f, 0.f};
            ks = mma_split<KW, !F32>(cur.kf[tm], sh, sl, ks);
            qs = mma_split<KW, !F32>(cur.qf[tm], sh, sl, qs);
            red[buf][wave][0][tm][lane] = ks;
            red[buf][wave][1][tm][lane] = qs;
        }
        lds_barrier();

        // E = V - diag(gamma) K S (all 64 tokens, this lane's column)
        float E[4][4];
#pragma unroll
        for (int tm = 0; tm < 4; ++tm) {
            f32x4 s4 = red[buf][0][0][tm][lane];
#pragma unroll
            for (int w = 1; w < 4; ++w) {
                const f32x4 p = red[buf][w][0][tm][lane];
                s4[0] += p[0]; s4[1] += p[1]; s4[2] += p[2]; s4[3] += p[3];
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) E[tm][j] = cur.vv[tm][j] - cur.gv[tm][j] * s4[j];
        }
        f32x4 qsum = red[buf][0][1][wave][lane];
#pragma unroll
        for (int w = 1; w < 4; ++w) {
            const f32x4 p = red[buf][w][1][wave][lane];
            qsum[0] += p[0]; qsum[1] += p[1]; qsum[2] += p[2]; qsum[3] += p[3];
        }

        // E as the B operand: k-step s covers accumulator tiles 2s and 2s+1
        __bf16 eh[2][8], el[2][8];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            float ef[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                ef[j] = E[2 * s][j];
                ef[4 + j] = E[2 * s + 1][j];
            }
            split_bf16(ef, eh[s], el[s]);
        }
        // S' = gamma_C S + W E (this wave's rows)
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            f32x4 we = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 2; ++s) we = mma_split<8, false>(cur.wf[tt][s], eh[s], el[s], we);
#pragma unroll
            for (int j = 0; j < 4; ++j) Sv[tt][j] = cur.gC * Sv[tt][j] + we[j];
        }
        // O = diag(gamma) Q S + M E for tokens 16*wave + 4lg + j
        f32x4 me = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 2; ++s) me = mma_split<8, false>(cur.mf[s], eh[s], el[s], me);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 16 * wave + 4 * lg + j;
            const int tok = chunk * C + r;
            if (tok < L) {
                const float ov = cur.gv[wave][j] * qsum[j] + me[j];
                const int64_t row = tokb + tok;
                if constexpr (!LOOP) {
                    o[(row * H + h) * D + col] = ov;
                } else {
                    const int64_t hi = row * d + (int64_t)h * D + col;
                    const float hp = h_prev_bf16 ? (float)reinterpret_cast<const bf16 *>(h_prev)[hi]
                                                 : reinterpret_cast<const float *>(h_prev)[hi];
                    const float hn = ov + rho[h * D + col] * hp;
                    h_out[hi] = hn;
                    if (x_next) x_next[hi] = (bf16)hn;
                }
            }
        }
        if (chunk + 1 < Nc) cur = nxt;
    }
    if (s_final) {
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                s_final[sbase + (int64_t)(sr0 + 16 * tt + 4 * lg + j) * D + col] = Sv[tt][j];
    }
}

}  // namespace

hipError_t launch_scan_prep(bool f32, int B, int L, int H, int D, const void *q, const void *k,
                            const float *alpha, const float *beta, ChunkWs ws, hipStream_t s) {
    const int Nc = (L + C - 1) / C;
    dim3 grid(Nc, H, B);
#define PREP(DD, T)                                                                                \
    hipLaunchKernelGGL((k_scan_prep<DD, T>), grid, dim3(256), 0, s, (const T *)q, (const T *)k,   \
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
    dim3 grid(D / 16, H, B);
    const bool loop = out.h_out != nullptr;
#define CARRY(DD, T, LP)                                                                           \
    hipLaunchKernelGGL((k_scan_carry<DD, T, LP>), grid, dim3(256), 0, s, (const T *)q,            \
                       (const T *)k, (const T *)v, L, H, Nc, ws.W, ws.M, ws.g, s_init, s_final,   \
                       out.o, out.h_prev, out.h_prev_bf16 ? 1 : 0, out.rho, out.h_out, out.x_next)
#define CARRY_D(T, LP)                                                                             \
    do { if (D == 128) CARRY(128, T, LP); else CARRY(64, T, LP); } while (0)
    if (f32) {
        if (loop) CARRY_D(float, true); else CARRY_D(float, false);
    } else {
        if (loop) CARRY_D(bf16, true); else CARRY_D(bf16, false);
    }
#undef CARRY_D
#undef CARRY
    return hipGetLastError();
}

}  // namespace gdn
