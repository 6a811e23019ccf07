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

// Position of element (row, token c) of a per-chunk [R x 64] matrix (W: R = D
// rows of S; M: R = 64 output tokens) in the carry's fragment order.  Rows are
// split over the 4 waves (R/4 each, in 16-row tiles tt); the 64 tokens form
// two 32-token k-steps s.  Lane l = lr + 16 lg of the wave holds row
// 16 tt + lr and, in slot j of its 8-element fragment, token
// 32 s + 4 lg + j (j < 4) or 32 s + 16 + 4 lg + (j - 4) (j >= 4).  Layout:
// [wave][tt][s][part: hi, lo][lane][8] bf16, so each wave reads its fragments
// with fully coalesced 16-byte loads.  The lo part sits 8 * 64 elements after
// the hi part.
template <int R>
__device__ __forceinline__ int64_t frag_index(int row, int c) {
    constexpr int RW = R / 4, NT = RW / 16;
    const int w = row / RW, rem = row % RW, tt = rem / 16, lr = rem % 16;
    const int s = c / 32, o = c % 32;
    const int lg = (o % 16) / 4, j = (o % 4) + (o >= 16 ? 4 : 0);
    const int lane = lr + 16 * lg;
    return ((((int64_t)(w * NT + tt) * 2 + s) * 2) * 64 + lane) * 8 + j;
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
// Per-wave operand fragments of one chunk (registers).  K and Q rows are the
// A operand of K.S / Q.S over this wave's D/4 state rows; W and M rows (bf16
// hi/lo parts from the workspace) are the A operand of W.E / M.E over the
// chunk's 64 tokens.  For D == 128 the 32 state rows (and the 32 tokens of each
// E k-step) are taken in the order {4g..4g+3, 16+4g..16+4g+3} for lane group g,
// which is exactly the order in which an MFMA accumulator tile holds them, so S
// and E feed the next product straight from registers.
template <int D, typename TIn> struct Frags {
    static constexpr int NT = D / 64, KW = (D == 128) ? 8 : 4;
    TIn k[4][KW], q[4][KW];
    __bf16 wh[NT][2][8], wl[NT][2][8], mh[2][8], ml[2][8];
};

template <typename T> __device__ __forceinline__ void load4(const T *p, T *dst);
template <> __device__ __forceinline__ void load4<bf16>(const bf16 *p, bf16 *dst) {
    const bf16x4 v = *reinterpret_cast<const bf16x4 *>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = v[i];
}
template <> __device__ __forceinline__ void load4<float>(const float *p, float *dst) {
    const float4 v = *reinterpret_cast<const float4 *>(p);
    dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
}

template <int D, typename TIn>
__device__ __forceinline__ void load_frags(Frags<D, TIn> &F, int chunk, int L, int H, int h,
                                           int64_t tokb, const TIn *q, const TIn *k,
                                           const float *W, const float *M, int64_t cidb) {
    constexpr int NT = D / 64, RW = D / 4, KW = (D == 128) ? 8 : 4;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int c0 = chunk * C, sr0 = wave * RW;
    // Tokens past the end of the sequence read the last token instead (no
    // branch around the loads, so they stay in flight): the prep kernel gives
    // padded tokens beta = 0, which zeroes their columns of W and M, and their
    // outputs are never stored, so any finite value is harmless.
#pragma unroll
    for (int tm = 0; tm < 4; ++tm) {
        const int tok = min(c0 + 16 * tm + lr, L - 1);
        const int64_t base = ((tokb + tok) * H + h) * D + sr0 + 4 * lg;
#pragma unroll
        for (int part = 0; part < KW / 4; ++part) {
            load4<TIn>(k + base + 16 * part, &F.k[tm][4 * part]);
            load4<TIn>(q + base + 16 * part, &F.q[tm][4 * part]);
        }
    }
    const int64_t cid = cidb + chunk;
    // W and M come in fragment order (see frag_index): one 16-byte load per part
    const bf16x8 *Wf = reinterpret_cast<const bf16x8 *>(W + cid * D * C) + (int64_t)wave * NT * 4 * 64 + lane;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const bf16x8 hi = Wf[((tt * 2 + s) * 2 + 0) * 64];
            const bf16x8 lo = Wf[((tt * 2 + s) * 2 + 1) * 64];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                F.wh[tt][s][i] = hi[i];
                F.wl[tt][s][i] = lo[i];
            }
        }
    const bf16x8 *Mf = reinterpret_cast<const bf16x8 *>(M + cid * C * C) + (int64_t)wave * 4 * 64 + lane;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const bf16x8 hi = Mf[(s * 2 + 0) * 64];
        const bf16x8 lo = Mf[(s * 2 + 1) * 64];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            F.mh[s][i] = hi[i];
            F.ml[s][i] = lo[i];
        }
    }
}

// Per-chunk data shared by the four waves: V slice [64 tokens x 16 columns],
// gamma [64] and (loop form) the residual input h_prev [64 x 16].  Thread t
// loads token t/4, columns 4(t%4)..+3, and gamma[4(t%16)..+3] in raw form;
// conversion happens when the values are written to LDS, a chunk later, so the
// loads stay in flight.  Padded tokens read the last token (see load_frags).
template <typename TIn> struct VG {
    uint4 v;         // 4 values of V, raw (bf16: .x, .y hold 4 packed values)
    float4 g;
    uint4 hp;        // 4 values of h_prev, raw (bf16: .x, .y)
};

template <typename T> __device__ __forceinline__ uint4 load4_raw(const T *p);
template <> __device__ __forceinline__ uint4 load4_raw<bf16>(const bf16 *p) {
    const uint2 r = *reinterpret_cast<const uint2 *>(p);
    return make_uint4(r.x, r.y, 0u, 0u);
}
template <> __device__ __forceinline__ uint4 load4_raw<float>(const float *p) {
    return *reinterpret_cast<const uint4 *>(p);
}
template <typename T> __device__ __forceinline__ void unpack4(const uint4 &r, float *dst);
template <> __device__ __forceinline__ void unpack4<bf16>(const uint4 &r, float *dst) {
    dst[0] = __uint_as_float(r.x << 16);
    dst[1] = __uint_as_float(r.x & 0xFFFF0000u);
    dst[2] = __uint_as_float(r.y << 16);
    dst[3] = __uint_as_float(r.y & 0xFFFF0000u);
}
template <> __device__ __forceinline__ void unpack4<float>(const uint4 &r, float *dst) {
    dst[0] = __uint_as_float(r.x);
    dst[1] = __uint_as_float(r.y);
    dst[2] = __uint_as_float(r.z);
    dst[3] = __uint_as_float(r.w);
}

template <typename TIn, int RES>
__device__ __forceinline__ void load_vg(VG<TIn> &X, int chunk, int L, int H, int h, int D, int64_t tokb,
                                        int col0, const TIn *v, const float *g, int64_t cidb,
                                        const void *h_prev) {
    const int t = threadIdx.x;
    const int tok = min(chunk * C + (t >> 2), L - 1);
    X.v = load4_raw<TIn>(v + ((tokb + tok) * H + h) * D + col0 + 4 * (t & 3));
    X.g = *reinterpret_cast<const float4 *>(g + (cidb + chunk) * C + 4 * (t & 15));
    if constexpr (RES != 0) {
        const int64_t hi = (tokb + tok) * (int64_t)H * D + (int64_t)h * D + col0 + 4 * (t & 3);
        if constexpr (RES == 2) X.hp = load4_raw<bf16>(reinterpret_cast<const bf16 *>(h_prev) + hi);
        else X.hp = load4_raw<float>(reinterpret_cast<const float *>(h_prev) + hi);
    }
}

template <typename TIn, int RES>
__device__ __forceinline__ void store_vg(const VG<TIn> &X, float (*vl)[17], float *gl, float (*hl)[17]) {
    const int t = threadIdx.x, r = t >> 2, c = 4 * (t & 3);
    float f[4];
    unpack4<TIn>(X.v, f);
#pragma unroll
    for (int i = 0; i < 4; ++i) vl[r][c + i] = f[i];
    if (t < 16) {
        gl[4 * t] = X.g.x; gl[4 * t + 1] = X.g.y; gl[4 * t + 2] = X.g.z; gl[4 * t + 3] = X.g.w;
    }
    if constexpr (RES != 0) {
        if constexpr (RES == 2) unpack4<bf16>(X.hp, f);
        else unpack4<float>(X.hp, f);
#pragma unroll
        for (int i = 0; i < 4; ++i) hl[r][c + i] = f[i];
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
// ... or an A operand already given as hi/lo parts (3 passes)
__device__ __forceinline__ f32x4 mma_hl(const __bf16 (&ah)[8], const __bf16 (&al)[8],
                                        const __bf16 (&bh)[8], const __bf16 (&bl)[8], f32x4 c) {
    c = mma_bf<8>(ah, bh, c);
    c = mma_bf<8>(ah, bl, c);
    return mma_bf<8>(al, bh, c);
}

// One chunk of the carry for one wave: partial K.S / Q.S, exchange, E, S' and O.
template <int D, typename TIn, int RES>
__device__ __forceinline__ void carry_chunk(
    const Frags<D, TIn> &F, float (&Sv)[D / 64][4], int chunk, int L, int H, int h, int64_t tokb,
    int col, float rho_c, f32x4 (*red)[2][4][64], const float (*vl)[17], const float *gl,
    const float (*hl)[17], float *o, float *h_out, bf16 *x_next) {
    constexpr int NT = D / 64, KW = (D == 128) ? 8 : 4;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int d = H * D;

    // B operand of K.S / Q.S: this wave's state rows, split into bf16 hi/lo
    __bf16 sh[KW], sl[KW];
    {
        float sf[KW];
#pragma unroll
        for (int i = 0; i < KW; ++i) sf[i] = Sv[i / 4][i % 4];
        split_bf16(sf, sh, sl);
    }
#pragma unroll
    for (int tm = 0; tm < 4; ++tm) {
        f32x4 ks = {0.f, 0.f, 0.f, 0.f}, qs = {0.f, 0.f, 0.f, 0.f};
        ks = mma_a<KW>(F.k[tm], sh, sl, ks);
        qs = mma_a<KW>(F.q[tm], sh, sl, qs);
        red[wave][0][tm][lane] = ks;
        red[wave][1][tm][lane] = qs;
    }
    lds_barrier();

    // E = V - diag(gamma) K S for all 64 tokens of this lane's column
    float E[4][4];
#pragma unroll
    for (int tm = 0; tm < 4; ++tm) {
        f32x4 s4 = red[0][0][tm][lane];
#pragma unroll
        for (int w = 1; w < 4; ++w) {
            const f32x4 p = red[w][0][tm][lane];
            s4[0] += p[0]; s4[1] += p[1]; s4[2] += p[2]; s4[3] += p[3];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 16 * tm + 4 * lg + j;
            E[tm][j] = vl[r][lr] - gl[r] * s4[j];
        }
    }
    f32x4 qsum = red[0][1][wave][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
        const f32x4 p = red[w][1][wave][lane];
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
    const float gC = gl[C - 1];
    // S' = gamma_C S + W E (this wave's rows)
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
        f32x4 we = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 2; ++s) we = mma_hl(F.wh[tt][s], F.wl[tt][s], eh[s], el[s], we);
#pragma unroll
        for (int j = 0; j < 4; ++j) Sv[tt][j] = gC * Sv[tt][j] + we[j];
    }
    // O = diag(gamma) Q S + M E for tokens 16*wave + 4lg + j
    f32x4 me = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 2; ++s) me = mma_hl(F.mh[s], F.ml[s], eh[s], el[s], me);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 16 * wave + 4 * lg + j;
        const int tok = chunk * C + r;
        if (tok < L) {
            const float ov = gl[r] * qsum[j] + me[j];
            const int64_t row = tokb + tok;
            if constexpr (RES == 0) {
                o[(row * H + h) * D + col] = ov;
            } else {
                const int64_t hi = row * d + (int64_t)h * D + col;
                const float hn = ov + rho_c * hl[r][lr];
                h_out[hi] = hn;
                if (x_next) x_next[hi] = (bf16)hn;
            }
        }
    }
}

template <int D, typename TIn, int RES>
__global__ __launch_bounds__(256) void k_scan_carry(
    const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v, int L, int H,
    int Nc, const float *__restrict__ W, const float *__restrict__ M, const float *__restrict__ g,
    const float *__restrict__ s_init, float *__restrict__ s_final, float *__restrict__ o,
    const void *h_prev, const float *__restrict__ rho, float *h_out, bf16 *x_next) {
    constexpr int NT = D / 64, RW = D / 4;
    __shared__ __attribute__((aligned(16))) f32x4 red[2][4][2][4][64];  // [buf][wave][KS|QS][tile][lane]
    __shared__ float vls[2][C][17];
    __shared__ float hls[RES ? 2 : 1][C][17];
    __shared__ float gls[2][C];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    // heads run along x so that the D/16 column slices of one head, which read the
    // same K, Q, W and M, get workgroup ids that are congruent mod 8 and share an XCD
    const int h = blockIdx.x, slice = blockIdx.y, b = blockIdx.z;
    const int col0 = slice * 16, col = col0 + lr;
    const int sr0 = wave * RW;
    const int64_t tokb = (int64_t)b * L;
    const int64_t cidb = ((int64_t)b * H + h) * Nc;
    const float rho_c = RES ? rho[h * D + col] : 0.f;
    float (*hl0)[17] = hls[0];
    float (*hl1)[17] = hls[RES ? 1 : 0];

    // state slice: Sv[tt][j] = S[sr0 + 16tt + 4lg + j][col]
    float Sv[NT][4];
    const int64_t sbase = ((int64_t)b * H + h) * D * D;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            Sv[tt][j] = s_init ? s_init[sbase + (int64_t)(sr0 + 16 * tt + 4 * lg + j) * D + col] : 0.f;

    Frags<D, TIn> fa, fb;
    VG<TIn> vg;
    load_frags<D, TIn>(fa, 0, L, H, h, tokb, q, k, W, M, cidb);
    load_vg<TIn, RES>(vg, 0, L, H, h, D, tokb, col0, v, g, cidb, h_prev);
    store_vg<TIn, RES>(vg, vls[0], gls[0], hl0);
    __syncthreads();

    // two chunks per iteration so the register sets swap roles without copies
    for (int chunk = 0; chunk < Nc; chunk += 2) {
        const bool has1 = chunk + 1 < Nc;
        if (has1) {
            load_frags<D, TIn>(fb, chunk + 1, L, H, h, tokb, q, k, W, M, cidb);
            load_vg<TIn, RES>(vg, chunk + 1, L, H, h, D, tokb, col0, v, g, cidb, h_prev);
        }
        carry_chunk<D, TIn, RES>(fa, Sv, chunk, L, H, h, tokb, col, rho_c, red[0], vls[0], gls[0], hl0,
                                  o, h_out, x_next);
        if (!has1) break;
        // buffer 1 was last read before this chunk's barrier, which every wave has passed
        store_vg<TIn, RES>(vg, vls[1], gls[1], hl1);
        const bool has2 = chunk + 2 < Nc;
        if (has2) {
            load_frags<D, TIn>(fa, chunk + 2, L, H, h, tokb, q, k, W, M, cidb);
            load_vg<TIn, RES>(vg, chunk + 2, L, H, h, D, tokb, col0, v, g, cidb, h_prev);
        }
        carry_chunk<D, TIn, RES>(fb, Sv, chunk + 1, L, H, h, tokb, col, rho_c, red[1], vls[1], gls[1],
                                  hl1, o, h_out, x_next);
        if (has2) store_vg<TIn, RES>(vg, vls[0], gls[0], hl0);
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
#define CARRY(DD, T, R)                                                                            \
    launch_kernel((k_scan_carry<DD, T, R>), grid, dim3(256), 0, s, (const T *)q,             \
                       (const T *)k, (const T *)v, L, H, Nc, ws.W, ws.M, ws.g, s_init, s_final,   \
                       out.o, out.h_prev, out.rho, out.h_out, out.x_next)
#define CARRY_R(DD, T)                                                                             \
    do {                                                                                           \
        if (res == 0) CARRY(DD, T, 0); else if (res == 1) CARRY(DD, T, 1); else CARRY(DD, T, 2);   \
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
