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
// bf16 path, long inputs (>= 1024 tokens): k_proj_wide, 256 tokens x 384
// packed columns (one head's q|k|v for D = 128) per workgroup, eight waves of
// 128 x 96, and k_gates for the 2H gate columns.  Short inputs (decode steps):
// k_proj_bf16, 256 x 128 tiles of four 128 x 64 waves with the gate columns as
// one more tile.  Both stage operands through LDS with XOR-swizzled direct
// loads and accumulate in fp32.  The packed weight puts each head's q|k|v rows
// in whole 128-row sections, so every output tile holds complete head
// sections for the normalisation.
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
// Block tile 256 (tokens) x 128 (packed output columns) x 64 (channels); four
// waves in a 2 x 2 arrangement each own 128 x 64 of the tile as 4 x 2 MFMA
// 32x32x16 accumulator tiles (128 fp32 per lane).  Operand tiles move from
// global memory straight into LDS (global_load_lds_dwordx4: lane i of a wave
// instruction fills the 16 bytes at the wave's LDS base + 16 i), three k-blocks
// deep, so two k-blocks are in flight while one is multiplied.  The LDS tiles
// are XOR-swizzled by choosing, for each lane, the global 16-byte chunk that
// belongs at its LDS position.  Gate tiles (the 2H gate columns) come first in
// the grid and only run the MFMAs of the columns they use, so they finish
// early instead of adding a round.
constexpr int BM_BF = 256, BK_BF = 64, STAGES = 3;
constexpr int A_ELEMS = BM_BF * BK_BF;  // bf16 elements of the A tile (32 KB)
constexpr int B_ELEMS = BN * BK_BF;     // bf16 elements of the B tile (16 KB)
constexpr int STAGE_ELEMS = A_ELEMS + B_ELEMS;

// 16-byte chunk `ch` (0..7) of row `r` of a 64-wide bf16 tile, XOR-swizzled by
// row.  A 128-byte row covers half of the 64 LDS banks, so rows of equal parity
// share a bank half; keying the swizzle on r / 2 makes 16 consecutive rows
// reading the same chunk land on 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz_key(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int swz(int r, int ch) { return r * BK_BF + ((ch ^ swz_key(r)) << 3); }

// Direct loads of loads [I0, I1) of one k-block (starting at channel k0) into
// one stage: loads 0..7 fill the A tile (2048 chunks; wave w's load i covers
// LDS chunks [(4 i + w) 64, +64), i.e. rows 8 (4 i + w) .. + 7), loads 8..11 the
// B tile (1024 chunks, same rule).  LDS chunk p holds row p / 8, logical chunk
// (p % 8) ^ swz_key(row).  Only the first NA of the A loads are issued: with at
// most 64 tokens (NA = 2) the rows they skip are all past M.
template <int I0, int I1, int NA, int AE = A_ELEMS>
__device__ __forceinline__ void gemm_issue(bf16 *stage, const bf16 *__restrict__ x,
                                           const bf16 *__restrict__ Wp, int lane, int wave, int m0,
                                           int n0, int M, int K, int b_rows, int k0) {
#pragma unroll
    for (int i = I0; i < I1; ++i) {
        if (i < 8) {
            if (i >= NA) continue;
            const int base = (4 * i + wave) * 64, p = base + lane;
            const int r = p >> 3, ch = (p & 7) ^ swz_key(r);
            const int m = min(m0 + r, M - 1);   // tail rows re-read the last row; never stored
            __builtin_amdgcn_global_load_lds(x + (int64_t)m * K + k0 + ch * 8,
                                             (lds_void *)(stage + base * 8), 16, 0, 0);
        } else {
            const int base = (4 * (i - 8) + wave) * 64, p = base + lane;
            const int r = p >> 3, ch = (p & 7) ^ swz_key(r);
            const int rr = min(r, b_rows - 1);   // gate tile: unused rows repeat a used one
            __builtin_amdgcn_global_load_lds(Wp + (int64_t)(n0 + rr) * K + k0 + ch * 8,
                                             (lds_void *)(stage + AE + base * 8), 16, 0, 0);
        }
    }
}

// Operand fragments of one k-block (4 k-steps x (4 A + 2 B) 32x32x16 fragments).
struct KFrags {
    bf16x8 a[BK_BF / 16][4], b[BK_BF / 16][2];
};

// AE: bf16 elements of the stage's A area; TMR: A tiles read (the A area of
// AE = 64 x 64 holds rows 0 .. 63 only, read by every wave).
template <int AE = A_ELEMS, int TMR = 4>
__device__ __forceinline__ void read_frags_step(KFrags &F, const bf16 *stage, int s, int lane, int wm, int wn) {
    const bf16 *Ab = stage, *Bb = stage + AE;
    const int ch = 2 * s + (lane >> 5);
    const int wrow = AE == A_ELEMS ? wm * 128 : 0;
#pragma unroll
    for (int tm = 0; tm < TMR; ++tm)
        F.a[s][tm] = *reinterpret_cast<const bf16x8 *>(Ab + swz(wrow + tm * 32 + (lane & 31), ch));
#pragma unroll
    for (int tn = 0; tn < 2; ++tn)
        F.b[s][tn] = *reinterpret_cast<const bf16x8 *>(Bb + swz(wn * 64 + tn * 32 + (lane & 31), ch));
}

// The k-loop of one tile, software-pipelined over NST LDS stages and two
// fragment register sets.  Iteration kb: wait until k-block kb+1 has landed
// (kb+2 .. kb+NST-1 may stay in flight), barrier, then per k-step: issue a
// quarter of k-block kb+NST's direct loads (into the stage that held kb, whose
// fragments were read during the previous iteration), read k-block kb+1's
// fragments into the idle register set, and run k-block kb's MFMAs from the
// other set.  The direct loads go out in small groups between MFMAs so that
// issuing them never fills the memory pipeline's queue, which would stall the
// wave's MFMA issue.  Past the end the loads re-read the last k-block into a
// free stage, so every iteration has the same shape.  GATE: only the 32-column
// MFMA tiles holding used gate columns are computed (a wave-uniform
// condition).  NA < 8: only the tile's first 32 NA token rows can be valid; the
// other A rows are neither loaded nor multiplied (their outputs are never
// stored), and the wait counts follow the NA + 4 loads per k-block.  With
// NA = 2 (at most 64 tokens) a stage holds only those 64 A rows and the B
// tile (24 KB), so six stages fit where three full ones did: five k-blocks
// in flight instead of two, for a tile that streams its weights with little
// arithmetic per byte.
template <int NA> struct KloopCfg {
    static constexpr int AE = NA == 2 ? 64 * BK_BF : A_ELEMS;   // bf16 elements of a stage's A area
    static constexpr int SE = AE + B_ELEMS;                       // bf16 elements per stage
    static constexpr int NST = NA == 2 ? 6 : STAGES;
};
static_assert(KloopCfg<2>::NST * KloopCfg<2>::SE <= STAGES * STAGE_ELEMS, "the NA = 2 stages fit the LDS");
// K is the row stride of x and Wp; the loop covers channels [0, Kn) of the
// rows as given (a k-range split passes x and Wp advanced to its first channel).
template <bool GATE, int NA>
__device__ __forceinline__ void gemm_kloop(f32x16 (&acc)[4][2], bf16 *stages, const bf16 *__restrict__ x,
                                           const bf16 *__restrict__ Wp, int lane, int wave, int wm,
                                           int wn, int m0, int n0, int M, int K, int b_rows,
                                           int gate_cols, int Kn) {
    using CF = KloopCfg<NA>;
    constexpr int NST = CF::NST, SE = CF::SE, AE = CF::AE;
    const int nkb = Kn / BK_BF;   // >= 1
    auto kblock = [&](int kb) { return min(kb, nkb - 1) * BK_BF; };
    constexpr int NL = NA + 4;          // direct loads per k-block
    static_assert((NST - 1) * NL < 64, "the vector-memory counter holds 0..63");
    // 32-row A tiles a wave multiplies: each A load covers 8 rows in each of the
    // 4 waves, so NA loads cover the rows of NA tiles
    constexpr int TM = NA >= 8 ? 4 : NA;
    static_assert(NA == 8 || NA == 2, "NA < 8 covers rows 0 .. 63 of the tile only");
    // NA = 2: the 64 rows are one row of waves' work, so the two rows of waves
    // split each k-block instead: waves wm take its k-steps 2 wm and 2 wm + 1
    // (partial sums added in the epilogue)
    const bool rows_on = true;
    auto mine = [&](int s) { return NA >= 8 || (s >> 1) == wm; };
#pragma unroll
    for (int st = 0; st < NST; ++st)
        gemm_issue<0, 12, NA, AE>(stages + st * SE, x, Wp, lane, wave, m0, n0, M, K, b_rows, kblock(st));
    wait_vmcnt<(NST - 1) * NL>();   // k-block 0 landed
    lds_barrier();
    const bool tn_on[2] = {!GATE || wn * 64 < gate_cols, !GATE || wn * 64 + 32 < gate_cols};
    KFrags f0, f1;
#pragma unroll
    for (int s = 0; s < BK_BF / 16; ++s)
        if (mine(s)) read_frags_step<AE, TM>(f0, stages, s, lane, wm, wn);

    auto step = [&](int kb, const KFrags &cur, KFrags &nxt) __attribute__((always_inline)) {
        wait_vmcnt<(NST - 2) * NL>();   // k-block kb+1 landed (kb+2 .. kb+NST-1 may remain)
        lds_barrier();      // ... for every wave; every wave has read k-block kb's fragments
        bf16 *ld_stage = stages + (kb % NST) * SE;           // receives kb+NST
        const bf16 *rd_stage = stages + ((kb + 1) % NST) * SE;
        const int kn = kblock(kb + NST);
#pragma unroll
        for (int s = 0; s < BK_BF / 16; ++s) {
            if (s == 0) gemm_issue<0, 3, NA, AE>(ld_stage, x, Wp, lane, wave, m0, n0, M, K, b_rows, kn);
            if (s == 1) gemm_issue<3, 6, NA, AE>(ld_stage, x, Wp, lane, wave, m0, n0, M, K, b_rows, kn);
            if (s == 2) gemm_issue<6, 9, NA, AE>(ld_stage, x, Wp, lane, wave, m0, n0, M, K, b_rows, kn);
            if (s == 3) gemm_issue<9, 12, NA, AE>(ld_stage, x, Wp, lane, wave, m0, n0, M, K, b_rows, kn);
            if (mine(s)) {
                read_frags_step<AE, TM>(nxt, rd_stage, s, lane, wm, wn);
#pragma unroll
                for (int tn = 0; tn < 2; ++tn)
                    if (tn_on[tn] && rows_on)
#pragma unroll
                        for (int tm = 0; tm < TM; ++tm)
                            acc[tm][tn] = mfma32x32x16(cur.a[s][tm], cur.b[s][tn], acc[tm][tn]);
            }
        }
    };
    for (int kb = 0; kb < nkb; kb += 2) {
        step(kb, f0, f1);
        if (kb + 1 < nkb) step(kb + 1, f1, f0);
    }
    wait_vmcnt<0>();   // the re-reads past the end land before LDS is reused
}

// One workgroup per CU (the three LDS stages take 144 KB), i.e. one wave per
// SIMD: the compiler may use the whole register file for latency hiding.  NA:
// A loads per k-block (8; 2 for at most 64 tokens, e.g. a decode batch).
template <int D, int NA>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_proj_bf16(const bf16 *__restrict__ x,
                                                   const bf16 *__restrict__ Wp, int M, int K, int H,
                                                   int m_tiles, int n_main, bf16 *q, bf16 *k, bf16 *v,
                                                   float *alpha, float *beta, float alpha_lo,
                                                   float eps) {
    constexpr int LDS_MAIN = STAGES * STAGE_ELEMS * 2;          // bytes
    constexpr int LDS_EPI = 128 * CS_LD * 4 + 2 * 128 * 4;      // one 128-row half of the tile
    constexpr int LDS_BYTES = LDS_MAIN > LDS_EPI ? LDS_MAIN : LDS_EPI;
    __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];
    bf16 *stages = reinterpret_cast<bf16 *>(smem);

    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);   // wave-uniform
    const int wm = wave >> 1, wn = wave & 1;
    // tile order: m_tiles gate tiles, then the main tiles m-fastest
    const int id = blockIdx.x;
    const bool gate = id < m_tiles;
    const int m_tile = gate ? id : (id - m_tiles) % m_tiles;
    const int n_tile = gate ? n_main : (id - m_tiles) / m_tiles;
    const int m0 = m_tile * BM_BF, n0 = n_tile * BN;
    const int gate_cols = 2 * H;          // used columns of the gate tile
    const int b_rows = gate ? ((gate_cols + 31) / 32) * 32 : BN;

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    if (gate) gemm_kloop<true, NA>(acc, stages, x, Wp, lane, wave, wm, wn, m0, n0, M, K, b_rows, gate_cols, K);
    else gemm_kloop<false, NA>(acc, stages, x, Wp, lane, wave, wm, wn, m0, n0, M, K, b_rows, gate_cols, K);
    __syncthreads();   // all waves done reading the operand stages

    // epilogue in two 128-row halves through an fp32 tile in LDS (reuses the operand buffers)
    float *Cs = reinterpret_cast<float *>(smem);
    float *red = Cs + 128 * CS_LD;
    if constexpr (NA == 2) {
        // rows 0 .. 63: the k-step halves of the two rows of waves, added in the order wm = 0, 1; rows
        // 64 .. 127 (never stored) zero
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            if (wm == pass) {
#pragma unroll
                for (int tm = 0; tm < 4; ++tm)
#pragma unroll
                    for (int tn = 0; tn < 2; ++tn)
#pragma unroll
                        for (int e = 0; e < 16; ++e) {
                            if (pass == 1 && tm >= 2) continue;
                            const int r = tm * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                            const int c = wn * 64 + tn * 32 + (lane & 31);
                            const float a = tm < 2 ? acc[tm][tn][e] : 0.f;
                            Cs[r * CS_LD + c] = pass ? Cs[r * CS_LD + c] + a : a;
                        }
            }
            __syncthreads();
        }
        proj_epilogue<D, 128, bf16>(Cs, red, m0, n0, M, H, q, k, v, alpha, beta, alpha_lo, eps);
        return;
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        if (m0 + half * 128 >= M) break;   // no valid row in this half (uniform)
        if (wm == half) {
#pragma unroll
            for (int tm = 0; tm < 4; ++tm)
#pragma unroll
                for (int tn = 0; tn < 2; ++tn)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int r = tm * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                        const int c = wn * 64 + tn * 32 + (lane & 31);
                        Cs[r * CS_LD + c] = acc[tm][tn][e];
                    }
        }
        __syncthreads();
        proj_epilogue<D, 128, bf16>(Cs, red, m0 + half * 128, n0, M, H, q, k, v, alpha, beta, alpha_lo,
                                    eps);
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// decode-size projection (at most 64 tokens) split over the channels
// ---------------------------------------------------------------------------
// With at most 64 tokens the projection streams the 25 MB of packed weights
// (d = 2048) with little arithmetic per byte, and one workgroup per 128-column
// tile leaves 80% of the CUs idle.  k_proj_dpart splits the channels into S
// equal ranges: workgroup (column tile j, range s) runs the 64-token k-loop of
// k_proj_bf16 over its range and stores the fp32 tile to part[s][M][NP]
// (NP = packed rows; only the M token rows).  The decode step that consumes
// them (k_decode with partials) adds the S partials of each element in the
// order s = 0 .. S-1 and applies the epilogue itself (per-head norms of q and
// k, gates, bf16 rounding): each of its workgroups owns one (sequence, head).
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_proj_dpart(
    const bf16 *__restrict__ x, const bf16 *__restrict__ Wp, int M, int K, int Kn, int H, int n_main, int NP,
    float *__restrict__ part) {
    constexpr int LDS_MAIN = STAGES * STAGE_ELEMS * 2;
    __shared__ __attribute__((aligned(16))) char smem[LDS_MAIN];
    bf16 *stages = reinterpret_cast<bf16 *>(smem);
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int n_tile = blockIdx.x, s = blockIdx.y;
    const bool gate = n_tile == n_main;
    const int n0 = n_tile * BN, k0 = s * Kn;
    const int gate_cols = 2 * H;
    const int b_rows = gate ? ((gate_cols + 31) / 32) * 32 : BN;
    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    if (gate) gemm_kloop<true, 2>(acc, stages, x + k0, Wp + k0, lane, wave, wm, wn, 0, n0, M, K, b_rows, gate_cols, Kn);
    else gemm_kloop<false, 2>(acc, stages, x + k0, Wp + k0, lane, wave, wm, wn, 0, n0, M, K, b_rows, gate_cols, Kn);
    __syncthreads();   // all waves done reading the operand stages
    // the two rows of waves hold the k-step halves of rows 0 .. 63: added in the order wm = 0, 1
    float *Cs = reinterpret_cast<float *>(smem);
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
        if (wm == pass) {
#pragma unroll
            for (int tm = 0; tm < 2; ++tm)
#pragma unroll
                for (int tn = 0; tn < 2; ++tn)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int r = tm * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                        const int c = wn * 64 + tn * 32 + (lane & 31);
                        Cs[r * CS_LD + c] = pass ? Cs[r * CS_LD + c] + acc[tm][tn][e] : acc[tm][tn][e];
                    }
        }
        __syncthreads();
    }
    // rows 0 .. M-1 of the tile: 32 float4 per row
    float *dst = part + (int64_t)s * M * NP + n0;
    for (int idx = t; idx < M * (BN / 4); idx += 256) {
        const int r = idx / (BN / 4), c4 = idx % (BN / 4);
        const float *src = Cs + r * CS_LD + 4 * c4;
        *reinterpret_cast<float4 *>(dst + (int64_t)r * NP + 4 * c4) = make_float4(src[0], src[1], src[2], src[3]);
    }
}

// ---------------------------------------------------------------------------
// wide bf16 MFMA GEMM for long inputs
// ---------------------------------------------------------------------------
// Block tile 384 packed columns (q|k|v of one head for D = 128, of two heads for
// D = 64) x 256 tokens x 64 channels.  Eight waves (two per SIMD) own 96
// columns x 128 tokens each as 3 x 4 MFMA 32x32x16 tiles (192 fp32 accumulators
// per lane).  Per flop this tile moves 45% fewer bytes from L2 into the CU than
// a 256 x 128 tile, and each wave reads 22% fewer LDS bytes than with 128 x 64
// wave tiles; the second wave on each SIMD covers the other's LDS latency.
// The product is formed transposed (Wp rows as the A operand, tokens as B), so
// that a lane holds, for one token, runs of four consecutive output columns:
// the per-head norms then sum mostly inside the lane, and results leave as
// 8-byte pieces of output rows through a staging tile in LDS.
// With one head per column tile, a sequence of 4096 tokens and 16 heads is
// exactly 256 tiles, one per CU.
// Gate columns (GZ): the 2H <= 32 gate rows are one more 32-row A tile.  Column
// tile j takes the gate product over one pair of channel blocks (2p, 2p+1;
// d = H D gives at most two blocks per column tile, and the pairs p of the
// column tiles are a permutation of all pairs) and writes it as an fp32 partial
// zp[j][2H][M]; the consumer sums the partials of a token in tile order.  The
// k-loop of tile j starts at block 2p, so both gate blocks are in the two
// stages after the prologue, where the gate MFMAs run before the main
// accumulators are live.  Without GZ the gate columns run in k_gates.
constexpr int WM = 256, WN = 384, WK = 64, WSTAGES = 2;
constexpr int WA = WM * WK, WB = WN * WK, WSTAGE = WA + WB;   // bf16 elements per stage
constexpr int WOUT_LD = WN + 4;   // bf16 row stride of the output staging tile (776 bytes)
constexpr int WCOLS = 96;         // columns per wave
constexpr int W_LDS_MAIN = WSTAGES * WSTAGE * 2;
constexpr int W_LDS_EPI = 128 * WOUT_LD * 2;   // staging tile; the sums of squares (<= 24 KiB) come first
static_assert(W_LDS_EPI <= W_LDS_MAIN, "epilogue buffers reuse the operand stages");
// Direct loads per wave per k-block (10), of which the token tile's (4): wave w's
// load i covers LDS chunks [(8 i + w) 64, +64) of its tile.  LDS chunk p holds row
// p / 8, logical chunk (p % 8) ^ ((row / 2) % 8).  Token rows past M re-read the
// last token and column rows past the packed q|k|v rows re-read the last used
// one; their results are never stored.
constexpr int WLOADS = (WA + WB) / 8 / 64 / 8;
constexpr int WLOADS_A = WA / 8 / 64 / 8;

// 16-byte chunk `ch` (0..7) of row `r` of a 64-wide bf16 tile (128-byte rows),
// XOR-swizzled by r / 2: 16 consecutive rows reading the same chunk then hit 16
// distinct 16-byte bank groups.
__device__ __forceinline__ int wswz(int r, int ch) { return r * WK + ((ch ^ ((r >> 1) & 7)) << 3); }

struct WideSrc {
    unsigned off[WLOADS];
};
// With a row list (rows != nullptr) token row m of the tile is x row rows[m],
// and the token offsets are taken from the start of x instead of the tile's
// first row.
__device__ __forceinline__ WideSrc wide_src(int lane, int wave, int m0, int M, int K, int n_rows,
                                            const int *rows = nullptr) {
    WideSrc s;
#pragma unroll
    for (int i = 0; i < WLOADS; ++i) {
        const int base = (8 * (i < WLOADS_A ? i : i - WLOADS_A) + wave) * 64, p = base + lane;
        const int r = p >> 3, ch = (p & 7) ^ ((r >> 1) & 7);
        int row;
        if (i < WLOADS_A) row = rows ? rows[min(m0 + r, M - 1)] : min(m0 + r, M - 1) - m0;
        else row = min(r, n_rows - 1);
        s.off[i] = (unsigned)(((unsigned)row * (unsigned)K + ch * 8) * 2u);
    }
    return s;
}
__device__ __forceinline__ void wide_load(int i, bf16 *stage, const WideSrc &src, const bf16 *xk, const bf16 *wk,
                                          int wave) {
    if (i < WLOADS_A) dma16_async_s(xk, src.off[i], stage + (8 * i + wave) * 64 * 8);
    else dma16_async_s(wk, src.off[i], stage + WA + (8 * (i - WLOADS_A) + wave) * 64 * 8);
}

// Fragments of one k-step: 3 column tiles (A operand) and 4 token tiles (B).
struct WFr {
    bf16x8 a[3], b[4];
};
__device__ __forceinline__ void wide_read(WFr &F, const bf16 *stage, int ks, int lane, int wt, int wf) {
    const int ch = 2 * ks + (lane >> 5);
#pragma unroll
    for (int ft = 0; ft < 3; ++ft)
        F.a[ft] = *reinterpret_cast<const bf16x8 *>(stage + WA + wswz(wf * WCOLS + ft * 32 + (lane & 31), ch));
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
        F.b[tt] = *reinterpret_cast<const bf16x8 *>(stage + wswz(wt * 128 + tt * 32 + (lane & 31), ch));
}

// Epilogue of one wave.  WF (the wave's column quarter) is a template
// parameter so that every section index is a compile-time constant; a tile
// starts at a q section, so section s has kind s % 3.
//   1. per-token sums of squares of each q/k section this wave touches (in-lane
//      sums plus one exchange between lane halves) into LDS;
//   2. the per-(token, section) scales 1/sqrt(sum + eps), once, in registers;
//   3. two passes of 128 tokens (all eight waves stage 2 token tiles each) through
//      a bf16 staging tile, then 16-byte stores of whole output row sections.
template <int D, int WF>
__device__ __forceinline__ void wide_epilogue(const f32x16 (&acc)[3][4], char *smem, int lane, int wt, int t,
                                              int m0, int n0, int M, int H, bf16 *q, bf16 *k, bf16 *v,
                                              float eps, const int *rows) {
    constexpr int NSEC = WN / D;
    constexpr int S0 = (WF * WCOLS) / D, S1 = (WF * WCOLS + WCOLS - 1) / D, NS = S1 - S0 + 1;
    float *red = reinterpret_cast<float *>(smem);   // [4 column quarters][NSEC][WM tokens]
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        float ss[NS];
#pragma unroll
        for (int i = 0; i < NS; ++i) ss[i] = 0.f;
#pragma unroll
        for (int ft = 0; ft < 3; ++ft) {
            const int si = (WF * WCOLS + ft * 32) / D - S0;
#pragma unroll
            for (int i = 0; i < 16; ++i) ss[si] += acc[ft][tt][i] * acc[ft][tt][i];
        }
        const int tok = wt * 128 + tt * 32 + (lane & 31);
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            if ((S0 + i) % 3 == 2) continue;   // v sections: no norm
            const float tot = ss[i] + __shfl_xor(ss[i], 32);
            if (lane < 32) red[(WF * NSEC + S0 + i) * WM + tok] = tot;
        }
    }
    lds_barrier();
    // scaled bf16 results, [ft][tt][g] = 4 consecutive columns of one token;
    // the fp32 accumulators are dead from here on
    bf16x4 res[3][4][4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        const int tok = wt * 128 + tt * 32 + (lane & 31);
        float sc[NS];
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const int s = S0 + i;
            sc[i] = 1.f;
            if (s % 3 != 2) {   // q or k section: L2 norm over the section
                float tot = 0.f;
#pragma unroll
                for (int w = 0; w < 4; ++w)
                    if (s * D < (w + 1) * WCOLS && (s + 1) * D > w * WCOLS) tot += red[(w * NSEC + s) * WM + tok];
                sc[i] = 1.f / sqrtf(tot + eps);
            }
        }
#pragma unroll
        for (int ft = 0; ft < 3; ++ft) {
            const float scale = sc[(WF * WCOLS + ft * 32) / D - S0];
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int j = 0; j < 4; ++j) res[ft][tt][g][j] = (bf16)(acc[ft][tt][4 * g + j] * scale);
        }
    }
    lds_barrier();   // the staging tile below overwrites the sums
    bf16 *out_s = reinterpret_cast<bf16 *>(smem);
    constexpr int PIECES = WN / 8;   // 16-byte pieces per staged token row
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            const int tt = 2 * pass + h2;
            const int row = wt * 64 + h2 * 32 + (lane & 31);
#pragma unroll
            for (int ft = 0; ft < 3; ++ft)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    *reinterpret_cast<bf16x4 *>(out_s + row * WOUT_LD + WF * WCOLS + ft * 32 + 8 * g +
                                                4 * (lane >> 5)) = res[ft][tt][g];
        }
        lds_barrier();
        // Staging row r holds token (r / 64) 128 + 64 pass + r % 64 of the tile.
        // Threads 0..383 each own one 16-byte column piece of the rows and store
        // 16 rows, 4 at a time; the destination row advances by a fixed stride.
        if (t < 8 * PIECES) {
            const int r0 = t / PIECES, f = (t % PIECES) * 8, n = n0 + f;
            const int head = n / (3 * D), kind = (n % (3 * D)) / D, off = n % D;
            const int64_t rs = (int64_t)H * D;   // elements between consecutive tokens
            bf16 *dst0 = (kind == 0 ? q : (kind == 1 ? k : v)) + (int64_t)head * D + off;
            bf16 *dst = dst0 + (int64_t)(m0 + pass * 64 + r0) * rs;
            const bool col_ok = head < H;
            const int mb = m0 + pass * 64 + r0;
#pragma unroll
            for (int i0 = 0; i0 < 16; i0 += 4) {
                uint4 val[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = r0 + 8 * (i0 + i);
                    const bf16 *srow = out_s + r * WOUT_LD + f;
                    const uint2 lo = *reinterpret_cast<const uint2 *>(srow);
                    const uint2 hi = *reinterpret_cast<const uint2 *>(srow + 4);
                    val[i] = make_uint4(lo.x, lo.y, hi.x, hi.y);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int ii = i0 + i, dm = (ii / 8) * 128 + 8 * (ii % 8);   // token offset of row r0 + 8 ii
                    if (col_ok && mb + dm < M) {
                        bf16 *d2 = rows ? dst0 + (int64_t)rows[mb + dm] * rs : dst + dm * rs;
                        *reinterpret_cast<uint4 *>(d2) = val[i];
                    }
                }
            }
        }
        if (pass == 0) lds_barrier();   // every staged row read before the second pass overwrites
    }
}

// ROWS: the tile's token rows are the entries m0 .. of the row list `rows`
// (count in *rows_count, read on the device), gathered from x and scattered to
// q, k, v and the gate partials; tiles past the count return at once.  M stays
// the row stride of the gate partials.
// RAW: also store the raw fp32 projections (yraw) before the epilogue.
template <int D, bool GZ, bool ROWS, bool RAW>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_proj_wide(
    const bf16 *__restrict__ x, const bf16 *__restrict__ Wp, int M, int K, int H, int m_tiles, int n_tiles,
    bf16 *q, bf16 *k, bf16 *v, float eps, float *__restrict__ zp, const int *__restrict__ rows,
    const int *__restrict__ rows_count, float *__restrict__ yraw, int64_t ldy) {
    __shared__ __attribute__((aligned(16))) char smem[W_LDS_MAIN];
    bf16 *stages = reinterpret_cast<bf16 *>(smem);

    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wt = wave >> 2, wf = wave & 3;
    // Workgroup ids are dealt to the 8 XCDs round-robin.  XCD x takes the
    // column tiles x, x + 8, ..., token tile by token tile (for each token
    // tile, its column tiles in turn), so its L2 serves few column tiles, the
    // column tiles of one token tile run side by side and read its x lines
    // once, and column tile n (one head for 128-wide heads) is written on XCD
    // n mod 8, where the scan kernels of that head run.  Otherwise each XCD
    // takes a contiguous run of tiles, column-tile major.
    const int ntot = m_tiles * n_tiles;
    const int id = blockIdx.x;
    const bool x8 = n_tiles % 8 == 0;
    int n_tile, m_tile;
    if (x8) {
        const int kx = id / 8, per = n_tiles / 8;
        n_tile = id % 8 + 8 * (kx % per);
        m_tile = kx / per;
    } else {
        const int tix = (ntot % 8 == 0) ? (id % 8) * (ntot / 8) + id / 8 : id;
        n_tile = tix / m_tiles;
        m_tile = tix % m_tiles;
    }
    const int m0 = m_tile * WM, n0 = n_tile * WN;
    const int qkv_rows = H * 3 * D;
    const int n_rows = min(WN, qkv_rows - n0);
    int Mv = M;   // rows of this launch
    if constexpr (ROWS) {
        Mv = *rows_count;
        if (m0 >= Mv) return;   // uniform over the workgroup, before any barrier
    }

    const WideSrc src = wide_src(lane, wave, m0, Mv, K, n_rows, ROWS ? rows : nullptr);
    const bf16 *xb = x + (ROWS ? (int64_t)0 : (int64_t)m0 * K), *wb = Wp + (int64_t)n0 * K;
    const int nkb = K / WK;
    // channel offset of the i-th block of this tile's k order (blocks kb0,
    // kb0+1, ... wrapping around); past the end it repeats the last one.  The
    // gate block pair of column tile n is pair n, or with the XCD dealing above
    // pair r (n mod 8) + n / 8 (r = n_tiles / 8), so that the column tiles of
    // one XCD start next to each other in k and share their token tile's lines
    // in L2.
    const int gpair = x8 ? (n_tiles / 8) * (n_tile % 8) + n_tile / 8 : n_tile;
    const int kb0 = GZ ? 2 * gpair : 0;
    auto kblock = [&](int i) {
        const int b = kb0 + min(i, nkb - 1);
        return (b < nkb ? b : b - nkb) * WK;
    };

    // prologue: the first two blocks into the two stages
#pragma unroll
    for (int i = 0; i < WLOADS; ++i) wide_load(i, stages, src, xb + kblock(0), wb + kblock(0), wave);
    if (nkb > 1) {
#pragma unroll
        for (int i = 0; i < WLOADS; ++i)
            wide_load(i, stages + WSTAGE, src, xb + kblock(1), wb + kblock(1), wave);
    }
    if constexpr (GZ) {
        // gate partial of this wave's 32 tokens (token tile wf of its half) over
        // the tile's gate blocks: gate rows as A (8 fragments straight from
        // global memory), the staged token tile as B
        const bf16 *Wg = Wp + qkv_rows_padded(H, D) * K;   // 128-row gate tile
        const bf16 *gsrc = Wg + (int64_t)(lane & 31) * K + kb0 * WK + 8 * (lane >> 5);
        const bool two = kb0 + 1 < nkb;   // the tile's second gate block exists
        bf16x8 ga[8];
#pragma unroll
        for (int gk = 0; gk < 8; ++gk)
            ga[gk] = *reinterpret_cast<const bf16x8 *>(gsrc + 16 * (two ? gk : gk % 4));
        wait_vmcnt<0>();
        lds_barrier();
        f32x16 gacc;
#pragma unroll
        for (int e = 0; e < 16; ++e) gacc[e] = 0.f;
        auto gate_steps = [&](int st) __attribute__((always_inline)) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int ch = 2 * ks + (lane >> 5);
                const bf16x8 b = *reinterpret_cast<const bf16x8 *>(stages + st * WSTAGE +
                                                                   wswz(wt * 128 + wf * 32 + (lane & 31), ch));
                gacc = mfma32x32x16(ga[4 * st + ks], b, gacc);
            }
        };
        gate_steps(0);
        if (two) gate_steps(1);
        // C lane layout: token (lane % 32), gate rows 8 (e / 4) + 4 (lane / 32) + e % 4
        const int gh2 = 2 * H, tok = m0 + wt * 128 + wf * 32 + (lane & 31);
        if (tok < Mv) {
            float *zdst = zp + (int64_t)n_tile * gh2 * M + (ROWS ? rows[tok] : tok);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int r = 8 * (e / 4) + 4 * (lane >> 5) + e % 4;
                if (r < gh2) zdst[(int64_t)r * M] = gacc[e];
            }
        }
    } else {
        if (nkb > 1) wait_vmcnt<WLOADS>();   // the first stage's loads (the second may be in flight)
        else wait_vmcnt<0>();
    }

    f32x16 acc[3][4];
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    // k-loop over two stages of 64 channels: step i waits for its own loads,
    // barriers (every wave is also done with step i-1, whose stage takes block
    // i+1), then runs four k-steps of 12 MFMAs, reading the next k-step's
    // fragments into the other register set, with block i+1's ten direct loads
    // spread between the MFMAs.  Step 0 finds both stages loaded by the prologue.
    auto kstep = [&](auto load_c, int it) __attribute__((always_inline)) {
        constexpr bool LOAD = decltype(load_c)::value;
        if constexpr (LOAD) wait_vmcnt<0>();
        lds_barrier();
        const bf16 *cur = stages + (it & 1) * WSTAGE;
        bf16 *ld = stages + ((it + 1) & 1) * WSTAGE;
        const int k1 = kblock(it + 1);
        WFr fr[2];
        wide_read(fr[0], cur, 0, lane, wt, wf);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (s < 3) wide_read(fr[(s + 1) & 1], cur, s + 1, lane, wt, wf);
#pragma unroll
            for (int j = 0; j < 12; ++j) {
                const int i = 12 * s + j, ft = j / 4, tt = j % 4;
                acc[ft][tt] = mfma32x32x16(fr[s & 1].a[ft], fr[s & 1].b[tt], acc[ft][tt]);
                if (LOAD && i % 4 == 1 && i / 4 < WLOADS) wide_load(i / 4, ld, src, xb + k1, wb + k1, wave);
            }
        }
    };
    kstep(std::false_type(), 0);
    for (int it = 1; it < nkb; ++it) kstep(std::true_type(), it);
    wait_vmcnt<0>();   // the re-reads past the end land before LDS is reused
    __syncthreads();

    if constexpr (RAW) {
        // the raw fp32 projections before the epilogue (for the backward pass): yraw[token][packed row], the
        // q|k|v rows only; a lane's four consecutive rows of a token as one 16-byte store
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const int m = m0 + wt * 128 + tt * 32 + (lane & 31);
            if (m < Mv) {
                const int nl = n0 + wf * WCOLS + 4 * (lane >> 5);
                float *yr = yraw + (int64_t)m * ldy + nl;
#pragma unroll
                for (int ft = 0; ft < 3; ++ft)
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        if (nl + ft * 32 + 8 * g < qkv_rows)
                            *reinterpret_cast<float4 *>(yr + ft * 32 + 8 * g) =
                                float4{acc[ft][tt][4 * g], acc[ft][tt][4 * g + 1], acc[ft][tt][4 * g + 2],
                                       acc[ft][tt][4 * g + 3]};
            }
        }
    }

    switch (wf) {
        case 0: wide_epilogue<D, 0>(acc, smem, lane, wt, t, m0, n0, Mv, H, q, k, v, eps, ROWS ? rows : nullptr); break;
        case 1: wide_epilogue<D, 1>(acc, smem, lane, wt, t, m0, n0, Mv, H, q, k, v, eps, ROWS ? rows : nullptr); break;
        case 2: wide_epilogue<D, 2>(acc, smem, lane, wt, t, m0, n0, Mv, H, q, k, v, eps, ROWS ? rows : nullptr); break;
        default: wide_epilogue<D, 3>(acc, smem, lane, wt, t, m0, n0, Mv, H, q, k, v, eps, ROWS ? rows : nullptr); break;
    }
}

// Gates for long inputs: a = x.wa and b = x.wb for 16 tokens per workgroup.
// Eight waves take the channel steps (32 channels each) round-robin, R per
// round with every operand load of the round issued up front, as MFMA
// 16x16x32 products (tokens x gate columns, operands straight from global
// memory); the partial sums meet in LDS.  NG 16-column tiles cover the 2H gate
// columns.
template <int NG>
__global__ __launch_bounds__(512) void k_gates(const bf16 *__restrict__ x, const bf16 *__restrict__ Wg, int M,
                                               int K, int H, float *alpha, float *beta, float alpha_lo) {
    constexpr int R = NG <= 2 ? 8 : 4;   // channel steps per wave and round
    __shared__ float red[8][16][NG * 16 + 1];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int m0 = blockIdx.x * 16;
    const bf16 *xr = x + (int64_t)min(m0 + (lane & 15), M - 1) * K + 8 * (lane >> 4);
    const bf16 *wr[NG];
#pragma unroll
    for (int c = 0; c < NG; ++c) wr[c] = Wg + (int64_t)min(c * 16 + (lane & 15), 2 * H - 1) * K + 8 * (lane >> 4);
    f32x4 acc[NG];
#pragma unroll
    for (int c = 0; c < NG; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int nsteps = K / 32;
    for (int j0 = wave; j0 < nsteps; j0 += 8 * R) {
        bf16x8 a[R], b[R][NG];
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int kk = min(j0 + 8 * i, nsteps - 1) * 32;
            a[i] = *reinterpret_cast<const bf16x8 *>(xr + kk);
#pragma unroll
            for (int c = 0; c < NG; ++c) b[i][c] = *reinterpret_cast<const bf16x8 *>(wr[c] + kk);
        }
#pragma unroll
        for (int i = 0; i < R; ++i)
            if (j0 + 8 * i < nsteps)
#pragma unroll
                for (int c = 0; c < NG; ++c) acc[c] = mfma16x16x32(a[i], b[i][c], acc[c]);
    }
#pragma unroll
    for (int c = 0; c < NG; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[wave][4 * (lane >> 4) + e][c * 16 + (lane & 15)] = acc[c][e];
    __syncthreads();
    for (int idx = t; idx < 16 * 2 * H; idx += 512) {
        const int r = idx / (2 * H), c = idx % (2 * H), m = m0 + r;
        if (m >= M) continue;
        float z = 0.f;
#pragma unroll
        for (int w = 0; w < 8; ++w) z += red[w][r][c];
        if (c < H) alpha[(int64_t)m * H + c] = alpha_lo + (1.f - alpha_lo) / (1.f + expf(z));
        else beta[(int64_t)m * H + (c - H)] = 1.f / (1.f + expf(-z));
    }
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
        launch_kernel(k_pack<float>, dim3((unsigned)blocks), dim3(threads), 0, s, d, H, D,
                           (const float *)Wq, (const float *)Wk, (const float *)Wv,
                           (const float *)wa, (const float *)wb, (float *)Wpack, total);
    else
        launch_kernel(k_pack<bf16>, dim3((unsigned)blocks), dim3(threads), 0, s, d, H, D,
                           (const bf16 *)Wq, (const bf16 *)Wk, (const bf16 *)Wv, (const bf16 *)wa,
                           (const bf16 *)wb, (bf16 *)Wpack, total);
    return hipGetLastError();
}

// bf16 inputs of at least this many tokens take the wide tiles (k_gates +
// k_proj_wide); shorter ones (decode steps, short prompts) the 256 x 128 tiles,
// which spread a short input over more workgroups.
constexpr int WIDE_MIN_TOKENS = 1024;

bool project_separate_gates(bool f32, int M) { return !f32 && M >= WIDE_MIN_TOKENS; }

hipError_t launch_gates(int M, int d, int H, int D, const void *x, const void *Wpack, float *alpha,
                        float *beta, float alpha_lo, hipStream_t s) {
    const int ng = (2 * H + 15) / 16;
    const bf16 *Wg = (const bf16 *)Wpack + qkv_rows_padded(H, D) * d;
    const dim3 grid((M + 15) / 16);
#define GATES(NG) launch_kernel(k_gates<NG>, grid, dim3(512), 0, s, (const bf16 *)x, Wg, M, d, H, alpha, beta, alpha_lo)
    if (ng <= 1) GATES(1);
    else if (ng <= 2) GATES(2);
    else if (ng <= 4) GATES(4);
    else GATES(8);
#undef GATES
    return hipGetLastError();
}

int decode_k_splits(bool f32, int M, int d) {
    if (f32 || M > 64 || d % BK_BF) return 1;
    const int nkb = d / BK_BF;
    for (int S = 4; S > 1; S /= 2)
        if (nkb % S == 0) return S;
    return 1;
}

size_t decode_part_bytes(bool f32, int M, int d, int H, int D) {
    const int S = decode_k_splits(f32, M, d);
    return S > 1 ? (size_t)S * M * packed_rows(H, D) * 4 : 0;
}

hipError_t launch_project_decode_parts(int M, int d, int H, int D, const void *x, const void *Wpack, float *part,
                                       hipStream_t s) {
    const int S = decode_k_splits(false, M, d);
    if (S < 2 || !part || M < 1) return hipErrorInvalidValue;
    const int n_main = (int)(qkv_rows_padded(H, D) / BN), NP = (int)packed_rows(H, D);
    const dim3 grid1(n_main + 1, S);
#define DPART(DD)                                                                                  \
    launch_kernel(k_proj_dpart<DD>, grid1, dim3(256), 0, s, (const bf16 *)x, (const bf16 *)Wpack, M, d, d / S, H, \
                  n_main, NP, part)
    if (D == 128) DPART(128); else DPART(64);
#undef DPART
    return hipGetLastError();
}

int gate_partials(bool f32, int M, int d, int H) {
    if (!project_separate_gates(f32, M) || 2 * H > 32) return 0;
    return (d / WK + 1) / 2;
}

hipError_t launch_project(bool f32, int M, int d, int H, int D, const void *x, const void *Wpack,
                          void *q, void *k, void *v, float *alpha, float *beta, float alpha_lo,
                          float eps, float *zp, hipStream_t s, const int *rows, const int *rows_count,
                          float *yraw, int64_t ldy) {
    if (rows && (f32 || !project_separate_gates(f32, M) || !zp || (int64_t)M * d * 2 >= (int64_t(1) << 32)))
        return hipErrorInvalidValue;
    if (yraw && (rows || !project_separate_gates(f32, M) || ldy < H * 3 * D || ldy % 4)) return hipErrorInvalidValue;
    const int ntiles = (int)(packed_rows(H, D) / BN);
    if (f32) {
        dim3 grid(ntiles, (M + BM_F - 1) / BM_F);
        if (D == 128)
            launch_kernel(k_proj_f32<128>, grid, dim3(256), 0, s, (const float *)x,
                               (const float *)Wpack, M, d, H, (float *)q, (float *)k, (float *)v,
                               alpha, beta, alpha_lo, eps);
        else
            launch_kernel(k_proj_f32<64>, grid, dim3(256), 0, s, (const float *)x,
                               (const float *)Wpack, M, d, H, (float *)q, (float *)k, (float *)v,
                               alpha, beta, alpha_lo, eps);
    } else if (project_separate_gates(f32, M)) {
        const int m_tiles = (M + WM - 1) / WM, n_tiles = (H * 3 * D + WN - 1) / WN;
#define WIDE(DD, GZ, RW, RAW)                                                                      \
    launch_kernel(k_proj_wide<DD, GZ, RW, RAW>, dim3(m_tiles * n_tiles), dim3(512), 0, s, (const bf16 *)x, \
                  (const bf16 *)Wpack, M, d, H, m_tiles, n_tiles, (bf16 *)q, (bf16 *)k, (bf16 *)v, eps, zp, rows, \
                  rows_count, yraw, ldy)
        if (rows) {
            if (D == 128) WIDE(128, true, true, false); else WIDE(64, true, true, false);
        } else if (zp && yraw) {
            if (D == 128) WIDE(128, true, false, true); else WIDE(64, true, false, true);
        } else if (zp) {
            if (D == 128) WIDE(128, true, false, false); else WIDE(64, true, false, false);
        } else if (yraw) {
            if (D == 128) WIDE(128, false, false, true); else WIDE(64, false, false, true);
        } else {
            if (D == 128) WIDE(128, false, false, false); else WIDE(64, false, false, false);
        }
#undef WIDE
    } else {
        const int m_tiles = (M + BM_BF - 1) / BM_BF;
        const int n_main = (int)(qkv_rows_padded(H, D) / BN);   // the gate tile is n_main
        dim3 grid(m_tiles * (n_main + 1));
#define NARROW(DD, NA)                                                                            \
    launch_kernel(k_proj_bf16<DD, NA>, grid, dim3(256), 0, s, (const bf16 *)x, (const bf16 *)Wpack, M, d, H, \
                  m_tiles, n_main, (bf16 *)q, (bf16 *)k, (bf16 *)v, alpha, beta, alpha_lo, eps)
        if (M <= 64) {
            if (D == 128) NARROW(128, 2); else NARROW(64, 2);
        } else {
            if (D == 128) NARROW(128, 8); else NARROW(64, 8);
        }
#undef NARROW
    }
    return hipGetLastError();
}

}  // namespace gdn
