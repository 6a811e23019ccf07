// gdn_kernels.h -- host-side launchers of the gfx950 kernels (internal).
// Shapes are validated by the C ABI layer before any of these is called.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16;

// Events that the next kernel launch of this thread stamps with its own start
// and end (they ride on the dispatch packet, so they time the kernel alone, not
// the gap before it).  The stage timer arms them for one launch; null otherwise.
struct LaunchEvents {
    hipEvent_t start, stop;
};
LaunchEvents &launch_events();

// Records `msg` as the calling thread's last error (gdn_last_error) and
// returns `status` (a gdn_status).
int set_last_error(int status, const char *msg);

// Every kernel of the library is launched through here; the caller reads the
// launch status with hipGetLastError().
template <typename F, typename... Args>
inline void launch_kernel(F kernel, dim3 grid, dim3 block, unsigned shmem, hipStream_t s, Args... args) {
    LaunchEvents &ev = launch_events();
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, ev.start, ev.stop, 0u, args...);
    ev = LaunchEvents{nullptr, nullptr};
}

// Rows of the packed weight matrix: per head q|k|v (3*D rows), zero rows up to
// a multiple of 128 (qkv_rows_padded), then one 128-row tile holding wa (H
// rows) and wb (H rows) followed by zero rows.
__host__ __device__ inline int64_t qkv_rows_padded(int H, int D) { return ((int64_t)H * 3 * D + 127) / 128 * 128; }
__host__ __device__ inline int64_t packed_rows(int H, int D) { return qkv_rows_padded(H, D) + 128; }

// Wpack[n][c] = W_src[c][col(n)]  (transpose into K-contiguous rows).
hipError_t launch_pack_weights(bool f32, int d, int H, int D, const void *Wq, const void *Wk,
                               const void *Wv, const void *wa, const void *wb, void *Wpack,
                               hipStream_t s);

// X[M, d] x Wpack^T with the fused per-head epilogue (L2 norm of q and k,
// gates alpha/beta, dtype conversion of q/k/v).  When project_separate_gates
// is true, launch_project writes q, k, v only, and the gates come either from
// launch_gates (an independent launch: both read x), or, with zp != nullptr,
// from the GEMM itself as gate_partials(...) fp32 partial pre-activations
// zp[P][2H][M] (P = gate_partials, > 0 required), which the chunk preparation
// sums and turns into alpha and beta.
bool project_separate_gates(bool f32, int M);
int gate_partials(bool f32, int M, int d, int H);
// With rows != nullptr (bf16 wide projection with gate partials only) only the
// tokens rows[0 .. *rows_count) are projected (count read on the device); the
// other tokens' q, k, v and gate partials stay as they are.  With yraw
// (project_separate_gates inputs, no row list) the GEMM also stores the raw
// fp32 projections of the q|k|v columns, before the norms, to yraw[M][ldy].
hipError_t launch_project(bool f32, int M, int d, int H, int D, const void *x, const void *Wpack,
                          void *q, void *k, void *v, float *alpha, float *beta, float alpha_lo,
                          float eps, float *zp, hipStream_t s, const int *rows = nullptr,
                          const int *rows_count = nullptr, float *yraw = nullptr, int64_t ldy = 0);
hipError_t launch_gates(int M, int d, int H, int D, const void *x, const void *Wpack, float *alpha,
                        float *beta, float alpha_lo, hipStream_t s);
// The projection of at most 64 bf16 tokens (a decode step) split over the
// channels: decode_k_splits(...) = S > 1 ranges whose fp32 partial products
// (no epilogue) go to part (decode_part_bytes bytes: [S][M][packed rows]);
// launch_decode with part sums them.  S == 1: not split (use launch_project).
int decode_k_splits(bool f32, int M, int d);
size_t decode_part_bytes(bool f32, int M, int d, int H, int D);
hipError_t launch_project_decode_parts(int M, int d, int H, int D, const void *x, const void *Wpack, float *part,
                                       hipStream_t s);

// Chunk matrices that the backward pass takes from the forward preparation,
// per chunk (regions of a bwd_mats_bytes block): T, P, A [64][64] fp32
// row-major (A = strict_lower(Gam (.) K K^T), P = lower_incl(Gam (.) Q K^T),
// both zero in the rows of tokens past the end of the sequence; T =
// (I + diag(beta) A)^{-1}), the fp64 log-cumsum lg of alpha, gamma = e^lg and
// c = e^(lg_last - lg) [64] fp32; W^T = diag(beta) T^T diag(c) K [64][D] as
// bf16 hi and lo planes, K^T and Q^T [D][64] bf16 (fp32 inputs: hi and lo
// planes; zero for tokens past the end) and M^T = diag(beta) T^T P^T [64][64]
// fp32 (zero in the columns of tokens past the end).
struct PrepBwd {
    float *T, *P, *A;
    double *lg;
    float *gam, *c;
    bf16 *Wth, *Wtl, *Kth, *Ktl, *Qth, *Qtl;
    float *Mt;
};
// Chunk preparation: per (b, h, chunk) decay products, the UT-transform
// inverse and the derived matrices W [D x 64], M [64 x 64], gamma [64]; with
// bwd.T set, also the backward's chunk matrices.
struct ChunkWs {
    float *W;    // per chunk: bf16 hi plane [D][64] then bf16 lo plane [D][64] (D*64*4 bytes)
    float *M;    // per chunk: bf16 hi plane [64][64] then bf16 lo plane [64][64]
    float *g;    // per chunk: gamma [64] fp32
    PrepBwd bwd = {};
};
// Gates of the chunk preparation: alpha/beta [B*L, H], or (zp != nullptr) the
// P partial pre-activations zp[P][2H][B*L] of the projection, summed in order
// p = 0..P-1, with alpha = lo + (1 - lo) sigmoid(-z_a), beta = sigmoid(z_b);
// the gates formed from zp are stored to alpha_out/beta_out [B*L, H] when
// those are given (so that a caller can read the gates the scan used).
struct GateSrc {
    const float *alpha, *beta;
    const float *zp;
    int P;
    float alpha_lo;
    float *alpha_out, *beta_out;
};
hipError_t launch_scan_prep(bool f32, int B, int L, int H, int D, const void *q, const void *k,
                            GateSrc gates, ChunkWs ws, hipStream_t s);

// Outputs of the carry: either `o` (scan form) or the loop residual
// h_out = o + rho (.) h_prev with an optional bf16 copy x_next.
struct CarryOut {
    float *o;              // [B, L, H, D] or nullptr
    const void *h_prev;    // [B, L, H*D] (bf16 if h_prev_bf16, else fp32) or nullptr
    bool h_prev_bf16;
    const float *rho;      // [H*D]
    float *h_out;          // [B, L, H*D]
    bf16 *x_next;          // [B, L, H*D] or nullptr
    float *s_chunks;       // [B, H, Nc, D, D] chunk-start states, or nullptr
    const int *halted;     // [B * L]: nonzero marks a halted position (no residual update), or nullptr
};

// Adaptive halting of the loop driver: R (running halting sums) and halt
// (the loop after which a position halted, 0 while it runs) start at zero;
// after loop tau every running position adds p = sigmoid(w . h + b) (fp32) to
// R and halts (halt = tau) once R >= thr.  After loop T the outputs get the
// halting loop (T for positions that never halted) and R.
hipError_t launch_act_init(int M, float *R, int *halt, hipStream_t s);
hipError_t launch_act_halt(int M, int d, const float *h, const float *w, float b, float thr, int tau, int T, float *R,
                           int *halt, int *halt_out, float *ponder_out, hipStream_t s);
// ---- the LT2 block's token-local kernels (block.hip) ----
// out = h / sqrt(mean(h^2) + eps) * g per row of d (d a multiple of 4).
hipError_t launch_rmsnorm(bool in_f32, bool out_f32, int M, int d, const void *h, const float *g, float eps,
                          void *out, hipStream_t s);
// W13 [2F][d] from W1, W3 [d][F]: in each group of 64 packed rows, 32 columns
// of W1 then the same 32 columns of W3.
hipError_t launch_pack_w13(bool f32, int d, int F, const void *W1, const void *W3, void *W13, hipStream_t s);
hipError_t launch_bf16_to_f32(const bf16 *src, float *dst, int64_t n, hipStream_t s);
hipError_t launch_copy_f32(const float *src, float *dst, int64_t n, hipStream_t s);

// ---- token-local steps of the loop backward (loop_backward.hip) ----
// x[i] = bf16(h[i]) (round to nearest even), n elements, 16-byte aligned.
hipError_t launch_lb_round(int64_t n, const float *h, bf16 *x, hipStream_t s);
// Y <- dL/dY from the scan gradients, in place; the raw gates from Y's gate
// columns, or with zp the sums of its nzp partials; dY's padding columns zero.
hipError_t launch_lb_epilogue_grad(int M, int H, int D, float *Y, int64_t P, int64_t qkvp, float eps, float alpha_lo,
                                   const float *dq, const float *dk, const float *dv, const float *dalpha,
                                   const float *dbeta, const float *zp, int nzp, hipStream_t s);
// drho[c] = sum_r dh[r][c] hp[r][c] through lb_drho_blocks(M) x d partials.
int lb_drho_blocks(int M);
hipError_t launch_lb_drho(int M, int d, const float *dh, const void *hp, bool hp_f32, float *part, float *drho,
                          hipStream_t s);
// dWT [d][P], the sum of nparts partial arrays pstride floats apart (added in
// order), to dWq, dWk [d][H D], dWv [d][H D], dwa, dwb [d][H].
hipError_t launch_lb_unpack(int d, int H, int D, const float *dWT, int nparts, int64_t pstride, int64_t P,
                            int64_t qkvp, float *dWq, float *dWk, float *dWv, float *dwa, float *dwb, hipStream_t s);
hipError_t launch_fill_zero(float *p, int64_t n, hipStream_t s);

// ---- products and transposes of the loop backward (gemm_nt.hip) ----
// Operand modes: bf16 in memory; fp32 split into bf16 hi + lo; fp32 rounded to bf16.
// (Named enums: an enumerator of an unnamed enum inside a kernel's template
// signature is mangled differently by the host and device compilations.)
enum GemmOperand : int { OPND_BF16 = 0, OPND_F32_SPLIT = 1, OPND_F32_ROUND = 2 };
// Epilogues: C = acc; C += acc; C = acc + rho[n] D1[m][n]; C = acc + D1[m][n];
// C = acc + D1[m][n] + rho[n] D2[m][n]; C = D1[m][n] sigmoid(acc); and
// C[m][f] = silu(acc[m][64 g + r]) acc[m][64 g + 32 + r], f = 32 g + r (the
// gated FFN with W1 and W3 rows interleaved in groups of 32).
enum GemmEpilogue : int {
    EPI_STORE = 0, EPI_ACCUM = 1, EPI_RESID = 2, EPI_ADD = 3, EPI_ADD_RESID = 4, EPI_GATE = 5, EPI_SWIGLU = 6
};
// C[m][n] (op)= sum_k A[m][k] B[n][k] for m < M, n < N; A [M][lda], B [N][ldb]
// K-contiguous, K, lda, ldb multiples of 8, 16-byte aligned bases.  Pairs
// supported: (bf16, bf16), (round, bf16), (split, bf16), (split, split),
// (bf16, split).
hipError_t launch_gemm_nt(int mode_a, int mode_b, int epi, const void *A, int64_t lda, const void *B, int64_t ldb,
                          int M, int N, int K, float *C, int64_t ldc, const float *rho, const float *Dsrc,
                          int64_t ldd, hipStream_t s);
// The tiled bf16 product (gemm_tile.hip): C[m][n] = epi(sum_k A[m][k] B[n][k])
// with A2 / B2 the optional lo planes of an fp32 operand split into bf16 hi +
// lo (null when the operand is bf16).  K a multiple of 64, lda, ldb multiples
// of 8 and >= K; C fp32 or bf16 (EPI_ACCUM fp32 only).  With ksplit > 1 (store
// or accumulate only) the k-blocks of all passes are divided into ksplit
// contiguous ranges, range z's partial products going to C + z cstride.
hipError_t launch_gemm_tile(int epi, bool out_f32, const bf16 *A, const bf16 *A2, int64_t lda, const bf16 *B,
                            const bf16 *B2, int64_t ldb, int M, int N, int K, void *C, int64_t ldc, const float *rho,
                            const float *D1, int64_t ldd1, const float *D2, int64_t ldd2, hipStream_t s,
                            int ksplit = 1, int64_t cstride = 0);
// out = sum_z parts[z] (z < nparts, stride pstride) + rho[c] * add[r][c] (rho null: no term), n = rows * d.
hipError_t launch_sum_parts(int64_t rows, int d, const float *parts, int nparts, int64_t pstride, const float *rho,
                            const float *add, float *out, hipStream_t s);
// hi/lo [R][ldh] split planes of in [R][ldi] and, from the same read, the
// transposed planes hiT/loT [Cc][ldo] (rows r < Rp, zero past R).
hipError_t launch_split_both(const float *in, int64_t ldi, int R, int Cc, bf16 *hi, bf16 *lo, int64_t ldh, bf16 *hiT,
                             bf16 *loT, int64_t ldo, int Rp, hipStream_t s);
// The same product with every epilogue of launch_gemm_tile (C fp32 or bf16);
// operand pairs (split, split) and (bf16, bf16).
hipError_t launch_gemm_nt_ex(int mode_a, int mode_b, int epi, bool out_f32, const void *A, int64_t lda, const void *B,
                             int64_t ldb, int M, int N, int K, void *C, int64_t ldc, const float *rho,
                             const float *D1, int64_t ldd1, const float *D2, int64_t ldd2, hipStream_t s);
// out[c][r] = in[r][c] (r < R, c < Cc; fp32 or bf16 either side, RNE to bf16),
// and 0 for R <= r < Rp.
hipError_t launch_transpose(bool in_f32, bool out_f32, const void *in, int64_t ldi, int R, int Cc, void *out,
                            int64_t ldo, int Rp, hipStream_t s);

// The positions that ran loop tau (halt 0 or tau), in ascending order, and
// their count: the rows whose projection input changed for loop tau + 1.
hipError_t launch_act_rows(int M, const int *halt, int tau, int *rows, int *count, hipStream_t s);
// Carry: sequential over chunks per (b, h, 16-column slice of S); the chain
// updates the state, output waves of the same workgroup form
// O = diag(gamma) Q S_c + M E a chunk behind and write `out`; final state to
// s_final.
hipError_t launch_scan_carry(bool f32, int B, int L, int H, int D, const void *q, const void *k, const void *v,
                             ChunkWs ws, const float *s_init, float *s_final, CarryOut out, hipStream_t s);

// Backward of the chunkwise scan.  The forward preparation, given
// bwd_prep_out(mats, B*H*Nc, D), forms per (b, h, chunk) the matrices of
// PrepBwd in `mats` (bwd_mats_bytes for B*H*Nc chunks of width D), and
// launch_bwd_ops M^T dO = diag(beta) T^T P^T dO (fp32) from M^T and dO.  The
// reverse carry walks the chunks of
// each (b, h, 16-column slice) backwards on MFMA: dE = M^T dO + W^T dS'
// (written to dv), dS = gamma_C dS' + Q^T diag(gamma) dO - K^T diag(gamma) dE,
// with each chunk's dS' kept in ds_end [B, H, Nc, D, D] and ds_init given the
// final dS when non-null.  The chunk kernel then forms dq, dk, dalpha, dbeta
// per (b, h, chunk) from the chunk-start states s_chunks and ds_end.  fp32
// inputs need D = 64.
size_t bwd_mats_bytes(int64_t chunks, int D);
PrepBwd bwd_prep_out(float *mats, int64_t chunks, int D);
hipError_t launch_bwd_ops(int B, int L, int H, int D, const float *d_o, float *mats, hipStream_t s);
hipError_t launch_bwd_carry(bool f32, int B, int L, int H, int D, const float *d_o, const float *d_sfinal,
                            float *mats, float *dv, float *ds_end, float *ds_init, hipStream_t s);
hipError_t launch_bwd_chunk(bool f32, int B, int L, int H, int D, const void *q, const void *k, const void *v,
                            const float *alpha, const float *beta, const float *d_o, const float *dv,
                            const float *s_chunks, const float *ds_end, float *mats, float *dq, float *dk,
                            float *dalpha, float *dbeta, hipStream_t s);

// One recurrent token per sequence; states updated in place.  With
// h_out != nullptr the loop residual is applied as in CarryOut.  With part
// (bf16 only; the S channel-range partials of launch_project_decode_parts) the
// step forms its own q, k, v and gates from the partials (added in the order
// 0 .. S-1, q and k normalised with eps, q/k/v rounded to bf16) and stores
// them to q, k, v, alpha, beta instead of reading them.
hipError_t launch_decode(bool f32, int N, int H, int D, const void *q, const void *k, const void *v,
                         const float *alpha, const float *beta, float *states, float *o,
                         const void *h_prev, bool h_prev_bf16, const float *rho, float *h_out,
                         bf16 *x_next, hipStream_t s, const float *part = nullptr, int S = 0,
                         float alpha_lo = 0.f, float eps = 0.f);

}  // namespace gdn
