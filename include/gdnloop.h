/*
 * gdnloop.h -- C ABI of the looped gated-delta-rule (GDN) token mixer for
 * AMD Instinct MI355X (gfx950).
 *
 * What the library computes (LT2: Linear-Time Looped Transformers):
 *   - Section 2, "Looped Transformer (LT)" paragraph: a hidden sequence
 *     h in R^{L x d} passes T times through the same (weight-tied) block.
 *   - Section 2, "LT2" paragraph: the block's token mixer is a linear-time
 *     mixer with per-token projections q_t, k_t in R^{dk}, v_t in R^{dv} of
 *     h_t and a recurrent state S_t in R^{dk x dv}; a per-channel gate
 *     rho_tau in R^d adds the previous loop's stream back:
 *         h^(tau) = h~^(tau) + rho_tau (.) h^(tau-1).
 *   - Appendix C: the mixer is Gated DeltaNet, T = 4, use_residual = true.
 *   - Appendix B.1 and the Fig. 6 caption: one block applies a rank-1
 *     (diagonal-plus-low-rank) state update built from data-dependent gating
 *     and the delta rule.
 * The update the pages name but do not print is taken as the gated delta rule
 * (the GDN reference the pages cite), per head, token by token:
 *         S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T
 *         o_t = S_t^T q_t
 * with h~^(tau) = o (the mixer output, H*dv == d), q and k L2-normalised per
 * head, alpha = alpha_lo + (1 - alpha_lo) sigmoid(-h.wa), beta = sigmoid(h.wb)
 * and every loop scanning from S = 0 with its own state.
 *
 * Conventions for every entry point
 *   - Pointers named as device pointers are HIP device memory owned by the
 *     caller; the library never allocates, frees or synchronises device
 *     memory on the compute path.  Scratch comes from the caller's workspace
 *     (size from gdn_workspace_bytes).  Device pointers must be 16-byte
 *     aligned.
 *   - Layouts are dense row-major, last index fastest.  Head j of a width-d
 *     row owns columns [j*dv, (j+1)*dv).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued on that stream; calls return without waiting.
 *   - Arguments are validated on the host before anything is enqueued; on
 *     any error nothing is launched and no output is written.  Launch
 *     failures return GDN_ERR_HIP; device faults surface at the caller's next
 *     synchronisation.  gdn_last_error() describes the most recent failure
 *     of the calling thread.
 *   - Inputs are const and must not overlap outputs (except where a buffer
 *     is documented as in/out).  Identical calls give bitwise-identical
 *     results (no atomics in any reduction).
 */
#ifndef GDNLOOP_H
#define GDNLOOP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDN_OK = 0,
    GDN_ERR_NULL = -1,        /* a required pointer is NULL */
    GDN_ERR_SHAPE = -2,       /* a size is out of range or inconsistent */
    GDN_ERR_UNSUPPORTED = -3, /* a valid but unimplemented combination */
    GDN_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required */
    GDN_ERR_HIP = -5,         /* a HIP runtime call or launch failed */
    GDN_ERR_ALIGN = -6        /* a device pointer is not 16-byte aligned */
} gdn_status;

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

/* Problem description shared by all entry points.
 *   B      batch (sequences); for decode calls, the number of sequences
 *   L      tokens per sequence (decode calls: 1)
 *   H      heads; dk == dv in {64, 128}; d == H*dv (the mixer output is the
 *          residual stream, Section 2 "LT2" paragraph)
 *   T      loops (>= 1; the pages use 4, Appendix C)
 *   chunk  must be 64 (tokens per chunk of the chunkwise prefill)
 *   act    dtype of h0 / h_t, of the weights and of q, k, v: GDN_F32 or
 *          GDN_BF16.  alpha, beta, rho, states, o and h outputs are fp32.
 *   alpha_lo  lower bound of the decay gate, in [0, 1]; 1 makes alpha = 1 (the
 *             delta rule without decay)
 *   norm_eps  epsilon of the q/k L2 normalisation, x / sqrt(sum x^2 + eps)
 */
typedef struct {
    int32_t B, L, H, dk, dv, d, T, chunk;
    int32_t act;
    float alpha_lo;
    float norm_eps;
} gdn_desc;

/* ---- packed projection weights ---------------------------------------- */

/* Size in bytes of the packed weight buffer for `desc` (opaque layout that
 * puts each head's q|k|v columns in one contiguous tile range). */
gdn_status gdn_weights_packed_bytes(const gdn_desc *desc, size_t *bytes);

/* Packs the projection weights (LT2 Section 2 "LT2": q, k, v are projections
 * of h_t; the same weights serve every loop, Section 2 "LT" paragraph).
 *   Wq, Wk [d, H*dk], Wv [d, H*dv], wa, wb [d, H]   device, dtype desc->act
 *   Wpack  device, gdn_weights_packed_bytes bytes, written
 * q = h.Wq etc. with head j in columns [j*dk, (j+1)*dk). */
gdn_status gdn_weights_pack(const gdn_desc *desc, const void *Wq, const void *Wk,
                            const void *Wv, const void *wa, const void *wb,
                            void *Wpack, void *stream);

/* ---- workspace ---------------------------------------------------------- */

enum { GDN_OP_LOOP_PREFILL = 0, GDN_OP_LOOP_DECODE = 1, GDN_OP_SCAN_PREFILL = 2,
       GDN_OP_SCAN_DECODE = 3, GDN_OP_PROJECT = 4, GDN_OP_SCAN_BACKWARD = 5,
       GDN_OP_LOOP_PREFILL_ACT = 6, GDN_OP_LOOP_BACKWARD = 7 };

/* Device scratch bytes that operation `op` needs for `desc` (0 is valid). */
gdn_status gdn_workspace_bytes(const gdn_desc *desc, int op, size_t *bytes);

/* Regions of the looped calls' workspace that hold a loop's projections
 * (LT2 Section 2 "LT2" paragraph: q_t, k_t, v_t and the gates are per-token
 * functions of h_t):
 *   GDN_WS_Q, GDN_WS_K   [B*L, H, dk]  desc->act
 *   GDN_WS_V             [B*L, H, dv]  desc->act
 *   GDN_WS_ALPHA, GDN_WS_BETA  [B*L, H] fp32
 * After gdn_loop_prefill or gdn_loop_decode has completed on its stream, these
 * regions hold what the last loop (loop T) used: q and k after normalisation,
 * v, and the gates alpha, beta.  A caller can thus inspect the operands of any
 * loop tau by running the call with T = tau (loops 1..tau are computed
 * identically for every T).  `op` must be GDN_OP_LOOP_PREFILL or
 * GDN_OP_LOOP_DECODE; *offset is the region's byte offset from the start of
 * the workspace and *bytes its length.  Errors: GDN_ERR_UNSUPPORTED for
 * another op or an unknown region, the usual descriptor errors, GDN_ERR_NULL
 * for a NULL output pointer.  GDN_OP_LOOP_PREFILL_ACT has the same regions. */
enum { GDN_WS_Q = 0, GDN_WS_K = 1, GDN_WS_V = 2, GDN_WS_ALPHA = 3, GDN_WS_BETA = 4 };
gdn_status gdn_workspace_region(const gdn_desc *desc, int op, int region, size_t *offset,
                                size_t *bytes);

/* ---- one loop's projection (P1 + fused epilogue) ------------------------- */

/* Projects token rows x [B*L, d] (device, desc->act) with the packed weights:
 *   q, k [B*L, H, dk], v [B*L, H, dv]   device, desc->act, written
 *   alpha, beta [B*L, H]                device, fp32, written
 * q and k are L2-normalised per head; alpha = alpha_lo + (1-alpha_lo)
 * sigmoid(-x.wa); beta = sigmoid(x.wb). */
gdn_status gdn_project(const gdn_desc *desc, const void *x, const void *Wpack,
                       void *q, void *k, void *v, float *alpha, float *beta,
                       void *stream);

/* ---- single scan passes ------------------------------------------------- */

/* One chunkwise-parallel pass of the gated delta rule over given inputs
 * (q and k are used as given: no normalisation inside).
 * Passage: LT2 Section 2 "LT2" paragraph (the mixer's recurrent state S_t in
 * R^{dk x dv} updated from q_t, k_t, v_t) with the Gated DeltaNet mixer of
 * Appendix C; the update is the rank-1 data-dependent transition of Appendix
 * B.1 / Fig. 6 caption, read as the gated delta rule stated at the top of
 * this header; o_t = S_t^T q_t.  The pages cite the chunkwise (WY/UT)
 * rewrite as the fused chunkwise kernel of Section 3.2; the result equals the
 * token recurrence up to rounding.
 * Sequences of B are independent; each starts from s_init (or 0).  Errors:
 * GDN_ERR_SHAPE also for B > 65535.
 *   q, k [B, L, H, dk], v [B, L, H, dv]   device, desc->act
 *   alpha, beta [B, L, H]                 device, fp32; alpha in (0, 1]
 *   s_init [B, H, dk, dv]                 device fp32, or NULL for S_0 = 0
 *   o [B, L, H, dv]                       device fp32, written
 *   s_final [B, H, dk, dv]                device fp32 or NULL, written
 *   ws, ws_bytes                          gdn_workspace_bytes(SCAN_PREFILL)
 * desc->T is ignored.  s_final may not alias s_init. */
gdn_status gdn_scan_prefill(const gdn_desc *desc, const void *q, const void *k,
                            const void *v, const float *alpha, const float *beta,
                            const float *s_init, float *o, float *s_final,
                            void *ws, size_t ws_bytes, void *stream);

/* One recurrent step (one token per sequence) of the gated delta rule; the
 * state is read once and written once (in place).
 * Passage: the same recurrence as gdn_scan_prefill, taken one token at a time
 * (LT2 Section 3.2 measures decode throughput; the linear-time mixer decodes
 * at constant cost per token from its state, Section 2 "LT2" paragraph).
 *   desc->L must be 1; B = number of sequences
 *   q, k [B, H, dk], v [B, H, dv]   device, desc->act
 *   alpha, beta [B, H]              device fp32
 *   states [B, H, dk, dv]           device fp32, in/out
 *   o [B, H, dv]                    device fp32, written */
gdn_status gdn_scan_decode(const gdn_desc *desc, const void *q, const void *k,
                           const void *v, const float *alpha, const float *beta,
                           float *states, float *o, void *stream);

/* Gradients of one gdn_scan_prefill pass (training: LT2 Appendix C trains
 * every looped model through this mixer with bf16 mixed precision).  For a
 * loss L of the scan's outputs o and final state S_final, given
 *   d_o [B, L, H, dv]        device fp32, dL/do
 *   d_sfinal [B, H, dk, dv]  device fp32 or NULL (zero), dL/dS_final
 * and the forward inputs (q, k, v in desc->act, alpha, beta, s_init as for
 * gdn_scan_prefill), it writes
 *   dq, dk [B, L, H, dk], dv [B, L, H, dv], dalpha, dbeta [B, L, H]   device fp32
 *   ds_init [B, H, dk, dv]   device fp32 or NULL
 * The forward pass is recomputed (chunk-start states into the workspace);
 * ws is gdn_workspace_bytes(GDN_OP_SCAN_BACKWARD).  The gradients are those
 * of the token recurrence (the chunkwise form is exact up to rounding); q
 * and k are treated as given (no normalisation).  alpha must be in (0, 1]:
 * dalpha divides by alpha.  GDN_ERR_UNSUPPORTED for fp32 inputs with
 * dk = 128.  Outputs must not alias inputs. */
gdn_status gdn_scan_backward(const gdn_desc *desc, const void *q, const void *k, const void *v,
                             const float *alpha, const float *beta, const float *s_init,
                             const float *d_o, const float *d_sfinal, float *dq, float *dk,
                             float *dv, float *dalpha, float *dbeta, float *ds_init, void *ws,
                             size_t ws_bytes, void *stream);

/* ---- the looped mixer --------------------------------------------------- */

/* T weight-tied loops over a whole prompt (prefill).
 * Passage: LT2 Section 2, "Looped Transformer (LT)" paragraph (the same block
 * applied T times to the whole sequence) and "LT2" paragraph (per-loop
 * residual gate h^(tau) = h~^(tau) + rho_tau (.) h^(tau-1)); Appendix C (T = 4,
 * use_residual = true).  Each loop projects bf16(h^(tau-1)) (or h^(tau-1) for
 * fp32 workloads) with the packed weights, normalises q and k, forms the
 * gates, scans from S = 0 and applies the residual gate; h~^(tau) = o.
 *   h0 [B, L, d]                 device, desc->act (h^(0))
 *   Wpack                        from gdn_weights_pack
 *   rho [T, d]                   device fp32 (rho_1 .. rho_T)
 *   h_out [B, L, d]              device fp32, written (h^(T))
 *   states_out [T, B, H, dk, dv] device fp32 or NULL: each loop's final state
 *   h_loops [T, B, L, d]         device fp32 or NULL: h^(1) .. h^(T)
 *   ws, ws_bytes                 gdn_workspace_bytes(LOOP_PREFILL)
 * For bf16 workloads the per-loop GEMM operand is bf16(h^(tau-1)); the
 * residual stream itself stays fp32. */
gdn_status gdn_loop_prefill(const gdn_desc *desc, const void *h0, const void *Wpack,
                            const float *rho, float *h_out, float *states_out,
                            float *h_loops, void *ws, size_t ws_bytes, void *stream);

/* How gdn_loop_prefill orders its work (a process-wide setting).
 * Passage: LT2 Section 2 "LT2" paragraph: loop tau's projections of a token
 * need only h^(tau-1) of that token, and its scan state needs only the tokens
 * before it; so loop tau+1 can start on the first tokens of a prompt while
 * loop tau is still scanning later ones (a wavefront over loops and pieces).
 * With pieces, gdn_loop_prefill splits each sequence into runs of whole
 * chunks of about `tokens` tokens (a multiple of 256, at least 1024; a last
 * run shorter than 1024 joins the one before).  The projections and chunk
 * preparations of all loops run on one internal stream and each loop's
 * carries on another (three carry streams, shared round-robin beyond three
 * loops); loop tau+1's projection of piece j waits (a stream wait on an
 * event, never a spin) for loop tau's carry of piece j, so it runs on the CUs
 * that the carries leave idle.  The call still orders against `stream` as one
 * operation: its work starts after what was queued on `stream` before it,
 * and what is queued there after it waits for all of it.  Every output is
 * the same as in the loop-by-loop order up to the carry's slice width, which
 * each launch chooses by its own workgroup count (the rounding of the
 * state's sums can differ in the last bits).  Pieces apply to bf16 workloads
 * of T >= 2 whose projection forms the gate partials (2H <= 32) and whose
 * sequences give at least two pieces (L >= 2048, or B >= 2 with L >= 1024);
 * gdn_workspace_bytes(GDN_OP_LOOP_PREFILL) includes the pieces' state buffer
 * for those shapes whatever the setting.  Calls from several host threads on
 * one device take turns while they enqueue.
 *   tokens  -1: loop by loop always; 0 (the default): two pieces per
 *           sequence where L >= 16384 and the whole call's carry would fill
 *           at most half the CUs (one workgroup per sequence, head and
 *           16-column slice); > 0: pieces of that many tokens wherever they
 *           apply
 * Errors: GDN_ERR_SHAPE for tokens < -1. */
gdn_status gdn_loop_prefill_set_pieces(int tokens);

/* The piece length gdn_loop_prefill would use for `desc` under the current
 * setting (0: loop by loop).  Passage: as gdn_loop_prefill_set_pieces (LT2
 * Section 2 "LT2" paragraph).  Host only, nothing enqueued.  Errors: the
 * usual descriptor errors, GDN_ERR_NULL for a NULL `tokens`. */
gdn_status gdn_loop_prefill_pieces(const gdn_desc *desc, int *tokens);

/* T loops with per-token adaptive halting (ACT).
 * Passage: LT2 Appendix A: after loop tau a linear layer with a sigmoid gives
 * each position a halting probability p_t = sigmoid(w_halt . h_t^(tau) +
 * b_halt); the probabilities accumulate over the loops, and once the running
 * sum reaches 1 - eps (the pages use eps = 0.01) the position halts: its
 * hidden state is frozen at h_t^(tau) and takes no further update.  Reading
 * of the pages for this mixer: every position is still projected and scanned
 * in every loop (a halted position's frozen state stays context for the
 * positions after it); only the residual update is withheld.  The halting
 * decision is taken in fp32.
 *   h0, Wpack, rho               as for gdn_loop_prefill
 *   w_halt [d]                   device fp32; b_halt, eps host floats (0 <= eps < 1)
 *   h_out [B, L, d]              device fp32, written: each position's final state
 *   halt_loop [B, L]             device int32 or NULL: the loop after which the
 *                                position halted (T if it never did)
 *   ponder [B, L]                device fp32 or NULL: the running sum of p
 *   ws, ws_bytes                 gdn_workspace_bytes(GDN_OP_LOOP_PREFILL_ACT)
 * h_out may not alias h0. */
gdn_status gdn_loop_prefill_act(const gdn_desc *desc, const void *h0, const void *Wpack, const float *rho,
                                const float *w_halt, float b_halt, float eps, float *h_out,
                                int32_t *halt_loop, float *ponder, void *ws, size_t ws_bytes,
                                void *stream);

/* One generated token per sequence through the T loops (decode).
 * Passage: as gdn_loop_prefill, for one new token per sequence; each loop
 * tau continues its own state (every loop scans the sequence from S = 0 in
 * prefill, so decode keeps T states per sequence and head; the pages' looped
 * cache grows with T, Section 3.2) with loop tau's projections of the token.
 * The projection and residual are token-local, so the result equals the
 * last row of gdn_loop_prefill over the prompt plus this token.
 *   desc->L must be 1; B = number of sequences
 *   h_t [B, d]                   device, desc->act
 *   rho [T, d]                   device fp32
 *   states [T, B, H, dk, dv]     device fp32, in/out (loop tau advances its own)
 *   h_out [B, d]                 device fp32, written (h^(T) of the token)
 *   ws, ws_bytes                 gdn_workspace_bytes(LOOP_DECODE); for at most 64
 *                                bf16 sequences its last region holds the
 *                                projection's partial products (the projection
 *                                split over the channels), and a workspace of
 *                                the size without that region runs the
 *                                projection unsplit */
gdn_status gdn_loop_decode(const gdn_desc *desc, const void *h_t, const void *Wpack,
                           const float *rho, float *states, float *h_out,
                           void *ws, size_t ws_bytes, void *stream);

/* The same decode step without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Arguments and results are those of
 * gdn_loop_decode; the scratch is a library-held device array of
 * GDN_NOALLOC_SCRATCH_BYTES per GPU, kept until the process ends, so the
 * call allocates and frees nothing.  A step whose workspace
 * (gdn_workspace_bytes with GDN_OP_LOOP_DECODE) exceeds that size returns
 * GDN_ERR_WORKSPACE before anything is enqueued (bf16 at d = 2048: up to 508
 * sequences).  Every call on one GPU uses the same array: calls that overlap
 * on one GPU (other streams, other threads) race and must be serialised by
 * the caller; calls on the same stream are ordered and safe. */
#define GDN_NOALLOC_SCRATCH_BYTES (8u << 20)
gdn_status gdn_loop_decode_noalloc(const gdn_desc *desc, const void *h_t, const void *Wpack,
                                   const float *rho, float *states, float *h_out, void *stream);

/* Gradients of gdn_loop_prefill through its T loops.
 * Passage: LT2: Linear-Time Looped Transformers, Appendix C (every looped
 * model is trained through this path with bf16 mixed precision); the
 * forward is that of gdn_loop_prefill (Section 2, "Looped Transformer (LT)"
 * and "LT2" paragraphs: weight tying and the per-loop residual gate).  For a
 * loss L of h^(T), given dh = dL/dh^(T), each loop tau = T..1 is recomputed
 * from its input h^(tau-1) (raw projections, L2 norm, gates; then the scan's
 * chunk matrices and states) and taken in reverse: the scan backward with
 * dO = dL/dh^(tau), the gradient through the normalisation and the gates,
 *     dW += x^T dY,   drho_tau = sum over positions of dL/dh^(tau) (.) h^(tau-1),
 *     dL/dh^(tau-1) = rho_tau (.) dL/dh^(tau) + dY W.
 * The forward's bf16 roundings (the loop operand x = bf16(h), q/k/v) pass
 * the gradient through unchanged.  Every loop's scan starts from S = 0 and
 * its final state is not an input of L.
 *   h0 [B, L, d]                 device, desc->act (as given to gdn_loop_prefill)
 *   Wpack, rho [T, d]            as for gdn_loop_prefill
 *   h_loops [T, B, L, d]         device fp32: h^(1..T) as gdn_loop_prefill's h_loops
 *                                wrote them (slices 0..T-2 are read; NULL allowed when T == 1)
 *   dh [B, L, d]                 device fp32, dL/dh^(T) (read only)
 *   dh0 [B, L, d]                device fp32, written: dL/dh0
 *   dWq, dWk [d, H*dk], dWv [d, H*dv], dwa, dwb [d, H]   device fp32, written: the
 *                                gradients of the unpacked weights (gdn_weights_pack's inputs)
 *   drho [T, d]                  device fp32, written
 *   ws, ws_bytes                 gdn_workspace_bytes(GDN_OP_LOOP_BACKWARD)
 * Products run on bf16 MFMA with fp32 operands split into two bf16 parts.
 * alpha must stay above 0 (dalpha divides by it).  GDN_ERR_UNSUPPORTED for
 * fp32 inputs with dk = 128; GDN_ERR_SHAPE beyond 65535 * 64 tokens or when dh0
 * aliases dh. */
gdn_status gdn_loop_backward(const gdn_desc *desc, const void *h0, const void *Wpack, const float *rho,
                             const float *h_loops, const float *dh, float *dh0, float *dWq, float *dWk,
                             float *dWv, float *dwa, float *dwb, float *drho, void *ws, size_t ws_bytes,
                             void *stream);

/* ---- the LT2 block around the mixer ------------------------------------- */

/* Passage: LT2: Linear-Time Looped Transformers, Section 2 ("Looped
 * Transformer (LT)": a block is a token mixer and a position-wise FFN, each
 * with an identity residual, pre-norm omitted from Eq. (1) for brevity, and
 * the N blocks are reused for T iterations; "LT2": the mixer is the linear
 * one and h^(tau) = (F_N o ... o F_1)(h^(tau-1)) + rho_tau (.) h^(tau-1)), and
 * Section 3's attention-sink paragraph (the head-specific sigmoid output gate
 * of Gated Attention, applied inside the looped block).  One block:
 *     x1 = RMSNorm(h; g1)            [x / sqrt(mean(x^2) + norm_eps) * g]
 *     o  = the gated-delta-rule mixer of x1 (projections, L2 norm, gates and
 *          the scan from S = 0, exactly as one loop of gdn_loop_prefill)
 *     z  = o (.) sigmoid(x1 Wg)       Wg [d, H*dv]: one gate per head channel
 *     h1 = h + z Wo                   Wo [H*dv, d]
 *     x2 = RMSNorm(h1; g2)
 *     F(h) = h1 + (silu(x2 W1) (.) (x2 W3)) W2     W1, W3 [d, ffn], W2 [ffn, d]
 * For bf16 workloads x1, q/k/v, z, x2 and silu(.)(.) are rounded to bf16 (the
 * products' operands); h, h1, o, the norms' statistics and the gates stay
 * fp32.  ffn must be a positive multiple of 64. */

/* Bytes of one packed block (desc->act weights plus the fp32 norm weights). */
gdn_status gdn_block_packed_bytes(const gdn_desc *desc, int ffn, size_t *bytes);
/* Pack one block's weights (device pointers): g1, g2 [d] fp32; Wq, Wk [d, H*dk],
 * Wv [d, H*dv], wa, wb [d, H] (as gdn_weights_pack), Wg [d, H*dv], Wo [H*dv, d],
 * W1, W3 [d, ffn], W2 [ffn, d] in desc->act.  Wblock: gdn_block_packed_bytes,
 * opaque, 256-byte aligned. */
gdn_status gdn_block_pack(const gdn_desc *desc, int ffn, const float *g1, const void *Wq, const void *Wk,
                          const void *Wv, const void *wa, const void *wb, const void *Wg, const void *Wo,
                          const float *g2, const void *W1, const void *W3, const void *W2, void *Wblock,
                          void *stream);
/* Workspace of gdn_block_forward and gdn_block_loop_prefill. */
gdn_status gdn_block_workspace_bytes(const gdn_desc *desc, int ffn, size_t *bytes);
/* Regions of that workspace that hold, after gdn_block_forward (or after the
 * last block of gdn_block_loop_prefill), that block's intermediates:
 *   GDN_BWS_X1, GDN_BWS_X2 [B*L, d] desc->act; GDN_BWS_O [B*L, H*dv] fp32;
 *   GDN_BWS_Z [B*L, H*dv] desc->act; GDN_BWS_H1 [B*L, d] fp32;
 *   GDN_BWS_U [B*L, ffn] desc->act; GDN_WS_Q .. GDN_WS_BETA as for the loop. */
enum { GDN_BWS_X1 = 16, GDN_BWS_O = 17, GDN_BWS_Z = 18, GDN_BWS_H1 = 19, GDN_BWS_X2 = 20, GDN_BWS_U = 21 };
gdn_status gdn_block_workspace_region(const gdn_desc *desc, int ffn, int region, size_t *offset, size_t *bytes);
/* One block on h [B, L, d] device fp32: out = F(h) [B, L, d] device fp32
 * (desc->T is ignored).  out may not alias h. */
gdn_status gdn_block_forward(const gdn_desc *desc, int ffn, const float *h, const void *Wblock, float *out,
                             void *ws, size_t ws_bytes, void *stream);
/* T loops of a stack of `layers` blocks (Wblocks: that many packed blocks
 * back to back, each gdn_block_packed_bytes): h^(tau) = F_N(...F_1(h^(tau-1)))
 * + rho_tau (.) h^(tau-1).  h0 [B, L, d] desc->act, rho [T, d] fp32, h_out
 * [B, L, d] fp32 (may not alias h0). */
gdn_status gdn_block_loop_prefill(const gdn_desc *desc, int ffn, int layers, const void *h0, const void *Wblocks,
                                  const float *rho, float *h_out, void *ws, size_t ws_bytes, void *stream);

/* ---- diagnostics -------------------------------------------------------- */

const char *gdn_status_string(gdn_status s);
/* Human-readable description of the calling thread's most recent error. */
const char *gdn_last_error(void);
/* Library version string. */
const char *gdn_version(void);

/* ---- optional device timing of one stage -------------------------------- */

/* Stages that a timer can bracket.  4 and 8 are not stages, and
 * gdn_timer_create rejects them: 4 named a separate output pass that the carry
 * now performs, 8 a backward preparation whose matrices the forward's chunk
 * preparation now writes. */
enum { GDN_STAGE_PROJECT = 0, GDN_STAGE_SCAN_PREP = 1, GDN_STAGE_SCAN_CARRY = 2,
       GDN_STAGE_DECODE = 3, GDN_STAGE_GATES = 5, GDN_STAGE_BWD_CARRY = 6, GDN_STAGE_BWD_CHUNK = 7,
       GDN_STAGE_BWD_GEMM = 9, GDN_STAGE_BWD_OPS = 10, GDN_STAGE_BLOCK_GEMM = 11 };
/* GDN_STAGE_BLOCK_GEMM times the four products of an LT2 block around its
 * mixer (the gate with o, the output projection, the FFN's up and down
 * projections); the mixer's own launches keep their stages. */
/* GDN_STAGE_BWD_GEMM times the three products of each loop of
 * gdn_loop_backward (the projections recomputed, the input gradient and the
 * weight gradient). */
/* GDN_STAGE_BWD_OPS, GDN_STAGE_BWD_CARRY and GDN_STAGE_BWD_CHUNK time the
 * three kernels of the scan backward (in gdn_scan_backward and in each loop
 * of gdn_loop_backward) that follow its forward recomputation, whose prep
 * (which also forms the backward's chunk matrices) and carry are timed as
 * GDN_STAGE_SCAN_PREP and GDN_STAGE_SCAN_CARRY. */
/* GDN_STAGE_SCAN_CARRY times the carry kernel, which computes the chunk outputs
 * (and the loop residual) as well.  GDN_STAGE_PROJECT times the projection GEMM.  For bf16 inputs of 1024 or
 * more tokens the gates alpha/beta leave the GEMM's epilogue: gdn_project and
 * gdn_loop_decode compute them in a launch of their own, timed as
 * GDN_STAGE_GATES; gdn_loop_prefill with H <= 16 has the GEMM write partial
 * gate pre-activations (in its workspace) that the chunk preparation sums,
 * so no gate launch occurs.  Shorter inputs compute the gates inside the GEMM. */

/* While a timer is attached, every launch of its stage carries a pair of HIP
 * events on its dispatch (hipExtLaunchKernel start/stop events), so each pair
 * spans that kernel's execution on its stream and nothing else (at most
 * `capacity` launches are recorded).  One timer per stage can be attached at
 * a time (attaching replaces that stage's timer; detach removes all).
 * Attaching is process-wide and meant for profiling runs; it is not
 * thread-safe.  gdn_timer_read waits for the recorded events and returns the
 * number of bracketed launches and their summed duration in milliseconds.
 * Each armed dispatch costs the GPU a few microseconds; gdn_timer_set_stride
 * (stride >= 1, default 1) arms only every stride-th launch of the stage made
 * while the timer is attached, counted from the call (and from each reset),
 * so that a long run can be sampled at a small cost.  gdn_timer_reset
 * forgets the recorded launches. */
typedef struct gdn_timer gdn_timer;
gdn_status gdn_timer_create(int stage, int capacity, gdn_timer **out);
gdn_status gdn_timer_set_stride(gdn_timer *t, int stride);
gdn_status gdn_timer_attach(gdn_timer *t);
gdn_status gdn_timer_detach(void);
gdn_status gdn_timer_reset(gdn_timer *t);
gdn_status gdn_timer_read(gdn_timer *t, int *launches, double *total_ms);
gdn_status gdn_timer_destroy(gdn_timer *t);

#ifdef __cplusplus
}
#endif
#endif /* GDNLOOP_H */
