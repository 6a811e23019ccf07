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
       GDN_OP_SCAN_DECODE = 3, GDN_OP_PROJECT = 4 };

/* Device scratch bytes that operation `op` needs for `desc` (0 is valid). */
gdn_status gdn_workspace_bytes(const gdn_desc *desc, int op, size_t *bytes);

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
 *   desc->L must be 1; B = number of sequences
 *   q, k [B, H, dk], v [B, H, dv]   device, desc->act
 *   alpha, beta [B, H]              device fp32
 *   states [B, H, dk, dv]           device fp32, in/out
 *   o [B, H, dv]                    device fp32, written */
gdn_status gdn_scan_decode(const gdn_desc *desc, const void *q, const void *k,
                           const void *v, const float *alpha, const float *beta,
                           float *states, float *o, void *stream);

/* ---- the looped mixer --------------------------------------------------- */

/* T weight-tied loops over a whole prompt (prefill):
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

/* One generated token per sequence through the T loops (decode):
 *   desc->L must be 1; B = number of sequences
 *   h_t [B, d]                   device, desc->act
 *   rho [T, d]                   device fp32
 *   states [T, B, H, dk, dv]     device fp32, in/out (loop tau advances its own)
 *   h_out [B, d]                 device fp32, written (h^(T) of the token)
 *   ws, ws_bytes                 gdn_workspace_bytes(LOOP_DECODE) */
gdn_status gdn_loop_decode(const gdn_desc *desc, const void *h_t, const void *Wpack,
                           const float *rho, float *states, float *h_out,
                           void *ws, size_t ws_bytes, void *stream);

/* ---- diagnostics -------------------------------------------------------- */

const char *gdn_status_string(gdn_status s);
/* Human-readable description of the calling thread's most recent error. */
const char *gdn_last_error(void);
/* Library version string. */
const char *gdn_version(void);

/* ---- optional device timing of one stage -------------------------------- */

/* Stages that a timer can bracket. */
enum { GDN_STAGE_PROJECT = 0, GDN_STAGE_SCAN_PREP = 1, GDN_STAGE_SCAN_CARRY = 2,
       GDN_STAGE_DECODE = 3, GDN_STAGE_SCAN_OUT = 4, GDN_STAGE_GATES = 5 };
/* GDN_STAGE_SCAN_CARRY times the carry kernel, which computes the chunk outputs
 * (and the loop residual) as well; GDN_STAGE_SCAN_OUT names no launch any more
 * and is kept so that stage numbers stay stable (a timer on it records none).
 * GDN_STAGE_PROJECT times the projection GEMM.  For bf16 inputs of 1024 or
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
