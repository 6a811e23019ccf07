// gdnloop_api.cpp -- C ABI of the looped gated-delta-rule mixer: host-side
// validation, workspace carving, launch sequencing and the T-loop driver.
//
// LT2: Linear-Time Looped Transformers, Section 2 ("Looped Transformer (LT)"
// and "LT2" paragraphs): the same block runs T times; loop tau maps h^(tau-1)
// to h~^(tau) and the per-channel gate adds h^(tau) = h~^(tau) + rho_tau (.) h^(tau-1).
// Appendix C: T = 4 with use_residual = true.  Each loop runs
//   project (q, k, v, alpha, beta from h^(tau-1), same weights every loop)
//   -> chunk prep -> state carry with the residual fused into its output.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/gdnloop.h"
#include "gdn_kernels.h"

using namespace gdn;

namespace {

thread_local std::string g_last_error = "no error";

gdn_status fail(gdn_status s, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

gdn_status hip_fail(hipError_t e, const char *what) {
    return fail(GDN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int CHUNK = 64;
constexpr size_t ALIGN = 256;

size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t act_bytes(const gdn_desc *d) { return d->act == GDN_F32 ? 4 : 2; }

// Shape checks common to every entry point.  `decode`: L must be 1.
gdn_status check_desc(const gdn_desc *d, bool decode) {
    if (!d) return fail(GDN_ERR_NULL, "desc is NULL");
    if (d->act != GDN_F32 && d->act != GDN_BF16)
        return fail(GDN_ERR_UNSUPPORTED, "act must be GDN_F32 or GDN_BF16 (got %d)", d->act);
    if (d->B < 1 || d->L < 1 || d->H < 1 || d->T < 1)
        return fail(GDN_ERR_SHAPE, "B, L, H, T must be >= 1 (B=%d L=%d H=%d T=%d)", d->B, d->L,
                    d->H, d->T);
    if (d->chunk != CHUNK) return fail(GDN_ERR_UNSUPPORTED, "chunk must be 64 (got %d)", d->chunk);
    if (d->dk != d->dv || (d->dk != 64 && d->dk != 128))
        return fail(GDN_ERR_UNSUPPORTED, "dk == dv in {64, 128} required (dk=%d dv=%d)", d->dk, d->dv);
    if (d->H > 64) return fail(GDN_ERR_UNSUPPORTED, "at most 64 heads (got %d)", d->H);
    if ((int64_t)d->H * d->dv != d->d)
        return fail(GDN_ERR_SHAPE, "d must equal H*dv (d=%d H=%d dv=%d)", d->d, d->H, d->dv);
    if (decode && d->L != 1) return fail(GDN_ERR_SHAPE, "decode calls need L == 1 (got %d)", d->L);
    if (!(d->alpha_lo >= 0.f && d->alpha_lo <= 1.f))
        return fail(GDN_ERR_SHAPE, "alpha_lo must be in [0, 1] (got %g)", (double)d->alpha_lo);
    if (!(d->norm_eps > 0.f) || !std::isfinite(d->norm_eps))
        return fail(GDN_ERR_SHAPE, "norm_eps must be positive and finite");
    // every tensor must be addressable with 64-bit offsets; keep element counts sane
    const int64_t tokens = (int64_t)d->B * d->L;
    if (tokens * d->d > (int64_t)1 << 40) return fail(GDN_ERR_SHAPE, "problem too large");
    // token counts are 32-bit inside the kernels
    if (tokens > INT32_MAX) return fail(GDN_ERR_SHAPE, "B*L must be below 2^31 (got %lld)", (long long)tokens);
    return GDN_OK;
}

// Launch-grid limits of the chunkwise prefill (checked before anything is
// enqueued, so that no launch of a multi-kernel call can fail on its shape):
// the chunk prep runs (chunk, head) pairs along x and sequences along y, the
// carry sequences along z; both y and z hold at most 65535.
gdn_status check_prefill_grid(const gdn_desc *d) {
    if (d->B > 65535) return fail(GDN_ERR_SHAPE, "prefill calls take at most 65535 sequences (got %d)", d->B);
    const int64_t nc = (d->L + 63) / 64;
    if (nc * d->H > INT32_MAX) return fail(GDN_ERR_SHAPE, "too many (chunk, head) pairs per sequence");
    // the fp32 projection runs 64-token row tiles along y
    if (d->act == GDN_F32 && ((int64_t)d->B * d->L + 63) / 64 > 65535)
        return fail(GDN_ERR_SHAPE, "fp32 projections take at most 65535 * 64 tokens");
    return GDN_OK;
}

// Sizes the loop backward's products and row-block reductions can take.
gdn_status check_loop_backward(const gdn_desc *d) {
    const int64_t M = (int64_t)d->B * d->L, Mp = (M + 63) / 64 * 64;
    if ((M + 127) / 128 > 65535 || Mp / 64 > 65535 || (packed_rows(d->H, d->dk) + 127) / 128 > 65535)
        return fail(GDN_ERR_SHAPE, "the loop backward takes at most 65535 * 64 tokens");
    return GDN_OK;
}

#define REQUIRE_PTR(p)                                                                             \
    do {                                                                                           \
        if (!(p)) return fail(GDN_ERR_NULL, "%s is NULL", #p);                                     \
        if (!aligned16(p)) return fail(GDN_ERR_ALIGN, "%s is not 16-byte aligned", #p);            \
    } while (0)
#define OPTIONAL_PTR(p)                                                                            \
    do {                                                                                           \
        if ((p) && !aligned16(p)) return fail(GDN_ERR_ALIGN, "%s is not 16-byte aligned", #p);     \
    } while (0)

// The loop backward's products split their k range into partial sums when
// their tiles alone would leave CUs idle (one 384 x 256 tile per CU at a time):
// dY W into at most LB_DX_SPLIT (summed with the residual), x^T dY into at
// most LB_DW_SPLIT accumulators (summed when unpacked).  The count minimises
// the rounds of tiles per unit of work plus `cost` per extra partial sum (its
// traffic, in rounds).  Sized for 256 CUs, so that workspace sizes do not
// depend on the device.
constexpr int LB_DX_SPLIT = 4, LB_DW_SPLIT = 3;
static int lb_split(int64_t tiles, int max_split, double cost) {
    int best = 1;
    double best_c = 1e30;
    for (int sp = 1; sp <= max_split; ++sp) {
        const double c = (double)((tiles * sp + 255) / 256) / sp + cost * (sp - 1);
        if (c < best_c - 1e-9) {
            best_c = c;
            best = sp;
        }
    }
    return best;
}
static int lb_dx_split(int64_t tokens, int d) {
    return lb_split(((tokens + 383) / 384) * ((d + 255) / 256), LB_DX_SPLIT, 0.025);
}
static int lb_dw_split(int d, int64_t P, bool f32) {
    return f32 ? 1 : lb_split(((int64_t)(d + 383) / 384) * ((P + 255) / 256), LB_DW_SPLIT, 0.05);
}

// ---- the loop prefill as a pipeline over pieces ------------------------------
// A piece is one sequence's run of whole chunks (at least PIPE_MIN_PIECE
// tokens, so that its projection takes the same wide GEMM as the whole call).
// Every step of a loop is local to its piece except the state, which crosses
// from piece to piece of a sequence; so loop tau+1 can project and scan piece
// j as soon as loop tau has finished piece j, while loop tau goes on with
// piece j+1.  The projections and chunk preps of all loops run on one stream,
// each loop's carries on a stream of their own, so that the projection of the
// next piece runs on the CUs that a carry leaves idle; the only waits are
// stream waits on events, so no kernel ever spins on another.
constexpr int PIPE_MIN_PIECE = 1024;
constexpr int PIPE_AUTO_MIN_L = 16384;   // shortest sequence the automatic setting splits
constexpr int PIPE_STREAMS = 4;
std::atomic<int> g_pipe_piece{0};   // gdn_loop_prefill_set_pieces: 0 automatic, -1 off, > 0 tokens per piece

// bf16 workloads of at least two loops whose projection forms the gate
// partials (P > 0), with pieces to form: more than one sequence, or one
// sequence of at least two pieces.
bool pipeline_capable(const gdn_desc *d, int P) {
    return d->act == GDN_BF16 && d->T >= 2 && P > 0 && d->L >= PIPE_MIN_PIECE &&
           (d->B >= 2 || d->L >= 2 * PIPE_MIN_PIECE);
}

// ---- workspace layout ------------------------------------------------------
struct Layout {
    size_t q = 0, k = 0, v = 0, alpha = 0, beta = 0, zp = 0, W = 0, M = 0, g = 0, x = 0, sc = 0, dse = 0, bm = 0;
    size_t R = 0, halt = 0, rows = 0, rows_count = 0;
    // the loop backward: raw projections (then their gradient) [M][P] and its
    // transpose [P][Mp], the loop input and the weights transposed, the scan
    // gradients, two dh buffers, the weight-gradient accumulator [d][P], rho partials
    size_t Y = 0, YT = 0, XT = 0, WT = 0, gq = 0, gk = 0, gv = 0, gal = 0, gbe = 0, dhA = 0, dhB = 0, dW = 0, part = 0;
    size_t Yhl = 0;   // bf16 workloads: dY as bf16 hi and lo planes (the transpose's planes reuse YT)
    size_t Gp = 0;    // bf16 workloads: the split-k partial sums of dY W
    size_t st = 0;    // the pipelined loop prefill: each (loop, sequence)'s state between pieces [T][B][H][D][D]
    size_t dpart = 0; // the loop decode: partial products of the channel-split projection (0: not split)
    size_t total = 0;
    int P = 0;   // gate partials of the projection (0: alpha and beta directly)
};

Layout layout(const gdn_desc *d, int op) {
    Layout lo;
    const int64_t tokens = (int64_t)d->B * d->L;
    const int64_t D = d->dk;
    const int64_t Nc = (d->L + CHUNK - 1) / CHUNK;
    const int64_t bh = (int64_t)d->B * d->H;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += align_up(bytes);
        return at;
    };
    const bool act = op == GDN_OP_LOOP_PREFILL_ACT;
    if (act) op = GDN_OP_LOOP_PREFILL;   // the loop prefill's regions, then the halting state
    const bool lbwd = op == GDN_OP_LOOP_BACKWARD;
    const bool proj = op == GDN_OP_LOOP_PREFILL || op == GDN_OP_LOOP_DECODE || lbwd;
    const bool chunks = op == GDN_OP_LOOP_PREFILL || op == GDN_OP_SCAN_PREFILL || op == GDN_OP_SCAN_BACKWARD || lbwd;
    if (proj) {
        lo.q = take(tokens * d->H * D * act_bytes(d));
        lo.k = take(tokens * d->H * D * act_bytes(d));
        lo.v = take(tokens * d->H * D * act_bytes(d));
        lo.alpha = take(tokens * d->H * 4);
        lo.beta = take(tokens * d->H * 4);
        if (d->act == GDN_BF16 && d->T > 1) lo.x = take(tokens * d->d * 2);
        if (op == GDN_OP_LOOP_PREFILL || lbwd) {
            lo.P = gate_partials(d->act == GDN_F32, (int)tokens, d->d, d->H);
            if (lo.P) lo.zp = take((size_t)lo.P * 2 * d->H * tokens * 4);
        }
    }
    if (chunks) {
        lo.W = take(bh * Nc * D * CHUNK * 4);
        lo.M = take(bh * Nc * CHUNK * CHUNK * 4);
        lo.g = take(bh * Nc * CHUNK * 4);
    }
    if (op == GDN_OP_SCAN_BACKWARD || lbwd) {   // chunk-start states and the gradient at each chunk's end
        lo.sc = take(bh * Nc * D * D * 4);
        lo.dse = take(bh * Nc * D * D * 4);
        lo.bm = take(bwd_mats_bytes(bh * Nc, (int)D));
    }
    if (lbwd) {
        const int64_t P = packed_rows(d->H, d->dk), Mp = (tokens + 63) / 64 * 64, ab = act_bytes(d);
        lo.Y = take(tokens * P * 4);
        if (d->act == GDN_BF16) lo.Yhl = take(tokens * P * 4);
        lo.YT = take(P * Mp * 4);
        lo.XT = take(d->d * Mp * ab);
        lo.WT = take(d->d * P * ab);
        lo.gq = take(tokens * d->H * D * 4);
        lo.gk = take(tokens * d->H * D * 4);
        lo.gv = take(tokens * d->H * D * 4);
        lo.gal = take(tokens * d->H * 4);
        lo.gbe = take(tokens * d->H * 4);
        lo.dhA = take(tokens * d->d * 4);
        lo.dhB = take(tokens * d->d * 4);
        lo.dW = take(d->d * P * 4 * lb_dw_split(d->d, P, d->act == GDN_F32));
        const int dxs = lb_dx_split(tokens, d->d);
        if (d->act == GDN_BF16 && dxs > 1) lo.Gp = take((size_t)dxs * tokens * d->d * 4);
        lo.part = take((size_t)lb_drho_blocks((int)tokens) * d->d * 4);
    }
    if (act) {
        lo.R = take(tokens * 4);
        lo.halt = take(tokens * 4);
        lo.rows = take(tokens * 4);   // positions re-projected in the next loop, and their count
        lo.rows_count = take(4);
    }
    // shapes the loop prefill can run as a pipeline of pieces (below) carry
    // each (loop, sequence)'s state from one piece to the next through here
    if (op == GDN_OP_LOOP_PREFILL && !act && pipeline_capable(d, lo.P)) lo.st = take((size_t)d->T * bh * D * D * 4);
    if (op == GDN_OP_LOOP_DECODE) {
        const size_t pb = decode_part_bytes(d->act == GDN_F32, (int)tokens, d->d, d->H, (int)D);
        if (pb) lo.dpart = take(pb);
    }
    lo.total = off;
    return lo;
}

char *at(void *ws, size_t off) { return static_cast<char *>(ws) + off; }

// ---- optional stage timing ---------------------------------------------------
}  // namespace

struct gdn_timer {
    int stage = 0;
    int capacity = 0;
    int used = 0;
    int stride = 1;   // record launches stride-1, 2 stride-1, ... of the stage
    int seen = 0;     // launches of the stage while attached
    std::vector<hipEvent_t> start, stop;
};

namespace {

constexpr int N_STAGES = GDN_STAGE_BLOCK_GEMM + 1;
thread_local LaunchEvents t_launch_events{nullptr, nullptr};
gdn_timer *g_timers[N_STAGES] = {};

// Runs `launch` (exactly one kernel launch) with the stage timer's next event
// pair armed, when a timer for `stage` is attached.
template <typename F>
hipError_t timed(int stage, hipStream_t s, F &&launch) {
    gdn_timer *tm = g_timers[stage];
    if (!tm || tm->stage != stage || tm->used >= tm->capacity) return launch();
    if (++tm->seen % tm->stride != 0) return launch();
    (void)s;
    launch_events() = LaunchEvents{tm->start[tm->used], tm->stop[tm->used]};
    hipError_t e = launch();
    launch_events() = LaunchEvents{nullptr, nullptr};
    if (e == hipSuccess) tm->used++;
    return e;
}

// The projection of M tokens: the GEMM launch, plus the gate launch when the
// GEMM leaves the gates to it and does not write gate partials (zp).
hipError_t project(bool f32, int M, int d, int H, int D, const void *x, const void *Wpack, void *q, void *k,
                   void *v, float *al, float *be, float alpha_lo, float eps, float *zp, hipStream_t s,
                   const int *rows = nullptr, const int *rows_count = nullptr, float *yraw = nullptr,
                   int64_t ldy = 0) {
    hipError_t e = timed(GDN_STAGE_PROJECT, s, [&] {
        return launch_project(f32, M, d, H, D, x, Wpack, q, k, v, al, be, alpha_lo, eps, zp, s, rows, rows_count,
                              yraw, ldy);
    });
    if (e == hipSuccess && !zp && project_separate_gates(f32, M))
        e = timed(GDN_STAGE_GATES, s, [&] { return launch_gates(M, d, H, D, x, Wpack, al, be, alpha_lo, s); });
    return e;
}

}  // namespace

LaunchEvents &gdn::launch_events() { return t_launch_events; }

int gdn::set_last_error(int status, const char *msg) { return fail((gdn_status)status, "%s", msg); }

extern "C" {

const char *gdn_status_string(gdn_status s) {
    switch (s) {
        case GDN_OK: return "GDN_OK";
        case GDN_ERR_NULL: return "GDN_ERR_NULL: a required pointer is NULL";
        case GDN_ERR_SHAPE: return "GDN_ERR_SHAPE: size out of range or inconsistent";
        case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED: combination not implemented";
        case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE: workspace missing or too small";
        case GDN_ERR_HIP: return "GDN_ERR_HIP: HIP runtime call or launch failed";
        case GDN_ERR_ALIGN: return "GDN_ERR_ALIGN: device pointer not 16-byte aligned";
    }
    return "unknown gdn_status";
}

const char *gdn_last_error(void) { return g_last_error.c_str(); }

const char *gdn_version(void) { return "gdnloop 0.1 (gfx950)"; }

gdn_status gdn_weights_packed_bytes(const gdn_desc *desc, size_t *bytes) {
    gdn_status st = check_desc(desc, false);
    if (st != GDN_OK) return st;
    if (!bytes) return fail(GDN_ERR_NULL, "bytes is NULL");
    *bytes = (size_t)packed_rows(desc->H, desc->dk) * desc->d * act_bytes(desc);
    return GDN_OK;
}

gdn_status gdn_weights_pack(const gdn_desc *desc, const void *Wq, const void *Wk, const void *Wv,
                            const void *wa, const void *wb, void *Wpack, void *stream) {
    gdn_status st = check_desc(desc, false);
    if (st != GDN_OK) return st;
    REQUIRE_PTR(Wq); REQUIRE_PTR(Wk); REQUIRE_PTR(Wv); REQUIRE_PTR(wa); REQUIRE_PTR(wb);
    REQUIRE_PTR(Wpack);
    hipError_t e = launch_pack_weights(desc->act == GDN_F32, desc->d, desc->H, desc->dk, Wq, Wk, Wv,
                                       wa, wb, Wpack, (hipStream_t)stream);
    return e == hipSuccess ? GDN_OK : hip_fail(e, "weight pack launch");
}

gdn_status gdn_workspace_bytes(const gdn_desc *desc, int op, size_t *bytes) {
    if (op < GDN_OP_LOOP_PREFILL || op > GDN_OP_LOOP_BACKWARD)
        return fail(GDN_ERR_UNSUPPORTED, "unknown op %d", op);
    gdn_status st = check_desc(desc, op == GDN_OP_LOOP_DECODE || op == GDN_OP_SCAN_DECODE);
    if (st != GDN_OK) return st;
    if ((op == GDN_OP_LOOP_PREFILL || op == GDN_OP_SCAN_PREFILL || op == GDN_OP_SCAN_BACKWARD ||
         op == GDN_OP_LOOP_PREFILL_ACT || op == GDN_OP_LOOP_BACKWARD) &&
        (st = check_prefill_grid(desc)) != GDN_OK)
        return st;
    if ((op == GDN_OP_SCAN_BACKWARD || op == GDN_OP_LOOP_BACKWARD) && desc->act == GDN_F32 && desc->dk == 128)
        return fail(GDN_ERR_UNSUPPORTED, "the backward pass takes fp32 inputs with dk = 64 only");
    if (op == GDN_OP_LOOP_BACKWARD && (st = check_loop_backward(desc)) != GDN_OK) return st;
    if (!bytes) return fail(GDN_ERR_NULL, "bytes is NULL");
    *bytes = layout(desc, op).total;
    return GDN_OK;
}

gdn_status gdn_workspace_region(const gdn_desc *desc, int op, int region, size_t *offset, size_t *bytes) {
    if (op != GDN_OP_LOOP_PREFILL && op != GDN_OP_LOOP_DECODE && op != GDN_OP_LOOP_PREFILL_ACT)
        return fail(GDN_ERR_UNSUPPORTED, "only the looped calls expose workspace regions (op %d)", op);
    gdn_status st = check_desc(desc, op == GDN_OP_LOOP_DECODE);
    if (st != GDN_OK) return st;
    if (!offset || !bytes) return fail(GDN_ERR_NULL, "offset or bytes is NULL");
    const Layout lo = layout(desc, op);
    const size_t tokens = (size_t)desc->B * desc->L, H = desc->H;
    const size_t qkv = tokens * H * desc->dk * act_bytes(desc), gate = tokens * H * 4;
    switch (region) {
        case GDN_WS_Q: *offset = lo.q; *bytes = qkv; break;
        case GDN_WS_K: *offset = lo.k; *bytes = qkv; break;
        case GDN_WS_V: *offset = lo.v; *bytes = qkv; break;
        case GDN_WS_ALPHA: *offset = lo.alpha; *bytes = gate; break;
        case GDN_WS_BETA: *offset = lo.beta; *bytes = gate; break;
        default: return fail(GDN_ERR_UNSUPPORTED, "unknown workspace region %d", region);
    }
    return GDN_OK;
}

gdn_status gdn_project(const gdn_desc *desc, const void *x, const void *Wpack, void *q, void *k,
                       void *v, float *alpha, float *beta, void *stream) {
    gdn_status st = check_desc(desc, false);
    if (st != GDN_OK) return st;
    REQUIRE_PTR(x); REQUIRE_PTR(Wpack); REQUIRE_PTR(q); REQUIRE_PTR(k); REQUIRE_PTR(v);
    REQUIRE_PTR(alpha); REQUIRE_PTR(beta);
    const hipStream_t s = (hipStream_t)stream;
    const int M = desc->B * desc->L;
    hipError_t e = project(desc->act == GDN_F32, M, desc->d, desc->H, desc->dk, x, Wpack, q, k, v, alpha,
                           beta, desc->alpha_lo, desc->norm_eps, nullptr, s);
    return e == hipSuccess ? GDN_OK : hip_fail(e, "projection launch");
}

// The chunk preparation and the carry.  With `bwd_mats` the preparation also
// writes the chunk matrices of the backward pass there.
static gdn_status scan_chunks(const gdn_desc *d, const void *q, const void *k, const void *v,
                              GateSrc gates, const float *s_init, float *s_final, CarryOut out, void *ws,
                              const Layout &lo, hipStream_t s, float *bwd_mats = nullptr,
                              hipStream_t carry_stream = nullptr, hipEvent_t prep_done = nullptr) {
    const bool f32 = d->act == GDN_F32;
    ChunkWs cw{(float *)at(ws, lo.W), (float *)at(ws, lo.M), (float *)at(ws, lo.g)};
    if (bwd_mats) cw.bwd = bwd_prep_out(bwd_mats, (int64_t)d->B * d->H * ((d->L + 63) / 64), d->dk);
    hipError_t e = timed(GDN_STAGE_SCAN_PREP, s, [&] {
        return launch_scan_prep(f32, d->B, d->L, d->H, d->dk, q, k, gates, cw, s);
    });
    if (e != hipSuccess) return hip_fail(e, "chunk prep launch");
    // the carry on a stream of its own (the pipelined loop prefill): it waits for the prep's event
    hipStream_t cs = s;
    if (carry_stream && carry_stream != s) {
        if ((e = hipEventRecord(prep_done, s)) != hipSuccess || (e = hipStreamWaitEvent(carry_stream, prep_done, 0)) != hipSuccess)
            return hip_fail(e, "carry stream wait");
        cs = carry_stream;
    }
    e = timed(GDN_STAGE_SCAN_CARRY, cs, [&] {
        return launch_scan_carry(f32, d->B, d->L, d->H, d->dk, q, k, v, cw, s_init, s_final, out, cs);
    });
    if (e != hipSuccess) return hip_fail(e, "carry launch");
    return GDN_OK;
}

gdn_status gdn_scan_prefill(const gdn_desc *desc, const void *q, const void *k, const void *v,
                            const float *alpha, const float *beta, const float *s_init, float *o,
                            float *s_final, void *ws, size_t ws_bytes, void *stream) {
    gdn_status st = check_desc(desc, false);
    if (st != GDN_OK) return st;
    if ((st = check_prefill_grid(desc)) != GDN_OK) return st;
    REQUIRE_PTR(q); REQUIRE_PTR(k); REQUIRE_PTR(v); REQUIRE_PTR(alpha); REQUIRE_PTR(beta);
    REQUIRE_PTR(o); OPTIONAL_PTR(s_init); OPTIONAL_PTR(s_final);
    if (s_init && s_init == s_final) return fail(GDN_ERR_SHAPE, "s_final may not alias s_init");
    const Layout lo = layout(desc, GDN_OP_SCAN_PREFILL);
    if (!ws || ws_bytes < lo.total)
        return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", lo.total, ws_bytes);
    if (!aligned16(ws)) return fail(GDN_ERR_ALIGN, "ws is not 16-byte aligned");
    CarryOut out{o, nullptr, false, nullptr, nullptr, nullptr};
    return scan_chunks(desc, q, k, v, GateSrc{alpha, beta, nullptr, 0, desc->alpha_lo, nullptr, nullptr}, s_init,
                       s_final, out,
                       ws, lo, (hipStream_t)stream);
}

gdn_status gdn_scan_backward(const gdn_desc *desc, const void *q, const void *k, const void *v,
                             const float *alpha, const float *beta, const float *s_init, const float *d_o,
                             const float *d_sfinal, float *dq, float *dk, float *dv, float *dalpha, float *dbeta,
                             float *ds_init, void *ws, size_t ws_bytes, void *stream) {
    gdn_status st = check_desc(desc, false);
    if (st != GDN_OK) return st;
    if ((st = check_prefill_grid(desc)) != GDN_OK) return st;
    if (desc->act == GDN_F32 && desc->dk == 128)
        return fail(GDN_ERR_UNSUPPORTED, "the backward pass takes fp32 inputs with dk = 64 only");
    REQUIRE_PTR(q); REQUIRE_PTR(k); REQUIRE_PTR(v); REQUIRE_PTR(alpha); REQUIRE_PTR(beta); REQUIRE_PTR(d_o);
    REQUIRE_PTR(dq); REQUIRE_PTR(dk); REQUIRE_PTR(dv); REQUIRE_PTR(dalpha); REQUIRE_PTR(dbeta);
    OPTIONAL_PTR(s_init); OPTIONAL_PTR(d_sfinal); OPTIONAL_PTR(ds_init);
    const Layout lo = layout(desc, GDN_OP_SCAN_BACKWARD);
    if (!ws || ws_bytes < lo.total)
        return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", lo.total, ws_bytes);
    if (!aligned16(ws)) return fail(GDN_ERR_ALIGN, "ws is not 16-byte aligned");
    const hipStream_t s = (hipStream_t)stream;
    const bool f32 = desc->act == GDN_F32;
    const int B = desc->B, L = desc->L, H = desc->H, D = desc->dk;
    // forward recomputation: the chunk matrices, then the state chain with the chunk-start states kept
    float *sc = (float *)at(ws, lo.sc), *dse = (float *)at(ws, lo.dse), *bm = (float *)at(ws, lo.bm);
    CarryOut out{nullptr, nullptr, false, nullptr, nullptr, nullptr, sc};
    st = scan_chunks(desc, q, k, v, GateSrc{alpha, beta, nullptr, 0, desc->alpha_lo, nullptr, nullptr}, s_init,
                     nullptr, out, ws, lo, s, bm);
    if (st != GDN_OK) return st;
    hipError_t e = timed(GDN_STAGE_BWD_OPS, s, [&] { return launch_bwd_ops(B, L, H, D, d_o, bm, s); });
    if (e != hipSuccess) return hip_fail(e, "backward carry operands launch");
    e = timed(GDN_STAGE_BWD_CARRY, s, [&] {
        return launch_bwd_carry(f32, B, L, H, D, d_o, d_sfinal, bm, dv, dse, ds_init, s);
    });
    if (e != hipSuccess) return hip_fail(e, "backward carry launch");
    e = timed(GDN_STAGE_BWD_CHUNK, s, [&] {
        return launch_bwd_chunk(f32, B, L, H, D, q, k, v, alpha, beta, d_o, dv, sc, dse, bm, dq, dk, dalpha, dbeta,
                                s);
    });
    if (e != hipSuccess) return hip_fail(e, "backward chunk launch");
    return GDN_OK;
}

gdn_status gdn_loop_backward(const gdn_desc *desc, const void *h0, const void *Wpack, const float *rho,
                             const float *h_loops, const float *dh, float *dh0, float *dWq, float *dWk, float *dWv,
                             float *dwa, float *dwb, float *drho, void *ws, size_t ws_bytes, void *stream) {
    gdn_status st = check_desc(desc, false);
    if (st != GDN_OK) return st;
    if ((st = check_prefill_grid(desc)) != GDN_OK) return st;
    if ((st = check_loop_backward(desc)) != GDN_OK) return st;
    const bool f32 = desc->act == GDN_F32;
    if (f32 && desc->dk == 128)
        return fail(GDN_ERR_UNSUPPORTED, "the backward pass takes fp32 inputs with dk = 64 only");
    REQUIRE_PTR(h0); REQUIRE_PTR(Wpack); REQUIRE_PTR(rho); REQUIRE_PTR(dh); REQUIRE_PTR(dh0);
    REQUIRE_PTR(dWq); REQUIRE_PTR(dWk); REQUIRE_PTR(dWv); REQUIRE_PTR(dwa); REQUIRE_PTR(dwb); REQUIRE_PTR(drho);
    if (desc->T > 1) REQUIRE_PTR(h_loops);
    else OPTIONAL_PTR(h_loops);
    if (dh0 == dh) return fail(GDN_ERR_SHAPE, "dh0 may not alias dh");
    const Layout lo = layout(desc, GDN_OP_LOOP_BACKWARD);
    if (!ws || ws_bytes < lo.total)
        return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", lo.total, ws_bytes);
    if (!aligned16(ws)) return fail(GDN_ERR_ALIGN, "ws is not 16-byte aligned");

    const hipStream_t s = (hipStream_t)stream;
    const int B = desc->B, L = desc->L, H = desc->H, D = desc->dk, d = desc->d, T = desc->T;
    const int M = B * L, Mp = (M + 63) / 64 * 64;
    float *zp = lo.P ? (float *)at(ws, lo.zp) : nullptr;   // gate partials, as in the forward
    bf16 *xb = f32 ? nullptr : (bf16 *)at(ws, lo.x);
    const int P = (int)packed_rows(H, D);
    const int64_t qkvp = qkv_rows_padded(H, D);
    void *q = at(ws, lo.q), *k = at(ws, lo.k), *v = at(ws, lo.v);
    float *al = (float *)at(ws, lo.alpha), *be = (float *)at(ws, lo.beta);
    float *Y = (float *)at(ws, lo.Y), *YT = (float *)at(ws, lo.YT), *dW = (float *)at(ws, lo.dW);
    void *XT = at(ws, lo.XT), *WT = at(ws, lo.WT);
    float *gq = (float *)at(ws, lo.gq), *gk = (float *)at(ws, lo.gk), *gv = (float *)at(ws, lo.gv);
    float *gal = (float *)at(ws, lo.gal), *gbe = (float *)at(ws, lo.gbe), *part = (float *)at(ws, lo.part);
    float *bufs[2] = {(float *)at(ws, lo.dhA), (float *)at(ws, lo.dhB)};
    float *sc = (float *)at(ws, lo.sc), *dse = (float *)at(ws, lo.dse), *bm = (float *)at(ws, lo.bm);
    const int wmode = f32 ? OPND_F32_SPLIT : OPND_BF16;
    const int64_t tokd = (int64_t)M * d;

    hipError_t e = launch_transpose(f32, f32, Wpack, d, P, d, WT, P, P, s);   // W^T [d][P]
    if (e != hipSuccess) return hip_fail(e, "weight transpose launch");
    // bf16: dY W and x^T dY split their k ranges so that their tiles fill the chip
    const int dx_split = f32 ? 1 : lb_dx_split(M, d), dw_split = lb_dw_split(d, P, f32);
    // (the first loop's x^T dY stores the accumulators, later loops add to them; the fp32 path accumulates
    // from zero)
    if (f32 && (e = launch_fill_zero(dW, (int64_t)d * P * dw_split, s)) != hipSuccess) return hip_fail(e, "fill launch");
    for (int tau = T - 1; tau >= 0; --tau) {
        // loop tau + 1 of the forward: input h^(tau), incoming gradient dL/dh^(tau+1)
        const bool hp_f32 = f32 || tau > 0;
        const void *hp = tau == 0 ? h0 : (const void *)(h_loops + (int64_t)(tau - 1) * tokd);
        const float *g_in = tau == T - 1 ? dh : bufs[(T - 2 - tau) & 1];
        float *g_out = tau == 0 ? dh0 : bufs[(T - 1 - tau) & 1];
        // The loop's operand (bf16(h) for bf16 workloads, rounded as the forward's carry rounds it) and its
        // q, k, v and gates from the forward's own kernels, launched as gdn_loop_prefill launches them: the
        // same values bit for bit, so this is the gradient of the forward that produced h_loops.
        const void *x = hp;
        if (!f32 && tau > 0) {
            if ((e = launch_lb_round(tokd, (const float *)hp, xb, s)) != hipSuccess) return hip_fail(e, "round launch");
            x = xb;
        }
        // the raw projections in fp32 (the normalisation's and the gates' gradients need them): from the
        // projection GEMM itself where it forms the gate partials (the raw gates are their sums), else from
        // one more product
        const bool raw_in_gemm = zp != nullptr;
        e = project(f32, M, d, H, D, x, Wpack, q, k, v, al, be, desc->alpha_lo, desc->norm_eps, zp, s, nullptr,
                    nullptr, raw_in_gemm ? Y : nullptr, P);
        if (e != hipSuccess) return hip_fail(e, "projection launch");
        if (!raw_in_gemm) {
            e = timed(GDN_STAGE_BWD_GEMM, s, [&] {
                if (f32)
                    return launch_gemm_nt(OPND_F32_SPLIT, wmode, EPI_STORE, x, d, Wpack, d, M, P, d, Y, P, nullptr,
                                          nullptr, 0, s);
                return launch_gemm_tile(EPI_STORE, true, (const bf16 *)x, nullptr, d, (const bf16 *)Wpack, nullptr,
                                        d, M, P, d, Y, P, nullptr, nullptr, 0, nullptr, 0, s);
            });
            if (e != hipSuccess) return hip_fail(e, "projection recompute launch");
        }
        // the scan backward from S = 0 with dO = dL/dh^(tau+1) (the mixer output is h's width); with gate
        // partials the prep forms alpha and beta into their workspace regions, as in the forward
        CarryOut out{nullptr, nullptr, false, nullptr, nullptr, nullptr, sc};
        st = scan_chunks(desc, q, k, v, GateSrc{al, be, zp, lo.P, desc->alpha_lo, zp ? al : nullptr, zp ? be : nullptr},
                         nullptr, nullptr, out, ws, lo, s, bm);
        if (st != GDN_OK) return st;
        e = timed(GDN_STAGE_BWD_OPS, s, [&] { return launch_bwd_ops(B, L, H, D, g_in, bm, s); });
        if (e != hipSuccess) return hip_fail(e, "backward carry operands launch");
        e = timed(GDN_STAGE_BWD_CARRY, s, [&] {
            return launch_bwd_carry(f32, B, L, H, D, g_in, nullptr, bm, gv, dse, nullptr, s);
        });
        if (e != hipSuccess) return hip_fail(e, "backward carry launch");
        e = timed(GDN_STAGE_BWD_CHUNK, s, [&] {
            return launch_bwd_chunk(f32, B, L, H, D, q, k, v, al, be, g_in, gv, sc, dse, bm, gq, gk, gal, gbe, s);
        });
        if (e != hipSuccess) return hip_fail(e, "backward chunk launch");
        // through the normalisation and the gates: Y <- dY
        e = launch_lb_epilogue_grad(M, H, D, Y, P, qkvp, desc->norm_eps, desc->alpha_lo, gq, gk, gv, gal, gbe,
                                    raw_in_gemm ? zp : nullptr, lo.P, s);
        if (e != hipSuccess) return hip_fail(e, "epilogue gradient launch");
        e = launch_lb_drho(M, d, g_in, hp, hp_f32, part, drho + (int64_t)tau * d, s);
        if (e != hipSuccess) return hip_fail(e, "rho gradient launch");
        // dL/dh^(tau) = rho_tau (.) dL/dh^(tau+1) + dY W, then dW^T [d][P] += x^T dY; dY enters the bf16
        // products as two bf16 planes (hi + lo)
        if (f32) {
            e = timed(GDN_STAGE_BWD_GEMM, s, [&] {
                return launch_gemm_nt(OPND_F32_SPLIT, wmode, EPI_RESID, Y, P, WT, P, M, d, P, g_out, d,
                                      rho + (int64_t)tau * d, g_in, d, s);
            });
            if (e != hipSuccess) return hip_fail(e, "input gradient launch");
            if ((e = launch_transpose(f32, f32, x, d, M, d, XT, Mp, Mp, s)) != hipSuccess ||
                (e = launch_transpose(true, true, Y, P, M, P, YT, Mp, Mp, s)) != hipSuccess)
                return hip_fail(e, "transpose launch");
            e = timed(GDN_STAGE_BWD_GEMM, s, [&] {
                return launch_gemm_nt(OPND_F32_SPLIT, OPND_F32_SPLIT, EPI_ACCUM, XT, Mp, YT, Mp, d, P, Mp, dW, P,
                                      nullptr, nullptr, 0, s);
            });
        } else {
            bf16 *Yh = (bf16 *)at(ws, lo.Yhl), *Yl = Yh + (int64_t)M * P;
            bf16 *YTh = (bf16 *)YT, *YTl = YTh + (int64_t)P * Mp;
            // dY as bf16 hi/lo planes for dY W, and transposed for x^T dY, from one read
            if ((e = launch_split_both(Y, P, M, P, Yh, Yl, P, YTh, YTl, Mp, Mp, s)) != hipSuccess)
                return hip_fail(e, "split launch");
            if (dx_split == 1) {
                e = timed(GDN_STAGE_BWD_GEMM, s, [&] {
                    return launch_gemm_tile(EPI_RESID, true, Yh, Yl, P, (const bf16 *)WT, nullptr, P, M, d, P, g_out,
                                            d, rho + (int64_t)tau * d, g_in, d, nullptr, 0, s);
                });
            } else {
                float *Gp = (float *)at(ws, lo.Gp);
                e = timed(GDN_STAGE_BWD_GEMM, s, [&] {
                    return launch_gemm_tile(EPI_STORE, true, Yh, Yl, P, (const bf16 *)WT, nullptr, P, M, d, P, Gp, d,
                                            nullptr, nullptr, 0, nullptr, 0, s, dx_split, (int64_t)M * d);
                });
                if (e == hipSuccess)
                    e = launch_sum_parts(M, d, Gp, dx_split, (int64_t)M * d, rho + (int64_t)tau * d, g_in, g_out, s);
            }
            if (e != hipSuccess) return hip_fail(e, "input gradient launch");
            if ((e = launch_transpose(false, false, x, d, M, d, XT, Mp, Mp, s)) != hipSuccess)
                return hip_fail(e, "transpose launch");
            e = timed(GDN_STAGE_BWD_GEMM, s, [&] {
                return launch_gemm_tile(tau == T - 1 ? EPI_STORE : EPI_ACCUM, true, (const bf16 *)XT, nullptr, Mp,
                                        YTh, YTl, Mp, d, P, Mp, dW, P, nullptr, nullptr, 0, nullptr, 0, s, dw_split,
                                        (int64_t)d * P);
            });
        }
        if (e != hipSuccess) return hip_fail(e, "weight gradient launch");
    }
    e = launch_lb_unpack(d, H, D, dW, dw_split, (int64_t)d * P, P, qkvp, dWq, dWk, dWv, dwa, dwb, s);
    return e == hipSuccess ? GDN_OK : hip_fail(e, "weight gradient unpack launch");
}

// ---- the LT2 block ------------------------------------------------------------
namespace {

// Offsets (bytes) of a packed block: the mixer's packed weights, Wg^T [HD][d],
// Wo^T [d][HD], W13 [2F][d] (interleaved), W2^T [d][F], g1, g2 [d] fp32.
struct BlockPack {
    size_t mix = 0, wg = 0, wo = 0, w13 = 0, w2 = 0, g1 = 0, g2 = 0, total = 0;
};
BlockPack block_pack_layout(const gdn_desc *d, int F) {
    BlockPack b;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += align_up(bytes);
        return at;
    };
    const size_t ab = act_bytes(d), HD = (size_t)d->H * d->dv, D = d->d;
    b.mix = take((size_t)packed_rows(d->H, d->dk) * D * ab);
    b.wg = take(HD * D * ab);
    b.wo = take(D * HD * ab);
    b.w13 = take((size_t)2 * F * D * ab);
    b.w2 = take(D * (size_t)F * ab);
    b.g1 = take(D * 4);
    b.g2 = take(D * 4);
    b.total = off;
    return b;
}

// The block's workspace: the loop prefill's (q, k, v, gates, gate partials,
// chunk matrices), then X1, O, Z, H1, X2, U and the fp32 stream buffers of
// the loop (its converted input, two loop outputs, two block outputs).
struct BlockLayout {
    Layout lo;
    size_t x1 = 0, o = 0, z = 0, h1 = 0, x2 = 0, u = 0, hin = 0, lp[2] = {0, 0}, ch[2] = {0, 0}, total = 0;
};
BlockLayout block_layout(const gdn_desc *d, int F) {
    BlockLayout b;
    b.lo = layout(d, GDN_OP_LOOP_PREFILL);
    size_t off = b.lo.total;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += align_up(bytes);
        return at;
    };
    const size_t M = (size_t)d->B * d->L, ab = act_bytes(d), HD = (size_t)d->H * d->dv, D = d->d;
    b.x1 = take(M * D * ab);
    b.o = take(M * HD * 4);
    b.z = take(M * HD * ab);
    b.h1 = take(M * D * 4);
    b.x2 = take(M * D * ab);
    b.u = take(M * (size_t)F * ab);
    b.hin = take(M * D * 4);
    b.lp[0] = take(M * D * 4);
    b.lp[1] = take(M * D * 4);
    b.ch[0] = take(M * D * 4);
    b.ch[1] = take(M * D * 4);
    b.total = off;
    return b;
}

gdn_status check_block(const gdn_desc *desc, int ffn) {
    gdn_status st = check_desc(desc, false);
    if (st != GDN_OK) return st;
    if ((st = check_prefill_grid(desc)) != GDN_OK) return st;
    if (ffn <= 0 || ffn % 64) return fail(GDN_ERR_SHAPE, "ffn must be a positive multiple of 64 (got %d)", ffn);
    if ((int64_t)desc->B * desc->L * ffn > ((int64_t)1 << 40)) return fail(GDN_ERR_SHAPE, "problem too large");
    return GDN_OK;
}

// One product of the block: bf16 workloads on the tiled kernel, fp32 ones on
// the split-operand kernel.
hipError_t block_gemm(bool f32, int epi, bool out_f32, const void *A, int64_t lda, const void *B, int64_t ldb, int M,
                      int N, int K, void *C, int64_t ldc, const float *rho, const float *D1, int64_t ldd1,
                      const float *D2, int64_t ldd2, hipStream_t s) {
    return timed(GDN_STAGE_BLOCK_GEMM, s, [&] {
        if (f32)
            return launch_gemm_nt_ex(OPND_F32_SPLIT, OPND_F32_SPLIT, epi, out_f32, A, lda, B, ldb, M, N, K, C, ldc,
                                     rho, D1, ldd1, D2, ldd2, s);
        return launch_gemm_tile(epi, out_f32, (const bf16 *)A, nullptr, lda, (const bf16 *)B, nullptr, ldb, M, N, K,
                                C, ldc, rho, D1, ldd1, D2, ldd2, s);
    });
}

// out = F(hin) (+ rho (.) hres when rho is given: the loop residual of the
// stack's last block, fused into the down projection).
gdn_status block_apply(const gdn_desc *desc, int F, const float *hin, const char *Wb, float *out, const float *rho,
                       const float *hres, void *ws, const BlockLayout &bl, hipStream_t s) {
    const bool f32 = desc->act == GDN_F32;
    const int M = desc->B * desc->L, d = desc->d, H = desc->H, D = desc->dk, HD = desc->H * desc->dv;
    const BlockPack bp = block_pack_layout(desc, F);
    const Layout &lo = bl.lo;
    void *x1 = at(ws, bl.x1), *z = at(ws, bl.z), *x2 = at(ws, bl.x2), *u = at(ws, bl.u);
    float *o = (float *)at(ws, bl.o), *h1 = (float *)at(ws, bl.h1);
    void *q = at(ws, lo.q), *k = at(ws, lo.k), *v = at(ws, lo.v);
    float *al = (float *)at(ws, lo.alpha), *be = (float *)at(ws, lo.beta);
    float *zp = lo.P ? (float *)at(ws, lo.zp) : nullptr;
    const float *g1 = (const float *)(Wb + bp.g1), *g2 = (const float *)(Wb + bp.g2);
    hipError_t e = launch_rmsnorm(true, f32, M, d, hin, g1, desc->norm_eps, x1, s);
    if (e != hipSuccess) return hip_fail(e, "norm launch");
    e = project(f32, M, d, H, D, x1, Wb + bp.mix, q, k, v, al, be, desc->alpha_lo, desc->norm_eps, zp, s);
    if (e != hipSuccess) return hip_fail(e, "projection launch");
    CarryOut out_o{o, nullptr, false, nullptr, nullptr, nullptr, nullptr, nullptr};
    gdn_status st = scan_chunks(desc, q, k, v,
                                GateSrc{al, be, zp, lo.P, desc->alpha_lo, zp ? al : nullptr, zp ? be : nullptr},
                                nullptr, nullptr, out_o, ws, lo, s);
    if (st != GDN_OK) return st;
    // z = o (.) sigmoid(x1 Wg); h1 = h + z Wo
    if ((e = block_gemm(f32, EPI_GATE, f32, x1, d, Wb + bp.wg, d, M, HD, d, z, HD, nullptr, o, HD, nullptr, 0, s)) !=
        hipSuccess)
        return hip_fail(e, "gate product launch");
    if ((e = block_gemm(f32, EPI_ADD, true, z, HD, Wb + bp.wo, HD, M, d, HD, h1, d, nullptr, hin, d, nullptr, 0, s)) !=
        hipSuccess)
        return hip_fail(e, "output projection launch");
    // FFN: u = silu(x2 W1) (.) (x2 W3); out = h1 + u W2 (+ rho (.) hres)
    if ((e = launch_rmsnorm(true, f32, M, d, h1, g2, desc->norm_eps, x2, s)) != hipSuccess)
        return hip_fail(e, "norm launch");
    if ((e = block_gemm(f32, EPI_SWIGLU, f32, x2, d, Wb + bp.w13, d, M, 2 * F, d, u, F, nullptr, nullptr, 0, nullptr,
                        0, s)) != hipSuccess)
        return hip_fail(e, "FFN up-projection launch");
    e = block_gemm(f32, rho ? EPI_ADD_RESID : EPI_ADD, true, u, F, Wb + bp.w2, F, M, d, F, out, d, rho, h1, d, hres,
                   d, s);
    return e == hipSuccess ? GDN_OK : hip_fail(e, "FFN down-projection launch");
}

}  // namespace

gdn_status gdn_block_packed_bytes(const gdn_desc *desc, int ffn, size_t *bytes) {
    gdn_status st = check_desc(desc, false);
    if (st != GDN_OK) return st;
    if (ffn <= 0 || ffn % 64) return fail(GDN_ERR_SHAPE, "ffn must be a positive multiple of 64 (got %d)", ffn);
    if (!bytes) return fail(GDN_ERR_NULL, "bytes is NULL");
    *bytes = block_pack_layout(desc, ffn).total;
    return GDN_OK;
}

gdn_status gdn_block_pack(const gdn_desc *desc, int ffn, const float *g1, const void *Wq, const void *Wk,
                          const void *Wv, const void *wa, const void *wb, const void *Wg, const void *Wo,
                          const float *g2, const void *W1, const void *W3, const void *W2, void *Wblock,
                          void *stream) {
    gdn_status st = check_desc(desc, false);
    if (st != GDN_OK) return st;
    if (ffn <= 0 || ffn % 64) return fail(GDN_ERR_SHAPE, "ffn must be a positive multiple of 64 (got %d)", ffn);
    REQUIRE_PTR(g1); REQUIRE_PTR(Wq); REQUIRE_PTR(Wk); REQUIRE_PTR(Wv); REQUIRE_PTR(wa); REQUIRE_PTR(wb);
    REQUIRE_PTR(Wg); REQUIRE_PTR(Wo); REQUIRE_PTR(g2); REQUIRE_PTR(W1); REQUIRE_PTR(W3); REQUIRE_PTR(W2);
    REQUIRE_PTR(Wblock);
    if (((uintptr_t)Wblock) % 256) return fail(GDN_ERR_ALIGN, "Wblock is not 256-byte aligned");
    const hipStream_t s = (hipStream_t)stream;
    const bool f32 = desc->act == GDN_F32;
    const int d = desc->d, HD = desc->H * desc->dv;
    const BlockPack bp = block_pack_layout(desc, ffn);
    char *W = (char *)Wblock;
    hipError_t e = launch_pack_weights(f32, d, desc->H, desc->dk, Wq, Wk, Wv, wa, wb, W + bp.mix, s);
    if (e == hipSuccess) e = launch_transpose(f32, f32, Wg, HD, d, HD, W + bp.wg, d, d, s);     // [HD][d]
    if (e == hipSuccess) e = launch_transpose(f32, f32, Wo, d, HD, d, W + bp.wo, HD, HD, s);    // [d][HD]
    if (e == hipSuccess) e = launch_pack_w13(f32, d, ffn, W1, W3, W + bp.w13, s);
    if (e == hipSuccess) e = launch_transpose(f32, f32, W2, d, ffn, d, W + bp.w2, ffn, ffn, s); // [d][F]
    if (e == hipSuccess) e = launch_copy_f32(g1, (float *)(W + bp.g1), d, s);
    if (e == hipSuccess) e = launch_copy_f32(g2, (float *)(W + bp.g2), d, s);
    return e == hipSuccess ? GDN_OK : hip_fail(e, "block pack launch");
}

gdn_status gdn_block_workspace_bytes(const gdn_desc *desc, int ffn, size_t *bytes) {
    gdn_status st = check_block(desc, ffn);
    if (st != GDN_OK) return st;
    if (!bytes) return fail(GDN_ERR_NULL, "bytes is NULL");
    *bytes = block_layout(desc, ffn).total;
    return GDN_OK;
}

gdn_status gdn_block_workspace_region(const gdn_desc *desc, int ffn, int region, size_t *offset, size_t *bytes) {
    gdn_status st = check_block(desc, ffn);
    if (st != GDN_OK) return st;
    if (!offset || !bytes) return fail(GDN_ERR_NULL, "offset or bytes is NULL");
    const BlockLayout bl = block_layout(desc, ffn);
    const size_t M = (size_t)desc->B * desc->L, ab = act_bytes(desc), HD = (size_t)desc->H * desc->dv;
    const size_t D = desc->d, qkv = M * desc->H * desc->dk * ab, gate = M * desc->H * 4;
    switch (region) {
        case GDN_WS_Q: *offset = bl.lo.q; *bytes = qkv; break;
        case GDN_WS_K: *offset = bl.lo.k; *bytes = qkv; break;
        case GDN_WS_V: *offset = bl.lo.v; *bytes = qkv; break;
        case GDN_WS_ALPHA: *offset = bl.lo.alpha; *bytes = gate; break;
        case GDN_WS_BETA: *offset = bl.lo.beta; *bytes = gate; break;
        case GDN_BWS_X1: *offset = bl.x1; *bytes = M * D * ab; break;
        case GDN_BWS_O: *offset = bl.o; *bytes = M * HD * 4; break;
        case GDN_BWS_Z: *offset = bl.z; *bytes = M * HD * ab; break;
        case GDN_BWS_H1: *offset = bl.h1; *bytes = M * D * 4; break;
        case GDN_BWS_X2: *offset = bl.x2; *bytes = M * D * ab; break;
        case GDN_BWS_U: *offset = bl.u; *bytes = M * (size_t)ffn * ab; break;
        default: return fail(GDN_ERR_UNSUPPORTED, "unknown block workspace region %d", region);
    }
    return GDN_OK;
}

gdn_status gdn_block_forward(const gdn_desc *desc, int ffn, const float *h, const void *Wblock, float *out,
                             void *ws, size_t ws_bytes, void *stream) {
    gdn_status st = check_block(desc, ffn);
    if (st != GDN_OK) return st;
    REQUIRE_PTR(h); REQUIRE_PTR(Wblock); REQUIRE_PTR(out);
    if ((const void *)out == (const void *)h) return fail(GDN_ERR_SHAPE, "out may not alias h");
    const BlockLayout bl = block_layout(desc, ffn);
    if (!ws || ws_bytes < bl.total)
        return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", bl.total, ws_bytes);
    if (!aligned16(ws)) return fail(GDN_ERR_ALIGN, "ws is not 16-byte aligned");
    return block_apply(desc, ffn, h, (const char *)Wblock, out, nullptr, nullptr, ws, bl, (hipStream_t)stream);
}

gdn_status gdn_block_loop_prefill(const gdn_desc *desc, int ffn, int layers, const void *h0, const void *Wblocks,
                                  const float *rho, float *h_out, void *ws, size_t ws_bytes, void *stream) {
    gdn_status st = check_block(desc, ffn);
    if (st != GDN_OK) return st;
    if (layers < 1) return fail(GDN_ERR_SHAPE, "layers must be >= 1 (got %d)", layers);
    REQUIRE_PTR(h0); REQUIRE_PTR(Wblocks); REQUIRE_PTR(rho); REQUIRE_PTR(h_out);
    if ((const void *)h_out == h0) return fail(GDN_ERR_SHAPE, "h_out may not alias h0");
    const BlockLayout bl = block_layout(desc, ffn);
    if (!ws || ws_bytes < bl.total)
        return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", bl.total, ws_bytes);
    if (!aligned16(ws)) return fail(GDN_ERR_ALIGN, "ws is not 16-byte aligned");
    const hipStream_t s = (hipStream_t)stream;
    const bool f32 = desc->act == GDN_F32;
    const int64_t n = (int64_t)desc->B * desc->L * desc->d;
    const size_t stride = block_pack_layout(desc, ffn).total;
    // the loop stream is fp32: a bf16 h0 is widened once
    const float *hin0 = (const float *)h0;
    if (!f32) {
        hipError_t e = launch_bf16_to_f32((const bf16 *)h0, (float *)at(ws, bl.hin), n, s);
        if (e != hipSuccess) return hip_fail(e, "widen launch");
        hin0 = (const float *)at(ws, bl.hin);
    }
    const int T = desc->T;
    for (int tau = 0; tau < T; ++tau) {
        const float *hp = tau == 0 ? hin0 : (const float *)at(ws, bl.lp[(tau - 1) & 1]);
        float *loop_out = tau == T - 1 ? h_out : (float *)at(ws, bl.lp[tau & 1]);
        const float *x = hp;
        for (int l = 0; l < layers; ++l) {
            const bool last = l == layers - 1;
            float *dst = last ? loop_out : (float *)at(ws, bl.ch[l & 1]);
            st = block_apply(desc, ffn, x, (const char *)Wblocks + (size_t)l * stride, dst,
                             last ? rho + (int64_t)tau * desc->d : nullptr, last ? hp : nullptr, ws, bl, s);
            if (st != GDN_OK) return st;
            x = dst;
        }
    }
    return GDN_OK;
}

gdn_status gdn_scan_decode(const gdn_desc *desc, const void *q, const void *k, const void *v,
                           const float *alpha, const float *beta, float *states, float *o,
                           void *stream) {
    gdn_status st = check_desc(desc, true);
    if (st != GDN_OK) return st;
    REQUIRE_PTR(q); REQUIRE_PTR(k); REQUIRE_PTR(v); REQUIRE_PTR(alpha); REQUIRE_PTR(beta);
    REQUIRE_PTR(states); REQUIRE_PTR(o);
    const hipStream_t s = (hipStream_t)stream;
    hipError_t e = timed(GDN_STAGE_DECODE, s, [&] {
        return launch_decode(desc->act == GDN_F32, desc->B, desc->H, desc->dk, q, k, v, alpha, beta,
                             states, o, nullptr, false, nullptr, nullptr, nullptr, s);
    });
    return e == hipSuccess ? GDN_OK : hip_fail(e, "decode launch");
}

// The halting of gdn_loop_prefill_act (nullptr for the plain loops).
struct ActArgs {
    const float *w;
    float b, thr;
    float *R;
    int *halt;
    int *rows, *rows_count;   // the positions re-projected in the next loop
    int32_t *halt_out;
    float *ponder;
};

static gdn_status loop_prefill_impl(const gdn_desc *desc, const void *h0, const void *Wpack, const float *rho,
                                    float *h_out, float *states_out, float *h_loops, void *ws, const Layout &lo,
                                    hipStream_t s, const ActArgs *act) {
    const bool f32 = desc->act == GDN_F32;
    const int M = desc->B * desc->L, D = desc->dk, d = desc->d;
    const int64_t tokd = (int64_t)M * d;
    void *q = at(ws, lo.q), *k = at(ws, lo.k), *v = at(ws, lo.v);
    float *al = (float *)at(ws, lo.alpha), *be = (float *)at(ws, lo.beta);
    float *zp = lo.P ? (float *)at(ws, lo.zp) : nullptr;   // gate partials, when the GEMM makes them
    bf16 *xbuf = f32 ? nullptr : (bf16 *)at(ws, lo.x);
    const int64_t state_elems = (int64_t)desc->B * desc->H * D * D;
    hipError_t e;
    if (act && (e = launch_act_init(M, act->R, act->halt, s)) != hipSuccess) return hip_fail(e, "halting init launch");

    const void *x = h0;            // GEMM operand of loop tau
    const void *hprev = h0;        // h^(tau-1) for the residual
    bool hprev_bf16 = !f32;
    for (int tau = 0; tau < desc->T; ++tau) {
        const bool last = tau == desc->T - 1;
        float *hdst = h_loops ? h_loops + tau * tokd : h_out;  // h^(tau+1), in place over h_out
        // Under halting a position that did not run the previous loop keeps its
        // projection input, so its q, k, v and gates from then stand; with the
        // row-list projection only the positions that ran it are projected again.
        // (the row-list loads address x with 32-bit byte offsets)
        const bool compact = act && tau > 0 && zp && (int64_t)M * d * 2 < (int64_t(1) << 32);
        if (compact && (e = launch_act_rows(M, act->halt, tau, act->rows, act->rows_count, s)) != hipSuccess)
            return hip_fail(e, "halting row list launch");
        e = project(f32, M, d, desc->H, D, x, Wpack, q, k, v, al, be, desc->alpha_lo, desc->norm_eps, zp, s,
                    compact ? act->rows : nullptr, compact ? act->rows_count : nullptr);
        if (e != hipSuccess) return hip_fail(e, "projection launch");
        // (no position has halted before the first loop's decision)
        CarryOut out{nullptr, hprev, hprev_bf16, rho + (int64_t)tau * d, hdst, (!f32 && !last) ? xbuf : nullptr,
                     nullptr, (act && tau > 0) ? act->halt : nullptr};
        // with gate partials the prep forms alpha and beta and stores them in the
        // workspace's gate regions, where gdn_loop_prefill documents them
        gdn_status st = scan_chunks(desc, q, k, v,
                                    GateSrc{al, be, zp, lo.P, desc->alpha_lo, zp ? al : nullptr, zp ? be : nullptr},
                                    nullptr, states_out ? states_out + tau * state_elems : nullptr, out, ws, lo, s);
        if (st != GDN_OK) return st;
        if (act) {
            e = launch_act_halt(M, d, hdst, act->w, act->b, act->thr, tau + 1, desc->T, act->R, act->halt,
                                act->halt_out, act->ponder, s);
            if (e != hipSuccess) return hip_fail(e, "halting launch");
        }
        hprev = hdst;
        hprev_bf16 = false;
        x = f32 ? (const void *)hdst : (const void *)xbuf;
    }
    if (h_loops) {
        e = hipMemcpyAsync(h_out, h_loops + (desc->T - 1) * tokd, tokd * sizeof(float), hipMemcpyDeviceToDevice, s);
        if (e != hipSuccess) return hip_fail(e, "copy of h^(T)");
    }
    return GDN_OK;
}

// ---- the pipelined loop prefill ----------------------------------------------
struct PipeRes {
    hipStream_t st[PIPE_STREAMS] = {};
    hipEvent_t fork = nullptr, done[PIPE_STREAMS] = {};
    std::vector<hipEvent_t> ev;   // two per loop: the end of loop tau's carry of piece j in ev[2 tau + j % 2]
    std::vector<hipEvent_t> evp;  // two per loop: the end of loop tau's chunk prep of piece j
};
std::mutex g_pipe_mu;   // one submission at a time: the streams and events are shared per device
PipeRes g_pipe_res[64];

int device_cus() {
    static int cus[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cus[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

// Tokens per piece for this call (0: the loops run one after another).
int pipe_piece_tokens(const gdn_desc *d, const Layout &lo) {
    int want = g_pipe_piece.load(std::memory_order_relaxed);
    if (!lo.st || want < 0) return 0;
    if (want == 0) {
        // automatic: two pieces per sequence, where the whole call's carry would
        // leave at least half the CUs idle (one 16-column slice workgroup per
        // CU) and the sequences are long enough for the projection of one loop
        // to hide behind the carry of another (measured on MI355X at 16 heads
        // of 128: one sequence of 16384 tokens 3.55 -> 3.07 ms, of 32768 tokens
        // 6.89 -> 5.79 ms; pieces of 4096 or 8192 gained less, and at 4096
        // tokens, or where the carry fills the CUs, pieces lose)
        if ((int64_t)d->B * d->H * (d->dk / 16) * 2 > device_cus() || d->L < PIPE_AUTO_MIN_L) return 0;
        want = (d->L + 1) / 2;
    }
    want = std::max(PIPE_MIN_PIECE, (int)std::min<int64_t>(((int64_t)want + 255) / 256 * 256, INT32_MAX / 2));
    if (want >= d->L && d->B == 1) return 0;   // a single piece: nothing to overlap
    return std::min(want, d->L);
}

// Per-device streams (non-blocking, default priority) and events, made on
// first use and kept until the process ends.
hipError_t pipe_resources(int T, PipeRes **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    PipeRes &r = g_pipe_res[dev];
    if (!r.fork) {
        for (int i = 0; i < PIPE_STREAMS; ++i) {
            if ((e = hipStreamCreateWithFlags(&r.st[i], hipStreamNonBlocking)) != hipSuccess) return e;
            if ((e = hipEventCreateWithFlags(&r.done[i], hipEventDisableTiming)) != hipSuccess) return e;
        }
        if ((e = hipEventCreateWithFlags(&r.fork, hipEventDisableTiming)) != hipSuccess) return e;
    }
    while ((int)r.ev.size() < 2 * T) {
        hipEvent_t ev;
        if ((e = hipEventCreateWithFlags(&ev, hipEventDisableTiming)) != hipSuccess) return e;
        r.ev.push_back(ev);
        if ((e = hipEventCreateWithFlags(&ev, hipEventDisableTiming)) != hipSuccess) return e;
        r.evp.push_back(ev);
    }
    *out = &r;
    return hipSuccess;
}

// The loops over pieces in wavefront order: step w issues piece w - tau of
// every loop tau, so each event is recorded (host order) before the wait on
// it, and any mapping of the streams onto hardware queues keeps the order of
// the dependencies.  Edges: loop tau's projection of piece j waits for loop
// tau-1's carry of piece j (its h rows and the q/k/v, gate-partial and chunk
// sub-regions it overwrites); loop tau's carry of piece j waits for the prep
// of piece j and follows its carry of piece j-1 on its stream (the state).  Within a piece the launches are those of the whole call
// (projection with gate partials, chunk prep, carry with the loop residual)
// on that piece's rows, its own gate-partial and chunk-matrix sub-regions, and
// the state of the previous piece of its sequence as the carry's start.  The
// arithmetic of every row is that of the whole call; only the carry's slice
// width may differ (it is chosen by the workgroup count of each launch).
static gdn_status loop_prefill_pipelined(const gdn_desc *desc, const void *h0, const void *Wpack, const float *rho,
                                         float *h_out, float *states_out, float *h_loops, void *ws, const Layout &lo,
                                         hipStream_t s, int piece) {
    const int B = desc->B, L = desc->L, H = desc->H, D = desc->dk, d = desc->d, T = desc->T;
    const int64_t M = (int64_t)B * L, tokd = M * d, Nc = (L + CHUNK - 1) / CHUNK;
    const int64_t state_elems = (int64_t)B * H * D * D, seq_state = (int64_t)H * D * D;
    struct Piece { int b, t0, len; bool first, last; int64_t cu; };   // cu: chunk units (b, h, c) before it
    std::vector<Piece> pieces;
    for (int b = 0; b < B; ++b)
        for (int t0 = 0; t0 < L;) {
            int len = std::min(piece, L - t0);
            if (L - (t0 + len) < PIPE_MIN_PIECE) len = L - t0;   // no short last piece
            pieces.push_back(Piece{b, t0, len, t0 == 0, t0 + len == L, 0});
            t0 += len;
        }
    int64_t cu = 0;
    for (Piece &p : pieces) {
        p.cu = cu;
        cu += (int64_t)H * ((p.len + CHUNK - 1) / CHUNK);
    }
    if (cu != (int64_t)B * H * Nc) return fail(GDN_ERR_SHAPE, "pieces do not tile the chunks");

    std::lock_guard<std::mutex> lock(g_pipe_mu);
    PipeRes *r = nullptr;
    hipError_t e = pipe_resources(T, &r);
    if (e != hipSuccess) return hip_fail(e, "pipeline streams");
    // stream 0: every projection and chunk prep, in submission order; streams
    // 1 .. NC: the carries, loop tau's on stream 1 + tau % NC
    const int NC = std::min(T, PIPE_STREAMS - 1), NS = NC + 1;
    hipStream_t ps = r->st[0];
    if ((e = hipEventRecord(r->fork, s)) != hipSuccess) return hip_fail(e, "pipeline fork");
    for (int i = 0; i < NS; ++i)
        if ((e = hipStreamWaitEvent(r->st[i], r->fork, 0)) != hipSuccess) return hip_fail(e, "pipeline fork");

    const size_t ab = 2;   // bf16 activations
    char *q = at(ws, lo.q), *k = at(ws, lo.k), *v = at(ws, lo.v);
    float *al = (float *)at(ws, lo.alpha), *be = (float *)at(ws, lo.beta);
    float *zp = (float *)at(ws, lo.zp), *stb = (float *)at(ws, lo.st);
    bf16 *xbuf = (bf16 *)at(ws, lo.x);
    const int npc = (int)pieces.size();
    gdn_status st = GDN_OK;
    for (int w = 0; w < npc + T - 1 && st == GDN_OK; ++w) {
        for (int tau = 0; tau < T && st == GDN_OK; ++tau) {
            const int j = w - tau;
            if (j < 0 || j >= npc) continue;
            const Piece &p = pieces[j];
            hipStream_t cs = r->st[1 + tau % NC];
            const bool last = tau == T - 1;
            const int64_t tok0 = (int64_t)p.b * L + p.t0;   // first row of the piece
            if (tau > 0 && (e = hipStreamWaitEvent(ps, r->ev[2 * (tau - 1) + j % 2], 0)) != hipSuccess) {
                st = hip_fail(e, "pipeline wait");
                break;
            }
            float *hdst = (h_loops ? h_loops + tau * tokd : h_out) + tok0 * d;
            const void *x = tau == 0 ? (const void *)((const char *)h0 + tok0 * d * ab) : (const void *)(xbuf + tok0 * d);
            const void *hprev = tau == 0 ? (const void *)((const char *)h0 + tok0 * d * ab)
                                         : (const void *)((h_loops ? h_loops + (tau - 1) * tokd : h_out) + tok0 * d);
            const int64_t qo = tok0 * H * D * ab;
            float *zpp = zp + (int64_t)lo.P * 2 * H * tok0;   // the piece's partials [P][2H][len]
            e = project(false, p.len, d, H, D, x, Wpack, q + qo, k + qo, v + qo, al + tok0 * H, be + tok0 * H,
                        desc->alpha_lo, desc->norm_eps, zpp, ps);
            if (e != hipSuccess) {
                st = hip_fail(e, "projection launch");
                break;
            }
            gdn_desc pd = *desc;
            pd.B = 1;
            pd.L = p.len;
            Layout pl = lo;   // the piece's chunk matrices follow those of the pieces before it
            pl.W = lo.W + (size_t)p.cu * D * CHUNK * 4;
            pl.M = lo.M + (size_t)p.cu * CHUNK * CHUNK * 4;
            pl.g = lo.g + (size_t)p.cu * CHUNK * 4;
            float *sbuf = stb + ((int64_t)tau * B + p.b) * seq_state;
            const float *s_init = p.first ? nullptr : sbuf;
            float *s_final = p.last ? (states_out ? states_out + tau * state_elems + p.b * seq_state : nullptr) : sbuf;
            CarryOut out{nullptr, hprev, tau == 0, rho + (int64_t)tau * d, hdst, last ? nullptr : xbuf + tok0 * d,
                         nullptr, nullptr};
            st = scan_chunks(&pd, q + qo, k + qo, v + qo,
                             GateSrc{al + tok0 * H, be + tok0 * H, zpp, lo.P, desc->alpha_lo, al + tok0 * H,
                                     be + tok0 * H},
                             s_init, s_final, out, ws, pl, ps, nullptr, cs, r->evp[2 * tau + j % 2]);
            if (st != GDN_OK) break;
            if (!last && (e = hipEventRecord(r->ev[2 * tau + j % 2], cs)) != hipSuccess) st = hip_fail(e, "pipeline event");
        }
    }
    // join (also after a failed launch, so that the caller's stream never runs ahead of work already queued)
    for (int i = 0; i < NS; ++i) {
        if ((e = hipEventRecord(r->done[i], r->st[i])) != hipSuccess) return st != GDN_OK ? st : hip_fail(e, "pipeline join");
        if ((e = hipStreamWaitEvent(s, r->done[i], 0)) != hipSuccess) return st != GDN_OK ? st : hip_fail(e, "pipeline join");
    }
    if (st != GDN_OK) return st;
    if (h_loops) {
        e = hipMemcpyAsync(h_out, h_loops + (T - 1) * tokd, tokd * sizeof(float), hipMemcpyDeviceToDevice, s);
        if (e != hipSuccess) return hip_fail(e, "copy of h^(T)");
    }
    return GDN_OK;
}

gdn_status gdn_loop_prefill(const gdn_desc *desc, const void *h0, const void *Wpack,
                            const float *rho, float *h_out, float *states_out, float *h_loops,
                            void *ws, size_t ws_bytes, void *stream) {
    gdn_status st = check_desc(desc, false);
    if (st != GDN_OK) return st;
    if ((st = check_prefill_grid(desc)) != GDN_OK) return st;
    REQUIRE_PTR(h0); REQUIRE_PTR(Wpack); REQUIRE_PTR(rho); REQUIRE_PTR(h_out);
    OPTIONAL_PTR(states_out); OPTIONAL_PTR(h_loops);
    if ((const void *)h_out == h0) return fail(GDN_ERR_SHAPE, "h_out may not alias h0");
    const Layout lo = layout(desc, GDN_OP_LOOP_PREFILL);
    if (!ws || ws_bytes < lo.total)
        return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", lo.total, ws_bytes);
    if (!aligned16(ws)) return fail(GDN_ERR_ALIGN, "ws is not 16-byte aligned");
    const int piece = pipe_piece_tokens(desc, lo);
    if (piece > 0)
        return loop_prefill_pipelined(desc, h0, Wpack, rho, h_out, states_out, h_loops, ws, lo, (hipStream_t)stream,
                                      piece);
    return loop_prefill_impl(desc, h0, Wpack, rho, h_out, states_out, h_loops, ws, lo, (hipStream_t)stream, nullptr);
}

gdn_status gdn_loop_prefill_set_pieces(int tokens) {
    if (tokens < -1) return fail(GDN_ERR_SHAPE, "tokens per piece must be -1, 0 or positive (got %d)", tokens);
    g_pipe_piece.store(tokens, std::memory_order_relaxed);
    return GDN_OK;
}

gdn_status gdn_loop_prefill_pieces(const gdn_desc *desc, int *tokens) {
    gdn_status st = check_desc(desc, false);
    if (st != GDN_OK) return st;
    if ((st = check_prefill_grid(desc)) != GDN_OK) return st;
    if (!tokens) return fail(GDN_ERR_NULL, "tokens is NULL");
    *tokens = pipe_piece_tokens(desc, layout(desc, GDN_OP_LOOP_PREFILL));
    return GDN_OK;
}

gdn_status gdn_loop_prefill_act(const gdn_desc *desc, const void *h0, const void *Wpack, const float *rho,
                                const float *w_halt, float b_halt, float eps, float *h_out, int32_t *halt_loop,
                                float *ponder, void *ws, size_t ws_bytes, void *stream) {
    gdn_status st = check_desc(desc, false);
    if (st != GDN_OK) return st;
    if ((st = check_prefill_grid(desc)) != GDN_OK) return st;
    REQUIRE_PTR(h0); REQUIRE_PTR(Wpack); REQUIRE_PTR(rho); REQUIRE_PTR(w_halt); REQUIRE_PTR(h_out);
    OPTIONAL_PTR(halt_loop); OPTIONAL_PTR(ponder);
    if ((const void *)h_out == h0) return fail(GDN_ERR_SHAPE, "h_out may not alias h0");
    if (!(eps >= 0.f && eps < 1.f)) return fail(GDN_ERR_SHAPE, "eps must be in [0, 1) (got %g)", (double)eps);
    if (!std::isfinite(b_halt)) return fail(GDN_ERR_SHAPE, "b_halt must be finite");
    const Layout lo = layout(desc, GDN_OP_LOOP_PREFILL_ACT);
    if (!ws || ws_bytes < lo.total)
        return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", lo.total, ws_bytes);
    if (!aligned16(ws)) return fail(GDN_ERR_ALIGN, "ws is not 16-byte aligned");
    const ActArgs act{w_halt, b_halt, 1.0f - eps, (float *)at(ws, lo.R), (int *)at(ws, lo.halt),
                      (int *)at(ws, lo.rows), (int *)at(ws, lo.rows_count), halt_loop, ponder};
    return loop_prefill_impl(desc, h0, Wpack, rho, h_out, nullptr, nullptr, ws, lo, (hipStream_t)stream, &act);
}

gdn_status gdn_loop_decode(const gdn_desc *desc, const void *h_t, const void *Wpack,
                           const float *rho, float *states, float *h_out, void *ws,
                           size_t ws_bytes, void *stream) {
    gdn_status st = check_desc(desc, true);
    if (st != GDN_OK) return st;
    REQUIRE_PTR(h_t); REQUIRE_PTR(Wpack); REQUIRE_PTR(rho); REQUIRE_PTR(states); REQUIRE_PTR(h_out);
    if ((const void *)h_out == h_t) return fail(GDN_ERR_SHAPE, "h_out may not alias h_t");
    const Layout lo = layout(desc, GDN_OP_LOOP_DECODE);
    // the projection's partials are the last region: a workspace that holds
    // everything before them runs the step with the projection unsplit
    const bool split = lo.dpart && ws && ws_bytes >= lo.total;
    const size_t need = lo.dpart ? lo.dpart : lo.total;
    if (!ws || ws_bytes < need)
        return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
    if (!aligned16(ws)) return fail(GDN_ERR_ALIGN, "ws is not 16-byte aligned");

    const hipStream_t s = (hipStream_t)stream;
    const bool f32 = desc->act == GDN_F32;
    const int N = desc->B, D = desc->dk, d = desc->d;
    void *q = at(ws, lo.q), *k = at(ws, lo.k), *v = at(ws, lo.v);
    float *al = (float *)at(ws, lo.alpha), *be = (float *)at(ws, lo.beta);
    bf16 *xbuf = f32 ? nullptr : (bf16 *)at(ws, lo.x);
    const int64_t state_elems = (int64_t)N * desc->H * D * D;
    const void *x = h_t, *hprev = h_t;
    bool hprev_bf16 = !f32;
    for (int tau = 0; tau < desc->T; ++tau) {
        const bool last = tau == desc->T - 1;
        // at most 64 bf16 tokens: the projection split over the channels into
        // partial products, which the decode step itself sums and normalises
        // (not stage-timed: a stage timer times single launches)
        float *part = split ? (float *)at(ws, lo.dpart) : nullptr;
        hipError_t e = part ? launch_project_decode_parts(N, d, desc->H, D, x, Wpack, part, s)
                            : project(f32, N, d, desc->H, D, x, Wpack, q, k, v, al, be, desc->alpha_lo,
                                      desc->norm_eps, nullptr, s);
        if (e != hipSuccess) return hip_fail(e, "projection launch");
        e = timed(GDN_STAGE_DECODE, s, [&] {
            return launch_decode(f32, N, desc->H, D, q, k, v, al, be, states + tau * state_elems,
                                 nullptr, hprev, hprev_bf16, rho + (int64_t)tau * d, h_out,
                                 (!f32 && !last) ? xbuf : nullptr, s, part, part ? decode_k_splits(f32, N, d) : 0,
                                 desc->alpha_lo, desc->norm_eps);
        });
        if (e != hipSuccess) return hip_fail(e, "decode launch");
        hprev = h_out;
        hprev_bf16 = false;
        x = f32 ? (const void *)h_out : (const void *)xbuf;
    }
    return GDN_OK;
}

// ---- timers -------------------------------------------------------------------
gdn_status gdn_timer_create(int stage, int capacity, gdn_timer **out) {
    if (!out) return fail(GDN_ERR_NULL, "out is NULL");
    if (stage < GDN_STAGE_PROJECT || stage > GDN_STAGE_BLOCK_GEMM || stage == 4 || stage == 8 || capacity < 1 ||
        capacity > (1 << 20))
        return fail(GDN_ERR_SHAPE, "bad timer stage %d or capacity %d", stage, capacity);
    gdn_timer *t = new gdn_timer;
    t->stage = stage;
    t->capacity = capacity;
    t->start.resize(capacity);
    t->stop.resize(capacity);
    for (int i = 0; i < capacity; ++i) {
        hipError_t e = hipEventCreate(&t->start[i]);
        if (e == hipSuccess) e = hipEventCreate(&t->stop[i]);
        if (e != hipSuccess) {
            for (int j = 0; j <= i; ++j) {
                if (t->start[j]) (void)hipEventDestroy(t->start[j]);
                if (j < i && t->stop[j]) (void)hipEventDestroy(t->stop[j]);
            }
            delete t;
            return hip_fail(e, "hipEventCreate");
        }
    }
    *out = t;
    return GDN_OK;
}

gdn_status gdn_timer_attach(gdn_timer *t) {
    if (!t) return fail(GDN_ERR_NULL, "timer is NULL");
    g_timers[t->stage] = t;
    return GDN_OK;
}

gdn_status gdn_timer_detach(void) {
    for (auto &t : g_timers) t = nullptr;
    return GDN_OK;
}

gdn_status gdn_timer_set_stride(gdn_timer *t, int stride) {
    if (!t) return fail(GDN_ERR_NULL, "timer is NULL");
    if (stride < 1) return fail(GDN_ERR_SHAPE, "timer stride must be >= 1 (got %d)", stride);
    t->stride = stride;
    t->seen = 0;
    return GDN_OK;
}

gdn_status gdn_timer_reset(gdn_timer *t) {
    if (!t) return fail(GDN_ERR_NULL, "timer is NULL");
    t->used = 0;
    t->seen = 0;
    return GDN_OK;
}

gdn_status gdn_timer_read(gdn_timer *t, int *launches, double *total_ms) {
    if (!t || !launches || !total_ms) return fail(GDN_ERR_NULL, "NULL argument");
    double sum = 0.0;
    for (int i = 0; i < t->used; ++i) {
        hipError_t e = hipEventSynchronize(t->stop[i]);
        if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
        float ms = 0.f;
        e = hipEventElapsedTime(&ms, t->start[i], t->stop[i]);
        if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
        sum += ms;
    }
    *launches = t->used;
    *total_ms = sum;
    return GDN_OK;
}

gdn_status gdn_timer_destroy(gdn_timer *t) {
    if (!t) return GDN_OK;
    if (g_timers[t->stage] == t) g_timers[t->stage] = nullptr;
    for (int i = 0; i < t->capacity; ++i) {
        (void)hipEventDestroy(t->start[i]);
        (void)hipEventDestroy(t->stop[i]);
    }
    delete t;
    return GDN_OK;
}

}  // extern "C"
