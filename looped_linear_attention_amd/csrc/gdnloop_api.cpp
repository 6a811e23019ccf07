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

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
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

// ---- workspace layout ------------------------------------------------------
struct Layout {
    size_t q = 0, k = 0, v = 0, alpha = 0, beta = 0, zp = 0, W = 0, M = 0, g = 0, x = 0, total = 0;
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
    const bool proj = op == GDN_OP_LOOP_PREFILL || op == GDN_OP_LOOP_DECODE;
    const bool chunks = op == GDN_OP_LOOP_PREFILL || op == GDN_OP_SCAN_PREFILL;
    if (proj) {
        lo.q = take(tokens * d->H * D * act_bytes(d));
        lo.k = take(tokens * d->H * D * act_bytes(d));
        lo.v = take(tokens * d->H * D * act_bytes(d));
        lo.alpha = take(tokens * d->H * 4);
        lo.beta = take(tokens * d->H * 4);
        if (d->act == GDN_BF16 && d->T > 1) lo.x = take(tokens * d->d * 2);
        if (op == GDN_OP_LOOP_PREFILL) {
            lo.P = gate_partials(d->act == GDN_F32, (int)tokens, d->d, d->H);
            if (lo.P) lo.zp = take((size_t)lo.P * 2 * d->H * tokens * 4);
        }
    }
    if (chunks) {
        lo.W = take(bh * Nc * D * CHUNK * 4);
        lo.M = take(bh * Nc * CHUNK * CHUNK * 4);
        lo.g = take(bh * Nc * CHUNK * 4);
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

constexpr int N_STAGES = GDN_STAGE_GATES + 1;
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
                   void *v, float *al, float *be, float alpha_lo, float eps, float *zp, hipStream_t s) {
    hipError_t e = timed(GDN_STAGE_PROJECT, s, [&] {
        return launch_project(f32, M, d, H, D, x, Wpack, q, k, v, al, be, alpha_lo, eps, zp, s);
    });
    if (e == hipSuccess && !zp && project_separate_gates(f32, M))
        e = timed(GDN_STAGE_GATES, s, [&] { return launch_gates(M, d, H, D, x, Wpack, al, be, alpha_lo, s); });
    return e;
}

}  // namespace

LaunchEvents &gdn::launch_events() { return t_launch_events; }

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
    if (op < GDN_OP_LOOP_PREFILL || op > GDN_OP_PROJECT)
        return fail(GDN_ERR_UNSUPPORTED, "unknown op %d", op);
    gdn_status st = check_desc(desc, op == GDN_OP_LOOP_DECODE || op == GDN_OP_SCAN_DECODE);
    if (st != GDN_OK) return st;
    if (!bytes) return fail(GDN_ERR_NULL, "bytes is NULL");
    *bytes = layout(desc, op).total;
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

static gdn_status scan_chunks(const gdn_desc *d, const void *q, const void *k, const void *v,
                              GateSrc gates, const float *s_init, float *s_final, CarryOut out, void *ws,
                              const Layout &lo, hipStream_t s) {
    const bool f32 = d->act == GDN_F32;
    ChunkWs cw{(float *)at(ws, lo.W), (float *)at(ws, lo.M), (float *)at(ws, lo.g)};
    hipError_t e = timed(GDN_STAGE_SCAN_PREP, s, [&] {
        return launch_scan_prep(f32, d->B, d->L, d->H, d->dk, q, k, gates, cw, s);
    });
    if (e != hipSuccess) return hip_fail(e, "chunk prep launch");
    e = timed(GDN_STAGE_SCAN_CARRY, s, [&] {
        return launch_scan_carry(f32, d->B, d->L, d->H, d->dk, q, k, v, cw, s_init, s_final, out, s);
    });
    if (e != hipSuccess) return hip_fail(e, "carry launch");
    return GDN_OK;
}

gdn_status gdn_scan_prefill(const gdn_desc *desc, const void *q, const void *k, const void *v,
                            const float *alpha, const float *beta, const float *s_init, float *o,
                            float *s_final, void *ws, size_t ws_bytes, void *stream) {
    gdn_status st = check_desc(desc, false);
    if (st != GDN_OK) return st;
    REQUIRE_PTR(q); REQUIRE_PTR(k); REQUIRE_PTR(v); REQUIRE_PTR(alpha); REQUIRE_PTR(beta);
    REQUIRE_PTR(o); OPTIONAL_PTR(s_init); OPTIONAL_PTR(s_final);
    if (s_init && s_init == s_final) return fail(GDN_ERR_SHAPE, "s_final may not alias s_init");
    const Layout lo = layout(desc, GDN_OP_SCAN_PREFILL);
    if (!ws || ws_bytes < lo.total)
        return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", lo.total, ws_bytes);
    if (!aligned16(ws)) return fail(GDN_ERR_ALIGN, "ws is not 16-byte aligned");
    CarryOut out{o, nullptr, false, nullptr, nullptr, nullptr};
    return scan_chunks(desc, q, k, v, GateSrc{alpha, beta, nullptr, 0, desc->alpha_lo}, s_init, s_final, out,
                       ws, lo, (hipStream_t)stream);
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

gdn_status gdn_loop_prefill(const gdn_desc *desc, const void *h0, const void *Wpack,
                            const float *rho, float *h_out, float *states_out, float *h_loops,
                            void *ws, size_t ws_bytes, void *stream) {
    gdn_status st = check_desc(desc, false);
    if (st != GDN_OK) return st;
    REQUIRE_PTR(h0); REQUIRE_PTR(Wpack); REQUIRE_PTR(rho); REQUIRE_PTR(h_out);
    OPTIONAL_PTR(states_out); OPTIONAL_PTR(h_loops);
    if ((const void *)h_out == h0) return fail(GDN_ERR_SHAPE, "h_out may not alias h0");
    const Layout lo = layout(desc, GDN_OP_LOOP_PREFILL);
    if (!ws || ws_bytes < lo.total)
        return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", lo.total, ws_bytes);
    if (!aligned16(ws)) return fail(GDN_ERR_ALIGN, "ws is not 16-byte aligned");

    const hipStream_t s = (hipStream_t)stream;
    const bool f32 = desc->act == GDN_F32;
    const int M = desc->B * desc->L, D = desc->dk, d = desc->d;
    const int64_t tokd = (int64_t)M * d;
    void *q = at(ws, lo.q), *k = at(ws, lo.k), *v = at(ws, lo.v);
    float *al = (float *)at(ws, lo.alpha), *be = (float *)at(ws, lo.beta);
    float *zp = lo.P ? (float *)at(ws, lo.zp) : nullptr;   // gate partials, when the GEMM makes them
    bf16 *xbuf = f32 ? nullptr : (bf16 *)at(ws, lo.x);
    const int64_t state_elems = (int64_t)desc->B * desc->H * D * D;

    const void *x = h0;            // GEMM operand of loop tau
    const void *hprev = h0;        // h^(tau-1) for the residual
    bool hprev_bf16 = !f32;
    for (int tau = 0; tau < desc->T; ++tau) {
        const bool last = tau == desc->T - 1;
        float *hdst = h_loops ? h_loops + tau * tokd : h_out;  // h^(tau+1), in place over h_out
        hipError_t e = project(f32, M, d, desc->H, D, x, Wpack, q, k, v, al, be, desc->alpha_lo,
                               desc->norm_eps, zp, s);
        if (e != hipSuccess) return hip_fail(e, "projection launch");
        CarryOut out{nullptr, hprev, hprev_bf16, rho + (int64_t)tau * d, hdst,
                     (!f32 && !last) ? xbuf : nullptr};
        st = scan_chunks(desc, q, k, v, GateSrc{al, be, zp, lo.P, desc->alpha_lo}, nullptr,
                         states_out ? states_out + tau * state_elems : nullptr, out, ws, lo, s);
        if (st != GDN_OK) return st;
        hprev = hdst;
        hprev_bf16 = false;
        x = f32 ? (const void *)hdst : (const void *)xbuf;
    }
    if (h_loops) {
        hipError_t e = hipMemcpyAsync(h_out, h_loops + (desc->T - 1) * tokd, tokd * sizeof(float),
                                      hipMemcpyDeviceToDevice, s);
        if (e != hipSuccess) return hip_fail(e, "copy of h^(T)");
    }
    return GDN_OK;
}

gdn_status gdn_loop_decode(const gdn_desc *desc, const void *h_t, const void *Wpack,
                           const float *rho, float *states, float *h_out, void *ws,
                           size_t ws_bytes, void *stream) {
    gdn_status st = check_desc(desc, true);
    if (st != GDN_OK) return st;
    REQUIRE_PTR(h_t); REQUIRE_PTR(Wpack); REQUIRE_PTR(rho); REQUIRE_PTR(states); REQUIRE_PTR(h_out);
    if ((const void *)h_out == h_t) return fail(GDN_ERR_SHAPE, "h_out may not alias h_t");
    const Layout lo = layout(desc, GDN_OP_LOOP_DECODE);
    if (!ws || ws_bytes < lo.total)
        return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", lo.total, ws_bytes);
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
        hipError_t e = project(f32, N, d, desc->H, D, x, Wpack, q, k, v, al, be, desc->alpha_lo,
                               desc->norm_eps, nullptr, s);
        if (e != hipSuccess) return hip_fail(e, "projection launch");
        e = timed(GDN_STAGE_DECODE, s, [&] {
            return launch_decode(f32, N, desc->H, D, q, k, v, al, be, states + tau * state_elems,
                                 nullptr, hprev, hprev_bf16, rho + (int64_t)tau * d, h_out,
                                 (!f32 && !last) ? xbuf : nullptr, s);
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
    if (stage < GDN_STAGE_PROJECT || stage > GDN_STAGE_GATES || capacity < 1 || capacity > (1 << 20))
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
