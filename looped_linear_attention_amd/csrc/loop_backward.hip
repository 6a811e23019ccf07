// loop_backward.hip -- the token-local steps of the backward through the T
// loops on gfx950: the bf16 loop operand, the gradient of the projection's
// epilogue from the raw projections, the residual gate's rho gradient, and
// the weight gradients handed back in the layout of the unpacked weights.
//
// LT2: Linear-Time Looped Transformers, Section 2 ("Looped Transformer (LT)":
// weight tying; "LT2": the per-loop residual gate h^(tau) = o + rho_tau (.)
// h^(tau-1)); Appendix C: the looped stack is trained with bf16 mixed
// precision.  Forward epilogue per (token, head): q = qr / r_q, k = kr / r_k,
// r = sqrt(|raw|^2 + eps); alpha = alpha_lo + (1 - alpha_lo) s,
// s = 1 / (1 + e^a); beta = 1 / (1 + e^-b).  Its gradient:
//     dqr = (dq - q (q . dq)) / r_q   (likewise k),   dvr = dv,
//     da = -dalpha (1 - alpha_lo) s (1 - s),          db = dbeta beta (1 - beta).
// The bf16 roundings of the forward pass the gradient through unchanged.
#include "gdn_device.h"
#include "gdn_kernels.h"

namespace gdn {

namespace {

// x = bf16(h), round to nearest even (the forward's carry writes the same copy).
__global__ __launch_bounds__(256) void k_lb_round(const float *__restrict__ h, bf16 *__restrict__ x, int64_t n) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i + 3 < n) {
        const float4 v = *reinterpret_cast<const float4 *>(h + i);
        const bf16 r[4] = {(bf16)v.x, (bf16)v.y, (bf16)v.z, (bf16)v.w};
        *reinterpret_cast<bf16x4 *>(x + i) = pack4(r);
    } else {
        for (int64_t j = i; j < n; ++j) x[j] = (bf16)h[j];
    }
}

// The gradient of the epilogue, one wave per (token, head), written over the
// raw projections Y [M][P] in place (packed order: head j's q|k|v at columns
// 3 D j .., the gates at qkvp + j and qkvp + H + j); each lane reads its own
// elements of Y before it writes them.  With zp the raw gate pre-activations
// are the sums of the projection's nzp partials zp[p][2H][M] in the order
// p = 0, 1, ... (as the chunk preparation forms them) rather than Y's gate
// columns.  The padding columns of dY (between the q|k|v columns and qkvp,
// and after the 2H gate columns) are set to zero.
template <int D>
__global__ __launch_bounds__(256) void k_lb_epilogue_grad(float *Y, int64_t P, int64_t qkvp, int M, int H, float eps,
                                                          float alpha_lo, const float *__restrict__ dq,
                                                          const float *__restrict__ dk, const float *__restrict__ dv,
                                                          const float *__restrict__ dalpha,
                                                          const float *__restrict__ dbeta,
                                                          const float *__restrict__ zp, int nzp) {
    constexpr int E = D / 64;
    const int lane = threadIdx.x & 63;
    const int64_t u = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (u >= (int64_t)M * H) return;
    const int64_t m = u / H;
    const int j = (int)(u % H);
    float *y = Y + m * P + (int64_t)j * 3 * D;
    const int64_t o = u * D;
    float qv[E], kv[E], gq[E], gk[E], sq = 0.f, sk = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        qv[e] = y[lane + 64 * e];
        kv[e] = y[D + lane + 64 * e];
        gq[e] = dq[o + lane + 64 * e];
        gk[e] = dk[o + lane + 64 * e];
        sq = fmaf(qv[e], qv[e], sq);
        sk = fmaf(kv[e], kv[e], sk);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        sq += __shfl_xor(sq, off, 64);
        sk += __shfl_xor(sk, off, 64);
    }
    const float iq = 1.f / sqrtf(sq + eps), ik = 1.f / sqrtf(sk + eps);
    float pq = 0.f, pk = 0.f;   // q . dq, k . dk with the normalised q, k
#pragma unroll
    for (int e = 0; e < E; ++e) {
        qv[e] *= iq;
        kv[e] *= ik;
        pq = fmaf(qv[e], gq[e], pq);
        pk = fmaf(kv[e], gk[e], pk);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        pq += __shfl_xor(pq, off, 64);
        pk += __shfl_xor(pk, off, 64);
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
        y[lane + 64 * e] = (gq[e] - qv[e] * pq) * iq;
        y[D + lane + 64 * e] = (gk[e] - kv[e] * pk) * ik;
        y[2 * D + lane + 64 * e] = dv[o + lane + 64 * e];
    }
    if (lane == 0) {
        float *ya = Y + m * P + qkvp + j, *yb = Y + m * P + qkvp + H + j;
        float za = 0.f, zb = 0.f;
        if (zp) {
            for (int p = 0; p < nzp; ++p) {
                za += zp[((int64_t)p * 2 * H + j) * M + m];
                zb += zp[((int64_t)p * 2 * H + H + j) * M + m];
            }
        } else {
            za = *ya;
            zb = *yb;
        }
        const float s = 1.f / (1.f + expf(za)), be = 1.f / (1.f + expf(-zb));
        *ya = -dalpha[u] * (1.f - alpha_lo) * s * (1.f - s);
        *yb = dbeta[u] * be * (1.f - be);
    }
    const int64_t qkv = (int64_t)H * 3 * D, pad1 = qkvp - qkv, pad2 = P - qkvp - 2 * H;
    for (int64_t i = (int64_t)j * 64 + lane; i < pad1 + pad2; i += (int64_t)H * 64)
        Y[m * P + (i < pad1 ? qkv + i : qkvp + 2 * H + (i - pad1))] = 0.f;
}

// drho partials: part[rb][c] = sum over rows r of block rb (DR_ROWS rows, in
// order) of dh[r][c] hp[r][c]; then drho[c] = sum over rb in order.  A thread
// takes 4 adjacent columns (16-byte loads of dh) and issues the loads of 8
// rows before it adds them up.
constexpr int DR_ROWS = 32;
template <typename TH> struct Quad;
template <> struct Quad<float> {
    __device__ static float4 load(const float *p) { return *reinterpret_cast<const float4 *>(p); }
};
template <> struct Quad<bf16> {
    __device__ static float4 load(const bf16 *p) {
        const bf16x4 v = *reinterpret_cast<const bf16x4 *>(p);
        return float4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
    }
};
template <typename TH>
__global__ __launch_bounds__(256) void k_lb_drho_part(const float *__restrict__ dh, const TH *__restrict__ hp, int M,
                                                      int d, float *__restrict__ part) {
    const int c = (blockIdx.x * 256 + threadIdx.x) * 4, rb = blockIdx.y;
    if (c >= d) return;
    const int r0 = rb * DR_ROWS, r1 = min(M, r0 + DR_ROWS);
    float4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int r = r0; r < r1; r += 8) {
        float4 a[8], b[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int64_t o = (int64_t)min(r + u, r1 - 1) * d + c;
            a[u] = *reinterpret_cast<const float4 *>(dh + o);
            b[u] = Quad<TH>::load(hp + o);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (r + u < r1) {
                acc.x = fmaf(a[u].x, b[u].x, acc.x);
                acc.y = fmaf(a[u].y, b[u].y, acc.y);
                acc.z = fmaf(a[u].z, b[u].z, acc.z);
                acc.w = fmaf(a[u].w, b[u].w, acc.w);
            }
        }
    }
    *reinterpret_cast<float4 *>(part + (int64_t)rb * d + c) = acc;
}
// 64 columns per workgroup: wave g sums the partials of row blocks
// [g nrb / 4, (g + 1) nrb / 4) in order, then the four sums are added in the
// order g = 0..3.
__global__ __launch_bounds__(256) void k_lb_drho_sum(const float *__restrict__ part, int nrb, int d,
                                                     float *__restrict__ drho) {
    __shared__ float s4[4][64];
    const int lane = threadIdx.x & 63, g = threadIdx.x >> 6;
    const int c = blockIdx.x * 64 + lane;
    float acc = 0.f;
    if (c < d)
        for (int rb = nrb * g / 4; rb < nrb * (g + 1) / 4; ++rb) acc += part[(int64_t)rb * d + c];
    s4[g][lane] = acc;
    __syncthreads();
    if (g == 0 && c < d) drho[c] = ((s4[0][lane] + s4[1][lane]) + s4[2][lane]) + s4[3][lane];
}

// dWT [d][P] (the weight gradient in the orientation x^T dY) to the unpacked
// layouts: dWq[c][j D + i] = dWT[c][3 D j + i], dWk at + D, dWv at + 2 D,
// dwa[c][j] = dWT[c][qkvp + j], dwb[c][j] = dWT[c][qkvp + H + j].
template <int D>
__global__ __launch_bounds__(256) void k_lb_unpack(const float *__restrict__ dWT, int nparts, int64_t pstride,
                                                   int64_t P, int64_t qkvp, int d, int H,
                                                   float *__restrict__ dWq, float *__restrict__ dWk,
                                                   float *__restrict__ dWv, float *__restrict__ dwa,
                                                   float *__restrict__ dwb) {
    const int64_t HD = (int64_t)H * D;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t per_row = 3 * HD + 2 * H;
    if (idx >= (int64_t)d * per_row) return;
    const int64_t c = idx / per_row, w = idx % per_row;
    const float *row = dWT + c * P;
    auto get = [&](int64_t col) {   // the k-range partial sums, in order
        float acc = row[col];
        for (int z = 1; z < nparts; ++z) acc += row[(int64_t)z * pstride + col];
        return acc;
    };
    if (w < 3 * HD) {
        const int64_t kind = w / HD, col = w % HD, j = col / D, i = col % D;
        float *dst = kind == 0 ? dWq : (kind == 1 ? dWk : dWv);
        dst[c * HD + col] = get(3 * D * j + kind * D + i);
    } else if (w < 3 * HD + H) {
        const int64_t j = w - 3 * HD;
        dwa[c * H + j] = get(qkvp + j);
    } else {
        const int64_t j = w - 3 * HD - H;
        dwb[c * H + j] = get(qkvp + H + j);
    }
}

__global__ __launch_bounds__(256) void k_sum_parts(int64_t n, int d, const float *__restrict__ parts, int nparts,
                                                   int64_t pstride, const float *__restrict__ rho,
                                                   const float *__restrict__ add, float *__restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    float acc = parts[i];
    for (int z = 1; z < nparts; ++z) acc += parts[(int64_t)z * pstride + i];
    if (rho) acc = fmaf(rho[i % d], add[i], acc);
    out[i] = acc;
}

__global__ __launch_bounds__(256) void k_fill_zero(float *p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0.f;
}

}  // namespace

hipError_t launch_lb_round(int64_t n, const float *h, bf16 *x, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const int64_t groups = (n + 3) / 4;
    launch_kernel(k_lb_round, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, s, h, x, n);
    return hipGetLastError();
}

hipError_t launch_lb_epilogue_grad(int M, int H, int D, float *Y, int64_t P, int64_t qkvp, float eps, float alpha_lo,
                                   const float *dq, const float *dk, const float *dv, const float *dalpha,
                                   const float *dbeta, const float *zp, int nzp, hipStream_t s) {
    const int64_t units = (int64_t)M * H;
    const dim3 grid((unsigned)((units + 3) / 4));
    if (D == 128)
        launch_kernel(k_lb_epilogue_grad<128>, grid, dim3(256), 0, s, Y, P, qkvp, M, H, eps, alpha_lo, dq, dk, dv,
                      dalpha, dbeta, zp, nzp);
    else if (D == 64)
        launch_kernel(k_lb_epilogue_grad<64>, grid, dim3(256), 0, s, Y, P, qkvp, M, H, eps, alpha_lo, dq, dk, dv,
                      dalpha, dbeta, zp, nzp);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

int lb_drho_blocks(int M) { return (M + DR_ROWS - 1) / DR_ROWS; }

hipError_t launch_lb_drho(int M, int d, const float *dh, const void *hp, bool hp_f32, float *part, float *drho,
                          hipStream_t s) {
    const int nrb = lb_drho_blocks(M);
    if (nrb > 65535 || d % 4) return hipErrorInvalidValue;
    const dim3 g1((d / 4 + 255) / 256, nrb);
    if (hp_f32) launch_kernel(k_lb_drho_part<float>, g1, dim3(256), 0, s, dh, (const float *)hp, M, d, part);
    else launch_kernel(k_lb_drho_part<bf16>, g1, dim3(256), 0, s, dh, (const bf16 *)hp, M, d, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    launch_kernel(k_lb_drho_sum, dim3((d + 63) / 64), dim3(256), 0, s, (const float *)part, nrb, d, drho);
    return hipGetLastError();
}

hipError_t launch_lb_unpack(int d, int H, int D, const float *dWT, int nparts, int64_t pstride, int64_t P,
                            int64_t qkvp, float *dWq, float *dWk, float *dWv, float *dwa, float *dwb, hipStream_t s) {
    const int64_t n = (int64_t)d * (3LL * H * D + 2 * H);
    const dim3 grid((unsigned)((n + 255) / 256));
    if (nparts < 1) return hipErrorInvalidValue;
    if (D == 128)
        launch_kernel(k_lb_unpack<128>, grid, dim3(256), 0, s, dWT, nparts, pstride, P, qkvp, d, H, dWq, dWk, dWv,
                      dwa, dwb);
    else if (D == 64)
        launch_kernel(k_lb_unpack<64>, grid, dim3(256), 0, s, dWT, nparts, pstride, P, qkvp, d, H, dWq, dWk, dWv,
                      dwa, dwb);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_sum_parts(int64_t rows, int d, const float *parts, int nparts, int64_t pstride, const float *rho,
                            const float *add, float *out, hipStream_t s) {
    const int64_t n = rows * d;
    if (n <= 0) return hipSuccess;
    launch_kernel(k_sum_parts, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, n, d, parts, nparts, pstride, rho,
                  add, out);
    return hipGetLastError();
}

hipError_t launch_fill_zero(float *p, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    launch_kernel(k_fill_zero, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

}  // namespace gdn
