// decode.hip -- one recurrent token of the gated delta rule per sequence, gfx950.
//
// LT2: Linear-Time Looped Transformers, related-work paragraph on linear
// attention: inference is a recurrent state update at constant cost per step.
// Per (sequence n, head h), with the state S [dk x dv] read once and written once:
//     a = S^T k,   b = S^T q                    (one pass over S)
//     u = beta (v - alpha a)
//     o = S'^T q = alpha b + (k.q) u            (S' the updated state)
//     S' = alpha S + k u^T
// which is S' = alpha (I - beta k k^T) S + beta k v^T, o = S'^T q.
// The kernel is HBM-bound: one workgroup per (n, h) streams the state with
// 16-byte accesses (each wave touches whole 512-byte rows).
#include "gdn_device.h"
#include "gdn_kernels.h"

namespace gdn {

namespace {

// Projection partials (the loop decode's channel-split projection, S > 0):
// instead of reading q, k, v, alpha, beta, workgroup (n, h) adds its head's S
// partial products part[s][n][NP] in the order s = 0 .. S-1, normalises q and k
// (x / sqrt(sum x^2 + eps)), rounds q, k, v to bf16, forms the gates from their
// pre-activations, stores all five to q_out .. beta_out (where the loop decode
// documents them) and continues with those values.
struct DecParts {
    const float *part;   // [S][N][NP] or nullptr
    int S, NP, gate_row; // gate_row: first packed row of the gate tile (wa rows, then wb rows)
    float alpha_lo, eps;
    bf16 *q_out, *k_out, *v_out;     // [N, H, D]
    float *alpha_out, *beta_out;     // [N, H]
};

template <int D, typename TIn, bool PARTS>
__global__ __launch_bounds__(256) void k_decode(const TIn *__restrict__ q, const TIn *__restrict__ k,
                                                const TIn *__restrict__ v,
                                                const float *__restrict__ alpha,
                                                const float *__restrict__ beta, float *states,
                                                float *__restrict__ o, const void *h_prev,
                                                int h_prev_bf16, const float *__restrict__ rho,
                                                float *h_out, bf16 *x_next,
                                                int H, DecParts dp) {
    constexpr int CG = D / 4;       // float4 column groups
    constexpr int RG = 256 / CG;    // row groups
    constexpr int RPT = D / RG;     // rows per thread
    __shared__ float ks[D], qs[D], vs[D];
    __shared__ __attribute__((aligned(16))) float4 pa[RG][CG], pb[RG][CG];
    __shared__ float kq_s;
    __shared__ float nred[2][4], gate_s[2];

    const int t = threadIdx.x;
    const int nh = blockIdx.x;  // n * H + h
    const int h = nh % H;
    const int64_t vec = (int64_t)nh * D;
    const int cg = t % CG, rg = t / CG;
    float4 *S = reinterpret_cast<float4 *>(states + (int64_t)nh * D * D);
    float4 sr[RPT];
#pragma unroll
    for (int ii = 0; ii < RPT; ++ii) sr[ii] = S[(rg + RG * ii) * CG + cg];
    float al, be;
    if constexpr (PARTS) {
        // threads 0 .. D-1: q, k, v of column t; thread D: the two gate pre-activations
        const int64_t n = nh / H;
        const float *pr = dp.part + n * dp.NP;
        const int64_t sstride = (int64_t)(gridDim.x / H) * dp.NP;
        float qv = 0.f, kv = 0.f, vv = 0.f;
        if (t < D) {
            const float *c = pr + (int64_t)h * 3 * D + t;
            float pq[8], pk[8], pv[8];
#pragma unroll
            for (int s = 0; s < 8; ++s)
                if (s < dp.S) {
                    pq[s] = c[s * sstride];
                    pk[s] = c[s * sstride + D];
                    pv[s] = c[s * sstride + 2 * D];
                }
            qv = pq[0], kv = pk[0], vv = pv[0];
#pragma unroll
            for (int s = 1; s < 8; ++s)
                if (s < dp.S) {
                    qv += pq[s];
                    kv += pk[s];
                    vv += pv[s];
                }
            // per-head sums of squares: in-wave, then across the D / 64 waves
            float sq = qv * qv, sk = kv * kv;
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) {
                sq += __shfl_xor(sq, off, 64);
                sk += __shfl_xor(sk, off, 64);
            }
            if ((t & 63) == 0) {
                nred[0][t >> 6] = sq;
                nred[1][t >> 6] = sk;
            }
        } else if (t == D) {
            float za = 0.f, zb = 0.f;
            for (int s = 0; s < dp.S; ++s) {
                za += pr[s * sstride + dp.gate_row + h];
                zb += pr[s * sstride + dp.gate_row + H + h];
            }
            gate_s[0] = dp.alpha_lo + (1.f - dp.alpha_lo) / (1.f + expf(za));
            gate_s[1] = 1.f / (1.f + expf(-zb));
        }
        __syncthreads();
        if (t < D) {
            float tq = 0.f, tk = 0.f;
#pragma unroll
            for (int w = 0; w < D / 64; ++w) {
                tq += nred[0][w];
                tk += nred[1][w];
            }
            const bf16 qb = (bf16)(qv * (1.f / sqrtf(tq + dp.eps))), kb = (bf16)(kv * (1.f / sqrtf(tk + dp.eps)));
            const bf16 vb = (bf16)vv;
            dp.q_out[vec + t] = qb;
            dp.k_out[vec + t] = kb;
            dp.v_out[vec + t] = vb;
            qs[t] = (float)qb;
            ks[t] = (float)kb;
            vs[t] = (float)vb;
        }
        al = gate_s[0];
        be = gate_s[1];
        if (t == 0) {
            dp.alpha_out[nh] = al;
            dp.beta_out[nh] = be;
        }
    } else {
        if (t < D) {
            ks[t] = to_f32(k[vec + t]);
            qs[t] = to_f32(q[vec + t]);
            vs[t] = to_f32(v[vec + t]);
        }
        al = alpha[nh];
        be = beta[nh];
    }
    __syncthreads();
    if (t < 64) {
        float p = 0.f;
        for (int i = t; i < D; i += 64) p += ks[i] * qs[i];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) p += __shfl_xor(p, off, 64);
        if (t == 0) kq_s = p;
    }
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), bq = a;
#pragma unroll
    for (int ii = 0; ii < RPT; ++ii) {
        const int i = rg + RG * ii;
        const float ki = ks[i], qi = qs[i];
        a.x += ki * sr[ii].x; a.y += ki * sr[ii].y; a.z += ki * sr[ii].z; a.w += ki * sr[ii].w;
        bq.x += qi * sr[ii].x; bq.y += qi * sr[ii].y; bq.z += qi * sr[ii].z; bq.w += qi * sr[ii].w;
    }
    pa[rg][cg] = a;
    pb[rg][cg] = bq;
    __syncthreads();
    float4 at = pa[0][cg], bt = pb[0][cg];
#pragma unroll
    for (int r = 1; r < RG; ++r) {
        const float4 x = pa[r][cg], y = pb[r][cg];
        at.x += x.x; at.y += x.y; at.z += x.z; at.w += x.w;
        bt.x += y.x; bt.y += y.y; bt.z += y.z; bt.w += y.w;
    }
    const float kq = kq_s;
    const int j0 = 4 * cg;
    float u[4], ov[4];
    const float av[4] = {at.x, at.y, at.z, at.w}, bv[4] = {bt.x, bt.y, bt.z, bt.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        u[c] = be * (vs[j0 + c] - al * av[c]);
        ov[c] = al * bv[c] + kq * u[c];
    }
    if (rg == 0) {
        if (h_out) {
            const int d = H * D;
            const int64_t n = nh / H;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int64_t hi = n * d + (int64_t)h * D + j0 + c;
                const float hp = h_prev_bf16 ? (float)reinterpret_cast<const bf16 *>(h_prev)[hi]
                                             : reinterpret_cast<const float *>(h_prev)[hi];
                const float hn = ov[c] + rho[h * D + j0 + c] * hp;
                h_out[hi] = hn;
                if (x_next) x_next[hi] = (bf16)hn;
            }
        } else {
            *reinterpret_cast<float4 *>(o + vec + j0) = make_float4(ov[0], ov[1], ov[2], ov[3]);
        }
    }
    // the updated state is written with non-temporal stores: the next step of
    // this loop comes after the other loops' states have streamed through
    typedef float f32x4v __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int ii = 0; ii < RPT; ++ii) {
        const float ki = ks[rg + RG * ii];
        const float4 s = sr[ii];
        const f32x4v sv = {al * s.x + ki * u[0], al * s.y + ki * u[1], al * s.z + ki * u[2], al * s.w + ki * u[3]};
        __builtin_nontemporal_store(sv, reinterpret_cast<f32x4v *>(&S[(rg + RG * ii) * CG + cg]));
    }
}

}  // namespace

hipError_t launch_decode(bool f32, int N, int H, int D, const void *q, const void *k, const void *v,
                         const float *alpha, const float *beta, float *states, float *o,
                         const void *h_prev, bool h_prev_bf16, const float *rho, float *h_out,
                         bf16 *x_next, hipStream_t s, const float *part, int S, float alpha_lo, float eps) {
    dim3 grid((unsigned)((int64_t)N * H));
    if (part && (f32 || S < 1 || S > 8)) return hipErrorInvalidValue;
    // with partials, q .. beta are where the step's operands are stored (nothing is read from them)
    const DecParts dp{part, S, (int)packed_rows(H, D), (int)qkv_rows_padded(H, D), alpha_lo, eps,
                      part ? (bf16 *)q : nullptr, part ? (bf16 *)k : nullptr, part ? (bf16 *)v : nullptr,
                      part ? (float *)alpha : nullptr, part ? (float *)beta : nullptr};
#define DEC(DD, T, PS)                                                                             \
    launch_kernel((k_decode<DD, T, PS>), grid, dim3(256), 0, s, (const T *)q, (const T *)k,  \
                       (const T *)v, alpha, beta, states, o, h_prev, h_prev_bf16 ? 1 : 0, rho,    \
                       h_out, x_next, H, dp)
    if (f32) {
        if (D == 128) DEC(128, float, false); else DEC(64, float, false);
    } else if (part) {
        if (D == 128) DEC(128, bf16, true); else DEC(64, bf16, true);
    } else {
        if (D == 128) DEC(128, bf16, false); else DEC(64, bf16, false);
    }
#undef DEC
    return hipGetLastError();
}

}  // namespace gdn
