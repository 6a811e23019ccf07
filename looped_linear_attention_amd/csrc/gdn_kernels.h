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
hipError_t launch_project(bool f32, int M, int d, int H, int D, const void *x, const void *Wpack,
                          void *q, void *k, void *v, float *alpha, float *beta, float alpha_lo,
                          float eps, float *zp, hipStream_t s);
hipError_t launch_gates(int M, int d, int H, int D, const void *x, const void *Wpack, float *alpha,
                        float *beta, float alpha_lo, hipStream_t s);

// Chunk preparation: per (b, h, chunk) decay products, the UT-transform
// inverse and the derived matrices W [D x 64], M [64 x 64], gamma [64].
struct ChunkWs {
    float *W;    // per chunk: bf16 hi plane [D][64] then bf16 lo plane [D][64] (D*64*4 bytes)
    float *M;    // per chunk: bf16 hi plane [64][64] then bf16 lo plane [64][64]
    float *g;    // per chunk: gamma [64] fp32
};
// Gates of the chunk preparation: alpha/beta [B*L, H], or (zp != nullptr) the
// P partial pre-activations zp[P][2H][B*L] of the projection, summed in order
// p = 0..P-1, with alpha = lo + (1 - lo) sigmoid(-z_a), beta = sigmoid(z_b).
struct GateSrc {
    const float *alpha, *beta;
    const float *zp;
    int P;
    float alpha_lo;
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
};
// Carry: sequential over chunks per (b, h, 16-column slice of S); the chain
// updates the state, output waves of the same workgroup form
// O = diag(gamma) Q S_c + M E a chunk behind and write `out`; final state to
// s_final.
hipError_t launch_scan_carry(bool f32, int B, int L, int H, int D, const void *q, const void *k, const void *v,
                             ChunkWs ws, const float *s_init, float *s_final, CarryOut out, hipStream_t s);

// One recurrent token per sequence; states updated in place.  With
// h_out != nullptr the loop residual is applied as in CarryOut.
hipError_t launch_decode(bool f32, int N, int H, int D, const void *q, const void *k, const void *v,
                         const float *alpha, const float *beta, float *states, float *o,
                         const void *h_prev, bool h_prev_bf16, const float *rho, float *h_out,
                         bf16 *x_next, hipStream_t s);

}  // namespace gdn
