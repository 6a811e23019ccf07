// block.hip -- the token-local kernels of the LT2 block around the mixer on
// gfx950: the pre-norm of each sub-layer and the packing of a block's weights.
//
// LT2: Linear-Time Looped Transformers, Section 2 ("Looped Transformer (LT)":
// each block is a token mixer and a position-wise FFN with residual
// connections, pre-norm omitted from its Eq. (1) for brevity; "LT2": the
// mixer is the linear one).  The norm is read as RMSNorm,
// x / sqrt(mean(x^2) + eps) * g, statistics in fp32.
#include "gdn_device.h"
#include "gdn_kernels.h"

namespace gdn {

namespace {

// One wave per token row: each lane sums the squares of its float4 groups
// (lane-strided), a butterfly gives the row's sum, then the row is scaled.
template <typename TIn, typename TOut>
__global__ __launch_bounds__(256) void k_rmsnorm(const TIn *__restrict__ h, const float *__restrict__ g, int M, int d,
                                                 float eps, TOut *__restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int64_t m = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (m >= M) return;
    const TIn *row = h + m * d;
    float ss = 0.f;
    for (int c = 4 * lane; c < d; c += 256) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float x = to_f32(row[c + j]);
            ss = fmaf(x, x, ss);
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
    const float inv = 1.f / sqrtf(ss / (float)d + eps);
    TOut *o = out + m * d;
    for (int c = 4 * lane; c < d; c += 256) {
#pragma unroll
        for (int j = 0; j < 4; ++j) o[c + j] = from_f32<TOut>(to_f32(row[c + j]) * inv * g[c + j]);
    }
}

// The interleaved up-projection of the gated FFN: packed row n of W13 [2F][d]
// is, in group n / 64, column 32 (n / 64) + n % 32 of W1 (n % 64 < 32) or of W3.
template <typename T>
__global__ __launch_bounds__(256) void k_pack_w13(const T *__restrict__ W1, const T *__restrict__ W3, int d, int F,
                                                  T *__restrict__ W13) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)2 * F * d) return;
    const int64_t n = idx / d;
    const int c = (int)(idx % d);
    const int grp = (int)(n / 64), r = (int)(n % 64);
    const int f = 32 * grp + (r & 31);
    W13[idx] = (r < 32 ? W1 : W3)[(int64_t)c * F + f];
}

__global__ __launch_bounds__(256) void k_bf16_to_f32(const bf16 *__restrict__ src, float *__restrict__ dst, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) dst[i] = (float)src[i];
}

__global__ __launch_bounds__(256) void k_copy_f32(const float *__restrict__ src, float *__restrict__ dst, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) dst[i] = src[i];
}

}  // namespace

hipError_t launch_rmsnorm(bool in_f32, bool out_f32, int M, int d, const void *h, const float *g, float eps,
                          void *out, hipStream_t s) {
    if (M <= 0 || d % 4) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(((int64_t)M + 3) / 4));
    if (in_f32 && out_f32)
        launch_kernel(k_rmsnorm<float, float>, grid, dim3(256), 0, s, (const float *)h, g, M, d, eps, (float *)out);
    else if (in_f32)
        launch_kernel(k_rmsnorm<float, bf16>, grid, dim3(256), 0, s, (const float *)h, g, M, d, eps, (bf16 *)out);
    else if (out_f32)
        launch_kernel(k_rmsnorm<bf16, float>, grid, dim3(256), 0, s, (const bf16 *)h, g, M, d, eps, (float *)out);
    else
        launch_kernel(k_rmsnorm<bf16, bf16>, grid, dim3(256), 0, s, (const bf16 *)h, g, M, d, eps, (bf16 *)out);
    return hipGetLastError();
}

hipError_t launch_pack_w13(bool f32, int d, int F, const void *W1, const void *W3, void *W13, hipStream_t s) {
    if (F % 32) return hipErrorInvalidValue;
    const int64_t n = (int64_t)2 * F * d;
    const dim3 grid((unsigned)((n + 255) / 256));
    if (f32) launch_kernel(k_pack_w13<float>, grid, dim3(256), 0, s, (const float *)W1, (const float *)W3, d, F, (float *)W13);
    else launch_kernel(k_pack_w13<bf16>, grid, dim3(256), 0, s, (const bf16 *)W1, (const bf16 *)W3, d, F, (bf16 *)W13);
    return hipGetLastError();
}

hipError_t launch_bf16_to_f32(const bf16 *src, float *dst, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    launch_kernel(k_bf16_to_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, src, dst, n);
    return hipGetLastError();
}

hipError_t launch_copy_f32(const float *src, float *dst, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    launch_kernel(k_copy_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, src, dst, n);
    return hipGetLastError();
}

}  // namespace gdn
