// gemm_epi.h -- the element epilogues shared by the library's generic
// products (k_gemm_nt, k_gemm_tile): given the fp32 sum x of output (m, n),
// store it, add it, add a residual and/or a gated loop residual, or gate a
// second operand with sigmoid(x).  The gated-FFN epilogue (EPI_SWIGLU) pairs
// two sums per output and lives in the kernels themselves.
#pragma once

#include "gdn_device.h"
#include "gdn_kernels.h"

namespace gdn {

template <int EPI, typename TOut>
__device__ __forceinline__ void epi_apply(float x, int m, int n, TOut *C, int64_t ldc, const float *rho,
                                          const float *D1, int64_t ldd1, const float *D2, int64_t ldd2) {
    TOut *c = C + (int64_t)m * ldc + n;
    if constexpr (EPI == EPI_STORE) *c = from_f32<TOut>(x);
    else if constexpr (EPI == EPI_ACCUM) *c = from_f32<TOut>(to_f32(*c) + x);
    else if constexpr (EPI == EPI_RESID) *c = from_f32<TOut>(x + rho[n] * D1[(int64_t)m * ldd1 + n]);
    else if constexpr (EPI == EPI_ADD) *c = from_f32<TOut>(x + D1[(int64_t)m * ldd1 + n]);
    else if constexpr (EPI == EPI_ADD_RESID)
        *c = from_f32<TOut>(x + D1[(int64_t)m * ldd1 + n] + rho[n] * D2[(int64_t)m * ldd2 + n]);
    else if constexpr (EPI == EPI_GATE) *c = from_f32<TOut>(D1[(int64_t)m * ldd1 + n] / (1.f + expf(-x)));
}

// silu(a) b, the gated FFN's product of its two projections
__device__ __forceinline__ float swiglu(float a, float b) { return a / (1.f + expf(-a)) * b; }

}  // namespace gdn
