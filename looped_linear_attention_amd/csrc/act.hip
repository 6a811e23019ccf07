// act.hip -- per-token adaptive halting of the loop driver on gfx950.
//
// LT2: Linear-Time Looped Transformers, Appendix A (adaptive computation
// time): after loop tau a single linear layer with a sigmoid maps the hidden
// state of position t to a halting probability p_t = sigmoid(w . h_t + b);
// the probabilities accumulate over the loops and the position halts once the
// running sum reaches 1 - eps (the threshold form, so that one loop can
// suffice).  A halted position's hidden state is frozen.  The decision is
// taken here in fp32: the dot product, the sigmoid and the running sum.
#include "gdn_device.h"
#include "gdn_kernels.h"

namespace gdn {

namespace {

__global__ __launch_bounds__(256) void k_act_init(float *R, int *halt, int M) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < M) {
        R[i] = 0.f;
        halt[i] = 0;
    }
}

// One wave per position: the dot product over d channels in a fixed order
// (each lane sums its 16-byte groups 4 l, 4 l + 256, ..., then a butterfly),
// so the decision is deterministic.  d is a multiple of 4.  Waves with no
// position return at once (no barriers here).
__global__ __launch_bounds__(256) void k_act_halt(const float *__restrict__ h, const float *__restrict__ w, float b,
                                                  float thr, int d, int M, int tau, int T, float *__restrict__ R,
                                                  int *__restrict__ halt, int *__restrict__ halt_out,
                                                  float *__restrict__ ponder_out) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= M) return;
    const float *ht = h + t * d;
    float acc = 0.f;
    for (int i = 4 * lane; i < d; i += 256) {
        const float4 x = *reinterpret_cast<const float4 *>(ht + i), y = *reinterpret_cast<const float4 *>(w + i);
        acc = fmaf(x.x, y.x, acc);
        acc = fmaf(x.y, y.y, acc);
        acc = fmaf(x.z, y.z, acc);
        acc = fmaf(x.w, y.w, acc);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (lane == 0) {
        int hv = halt[t];
        float r = R[t];
        if (hv == 0) {
            const float p = 1.f / (1.f + expf(-(acc + b)));
            r += p;
            R[t] = r;
            if (r >= thr) {
                hv = tau;
                halt[t] = tau;
            }
        }
        if (tau == T) {
            if (halt_out) halt_out[t] = hv ? hv : T;
            if (ponder_out) ponder_out[t] = r;
        }
    }
}

// One workgroup of 16 waves: wave w takes a contiguous range of positions in
// steps of 64 (one position per lane), counts the ones that ran loop tau with
// ballots, and after an exclusive sum of the 16 counts writes their indices
// in ascending order.
__global__ __launch_bounds__(1024) void k_act_rows(const int *__restrict__ halt, int tau, int M,
                                                   int *__restrict__ rows, int *__restrict__ count) {
    __shared__ int wsum[16];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int per = ((M + 15) / 16 + 63) / 64 * 64;
    const int lo = min(M, wave * per), hi = min(M, lo + per);
    auto ran = [&](int i) {
        if (i >= hi) return false;
        const int hv = halt[i];
        return hv == 0 || hv == tau;
    };
    int c = 0;
    for (int i0 = lo; i0 < hi; i0 += 64) c += __popcll(__ballot(ran(i0 + lane)));
    if (lane == 0) wsum[wave] = c;
    __syncthreads();
    int o = 0;
    for (int u = 0; u < wave; ++u) o += wsum[u];
    const unsigned long long below = (1ull << lane) - 1ull;
    for (int i0 = lo; i0 < hi; i0 += 64) {
        const bool r = ran(i0 + lane);
        const unsigned long long m = __ballot(r);
        if (r) rows[o + __popcll(m & below)] = i0 + lane;
        o += __popcll(m);
    }
    if (t == 0) {
        int tot = 0;
        for (int u = 0; u < 16; ++u) tot += wsum[u];
        *count = tot;
    }
}

}  // namespace

hipError_t launch_act_rows(int M, const int *halt, int tau, int *rows, int *count, hipStream_t s) {
    launch_kernel(k_act_rows, dim3(1), dim3(1024), 0, s, halt, tau, M, rows, count);
    return hipGetLastError();
}

hipError_t launch_act_init(int M, float *R, int *halt, hipStream_t s) {
    launch_kernel(k_act_init, dim3((unsigned)((M + 255) / 256)), dim3(256), 0, s, R, halt, M);
    return hipGetLastError();
}

hipError_t launch_act_halt(int M, int d, const float *h, const float *w, float b, float thr, int tau, int T, float *R,
                           int *halt, int *halt_out, float *ponder_out, hipStream_t s) {
    if (d % 4) return hipErrorInvalidValue;
    launch_kernel(k_act_halt, dim3((unsigned)((M + 3) / 4)), dim3(256), 0, s, h, w, b, thr, d, M, tau, T, R, halt,
                  halt_out, ponder_out);
    return hipGetLastError();
}

}  // namespace gdn
