// gdn_device.h -- device helpers shared by the gfx950 kernels of the looped
// gated-delta-rule mixer (bf16 conversion, MFMA fragment types, split-bf16).
//
// MFMA lane layouts used throughout (CDNA4 matrix cores, 64-lane wavefront):
//   v_mfma_f32_16x16x32_bf16: A lane l holds row l%16, k = 8*(l/16) + i (i<8);
//                             B lane l holds col l%16, k = 8*(l/16) + i;
//                             C lane l holds col l%16, rows 4*(l/16) + i (i<4).
//   v_mfma_f32_16x16x16_bf16: as above with k = 4*(l/16) + i (i<4); its B
//                             k-slots coincide with the C rows of a lane, so an
//                             accumulator tile can feed the next product as B.
//   v_mfma_f32_32x32x16_bf16: A row l%32, k = 8*(l/32) + i; B col l%32;
//                             C col l%32, rows 8*(i/4) + 4*(l/32) + i%4 (i<16).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x16(const bf16x4 &a, const bf16x4 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                      __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// x ~= hi + lo with hi = bf16(x), lo = bf16(x - hi): about 16 significant bits.
template <int N>
__device__ __forceinline__ void split_bf16(const float (&x)[N], __bf16 (&hi)[N], __bf16 (&lo)[N]) {
    static_assert(N % 2 == 0, "pairs");
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    // two elements per conversion; a bf16 value widens to fp32 by moving its
    // bits to the upper half of the word
#pragma unroll
    for (int i = 0; i < N; i += 2) {
        const bf16x2 h = __builtin_convertvector((f32x2{x[i], x[i + 1]}), bf16x2);
        unsigned hu;
        __builtin_memcpy(&hu, &h, 4);
        const f32x2 r = {x[i] - __uint_as_float(hu << 16), x[i + 1] - __uint_as_float(hu & 0xffff0000u)};
        const bf16x2 l = __builtin_convertvector(r, bf16x2);
        hi[i] = h[0];
        hi[i + 1] = h[1];
        lo[i] = l[0];
        lo[i + 1] = l[1];
    }
}

__device__ __forceinline__ bf16x8 pack8(const __bf16 (&v)[8]) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = v[i];
    return r;
}
__device__ __forceinline__ bf16x4 pack4(const __bf16 (&v)[4]) {
    bf16x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = v[i];
    return r;
}

// Workgroup barrier that waits only for LDS traffic (outstanding global loads
// issued for a later step stay in flight across it).
// Built from the builtins (not inline asm) so that the compiler's own wait
// tracking knows every LDS access has completed here and adds no wait of its
// own for them later; the empty asm statements keep memory operations from
// being scheduled across the barrier.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt unconstrained
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + expf(-x)); }

typedef __attribute__((address_space(3))) void lds_void;

// Direct global -> LDS load of 16 bytes per active lane: lane i of the wave
// writes the 16 bytes at wave_base + 16 i (wave_base must be wave-uniform).
// Completion is tracked by the vector-memory counter only (wait_vmcnt).
__device__ __forceinline__ void dma16(const void *g, void *wave_base) {
    __builtin_amdgcn_global_load_lds(g, (lds_void *)wave_base, 16, 0, 0);
}

// The same direct load, issued so that the compiler's wait-count tracking does
// not see it.  For the builtin form the compiler makes every later LDS access
// it cannot prove disjoint wait for all outstanding direct loads, which would
// stall each chunk on the prefetch of the next one.  Callers order the loaded
// data themselves: wait_vmcnt until the loads are done, then a workgroup
// barrier, before any lane reads the destination.  The instruction writes no
// register (the data goes to LDS), and the leading s_nop covers the one wait
// state an LDS direct load needs after M0 is written by a scalar instruction.
__device__ __forceinline__ void dma16_async(const void *g, void *wave_base) {
    const unsigned lds = __builtin_amdgcn_readfirstlane((unsigned)(unsigned long)(lds_void *)wave_base);
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(lds) : "memory");
}

// The same direct load to an LDS byte address given as a number (see lds_addr).
__device__ __forceinline__ void dma16_async_at(const void *g, unsigned lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(lds) : "memory");
}
// LDS byte address of a __shared__ object, wave-uniform.  Taking it once from
// the object itself (rather than from pointers derived later) lets the
// compiler fold the address-space conversion.
__device__ __forceinline__ unsigned lds_addr(const void *p) {
    return __builtin_amdgcn_readfirstlane((unsigned)(unsigned long)(const lds_void *)p);
}

// The same direct load with a wave-uniform base address (scalar registers)
// and a per-lane 32-bit byte offset: one vector register per load instead of
// a 64-bit address.
__device__ __forceinline__ void dma16_async_s(const void *sbase, unsigned voff, void *wave_base) {
    const unsigned lds = __builtin_amdgcn_readfirstlane((unsigned)(unsigned long)(lds_void *)wave_base);
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds) : "memory");
}

// ... and with the LDS byte address given as a number (see lds_addr).
__device__ __forceinline__ void dma16_async_s_at(const void *sbase, unsigned voff, unsigned lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds) : "memory");
}

// Buffer resource over `bytes` bytes at `base` (raw addressing, stride 0;
// the gfx9-family format word).  Stores whose byte range does not lie inside
// [0, bytes) are dropped by the hardware, so a tail can be masked without a
// branch around the store instruction.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(void *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, bytes, 0x00020000);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14; expcnt and lgkmcnt left at max).
// The builtin is visible to the compiler's own wait tracking; the empty asm
// statements on both sides keep memory operations from being scheduled across
// it (the builtin alone does not order them), so the count refers to exactly
// the operations issued before it in program order.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "the vector-memory counter holds 0..63");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
    asm volatile("" ::: "memory");
}

}  // namespace gdn
