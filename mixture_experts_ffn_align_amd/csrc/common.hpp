// Shared device helpers for the gfx950 MoE expert-FFN kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load of weights that are read once: marked nontemporal
// so they do not displace reused data (activations, intermediates) in cache.
__device__ __forceinline__ uint4 load_stream16(const uint32_t* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint4 load_stream16(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

constexpr int kWave = 64;

// Two OCP E4M3 codes (the low or the high 16 bits of w, low byte first) -> a
// bf16 pair in the same order. Exact: every E4M3 value is a bf16 value.
template <bool kHi>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHi));
}

// E8M0 block scale byte -> 2^(e - 127) in fp32 (e = 0 is the subnormal
// 2^-127, e = 255 is NaN).
__device__ __forceinline__ float e8m0_to_float(uint32_t e) {
  const uint32_t bits = e == 0 ? 0x00400000u : (e == 255 ? 0x7FC00000u : e << 23);
  return __uint_as_float(bits);
}

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// bf16 bit patterns (low / high half of a word) -> fp32, exact.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Eight int4 values of one word, biased by 128, as four bf16 pairs. Words
// use AWQ's interleaved nibble order (slot i holds element [0,2,4,6,1,3,5,7][i]),
// so (w >> 4i) & 0x000F000F puts elements 2i and 2i+1 in the low and high
// halves: pair i = (128 + q_{2i}, 128 + q_{2i+1}), the same element order as
// word i of eight consecutive bf16 activations. 0x4300 is bf16 128.0 with a
// zero mantissa, so OR-ing a 4-bit value into the mantissa gives 128 + q
// exactly.
__device__ __forceinline__ void unpack8_bias128(uint32_t w, uint32_t p[4]) {
  const uint32_t m = 0x000F000Fu, c = 0x43004300u;
  p[0] = (w & m) | c;
  p[1] = ((w >> 4) & m) | c;
  p[2] = ((w >> 8) & m) | c;
  p[3] = ((w >> 12) & m) | c;
}

// A value the compiler must keep in a VGPR. gfx9 VOP3 instructions take at
// most one scalar or literal operand, so with the nibble mask in a VGPR and
// the 0x43004300 constant in an SGPR each pair is a single v_and_or_b32.
__device__ __forceinline__ uint32_t in_vgpr(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// unpack8_bias128 with the nibble mask supplied in a VGPR (see in_vgpr).
__device__ __forceinline__ void unpack8_bias128_m(uint32_t w, uint32_t m, uint32_t p[4]) {
  const uint32_t c = 0x43004300u;
  p[0] = (w & m) | c;
  p[1] = ((w >> 4) & m) | c;
  p[2] = ((w >> 8) & m) | c;
  p[3] = ((w >> 12) & m) | c;
}

// Workgroup barrier for LDS data (and control) only. __syncthreads() also
// fences global memory: it waits for every load and store of the wave in
// flight (draining a load pipeline, or a store round trip per barrier).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
}

// Wave-uniform integer made explicitly scalar.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// The eight int4 values of one word as fp32, in element order.
__device__ __forceinline__ void unpack8_f32(uint32_t w, float q[8]) {
  const uint32_t lo = w & 0x0F0F0F0Fu;         // slots 0,2,4,6 -> elements 0,4,1,5
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;  // slots 1,3,5,7 -> elements 2,6,3,7
  q[0] = (float)(lo & 0xFF);
  q[4] = (float)((lo >> 8) & 0xFF);
  q[1] = (float)((lo >> 16) & 0xFF);
  q[5] = (float)(lo >> 24);
  q[2] = (float)(hi & 0xFF);
  q[6] = (float)((hi >> 8) & 0xFF);
  q[3] = (float)((hi >> 16) & 0xFF);
  q[7] = (float)(hi >> 24);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

// Butterfly sum over the 64 lanes of a wave; every lane ends with the same
// bits (each level adds the same two partial sums, and fp add commutes).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + expf(-g)) * u;
}

// Local expert index of route r: experts [ebase, ebase + E) are held here;
// any other value (an invalid route) maps to -1.
__device__ __forceinline__ int load_expert(const int32_t* ids, int r, int E, int ebase) {
  const int e = ids[r] - ebase;
  return (e >= 0 && e < E) ? e : -1;
}

// LDS byte address of a __shared__ object (low half of its generic address).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

// 16 bytes per lane from global memory to LDS at base + 16 * lane (LDS DMA).
// M0 carries the LDS base; nothing else in these kernels uses M0.
// It is issued from asm so that the compiler neither reorders it nor adds
// waits for it: the kernel waits for these loads itself (s_waitcnt vmcnt;
// the compiler's own waits stay right for loads issued after them).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(lds_base)
               : "memory", "m0");
}
#pragma clang diagnostic pop

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

}  // namespace moe
