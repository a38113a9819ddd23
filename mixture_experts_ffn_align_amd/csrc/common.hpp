// Shared device helpers for the gfx950 MoE expert-FFN kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// bf16 bit patterns (low / high half of a word) -> fp32, exact.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Eight int4 values of one word, biased by 128, as four bf16 pairs:
// pair i = (128 + q_i, 128 + q_{i+4}). 0x4300 is bf16 128.0 with a zero
// mantissa, so OR-ing a 4-bit value into the mantissa gives 128 + q exactly.
__device__ __forceinline__ void unpack8_bias128(uint32_t w, uint32_t p[4]) {
  const uint32_t m = 0x000F000Fu, c = 0x43004300u;
  p[0] = (w & m) | c;
  p[1] = ((w >> 4) & m) | c;
  p[2] = ((w >> 8) & m) | c;
  p[3] = ((w >> 12) & m) | c;
}

// Eight consecutive bf16 activations (four words, element 2i in the low
// half of word i) regrouped into the pairs (x_i, x_{i+4}) that match
// unpack8_bias128.
__device__ __forceinline__ void pair_x8(const uint32_t x[4], uint32_t p[4]) {
  p[0] = (x[0] & 0xFFFFu) | (x[2] << 16);
  p[1] = (x[0] >> 16) | (x[2] & 0xFFFF0000u);
  p[2] = (x[1] & 0xFFFFu) | (x[3] << 16);
  p[3] = (x[1] >> 16) | (x[3] & 0xFFFF0000u);
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

// Route-ID gathers that tolerate any value: invalid entries map to -1.
__device__ __forceinline__ int load_expert(const int32_t* ids, int r, int E) {
  int e = ids[r];
  return (e >= 0 && e < E) ? e : -1;
}

}  // namespace moe
