// Measurement kernels for the benchmark: a plain streaming read and a copy,
// 16-byte nontemporal loads per lane, each workgroup streaming whole tiles of
// 256 lanes x (loads per lane) x 16 bytes with all of a tile's loads in
// flight at once. Their best times over the loads-per-lane variants are the
// floor the layer's kernels are compared with. A third kernel measures the
// dense MFMA issue rate the grouped GEMMs are compared with.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>

#include "moe_bench.h"

namespace {

constexpr int kThreads = 256;
constexpr int kMaxGrid = 8192;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int kUnroll>
__global__ __launch_bounds__(kThreads) void stream_read(const u32x4* __restrict__ src, size_t n16,
                                                        uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const size_t per_tile = size_t(kThreads) * kUnroll;
  for (size_t base = size_t(blockIdx.x) * per_tile; base < n16; base += size_t(gridDim.x) * per_tile) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t i = base + size_t(u) * kThreads + threadIdx.x;
      v[u] = i < n16 ? __builtin_nontemporal_load(src + i) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // Workgroup XOR through LDS: one word per workgroup.
  __shared__ uint32_t red[kThreads];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] ^= red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0];
}

template <int kUnroll>
__global__ __launch_bounds__(kThreads) void copy16(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                   size_t n16) {
  const size_t per_tile = size_t(kThreads) * kUnroll;
  for (size_t base = size_t(blockIdx.x) * per_tile; base < n16; base += size_t(gridDim.x) * per_tile) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t i = base + size_t(u) * kThreads + threadIdx.x;
      if (i < n16) v[u] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t i = base + size_t(u) * kThreads + threadIdx.x;
      if (i < n16) dst[i] = v[u];
    }
  }
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

constexpr int kMfmaChains = 8;            // independent accumulation chains per wave
constexpr double kMfmaFlops = 2.0 * 16 * 16 * 32;   // one 16x16x32 MFMA

// Dense MFMA issue rate: every wave runs kMfmaChains independent chains of
// iters 16x16x32 MFMAs (fp16 or bf16 operands, fp32 accumulation) on register
// operands, with no memory traffic in the loop. pattern 0: every operand 1.0,
// so each accumulator element ends at exactly 32 * iters; pattern 1: seeded
// operands in [1, 2) (a realistic mix of bits). Lane 0 of each wave writes
// the sum of its chains' first elements, kMfmaChains * 32 * iters under
// pattern 0.
template <bool kHalf>
__global__ __launch_bounds__(kThreads) void mfma_issue(int pattern, int iters, float* __restrict__ sink) {
  const uint32_t one = kHalf ? 0x3C00u : 0x3F80u;
  const uint32_t mant = kHalf ? 0x03FFu : 0x007Fu;
  u32x4v a, b;
  uint32_t x = (blockIdx.x * kThreads + threadIdx.x) * 2654435761u + 12345u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t lo = one, hi = one, lo2 = one, hi2 = one;
    if (pattern != 0) {
      x = x * 1664525u + 1013904223u;
      lo = one | (x & mant);
      hi = one | ((x >> 10) & mant);
      lo2 = one | ((x >> 16) & mant);
      hi2 = one | ((x >> 22) & mant);
    }
    a[i] = lo | (hi << 16);
    b[i] = lo2 | (hi2 << 16);
  }
  // The chains start equal; the empty asm hides that from the compiler,
  // which would otherwise fold them together.
  floatx4 acc[kMfmaChains];
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c) {
    acc[c] = floatx4{0, 0, 0, 0};
    asm volatile("" : "+v"(acc[c]));
  }
#pragma unroll 1
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c) {
      if constexpr (kHalf)
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(halfx8, a), __builtin_bit_cast(halfx8, b),
                                                        acc[c], 0, 0, 0);
      else
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                         __builtin_bit_cast(bf16x8, b), acc[c], 0, 0, 0);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c) s += acc[c][0];
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (kThreads / 64) + threadIdx.x / 64] = s;
}

int grid_of(size_t bytes, int unroll) {
  const size_t tile = size_t(kThreads) * unroll * 16;
  const size_t tiles = (bytes + tile - 1) / tile;
  return static_cast<int>(tiles < 1 ? 1 : (tiles > size_t(kMaxGrid) ? kMaxGrid : tiles));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

bool unroll_ok(int u) { return u == 1 || u == 2 || u == 4 || u == 8 || u == 16; }

template <typename F, typename... Args>
void run(F kernel, int grid, hipStream_t stream, hipEvent_t start, hipEvent_t stop, Args... args) {
  if (start == nullptr && stop == nullptr)
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), 0, stream, args...);
  else
    hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), 0, stream, start, stop, 0, args...);
}

}  // namespace

extern "C" {

int32_t moe_bench_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t sink_words,
                              int32_t loads_per_lane, int32_t* grid_out, hipEvent_t start, hipEvent_t stop,
                              hipStream_t stream) {
  if (src == nullptr || sink == nullptr || sink_words < 1 || !aligned16(src) || (bytes % 16) != 0 ||
      !unroll_ok(loads_per_lane))
    return 1;
  int grid = grid_of(bytes, loads_per_lane);
  if (grid > sink_words) grid = sink_words;
  const auto* s = static_cast<const u32x4*>(src);
  const size_t n16 = bytes / 16;
  switch (loads_per_lane) {
    case 1: run(stream_read<1>, grid, stream, start, stop, s, n16, sink); break;
    case 2: run(stream_read<2>, grid, stream, start, stop, s, n16, sink); break;
    case 4: run(stream_read<4>, grid, stream, start, stop, s, n16, sink); break;
    case 8: run(stream_read<8>, grid, stream, start, stop, s, n16, sink); break;
    default: run(stream_read<16>, grid, stream, start, stop, s, n16, sink); break;
  }
  if (hipGetLastError() != hipSuccess) return 2;
  if (grid_out != nullptr) *grid_out = grid;
  return 0;
}

int32_t moe_bench_copy(const void* src, void* dst, size_t bytes, int32_t loads_per_lane, hipEvent_t start,
                       hipEvent_t stop, hipStream_t stream) {
  if (src == nullptr || dst == nullptr || !aligned16(src) || !aligned16(dst) || (bytes % 16) != 0 ||
      !unroll_ok(loads_per_lane))
    return 1;
  const auto* s = static_cast<const u32x4*>(src);
  auto* d = static_cast<u32x4*>(dst);
  const size_t n16 = bytes / 16;
  const int grid = grid_of(bytes, loads_per_lane);
  switch (loads_per_lane) {
    case 1: run(copy16<1>, grid, stream, start, stop, s, d, n16); break;
    case 2: run(copy16<2>, grid, stream, start, stop, s, d, n16); break;
    case 4: run(copy16<4>, grid, stream, start, stop, s, d, n16); break;
    case 8: run(copy16<8>, grid, stream, start, stop, s, d, n16); break;
    default: run(copy16<16>, grid, stream, start, stop, s, d, n16); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

int32_t moe_bench_mfma(int32_t fp16, int32_t pattern, int32_t iters, int32_t grid, float* sink, double* flops_out,
                       hipEvent_t start, hipEvent_t stop, hipStream_t stream) {
  if (sink == nullptr || iters < 1 || grid < 1 || grid > kMaxGrid || (pattern != 0 && pattern != 1)) return 1;
  if (fp16)
    run(mfma_issue<true>, grid, stream, start, stop, pattern, iters, sink);
  else
    run(mfma_issue<false>, grid, stream, start, stop, pattern, iters, sink);
  if (hipGetLastError() != hipSuccess) return 2;
  if (flops_out != nullptr) *flops_out = double(grid) * (kThreads / 64) * double(iters) * kMfmaChains * kMfmaFlops;
  return 0;
}

}  // extern "C"
