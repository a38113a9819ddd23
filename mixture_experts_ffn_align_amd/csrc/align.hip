// Route alignment ("Route-Block Membership Selects Packed-AWQ Arithmetic",
// first paragraph; A_e / B(e,j) paragraph; stable-construction paragraph).
//
// One workgroup of 1024 threads (16 wave64s). The result is integer and does
// not depend on scheduling:
//   1. per-expert histogram with LDS integer atomics (order-free);
//   2. exclusive scan of the padded counts ceil(c_e/b)*b (wave scans + one
//      scan over the 16 wave totals) gives each expert's first aligned row;
//   3. routes are placed in chunks of 1024 in route-ID order. Inside a wave,
//      lanes holding the same expert are found with one ballot per ID bit
//      (wave64 has no match instruction); a lane's rank is the popcount of
//      its equal-expert peers below it. Per-wave counts in LDS give the
//      offset of earlier waves, and a per-expert running count the offset of
//      earlier chunks, so each expert's routes land in ascending route ID;
//   4. padding rows keep the sentinel M*k and blocks past num_padded keep -1
//      from a coalesced prefill at the start (ordered before the placement
//      by the workgroup barriers in between); each expert writes its own
//      entries of the block vector.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;

__device__ __forceinline__ int padded_count(int c, int b) { return (c + b - 1) / b * b; }

__global__ __launch_bounds__(kThreads) void align_kernel(
    const int32_t* __restrict__ ids, int mk, int E, int b, int nbits,
    int32_t* __restrict__ sorted, int32_t* __restrict__ blocks,
    int32_t* __restrict__ num_padded, int cap) {
  extern __shared__ __align__(16) int lds[];
  int* cnt = lds;              // [E]    routes per expert
  int* off = cnt + E;          // [E+1]  first aligned row per expert; off[E] = total
  int* run = off + E + 1;      // [E]    routes of this expert placed by earlier chunks
  int* wtot = run + E;         // [32]   wave scan totals
  uint8_t* wcnt = reinterpret_cast<uint8_t*>(wtot + 32);  // [16][E] per-wave counts in a chunk

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int nblk = cap / b;

  // Prefill: every row is padding and every block is past the end until the
  // steps below overwrite them (the ids loads are in flight meanwhile).
  for (int p = tid; p < cap; p += kThreads) sorted[p] = mk;
  for (int i = tid; i < nblk; i += kThreads) blocks[i] = -1;
  for (int e = tid; e < E; e += kThreads) { cnt[e] = 0; run[e] = 0; }
  for (int i = tid; i < kWaves * E; i += kThreads) wcnt[i] = 0;
  __syncthreads();

  for (int r = tid; r < mk; r += kThreads) {
    const int e = ids[r];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();

  // Exclusive scan of padded counts; thread t owns experts [e0, e1).
  const int per = (E + kThreads - 1) / kThreads;
  const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
  int local = 0;
  for (int e = e0; e < e1; ++e) local += padded_count(cnt[e], b);
  int incl = local;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int v = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += v;
  }
  if (lane == kWave - 1) wtot[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    const int v = lane < kWaves ? wtot[lane] : 0;
    int inc = v;
#pragma unroll
    for (int d = 1; d < kWaves; d <<= 1) {
      const int u = __shfl_up(inc, d, kWave);
      if (lane >= d) inc += u;
    }
    if (lane < kWaves) wtot[lane] = inc - v;
    if (lane == kWaves - 1) wtot[kWaves] = inc;
  }
  __syncthreads();
  {
    int base = wtot[wave] + incl - local;
    for (int e = e0; e < e1; ++e) {
      off[e] = base;
      base += padded_count(cnt[e], b);
    }
  }
  const int total = wtot[kWaves];
  if (tid == 0) {
    off[E] = total;
    num_padded[0] = total;
  }
  __syncthreads();
  // Block vector: expert e owns blocks off[e]/b .. off[e+1]/b - 1.
  for (int e = tid; e < E; e += kThreads) {
    for (int p = off[e]; p < off[e + 1]; p += b) blocks[p / b] = e;
  }

  // Stable placement, one chunk of 1024 routes at a time.
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int base = 0; base < mk; base += kThreads) {
    const int r = base + tid;
    const int e = r < mk ? ids[r] : -1;
    const bool valid = e >= 0 && e < E;
    unsigned long long peers = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool set = valid && ((e >> bit) & 1);
      const unsigned long long m = __ballot(set);
      peers &= set ? m : ~m;
    }
    const int rank = __popcll(peers & below);
    const int nwave = __popcll(peers);
    const bool leader = valid && rank == 0;
    if (leader) wcnt[wave * E + e] = static_cast<uint8_t>(nwave);
    __syncthreads();
    if (valid) {
      int prior = 0;
      for (int w = 0; w < wave; ++w) prior += wcnt[w * E + e];
      sorted[off[e] + run[e] + prior + rank] = r;
    }
    __syncthreads();
    if (leader) {
      atomicAdd(&run[e], nwave);
      wcnt[wave * E + e] = 0;
    }
    __syncthreads();
  }
}

}  // namespace

size_t align_lds_bytes(int E) {
  return sizeof(int) * (3 * static_cast<size_t>(E) + 1 + 32) + static_cast<size_t>(kWaves) * E;
}

hipError_t launch_align(const int32_t* ids, int mk, int E, int b, int32_t* sorted,
                        int32_t* blocks, int32_t* num_padded, int cap, hipStream_t stream) {
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const size_t lds = align_lds_bytes(E);
  hipLaunchKernelGGL(align_kernel, dim3(1), dim3(kThreads), lds, stream, ids, mk, E, b, nbits,
                     sorted, blocks, num_padded, cap);
  return hipGetLastError();
}

}  // namespace moe
