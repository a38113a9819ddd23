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
//
// Prefill-size M*k uses three launches over G workgroups of R routes each,
// with the same result bit for bit:
//   align_count    per-workgroup expert histogram -> counts[g][e];
//   align_colscan  per expert, exclusive prefix of counts over g (the rows
//                  that earlier workgroups place) and the expert's total;
//   align_scatter  every workgroup scans the padded totals itself, places
//                  its routes in chunks of 1024 exactly as above, starting
//                  at the expert's offset plus its prefix, and writes its
//                  share of the padding, the tail and the block vector.
// Earlier workgroups hold earlier route IDs, so each expert's routes stay in
// ascending route ID.
//
// Only experts [ebase, ebase + E) are held here: an ID outside that range
// marks an invalid route, and block entries are local indices e - ebase.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kRegChunks = 4;     // chunks of route IDs a thread holds in registers
static_assert(kAlignRoutesPerGroup == kRegChunks * kThreads, "a workgroup's routes fit its registers");

__device__ __forceinline__ int padded_count(int c, int b) { return (c + b - 1) / b * b; }

// Local expert index of route r, or -1 when its expert is not held here.
__device__ __forceinline__ int local_expert(const int32_t* __restrict__ ids, int r, int E, int ebase) {
  const int e = ids[r] - ebase;
  return (e >= 0 && e < E) ? e : -1;
}

// Exclusive scan of the padded counts of experts [0, E) held in cnt[] into
// off[0..E] (off[E] = total), by the whole workgroup; wtot is [kWaves + 1]
// of scratch. Thread t owns a contiguous run of experts.
__device__ __forceinline__ void scan_padded(const int* cnt, int* off, int* wtot, int E, int b) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
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
  int base = wtot[wave] + incl - local;
  for (int e = e0; e < e1; ++e) {
    off[e] = base;
    base += padded_count(cnt[e], b);
  }
  if (tid == 0) off[E] = wtot[kWaves];
  __syncthreads();
}

// Local experts of routes base + 1024 c + tid, c < kRegChunks (-1 past r1;
// r1 > base). Every load is issued, unconditionally (routes past r1 read
// route r1 - 1), before any is used: one memory round trip for the batch,
// not one per chunk behind a branch.
__device__ __forceinline__ void load_chunks(const int32_t* __restrict__ ids, int base, int r1, int E, int ebase,
                                            int (&ev)[kRegChunks]) {
  int raw[kRegChunks];
#pragma unroll
  for (int c = 0; c < kRegChunks; ++c) {
    const int r = base + c * kThreads + threadIdx.x;
    raw[c] = ids[r < r1 ? r : r1 - 1];
  }
#pragma unroll
  for (int c = 0; c < kRegChunks; ++c) {
    const int r = base + c * kThreads + threadIdx.x;
    const int e = raw[c] - ebase;
    ev[c] = (r < r1 && e >= 0 && e < E) ? e : -1;
  }
}

// Places one chunk of 1024 routes (route r of this thread has local expert
// e, -1 if invalid or past the end): run[e] holds the rows of expert e
// already placed, off[e] its first row; wcnt is [kWaves][E] bytes of zeroed
// scratch. Advances run[]. Called by the whole workgroup; its barriers order
// LDS only, so the route stores of one chunk stay in flight during the next.
__device__ __forceinline__ void place_chunk(int e, int r, int E, int nbits, const int* off, int* run,
                                            uint8_t* wcnt, int32_t* __restrict__ sorted) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const unsigned long long below = (1ull << lane) - 1ull;
  const bool valid = e >= 0;
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
  lds_barrier();
  if (valid) {
    int prior = 0;
    for (int w = 0; w < wave; ++w) prior += wcnt[w * E + e];
    sorted[off[e] + run[e] + prior + rank] = r;
  }
  lds_barrier();
  if (leader) {
    atomicAdd(&run[e], nwave);
    wcnt[wave * E + e] = 0;
  }
  lds_barrier();
}

// Places routes [base, r1) (at most kRegChunks chunks) whose local experts
// are already in ev[].
__device__ __forceinline__ void place_loaded(const int (&ev)[kRegChunks], int base, int r1, int E, int nbits,
                                             const int* off, int* run, uint8_t* wcnt,
                                             int32_t* __restrict__ sorted) {
#pragma unroll
  for (int c = 0; c < kRegChunks; ++c) {
    if (base + c * kThreads >= r1) break;   // uniform over the workgroup
    place_chunk(ev[c], base + c * kThreads + threadIdx.x, E, nbits, off, run, wcnt, sorted);
  }
}

// Places routes [r0, r1) in route-ID order, kRegChunks chunks per batch of loads.
__device__ __forceinline__ void place_routes(const int32_t* __restrict__ ids, int r0, int r1, int E, int ebase,
                                             int nbits, const int* off, int* run, uint8_t* wcnt,
                                             int32_t* __restrict__ sorted) {
  for (int base = r0; base < r1; base += kRegChunks * kThreads) {
    int ev[kRegChunks];
    load_chunks(ids, base, r1, E, ebase, ev);
    place_loaded(ev, base, r1, E, nbits, off, run, wcnt, sorted);
  }
}

__global__ __launch_bounds__(kThreads) void align_kernel(
    const int32_t* __restrict__ ids, int mk, int E, int ebase, int b, int nbits,
    int32_t* __restrict__ sorted, int32_t* __restrict__ blocks,
    int32_t* __restrict__ num_padded, int cap) {
  extern __shared__ __align__(16) int lds[];
  int* cnt = lds;              // [E]    routes per expert
  int* off = cnt + E;          // [E+1]  first aligned row per expert; off[E] = total
  int* run = off + E + 1;      // [E]    routes of this expert placed by earlier chunks
  int* wtot = run + E;         // [32]   wave scan totals
  uint8_t* wcnt = reinterpret_cast<uint8_t*>(wtot + 32);  // [16][E] per-wave counts in a chunk

  const int tid = threadIdx.x;
  const int nblk = cap / b;

  // The first batch of route IDs is requested before the prefill stores.
  int ev[kRegChunks];
  load_chunks(ids, 0, mk, E, ebase, ev);
  // Prefill: every row is padding and every block is past the end until the
  // steps below overwrite them (the ids loads are in flight meanwhile).
  for (int p = tid; p < cap; p += kThreads) sorted[p] = mk;
  for (int i = tid; i < nblk; i += kThreads) blocks[i] = -1;
  for (int e = tid; e < E; e += kThreads) { cnt[e] = 0; run[e] = 0; }
  for (int i = tid; i < kWaves * E; i += kThreads) wcnt[i] = 0;
  __syncthreads();

  // Histogram, kRegChunks chunks per batch of loads; up to kRegChunks
  // chunks of routes stay in registers for the placement.
  for (int base = 0; base < mk; base += kRegChunks * kThreads) {
    if (base > 0) load_chunks(ids, base, mk, E, ebase, ev);
#pragma unroll
    for (int c = 0; c < kRegChunks; ++c)
      if (ev[c] >= 0) atomicAdd(&cnt[ev[c]], 1);
  }
  __syncthreads();
  scan_padded(cnt, off, wtot, E, b);
  if (tid == 0) num_padded[0] = off[E];
  // Block vector: expert e owns blocks off[e]/b .. off[e+1]/b - 1.
  for (int e = tid; e < E; e += kThreads) {
    for (int p = off[e]; p < off[e + 1]; p += b) blocks[p / b] = e;
  }
  if (mk <= kRegChunks * kThreads) place_loaded(ev, 0, mk, E, nbits, off, run, wcnt, sorted);
  else place_routes(ids, 0, mk, E, ebase, nbits, off, run, wcnt, sorted);
}

// Multi-workgroup alignment, launch 1 of 3: counts[g][e] = routes of local
// expert e among routes [g R, (g + 1) R).
__global__ __launch_bounds__(kThreads) void align_count(const int32_t* __restrict__ ids, int mk, int E, int ebase,
                                                        int R, int32_t* __restrict__ counts) {
  extern __shared__ __align__(16) int hist[];
  for (int e = threadIdx.x; e < E; e += kThreads) hist[e] = 0;
  __syncthreads();
  const int r0 = blockIdx.x * R, r1 = min(mk, r0 + R);
  for (int base = r0; base < r1; base += kRegChunks * kThreads) {
    int ev[kRegChunks];
    load_chunks(ids, base, r1, E, ebase, ev);
#pragma unroll
    for (int c = 0; c < kRegChunks; ++c)
      if (ev[c] >= 0) atomicAdd(&hist[ev[c]], 1);
  }
  __syncthreads();
  int32_t* row = counts + static_cast<size_t>(blockIdx.x) * E;
  for (int e = threadIdx.x; e < E; e += kThreads) row[e] = hist[e];
}

// Launch 2 of 3: per expert (one thread each), counts[g][e] becomes the
// exclusive prefix over g, and totals[e] the expert's route count.
__global__ __launch_bounds__(256) void align_colscan(int32_t* __restrict__ counts, int G, int E,
                                                    int32_t* __restrict__ totals) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= E) return;
  int run = 0;
  int g = 0;
  for (; g + 4 <= G; g += 4) {
    const int c0 = counts[static_cast<size_t>(g) * E + e], c1 = counts[static_cast<size_t>(g + 1) * E + e];
    const int c2 = counts[static_cast<size_t>(g + 2) * E + e], c3 = counts[static_cast<size_t>(g + 3) * E + e];
    counts[static_cast<size_t>(g) * E + e] = run;
    counts[static_cast<size_t>(g + 1) * E + e] = run + c0;
    counts[static_cast<size_t>(g + 2) * E + e] = run + c0 + c1;
    counts[static_cast<size_t>(g + 3) * E + e] = run + c0 + c1 + c2;
    run += c0 + c1 + c2 + c3;
  }
  for (; g < G; ++g) {
    const int c = counts[static_cast<size_t>(g) * E + e];
    counts[static_cast<size_t>(g) * E + e] = run;
    run += c;
  }
  totals[e] = run;
}

// Launch 3 of 3: workgroup g places routes [g R, (g + 1) R) and writes its
// share of the padding rows, the tail past num_padded and the block vector.
__global__ __launch_bounds__(kThreads) void align_scatter(
    const int32_t* __restrict__ ids, int mk, int E, int ebase, int b, int nbits, int R,
    const int32_t* __restrict__ prefix, const int32_t* __restrict__ totals, int32_t* __restrict__ sorted,
    int32_t* __restrict__ blocks, int32_t* __restrict__ num_padded, int cap) {
  extern __shared__ __align__(16) int lds[];
  int* cnt = lds;              // [E]    expert totals
  int* off = cnt + E;          // [E+1]  first aligned row per expert
  int* run = off + E + 1;      // [E]    rows of the expert placed before this workgroup's chunk
  int* wtot = run + E;         // [32]
  uint8_t* wcnt = reinterpret_cast<uint8_t*>(wtot + 32);  // [16][E]
  const int tid = threadIdx.x, g = blockIdx.x, G = gridDim.x;
  const int r0 = g * R, r1 = min(mk, r0 + R);
  int ev[kRegChunks];                      // this workgroup's routes (R <= kRegChunks chunks)
  load_chunks(ids, r0, r1, E, ebase, ev);
  for (int e = tid; e < E; e += kThreads) {
    cnt[e] = totals[e];
    run[e] = prefix[static_cast<size_t>(g) * E + e];
  }
  for (int i = tid; i < kWaves * E; i += kThreads) wcnt[i] = 0;
  __syncthreads();
  scan_padded(cnt, off, wtot, E, b);
  const int total = off[E];
  if (g == 0 && tid == 0) num_padded[0] = total;
  // Padding rows of experts e = g, g + G, ... and their blocks.
  for (int e = g; e < E; e += G) {
    for (int p = off[e] + cnt[e] + tid; p < off[e + 1]; p += kThreads) sorted[p] = mk;
    for (int p = off[e] + tid * b; p < off[e + 1]; p += kThreads * b) blocks[p / b] = e;
  }
  // Tail past num_padded, strided over the grid.
  for (int p = total + g * kThreads + tid; p < cap; p += G * kThreads) sorted[p] = mk;
  for (int i = total / b + g * kThreads + tid; i < cap / b; i += G * kThreads) blocks[i] = -1;
  place_loaded(ev, r0, r1, E, nbits, off, run, wcnt, sorted);
}

}  // namespace

size_t align_lds_bytes(int E) {
  return sizeof(int) * (3 * static_cast<size_t>(E) + 1 + 32) + static_cast<size_t>(kWaves) * E;
}

int align_groups(int mk) { return (mk + kAlignRoutesPerGroup - 1) / kAlignRoutesPerGroup; }

size_t align_ws_bytes(int mk, int E) {
  if (mk <= kAlignSingleMaxRoutes) return 0;
  const size_t words = static_cast<size_t>(align_groups(mk)) * E + E;
  return (words * sizeof(int32_t) + 255) & ~size_t(255);
}

hipError_t launch_align(const int32_t* ids, int mk, int E, int ebase, int b, int32_t* sorted,
                        int32_t* blocks, int32_t* num_padded, int cap, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const size_t lds = align_lds_bytes(E);
  const size_t need = align_ws_bytes(mk, E);
  if (need == 0 || ws == nullptr || ws_bytes < need) {
    launch(align_kernel, dim3(1), dim3(kThreads), lds, stream, ids, mk, E, ebase, b, nbits,
                       sorted, blocks, num_padded, cap);
    return hipGetLastError();
  }
  const int G = align_groups(mk);
  int32_t* counts = static_cast<int32_t*>(ws);
  int32_t* totals = counts + static_cast<size_t>(G) * E;
  launch(align_count, dim3(G), dim3(kThreads), sizeof(int) * static_cast<size_t>(E), stream, ids, mk,
                     E, ebase, kAlignRoutesPerGroup, counts);
  launch(align_colscan, dim3((E + 255) / 256), dim3(256), 0, stream, counts, G, E, totals);
  launch(align_scatter, dim3(G), dim3(kThreads), lds, stream, ids, mk, E, ebase, b, nbits,
                     kAlignRoutesPerGroup, counts, totals, sorted, blocks, num_padded, cap);
  return hipGetLastError();
}

}  // namespace moe
