// Grouped path: expert-centric bf16 MFMA GEMMs over the aligned rows, for
// batches large enough that tokens share experts (the warp-decode write-up,
// last section: expert-centric packing stays better for prefill and large
// batches; "Hardware-Native Joint Sparse-Quantization for Trillion-Scale MoE",
// Section 3.4: grouped GEMM over routing-dependent token counts, weights as
// the left operand so Y_e^T = W_e X_e^T).
//
// One kernel template serves both GEMMs. A workgroup of eight waves takes one
// aligned block (b <= 64 routes of one expert: up to four 16-column
// sub-tiles) and a tile of two row sets of 64 weight rows (gate/up: the gate
// rows and the up rows of 64 neurons; down: the two halves of 128 output
// rows); wave w owns rows 16 (w % 4) .. +15 of row set w / 4. Every product
// is v_mfma_f32_16x16x32_bf16 with the expert's weight rows on A and the
// block's columns on B:
//   A lane l: weight row l%16, 8 reduction elements of lane group l/16;
//   B lane l: column l%16, the same 8 reduction elements;
//   D lane l: rows 4*(l/16)+i (i < 4) of column l%16.
// The reduction runs in slabs of 128 (gate/up) or 64 (down) elements, MFMA
// steps of 32 (step j, lane group q: elements 32j+8q .. 32j+8q+7 of the
// slab), so every step lies inside one quantisation group whenever g is a
// multiple of 32.
//
// Data movement: the tile's weight rows and the block's activation rows
// (16 bytes per lane, per active sub-tile, step and plane) go global -> LDS
// with 16-byte LDS-DMA loads into one ring of slab-sized slots, issued
// depth - 1 slabs ahead; nothing passes through VGPRs. The depth follows
// from the slot size (the slot holds only active sub-tiles). Each slab costs
// one wait on the wave's own loads (an exact vmcnt: the loads of the later
// slabs stay in flight) and one LDS-only workgroup barrier. Weight and
// activation loads are spread over the eight waves; the tile's scales and
// zeros arrive with the first slab. Blocks of one sub-tile (b <= 16) use a
// smaller ring and fewer registers so that three workgroups share a CU.
//
// The int4 words become bf16 (128 + q) pairs with one AND-OR each (AWQ
// nibble order) and a second MFMA per step adds -(128 + z) times the same
// activations, so a group's partial holds sum x (q - z); it is scaled by the
// group scale in fp32. MXFP8 codes convert exactly to bf16; the partial is
// scaled by the block's power of two.
// gate/up: B is x; the epilogue writes silu(gate) * up for every valid route
//   as a bf16 hi/lo pair (a = hi + lo to within 2^-17 relative).
// down: B is the hi and the lo plane of the intermediate (both accumulate
//   into the same partial); each route's yhat row is written once.
// combine: y[t] = sum over j ascending of w[t,j] * yhat[t*k+j].
// Workgroups whose block lies past num_padded (read on the device) skip it,
// so the grid can be sized from the host-known capacity. No floating-point
// atomics; every sum has a fixed order.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kThreads = 256;            // combine workgroup
constexpr int kTileRows = 64;            // weight rows per row set of a GEMM tile (four waves of 16)
constexpr int kMaxTok = 64;              // block size limit: four 16-column sub-tiles
constexpr int kMaxSub = kMaxTok / 16;
constexpr int kMaxGpr = 32;              // K / g limit (the tile's scales live in LDS)

__device__ __forceinline__ floatx4 mfma_bf16(const bf16x8& a, const bf16x8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// One packed word -> eight bf16 (128 + q), element order.
__device__ __forceinline__ bf16x8 bias_pairs(uint32_t w, uint32_t m) {
  uint32_t p[4];
  unpack8_bias128_m(w, m, p);
  return __builtin_bit_cast(bf16x8, make_uint4(p[0], p[1], p[2], p[3]));
}

// Eight copies of the bf16 value -(128 + z), z in 0..15.
__device__ __forceinline__ bf16x8 neg_zero_pairs(uint32_t z) {
  const uint32_t h = 0xC300u | z;
  const uint32_t pr = h | (h << 16);
  return __builtin_bit_cast(bf16x8, make_uint4(pr, pr, pr, pr));
}

// LDS byte address of a __shared__ object (low half of its generic address).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

// 16 bytes per lane from global memory to LDS at base + 16 * lane (LDS DMA).
// M0 carries the LDS base; nothing else in these kernels uses M0.
// It is issued from asm so that the compiler neither reorders it nor adds
// waits for it; the kernel waits for these loads itself (wait_vm_le).
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

// Wait until at most about n vector-memory operations of this wave are in
// flight (n wave-uniform, rounded down to 0..4, 6, 8, 12, 16 or 24: a
// smaller count only waits longer). Loads complete in issue order, so this
// waits for every load issued before the last n. A short branch tree keeps
// the scalar work small.
__device__ __forceinline__ void wait_vm_le(int n) {
  if (n >= 8) {
    if (n >= 16) {
      if (n >= 24) wait_vm<24>(); else wait_vm<16>();
    } else {
      if (n >= 12) wait_vm<12>(); else wait_vm<8>();
    }
  } else if (n >= 4) {
    if (n >= 6) wait_vm<6>(); else wait_vm<4>();
  } else if (n >= 2) {
    if (n >= 3) wait_vm<3>(); else wait_vm<2>();
  } else {
    if (n >= 1) wait_vm<1>(); else wait_vm<0>();
  }
}

struct GemmParams {
  const uint16_t* b0;            // B rows (bf16, K per row): x [M] or a_hi [Mk]
  const uint16_t* b1;            // second plane (a_lo) or null
  const int32_t* sorted;         // aligned rows (null in the batched layout)
  const int32_t* blocks;
  const int32_t* num_padded;
  const int32_t* counts;         // batched layout: rows of each expert [E], else null
  int cap;                       // batched layout: rows reserved per expert
  int nbpe;                      // batched layout: blocks per expert, ceil(cap / b)
  const unsigned char* q;        // int4: u32 [E][rows][K/8]; MXFP8: E4M3 [E][rows][K]
  const unsigned char* sc;       // int4: fp16 [E][rows][K/g]; MXFP8: E8M0 [E][rows][K/32]
  const uint8_t* zp;
  uint16_t* a_hi;                // gate/up output planes [Mk][I]
  uint16_t* a_lo;
  float* yhat;                   // down output [Mk][H]
  int mk, k, E, b, nblk;
  int ntile;                     // tiles per block
  int rows_per_expert;           // weight rows per expert (2I or H)
  int set_stride;                // row offset of row set 1 (I: up rows; 64: next 64 rows)
  int tile_stride;               // row offset between tiles (64 or 128)
  int out_rows;                  // row length of the output (I or H)
  int K, g;
};

constexpr int kGemmWaves = 8;
constexpr int kGemmThreads = kGemmWaves * kWave;
constexpr int kRingBytes = 64 * 1024;        // two workgroups per CU
constexpr int kSmallRingBytes = 36 * 1024;   // int4 with b <= 16 (one sub-tile): three per CU
constexpr int kSmallRingMxBytes = 40 * 1024; // MXFP8 with b <= 16: three per CU
constexpr int kMaxDepth = 8;

// One workgroup of eight waves computes a tile of 2 x 64 weight rows against
// one aligned block: wave w takes row set w / 4 (gate/up: the gate rows or
// the up rows of 64 neurons; down: rows 0..63 or 64..127 of a 128-row tile),
// rows 16 (w % 4) .. +15 of it.
// kGateUp: epilogue silu(gate) * up (else yhat rows). kPlanes: B planes (1: x;
// 2: the hi and lo planes). kSteps: 32-element MFMA steps per slab (4 or 2).
// kFlush: steps per scaled partial (g / 32, at most kSteps). kRing: LDS ring
// bytes (kRingBytes, or a small ring for blocks of one sub-tile, where the
// kernel is held to 80 VGPRs so that three workgroups share a CU).
template <int kFmt, bool kGateUp, int kPlanes, int kSteps, int kFlush, int kRing>
__global__ __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(kRing == kRingBytes ? 1 : 6)))
void grouped_gemm(const GemmParams p) {
  constexpr bool kMx = kFmt == MOE_W_MXFP8;
  // Sub-tiles a block can have: four (b <= 64), or one with the small ring
  // (b <= 16, which the launch guarantees).
  constexpr int kSub = kRing == kRingBytes ? kMaxSub : 1;
  constexpr int kSlabK = 32 * kSteps;                  // reduction elements per slab
  constexpr int kRowBytes = kMx ? kSlabK : kSlabK / 2; // weight bytes per row and slab
  constexpr int kRowsPerDma = 1024 / kRowBytes;        // weight rows per 1 KB LDS-DMA
  constexpr int kABytes = 2 * kTileRows * kRowBytes;   // weight bytes per slab (128 rows)
  constexpr int kScStride = kTileRows * kMaxGpr * 2;   // bytes per row set (fp16 scales)
  constexpr int kZpStride = kTileRows * kMaxGpr;       // bytes per row set (u8 zeros)
  constexpr int kADma = kABytes / 1024;                // weight DMAs per slab
  static_assert(kADma == 4 || kADma == 8 || kADma == 16, "weight DMAs per slab");
  // The pipeline keeps at least two slots in flight at the largest slot (every
  // sub-tile active); the depth computed per task relies on it.
  static_assert(kRing >= 2 * (kABytes + kSub * kPlanes * kSteps * 1024), "ring holds two slabs");
  __shared__ __align__(16) unsigned char ring[kRing];
  __shared__ __align__(16) unsigned char ssh[2 * kScStride];
  __shared__ __align__(16) unsigned char szz[2 * kZpStride];
  __shared__ int cols[kMaxTok];    // route of each block column, -1 for padding
  __shared__ int brow[kMaxTok];    // B row of each column (0 for padding)

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = uniform(threadIdx.x / kWave);
  const int rs = wave >> 2;                         // this wave's row set
  const int rl = 16 * (wave & 3);                   // first row of this wave within the set
  const int n = lane & 15, lq = lane >> 4;
  const int ntasks = p.nblk * p.ntile;
  const bool batched = p.counts != nullptr;
  const int npad = batched ? 0 : p.num_padded[0];
  const int row_bytes = kMx ? p.K : p.K / 2, gpr = p.K / p.g;
  constexpr int kScBytes = kMx ? 1 : 2;                 // E8M0 byte or fp16 scale
  const int nslab = p.K / kSlabK;
  const uint32_t nib_mask = in_vgpr(0x000F000Fu);

  for (int task = blockIdx.x; task < ntasks; task += gridDim.x) {
    const int blk = task / p.ntile;
    const int ng = task - blk * p.ntile;
    int e, nrows;    // the block's expert and, in the batched layout, its valid rows
    if (batched) {
      // Block j of expert e covers rows e * cap + j * b .. +b-1 of the batched
      // operands; rows at or past the expert's count are padding.
      e = blk / p.nbpe;
      const int j = blk - e * p.nbpe;
      const int cnt = min(max(p.counts[e], 0), p.cap);
      if (j * p.b >= cnt) continue;
      nrows = min(p.b, cnt - j * p.b);
    } else {
      if (blk * p.b >= npad) continue;
      e = p.blocks[blk];
      if (e < 0 || e >= p.E) continue;
      nrows = p.b;
    }

    if (threadIdx.x < kMaxTok) {
      const int c = threadIdx.x;
      int r = -1;
      if (batched) {
        if (c < nrows) r = (blk / p.nbpe) * p.cap + (blk % p.nbpe) * p.b + c;
      } else if (c < p.b) {
        r = p.sorted[static_cast<size_t>(blk) * p.b + c];
        if (r < 0 || r >= p.mk) r = -1;
      }
      cols[c] = r;
      brow[c] = r < 0 ? 0 : ((kGateUp && !batched) ? r / p.k : r);
    }
    __syncthreads();
    // Active sub-tiles (wave-uniform), listed in order; static indices only,
    // so the lists stay in registers.
    int amask = 0;
#pragma unroll
    for (int st = 0; st < kSub; ++st) {
      if (__ballot(cols[16 * st + n] >= 0) != 0ull) amask |= 1 << st;
    }
    const int nact = __builtin_popcount(amask);
    int act[kSub];                    // sub-tile of each active index
    {
      int m = amask;
#pragma unroll
      for (int u = 0; u < kSub; ++u) {
        act[u] = m ? __builtin_ctz(m) : 0;
        m &= m - 1;
      }
    }
    // Ring geometry: one slot per slab holds the 128 weight rows, then the
    // activations of every (plane, active sub-tile, step), 1 KB each.
    const int nbdma = nact * kPlanes * kSteps;                 // activation DMAs per slab
    const int slot_bytes = kABytes + nbdma * 1024;
    const int depth_fit = kRing / slot_bytes;
    const int depth = depth_fit < kMaxDepth ? depth_fit : kMaxDepth;   // >= 2 (static_assert above)
    // This wave's DMAs per slab: weight DMA i goes to wave i, activation DMA
    // i to wave i % 8.
    const int my_b = nbdma > wave ? (nbdma - wave + kGemmWaves - 1) / kGemmWaves : 0;
    // Weight DMA m goes to wave m % 8 (kADma is 4, 8 or 16).
    constexpr int kAMax = (kADma + kGemmWaves - 1) / kGemmWaves;   // weight DMAs per wave, at most
    const int my_a = kADma >= kGemmWaves ? kADma / kGemmWaves : (wave < kADma ? 1 : 0);
    const int per_slab = my_b + my_a;

    // Everything before this point is a plain load the compiler waits for;
    // from here on the only vector-memory operations are the LDS-DMA loads
    // below (and the epilogue stores after the slab loop).
    wait_vm<0>();

    const size_t ebase = static_cast<size_t>(e) * p.rows_per_expert + static_cast<size_t>(ng) * p.tile_stride;
    // Scales and zeros of the tile's two row sets, all groups (whole 1 KB
    // DMAs: lanes past a region re-read its first chunk and land in the
    // set's unused tail).
#pragma unroll
    for (int set = 0; set < 2; ++set) {
      const size_t r0 = ebase + static_cast<size_t>(set) * p.set_stride;
      const int nsc = (kTileRows * gpr * kScBytes) / 16, nzp = kMx ? 0 : (kTileRows * gpr) / 16;
      const unsigned char* gsc = p.sc + r0 * gpr * kScBytes;
      const unsigned char* gzp = kMx ? p.sc : p.zp + r0 * gpr;
      const int w0 = set * 4;
      for (int m = wave - w0; m >= 0 && m < 4 && m * kWave < nsc; m += 4) {
        const int c = m * kWave + lane;
        dma16(gsc + 16 * (c < nsc ? c : 0), lds_addr(ssh + set * kScStride + m * 1024));
      }
      for (int m = wave - w0; m >= 0 && m < 4 && m * kWave < nzp; m += 4) {
        const int c = m * kWave + lane;
        dma16(gzp + 16 * (c < nzp ? c : 0), lds_addr(szz + set * kZpStride + m * 1024));
      }
    }

    // Weight DMAs of this wave: DMA m covers tile rows kRowsPerDma * m ..
    // +kRowsPerDma-1; lane l takes row l % kRowsPerDma, chunk l / kRowsPerDma.
    const unsigned char* qa[kAMax];
#pragma unroll
    for (int t = 0; t < kAMax; ++t) {
      const int m = wave + kGemmWaves * t;
      const int tr = kRowsPerDma * (m < kADma ? m : 0) + lane % kRowsPerDma;     // tile-local row
      const int ch = lane / kRowsPerDma;
      const size_t grow = ebase + static_cast<size_t>(tr / kTileRows) * p.set_stride + tr % kTileRows;
      qa[t] = p.q + grow * row_bytes + 16 * ch;
    }
    // This wave's activation DMAs (at most two per slab: nbdma <= 16):
    // DMA i = ((plane * nact + u) * kSteps + j) is issued by wave i % 8 and
    // reads step j of this lane's column in active sub-tile u.
    const uint16_t* bsrc[2] = {p.b0, p.b0};
    int boff[2] = {0, 0};
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int i = wave + kGemmWaves * t;
      if (i >= nbdma) continue;
      const int j = i % kSteps;
      const int pu = i / kSteps;
      const int pl = (kPlanes == 2 && pu >= nact) ? 1 : 0;
      int m = amask;                      // the (pu - pl * nact)-th active sub-tile
      for (int v = pu - pl * nact; v > 0; --v) m &= m - 1;
      const int st = __builtin_ctz(m);
      const uint16_t* base = pl ? p.b1 : p.b0;
      bsrc[t] = base + static_cast<size_t>(brow[16 * st + n]) * p.K + 32 * j + 8 * lq;
      boff[t] = kABytes + i * 1024;
    }
    // Ring slots are walked with running offsets, and the DMA sources with
    // running pointers: no divisions in the slab loop.
    const int ring_used = depth * slot_bytes;
    const uint16_t* bnext0 = bsrc[0];
    const uint16_t* bnext1 = bsrc[1];
    const unsigned char* anext[kAMax];
#pragma unroll
    for (int t = 0; t < kAMax; ++t) anext[t] = qa[t];
    auto issue_next = [&](int off) {
      unsigned char* slot = ring + off;
      if (my_b > 0) dma16(bnext0, lds_addr(slot + boff[0]));
      if (my_b > 1) dma16(bnext1, lds_addr(slot + boff[1]));
#pragma unroll
      for (int t = 0; t < kAMax; ++t) {
        if (t < my_a) dma16(anext[t], lds_addr(slot + (wave + kGemmWaves * t) * 1024));
        anext[t] += kRowBytes;
      }
      bnext0 += kSlabK;
      bnext1 += kSlabK;
    };

    floatx4 acc[kSub];            // per active index u (sub-tile act[u])
#pragma unroll
    for (int u = 0; u < kSub; ++u) acc[u] = floatx4{0, 0, 0, 0};

    // This lane's weight row within the tile, and where its words sit in a slot.
    // Step j, lane group q reads elements 32j + 8q .. +7 of the row's slab:
    // int4 bytes 16j + 4q (word q of chunk j), MXFP8 bytes 32j + 8q (half
    // q % 2 of chunk 2j + q / 2); chunk c of row r sits at 16 (r + R c).
    const int arow = 64 * rs + rl + n;
    const int a_off = (arow / kRowsPerDma) * 1024 + 16 * (arow % kRowsPerDma) +
                      (kMx ? 16 * kRowsPerDma * (lq >> 1) + 8 * (lq & 1) : 4 * lq);
    constexpr int kAStep = kMx ? 32 * kRowsPerDma : 16 * kRowsPerDma;   // LDS bytes per step
    // Scale and zero addresses of this lane (group 0); the group index is
    // added per partial.
    const unsigned char* sp = ssh + rs * kScStride + (rl + 4 * lq) * gpr * kScBytes;
    const unsigned char* zpl = szz + rs * kZpStride + (rl + n) * gpr;
    // Group of the first partial of a slab: slab s covers groups s * gps ..
    // (g below the slab) or group s / spg (g a multiple of the slab).
    const int gps = p.g < kSlabK ? kSlabK / p.g : 1;
    const int spg = p.g < kSlabK ? 1 : p.g / kSlabK;

    int wr = 0;
    for (int s = 0; s < depth - 1 && s < nslab; ++s) {
      issue_next(wr);
      wr += slot_bytes;
    }
    const int n_steady = (depth - 2) * per_slab;
    int rd = 0, grp0 = 0, gcount = 0;
    for (int s = 0; s < nslab; ++s) {
      const bool more = s + depth - 1 < nslab;
      wait_vm_le(more ? n_steady : (nslab - 1 - s) * per_slab);
      lds_barrier();
      if (more) {
        issue_next(wr);
        wr += slot_bytes;
        if (wr == ring_used) wr = 0;
      }
      const unsigned char* slot = ring + rd;
      rd += slot_bytes;
      if (rd == ring_used) rd = 0;
      // Step j, lane group q: word 4j + q of the row = word q of chunk j.
      uint32_t aw[kSteps][kMx ? 2 : 1];
#pragma unroll
      for (int j = 0; j < kSteps; ++j) {
        if constexpr (kMx) {
          const uint2 v = *reinterpret_cast<const uint2*>(slot + a_off + kAStep * j);
          aw[j][0] = v.x;
          aw[j][1] = v.y;
        } else {
          aw[j][0] = *reinterpret_cast<const uint32_t*>(slot + a_off + kAStep * j);
        }
      }
#pragma unroll
      for (int f = 0; f < kSteps / kFlush; ++f) {
        const int grp = grp0 + f;
        bf16x8 Z;
        float cs[4];
        if constexpr (kMx) {
#pragma unroll
          for (int i = 0; i < 4; ++i) cs[i] = e8m0_to_float(sp[i * gpr + grp]);
        } else {
          Z = neg_zero_pairs(zpl[grp]);
          const uint16_t* sp16 = reinterpret_cast<const uint16_t*>(sp);
#pragma unroll
          for (int i = 0; i < 4; ++i) cs[i] = half_bits_to_float(sp16[i * gpr + grp]);
        }
        bf16x8 A[kFlush];
#pragma unroll
        for (int jj = 0; jj < kFlush; ++jj) {
          if constexpr (kMx) {
            const uint32_t* w = aw[kFlush * f + jj];
            A[jj] = __builtin_bit_cast(bf16x8, make_uint4(fp8x2_to_bf16x2<false>(w[0]), fp8x2_to_bf16x2<true>(w[0]),
                                                          fp8x2_to_bf16x2<false>(w[1]), fp8x2_to_bf16x2<true>(w[1])));
          } else {
            A[jj] = bias_pairs(aw[kFlush * f + jj][0], nib_mask);
          }
        }
#pragma unroll
        for (int u = 0; u < kSub; ++u) {
          if (u >= nact) break;
          // One chain per active sub-tile: the bias product and the
          // zero-point product accumulate into the same partial.
          floatx4 d = {0, 0, 0, 0};
#pragma unroll
          for (int jj = 0; jj < kFlush; ++jj) {
            const int j = kFlush * f + jj;
#pragma unroll
            for (int pl = 0; pl < kPlanes; ++pl) {
              const bf16x8 B = __builtin_bit_cast(
                  bf16x8, *reinterpret_cast<const uint4*>(slot + kABytes + (((pl * nact + u) * kSteps + j) * 1024) + 16 * lane));
              d = mfma_bf16(A[jj], B, d);
              if constexpr (!kMx) d = mfma_bf16(Z, B, d);
            }
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[u][i] = fmaf(cs[i], d[i], acc[u][i]);
          // Keep this sub-tile's accumulation in its own iteration: the
          // compiler can otherwise merge the accumulations into one tail that
          // the loop exit jumps into right after an MFMA whose result it
          // reads, without the wait states that read needs (seen on gfx950
          // with ROCm 7.2: wrong sums for the last of two or three sub-tiles).
          asm volatile("" : "+v"(acc[u]));
        }
      }
      if (++gcount == spg) {
        gcount = 0;
        grp0 += gps;
      }
    }

    // Epilogue: every valid column's rows are written once.
    if constexpr (kGateUp) {
      // The up waves hand their sums to the gate waves through the ring.
      lds_barrier();
      float* xch = reinterpret_cast<float*>(ring);
      if (rs == 1) {
#pragma unroll
        for (int u = 0; u < kSub; ++u)
          *reinterpret_cast<floatx4*>(xch + (((wave & 3) * kSub + u) * kWave + lane) * 4) = acc[u];
      }
      lds_barrier();
      if (rs == 0) {
#pragma unroll
        for (int u = 0; u < kSub; ++u) {
          if (u >= nact) break;
          const int r = cols[16 * act[u] + n];
          if (r < 0) continue;
          const floatx4 up = *reinterpret_cast<const floatx4*>(xch + ((wave * kSub + u) * kWave + lane) * 4);
          uint32_t hi2[2], lo2[2];
#pragma unroll
          for (int i = 0; i < 4; i += 2) {
            const float v0 = silu_mul(acc[u][i], up[i]);
            const float v1 = silu_mul(acc[u][i + 1], up[i + 1]);
            const bf16x2 h = {static_cast<__bf16>(v0), static_cast<__bf16>(v1)};
            const uint32_t hb = __builtin_bit_cast(uint32_t, h);
            const bf16x2 l = {static_cast<__bf16>(v0 - bf16_lo(hb)), static_cast<__bf16>(v1 - bf16_hi(hb))};
            hi2[i / 2] = hb;
            lo2[i / 2] = __builtin_bit_cast(uint32_t, l);
          }
          const size_t off = static_cast<size_t>(r) * p.out_rows + ng * p.tile_stride + rl + 4 * lq;
          *reinterpret_cast<uint2*>(p.a_hi + off) = make_uint2(hi2[0], hi2[1]);
          *reinterpret_cast<uint2*>(p.a_lo + off) = make_uint2(lo2[0], lo2[1]);
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < kSub; ++u) {
        if (u >= nact) break;
        const int r = cols[16 * act[u] + n];
        if (r < 0) continue;
        const size_t off = static_cast<size_t>(r) * p.out_rows + ng * p.tile_stride + 64 * rs + rl + 4 * lq;
        *reinterpret_cast<float4*>(p.yhat + off) = make_float4(acc[u][0], acc[u][1], acc[u][2], acc[u][3]);
      }
    }
    __syncthreads();   // cols, brow and the ring are reused by the next task
  }
}

// Routes of a token taken per round of the combine: their ids, weights and
// yhat segments are all loaded before any is used (one memory round trip
// per round instead of one per route).
constexpr int kCombineChunk = 8;

__global__ __launch_bounds__(kThreads) void combine_topk(
    const float* __restrict__ yhat, const int32_t* __restrict__ ids,
    const float* __restrict__ topk_w, float* __restrict__ y, int M, int k, int E, int ebase, int H) {
  const int quads = H >> 2;
  const int total = M * quads;
  for (int i = blockIdx.x * kThreads + threadIdx.x; i < total; i += gridDim.x * kThreads) {
    const int t = i / quads;
    const int h = (i - t * quads) << 2;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j0 = 0; j0 < k; j0 += kCombineChunk) {
      // Every route row of yhat exists (it may hold stale values for an
      // invalid route, which the select below never adds); slots past k
      // re-read the token's first route.
      int e[kCombineChunk];
      float w[kCombineChunk];
      float4 v[kCombineChunk];
#pragma unroll
      for (int c = 0; c < kCombineChunk; ++c) {
        const int r = t * k + (j0 + c < k ? j0 + c : 0);
        e[c] = ids[r] - ebase;
        w[c] = topk_w[r];
        v[c] = *reinterpret_cast<const float4*>(yhat + static_cast<size_t>(r) * H + h);
      }
      // Each product is formed and then kept or dropped by a select (no
      // branch the loads could be moved into).
#pragma unroll
      for (int c = 0; c < kCombineChunk; ++c) {
        const bool ok = j0 + c < k && e[c] >= 0 && e[c] < E;
        const float4 n = make_float4(fmaf(w[c], v[c].x, acc.x), fmaf(w[c], v[c].y, acc.y),
                                     fmaf(w[c], v[c].z, acc.z), fmaf(w[c], v[c].w, acc.w));
        acc.x = ok ? n.x : acc.x;
        acc.y = ok ? n.y : acc.y;
        acc.z = ok ? n.z : acc.z;
        acc.w = ok ? n.w : acc.w;
      }
    }
    *reinterpret_cast<float4*>(y + static_cast<size_t>(t) * H + h) = acc;
  }
}

// Steps per scaled partial: g / 32 for g below the slab, else a whole slab
// (g a multiple of the slab).
int flush_steps(int g, int steps) { return g >= 32 * steps ? steps : g / 32; }

bool group_ok(int K, int g, int slab) {
  if (g < 32 || (g % 32) != 0 || (K % g) != 0 || K / g > kMaxGpr) return false;
  return g < slab ? (slab % g) == 0 : (g % slab) == 0;
}

template <int kFmt, bool kGateUp, int kPlanes, int kSteps, int kRing>
hipError_t launch_gemm_ring(const GemmParams& gp, int wgs, hipStream_t stream) {
  if constexpr (kFmt == MOE_W_MXFP8) {
    hipLaunchKernelGGL((grouped_gemm<kFmt, kGateUp, kPlanes, kSteps, 1, kRing>), dim3(wgs), dim3(kGemmThreads), 0,
                       stream, gp);
    return hipGetLastError();
  }
  switch (flush_steps(gp.g, kSteps)) {
    case 1:
      hipLaunchKernelGGL((grouped_gemm<kFmt, kGateUp, kPlanes, kSteps, 1, kRing>), dim3(wgs), dim3(kGemmThreads), 0,
                         stream, gp);
      break;
    case 2:
      hipLaunchKernelGGL((grouped_gemm<kFmt, kGateUp, kPlanes, kSteps, 2, kRing>), dim3(wgs), dim3(kGemmThreads), 0,
                         stream, gp);
      break;
    default:
      hipLaunchKernelGGL((grouped_gemm<kFmt, kGateUp, kPlanes, kSteps, kSteps, kRing>), dim3(wgs),
                         dim3(kGemmThreads), 0, stream, gp);
      break;
  }
  return hipGetLastError();
}

// MXFP8 blocks are 32 elements: one scaled partial per MFMA step. Layers
// aligned with b <= 16 have one 16-column sub-tile per block, whose ring
// slots are small: a 36 KB ring (int4; 40 KB for MXFP8's wider weight rows)
// keeps two or more slots in flight and lets three workgroups share a CU
// (more tasks per round).
template <bool kGateUp, int kPlanes, int kSteps>
hipError_t launch_gemm(int fmt, const GemmParams& gp, int wgs, hipStream_t stream) {
  if (fmt == MOE_W_MXFP8) {
    if (gp.b <= 16)
      return launch_gemm_ring<MOE_W_MXFP8, kGateUp, kPlanes, kSteps, kSmallRingMxBytes>(gp, wgs, stream);
    return launch_gemm_ring<MOE_W_MXFP8, kGateUp, kPlanes, kSteps, kRingBytes>(gp, wgs, stream);
  }
  if (gp.b <= 16) return launch_gemm_ring<MOE_W_INT4_AWQ, kGateUp, kPlanes, kSteps, kSmallRingBytes>(gp, wgs, stream);
  return launch_gemm_ring<MOE_W_INT4_AWQ, kGateUp, kPlanes, kSteps, kRingBytes>(gp, wgs, stream);
}

constexpr int kGateUpSteps = 4;   // 128-element slabs
constexpr int kDownSteps = 2;     // 64-element slabs (two planes of activations)

}  // namespace

bool grouped_shape_ok(int fmt, int H, int I, int b, int g13, int g2) {
  // Whole slabs and whole tiles in both GEMMs (gate/up: 64 neurons; down:
  // 128 rows); the tile's scales (and int4 zeros) are staged in LDS: int4 at
  // most 32 groups per row, MXFP8 at most 64 blocks of 32 per row.
  if (b < 1 || b > kMaxTok || (H % 128) != 0 || (I % 64) != 0 || (H % (32 * kGateUpSteps)) != 0 ||
      (I % (32 * kDownSteps)) != 0)
    return false;
  if (fmt == MOE_W_MXFP8) return g13 == 32 && g2 == 32 && H / 32 <= 2 * kMaxGpr && I / 32 <= 2 * kMaxGpr;
  return group_ok(H, g13, 32 * kGateUpSteps) && group_ok(I, g2, 32 * kDownSteps);
}

hipError_t launch_grouped_gate_up(const GroupedArgs& p, hipStream_t stream) {
  GemmParams gp{};
  gp.b0 = p.x;
  gp.b1 = nullptr;
  gp.sorted = p.sorted;
  gp.blocks = p.blocks;
  gp.num_padded = p.num_padded;
  gp.q = static_cast<const unsigned char*>(p.w13.q);
  gp.sc = static_cast<const unsigned char*>(p.w13.scale);
  gp.zp = p.w13.zero;
  gp.a_hi = p.a_hi;
  gp.a_lo = p.a_lo;
  gp.mk = p.M * p.k;
  gp.k = p.k;
  gp.E = p.E;
  gp.b = p.b;
  gp.nblk = p.nblk;
  gp.ntile = p.I / kTileRows;
  gp.rows_per_expert = 2 * p.I;
  gp.set_stride = p.I;
  gp.tile_stride = kTileRows;
  gp.out_rows = p.I;
  gp.K = p.H;
  gp.g = p.w13.group;
  const int wgs = grid_for(int64_t(p.nblk) * gp.ntile, p.max_workgroups);
  return launch_gemm<true, 1, kGateUpSteps>(p.w13.fmt, gp, wgs, stream);
}

hipError_t launch_grouped_down(const GroupedArgs& p, hipStream_t stream) {
  GemmParams gp{};
  gp.b0 = p.a_hi;
  gp.b1 = p.a_lo;
  gp.sorted = p.sorted;
  gp.blocks = p.blocks;
  gp.num_padded = p.num_padded;
  gp.q = static_cast<const unsigned char*>(p.w2.q);
  gp.sc = static_cast<const unsigned char*>(p.w2.scale);
  gp.zp = p.w2.zero;
  gp.yhat = p.yhat;
  gp.mk = p.M * p.k;
  gp.k = p.k;
  gp.E = p.E;
  gp.b = p.b;
  gp.nblk = p.nblk;
  gp.ntile = p.H / (2 * kTileRows);
  gp.rows_per_expert = p.H;
  gp.set_stride = kTileRows;
  gp.tile_stride = 2 * kTileRows;
  gp.out_rows = p.H;
  gp.K = p.I;
  gp.g = p.w2.group;
  const int wgs = grid_for(int64_t(p.nblk) * gp.ntile, p.max_workgroups);
  return launch_gemm<false, 2, kDownSteps>(p.w2.fmt, gp, wgs, stream);
}

hipError_t launch_grouped_gate_up_batched(const GroupedArgs& p, const int32_t* counts, int cap, hipStream_t stream) {
  GemmParams gp{};
  gp.b0 = p.x;
  gp.counts = counts;
  gp.cap = cap;
  gp.nbpe = (cap + p.b - 1) / p.b;
  gp.q = static_cast<const unsigned char*>(p.w13.q);
  gp.sc = static_cast<const unsigned char*>(p.w13.scale);
  gp.zp = p.w13.zero;
  gp.a_hi = p.a_hi;
  gp.a_lo = p.a_lo;
  gp.mk = p.E * cap;
  gp.k = 1;
  gp.E = p.E;
  gp.b = p.b;
  gp.nblk = p.E * gp.nbpe;
  gp.ntile = p.I / kTileRows;
  gp.rows_per_expert = 2 * p.I;
  gp.set_stride = p.I;
  gp.tile_stride = kTileRows;
  gp.out_rows = p.I;
  gp.K = p.H;
  gp.g = p.w13.group;
  const int wgs = grid_for(int64_t(gp.nblk) * gp.ntile, p.max_workgroups);
  return launch_gemm<true, 1, kGateUpSteps>(p.w13.fmt, gp, wgs, stream);
}

hipError_t launch_grouped_down_batched(const GroupedArgs& p, const int32_t* counts, int cap, hipStream_t stream) {
  GemmParams gp{};
  gp.b0 = p.a_hi;
  gp.b1 = p.a_lo;
  gp.counts = counts;
  gp.cap = cap;
  gp.nbpe = (cap + p.b - 1) / p.b;
  gp.q = static_cast<const unsigned char*>(p.w2.q);
  gp.sc = static_cast<const unsigned char*>(p.w2.scale);
  gp.zp = p.w2.zero;
  gp.yhat = p.yhat;
  gp.mk = p.E * cap;
  gp.k = 1;
  gp.E = p.E;
  gp.b = p.b;
  gp.nblk = p.E * gp.nbpe;
  gp.ntile = p.H / (2 * kTileRows);
  gp.rows_per_expert = p.H;
  gp.set_stride = kTileRows;
  gp.tile_stride = 2 * kTileRows;
  gp.out_rows = p.H;
  gp.K = p.I;
  gp.g = p.w2.group;
  const int wgs = grid_for(int64_t(gp.nblk) * gp.ntile, p.max_workgroups);
  return launch_gemm<false, 2, kDownSteps>(p.w2.fmt, gp, wgs, stream);
}

hipError_t launch_combine(const GroupedArgs& p, hipStream_t stream) {
  const int64_t total = int64_t(p.M) * (p.H / 4);
  const int wgs = grid_for((total + kThreads - 1) / kThreads, p.max_workgroups);
  hipLaunchKernelGGL(combine_topk, dim3(wgs), dim3(kThreads), 0, stream, p.yhat, p.ids, p.topk_w,
                     p.y, p.M, p.k, p.E, p.ebase, p.H);
  return hipGetLastError();
}

}  // namespace moe
