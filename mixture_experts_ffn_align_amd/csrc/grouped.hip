// Grouped path: expert-centric bf16 MFMA GEMMs over the aligned rows, for
// batches large enough that tokens share experts (the warp-decode write-up,
// last section: expert-centric packing stays better for prefill and large
// batches; "Hardware-Native Joint Sparse-Quantization for Trillion-Scale MoE",
// Section 3.4: grouped GEMM over routing-dependent token counts, weights as
// the left operand so Y_e^T = W_e X_e^T).
//
// One kernel template serves both GEMMs. A workgroup of eight waves takes up
// to 64 routes of one aligned block (one expert; up to four 16-column
// sub-tiles; a block of b > 64 routes is taken in parts of 64) and a tile of
// two row sets of 64 weight rows (gate/up: the gate
// rows and the up rows of 64 neurons; down: the two halves of 128 output
// rows); wave w owns rows 16 (w % 4) .. +15 of row set w / 4. Every product
// is a 16x16x32 MFMA (bf16 for gate/up, fp16 for down) with the expert's
// weight rows on A and the block's columns on B:
//   A lane l: weight row l%16, 8 reduction elements of lane group l/16;
//   B lane l: column l%16, the same 8 reduction elements;
//   D lane l: rows 4*(l/16)+i (i < 4) of column l%16.
// The reduction runs in slabs of 128 elements, MFMA steps of 32 (step j,
// lane group q: elements 32j+8q .. 32j+8q+7 of the slab), so every step lies
// inside one quantisation group whenever g is a multiple of 32.
//
// Data movement: the tile's weight rows and the block's activation rows go
// global -> LDS with 16-byte LDS-DMA loads into one ring of slab-sized slots,
// issued depth - 1 slabs ahead; nothing passes through VGPRs. An activation
// DMA fills 1 KB with eight columns times two steps (128 contiguous bytes,
// one cache line, per column; half the lines of a column-per-lane layout),
// its 16-byte pieces placed with an XOR of the column so that the MFMA's
// 16-byte LDS reads of a step stay free of bank conflicts. The depth follows from the slot
// size (the slot holds only active sub-tiles). Each slab costs one wait on
// the wave's own loads (an exact vmcnt: the loads of the later slabs stay in
// flight) and one LDS-only workgroup barrier. Weight and activation loads
// are spread over the eight waves; the tile's scales and zeros arrive with
// the first slab. Blocks of one sub-tile (b <= 16) use a smaller ring and
// fewer registers so that three workgroups share a CU.
//
// The int4 words become (128 + q) pairs with one AND-OR each (AWQ nibble
// order; bf16 or fp16, both exact) and a second MFMA per step adds
// -(128 + z) times the same activations, so a group's partial holds
// sum x (q - z); it is scaled by the group scale in fp32. MXFP8 codes convert
// exactly to bf16 or fp16; the partial is scaled by the block's power of two.
// gate/up: B is x (bf16); the epilogue writes a = silu(gate) * up for every
//   valid route as one fp16 plane: each route's 64 neurons of the tile are
//   multiplied by a power of two that puts their largest magnitude in
//   [2^14, 2^15) (no overflow; relative rounding 2^-11 for every value of
//   the chunk down to 2^-28 of its largest), and the inverse power of two is
//   stored beside it.
// down: B is that fp16 plane, plus per slab one page with each column's two
//   chunk multipliers, applied to the partial of each 64-element chunk;
//   each route's yhat row is written once.
// combine: y[t] = sum over j ascending of w[t,j] * yhat[t*k+j].
// Workgroups whose block lies past num_padded (read on the device) skip it,
// so the grid can be sized from the host-known capacity. No floating-point
// atomics; every sum has a fixed order.
// H and I need only be multiples of 32: when a GEMM's K or output rows are
// off the 128 grid, its last slab holds fewer MFMA steps and its last tile
// reaches past the output rows (the kRagged instantiation handles both; the
// loads stay inside their rows and the rows past the end are not written).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kThreads = 256;            // combine workgroup
constexpr int kTileRows = 64;            // weight rows per row set of a GEMM tile (four waves of 16)
constexpr int kMaxTok = 64;              // columns per task: four 16-column sub-tiles (a larger
                                         // block is split into parts of 64 columns)
constexpr int kMaxBlock = 1024;          // block size limit
constexpr int kMaxSub = kMaxTok / 16;
constexpr int kMaxGpr = 256;             // K / g limit (the tile's scales live in LDS; see lds_fits)
constexpr int kLdsPerCu = 160 * 1024;

constexpr int kSteps = 4;                // 32-element MFMA steps per slab
constexpr int kSlabK = 32 * kSteps;      // reduction elements per slab

typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef _Float16 halfx2 __attribute__((ext_vector_type(2)));

// A and B travel as raw 16-byte words; kHalf selects the fp16 MFMA (down:
// the intermediate is fp16) or the bf16 one (gate/up: x is bf16).
template <bool kHalf>
__device__ __forceinline__ floatx4 mfma16(const uint4& a, const uint4& b, const floatx4& c) {
  if constexpr (kHalf)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(halfx8, a), __builtin_bit_cast(halfx8, b), c,
                                                  0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

// Nibble mask of bias_pairs, to be held in a VGPR (one v_and_or_b32 per pair).
template <bool kHalf>
constexpr uint32_t kNibMask = kHalf ? 0x00780078u : 0x000F000Fu;

// One packed word -> eight (128 + q) values in element order. AWQ's nibble
// order puts elements 2i and 2i+1 in slots i and i+4 (bits 4i and 4i+16).
// bf16: 0x4300 is 128.0 with a mantissa step of 1, so (w >> 4i) & 0x000F000F
// OR 0x43004300 is the pair. fp16: 0x5800 is 128.0 with a step of 1/8, so
// the nibbles go three bits higher (mask 0x00780078).
template <bool kHalf>
__device__ __forceinline__ uint4 bias_pairs(uint32_t w, uint32_t m) {
  if constexpr (kHalf) {
    const uint32_t c = 0x58005800u;
    return make_uint4(((w << 3) & m) | c, ((w >> 1) & m) | c, ((w >> 5) & m) | c, ((w >> 9) & m) | c);
  } else {
    uint32_t p[4];
    unpack8_bias128_m(w, m, p);
    return make_uint4(p[0], p[1], p[2], p[3]);
  }
}

// Eight copies of -(128 + z), z in 0..15 (bf16 0xC300 | z, fp16 0xD800 | 8z).
template <bool kHalf>
__device__ __forceinline__ uint4 neg_zero_pairs(uint32_t z) {
  const uint32_t h = kHalf ? (0xD800u | (z << 3)) : (0xC300u | z);
  const uint32_t pr = h | (h << 16);
  return make_uint4(pr, pr, pr, pr);
}

// Two E4M3 codes (the low or the high 16 bits of w) -> an fp16 pair, exact.
template <bool kHi>
__device__ __forceinline__ uint32_t fp8x2_to_f16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, kHi));
}

// Four E4M3 codes of each of two words -> eight bf16 or fp16 values.
template <bool kHalf>
__device__ __forceinline__ uint4 fp8_operand(uint32_t w0, uint32_t w1) {
  if constexpr (kHalf)
    return make_uint4(fp8x2_to_f16x2<false>(w0), fp8x2_to_f16x2<true>(w0), fp8x2_to_f16x2<false>(w1),
                      fp8x2_to_f16x2<true>(w1));
  else
    return make_uint4(fp8x2_to_bf16x2<false>(w0), fp8x2_to_bf16x2<true>(w0), fp8x2_to_bf16x2<false>(w1),
                      fp8x2_to_bf16x2<true>(w1));
}

// Power-of-two shift t of a chunk whose largest magnitude is m: m * 2^t lies
// in [2^14, 2^15) (t = 14 - (exponent of m)); zero, infinite and NaN chunks
// keep t = 0, and t stays in [-126, 126] so that 2^t and 2^-t are normal.
__device__ __forceinline__ int chunk_shift(float m) {
  const int eb = static_cast<int>((__float_as_uint(m) >> 23) & 0xFFu);
  const int t = (m > 0.0f && eb < 255) ? 141 - eb : 0;
  return t < -126 ? -126 : (t > 126 ? 126 : t);
}

__device__ __forceinline__ float pow2f(int t) { return __uint_as_float(static_cast<uint32_t>(t + 127) << 23); }

// Largest v over the four lanes of a wave that share l % 16 (one per 16-lane
// row), in each of them: gfx950's lane swaps across row pairs, no LDS.
__device__ __forceinline__ float max_over_rows(float v) {
  const uint32_t b = __float_as_uint(v);
  const auto s32 = __builtin_amdgcn_permlane32_swap(b, b, false, false);   // rows 0,1 <-> 2,3
  const float m = fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
  const uint32_t c = __float_as_uint(m);
  const auto s16 = __builtin_amdgcn_permlane16_swap(c, c, false, false);   // rows 0,2 <-> 1,3
  return fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
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
  const uint16_t* b0;            // B rows (K per row): x [M] bf16, or the intermediate [Mk] fp16
  const float* bsc;              // down: chunk multipliers of the B rows [Mk][K/128][4], else null
  const int32_t* sorted;         // aligned rows (null in the batched layout)
  const int32_t* blocks;
  const int32_t* num_padded;
  const int32_t* counts;         // batched layout: rows of each expert [E], else null
  int cap;                       // batched layout: rows reserved per expert
  int nbpe;                      // batched layout: blocks per expert, ceil(cap / b)
  const unsigned char* q;        // int4: u32 [E][rows][K/8]; MXFP8: E4M3 [E][rows][K]
  const unsigned char* sc;       // int4: fp16 [E][rows][K/g]; MXFP8: E8M0 [E][rows][K/32]
  const uint8_t* zp;
  uint16_t* a16;                 // gate/up output: fp16 [Mk][I], scaled per 64-neuron chunk
  float* a_scale;                // gate/up output: [Mk][ceil(I/128)][4], entries 0, 1 undo the two chunks' scaling
  float* yhat;                   // down output [Mk][H]
  float* w13_out;                // gate/up: fp32 [Mk][2I] W13 outputs (gate, up) or null
  int mk, k, E, b, nblk;
  int ntile;                     // weight tiles per block
  int col0;                      // first column of every block this launch takes (blocks of more
                                 // than 64 routes take one launch per 64 columns)
  int rows_per_expert;           // weight rows per expert (2I or H)
  int set_stride;                // row offset of row set 1 (I: up rows; 64: next 64 rows)
  int tile_stride;               // row offset between tiles (64 or 128)
  int out_rows;                  // row length of the output (I or H): output rows past it in the last
                                 // tile are not written, and their weight rows are read as row out_rows - 1
  int K, g;                      // K a multiple of 32: the last slab may hold fewer than four steps
  int sc_set, zp_set;            // LDS bytes per row set of the tile's scales / zeros (set at launch)
};

constexpr int kGemmWaves = 8;
constexpr int kGemmThreads = kGemmWaves * kWave;
constexpr int kMaxDepth = 8;

// LDS ring of one GEMM instantiation. A slot holds one slab: the tile's 128
// weight rows, 1 KB per (active sub-tile, step) of activations and, for the
// down GEMM, a 1 KB page of chunk multipliers. Tasks of up to four
// sub-tiles (b > 16) get at least 64 KB and two slots at the largest slot
// (two workgroups per CU); blocks of one sub-tile (b <= 16) get three int4
// slots or two MXFP8 slots (three workgroups per CU).
template <int kFmt, bool kGateUp, bool kSmall>
struct Ring {
  static constexpr bool kMx = kFmt == MOE_W_MXFP8;
  static constexpr int kSub = kSmall ? 1 : kMaxSub;
  static constexpr int kABytes = 2 * kTileRows * (kMx ? kSlabK : kSlabK / 2);
  static constexpr int kPages = kGateUp ? 0 : 1;
  static constexpr int kSlotMax = kABytes + (kSub * kSteps + kPages) * 1024;
  static constexpr int kBytes =
      kSmall ? (kMx ? 2 : 3) * kSlotMax : (2 * kSlotMax > 64 * 1024 ? 2 * kSlotMax : 64 * 1024);
};

// One workgroup of eight waves computes a tile of 2 x 64 weight rows against
// one aligned block: wave w takes row set w / 4 (gate/up: the gate rows or
// the up rows of 64 neurons; down: rows 0..63 or 64..127 of a 128-row tile),
// rows 16 (w % 4) .. +15 of it.
// kGateUp: bf16 products and the silu(gate) * up epilogue (else fp16
// products and yhat rows). kFlush: steps per scaled partial (g / 32, at most
// kSteps). kSmall: blocks of one sub-tile (b <= 16, which the launch
// guarantees), a small ring and an 80-VGPR budget so that three workgroups
// share a CU.
template <int kFmt, bool kGateUp, int kFlush, bool kSmall, bool kRagged>
__global__ __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(kSmall ? 6 : 1)))
void grouped_gemm(const GemmParams p) {
  constexpr bool kMx = kFmt == MOE_W_MXFP8;
  constexpr bool kHalf = !kGateUp;                     // fp16 operands
  constexpr int kSub = Ring<kFmt, kGateUp, kSmall>::kSub;
  constexpr int kRing = Ring<kFmt, kGateUp, kSmall>::kBytes;
  constexpr int kRowBytes = kMx ? kSlabK : kSlabK / 2; // weight bytes per row and slab
  constexpr int kRowsPerDma = 1024 / kRowBytes;        // weight rows per 1 KB LDS-DMA
  constexpr int kABytes = 2 * kTileRows * kRowBytes;   // weight bytes per slab (128 rows)
  constexpr int kADma = kABytes / 1024;                // weight DMAs per slab
  static_assert(kADma == 4 || kADma == 8 || kADma == 16, "weight DMAs per slab");
  // The pipeline keeps at least two slots in flight at the largest slot (every
  // sub-tile active); the depth computed per task relies on it.
  static_assert(kRing >= 2 * Ring<kFmt, kGateUp, kSmall>::kSlotMax, "ring holds two slabs");
  static_assert(kABytes == Ring<kFmt, kGateUp, kSmall>::kABytes, "weight bytes per slab");
  __shared__ __align__(16) unsigned char ring[kRing];
  // The tile's scales and zeros, two row sets each, sized per launch
  // (p.sc_set, p.zp_set bytes per set: whole 1 KB DMA pieces).
  extern __shared__ __align__(16) unsigned char dyn_lds[];
  unsigned char* ssh = dyn_lds;
  unsigned char* szz = dyn_lds + 2 * p.sc_set;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = uniform(threadIdx.x / kWave);
  const int rs = wave >> 2;                         // this wave's row set
  const int rl = 16 * (wave & 3);                   // first row of this wave within the set
  const int n = lane & 15, lq = lane >> 4;
  const int ntasks = p.nblk * p.ntile;
  const int cb = p.col0;                               // this launch's first column of each block
  const int bw = min(p.b - cb, kMaxTok);               // and its columns
  const bool batched = p.counts != nullptr;
  const int npad = batched ? 0 : p.num_padded[0];
  const int row_bytes = kMx ? p.K : p.K / 2, gpr = p.K / p.g;
  constexpr int kScBytes = kMx ? 1 : 2;                 // E8M0 byte or fp16 scale
  // kRagged: K or the output rows off the 128 grid (multiples of 32): the
  // last slab may hold fewer than four MFMA steps and the last tile may
  // reach past the output rows.
  const int nslab = kRagged ? (p.K + kSlabK - 1) / kSlabK : p.K / kSlabK;
  const int last_steps = kRagged ? (p.K - (nslab - 1) * kSlabK) / 32 : kSteps;
  const uint32_t nib_mask = in_vgpr(kNibMask<kHalf>);

  for (int task = blockIdx.x; task < ntasks; task += gridDim.x) {
    const int blk = task / p.ntile;
    const int ng = task - blk * p.ntile;
    // Every wave holds the task's columns itself, lane c column cb + c of the
    // block (cb: this launch's part): rc is its route (batched layout: its
    // row), -1 for padding, and bc the
    // B row it reads. The expert ID and the routes are loaded together, and
    // the active sub-tiles, B rows and output rows come from ballots and
    // lane reads, with no LDS round trip or barrier before the first DMA.
    int e, rc = -1;
    if (batched) {
      // Block j of expert e covers rows e * cap + j * b .. +b-1 of the batched
      // operands; rows at or past the expert's count are padding.
      e = blk / p.nbpe;
      const int j = blk - e * p.nbpe;
      const int cnt = min(max(p.counts[e], 0), p.cap);
      if (j * p.b + cb >= cnt) continue;
      if (lane < min(bw, cnt - j * p.b - cb)) rc = e * p.cap + j * p.b + cb + lane;
    } else {
      if (blk * p.b >= npad) continue;
      // blk < nblk keeps the index inside the alignment's capacity.
      const int rr = lane < bw ? p.sorted[static_cast<size_t>(blk) * p.b + cb + lane] : -1;
      e = p.blocks[blk];
      if (e < 0 || e >= p.E) continue;
      rc = (rr >= 0 && rr < p.mk) ? rr : -1;
    }
    const int bc = rc < 0 ? 0 : ((kGateUp && !batched) ? rc / p.k : rc);
    // Active sub-tiles (wave-uniform), listed in order; static indices only,
    // so the lists stay in registers.
    const uint64_t valid = __ballot(rc >= 0);
    int amask = 0;
#pragma unroll
    for (int st = 0; st < kSub; ++st) {
      if (((valid >> (16 * st)) & 0xFFFFull) != 0ull) amask |= 1 << st;
    }
    const int nact = __builtin_popcount(amask);
    // A part of a block with no valid route has nothing to write (the same
    // decision in every wave: all of them hold the same columns).
    if (nact == 0) continue;
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
    // activations of every (active sub-tile, step), 1 KB each, then (down)
    // the page of chunk multipliers.
    constexpr int kPages = Ring<kFmt, kGateUp, kSmall>::kPages;
    const int nbdma = nact * kSteps;                           // activation DMAs per slab
    const int page_off = kABytes + nbdma * 1024;               // multiplier page within a slot
    const int slot_bytes = page_off + kPages * 1024;
    const int depth_fit = kRing / slot_bytes;
    const int depth = depth_fit < kMaxDepth ? depth_fit : kMaxDepth;   // >= 2 (static_assert above)
    // This wave's DMAs per slab: weight DMA i goes to wave i, activation DMA
    // i to wave i % 8.
    const int my_b = nbdma > wave ? (nbdma - wave + kGemmWaves - 1) / kGemmWaves : 0;
    // Weight DMA m goes to wave m % 8 (kADma is 4, 8 or 16).
    constexpr int kAMax = (kADma + kGemmWaves - 1) / kGemmWaves;   // weight DMAs per wave, at most
    const int my_a = kADma >= kGemmWaves ? kADma / kGemmWaves : (wave < kADma ? 1 : 0);
    // The multiplier page goes to the last wave (it has no more activation
    // DMAs than any other).
    const bool my_page = kPages > 0 && wave == kGemmWaves - 1;
    const int per_slab = my_b + my_a + (my_page ? 1 : 0);

    // Everything before this point is a plain load the compiler waits for
    // (or a store of the previous task's epilogue); from here on the only
    // vector-memory operations are the LDS-DMA loads below (and the epilogue
    // stores after the slab loop).
    wait_vm<0>();

    const size_t ebase = static_cast<size_t>(e) * p.rows_per_expert + static_cast<size_t>(ng) * p.tile_stride;
    // First output row of row set `set` of this tile (gate/up: both sets
    // cover the same 64 neurons), and how many of its 64 rows exist (at
    // least 32 in set 0: out_rows is a multiple of 32).
    auto set_first = [&](int set) { return ng * p.tile_stride + (kGateUp ? 0 : set * kTileRows); };
    auto set_rows = [&](int set) { return kRagged ? min(max(p.out_rows - set_first(set), 0), kTileRows) : kTileRows; };
    // Scales and zeros of the tile's two row sets, all groups (whole 1 KB
    // DMAs: lanes past a set's rows re-read the first chunk of set 0 and
    // land in the set's unused tail).
#pragma unroll
    for (int set = 0; set < 2; ++set) {
      const size_t r0 = ebase + static_cast<size_t>(set) * p.set_stride;
      const int nsc = (kTileRows * gpr * kScBytes) / 16, nzp = kMx ? 0 : (kTileRows * gpr) / 16;
      const int vsc = (set_rows(set) * gpr * kScBytes) / 16, vzp = kMx ? 0 : (set_rows(set) * gpr) / 16;
      const unsigned char* gsc = p.sc + r0 * gpr * kScBytes;
      const unsigned char* gzp = kMx ? p.sc : p.zp + r0 * gpr;
      const unsigned char* gsc0 = p.sc + ebase * gpr * kScBytes;
      const unsigned char* gzp0 = kMx ? p.sc : p.zp + ebase * gpr;
      // Waves 4 set .. 4 set + 3 move this set's pieces, every fourth each.
      const int w0 = set * 4;
      if (wave >= w0 && wave < w0 + 4) {
        for (int m = wave - w0; m * kWave < nsc; m += 4) {
          const int c = m * kWave + lane;
          dma16(c < vsc ? gsc + 16 * c : gsc0, lds_addr(ssh + set * p.sc_set + m * 1024));
        }
        for (int m = wave - w0; m * kWave < nzp; m += 4) {
          const int c = m * kWave + lane;
          dma16(c < vzp ? gzp + 16 * c : gzp0, lds_addr(szz + set * p.zp_set + m * 1024));
        }
      }
    }

    // Weight DMAs of this wave: DMA m covers tile rows kRowsPerDma * m ..
    // +kRowsPerDma-1; lane l takes row l % kRowsPerDma, chunk l / kRowsPerDma.
    // Rows past out_rows read row out_rows - 1 of the same set; chunks of the
    // last slab past its steps read the slab's first chunk (a_back bytes
    // back) and are not used.
    const unsigned char* qa[kAMax];
    int a_back[kAMax];
#pragma unroll
    for (int t = 0; t < kAMax; ++t) {
      const int m = wave + kGemmWaves * t;
      const int tr = kRowsPerDma * (m < kADma ? m : 0) + lane % kRowsPerDma;     // tile-local row
      const int ch = lane / kRowsPerDma;
      const int set = tr / kTileRows;
      const int o = kRagged ? min(set_first(set) + tr % kTileRows, p.out_rows - 1) : set_first(set) + tr % kTileRows;
      const size_t grow = static_cast<size_t>(e) * p.rows_per_expert +
                          (kGateUp ? static_cast<size_t>(set) * p.set_stride : 0) + o;
      qa[t] = p.q + grow * row_bytes + 16 * ch;
      a_back[t] = (kMx ? ch / 2 : ch) < last_steps ? 0 : 16 * ch;
    }
    // This wave's activation DMAs (at most kBMax per slab: nbdma <= 4 kSub):
    // DMA i = (u * kSteps + j) is issued by wave i % 8 and reads step j of
    // this lane's column in active sub-tile u.
    constexpr int kBMax = (kSub * kSteps + kGemmWaves - 1) / kGemmWaves;
    const uint16_t* bsrc[kBMax];
    int boff[kBMax];
    int b_back[kBMax];                    // last slab: elements back to its first piece
#pragma unroll
    for (int t = 0; t < kBMax; ++t) {
      bsrc[t] = p.b0;
      boff[t] = 0;
      b_back[t] = 0;
      const int i = wave + kGemmWaves * t;
      if (i >= nbdma) continue;
      const int j = i % kSteps;
      int m = amask;                      // the (i / kSteps)-th active sub-tile
      for (int v = i / kSteps; v > 0; --v) m &= m - 1;
      const int st = __builtin_ctz(m);
      // DMA j of a sub-tile: columns 8 (j & 1) .. +7, steps 2 (j >> 1) and
      // +1, 128 contiguous bytes per column; lane L takes column L / 8 of the
      // half and 16-byte piece (L % 8) ^ (column / 2) of its 128 bytes.
      const int c = 8 * (j & 1) + (lane >> 3);
      const int pc = (lane & 7) ^ (c >> 1);
      bsrc[t] = p.b0 + static_cast<size_t>(__shfl(bc, 16 * st + c, kWave)) * p.K + 64 * (j >> 1) + 8 * pc;
      boff[t] = kABytes + i * 1024;
      // Pieces of the last slab past its steps read the slab's first piece.
      const int eo = 64 * (j >> 1) + 8 * pc;
      b_back[t] = eo < 32 * last_steps ? 0 : eo;
    }
    // Multiplier page (down): lane 16 u + c reads the 16-byte entry of column
    // c of active sub-tile u for the slab (lanes past the active sub-tiles
    // read row 0's and are not used).
    const float* pnext = p.bsc;
    if (my_page) {
      int m = amask;
      for (int v = lane >> 4; v > 0 && m != 0; --v) m &= m - 1;
      const int row_src = __shfl(bc, m != 0 ? 16 * __builtin_ctz(m) + n : n, kWave);
      const int row = m != 0 ? row_src : 0;
      pnext = p.bsc + static_cast<size_t>(row) * nslab * 4;
    }
    // Ring slots are walked with running offsets, and the DMA sources with
    // running pointers: no divisions in the slab loop.
    const int ring_used = depth * slot_bytes;
    const uint16_t* bnext[kBMax];
#pragma unroll
    for (int t = 0; t < kBMax; ++t) bnext[t] = bsrc[t];
    const unsigned char* anext[kAMax];
#pragma unroll
    for (int t = 0; t < kAMax; ++t) anext[t] = qa[t];
    int issued = 0;                       // slabs issued so far
    auto issue_next = [&](int off) {
      unsigned char* slot = ring + off;
      const bool tail = kRagged && ++issued == nslab;
#pragma unroll
      for (int t = 0; t < kBMax; ++t) {
        if (t < my_b) dma16(bnext[t] - (tail ? b_back[t] : 0), lds_addr(slot + boff[t]));
        bnext[t] += kSlabK;
      }
#pragma unroll
      for (int t = 0; t < kAMax; ++t) {
        if (t < my_a) dma16(anext[t] - (tail ? a_back[t] : 0), lds_addr(slot + (wave + kGemmWaves * t) * 1024));
        anext[t] += kRowBytes;
      }
      if (my_page) dma16(pnext, lds_addr(slot + page_off));
      pnext += 4;
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
    const unsigned char* sp = ssh + rs * p.sc_set + (rl + 4 * lq) * gpr * kScBytes;
    const unsigned char* zpl = szz + rs * p.zp_set + (rl + n) * gpr;
    // Group of the first partial of a slab: slab s covers groups s * gps ..
    // (g below the slab) or group s / spg (g a multiple of the slab).
    // B operand of step j for lane (n, lq): column n, piece 4 (j & 1) + lq
    // of DMA 2 (j >> 1) + n / 8, stored at lane 8 (n % 8) + (piece ^ n / 2).
    static_assert(kSteps == 4, "two 128-byte column halves per slab");
    const int boff_b0 = (n >> 3) * 1024 + 16 * (8 * (n & 7) + (lq ^ (n >> 1)));
    const int boff_b1 = (n >> 3) * 1024 + 16 * (8 * (n & 7) + ((4 + lq) ^ (n >> 1)));
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
      // The last slab may hold fewer steps (a multiple of kFlush: g divides K).
      const int steps_here = kRagged && s == nslab - 1 ? last_steps : kSteps;
#pragma unroll
      for (int f = 0; f < kSteps / kFlush; ++f) {
        // (A guard rather than a break: the trip count stays exact, so the
        // loop unrolls in every instantiation.)
        if (kFlush * f < steps_here) {
        const int grp = grp0 + f;
        uint4 Z;
        float cs[4];
        if constexpr (kMx) {
#pragma unroll
          for (int i = 0; i < 4; ++i) cs[i] = e8m0_to_float(sp[i * gpr + grp]);
        } else {
          Z = neg_zero_pairs<kHalf>(zpl[grp]);
          const uint16_t* sp16 = reinterpret_cast<const uint16_t*>(sp);
#pragma unroll
          for (int i = 0; i < 4; ++i) cs[i] = half_bits_to_float(sp16[i * gpr + grp]);
        }
        // Unpacked once per group for every active sub-tile; with one
        // sub-tile (small blocks) each step's operand is formed right before
        // its products instead, which keeps three of the four out of the
        // registers.
        auto a_operand = [&](int jj) {
          if constexpr (kMx) {
            const uint32_t* w = aw[kFlush * f + jj];
            return fp8_operand<kHalf>(w[0], w[1]);
          } else {
            return bias_pairs<kHalf>(aw[kFlush * f + jj][0], nib_mask);
          }
        };
        uint4 A[kSub > 1 ? kFlush : 1];
        if constexpr (kSub > 1) {
#pragma unroll
          for (int jj = 0; jj < kFlush; ++jj) A[jj] = a_operand(jj);
        }
        // Down: the intermediate's scaling is uniform over 64-element chunks
        // (two steps), so a partial spans at most one chunk.
        constexpr int kPart = (kHalf && kFlush > 2) ? 2 : kFlush;
#pragma unroll
        for (int u = 0; u < kSub; ++u) {
          if (u >= nact) break;
          // Every B operand of this sub-tile's steps is read before its first
          // product (held in place by the scheduling barrier), so the chain
          // waits on one LDS round trip instead of one per pair of steps.
          uint4 Bs[kFlush];
#pragma unroll
          for (int jj = 0; jj < kFlush; ++jj) {
            const int j = kFlush * f + jj;
            Bs[jj] = *reinterpret_cast<const uint4*>(slot + kABytes + (u * kSteps + 2 * (j >> 1)) * 1024 +
                                                     ((j & 1) ? boff_b1 : boff_b0));
          }
          __builtin_amdgcn_sched_barrier(0);
          float pm[2] = {1.0f, 1.0f};
          if constexpr (kHalf) {
            const float2 v = *reinterpret_cast<const float2*>(slot + page_off + 16 * (16 * u + n));
            pm[0] = v.x;
            pm[1] = v.y;
          }
#pragma unroll
          for (int h = 0; h < kFlush / kPart; ++h) {
            // One chain per active sub-tile and partial: the bias product and
            // the zero-point product accumulate into the same partial.
            floatx4 d = {0, 0, 0, 0};
#pragma unroll
            for (int jj = h * kPart; jj < (h + 1) * kPart; ++jj) {
              const uint4 Aj = kSub > 1 ? A[kSub > 1 ? jj : 0] : a_operand(jj);
              d = mfma16<kHalf>(Aj, Bs[jj], d);
              if constexpr (!kMx) d = mfma16<kHalf>(Z, Bs[jj], d);
            }
            if constexpr (kHalf) {
              const float m = pm[(kFlush * f + h * kPart) / 2];
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[u][i] = fmaf(cs[i] * m, d[i], acc[u][i]);
            } else {
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[u][i] = fmaf(cs[i], d[i], acc[u][i]);
            }
          }
          // Keep this sub-tile's accumulation in its own iteration: the
          // compiler can otherwise merge the accumulations into one tail that
          // the loop exit jumps into right after an MFMA whose result it
          // reads, without the wait states that read needs (seen on gfx950
          // with ROCm 7.2: wrong sums for the last of two or three sub-tiles).
          asm volatile("" : "+v"(acc[u]));
        }
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
      // Gate waves: a = silu(gate) * up in place, and each column's largest
      // |a| over this wave's 16 neurons into LDS beside the hand-off area.
      float* xmax = xch + 4 * kSub * kWave * 4;    // [gate wave][active index][column]
      // This lane's four neurons exist (out_rows is a multiple of 32, so the
      // four are all in or all out); those that do not are left out of the
      // chunk's maximum and not written.
      const bool nvalid = !kRagged || ng * p.tile_stride + rl + 4 * lq < p.out_rows;
      if (rs == 0) {
#pragma unroll
        for (int u = 0; u < kSub; ++u) {
          if (u >= nact) break;
          const floatx4 up = *reinterpret_cast<const floatx4*>(xch + ((wave * kSub + u) * kWave + lane) * 4);
          if (p.w13_out != nullptr) {
            // The W13 outputs themselves (capture surface): gate, then up.
            const int r = __shfl(rc, 16 * act[u] + n, kWave);
            if (r >= 0 && nvalid) {
              float* o = p.w13_out + static_cast<size_t>(r) * (2 * p.out_rows) + ng * p.tile_stride + rl + 4 * lq;
              *reinterpret_cast<float4*>(o) = make_float4(acc[u][0], acc[u][1], acc[u][2], acc[u][3]);
              *reinterpret_cast<float4*>(o + p.out_rows) = make_float4(up[0], up[1], up[2], up[3]);
            }
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[u][i] = nvalid ? silu_mul(acc[u][i], up[i]) : 0.0f;
          const float m = max_over_rows(
              fmaxf(fmaxf(fabsf(acc[u][0]), fabsf(acc[u][1])), fmaxf(fabsf(acc[u][2]), fabsf(acc[u][3]))));
          if (lq == 0) xmax[(wave * kSub + u) * 16 + n] = m;
        }
      }
      lds_barrier();
      // Each valid column's 64 neurons are scaled by 2^t (the largest
      // magnitude into [2^14, 2^15)) and written as fp16; the gate wave of
      // the first 16 neurons stores 2^-t in the column's chunk entry.
      if (rs == 0) {
#pragma unroll
        for (int u = 0; u < kSub; ++u) {
          if (u >= nact) break;
          const int r = __shfl(rc, 16 * act[u] + n, kWave);
          if (r < 0) continue;
          const float m = fmaxf(fmaxf(xmax[u * 16 + n], xmax[(kSub + u) * 16 + n]),
                                fmaxf(xmax[(2 * kSub + u) * 16 + n], xmax[(3 * kSub + u) * 16 + n]));
          const int t = chunk_shift(m);
          const float sup = pow2f(t);
          const halfx2 h01 = {static_cast<_Float16>(acc[u][0] * sup), static_cast<_Float16>(acc[u][1] * sup)};
          const halfx2 h23 = {static_cast<_Float16>(acc[u][2] * sup), static_cast<_Float16>(acc[u][3] * sup)};
          const size_t off = static_cast<size_t>(r) * p.out_rows + ng * p.tile_stride + rl + 4 * lq;
          if (nvalid)
            *reinterpret_cast<uint2*>(p.a16 + off) =
                make_uint2(__builtin_bit_cast(uint32_t, h01), __builtin_bit_cast(uint32_t, h23));
          // (Neuron ng * 64 of wave 0, lane group 0, always exists.)
          const int nslab_out = (p.out_rows + kSlabK - 1) / kSlabK;
          if (wave == 0 && lq == 0)
            p.a_scale[(static_cast<size_t>(r) * nslab_out + (ng >> 1)) * 4 + (ng & 1)] = pow2f(-t);
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < kSub; ++u) {
        if (u >= nact) break;
        const int r = __shfl(rc, 16 * act[u] + n, kWave);
        if (r < 0 || (kRagged && ng * p.tile_stride + 64 * rs + rl + 4 * lq >= p.out_rows)) continue;
        const size_t off = static_cast<size_t>(r) * p.out_rows + ng * p.tile_stride + 64 * rs + rl + 4 * lq;
        *reinterpret_cast<float4*>(p.yhat + off) = make_float4(acc[u][0], acc[u][1], acc[u][2], acc[u][3]);
      }
    }
    // The ring is reused by the next task. LDS only: the epilogue's global
    // stores need not land first (the next task's first wait covers them).
    lds_barrier();
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

// LDS bytes per row set of a tile's scales and (int4) zeros: all K / g
// groups of 64 rows, rounded up to whole 1 KB DMA pieces.
int scale_set_bytes(int fmt, int gpr) { return (kTileRows * gpr * (fmt == MOE_W_MXFP8 ? 1 : 2) + 1023) / 1024 * 1024; }
int zero_set_bytes(int fmt, int gpr) { return fmt == MOE_W_MXFP8 ? 0 : (kTileRows * gpr + 1023) / 1024 * 1024; }

// One workgroup's LDS (its ring and both row sets' scales and zeros) fits a
// CU: above 128 groups per row only one workgroup per CU does.
template <int kFmt, bool kGateUp, bool kSmall>
bool lds_fits_as(int gpr) {
  return Ring<kFmt, kGateUp, kSmall>::kBytes + 2 * scale_set_bytes(kFmt, gpr) + 2 * zero_set_bytes(kFmt, gpr) <=
         kLdsPerCu;
}

template <bool kGateUp>
bool lds_fits(int fmt, int b, int gpr) {
  if (fmt == MOE_W_MXFP8)
    return b <= 16 ? lds_fits_as<MOE_W_MXFP8, kGateUp, true>(gpr) : lds_fits_as<MOE_W_MXFP8, kGateUp, false>(gpr);
  return b <= 16 ? lds_fits_as<MOE_W_INT4_AWQ, kGateUp, true>(gpr) : lds_fits_as<MOE_W_INT4_AWQ, kGateUp, false>(gpr);
}

bool group_ok(int K, int g, int slab) {
  if (g < 32 || (g % 32) != 0 || (K % g) != 0 || K / g > kMaxGpr) return false;
  return g < slab ? (slab % g) == 0 : (g % slab) == 0;
}

template <int kFmt, bool kGateUp, bool kSmall, bool kRagged>
hipError_t launch_gemm_ring_as(const GemmParams& gp, int wgs, uint32_t lds, hipStream_t stream) {
  if constexpr (kFmt == MOE_W_MXFP8) {
    launch(grouped_gemm<kFmt, kGateUp, 1, kSmall, kRagged>, dim3(wgs), dim3(kGemmThreads), lds, stream, gp);
  } else {
    switch (flush_steps(gp.g, kSteps)) {
      case 1:
        launch(grouped_gemm<kFmt, kGateUp, 1, kSmall, kRagged>, dim3(wgs), dim3(kGemmThreads), lds, stream, gp);
        break;
      case 2:
        launch(grouped_gemm<kFmt, kGateUp, 2, kSmall, kRagged>, dim3(wgs), dim3(kGemmThreads), lds, stream, gp);
        break;
      default:
        launch(grouped_gemm<kFmt, kGateUp, kSteps, kSmall, kRagged>, dim3(wgs), dim3(kGemmThreads), lds, stream,
               gp);
        break;
    }
  }
  return hipGetLastError();
}

template <int kFmt, bool kGateUp, bool kSmall>
hipError_t launch_gemm_ring(const GemmParams& gp_in, int wgs, hipStream_t stream) {
  // The tile's scales (and int4 zeros) for all K / g groups of its two row
  // sets, each set rounded up to whole 1 KB DMA pieces.
  GemmParams gp = gp_in;
  const int gpr = gp.K / gp.g;
  gp.sc_set = scale_set_bytes(kFmt, gpr);
  gp.zp_set = zero_set_bytes(kFmt, gpr);
  const uint32_t lds = static_cast<uint32_t>(2 * gp.sc_set + 2 * gp.zp_set);
  // Shapes on the 128 grid take the instantiation without the tail checks.
  if ((gp.K % kSlabK) != 0 || (gp.out_rows % gp.tile_stride) != 0)
    return launch_gemm_ring_as<kFmt, kGateUp, kSmall, true>(gp, wgs, lds, stream);
  return launch_gemm_ring_as<kFmt, kGateUp, kSmall, false>(gp, wgs, lds, stream);
}

// MXFP8 blocks are 32 elements: one scaled partial per MFMA step. Layers
// aligned with b <= 16 have one 16-column sub-tile per block, whose ring
// slots are small: the small ring keeps two or more slots in flight and lets
// three workgroups share a CU (more tasks per round).
template <bool kGateUp>
hipError_t launch_gemm_part(int fmt, const GemmParams& gp, int wgs, hipStream_t stream) {
  if (fmt == MOE_W_MXFP8) {
    if (gp.b <= 16) return launch_gemm_ring<MOE_W_MXFP8, kGateUp, true>(gp, wgs, stream);
    return launch_gemm_ring<MOE_W_MXFP8, kGateUp, false>(gp, wgs, stream);
  }
  if (gp.b <= 16) return launch_gemm_ring<MOE_W_INT4_AWQ, kGateUp, true>(gp, wgs, stream);
  return launch_gemm_ring<MOE_W_INT4_AWQ, kGateUp, false>(gp, wgs, stream);
}

// Blocks of more than 64 routes: one launch per 64 columns of every block
// (the parts write disjoint rows of the output).
template <bool kGateUp>
hipError_t launch_gemm(int fmt, const GemmParams& gp_in, int wgs, hipStream_t stream) {
  GemmParams gp = gp_in;
  for (gp.col0 = 0; gp.col0 < gp.b; gp.col0 += kMaxTok) {
    const hipError_t err = launch_gemm_part<kGateUp>(fmt, gp, wgs, stream);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace

bool grouped_shape_ok(int fmt, int H, int I, int b, int g13, int g2) {
  // H and I multiples of 32 (one MFMA step): the last tile of a GEMM may be
  // partly outside the output rows and the last slab shorter than 128; the
  // tile's scales (and int4 zeros) are staged in LDS: at most 256 groups
  // (int4) or blocks of 32 (MXFP8) per row, within one CU's LDS.
  if (b < 1 || b > kMaxBlock || H < 32 || I < 32 || (H % 32) != 0 || (I % 32) != 0) return false;
  if (fmt == MOE_W_MXFP8) {
    if (g13 != 32 || g2 != 32 || H / 32 > kMaxGpr || I / 32 > kMaxGpr) return false;
  } else if (!group_ok(H, g13, kSlabK) || !group_ok(I, g2, kSlabK)) {
    return false;
  }
  return lds_fits<true>(fmt, b, H / g13) && lds_fits<false>(fmt, b, I / g2);
}

hipError_t launch_grouped_gate_up(const GroupedArgs& p, hipStream_t stream) {
  GemmParams gp{};
  gp.b0 = p.x;
  gp.sorted = p.sorted;
  gp.blocks = p.blocks;
  gp.num_padded = p.num_padded;
  gp.q = static_cast<const unsigned char*>(p.w13.q);
  gp.sc = static_cast<const unsigned char*>(p.w13.scale);
  gp.zp = p.w13.zero;
  gp.a16 = p.a16;
  gp.a_scale = p.a_scale;
  gp.w13_out = p.w13_out;
  gp.mk = p.M * p.k;
  gp.k = p.k;
  gp.E = p.E;
  gp.b = p.b;
  gp.nblk = p.nblk;
  gp.ntile = (p.I + kTileRows - 1) / kTileRows;
  gp.rows_per_expert = 2 * p.I;
  gp.set_stride = p.I;
  gp.tile_stride = kTileRows;
  gp.out_rows = p.I;
  gp.K = p.H;
  gp.g = p.w13.group;
  const int wgs = grid_for(int64_t(p.nblk) * gp.ntile, p.max_workgroups);
  return launch_gemm<true>(p.w13.fmt, gp, wgs, stream);
}

hipError_t launch_grouped_down(const GroupedArgs& p, hipStream_t stream) {
  GemmParams gp{};
  gp.b0 = p.a16;
  gp.bsc = p.a_scale;
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
  gp.ntile = (p.H + 2 * kTileRows - 1) / (2 * kTileRows);
  gp.rows_per_expert = p.H;
  gp.set_stride = kTileRows;
  gp.tile_stride = 2 * kTileRows;
  gp.out_rows = p.H;
  gp.K = p.I;
  gp.g = p.w2.group;
  const int wgs = grid_for(int64_t(p.nblk) * gp.ntile, p.max_workgroups);
  return launch_gemm<false>(p.w2.fmt, gp, wgs, stream);
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
  gp.a16 = p.a16;
  gp.a_scale = p.a_scale;
  gp.mk = p.E * cap;
  gp.k = 1;
  gp.E = p.E;
  gp.b = p.b;
  gp.nblk = p.E * gp.nbpe;
  gp.ntile = (p.I + kTileRows - 1) / kTileRows;
  gp.rows_per_expert = 2 * p.I;
  gp.set_stride = p.I;
  gp.tile_stride = kTileRows;
  gp.out_rows = p.I;
  gp.K = p.H;
  gp.g = p.w13.group;
  const int wgs = grid_for(int64_t(gp.nblk) * gp.ntile, p.max_workgroups);
  return launch_gemm<true>(p.w13.fmt, gp, wgs, stream);
}

hipError_t launch_grouped_down_batched(const GroupedArgs& p, const int32_t* counts, int cap, hipStream_t stream) {
  GemmParams gp{};
  gp.b0 = p.a16;
  gp.bsc = p.a_scale;
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
  gp.ntile = (p.H + 2 * kTileRows - 1) / (2 * kTileRows);
  gp.rows_per_expert = p.H;
  gp.set_stride = kTileRows;
  gp.tile_stride = 2 * kTileRows;
  gp.out_rows = p.H;
  gp.K = p.I;
  gp.g = p.w2.group;
  const int wgs = grid_for(int64_t(gp.nblk) * gp.ntile, p.max_workgroups);
  return launch_gemm<false>(p.w2.fmt, gp, wgs, stream);
}

hipError_t launch_combine(const GroupedArgs& p, hipStream_t stream) {
  const int64_t total = int64_t(p.M) * (p.H / 4);
  const int wgs = grid_for((total + kThreads - 1) / kThreads, p.max_workgroups);
  launch(combine_topk, dim3(wgs), dim3(kThreads), 0, stream, p.yhat, p.ids, p.topk_w,
                     p.y, p.M, p.k, p.E, p.ebase, p.H);
  return hipGetLastError();
}

}  // namespace moe
