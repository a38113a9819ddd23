// Grouped path: expert-centric bf16 MFMA GEMMs over the aligned rows, for
// batches large enough that tokens share experts (the warp-decode write-up,
// last section: expert-centric packing stays better for prefill and large
// batches; "Hardware-Native Joint Sparse-Quantization for Trillion-Scale MoE",
// Section 3.4: grouped GEMM over routing-dependent token counts, weights as
// the left operand so Y_e^T = W_e X_e^T).
//
// A workgroup takes one aligned block (b <= 64 routes of one expert, four
// 16-token sub-tiles) and 64 output rows; wave w owns rows 16w..16w+15.
// Every GEMM uses v_mfma_f32_16x16x32_bf16 with the expert's weight rows on
// the A operand and the block's tokens on B:
//   A lane l: weight row l%16, 8 reduction elements of lane group l/16;
//   B lane l: token column l%16, the same 8 reduction elements;
//   D lane l: rows 4*(l/16)+i (i < 4) of column l%16.
// The reduction runs in slabs of 32*kSpw elements, each inside one
// quantisation group; lane group q holds words kSpw*q .. kSpw*q+kSpw-1 of a
// slab row and MFMA step j uses word kSpw*q + j. The block's activations for
// a slab are staged in LDS (double-buffered: the next slab's global loads
// are in flight while the current slab's MFMAs run) and shared by the four
// waves; each wave streams only its own weight rows, one slab ahead, straight
// into registers. Sub-tiles with no valid route are skipped.
//
// gate/up: the int4 words become bf16 (128 + q) pairs with one AND-OR (AWQ
//   nibble order) and a second MFMA per step adds -(128 + z) times the same
//   activations, so each slab's accumulator holds sum x (q - z) for the
//   group; it is scaled by the group scale in fp32. The epilogue writes
//   silu(gate) * up for every valid route as a bf16 hi/lo pair (a = hi + lo
//   to within 2^-17 relative), the B operand of the down GEMM.
// down: the weights are dequantised exactly to bf16 integers (q - z lies in
//   [-15, 15]) and two MFMAs per step take the hi and lo planes of the
//   intermediate. Each route's yhat row is written once.
// combine: y[t] = sum over j ascending of w[t,j] * yhat[t*k+j].
// Workgroups whose block lies past num_padded (read on the device) exit at
// once, so the grid can be sized from the host-known capacity. No
// floating-point atomics; every sum has a fixed order.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kTileRows = 16 * kWaves;   // output rows per workgroup
constexpr int kMaxTok = 64;              // block size limit: four 16-token sub-tiles
constexpr int kMaxSub = kMaxTok / 16;

__device__ __forceinline__ floatx4 mfma_bf16(const bf16x8& a, const bf16x8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// One packed word -> eight bf16 (128 + q), element order.
__device__ __forceinline__ bf16x8 bias_pairs(uint32_t w) {
  uint32_t p[4];
  unpack8_bias128(w, p);
  return __builtin_bit_cast(bf16x8, make_uint4(p[0], p[1], p[2], p[3]));
}

// Eight copies of the bf16 value -(128 + z), z in 0..15.
__device__ __forceinline__ bf16x8 neg_zero_pairs(uint32_t z) {
  const uint32_t h = 0xC300u | z;
  const uint32_t pr = h | (h << 16);
  return __builtin_bit_cast(bf16x8, make_uint4(pr, pr, pr, pr));
}

// One packed word -> eight exact bf16 values (q - z), element order.
__device__ __forceinline__ bf16x8 dequant8_exact(uint32_t w, float z) {
  float qf[8];
  unpack8_f32(w, qf);
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = static_cast<__bf16>(qf[i] - z);
  return r;
}

template <int kSpw>
__device__ __forceinline__ void load_words(const uint32_t* p, uint32_t (&w)[kSpw]) {
  if constexpr (kSpw == 4) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else if constexpr (kSpw == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    w[0] = v.x; w[1] = v.y;
  } else {
    w[0] = p[0];
  }
}

// Route of every column of the block (-1 for padding), staged in LDS, and
// the per-lane view: route of column n of each sub-tile and which sub-tiles
// hold a valid route.
struct BlockView {
  int rid[kMaxSub];
  bool act[kMaxSub];
};

__device__ __forceinline__ BlockView stage_block(const int32_t* sorted, int blk, int b, int mk,
                                                 int* cols, int n) {
  if (threadIdx.x < kMaxTok) {
    int r = -1;
    if (static_cast<int>(threadIdx.x) < b) {
      r = sorted[static_cast<size_t>(blk) * b + threadIdx.x];
      if (r < 0 || r >= mk) r = -1;
    }
    cols[threadIdx.x] = r;
  }
  __syncthreads();
  BlockView v;
#pragma unroll
  for (int st = 0; st < kMaxSub; ++st) {
    v.rid[st] = cols[16 * st + n];
    v.act[st] = __ballot(v.rid[st] >= 0) != 0ull;
  }
  return v;
}

// Weight words of a wave run kDepth slabs ahead of the MFMAs in a register
// ring (the ring index is static: the slab loop is unrolled by kDepth), so
// each wave keeps kDepth slabs of its weight rows in flight; kDepth * kSpw
// words (256 reduction elements) per lane and row.
#ifndef MOE_RING_WORDS
#define MOE_RING_WORDS 4
#endif
template <int kSpw>
constexpr int ring_depth() { return MOE_RING_WORDS / kSpw > 0 ? MOE_RING_WORDS / kSpw : 1; }

template <int kSpw>
__global__ __launch_bounds__(kThreads) void grouped_gate_up_int4(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ sorted,
    const int32_t* __restrict__ blocks, const int32_t* __restrict__ num_padded,
    const uint32_t* __restrict__ q, const uint16_t* __restrict__ sc,
    const uint8_t* __restrict__ zp, uint16_t* __restrict__ a_hi, uint16_t* __restrict__ a_lo,
    int mk, int k, int E, int H, int I, int g, int b, int nblk) {
  constexpr int kSlab = 32 * kSpw;
  constexpr int kRowB = kSlab * 2 + 16;          // bytes per staged token row (padded)
  constexpr int kChunks = kSlab / 8;             // 16-byte chunks per token row
  constexpr int kMaxGroups = 64;                 // H / g held in LDS (H <= 8192 at g = 128)
  constexpr int kDepth = ring_depth<kSpw>();
  __shared__ __align__(16) unsigned char bs[2][kMaxTok * kRowB];
  __shared__ uint16_t ssh[2 * kTileRows * kMaxGroups / 4];   // this tile's scales: [2*64 rows][gpr]
  __shared__ uint8_t szz[2 * kTileRows * kMaxGroups / 4];    // and zeros
  __shared__ int cols[kMaxTok];
  __shared__ int toks[kMaxTok];                              // token of each block column, -1 if none
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int n = lane & 15, lq = lane >> 4;
  const int ngroups = I / kTileRows;
  const int ntasks = nblk * ngroups;
  const int npad = num_padded[0];
  const int words = H >> 3, gpr = H / g;
  const int nslab = H / kSlab;

  for (int task = blockIdx.x; task < ntasks; task += gridDim.x) {
    const int blk = task / ngroups;
    const int ng = task - blk * ngroups;
    if (blk * b >= npad) continue;
    const int e = blocks[blk];
    if (e < 0 || e >= E) continue;

    // Weight rows of this wave: gate rows and up rows of 16 neurons.
    const size_t tile0 = static_cast<size_t>(e) * (2 * I) + ng * kTileRows;
    const size_t rowg = tile0 + wave * 16;
    const size_t rowu = rowg + I;
    const uint32_t* qg = q + (rowg + n) * words + kSpw * lq;
    const uint32_t* qu = q + (rowu + n) * words + kSpw * lq;
    uint32_t wg[kDepth][kSpw], wu[kDepth][kSpw];
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      if (d < nslab) {
        load_words<kSpw>(qg + d * 4 * kSpw, wg[d]);
        load_words<kSpw>(qu + d * 4 * kSpw, wu[d]);
      }
    }
    // Scales and zeros of the tile's 64 gate and 64 up rows, for all groups.
    for (int v = threadIdx.x; v < 2 * kTileRows * gpr; v += kThreads) {
      const int half = v / (kTileRows * gpr);
      const size_t off = (tile0 + half * static_cast<size_t>(I)) * gpr + (v - half * kTileRows * gpr);
      ssh[v] = sc[off];
      szz[v] = zp[off];
    }
    if (threadIdx.x < kMaxTok) {
      const int c = threadIdx.x;
      int r = c < b ? sorted[static_cast<size_t>(blk) * b + c] : -1;
      toks[c] = (r >= 0 && r < mk) ? r / k : -1;
    }
    const BlockView bv = stage_block(sorted, blk, b, mk, cols, n);   // includes a barrier

    uint4 breg[kSpw];
    auto load_b = [&](int s) {
#pragma unroll
      for (int u = 0; u < kSpw; ++u) {
        const int idx = threadIdx.x + kThreads * u;
        const int col = idx / kChunks, ch = idx - col * kChunks;
        const int t = toks[col];
        breg[u] = t >= 0 ? *reinterpret_cast<const uint4*>(x + static_cast<size_t>(t) * H + s * kSlab + ch * 8)
                         : make_uint4(0, 0, 0, 0);
      }
    };
    auto store_b = [&](int buf) {
#pragma unroll
      for (int u = 0; u < kSpw; ++u) {
        const int idx = threadIdx.x + kThreads * u;
        const int col = idx / kChunks, ch = idx - col * kChunks;
        *reinterpret_cast<uint4*>(&bs[buf][col * kRowB + ch * 16]) = breg[u];
      }
    };

    floatx4 accg[kMaxSub], accu[kMaxSub];
#pragma unroll
    for (int st = 0; st < kMaxSub; ++st) { accg[st] = floatx4{0, 0, 0, 0}; accu[st] = floatx4{0, 0, 0, 0}; }

    load_b(0);
    store_b(0);
    __syncthreads();
    const int lg = wave * 16 + n;               // local row of this lane's A operand
    for (int s0 = 0; s0 < nslab; s0 += kDepth) {
#pragma unroll
      for (int d = 0; d < kDepth; ++d) {
        const int s = s0 + d;
        if (s >= nslab) break;
        const int cur = s & 1;
        const int grp = (s * kSlab) / g;
        bf16x8 Ag[kSpw], Au[kSpw];
#pragma unroll
        for (int j = 0; j < kSpw; ++j) { Ag[j] = bias_pairs(wg[d][j]); Au[j] = bias_pairs(wu[d][j]); }
        // Activation loads before the weight-ring loads: the wait before
        // store_b then leaves the (later) weight loads in flight.
        if (s + 1 < nslab) load_b(s + 1);
        if (s + kDepth < nslab) {
          load_words<kSpw>(qg + (s + kDepth) * 4 * kSpw, wg[d]);
          load_words<kSpw>(qu + (s + kDepth) * 4 * kSpw, wu[d]);
        }
        const bf16x8 Zg = neg_zero_pairs(szz[lg * gpr + grp]);
        const bf16x8 Zu = neg_zero_pairs(szz[(kTileRows + lg) * gpr + grp]);
        float cg[4], cu[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          cg[i] = half_bits_to_float(ssh[(wave * 16 + 4 * lq + i) * gpr + grp]);
          cu[i] = half_bits_to_float(ssh[(kTileRows + wave * 16 + 4 * lq + i) * gpr + grp]);
        }
#pragma unroll
        for (int st = 0; st < kMaxSub; ++st) {
          if (!bv.act[st]) continue;
          const unsigned char* brow = &bs[cur][(16 * st + n) * kRowB + 16 * kSpw * lq];
          floatx4 dg = {0, 0, 0, 0}, du = {0, 0, 0, 0};
#pragma unroll
          for (int j = 0; j < kSpw; ++j) {
            const bf16x8 B = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(brow + 16 * j));
            dg = mfma_bf16(Ag[j], B, dg);
            dg = mfma_bf16(Zg, B, dg);
            du = mfma_bf16(Au[j], B, du);
            du = mfma_bf16(Zu, B, du);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            accg[st][i] = fmaf(cg[i], dg[i], accg[st][i]);
            accu[st][i] = fmaf(cu[i], du[i], accu[st][i]);
          }
        }
        if (s + 1 < nslab) store_b(cur ^ 1);
        __syncthreads();
      }
    }
#pragma unroll
    for (int st = 0; st < kMaxSub; ++st) {
      const int r = bv.rid[st];
      if (r < 0) continue;
      uint32_t hi2[2], lo2[2];
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        const float v0 = silu_mul(accg[st][i], accu[st][i]);
        const float v1 = silu_mul(accg[st][i + 1], accu[st][i + 1]);
        const bf16x2 h = {static_cast<__bf16>(v0), static_cast<__bf16>(v1)};
        const uint32_t hb = __builtin_bit_cast(uint32_t, h);
        const bf16x2 l = {static_cast<__bf16>(v0 - bf16_lo(hb)), static_cast<__bf16>(v1 - bf16_hi(hb))};
        hi2[i / 2] = hb;
        lo2[i / 2] = __builtin_bit_cast(uint32_t, l);
      }
      const size_t off = static_cast<size_t>(r) * I + ng * kTileRows + wave * 16 + 4 * lq;
      *reinterpret_cast<uint2*>(a_hi + off) = make_uint2(hi2[0], hi2[1]);
      *reinterpret_cast<uint2*>(a_lo + off) = make_uint2(lo2[0], lo2[1]);
    }
  }
}

template <int kSpw>
__global__ __launch_bounds__(kThreads) void grouped_down_int4(
    const uint16_t* __restrict__ a_hi, const uint16_t* __restrict__ a_lo,
    const int32_t* __restrict__ sorted, const int32_t* __restrict__ blocks,
    const int32_t* __restrict__ num_padded, const uint32_t* __restrict__ q,
    const uint16_t* __restrict__ sc, const uint8_t* __restrict__ zp, float* __restrict__ yhat,
    int mk, int E, int H, int I, int g, int b, int nblk) {
  constexpr int kSlab = 32 * kSpw;
  constexpr int kRowB = kSlab * 2 + 16;
  constexpr int kChunks = kSlab / 8;
  constexpr int kLoads = 2 * kSpw;               // hi and lo planes
  constexpr int kMaxGroups = 64;
  constexpr int kDepth = ring_depth<kSpw>();
  __shared__ __align__(16) unsigned char bs[2][2][kMaxTok * kRowB];
  __shared__ uint16_t ssh[kTileRows * kMaxGroups / 2];
  __shared__ uint8_t szz[kTileRows * kMaxGroups / 2];
  __shared__ int cols[kMaxTok];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int n = lane & 15, lq = lane >> 4;
  const int ngroups = H / kTileRows;
  const int ntasks = nblk * ngroups;
  const int npad = num_padded[0];
  const int words = I >> 3, gpr = I / g;
  const int nslab = I / kSlab;

  for (int task = blockIdx.x; task < ntasks; task += gridDim.x) {
    const int blk = task / ngroups;
    const int ng = task - blk * ngroups;
    if (blk * b >= npad) continue;
    const int e = blocks[blk];
    if (e < 0 || e >= E) continue;

    const size_t tile0 = static_cast<size_t>(e) * H + ng * kTileRows;
    const size_t row0 = tile0 + wave * 16;
    const uint32_t* qa = q + (row0 + n) * words + kSpw * lq;
    uint32_t wa[kDepth][kSpw];
#pragma unroll
    for (int d = 0; d < kDepth; ++d)
      if (d < nslab) load_words<kSpw>(qa + d * 4 * kSpw, wa[d]);
    for (int v = threadIdx.x; v < kTileRows * gpr; v += kThreads) {
      ssh[v] = sc[tile0 * gpr + v];
      szz[v] = zp[tile0 * gpr + v];
    }
    const BlockView bv = stage_block(sorted, blk, b, mk, cols, n);   // includes a barrier

    uint4 breg[kLoads];
    auto load_b = [&](int s) {
#pragma unroll
      for (int u = 0; u < kLoads; ++u) {
        const int idx = threadIdx.x + kThreads * (u >> 1);
        const int col = idx / kChunks, ch = idx - col * kChunks;
        const int r = cols[col];
        const uint16_t* src = (u & 1) ? a_lo : a_hi;
        breg[u] = r >= 0 ? *reinterpret_cast<const uint4*>(src + static_cast<size_t>(r) * I + s * kSlab + ch * 8)
                         : make_uint4(0, 0, 0, 0);
      }
    };
    auto store_b = [&](int buf) {
#pragma unroll
      for (int u = 0; u < kLoads; ++u) {
        const int idx = threadIdx.x + kThreads * (u >> 1);
        const int col = idx / kChunks, ch = idx - col * kChunks;
        *reinterpret_cast<uint4*>(&bs[buf][u & 1][col * kRowB + ch * 16]) = breg[u];
      }
    };

    floatx4 acc[kMaxSub];
#pragma unroll
    for (int st = 0; st < kMaxSub; ++st) acc[st] = floatx4{0, 0, 0, 0};

    load_b(0);
    store_b(0);
    __syncthreads();
    const int la = wave * 16 + n;
    for (int s0 = 0; s0 < nslab; s0 += kDepth) {
#pragma unroll
      for (int d = 0; d < kDepth; ++d) {
        const int s = s0 + d;
        if (s >= nslab) break;
        const int cur = s & 1;
        const int grp = (s * kSlab) / g;
        const float za = static_cast<float>(szz[la * gpr + grp]);
        bf16x8 A[kSpw];
#pragma unroll
        for (int j = 0; j < kSpw; ++j) A[j] = dequant8_exact(wa[d][j], za);
        if (s + 1 < nslab) load_b(s + 1);
        if (s + kDepth < nslab) load_words<kSpw>(qa + (s + kDepth) * 4 * kSpw, wa[d]);
        float cs[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) cs[i] = half_bits_to_float(ssh[(wave * 16 + 4 * lq + i) * gpr + grp]);
#pragma unroll
        for (int st = 0; st < kMaxSub; ++st) {
          if (!bv.act[st]) continue;
          const int boff = (16 * st + n) * kRowB + 16 * kSpw * lq;
          floatx4 dd = {0, 0, 0, 0};
#pragma unroll
          for (int j = 0; j < kSpw; ++j) {
            const bf16x8 Bh = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&bs[cur][0][boff + 16 * j]));
            const bf16x8 Bl = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&bs[cur][1][boff + 16 * j]));
            dd = mfma_bf16(A[j], Bh, dd);
            dd = mfma_bf16(A[j], Bl, dd);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[st][i] = fmaf(cs[i], dd[i], acc[st][i]);
        }
        if (s + 1 < nslab) store_b(cur ^ 1);
        __syncthreads();
      }
    }
#pragma unroll
    for (int st = 0; st < kMaxSub; ++st) {
      const int r = bv.rid[st];
      if (r < 0) continue;
      *reinterpret_cast<float4*>(yhat + static_cast<size_t>(r) * H + ng * kTileRows + wave * 16 + 4 * lq) =
          make_float4(acc[st][0], acc[st][1], acc[st][2], acc[st][3]);
    }
  }
}

__global__ __launch_bounds__(kThreads) void combine_topk(
    const float* __restrict__ yhat, const int32_t* __restrict__ ids,
    const float* __restrict__ topk_w, float* __restrict__ y, int M, int k, int E, int H) {
  const int quads = H >> 2;
  const int total = M * quads;
  for (int i = blockIdx.x * kThreads + threadIdx.x; i < total; i += gridDim.x * kThreads) {
    const int t = i / quads;
    const int h = (i - t * quads) << 2;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
      const int r = t * k + j;
      const int e = ids[r];
      if (e < 0 || e >= E) continue;
      const float w = topk_w[r];
      const float4 v = *reinterpret_cast<const float4*>(yhat + static_cast<size_t>(r) * H + h);
      acc.x = fmaf(w, v.x, acc.x);
      acc.y = fmaf(w, v.y, acc.y);
      acc.z = fmaf(w, v.z, acc.z);
      acc.w = fmaf(w, v.w, acc.w);
    }
    *reinterpret_cast<float4*>(y + static_cast<size_t>(t) * H + h) = acc;
  }
}

int grid_for(int work_groups, int max_workgroups) {
  if (work_groups < 1) work_groups = 1;
  return (max_workgroups > 0 && max_workgroups < work_groups) ? max_workgroups : work_groups;
}

int slab_words(int K, int g, int max_spw) {
  // Largest of 4, 2, 1 words per lane (slabs of 128, 64, 32 elements), at
  // most max_spw, such that a slab stays inside one group and K is a whole
  // number of slabs.
  for (int spw = max_spw; spw >= 1; spw >>= 1) {
    const int slab = 32 * spw;
    if (g % slab == 0 && K % slab == 0) return spw;
  }
  return 0;
}

// The down kernel stages two planes, so its slab is at most 64 elements to
// keep the double-buffered LDS tile small.
#ifndef MOE_GATE_UP_MAX_SPW
#define MOE_GATE_UP_MAX_SPW 4
#endif
constexpr int kGateUpMaxSpw = MOE_GATE_UP_MAX_SPW;
constexpr int kDownMaxSpw = 2;

}  // namespace

bool grouped_shape_ok(int H, int I, int b, int g13, int g2) {
  // The scale/zero tiles of a workgroup live in LDS: at most 16 groups per
  // row for W13 and 32 for W2.
  return b >= 1 && b <= kMaxTok && (I % kTileRows) == 0 && (H % kTileRows) == 0 &&
         slab_words(H, g13, kGateUpMaxSpw) > 0 && slab_words(I, g2, kDownMaxSpw) > 0 &&
         H / g13 <= 16 && I / g2 <= 32;
}

hipError_t launch_grouped_gate_up(const GroupedArgs& p, hipStream_t stream) {
  const int ntasks = p.nblk * (p.I / kTileRows);
  const int wgs = grid_for(ntasks, p.max_workgroups);
  const auto* q = static_cast<const uint32_t*>(p.w13.q);
  const auto* s = static_cast<const uint16_t*>(p.w13.scale);
  const int mk = p.M * p.k;
  switch (slab_words(p.H, p.w13.group, kGateUpMaxSpw)) {
    case 4:
      hipLaunchKernelGGL(grouped_gate_up_int4<4>, dim3(wgs), dim3(kThreads), 0, stream, p.x, p.sorted,
                         p.blocks, p.num_padded, q, s, p.w13.zero, p.a_hi, p.a_lo, mk, p.k, p.E, p.H,
                         p.I, p.w13.group, p.b, p.nblk);
      break;
    case 2:
      hipLaunchKernelGGL(grouped_gate_up_int4<2>, dim3(wgs), dim3(kThreads), 0, stream, p.x, p.sorted,
                         p.blocks, p.num_padded, q, s, p.w13.zero, p.a_hi, p.a_lo, mk, p.k, p.E, p.H,
                         p.I, p.w13.group, p.b, p.nblk);
      break;
    default:
      hipLaunchKernelGGL(grouped_gate_up_int4<1>, dim3(wgs), dim3(kThreads), 0, stream, p.x, p.sorted,
                         p.blocks, p.num_padded, q, s, p.w13.zero, p.a_hi, p.a_lo, mk, p.k, p.E, p.H,
                         p.I, p.w13.group, p.b, p.nblk);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_grouped_down(const GroupedArgs& p, hipStream_t stream) {
  const int ntasks = p.nblk * (p.H / kTileRows);
  const int wgs = grid_for(ntasks, p.max_workgroups);
  const auto* q = static_cast<const uint32_t*>(p.w2.q);
  const auto* s = static_cast<const uint16_t*>(p.w2.scale);
  const int mk = p.M * p.k;
  switch (slab_words(p.I, p.w2.group, kDownMaxSpw)) {
    case 2:
      hipLaunchKernelGGL(grouped_down_int4<2>, dim3(wgs), dim3(kThreads), 0, stream, p.a_hi, p.a_lo,
                         p.sorted, p.blocks, p.num_padded, q, s, p.w2.zero, p.yhat, mk, p.E, p.H,
                         p.I, p.w2.group, p.b, p.nblk);
      break;
    default:
      hipLaunchKernelGGL(grouped_down_int4<1>, dim3(wgs), dim3(kThreads), 0, stream, p.a_hi, p.a_lo,
                         p.sorted, p.blocks, p.num_padded, q, s, p.w2.zero, p.yhat, mk, p.E, p.H,
                         p.I, p.w2.group, p.b, p.nblk);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_combine(const GroupedArgs& p, hipStream_t stream) {
  const int total = p.M * (p.H / 4);
  const int wgs = grid_for((total + kThreads - 1) / kThreads, p.max_workgroups);
  hipLaunchKernelGGL(combine_topk, dim3(wgs), dim3(kThreads), 0, stream, p.yhat, p.ids, p.topk_w,
                     p.y, p.M, p.k, p.E, p.H);
  return hipGetLastError();
}

}  // namespace moe
