// Grouped path: expert-centric bf16 MFMA GEMMs over the aligned rows, for
// batches large enough that tokens share experts (the warp-decode write-up,
// last section: expert-centric packing stays better for prefill and large
// batches; "Hardware-Native Joint Sparse-Quantization for Trillion-Scale MoE",
// Section 3.4: grouped GEMM over routing-dependent token counts, weights as
// the left operand so Y_e^T = W_e X_e^T).
//
// Both GEMMs put the expert's weight rows on the MFMA A operand and the
// block's tokens (16 per sub-tile) on B, with v_mfma_f32_16x16x32_bf16:
//   A lane l: weight row l%16, 8 reduction elements of lane group l/16;
//   B lane l: token column l%16, the same 8 reduction elements;
//   D lane l: rows 4*(l/16)+i (i < 4) of column l%16.
// A slab of 32*kSpw reduction elements lies inside one quantisation group;
// lane group q holds words kSpw*q .. kSpw*q+kSpw-1 of the slab (one 4*kSpw-byte
// load per lane and row), and MFMA step j of the slab uses word kSpw*q + j.
// Weights are dequantised exactly to bf16 (q - z is an integer in [-15, 15]),
// and each slab's fp32 partial is multiplied by the group scale before it is
// added to the accumulator, so the only rounding is fp32 accumulation.
//
// gate/up: one workgroup per (aligned block, 16 neurons); the four waves
//   split the reduction (H) into quarters and their partials are summed in
//   wave order through LDS. Each wave prefetches its next slab's weights and
//   activations while the current slab's MFMAs run. The epilogue writes
//   silu(gate)*up for every valid route of the block as a bf16 hi/lo pair
//   (a = hi + lo to within 2^-17 relative), ready to be the B operand of the
//   down GEMM.
// down: one workgroup per (aligned block, 16 hidden rows), the same K split;
//   B = the hi and lo planes of the intermediate (two MFMAs per step). Each
//   route's yhat row is written once.
// combine: y[t] = sum over j ascending of w[t,j] * yhat[t*k+j].
// Workgroups whose block lies past num_padded (read on the device) exit at
// once, so the grid can be sized from the host-known capacity.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxSub = 4;        // 16-token sub-tiles per block (b <= 64)

__device__ __forceinline__ floatx4 mfma_bf16(const bf16x8& a, const bf16x8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
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

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

// Columns of one aligned block: route IDs (or -1) for the four sub-tiles of
// lane column n, and which sub-tiles hold at least one valid route.
struct BlockCols {
  int rid[kMaxSub];
  bool any[kMaxSub];
};

__device__ __forceinline__ BlockCols load_block_cols(const int32_t* sorted, int blk, int b, int nst,
                                                     int mk, int n) {
  BlockCols bc;
#pragma unroll
  for (int st = 0; st < kMaxSub; ++st) {
    const int col = 16 * st + n;
    int r = -1;
    if (st < nst && col < b) {
      r = sorted[static_cast<size_t>(blk) * b + col];
      if (r < 0 || r >= mk) r = -1;
    }
    bc.rid[st] = r;
    bc.any[st] = __ballot(r >= 0) != 0ull;
  }
  return bc;
}

// Reduction across the four waves of a workgroup, in wave order, through
// LDS. `part` holds kWaves x nvals x 64 floats.
template <int kVals>
__device__ __forceinline__ void reduce_waves(float (&v)[kVals], float* part, int wave, int lane) {
  constexpr int kWaves = kThreads / kWave;
#pragma unroll
  for (int i = 0; i < kVals; ++i) part[(wave * kVals + i) * kWave + lane] = v[i];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < kVals; ++i) {
      float s = part[i * kWave + lane];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) s += part[(w * kVals + i) * kWave + lane];
      v[i] = s;
    }
  }
  __syncthreads();
}

// gate/up: workgroup = (aligned block, 16 neurons); wave w reduces over the
// w-th quarter of H. Per slab, the wave dequantises its gate and up words
// once and runs them against every active 16-token sub-tile.
template <int kSpw>
__global__ __launch_bounds__(kThreads) void grouped_gate_up_int4(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ sorted,
    const int32_t* __restrict__ blocks, const int32_t* __restrict__ num_padded,
    const uint32_t* __restrict__ q, const uint16_t* __restrict__ sc,
    const uint8_t* __restrict__ zp, uint16_t* __restrict__ a_hi, uint16_t* __restrict__ a_lo,
    int mk, int k, int E, int H, int I, int g, int b, int nblk) {
  constexpr int kWaves = kThreads / kWave;
  constexpr int kSlab = 32 * kSpw;
  constexpr int kVals = kMaxSub * 8;  // gate and up, 4 rows each, per sub-tile
  __shared__ float part[kWaves * kVals * kWave];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int n = lane & 15, lq = lane >> 4;
  const int ntiles = I / 16;
  const int ntasks = nblk * ntiles;
  const int npad = num_padded[0];
  const int nst = (b + 15) / 16;
  const int words = H >> 3, gpr = H / g;
  const int kq = H / kWaves;                 // reduction range of one wave
  const int nslab = kq / kSlab;

  for (int task = blockIdx.x; task < ntasks; task += gridDim.x) {
    const int blk = task / ntiles;
    const int nt = (task - blk * ntiles) * 16;
    if (blk * b >= npad) continue;
    const int e = blocks[blk];
    if (e < 0 || e >= E) continue;
    const BlockCols bc = load_block_cols(sorted, blk, b, nst, mk, n);
    int tok[kMaxSub];
#pragma unroll
    for (int st = 0; st < kMaxSub; ++st) tok[st] = bc.rid[st] >= 0 ? bc.rid[st] / k : 0;

    const size_t rowg = static_cast<size_t>(e) * (2 * I) + nt;  // first gate row of the tile
    const size_t rowu = rowg + I;                                 // first up row
    const int kbeg = wave * kq;
    const uint32_t* qg = q + (rowg + n) * words + (kbeg >> 3) + kSpw * lq;
    const uint32_t* qu = q + (rowu + n) * words + (kbeg >> 3) + kSpw * lq;

    floatx4 accg[kMaxSub], accu[kMaxSub];
#pragma unroll
    for (int st = 0; st < kMaxSub; ++st) { accg[st] = floatx4{0, 0, 0, 0}; accu[st] = floatx4{0, 0, 0, 0}; }

    // Prefetch: the first slab's weights and activations.
    uint32_t wg[kSpw], wu[kSpw];
    bf16x8 Bn[kMaxSub][kSpw];
#pragma unroll
    for (int j = 0; j < kSpw; ++j) { wg[j] = qg[j]; wu[j] = qu[j]; }
#pragma unroll
    for (int st = 0; st < kMaxSub; ++st) {
      if (!bc.any[st]) continue;
      const uint16_t* xp = x + static_cast<size_t>(tok[st]) * H + kbeg + 8 * kSpw * lq;
#pragma unroll
      for (int j = 0; j < kSpw; ++j) Bn[st][j] = load_bf16x8(xp + 8 * j);
    }
    for (int sl = 0; sl < nslab; ++sl) {
      const int k0 = kbeg + sl * kSlab;
      const int grp = k0 / g;
      const float zg = static_cast<float>(zp[(rowg + n) * gpr + grp]);
      const float zu = static_cast<float>(zp[(rowu + n) * gpr + grp]);
      float sg[4], su[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sg[i] = half_bits_to_float(sc[(rowg + 4 * lq + i) * gpr + grp]);
        su[i] = half_bits_to_float(sc[(rowu + 4 * lq + i) * gpr + grp]);
      }
      bf16x8 Ag[kSpw], Au[kSpw], B[kMaxSub][kSpw];
#pragma unroll
      for (int j = 0; j < kSpw; ++j) { Ag[j] = dequant8_exact(wg[j], zg); Au[j] = dequant8_exact(wu[j], zu); }
#pragma unroll
      for (int st = 0; st < kMaxSub; ++st)
#pragma unroll
        for (int j = 0; j < kSpw; ++j) B[st][j] = Bn[st][j];
      if (sl + 1 < nslab) {   // next slab's loads overlap this slab's MFMAs
        const int w1 = (sl + 1) * kSpw * 4;
#pragma unroll
        for (int j = 0; j < kSpw; ++j) { wg[j] = qg[w1 + j]; wu[j] = qu[w1 + j]; }
#pragma unroll
        for (int st = 0; st < kMaxSub; ++st) {
          if (!bc.any[st]) continue;
          const uint16_t* xp = x + static_cast<size_t>(tok[st]) * H + k0 + kSlab + 8 * kSpw * lq;
#pragma unroll
          for (int j = 0; j < kSpw; ++j) Bn[st][j] = load_bf16x8(xp + 8 * j);
        }
      }
#pragma unroll
      for (int st = 0; st < kMaxSub; ++st) {
        if (!bc.any[st]) continue;
        floatx4 dg = {0, 0, 0, 0}, du = {0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < kSpw; ++j) {
          dg = mfma_bf16(Ag[j], B[st][j], dg);
          du = mfma_bf16(Au[j], B[st][j], du);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          accg[st][i] = fmaf(sg[i], dg[i], accg[st][i]);
          accu[st][i] = fmaf(su[i], du[i], accu[st][i]);
        }
      }
    }
    float v[kVals];
#pragma unroll
    for (int st = 0; st < kMaxSub; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) { v[st * 8 + i] = accg[st][i]; v[st * 8 + 4 + i] = accu[st][i]; }
    reduce_waves(v, part, wave, lane);
    if (wave == 0) {
#pragma unroll
      for (int st = 0; st < kMaxSub; ++st) {
        const int r = bc.rid[st];
        if (r < 0) continue;
        uint32_t hi2[2], lo2[2];
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          const float v0 = silu_mul(v[st * 8 + i], v[st * 8 + 4 + i]);
          const float v1 = silu_mul(v[st * 8 + i + 1], v[st * 8 + 4 + i + 1]);
          const bf16x2 h = {static_cast<__bf16>(v0), static_cast<__bf16>(v1)};
          const uint32_t hb = __builtin_bit_cast(uint32_t, h);
          const bf16x2 l = {static_cast<__bf16>(v0 - bf16_lo(hb)), static_cast<__bf16>(v1 - bf16_hi(hb))};
          hi2[i / 2] = hb;
          lo2[i / 2] = __builtin_bit_cast(uint32_t, l);
        }
        const size_t off = static_cast<size_t>(r) * I + nt + 4 * lq;
        *reinterpret_cast<uint2*>(a_hi + off) = make_uint2(hi2[0], hi2[1]);
        *reinterpret_cast<uint2*>(a_lo + off) = make_uint2(lo2[0], lo2[1]);
      }
    }
  }
}

// down: workgroup = (aligned block, 16 hidden rows); wave w reduces over the
// w-th quarter of I; B is the hi and lo planes of the intermediate.
template <int kSpw>
__global__ __launch_bounds__(kThreads) void grouped_down_int4(
    const uint16_t* __restrict__ a_hi, const uint16_t* __restrict__ a_lo,
    const int32_t* __restrict__ sorted, const int32_t* __restrict__ blocks,
    const int32_t* __restrict__ num_padded, const uint32_t* __restrict__ q,
    const uint16_t* __restrict__ sc, const uint8_t* __restrict__ zp, float* __restrict__ yhat,
    int mk, int E, int H, int I, int g, int b, int nblk) {
  constexpr int kWaves = kThreads / kWave;
  constexpr int kSlab = 32 * kSpw;
  constexpr int kVals = kMaxSub * 4;
  __shared__ float part[kWaves * kVals * kWave];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int n = lane & 15, lq = lane >> 4;
  const int ntiles = H / 16;
  const int ntasks = nblk * ntiles;
  const int npad = num_padded[0];
  const int nst = (b + 15) / 16;
  const int words = I >> 3, gpr = I / g;
  const int kq = I / kWaves;
  const int nslab = kq / kSlab;

  for (int task = blockIdx.x; task < ntasks; task += gridDim.x) {
    const int blk = task / ntiles;
    const int h0 = (task - blk * ntiles) * 16;
    if (blk * b >= npad) continue;
    const int e = blocks[blk];
    if (e < 0 || e >= E) continue;
    const BlockCols bc = load_block_cols(sorted, blk, b, nst, mk, n);
    int src[kMaxSub];
#pragma unroll
    for (int st = 0; st < kMaxSub; ++st) src[st] = bc.rid[st] >= 0 ? bc.rid[st] : 0;

    const size_t row0 = static_cast<size_t>(e) * H + h0;
    const int kbeg = wave * kq;
    const uint32_t* qa = q + (row0 + n) * words + (kbeg >> 3) + kSpw * lq;
    floatx4 acc[kMaxSub];
#pragma unroll
    for (int st = 0; st < kMaxSub; ++st) acc[st] = floatx4{0, 0, 0, 0};

    uint32_t wa[kSpw];
    bf16x8 Hn[kMaxSub][kSpw], Ln[kMaxSub][kSpw];
#pragma unroll
    for (int j = 0; j < kSpw; ++j) wa[j] = qa[j];
#pragma unroll
    for (int st = 0; st < kMaxSub; ++st) {
      if (!bc.any[st]) continue;
      const size_t boff = static_cast<size_t>(src[st]) * I + kbeg + 8 * kSpw * lq;
#pragma unroll
      for (int j = 0; j < kSpw; ++j) {
        Hn[st][j] = load_bf16x8(a_hi + boff + 8 * j);
        Ln[st][j] = load_bf16x8(a_lo + boff + 8 * j);
      }
    }
    for (int sl = 0; sl < nslab; ++sl) {
      const int k0 = kbeg + sl * kSlab;
      const int grp = k0 / g;
      const float za = static_cast<float>(zp[(row0 + n) * gpr + grp]);
      float sa[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) sa[i] = half_bits_to_float(sc[(row0 + 4 * lq + i) * gpr + grp]);
      bf16x8 A[kSpw], Bh[kMaxSub][kSpw], Bl[kMaxSub][kSpw];
#pragma unroll
      for (int j = 0; j < kSpw; ++j) A[j] = dequant8_exact(wa[j], za);
#pragma unroll
      for (int st = 0; st < kMaxSub; ++st)
#pragma unroll
        for (int j = 0; j < kSpw; ++j) { Bh[st][j] = Hn[st][j]; Bl[st][j] = Ln[st][j]; }
      if (sl + 1 < nslab) {
        const int w1 = (sl + 1) * kSpw * 4;
#pragma unroll
        for (int j = 0; j < kSpw; ++j) wa[j] = qa[w1 + j];
#pragma unroll
        for (int st = 0; st < kMaxSub; ++st) {
          if (!bc.any[st]) continue;
          const size_t boff = static_cast<size_t>(src[st]) * I + k0 + kSlab + 8 * kSpw * lq;
#pragma unroll
          for (int j = 0; j < kSpw; ++j) {
            Hn[st][j] = load_bf16x8(a_hi + boff + 8 * j);
            Ln[st][j] = load_bf16x8(a_lo + boff + 8 * j);
          }
        }
      }
#pragma unroll
      for (int st = 0; st < kMaxSub; ++st) {
        if (!bc.any[st]) continue;
        floatx4 d = {0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < kSpw; ++j) {
          d = mfma_bf16(A[j], Bh[st][j], d);
          d = mfma_bf16(A[j], Bl[st][j], d);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[st][i] = fmaf(sa[i], d[i], acc[st][i]);
      }
    }
    float v[kVals];
#pragma unroll
    for (int st = 0; st < kMaxSub; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) v[st * 4 + i] = acc[st][i];
    reduce_waves(v, part, wave, lane);
    if (wave == 0) {
#pragma unroll
      for (int st = 0; st < kMaxSub; ++st) {
        const int r = bc.rid[st];
        if (r < 0) continue;
        *reinterpret_cast<float4*>(yhat + static_cast<size_t>(r) * H + h0 + 4 * lq) =
            make_float4(v[st * 4], v[st * 4 + 1], v[st * 4 + 2], v[st * 4 + 3]);
      }
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

int slab_words(int K, int g) {
  // Largest of 2, 1 words per lane (slabs of 64, 32 elements) such that a
  // slab stays inside one group and each wave's quarter of K is a whole
  // number of slabs. (Four words per lane would double the prefetched
  // activation registers and halve occupancy.)
  for (int spw = 2; spw >= 1; spw >>= 1) {
    const int slab = 32 * spw;
    if (g % slab == 0 && K % (4 * slab) == 0) return spw;
  }
  return 0;
}

}  // namespace

bool grouped_shape_ok(int H, int I, int b, int g13, int g2) {
  return b >= 1 && b <= 16 * kMaxSub && (I % 16) == 0 && (H % 16) == 0 &&
         slab_words(H, g13) > 0 && slab_words(I, g2) > 0;
}

hipError_t launch_grouped_gate_up(const GroupedArgs& p, hipStream_t stream) {
  const int ntasks = p.nblk * (p.I / 16);
  const int wgs = grid_for(ntasks, p.max_workgroups);
  const auto* q = static_cast<const uint32_t*>(p.w13.q);
  const auto* s = static_cast<const uint16_t*>(p.w13.scale);
  const int mk = p.M * p.k;
  switch (slab_words(p.H, p.w13.group)) {
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
  const int ntasks = p.nblk * (p.H / 16);
  const int wgs = grid_for(ntasks, p.max_workgroups);
  const auto* q = static_cast<const uint32_t*>(p.w2.q);
  const auto* s = static_cast<const uint16_t*>(p.w2.scale);
  const int mk = p.M * p.k;
  switch (slab_words(p.I, p.w2.group)) {
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
