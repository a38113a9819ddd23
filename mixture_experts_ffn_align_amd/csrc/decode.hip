// Decode path: output-stationary expert FFN for small batches (the
// warp-decode write-up, "Qué cambiamos" and "Cómo funcionan los dos kernels").
//
// No alignment, gather, scatter or per-expert output buffer: each wave64 owns
// a fixed set of outputs, streams exactly the packed weight rows they need
// from HBM, reduces across its lanes in a fixed order, and writes each output
// once.
//
// Kernel 1 (gate/up): a wave owns kNpw intermediate neurons of one route
//   (token t, expert e) and streams their gate and up rows, lane l covering
//   the 32-element chunks c = l, l+64, ... of the reduction (H); waves are
//   independent (no workgroup barrier), so each computes as soon as its own
//   loads land. Weights are unpacked to bf16 (128 + q) pairs and
//   multiplied with the bf16 activation pairs by v_dot2c_f32_bf16 (exact
//   products, fp32 sums); per chunk the bias and zero point are removed in
//   fp32: s * (sum x(128+q) - (128+z) sum x). A DPP butterfly reduces each
//   row; silu(gate) * up goes to the intermediate as a bf16 hi/lo pair
//   (a = hi + lo to within 2^-17 relative).
// Kernel 2 (down + combine): a workgroup owns kDownRows hidden outputs of
//   one token; wave w streams the down rows of routes j = w, w+8, ... and
//   folds the routing weight into its fp32 accumulators. The token's
//   intermediate rows (hi and lo planes) and the tile's scales and zeros are
//   staged in LDS; the weights are again bf16 (128 + q) pairs and each pair
//   is dotted with the hi and the lo plane.
//   Lanes of a wave form slots of pow2(I/32) lanes; a slot owns some of the
//   rows and its lanes cover the I/32 chunks. The eight wave partials are
//   added in wave (= route) order and y is written once. No floating-point
//   atomics anywhere.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kGateUpThreads = 256;
constexpr int kGateUpWaves = kGateUpThreads / kWave;
constexpr int kNpw = 2;                       // neurons per wave
constexpr int kDownWaves = 8;
constexpr int kDownThreads = kDownWaves * kWave;
constexpr int kDownRows = 8;
constexpr size_t kMaxDownLds = 48 * 1024;     // staged intermediate rows + scales + zeros
constexpr int kMaxGroups = 32;                // scale groups per row held in LDS (K / g)

template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}

// Sum over the 64 lanes of a wave, the same bits in every lane: butterflies
// inside each 16-lane row with DPP (xor 1, xor 2, half-row mirror, row
// mirror), then the four row sums added as (r0 + r1) + (r2 + r3).
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror
  v += dpp<0x140>(v);  // row_mirror
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

__global__ __launch_bounds__(kGateUpThreads) void decode_gate_up_int4(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ ids,
    const uint32_t* __restrict__ q, const uint16_t* __restrict__ sc,
    const uint8_t* __restrict__ zp, uint16_t* __restrict__ a_hi, uint16_t* __restrict__ a_lo,
    int mk, int k, int E, int H, int I, int g_shift) {
  __shared__ float2 wsz[kGateUpWaves][2 * kNpw * kMaxGroups];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave_l = uniform(threadIdx.x / kWave);
  // Task indices are wave-uniform: keep them (and the row addresses) scalar.
  const int wave_id = uniform(blockIdx.x * kGateUpWaves + threadIdx.x / kWave);
  const int nwaves = gridDim.x * kGateUpWaves;
  const int tasks_per_route = I / kNpw;
  const int ntasks = mk * tasks_per_route;
  const int nch = H >> 5, words = H >> 3, gpr = H >> g_shift;
  const uint32_t nib_mask = in_vgpr(0x000F000Fu);

  for (int task = wave_id; task < ntasks; task += nwaves) {
    const int r = task / tasks_per_route;
    const int i0 = (task - r * tasks_per_route) * kNpw;
    const int e = uniform(load_expert(ids, r, E));
    if (e < 0) {
      if (lane < kNpw) {
        a_hi[static_cast<size_t>(r) * I + i0 + lane] = 0;
        a_lo[static_cast<size_t>(r) * I + i0 + lane] = 0;
      }
      continue;
    }
    const int t = r / k;
    const size_t row0 = static_cast<size_t>(e) * (2 * I) + i0;  // first gate row
    const uint32_t* qrow[2 * kNpw];
    const uint16_t* srow[2 * kNpw];
    const uint8_t* zrow[2 * kNpw];
#pragma unroll
    for (int j = 0; j < 2 * kNpw; ++j) {
      const size_t row = row0 + (j < kNpw ? j : I + j - kNpw);
      qrow[j] = q + row * words;
      srow[j] = sc + row * gpr;
      zrow[j] = zp + row * gpr;
    }
    float acc[2 * kNpw];
#pragma unroll
    for (int j = 0; j < 2 * kNpw; ++j) acc[j] = 0.0f;
    // The rows' scales and zeros: one coalesced load per lane into this
    // wave's LDS slice (a wave reads back only what it wrote, so no barrier).
    for (int v = lane; v < 2 * kNpw * gpr; v += kWave) {
      const int j = v / gpr, gi = v - j * gpr;
      wsz[wave_l][v] = make_float2(half_bits_to_float(srow[j][gi]), 128.0f + static_cast<float>(zrow[j][gi]));
    }
    const uint4* xrow = reinterpret_cast<const uint4*>(x + static_cast<size_t>(t) * H);
    for (int c = lane; c < nch; c += kWave) {
      // Issue the weight loads first so they are all in flight together.
      uint4 wv[2 * kNpw];
      float s[2 * kNpw], zb[2 * kNpw];
      const int grp = (c << 5) >> g_shift;
#pragma unroll
      for (int j = 0; j < 2 * kNpw; ++j) wv[j] = load_stream16(qrow[j] + 4 * c);
#pragma unroll
      for (int j = 0; j < 2 * kNpw; ++j) {
        const float2 sz = wsz[wave_l][j * gpr + grp];
        s[j] = sz.x;
        zb[j] = sz.y;
      }
      uint32_t xw[16];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint4 t4 = xrow[c * 4 + v];
        xw[4 * v] = t4.x; xw[4 * v + 1] = t4.y; xw[4 * v + 2] = t4.z; xw[4 * v + 3] = t4.w;
      }
      float sx = 0.0f;
#pragma unroll
      for (int v = 0; v < 16; ++v) sx = dot2_bf16(xw[v], 0x3F803F80u, sx);  // (1.0, 1.0)
#pragma unroll
      for (int j = 0; j < 2 * kNpw; ++j) {
        const uint32_t w4[4] = {wv[j].x, wv[j].y, wv[j].z, wv[j].w};
        float d = 0.0f;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          uint32_t p[4];
          unpack8_bias128_m(w4[v], nib_mask, p);
#pragma unroll
          for (int i = 0; i < 4; ++i) d = dot2_bf16(p[i], xw[4 * v + i], d);
        }
        acc[j] = fmaf(s[j], fmaf(-zb[j], sx, d), acc[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < 2 * kNpw; ++j) acc[j] = wave_sum_dpp(acc[j]);
    float gv = acc[0], uv = acc[kNpw];
#pragma unroll
    for (int j = 1; j < kNpw; ++j) {
      if (lane == j) { gv = acc[j]; uv = acc[kNpw + j]; }
    }
    if (lane < kNpw) {
      const float v = silu_mul(gv, uv);
      const __bf16 h = static_cast<__bf16>(v);
      const size_t off = static_cast<size_t>(r) * I + i0 + lane;
      a_hi[off] = __builtin_bit_cast(uint16_t, h);
      a_lo[off] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v - static_cast<float>(h)));
    }
  }
}

// kRps: rows per lane, ceil(kDownRows / slots); kKpw: routes per wave.
template <int kKpw, int kRps>
__global__ __launch_bounds__(kDownThreads) void decode_down_int4(
    const uint16_t* __restrict__ a_hi, const uint16_t* __restrict__ a_lo,
    const int32_t* __restrict__ ids, const float* __restrict__ topk_w,
    const uint32_t* __restrict__ q, const uint16_t* __restrict__ sc,
    const uint8_t* __restrict__ zp, float* __restrict__ y, int M, int k, int E, int H, int I,
    int g_shift) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int gpr = I >> g_shift;
  uint16_t* ah = reinterpret_cast<uint16_t*>(lds);                          // [k][I] hi plane
  uint16_t* al = ah + static_cast<size_t>(k) * I;                           // [k][I] lo plane
  float* ss = reinterpret_cast<float*>(al + static_cast<size_t>(k) * I);    // [k][kDownRows][gpr]
  float* zs = ss + k * kDownRows * gpr;                                     // 128 + zero
  __shared__ float part[kDownWaves][kDownRows];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = uniform(threadIdx.x / kWave);
  const int tiles_per_tok = H / kDownRows;
  const int ntiles = M * tiles_per_tok;
  const int nch = I >> 5, words = I >> 3;
  int span = 1;
  while (span < nch && span < kWave) span <<= 1;
  const int slots = kWave / span;
  const int slot = lane / span;
  const int c0 = lane - slot * span;
  const uint32_t nib_mask = in_vgpr(0x000F000Fu);

  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int t = tile / tiles_per_tok;
    const int h0 = (tile - t * tiles_per_tok) * kDownRows;
    int ex[kKpw];
    float wr[kKpw];
#pragma unroll
    for (int u = 0; u < kKpw; ++u) {
      const int j = wave + kDownWaves * u;
      ex[u] = j < k ? uniform(load_expert(ids, t * k + j, E)) : -1;
      wr[u] = j < k ? topk_w[t * k + j] : 0.0f;
    }
    // Weight loads of this wave's routes (two chunks per lane at most).
    constexpr int kMaxCh = 2;
    uint4 wv[kKpw][kMaxCh][kRps];
#pragma unroll
    for (int u = 0; u < kKpw; ++u) {
      if (ex[u] < 0) continue;
      const uint32_t* qt = q + (static_cast<size_t>(ex[u]) * H + h0) * words;
#pragma unroll
      for (int cc = 0; cc < kMaxCh; ++cc) {
        const int c = c0 + cc * span;
        if (c >= nch) continue;
#pragma unroll
        for (int i = 0; i < kRps; ++i) {
          const int m = slot + i * slots;
          if (m < kDownRows) wv[u][cc][i] = load_stream16(qt + m * words + 4 * c);
        }
      }
    }
    // Stage the token's intermediate rows, and the tile's scales and zeros.
    const uint4* gh = reinterpret_cast<const uint4*>(a_hi + static_cast<size_t>(t) * k * I);
    const uint4* gl = reinterpret_cast<const uint4*>(a_lo + static_cast<size_t>(t) * k * I);
    for (int v = threadIdx.x; v < k * I / 8; v += kDownThreads) {
      reinterpret_cast<uint4*>(ah)[v] = gh[v];
      reinterpret_cast<uint4*>(al)[v] = gl[v];
    }
    // Each wave stages the scales and zeros of its own routes' rows (one
    // coalesced load per lane); it is the only reader of that slice.
#pragma unroll
    for (int u = 0; u < kKpw; ++u) {
      if (ex[u] < 0) continue;
      const int j = wave + kDownWaves * u;
      const size_t base = (static_cast<size_t>(ex[u]) * H + h0) * gpr;
      for (int v = lane; v < kDownRows * gpr; v += kWave) {
        ss[j * kDownRows * gpr + v] = half_bits_to_float(sc[base + v]);
        zs[j * kDownRows * gpr + v] = 128.0f + static_cast<float>(zp[base + v]);
      }
    }
    __syncthreads();

    float acc[kRps];
#pragma unroll
    for (int i = 0; i < kRps; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int u = 0; u < kKpw; ++u) {
      if (ex[u] < 0) continue;
      const int j = wave + kDownWaves * u;
#pragma unroll
      for (int cc = 0; cc < kMaxCh; ++cc) {
        const int c = c0 + cc * span;
        if (c >= nch) continue;
        const int grp = (c << 5) >> g_shift;
        uint32_t hw[16], lw[16];
        const uint4* hp = reinterpret_cast<const uint4*>(ah + static_cast<size_t>(j) * I + (c << 5));
        const uint4* lp = reinterpret_cast<const uint4*>(al + static_cast<size_t>(j) * I + (c << 5));
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint4 th = hp[v], tl = lp[v];
          hw[4 * v] = th.x; hw[4 * v + 1] = th.y; hw[4 * v + 2] = th.z; hw[4 * v + 3] = th.w;
          lw[4 * v] = tl.x; lw[4 * v + 1] = tl.y; lw[4 * v + 2] = tl.z; lw[4 * v + 3] = tl.w;
        }
        float sa = 0.0f;
#pragma unroll
        for (int v = 0; v < 16; ++v) sa = dot2_bf16(lw[v], 0x3F803F80u, dot2_bf16(hw[v], 0x3F803F80u, sa));
#pragma unroll
        for (int i = 0; i < kRps; ++i) {
          const int m = slot + i * slots;
          if (m < kDownRows) {
            const int si = (j * kDownRows + m) * gpr + grp;
            const uint32_t w4[4] = {wv[u][cc][i].x, wv[u][cc][i].y, wv[u][cc][i].z, wv[u][cc][i].w};
            float d = 0.0f;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              uint32_t p[4];
              unpack8_bias128_m(w4[v], nib_mask, p);
#pragma unroll
              for (int e8 = 0; e8 < 4; ++e8) {
                d = dot2_bf16(p[e8], hw[4 * v + e8], d);
                d = dot2_bf16(p[e8], lw[4 * v + e8], d);
              }
            }
            acc[i] = fmaf(wr[u] * ss[si], fmaf(-zs[si], sa, d), acc[i]);
          }
        }
      }
    }
    // Sum each row over the lanes of its slot (butterfly inside the span).
#pragma unroll
    for (int i = 0; i < kRps; ++i) {
      float v = acc[i];
      for (int o = span >> 1; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
      acc[i] = v;
    }
    if (c0 == 0) {
#pragma unroll
      for (int i = 0; i < kRps; ++i) {
        const int m = slot + i * slots;
        if (m < kDownRows) part[wave][m] = acc[i];
      }
    }
    __syncthreads();
    if (threadIdx.x < kDownRows) {
      float v = part[0][threadIdx.x];
      for (int w = 1; w < kDownWaves; ++w) v += part[w][threadIdx.x];
      y[static_cast<size_t>(t) * H + h0 + threadIdx.x] = v;
    }
    __syncthreads();
  }
}

int grid_for(int work_groups, int max_workgroups) {
  if (work_groups < 1) work_groups = 1;
  return (max_workgroups > 0 && max_workgroups < work_groups) ? max_workgroups : work_groups;
}

size_t down_lds(int I, int k, int g) {
  return sizeof(uint16_t) * 2 * static_cast<size_t>(k) * I +
         sizeof(float) * 2 * static_cast<size_t>(k) * kDownRows * (I / g);
}

int log2_of(int g) {
  int s = 0;
  while ((1 << s) < g) ++s;
  return s;
}

template <int kKpw, int kRps>
void launch_down(const DecodeArgs& p, int wgs, hipStream_t stream) {
  hipLaunchKernelGGL((decode_down_int4<kKpw, kRps>), dim3(wgs), dim3(kDownThreads),
                     down_lds(p.I, p.k, p.w2.group), stream, p.a_hi, p.a_lo, p.ids, p.topk_w,
                     static_cast<const uint32_t*>(p.w2.q), static_cast<const uint16_t*>(p.w2.scale),
                     p.w2.zero, p.y, p.M, p.k, p.E, p.H, p.I, log2_of(p.w2.group));
}

template <int kKpw>
void launch_down_rps(const DecodeArgs& p, int wgs, hipStream_t stream) {
  int nch = p.I >> 5, span = 1;
  while (span < nch && span < kWave) span <<= 1;
  const int slots = kWave / span;
  const int rps = (kDownRows + slots - 1) / slots;
  if (rps <= 1) launch_down<kKpw, 1>(p, wgs, stream);
  else if (rps <= 2) launch_down<kKpw, 2>(p, wgs, stream);
  else if (rps <= 4) launch_down<kKpw, 4>(p, wgs, stream);
  else launch_down<kKpw, 8>(p, wgs, stream);
}

}  // namespace

bool decode_shape_ok(int H, int I, int k, int g13, int g2) {
  // Two 32-element chunks of a down row per lane at most (I <= 4096), the
  // staged intermediate rows of one token fit in LDS, and the W13 group is a
  // power of two (the gate/up kernel divides by shifting).
  return (H % 32) == 0 && (I % 32) == 0 && I <= 4096 && (I % kNpw) == 0 && (g13 & (g13 - 1)) == 0 &&
         H / g13 <= kMaxGroups &&
         (g2 & (g2 - 1)) == 0 &&
         (H % kDownRows) == 0 && k >= 1 && k <= 2 * kDownWaves && down_lds(I, k, g2) <= kMaxDownLds;
}

hipError_t launch_decode_gate_up(const DecodeArgs& p, hipStream_t stream) {
  const int mk = p.M * p.k;
  const int waves = mk * (p.I / kNpw);
  const int wgs = grid_for((waves + kGateUpWaves - 1) / kGateUpWaves, p.max_workgroups);
  hipLaunchKernelGGL(decode_gate_up_int4, dim3(wgs), dim3(kGateUpThreads), 0, stream, p.x, p.ids,
                     static_cast<const uint32_t*>(p.w13.q), static_cast<const uint16_t*>(p.w13.scale),
                     p.w13.zero, p.a_hi, p.a_lo, mk, p.k, p.E, p.H, p.I, log2_of(p.w13.group));
  return hipGetLastError();
}

hipError_t launch_decode_down(const DecodeArgs& p, hipStream_t stream) {
  const int wgs = grid_for(p.M * (p.H / kDownRows), p.max_workgroups);
  if (p.k <= kDownWaves) launch_down_rps<1>(p, wgs, stream);
  else launch_down_rps<2>(p, wgs, stream);
  return hipGetLastError();
}

}  // namespace moe
