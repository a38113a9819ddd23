// Decode path: output-stationary expert FFN for small batches (the
// warp-decode write-up, "Qué cambiamos" and "Cómo funcionan los dos kernels").
//
// No alignment, gather, scatter or per-expert output buffer: each wave64 owns
// a fixed set of outputs, streams exactly the packed weight rows they need
// from HBM, reduces across its lanes with a fixed butterfly, and writes each
// output once.
//
// Kernel 1 (gate/up): a wave owns kNpw intermediate neurons of one route
//   (token t, expert e) and streams their gate and up rows. Lane l covers the
//   32-element chunks c = l, l+64, ... of the reduction (H). Weights are
//   unpacked to bf16 (128 + q) pairs and multiplied with the bf16 activation
//   pairs by v_dot2c_f32_bf16 (exact products, fp32 sums); per chunk the bias
//   and zero point are removed in fp32: s * (sum x(128+q) - (128+z) sum x).
//   silu(gate) * up is written to the fp32 intermediate a[r][i].
// Kernel 2 (down + combine): a workgroup owns 8 hidden outputs of one token;
//   wave w streams the down rows of routes j = w, w+4, ... and folds the
//   routing weight into its fp32 accumulators (j ascending). Lanes of a wave
//   are split into slots of pow2(I/32) lanes; a slot owns rows of the 8 and
//   its lanes cover the I/32 chunks. The four wave partials are summed in
//   wave order and y is written once. No floating-point atomics anywhere.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kGateUpThreads = 256;
constexpr int kDownThreads = 256;
constexpr int kDownRows = 8;

template <int kNpw>
__global__ __launch_bounds__(kGateUpThreads) void decode_gate_up_int4(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ ids,
    const uint32_t* __restrict__ q, const uint16_t* __restrict__ sc,
    const uint8_t* __restrict__ zp, float* __restrict__ a, int mk, int k, int E, int H,
    int I, int g) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave_id = blockIdx.x * (kGateUpThreads / kWave) + threadIdx.x / kWave;
  const int nwaves = gridDim.x * (kGateUpThreads / kWave);
  const int tasks_per_route = I / kNpw;
  const int ntasks = mk * tasks_per_route;
  const int nch = H >> 5;
  const int words = H >> 3;
  const int gpr = H / g;

  for (int task = wave_id; task < ntasks; task += nwaves) {
    const int r = task / tasks_per_route;
    const int i0 = (task - r * tasks_per_route) * kNpw;
    const int e = load_expert(ids, r, E);
    if (e < 0) {
      if (lane < kNpw) a[static_cast<size_t>(r) * I + i0 + lane] = 0.0f;
      continue;
    }
    const int t = r / k;
    float acc[2 * kNpw];
#pragma unroll
    for (int j = 0; j < 2 * kNpw; ++j) acc[j] = 0.0f;

    const uint4* xrow = reinterpret_cast<const uint4*>(x + static_cast<size_t>(t) * H);
    for (int c = lane; c < nch; c += kWave) {
      // Issue the weight loads first so they are all in flight together.
      uint4 wv[2 * kNpw];
      float s[2 * kNpw], zb[2 * kNpw];
      const int grp = (c << 5) / g;
#pragma unroll
      for (int j = 0; j < 2 * kNpw; ++j) {
        const int n = j < kNpw ? i0 + j : I + i0 + (j - kNpw);
        const size_t row = static_cast<size_t>(e) * (2 * I) + n;
        wv[j] = load_stream16(q + row * words + 4 * c);
        s[j] = half_bits_to_float(sc[row * gpr + grp]);
        zb[j] = 128.0f + static_cast<float>(zp[row * gpr + grp]);
      }
      uint32_t xw[16];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint4 t4 = xrow[c * 4 + v];
        xw[4 * v + 0] = t4.x; xw[4 * v + 1] = t4.y; xw[4 * v + 2] = t4.z; xw[4 * v + 3] = t4.w;
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
          unpack8_bias128(w4[v], p);
#pragma unroll
          for (int i = 0; i < 4; ++i) d = dot2_bf16(p[i], xw[4 * v + i], d);
        }
        acc[j] = fmaf(s[j], fmaf(-zb[j], sx, d), acc[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < 2 * kNpw; ++j) acc[j] = wave_sum(acc[j]);
    float gv = acc[0], uv = acc[kNpw];
#pragma unroll
    for (int j = 1; j < kNpw; ++j) {
      if (lane == j) { gv = acc[j]; uv = acc[kNpw + j]; }
    }
    if (lane < kNpw) a[static_cast<size_t>(r) * I + i0 + lane] = silu_mul(gv, uv);
  }
}

__global__ __launch_bounds__(kDownThreads) void decode_down_int4(
    const float* __restrict__ a, const int32_t* __restrict__ ids,
    const float* __restrict__ topk_w, const uint32_t* __restrict__ q,
    const uint16_t* __restrict__ sc, const uint8_t* __restrict__ zp, float* __restrict__ y,
    int M, int k, int E, int H, int I, int g) {
  __shared__ float part[kDownThreads / kWave][kDownRows];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int nwv = kDownThreads / kWave;
  const int tiles_per_tok = H / kDownRows;
  const int ntiles = M * tiles_per_tok;
  const int nch = I >> 5;
  const int words = I >> 3;
  const int gpr = I / g;
  // Lanes form slots of `span` lanes (a power of two >= the chunk count, or
  // the whole wave when a row has more than 64 chunks).
  int span = 1;
  while (span < nch && span < kWave) span <<= 1;
  const int slots = kWave / span;
  const int slot = lane / span;
  const int c0 = lane - slot * span;
  const int rps = (kDownRows + slots - 1) / slots;  // rows per slot

  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int t = tile / tiles_per_tok;
    const int h0 = (tile - t * tiles_per_tok) * kDownRows;
    float acc[kDownRows];
#pragma unroll
    for (int i = 0; i < kDownRows; ++i) acc[i] = 0.0f;

    for (int j = wave; j < k; j += nwv) {
      const int r = t * k + j;
      const int e = load_expert(ids, r, E);
      if (e < 0) continue;
      const float wj = topk_w[r];
      for (int c = c0; c < nch; c += span) {
        uint4 wv[kDownRows];
        float s[kDownRows], z[kDownRows];
#pragma unroll
        for (int i = 0; i < kDownRows; ++i) {
          const int m = slot + i * slots;
          if (i < rps && m < kDownRows) {
            const size_t row = static_cast<size_t>(e) * H + h0 + m;
            const int grp = (c << 5) / g;
            wv[i] = load_stream16(q + row * words + 4 * c);
            s[i] = half_bits_to_float(sc[row * gpr + grp]);
            z[i] = static_cast<float>(zp[row * gpr + grp]);
          }
        }
        const float4* ap = reinterpret_cast<const float4*>(a + static_cast<size_t>(r) * I + (c << 5));
        float av[32];
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          const float4 t4 = ap[v];
          av[4 * v] = t4.x; av[4 * v + 1] = t4.y; av[4 * v + 2] = t4.z; av[4 * v + 3] = t4.w;
        }
        float sa = 0.0f;
#pragma unroll
        for (int v = 0; v < 32; ++v) sa += av[v];
#pragma unroll
        for (int i = 0; i < kDownRows; ++i) {
          const int m = slot + i * slots;
          if (i < rps && m < kDownRows) {
            const uint32_t w4[4] = {wv[i].x, wv[i].y, wv[i].z, wv[i].w};
            float d = 0.0f;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              float qf[8];
              unpack8_f32(w4[v], qf);
#pragma unroll
              for (int u = 0; u < 8; ++u) d = fmaf(av[8 * v + u], qf[u], d);
            }
            acc[i] = fmaf(wj * s[i], fmaf(-z[i], sa, d), acc[i]);
          }
        }
      }
    }
    // Sum each row over the lanes of its slot (butterfly inside the span).
#pragma unroll
    for (int i = 0; i < kDownRows; ++i) {
      if (i < rps) {
        float v = acc[i];
        for (int o = span >> 1; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
        acc[i] = v;
      }
    }
    if (c0 == 0) {
#pragma unroll
      for (int i = 0; i < kDownRows; ++i) {
        const int m = slot + i * slots;
        if (i < rps && m < kDownRows) part[wave][m] = acc[i];
      }
    }
    __syncthreads();
    if (threadIdx.x < kDownRows) {
      float v = part[0][threadIdx.x];
      for (int w = 1; w < nwv; ++w) v += part[w][threadIdx.x];
      y[static_cast<size_t>(t) * H + h0 + threadIdx.x] = v;
    }
    __syncthreads();
  }
}

int grid_for(int work_groups, int max_workgroups) {
  if (work_groups < 1) work_groups = 1;
  return (max_workgroups > 0 && max_workgroups < work_groups) ? max_workgroups : work_groups;
}

}  // namespace

constexpr int kDecodeNpw = 2;

bool decode_shape_ok(int H, int I, int k) {
  return (H % 32) == 0 && (I % 32) == 0 && (I % kDecodeNpw) == 0 && (H % kDownRows) == 0 && k >= 1;
}

hipError_t launch_decode_gate_up(const DecodeArgs& p, hipStream_t stream) {
  const int mk = p.M * p.k;
  const int waves = mk * (p.I / kDecodeNpw);
  const int wgs = grid_for((waves + 3) / 4, p.max_workgroups);
  hipLaunchKernelGGL(decode_gate_up_int4<kDecodeNpw>, dim3(wgs), dim3(kGateUpThreads), 0, stream,
                     p.x, p.ids, static_cast<const uint32_t*>(p.w13.q),
                     static_cast<const uint16_t*>(p.w13.scale), p.w13.zero, p.a, mk, p.k, p.E,
                     p.H, p.I, p.w13.group);
  return hipGetLastError();
}

hipError_t launch_decode_down(const DecodeArgs& p, hipStream_t stream) {
  const int tiles = p.M * (p.H / kDownRows);
  const int wgs = grid_for(tiles, p.max_workgroups);
  hipLaunchKernelGGL(decode_down_int4, dim3(wgs), dim3(kDownThreads), 0, stream, p.a, p.ids,
                     p.topk_w, static_cast<const uint32_t*>(p.w2.q),
                     static_cast<const uint16_t*>(p.w2.scale), p.w2.zero, p.y, p.M, p.k, p.E,
                     p.H, p.I, p.w2.group);
  return hipGetLastError();
}

}  // namespace moe
