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
// Kernel 2 (down + combine): a workgroup owns 8 (or, at larger M, 16)
//   hidden outputs of one token; wave w takes the routes j = w, w+8, ... and
//   folds the routing weight into its fp32 accumulators. Lanes of a wave form slots of
//   pow2(I/32) lanes; a slot owns some of the rows and its lanes cover the
//   I/32 chunks. Each lane loads its intermediate chunks (hi and lo planes)
//   straight into registers (16-row form: the wave's LDS region, by LDS-DMA),
//   then its weight words, scales and zeros, so a route costs a single wait
//   on memory; the weights are bf16 (128 + q)
//   pairs, each dotted with the hi and the lo plane. The eight wave partials
//   are added in wave order and y is written once. No floating-point atomics
//   anywhere.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kGateUpThreads = 256;
constexpr int kGateUpWaves = kGateUpThreads / kWave;
constexpr int kNpw = 2;                       // neurons per wave (the row folding assumes 2)
constexpr int kDownWaves = 8;
constexpr int kDownThreads = kDownWaves * kWave;
constexpr int kDownRows = 8;

template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}

// Sums over the 64 lanes of four values at once, the same bits in every lane
// of a 16-lane row: gfx950's lane swaps fold the four values into one
// register, one per 16-lane row (a: row 0, c: row 1, b: row 2, d: row 3),
// then a DPP butterfly finishes each row. Per value the order is
// ((l0 + l2) + (l1 + l3)) over the four rows' lanes, then the butterfly.
__device__ __forceinline__ float wave_sum4_dpp(float a, float b, float c, float d) {
  const auto ab = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  const auto cd = __builtin_amdgcn_permlane32_swap(__float_as_uint(c), __float_as_uint(d), false, false);
  // Lanes 0..31: a's rows 0,1 + rows 2,3; lanes 32..63 the same for b.
  const float sab = __uint_as_float(ab[0]) + __uint_as_float(ab[1]);
  const float scd = __uint_as_float(cd[0]) + __uint_as_float(cd[1]);
  const auto m = __builtin_amdgcn_permlane16_swap(__float_as_uint(sab), __float_as_uint(scd), false, false);
  float v = __uint_as_float(m[0]) + __uint_as_float(m[1]);   // rows: a, c, b, d
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror
  v += dpp<0x140>(v);  // row_mirror
  return v;
}

// One 32-element chunk of a weight row dotted with 16 bf16 activation pairs
// (xw). int4: 16 bytes, bf16 (128 + q) pairs, the caller removes the bias
// and zero point; MXFP8: 32 bytes of E4M3 codes, converted exactly to bf16
// pairs, the caller applies the block's power-of-two scale.
template <int kFmt>
struct ChunkRow {
  static constexpr int kVecs = kFmt == MOE_W_MXFP8 ? 2 : 1;   // 16-byte loads per chunk
  uint4 v[kVecs];
};

template <int kFmt>
__device__ __forceinline__ void load_chunk(const unsigned char* row, int c, ChunkRow<kFmt>& w) {
  const uint4* p = reinterpret_cast<const uint4*>(row) + c * ChunkRow<kFmt>::kVecs;
#pragma unroll
  for (int i = 0; i < ChunkRow<kFmt>::kVecs; ++i) w.v[i] = load_stream16(p + i);
}

template <int kFmt>
__device__ __forceinline__ float dot_chunk(const ChunkRow<kFmt>& w, const uint32_t (&xw)[16], uint32_t nib_mask,
                                           float d) {
  if constexpr (kFmt == MOE_W_MXFP8) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t w4[4] = {w.v[i].x, w.v[i].y, w.v[i].z, w.v[i].w};
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        d = dot2_bf16(fp8x2_to_bf16x2<false>(w4[v]), xw[8 * i + 2 * v], d);
        d = dot2_bf16(fp8x2_to_bf16x2<true>(w4[v]), xw[8 * i + 2 * v + 1], d);
      }
    }
  } else {
    const uint32_t w4[4] = {w.v[0].x, w.v[0].y, w.v[0].z, w.v[0].w};
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      uint32_t p[4];
      unpack8_bias128_m(w4[v], nib_mask, p);
#pragma unroll
      for (int i = 0; i < 4; ++i) d = dot2_bf16(p[i], xw[4 * v + i], d);
    }
  }
  return d;
}

// Piece pc (16 bytes: activations 8 pc .. 8 pc + 7 of the chunk, as four
// bf16 pairs xp) of dot_chunk, in dot_chunk's order: running pieces 0..3
// through it gives dot_chunk's sum bit for bit.
template <int kFmt>
__device__ __forceinline__ float dot_piece(const ChunkRow<kFmt>& w, int pc, const uint32_t (&xp)[4],
                                           uint32_t nib_mask, float d) {
  if constexpr (kFmt == MOE_W_MXFP8) {
    const uint4 v4 = w.v[pc >> 1];
    const uint32_t w4[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t wd = w4[2 * (pc & 1) + h];
      d = dot2_bf16(fp8x2_to_bf16x2<false>(wd), xp[2 * h], d);
      d = dot2_bf16(fp8x2_to_bf16x2<true>(wd), xp[2 * h + 1], d);
    }
  } else {
    const uint32_t w4[4] = {w.v[0].x, w.v[0].y, w.v[0].z, w.v[0].w};
    uint32_t p[4];
    unpack8_bias128_m(w4[pc], nib_mask, p);
#pragma unroll
    for (int i = 0; i < 4; ++i) d = dot2_bf16(p[i], xp[i], d);
  }
  return d;
}

// kCapture: also write the W13 outputs (gate, up) to w13_out; a separate
// instantiation, so the plain kernel carries no trace of it.
template <int kFmt, bool kCapture>
__global__ __launch_bounds__(kGateUpThreads) void decode_gate_up(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ ids,
    const unsigned char* __restrict__ q, const unsigned char* __restrict__ sc,
    const uint8_t* __restrict__ zp, uint16_t* __restrict__ a_hi, uint16_t* __restrict__ a_lo,
    float* __restrict__ w13_out, int mk, int k, int E, int ebase, int H, int I, int g_shift) {
  constexpr bool kMx = kFmt == MOE_W_MXFP8;
  const int lane = threadIdx.x & (kWave - 1);
  // Task indices are wave-uniform: keep them (and the row addresses) scalar.
  const int wave_id = uniform(blockIdx.x * kGateUpWaves + threadIdx.x / kWave);
  const int nwaves = gridDim.x * kGateUpWaves;
  const int tasks_per_route = I / kNpw;
  const int ntasks = mk * tasks_per_route;
  const int nch = H >> 5, gpr = H >> g_shift;
  const int row_bytes = kMx ? H : H / 2;
  const int sc_bytes = kMx ? 1 : 2;                // E8M0 byte or fp16 per group
  const uint32_t nib_mask = in_vgpr(0x000F000Fu);

  for (int task = wave_id; task < ntasks; task += nwaves) {
    const int r = task / tasks_per_route;
    const int i0 = (task - r * tasks_per_route) * kNpw;
    // The activations do not depend on the expert: their first chunk is
    // requested before the expert-ID load is waited for.
    const int t = r / k;
    const uint4* xrow = reinterpret_cast<const uint4*>(x + static_cast<size_t>(t) * H);
    uint4 xv[4];
    {
      const int cx = lane < nch ? lane : 0;
#pragma unroll
      for (int v = 0; v < 4; ++v) xv[v] = xrow[cx * 4 + v];
    }
    __builtin_amdgcn_sched_barrier(0);
    const int e = uniform(load_expert(ids, r, E, ebase));
    if (e < 0) {
      // A use of the activations on this (rare) side too, so that their
      // loads stay above the branch instead of being sunk below the ID wait.
      asm volatile("" ::"v"(xv[0].x));
      if (lane < kNpw) {
        a_hi[static_cast<size_t>(r) * I + i0 + lane] = 0;
        a_lo[static_cast<size_t>(r) * I + i0 + lane] = 0;
      }
      continue;
    }
    const size_t row0 = static_cast<size_t>(e) * (2 * I) + i0;  // first gate row
    const unsigned char* qrow[2 * kNpw];
    const unsigned char* srow[2 * kNpw];
    const uint8_t* zrow[2 * kNpw];
#pragma unroll
    for (int j = 0; j < 2 * kNpw; ++j) {
      const size_t row = row0 + (j < kNpw ? j : I + j - kNpw);
      qrow[j] = q + row * row_bytes;
      srow[j] = sc + row * gpr * sc_bytes;
      zrow[j] = kMx ? nullptr : zp + row * gpr;
    }
    float acc[2 * kNpw];
#pragma unroll
    for (int j = 0; j < 2 * kNpw; ++j) acc[j] = 0.0f;
    for (int c = lane; c < nch; c += kWave) {
      // Loads return in issue order, so the activations and the small scale
      // and zero loads go first and the four weight rows last: row j's sums
      // then wait only for row j's weights, and the rows before it are
      // computed while the later ones land.
      if (c != lane) {
#pragma unroll
        for (int v = 0; v < 4; ++v) xv[v] = xrow[c * 4 + v];
      }
      __builtin_amdgcn_sched_barrier(0);
      ChunkRow<kFmt> wv[2 * kNpw];
      const int grp = (c << 5) >> g_shift;
      uint32_t sv[2 * kNpw], zv[2 * kNpw];
#pragma unroll
      for (int j = 0; j < 2 * kNpw; ++j) {
        if constexpr (kMx) {
          sv[j] = srow[j][grp];
        } else {
          sv[j] = reinterpret_cast<const uint16_t*>(srow[j])[grp];
          zv[j] = zrow[j][grp];
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 2 * kNpw; ++j) load_chunk<kFmt>(qrow[j], c, wv[j]);
      // Keep every load above this point: the scheduler would otherwise sink
      // some of them below the first use of the others and add a round trip.
      __builtin_amdgcn_sched_barrier(0);
      uint32_t xw[16];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        xw[4 * v] = xv[v].x; xw[4 * v + 1] = xv[v].y; xw[4 * v + 2] = xv[v].z; xw[4 * v + 3] = xv[v].w;
      }
      if constexpr (kMx) {
#pragma unroll
        for (int j = 0; j < 2 * kNpw; ++j)
          acc[j] = fmaf(e8m0_to_float(sv[j]), dot_chunk<kFmt>(wv[j], xw, nib_mask, 0.0f), acc[j]);
      } else {
        // The activation sum and the per-row scale terms need only the loads
        // that land first; they are done before the first weight row's wait.
        float sx = 0.0f;
#pragma unroll
        for (int v = 0; v < 16; ++v) sx = dot2_bf16(xw[v], 0x3F803F80u, sx);  // (1.0, 1.0)
        float s[2 * kNpw], zb[2 * kNpw];
#pragma unroll
        for (int j = 0; j < 2 * kNpw; ++j) {
          s[j] = half_bits_to_float(static_cast<uint16_t>(sv[j]));
          zb[j] = 128.0f + static_cast<float>(zv[j]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 2 * kNpw; ++j)
          acc[j] = fmaf(s[j], fmaf(-zb[j], sx, dot_chunk<kFmt>(wv[j], xw, nib_mask, 0.0f)), acc[j]);
      }
    }
    // Rows of the folded sums: gate 0, up 0, gate 1, up 1.
    const float v = wave_sum4_dpp(acc[0], acc[1], acc[2], acc[3]);
    const float g0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float u0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float g1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float u1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    const float gv = lane == 0 ? g0 : g1;
    const float uv = lane == 0 ? u0 : u1;
    if (lane < kNpw) {
      const float v = silu_mul(gv, uv);
      const __bf16 h = static_cast<__bf16>(v);
      const size_t off = static_cast<size_t>(r) * I + i0 + lane;
      a_hi[off] = __builtin_bit_cast(uint16_t, h);
      a_lo[off] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v - static_cast<float>(h)));
      if constexpr (kCapture) {
        // The W13 outputs themselves (capture surface): gate, then up.
        w13_out[static_cast<size_t>(r) * (2 * I) + i0 + lane] = gv;
        w13_out[static_cast<size_t>(r) * (2 * I) + I + i0 + lane] = uv;
      }
    }
  }
}

// kSpan: lanes per slot, pow2(I/32) capped at 64; kCh: 32-element chunks of
// a down row per lane (1, or 2 when I/32 > 64). Routes j = wave, wave + 8, ...
// are taken in turn.
// kLds (one chunk per lane): the route's intermediate rows reach LDS by
// LDS-DMA into a region of the wave's own and are read in 16-byte pieces
// inside the dot products, so they hold no registers while in flight (more
// workgroups per CU); same products, same order, same bits.
template <int kFmt, int kCh, int kSpan, bool kLds, int kRows>
__global__ __launch_bounds__(kDownThreads) void decode_down(
    const uint16_t* __restrict__ a_hi, const uint16_t* __restrict__ a_lo,
    const int32_t* __restrict__ ids, const float* __restrict__ topk_w,
    const unsigned char* __restrict__ q, const unsigned char* __restrict__ sc,
    const uint8_t* __restrict__ zp, float* __restrict__ y, int M, int k, int E, int ebase, int H, int I,
    int g_shift) {
  constexpr bool kMx = kFmt == MOE_W_MXFP8;
  constexpr int kSlots = kWave / kSpan;
  constexpr int kRps = (kRows + kSlots - 1) / kSlots;  // rows per lane
  static_assert(!kLds || kCh == 1, "LDS-staged intermediate: one chunk per lane");
  constexpr int kPlane = kSpan * 64;                        // LDS bytes per intermediate plane
  __shared__ float part[kDownWaves][kRows];
  __shared__ __align__(16) unsigned char inter[kLds ? kDownWaves * 2 * kPlane : 16];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = uniform(threadIdx.x / kWave);
  const int tiles_per_tok = H / kRows;
  const int ntiles = M * tiles_per_tok;
  const int nch = I >> 5, gpr = I >> g_shift;
  const int row_bytes = kMx ? I : I / 2;
  const int span = kSpan, slots = kSlots;
  const int slot = lane / kSpan;
  const int c0 = lane - slot * kSpan;
  const uint32_t nib_mask = in_vgpr(0x000F000Fu);

  // Lanes past the last chunk, and slots past the last row (tiny I), read a
  // clamped in-bounds address and contribute zero: the loop body has no
  // per-lane branches, so the row chains can be interleaved.
  int cl[kCh];
  float cvalid[kCh];
#pragma unroll
  for (int cc = 0; cc < kCh; ++cc) {
    const int c = c0 + cc * span;
    cl[cc] = c < nch ? c : 0;
    cvalid[cc] = (c < nch && slot < kRows) ? 1.0f : 0.0f;
  }
  int mrow[kRps];
#pragma unroll
  for (int i = 0; i < kRps; ++i) {
    const int m = slot + i * slots;
    mrow[i] = m < kRows ? m : 0;
  }

  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int t = tile / tiles_per_tok;
    const int h0 = (tile - t * tiles_per_tok) * kRows;
    float acc[kRps];
#pragma unroll
    for (int i = 0; i < kRps; ++i) acc[i] = 0.0f;
    for (int j = wave; j < k; j += kDownWaves) {
      // Every load of this route is issued before the first wait: the
      // intermediate chunks (they do not depend on the expert id), then the
      // packed weights, then the scales and zeros.
      const size_t r = static_cast<size_t>(t) * k + j;
      uint4 hv[kCh][4], lv[kCh][4];
      unsigned char* const ih = inter + (wave * 2) * kPlane;
      if constexpr (kLds) {
        // Both planes of the route's row, 1 KB per DMA (the plane's bytes in
        // order; lanes past the row's 2I bytes re-read its start and land
        // in the region's unused tail). The previous route's LDS reads have
        // completed before its region is written again.
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const unsigned char* hs = reinterpret_cast<const unsigned char*>(a_hi + r * I);
        const unsigned char* ls = reinterpret_cast<const unsigned char*>(a_lo + r * I);
        for (int m = 0; m * 1024 < 2 * I; ++m) {
          const int off = 1024 * m + 16 * lane;
          const int so = off < 2 * I ? off : 0;
          dma16(hs + so, lds_addr(ih) + 1024 * m);
          dma16(ls + so, lds_addr(ih + kPlane) + 1024 * m);
        }
      } else {
#pragma unroll
        for (int cc = 0; cc < kCh; ++cc) {
          const uint4* hp = reinterpret_cast<const uint4*>(a_hi + r * I + (cl[cc] << 5));
          const uint4* lp = reinterpret_cast<const uint4*>(a_lo + r * I + (cl[cc] << 5));
#pragma unroll
          for (int v = 0; v < 4; ++v) { hv[cc][v] = hp[v]; lv[cc][v] = lp[v]; }
        }
      }
      // The scheduler must not move these loads below the expert-id wait,
      // nor (further down) the weight loads below the first use of any load.
      __builtin_amdgcn_sched_barrier(0);
      // An invalid route has a zero intermediate (the gate/up kernel writes
      // zeros for it); it reads expert 0's rows and adds exactly zero. No
      // branch here: the compiler would sink the loads above into it.
      const int e_raw = uniform(load_expert(ids, static_cast<int>(r), E, ebase));
      const int e = e_raw < 0 ? 0 : e_raw;
      const float wr = e_raw < 0 ? 0.0f : topk_w[r];
      const unsigned char* qt = q + (static_cast<size_t>(e) * H + h0) * row_bytes;
      const size_t gt = (static_cast<size_t>(e) * H + h0) * gpr;
      ChunkRow<kFmt> wv[kCh][kRps];
      uint32_t sv[kCh][kRps], zv[kCh][kRps];
#pragma unroll
      for (int cc = 0; cc < kCh; ++cc) {
#pragma unroll
        for (int i = 0; i < kRps; ++i) load_chunk<kFmt>(qt + mrow[i] * row_bytes, cl[cc], wv[cc][i]);
      }
#pragma unroll
      for (int cc = 0; cc < kCh; ++cc) {
        const int grp = (cl[cc] << 5) >> g_shift;
#pragma unroll
        for (int i = 0; i < kRps; ++i) {
          if constexpr (kMx) {
            sv[cc][i] = sc[gt + mrow[i] * gpr + grp];
          } else {
            sv[cc][i] = reinterpret_cast<const uint16_t*>(sc)[gt + mrow[i] * gpr + grp];
            zv[cc][i] = zp[gt + mrow[i] * gpr + grp];
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kLds) {
        // Every load of the route has landed (the DMAs are the oldest); the
        // pieces are read in order, so each chain below sees the dwords in
        // the register form's order.
        wait_vm<0>();
        const unsigned char* hc = ih + cl[0] * 64;
        const unsigned char* lc = ih + kPlane + cl[0] * 64;
        float sa4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        float dh[kRps], dl[kRps];
#pragma unroll
        for (int i = 0; i < kRps; ++i) dh[i] = dl[i] = 0.0f;
#pragma unroll
        for (int pc = 0; pc < 4; ++pc) {
          const uint4 h4 = *reinterpret_cast<const uint4*>(hc + 16 * pc);
          const uint4 l4 = *reinterpret_cast<const uint4*>(lc + 16 * pc);
          const uint32_t hp[4] = {h4.x, h4.y, h4.z, h4.w};
          const uint32_t lp[4] = {l4.x, l4.y, l4.z, l4.w};
          if constexpr (!kMx) {
#pragma unroll
            for (int u = 0; u < 4; ++u) sa4[u] = dot2_bf16(lp[u], 0x3F803F80u, dot2_bf16(hp[u], 0x3F803F80u, sa4[u]));
          }
#pragma unroll
          for (int i = 0; i < kRps; ++i) {
            dh[i] = dot_piece<kFmt>(wv[0][i], pc, hp, nib_mask, dh[i]);
            dl[i] = dot_piece<kFmt>(wv[0][i], pc, lp, nib_mask, dl[i]);
            // One row's unpacked weights live at a time (registers, not ILP,
            // bound this form: other waves fill the gaps).
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        const float sa = (sa4[0] + sa4[1]) + (sa4[2] + sa4[3]);
#pragma unroll
        for (int i = 0; i < kRps; ++i) {
          if constexpr (kMx) {
            const float s = cvalid[0] * e8m0_to_float(sv[0][i]);
            acc[i] = fmaf(wr * s, dh[i] + dl[i], acc[i]);
          } else {
            const float s = cvalid[0] * half_bits_to_float(static_cast<uint16_t>(sv[0][i]));
            const float zb = 128.0f + static_cast<float>(zv[0][i]);
            acc[i] = fmaf(wr * s, fmaf(-zb, sa, dh[i] + dl[i]), acc[i]);
          }
        }
        continue;
      }
#pragma unroll
      for (int cc = 0; cc < kCh; ++cc) {
        const uint32_t hw[16] = {hv[cc][0].x, hv[cc][0].y, hv[cc][0].z, hv[cc][0].w,
                                 hv[cc][1].x, hv[cc][1].y, hv[cc][1].z, hv[cc][1].w,
                                 hv[cc][2].x, hv[cc][2].y, hv[cc][2].z, hv[cc][2].w,
                                 hv[cc][3].x, hv[cc][3].y, hv[cc][3].z, hv[cc][3].w};
        const uint32_t lw[16] = {lv[cc][0].x, lv[cc][0].y, lv[cc][0].z, lv[cc][0].w,
                                 lv[cc][1].x, lv[cc][1].y, lv[cc][1].z, lv[cc][1].w,
                                 lv[cc][2].x, lv[cc][2].y, lv[cc][2].z, lv[cc][2].w,
                                 lv[cc][3].x, lv[cc][3].y, lv[cc][3].z, lv[cc][3].w};
        // Sum of the chunk's activations in four independent chains (int4:
        // the bias and zero-point term).
        float sa = 0.0f;
        if constexpr (!kMx) {
          float sa4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int v = 0; v < 16; ++v)
            sa4[v & 3] = dot2_bf16(lw[v], 0x3F803F80u, dot2_bf16(hw[v], 0x3F803F80u, sa4[v & 3]));
          sa = (sa4[0] + sa4[1]) + (sa4[2] + sa4[3]);
        }
        // Per row, the hi and lo planes are separate chains.
#pragma unroll
        for (int i = 0; i < kRps; ++i) {
          const float dh = dot_chunk<kFmt>(wv[cc][i], hw, nib_mask, 0.0f);
          const float dl = dot_chunk<kFmt>(wv[cc][i], lw, nib_mask, 0.0f);
          if constexpr (kMx) {
            const float s = cvalid[cc] * e8m0_to_float(sv[cc][i]);
            acc[i] = fmaf(wr * s, dh + dl, acc[i]);
          } else {
            const float s = cvalid[cc] * half_bits_to_float(static_cast<uint16_t>(sv[cc][i]));
            const float zb = 128.0f + static_cast<float>(zv[cc][i]);
            acc[i] = fmaf(wr * s, fmaf(-zb, sa, dh + dl), acc[i]);
          }
        }
      }
    }
    // Sum each row over the lanes of its slot: DPP butterflies inside 16-lane
    // rows, then (slots wider than 16 lanes) the row sums read out in lane
    // order. Fixed order, no LDS round trips.
    if constexpr (kSpan == 32 && kRps % 4 == 0) {
      // Two 32-lane slots (slot s, index i: row s + 2i), four indices at a
      // time. A lane swap of 16-lane rows adds each slot's two halves and
      // packs four rows into one register (16-lane rows: rows 0, 2, 1, 3 of
      // a pair of indices), so two butterflies finish eight rows.
#pragma unroll
      for (int g4 = 0; g4 < kRps / 4; ++g4) {
        const float* a = acc + 4 * g4;
        const auto p01 = __builtin_amdgcn_permlane16_swap(__float_as_uint(a[0]), __float_as_uint(a[1]), false, false);
        const auto p23 = __builtin_amdgcn_permlane16_swap(__float_as_uint(a[2]), __float_as_uint(a[3]), false, false);
        float v01 = __uint_as_float(p01[0]) + __uint_as_float(p01[1]);
        float v23 = __uint_as_float(p23[0]) + __uint_as_float(p23[1]);
        v01 += dpp<0xB1>(v01);  v23 += dpp<0xB1>(v23);
        v01 += dpp<0x4E>(v01);  v23 += dpp<0x4E>(v23);
        v01 += dpp<0x141>(v01); v23 += dpp<0x141>(v23);
        v01 += dpp<0x140>(v01); v23 += dpp<0x140>(v23);
        if ((lane & 15) == 0) {
          const int q = lane >> 4;
          const int row = 8 * g4 + ((q >> 1) | ((q & 1) << 1));
          part[wave][row] = v01;
          part[wave][row + 4] = v23;
        }
      }
    } else if constexpr (kSpan == 64 && kRps == 8) {
      // One 64-lane slot, eight rows: each group of four accumulators folds
      // into one register (16-lane rows: rows 0, 2, 1, 3 of the group).
      const float v0 = wave_sum4_dpp(acc[0], acc[1], acc[2], acc[3]);
      const float v1 = wave_sum4_dpp(acc[4], acc[5], acc[6], acc[7]);
      if ((lane & 15) == 0) {
        const int q = lane >> 4;
        const int row = (q >> 1) | ((q & 1) << 1);
        part[wave][row] = v0;
        part[wave][row + 4] = v1;
      }
    } else {
#pragma unroll
    for (int i = 0; i < kRps; ++i) {
      float v = acc[i];
      if constexpr (kSpan > 1) v += dpp<0xB1>(v);   // xor 1
      if constexpr (kSpan > 2) v += dpp<0x4E>(v);   // xor 2
      if constexpr (kSpan > 4) v += dpp<0x141>(v);  // half-row mirror
      if constexpr (kSpan > 8) v += dpp<0x140>(v);  // row mirror
      acc[i] = v;
    }
    if constexpr (kSpan <= 16) {
      if (c0 == 0) {
#pragma unroll
        for (int i = 0; i < kRps; ++i) {
          if (slot + i * kSlots < kRows) part[wave][slot + i * kSlots] = acc[i];
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < kRps; ++i) {
#pragma unroll
        for (int sl = 0; sl < kSlots; ++sl) {
          float v = 0.0f;
#pragma unroll
          for (int rr = 0; rr < kSpan / 16; ++rr)
            v += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc[i]), sl * kSpan + 16 * rr));
          if (lane == 0) part[wave][sl + i * kSlots] = v;
        }
      }
    }
    }
    __syncthreads();
    if (threadIdx.x < kRows) {
      float v = part[0][threadIdx.x];
      for (int w = 1; w < kDownWaves; ++w) v += part[w][threadIdx.x];
      y[static_cast<size_t>(t) * H + h0 + threadIdx.x] = v;
    }
    __syncthreads();
  }
}

int log2_of(int g) {
  int s = 0;
  while ((1 << s) < g) ++s;
  return s;
}

template <int kFmt, int kCh, int kSpan, bool kLds, int kRows>
void launch_down(const DecodeArgs& p, hipStream_t stream) {
  const int wgs = grid_for(int64_t(p.M) * (p.H / kRows), p.max_workgroups);
  launch(decode_down<kFmt, kCh, kSpan, kLds, kRows>, dim3(wgs), dim3(kDownThreads), 0, stream,
                     p.a_hi, p.a_lo, p.ids, p.topk_w, static_cast<const unsigned char*>(p.w2.q),
                     static_cast<const unsigned char*>(p.w2.scale), p.w2.zero, p.y, p.M, p.k, p.E,
                     p.ebase, p.H, p.I, log2_of(p.w2.group));
}

// Down workgroups of 16 rows with the intermediate staged in LDS (int4,
// 17..32 chunks per row): each wave streams twice the weight bytes per route
// at the same registers and workgroups per CU, once the layer has at least
// two such workgroups per CU of the 256; below that the 8-row form keeps
// more waves in flight.
constexpr int kDownWideRows = 16;
constexpr int64_t kDownWideMinGroups = 2 * 256;

template <int kFmt>
void launch_down_fmt(const DecodeArgs& p, hipStream_t stream) {
  const int nch = p.I >> 5;
  const bool wide = (p.H % kDownWideRows) == 0 && int64_t(p.M) * (p.H / kDownWideRows) >= kDownWideMinGroups;
  if (nch > 32) {
    if (nch > kWave) launch_down<kFmt, 2, 64, false, kDownRows>(p, stream);
    else launch_down<kFmt, 1, 64, false, kDownRows>(p, stream);
  } else if (nch > 16) {
    if constexpr (kFmt == MOE_W_INT4_AWQ) {
      if (wide) {
        launch_down<kFmt, 1, 32, true, kDownWideRows>(p, stream);
        return;
      }
    }
    launch_down<kFmt, 1, 32, false, kDownRows>(p, stream);
  } else if (nch > 8) launch_down<kFmt, 1, 16, false, kDownRows>(p, stream);
  else if (nch > 4) launch_down<kFmt, 1, 8, false, kDownRows>(p, stream);
  else if (nch > 2) launch_down<kFmt, 1, 4, false, kDownRows>(p, stream);
  else if (nch > 1) launch_down<kFmt, 1, 2, false, kDownRows>(p, stream);
  else launch_down<kFmt, 1, 1, false, kDownRows>(p, stream);
}

}  // namespace

bool decode_shape_ok(int fmt, int H, int I, int k, int g13, int g2) {
  if (fmt == MOE_W_MXFP8 && (g13 != 32 || g2 != 32)) return false;
  // Two 32-element chunks of a down row per lane at most (I <= 4096), at most
  // two routes per down wave (k <= 16), and power-of-two groups (the kernels
  // divide by shifting).
  return (H % 32) == 0 && (I % 32) == 0 && I <= 4096 && (I % kNpw) == 0 && (g13 & (g13 - 1)) == 0 &&
         (g2 & (g2 - 1)) == 0 &&
         (H % kDownRows) == 0 && k >= 1 && k <= 2 * kDownWaves;
}

namespace {

template <int kFmt, bool kCapture>
void launch_gate_up(const DecodeArgs& p, int wgs, hipStream_t stream) {
  launch(decode_gate_up<kFmt, kCapture>, dim3(wgs), dim3(kGateUpThreads), 0, stream, p.x, p.ids,
         static_cast<const unsigned char*>(p.w13.q), static_cast<const unsigned char*>(p.w13.scale), p.w13.zero,
         p.a_hi, p.a_lo, p.w13_out, p.M * p.k, p.k, p.E, p.ebase, p.H, p.I, log2_of(p.w13.group));
}

}  // namespace

hipError_t launch_decode_gate_up(const DecodeArgs& p, hipStream_t stream) {
  const int mk = p.M * p.k;
  const int64_t waves = int64_t(mk) * (p.I / kNpw);
  const int wgs = grid_for((waves + kGateUpWaves - 1) / kGateUpWaves, p.max_workgroups);
  const bool cap = p.w13_out != nullptr;
  if (p.w13.fmt == MOE_W_MXFP8) {
    if (cap) launch_gate_up<MOE_W_MXFP8, true>(p, wgs, stream);
    else launch_gate_up<MOE_W_MXFP8, false>(p, wgs, stream);
  } else {
    if (cap) launch_gate_up<MOE_W_INT4_AWQ, true>(p, wgs, stream);
    else launch_gate_up<MOE_W_INT4_AWQ, false>(p, wgs, stream);
  }
  return hipGetLastError();
}

hipError_t launch_decode_down(const DecodeArgs& p, hipStream_t stream) {
  if (p.w2.fmt == MOE_W_MXFP8) launch_down_fmt<MOE_W_MXFP8>(p, stream);
  else launch_down_fmt<MOE_W_INT4_AWQ>(p, stream);
  return hipGetLastError();
}

}  // namespace moe
