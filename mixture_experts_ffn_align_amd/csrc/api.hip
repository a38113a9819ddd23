// C ABI of the MoE expert-FFN library: argument validation, workspace layout,
// path selection and kernel launches. Nothing here allocates device memory or
// synchronises the host.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>

#include "kernels.hpp"
#include "moe_ffn.h"

namespace moe {

LaunchTiming*& launch_timing() {
  static thread_local LaunchTiming* t = nullptr;
  return t;
}

}  // namespace moe

namespace {

constexpr int32_t kMaxExperts = 2048;
constexpr int64_t kMaxRoutes = int64_t(1) << 24;
constexpr int32_t kAutoDecodeMaxM = 14;
constexpr int64_t kMaxTasks = int64_t(1) << 30;

size_t round256(size_t n) { return (n + 255) & ~size_t(255); }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t capacity_of(int64_t M, int64_t k, int64_t E, int64_t b) {
  const int64_t mk = M * k;
  const int64_t raw = mk + (E < mk ? E : mk) * (b - 1);
  return static_cast<size_t>((raw + b - 1) / b * b);
}

struct Layout {
  int path = MOE_PATH_DECODE;
  size_t cap = 0;        // alignment capacity (grouped)
  size_t off_sorted = 0, off_blocks = 0, off_npad = 0, off_align_ws = 0, align_ws = 0;
  size_t off_a = 0, off_aux = 0, off_yhat = 0;   // intermediate (see moe_ffn_intermediate), yhat
  size_t total = 0;
};

bool weights_ok(const moe_weights& w) {
  if (w.q == nullptr || w.scale == nullptr || w.group <= 0) return false;
  if (!aligned(w.q, 16)) return false;
  if (w.fmt == MOE_W_INT4_AWQ && w.zero == nullptr) return false;
  return true;
}

// MOE_PATH_AUTO: the decode path for M <= kAutoDecodeMaxM, else the grouped
// path (expert-centric packing wins once tokens share experts: the warp-decode
// write-up's last section). On the Qwen3-30B-A3B-sized layer (top-8 of 128
// experts, int4 g128, b = 8, cold weights) the decode path is faster on the
// median up to M = 14 and the grouped path from M = 15
// (profiles/batch_sweep_decode_vs_grouped.md, `bench.py --batch-sweep`).
int auto_path(const moe_ffn_desc* d) { return d->M <= kAutoDecodeMaxM ? MOE_PATH_DECODE : MOE_PATH_GROUPED; }

bool shape_ok(int path, const moe_ffn_desc* d) {
  if (path == MOE_PATH_DECODE)
    return moe::decode_shape_ok(d->w13.fmt, d->H, d->I, d->k, d->w13.group, d->w2.group);
  return moe::grouped_shape_ok(d->w13.fmt, d->H, d->I, d->b, d->w13.group, d->w2.group);
}

// Task counts of the path's kernels (waves or workgroups; the combine's
// threads) stay below kMaxTasks, so that int32 task indices and the
// grid-stride steps past the last task do not overflow.
bool tasks_fit(int path, const moe_ffn_desc* d, int64_t mk) {
  const int64_t M = d->M, H = d->H, I = d->I;
  if (path == MOE_PATH_DECODE) return mk * (I / 2) <= kMaxTasks && M * (H / 8) <= kMaxTasks;
  // Blocks of 64-column parts (blocks above 64 routes take several).
  const int64_t nblk = static_cast<int64_t>(capacity_of(d->M, d->k, d->E, d->b)) / d->b * ((d->b + 63) / 64);
  if (M * (H / 4) > kMaxTasks) return false;
  return nblk * ((I + 63) / 64) <= kMaxTasks && nblk * ((H + 127) / 128) <= kMaxTasks;
}

moe_status validate(const moe_ffn_desc* d, Layout* L, bool need_align_buffers) {
  if (d == nullptr) return MOE_ERR_INVALID_ARG;
  if (d->M < 0 || d->H <= 0 || d->I <= 0 || d->E < 1 || d->k < 1 || d->b < 1) return MOE_ERR_INVALID_ARG;
  if (d->expert_base < 0 || d->expert_base > INT32_MAX - d->E) return MOE_ERR_INVALID_ARG;
  if (d->path < MOE_PATH_AUTO || d->path > MOE_PATH_GROUPED) return MOE_ERR_INVALID_ARG;
  if (d->max_workgroups < 0) return MOE_ERR_INVALID_ARG;
  if (d->w13.fmt != d->w2.fmt) return MOE_ERR_INVALID_ARG;
  if (d->w13.fmt != MOE_W_INT4_AWQ && d->w13.fmt != MOE_W_MXFP8) return MOE_ERR_INVALID_ARG;
  if (!weights_ok(d->w13) || !weights_ok(d->w2)) return MOE_ERR_INVALID_ARG;
  if ((d->H % 32) != 0 || (d->I % 32) != 0) return MOE_ERR_INVALID_ARG;
  if ((d->H % d->w13.group) != 0 || (d->I % d->w2.group) != 0) return MOE_ERR_INVALID_ARG;
  if ((d->w13.group % 32) != 0 || (d->w2.group % 32) != 0) return MOE_ERR_INVALID_ARG;
  if (d->w13.fmt == MOE_W_MXFP8 && (d->w13.group != 32 || d->w2.group != 32)) return MOE_ERR_INVALID_ARG;
  if (d->E > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  const int64_t mk = int64_t(d->M) * d->k;
  if (mk > kMaxRoutes) return MOE_ERR_UNSUPPORTED;

  int path = d->path;
  if (path == MOE_PATH_AUTO) {
    // The size-based choice, else the other path when its shape rules fail.
    path = auto_path(d);
    if (!shape_ok(path, d)) path = path == MOE_PATH_DECODE ? MOE_PATH_GROUPED : MOE_PATH_DECODE;
  }
  if (need_align_buffers) path = MOE_PATH_GROUPED;
  L->path = path;
  if (!shape_ok(path, d)) return MOE_ERR_UNSUPPORTED;
  if (!tasks_fit(path, d, mk)) return MOE_ERR_UNSUPPORTED;
  if (path == MOE_PATH_DECODE) {
    L->off_a = 0;
    L->off_aux = round256(size_t(mk) * d->I * sizeof(uint16_t));
    L->total = L->off_aux + round256(size_t(mk) * d->I * sizeof(uint16_t));
    if (L->total == 0) L->total = 256;
    return MOE_OK;
  }
  L->cap = capacity_of(d->M, d->k, d->E, d->b);
  size_t o = 0;
  L->off_sorted = o; o += round256(L->cap * sizeof(int32_t));
  L->off_blocks = o; o += round256((L->cap / d->b) * sizeof(int32_t));
  L->off_npad = o;   o += 256;
  L->align_ws = moe::align_ws_bytes(static_cast<int>(mk), d->E);
  L->off_align_ws = o; o += L->align_ws;
  L->off_a = o;      o += round256(size_t(mk) * d->I * sizeof(uint16_t));
  L->off_aux = o;    o += round256(size_t(mk) * ((d->I + 127) / 128) * 4 * sizeof(float));
  L->off_yhat = o;   o += round256(size_t(mk) * d->H * sizeof(float));
  L->total = o;
  return MOE_OK;
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

int kernel_count_of(const Layout& L, bool aligned_input) {
  if (L.path == MOE_PATH_DECODE) return 2;
  return aligned_input ? 3 : 4;
}


template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// Stages of one forward call: kStageGateUp = step (2) (with step (1) on the
// grouped path), kStageDown = steps (3)-(4).
constexpr int kStageGateUp = 1;
constexpr int kStageDown = 2;

// Enqueues the kernels of the requested stages. `align_src` is null for the
// normal path (alignment computed into the workspace) or the caller's
// alignment for moe_ffn_forward_aligned. Events, when given, bracket every
// kernel.
moe_status run_forward(const moe_ffn_desc* d, const Layout& L, int stages, const uint16_t* x,
                       const int32_t* ids, const float* w, float* y, void* ws,
                       const int32_t* a_sorted, const int32_t* a_blocks, const int32_t* a_npad,
                       size_t a_cap, hipStream_t s, hipEvent_t* ev, float* w13_out = nullptr) {
  // Profiled calls: kernel i records its start in ev[2i] and its end in
  // ev[2i + 1] (see moe::LaunchTiming); the timing is removed on every exit.
  int kidx = 0;
  moe::LaunchTiming timing{nullptr, nullptr};
  struct Uninstall {
    ~Uninstall() { moe::launch_timing() = nullptr; }
  } uninstall;
  const int nk = ev == nullptr ? 0 : kernel_count_of(L, a_sorted != nullptr);
  auto arm = [&](void) {
    if (ev == nullptr || kidx >= nk) {
      moe::launch_timing() = nullptr;
      return;
    }
    timing = moe::LaunchTiming{ev[2 * kidx], ev[2 * kidx + 1]};
    moe::launch_timing() = &timing;
  };
  auto mark = [&](void) -> moe_status {
    ++kidx;
    arm();
    return MOE_OK;
  };
  arm();
  moe_status st;
  if (L.path == MOE_PATH_DECODE) {
    moe::DecodeArgs p{};
    p.x = x; p.ids = ids; p.topk_w = w; p.w13 = d->w13; p.w2 = d->w2;
    p.a_hi = at<uint16_t>(ws, L.off_a); p.a_lo = at<uint16_t>(ws, L.off_aux); p.y = y;
    p.w13_out = w13_out;
    p.M = d->M; p.H = d->H; p.I = d->I; p.E = d->E; p.k = d->k;
    p.ebase = d->expert_base;
    p.max_workgroups = d->max_workgroups;
    if (stages & kStageGateUp) {
      if ((st = hip_status(moe::launch_decode_gate_up(p, s))) != MOE_OK) return st;
      if ((st = mark()) != MOE_OK) return st;
    }
    if (stages & kStageDown) {
      if ((st = hip_status(moe::launch_decode_down(p, s))) != MOE_OK) return st;
      if ((st = mark()) != MOE_OK) return st;
    }
    return MOE_OK;
  }
  moe::GroupedArgs p{};
  const int64_t mk = int64_t(d->M) * d->k;
  p.x = x; p.ids = ids; p.topk_w = w; p.w13 = d->w13; p.w2 = d->w2;
  p.a16 = at<uint16_t>(ws, L.off_a); p.a_scale = at<float>(ws, L.off_aux);
  p.yhat = at<float>(ws, L.off_yhat); p.y = y;
  p.w13_out = w13_out;
  p.M = d->M; p.H = d->H; p.I = d->I; p.E = d->E; p.k = d->k; p.b = d->b;
  p.ebase = d->expert_base;
  p.max_workgroups = d->max_workgroups;
  if (a_sorted == nullptr) {
    p.sorted = at<int32_t>(ws, L.off_sorted);
    p.blocks = at<int32_t>(ws, L.off_blocks);
    p.num_padded = at<int32_t>(ws, L.off_npad);
    p.nblk = static_cast<int>(L.cap / d->b);
    if (stages & kStageGateUp) {
      if ((st = hip_status(moe::launch_align(ids, static_cast<int>(mk), d->E, d->expert_base, d->b,
                                             at<int32_t>(ws, L.off_sorted), at<int32_t>(ws, L.off_blocks),
                                             at<int32_t>(ws, L.off_npad), static_cast<int>(L.cap),
                                             L.align_ws ? at<void>(ws, L.off_align_ws) : nullptr, L.align_ws,
                                             s))) != MOE_OK)
        return st;
      if ((st = mark()) != MOE_OK) return st;
    }
  } else {
    p.sorted = a_sorted; p.blocks = a_blocks; p.num_padded = a_npad;
    p.nblk = static_cast<int>(a_cap / d->b);
  }
  if (stages & kStageGateUp) {
    if ((st = hip_status(moe::launch_grouped_gate_up(p, s))) != MOE_OK) return st;
    if ((st = mark()) != MOE_OK) return st;
  }
  if (stages & kStageDown) {
    if ((st = hip_status(moe::launch_grouped_down(p, s))) != MOE_OK) return st;
    if ((st = mark()) != MOE_OK) return st;
    if ((st = hip_status(moe::launch_combine(p, s))) != MOE_OK) return st;
    if ((st = mark()) != MOE_OK) return st;
  }
  return MOE_OK;
}

moe_status check_io(const moe_ffn_desc* d, const uint16_t* x, const int32_t* ids, const float* w,
                    float* y, void* ws, size_t ws_bytes, const Layout& L) {
  if (x == nullptr || ids == nullptr || w == nullptr || y == nullptr || ws == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(ws, 256) || !aligned(ids, 4) || !aligned(w, 4))
    return MOE_ERR_INVALID_ARG;
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  (void)d;
  return MOE_OK;
}

// Device scratch of moe_ffn_forward_noalloc: the workspace of one forward
// call, for callers that cannot allocate. One copy per GPU, held from the
// code object's load until the process ends. Its name is a host-side stand-in
// in host code; the device address comes from hipGetSymbolAddress, once per
// device, with that device current.
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
constexpr int kNoAllocMaxDevices = 64;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kNoAllocMaxDevices] = {};

// The current device's scratch address, looked up on its first use.
moe_status scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kNoAllocMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_align_capacity(int32_t M, int32_t k, int32_t E, int32_t b) {
  if (M < 0 || k < 1 || E < 1 || b < 1) return 0;
  return capacity_of(M, k, E, b);
}

moe_status moe_align_ex(const int32_t* topk_ids, int32_t M, int32_t k, int32_t E, int32_t expert_base,
                        int32_t b, int32_t* sorted_route_ids, int32_t* expert_block_ids, int32_t* num_padded,
                        size_t capacity, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (M < 0 || k < 1 || E < 1 || b < 1) return MOE_ERR_INVALID_ARG;
  if (expert_base < 0 || expert_base > INT32_MAX - E) return MOE_ERR_INVALID_ARG;
  if (M == 0) return MOE_OK;
  if (topk_ids == nullptr || sorted_route_ids == nullptr || expert_block_ids == nullptr ||
      num_padded == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (E > kMaxExperts || int64_t(M) * k > kMaxRoutes) return MOE_ERR_UNSUPPORTED;
  const size_t need = capacity_of(M, k, E, b);
  if (capacity < need) return MOE_ERR_CAPACITY;
  if (capacity > size_t(INT32_MAX)) return MOE_ERR_UNSUPPORTED;
  const size_t ws_need = moe::align_ws_bytes(M * k, E);
  if (ws_need > 0 && ws != nullptr) {
    if (!aligned(ws, 256)) return MOE_ERR_INVALID_ARG;
    if (ws_bytes < ws_need) return MOE_ERR_WORKSPACE;
  }
  return hip_status(moe::launch_align(topk_ids, M * k, E, expert_base, b, sorted_route_ids, expert_block_ids,
                                      num_padded, static_cast<int>(capacity), ws, ws_bytes, stream));
}

moe_status moe_align(const int32_t* topk_ids, int32_t M, int32_t k, int32_t E, int32_t b,
                     int32_t* sorted_route_ids, int32_t* expert_block_ids, int32_t* num_padded,
                     size_t capacity, hipStream_t stream) {
  return moe_align_ex(topk_ids, M, k, E, 0, b, sorted_route_ids, expert_block_ids, num_padded, capacity,
                      nullptr, 0, stream);
}

moe_status moe_align_ex_workspace_size(int32_t M, int32_t k, int32_t E, size_t* bytes) {
  if (bytes == nullptr || M < 0 || k < 1 || E < 1) return MOE_ERR_INVALID_ARG;
  if (E > kMaxExperts || int64_t(M) * k > kMaxRoutes) return MOE_ERR_UNSUPPORTED;
  *bytes = moe::align_ws_bytes(M * k, E);
  return MOE_OK;
}

moe_status moe_ffn_workspace_size(const moe_ffn_desc* d, size_t* bytes) {
  if (bytes == nullptr) return MOE_ERR_INVALID_ARG;
  Layout L;
  const moe_status st = validate(d, &L, false);
  if (st != MOE_OK) return st;
  *bytes = L.total;
  return MOE_OK;
}

moe_status moe_ffn_forward(const moe_ffn_desc* d, const uint16_t* x, const int32_t* topk_ids,
                           const float* topk_w, float* y, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  Layout L;
  moe_status st = validate(d, &L, false);
  if (st != MOE_OK) return st;
  if (d->M == 0) return MOE_OK;
  if ((st = check_io(d, x, topk_ids, topk_w, y, ws, ws_bytes, L)) != MOE_OK) return st;
  return run_forward(d, L, kStageGateUp | kStageDown, x, topk_ids, topk_w, y, ws, nullptr, nullptr, nullptr, 0,
                     stream, nullptr);
}

size_t moe_ffn_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

moe_status moe_ffn_forward_noalloc(const moe_ffn_desc* d, const uint16_t* x, const int32_t* topk_ids,
                                   const float* topk_w, float* y, hipStream_t stream) {
  Layout L;
  moe_status st = validate(d, &L, false);
  if (st != MOE_OK) return st;
  if (d->M == 0) return MOE_OK;
  if (L.total > kNoAllocScratchBytes) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  if ((st = scratch_for_current_device(&ws)) != MOE_OK) return st;
  if ((st = check_io(d, x, topk_ids, topk_w, y, ws, kNoAllocScratchBytes, L)) != MOE_OK) return st;
  return run_forward(d, L, kStageGateUp | kStageDown, x, topk_ids, topk_w, y, ws, nullptr, nullptr, nullptr, 0,
                     stream, nullptr);
}

moe_status moe_ffn_forward_aligned(const moe_ffn_desc* d, const uint16_t* x,
                                   const int32_t* topk_ids, const float* topk_w,
                                   const int32_t* sorted_route_ids,
                                   const int32_t* expert_block_ids,
                                   const int32_t* num_padded, size_t capacity, float* y,
                                   void* ws, size_t ws_bytes, hipStream_t stream) {
  Layout L;
  moe_status st = validate(d, &L, true);
  if (st != MOE_OK) return st;
  if (d->M == 0) return MOE_OK;
  if ((st = check_io(d, x, topk_ids, topk_w, y, ws, ws_bytes, L)) != MOE_OK) return st;
  if (sorted_route_ids == nullptr || expert_block_ids == nullptr || num_padded == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (capacity % size_t(d->b) != 0 || capacity > size_t(INT32_MAX)) return MOE_ERR_INVALID_ARG;
  if (capacity < capacity_of(d->M, d->k, d->E, d->b)) return MOE_ERR_CAPACITY;
  return run_forward(d, L, kStageGateUp | kStageDown, x, topk_ids, topk_w, y, ws, sorted_route_ids,
                     expert_block_ids, num_padded, capacity, stream, nullptr);
}

moe_status moe_ffn_forward_capture(const moe_ffn_desc* d, const uint16_t* x, const int32_t* topk_ids,
                                   const float* topk_w, float* y, void* ws, size_t ws_bytes, float* w13_out,
                                   hipStream_t stream) {
  Layout L;
  moe_status st = validate(d, &L, false);
  if (st != MOE_OK) return st;
  if (d->M == 0) return MOE_OK;
  if ((st = check_io(d, x, topk_ids, topk_w, y, ws, ws_bytes, L)) != MOE_OK) return st;
  if (w13_out == nullptr || !aligned(w13_out, 16)) return MOE_ERR_INVALID_ARG;
  return run_forward(d, L, kStageGateUp | kStageDown, x, topk_ids, topk_w, y, ws, nullptr, nullptr, nullptr, 0,
                     stream, nullptr, w13_out);
}

moe_status moe_ffn_forward_profiled(const moe_ffn_desc* d, const uint16_t* x,
                                    const int32_t* topk_ids, const float* topk_w, float* y,
                                    void* ws, size_t ws_bytes, hipStream_t stream,
                                    hipEvent_t* events, int32_t n_events) {
  Layout L;
  moe_status st = validate(d, &L, false);
  if (st != MOE_OK) return st;
  if (d->M == 0) return MOE_OK;
  if ((st = check_io(d, x, topk_ids, topk_w, y, ws, ws_bytes, L)) != MOE_OK) return st;
  if (events == nullptr || n_events != 2 * kernel_count_of(L, false)) return MOE_ERR_INVALID_ARG;
  for (int i = 0; i < n_events; ++i)
    if (events[i] == nullptr) return MOE_ERR_INVALID_ARG;
  return run_forward(d, L, kStageGateUp | kStageDown, x, topk_ids, topk_w, y, ws, nullptr, nullptr, nullptr, 0,
                     stream, events);
}

moe_status moe_ffn_gate_up(const moe_ffn_desc* d, const uint16_t* x, const int32_t* topk_ids,
                           void* ws, size_t ws_bytes, hipStream_t stream) {
  Layout L;
  moe_status st = validate(d, &L, false);
  if (st != MOE_OK) return st;
  if (d->M == 0) return MOE_OK;
  if (x == nullptr || topk_ids == nullptr || ws == nullptr) return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(ws, 256) || !aligned(topk_ids, 4)) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  return run_forward(d, L, kStageGateUp, x, topk_ids, nullptr, nullptr, ws, nullptr, nullptr, nullptr, 0,
                     stream, nullptr);
}

moe_status moe_ffn_down_combine(const moe_ffn_desc* d, const int32_t* topk_ids, const float* topk_w,
                                float* y, void* ws, size_t ws_bytes, hipStream_t stream) {
  Layout L;
  moe_status st = validate(d, &L, false);
  if (st != MOE_OK) return st;
  if (d->M == 0) return MOE_OK;
  if (topk_ids == nullptr || topk_w == nullptr || y == nullptr || ws == nullptr) return MOE_ERR_INVALID_ARG;
  if (!aligned(y, 16) || !aligned(ws, 256) || !aligned(topk_ids, 4) || !aligned(topk_w, 4))
    return MOE_ERR_INVALID_ARG;
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  return run_forward(d, L, kStageDown, nullptr, topk_ids, topk_w, y, ws, nullptr, nullptr, nullptr, 0,
                     stream, nullptr);
}

}  // extern "C"

namespace {

// Validation of the batched-layout GEMM calls: the layer shape and weights
// as for moe_ffn_forward (M, k, path and expert_base are not used), the
// grouped path's shape rules, and a capacity whose row indices fit int32.
moe_status validate_batched(const moe_ffn_desc* d, int32_t capacity) {
  if (d == nullptr || capacity < 1) return MOE_ERR_INVALID_ARG;
  moe_ffn_desc t = *d;
  t.M = 1;
  t.k = 1;
  t.path = MOE_PATH_GROUPED;
  t.expert_base = 0;
  Layout L;
  const moe_status st = validate(&t, &L, true);
  if (st != MOE_OK) return st;
  if (int64_t(d->E) * capacity > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  // GEMM tasks: E * ceil(capacity / b) blocks times the tiles per block.
  const int64_t nblk = int64_t(d->E) * ((int64_t(capacity) + d->b - 1) / d->b) * ((d->b + 63) / 64);
  if (nblk * ((d->I + 63) / 64) > kMaxTasks || nblk * ((d->H + 127) / 128) > kMaxTasks) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe::GroupedArgs batched_args(const moe_ffn_desc* d) {
  moe::GroupedArgs p{};
  p.w13 = d->w13;
  p.w2 = d->w2;
  p.H = d->H; p.I = d->I; p.E = d->E; p.b = d->b;
  p.max_workgroups = d->max_workgroups;
  return p;
}

}  // namespace

extern "C" {

moe_status moe_ffn_gate_up_batched(const moe_ffn_desc* d, const uint16_t* xb, const int32_t* counts,
                                   int32_t capacity, uint16_t* a16, float* a_scale, hipStream_t stream) {
  moe_status st = validate_batched(d, capacity);
  if (st != MOE_OK) return st;
  if (xb == nullptr || counts == nullptr || a16 == nullptr || a_scale == nullptr) return MOE_ERR_INVALID_ARG;
  if (!aligned(xb, 16) || !aligned(a16, 16) || !aligned(a_scale, 16) || !aligned(counts, 4))
    return MOE_ERR_INVALID_ARG;
  moe::GroupedArgs p = batched_args(d);
  p.x = xb;
  p.a16 = a16;
  p.a_scale = a_scale;
  return hip_status(moe::launch_grouped_gate_up_batched(p, counts, capacity, stream));
}

moe_status moe_ffn_down_batched(const moe_ffn_desc* d, const uint16_t* a16, const float* a_scale,
                                const int32_t* counts, int32_t capacity, float* yb, hipStream_t stream) {
  moe_status st = validate_batched(d, capacity);
  if (st != MOE_OK) return st;
  if (a16 == nullptr || a_scale == nullptr || counts == nullptr || yb == nullptr) return MOE_ERR_INVALID_ARG;
  if (!aligned(a16, 16) || !aligned(a_scale, 16) || !aligned(yb, 16) || !aligned(counts, 4))
    return MOE_ERR_INVALID_ARG;
  moe::GroupedArgs p = batched_args(d);
  p.a16 = const_cast<uint16_t*>(a16);        // read only: the down GEMM's input
  p.a_scale = const_cast<float*>(a_scale);
  p.yhat = yb;
  return hip_status(moe::launch_grouped_down_batched(p, counts, capacity, stream));
}

int32_t moe_ffn_kernel_count(const moe_ffn_desc* d) {
  Layout L;
  if (validate(d, &L, false) != MOE_OK) return 0;
  return kernel_count_of(L, false);
}

const char* moe_ffn_kernel_name(const moe_ffn_desc* d, int32_t i) {
  Layout L;
  if (validate(d, &L, false) != MOE_OK) return nullptr;
  // Kernel template names as a kernel trace shows them (before the template
  // arguments); the grouped GEMM is one template run for both projections.
  static const char* const kDecode[] = {"decode_gate_up", "decode_down"};
  static const char* const kGrouped[] = {"align_kernel", "grouped_gemm (gate/up)", "grouped_gemm (down)",
                                         "combine_topk"};
  if (L.path == MOE_PATH_DECODE) return (i >= 0 && i < 2) ? kDecode[i] : nullptr;
  return (i >= 0 && i < 4) ? kGrouped[i] : nullptr;
}

moe_status moe_ffn_intermediate(const moe_ffn_desc* d, size_t* offset, size_t* aux_offset,
                                int32_t* format) {
  if (offset == nullptr || aux_offset == nullptr || format == nullptr) return MOE_ERR_INVALID_ARG;
  Layout L;
  const moe_status st = validate(d, &L, false);
  if (st != MOE_OK) return st;
  *offset = L.off_a;
  *aux_offset = L.off_aux;
  *format = L.path == MOE_PATH_DECODE ? 1 : 2;
  return MOE_OK;
}

moe_status moe_ffn_route_outputs(const moe_ffn_desc* d, size_t* offset) {
  if (offset == nullptr) return MOE_ERR_INVALID_ARG;
  Layout L;
  const moe_status st = validate(d, &L, false);
  if (st != MOE_OK) return st;
  if (L.path != MOE_PATH_GROUPED) return MOE_ERR_UNSUPPORTED;
  *offset = L.off_yhat;
  return MOE_OK;
}

int32_t moe_ffn_auto_decode_max_m(void) { return kAutoDecodeMaxM; }

int32_t moe_ffn_resolved_path(const moe_ffn_desc* d) {
  Layout L;
  if (validate(d, &L, false) != MOE_OK) return -1;
  return L.path;
}

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape, format or path";
    case MOE_ERR_CAPACITY: return "alignment capacity too small";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

}  // extern "C"
