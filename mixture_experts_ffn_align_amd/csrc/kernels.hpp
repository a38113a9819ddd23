// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_ffn.h"

namespace moe {

// Per-kernel timing of moe_ffn_forward_profiled: while a LaunchTiming is
// installed (one per host thread), every launch records the kernel's own
// start and end timestamps into these events (hipExtLaunchKernel); the start
// event is consumed by the first launch of a stage, the end event is
// re-recorded by each launch, so a stage of several launches spans them all.
struct LaunchTiming {
  hipEvent_t start;
  hipEvent_t stop;
};
LaunchTiming*& launch_timing();

template <typename... KArgs, typename... Args>
void launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t lds_bytes, hipStream_t stream,
            Args... args) {
  LaunchTiming* t = launch_timing();
  if (t == nullptr) {
    hipLaunchKernelGGL(kernel, grid, block, lds_bytes, stream, args...);
  } else {
    hipExtLaunchKernelGGL(kernel, grid, block, lds_bytes, stream, t->start, t->stop, 0, args...);
    t->start = nullptr;
  }
}

// Every kernel strides over its tasks, so its grid may be smaller than its
// task count; launches are capped at kMaxGrid workgroups (and at a caller's
// max_workgroups > 0), which keeps the work-item count of a dispatch within
// 32 bits. Task counts themselves are int32 (the C ABI rejects larger layers).
constexpr int64_t kMaxGrid = int64_t(1) << 20;
inline int grid_for(int64_t work_groups, int max_workgroups) {
  if (work_groups < 1) work_groups = 1;
  if (work_groups > kMaxGrid) work_groups = kMaxGrid;
  return (max_workgroups > 0 && max_workgroups < work_groups) ? max_workgroups : static_cast<int>(work_groups);
}

// Route alignment (align.hip). Up to kAlignSingleMaxRoutes routes run as one
// workgroup; more (with a workspace of align_ws_bytes) as three launches over
// workgroups of kAlignRoutesPerGroup routes. Experts [ebase, ebase + E) are
// held here.
constexpr int kAlignSingleMaxRoutes = 8192;
constexpr int kAlignRoutesPerGroup = 4096;
size_t align_lds_bytes(int E);
size_t align_ws_bytes(int mk, int E);
hipError_t launch_align(const int32_t* ids, int mk, int E, int ebase, int b, int32_t* sorted, int32_t* blocks,
                        int32_t* num_padded, int cap, void* ws, size_t ws_bytes, hipStream_t stream);

// Decode path (decode.hip).
struct DecodeArgs {
  const uint16_t* x;
  const int32_t* ids;
  const float* topk_w;
  moe_weights w13, w2;
  uint16_t* a_hi;  // bf16 [M*k][I] intermediate, high part
  uint16_t* a_lo;  // bf16 [M*k][I] intermediate, low part
  float* w13_out;  // fp32 [M*k][2I] W13 outputs (gate, up) or null: capture surface
  float* y;        // fp32 [M][H]
  int M, H, I, E, k;
  int ebase;       // experts [ebase, ebase + E) are held here
  int max_workgroups;
};
bool decode_shape_ok(int fmt, int H, int I, int k, int g13, int g2);
hipError_t launch_decode_gate_up(const DecodeArgs& p, hipStream_t stream);
hipError_t launch_decode_down(const DecodeArgs& p, hipStream_t stream);

// Grouped path (grouped.hip).
struct GroupedArgs {
  const uint16_t* x;
  const int32_t* ids;
  const float* topk_w;
  const int32_t* sorted;
  const int32_t* blocks;
  const int32_t* num_padded;
  moe_weights w13, w2;
  uint16_t* a16;   // fp16 [M*k][I] intermediate, each 64-neuron chunk of a route scaled by a power of two
  float* a_scale;  // fp32 [M*k][ceil(I/128)][4]: entries 0 and 1 undo the scaling of the slab's two chunks
  float* yhat;     // fp32 [M*k][H]
  float* w13_out;  // fp32 [M*k][2I] W13 outputs (gate, up) or null: capture surface
  float* y;        // fp32 [M][H]
  int M, H, I, E, k, b;
  int ebase;       // experts [ebase, ebase + E) are held here
  int nblk;        // blocks in the alignment buffers (capacity / b)
  int max_workgroups;
};
bool grouped_shape_ok(int fmt, int H, int I, int b, int g13, int g2);
hipError_t launch_grouped_gate_up(const GroupedArgs& p, hipStream_t stream);
hipError_t launch_grouped_down(const GroupedArgs& p, hipStream_t stream);
hipError_t launch_combine(const GroupedArgs& p, hipStream_t stream);

// The two grouped GEMMs on the fixed-capacity batched layout: expert e's rows
// are e * cap .. e * cap + counts[e] - 1 of x / the intermediate (a16 and
// a_scale) / yhat (counts on the device, clamped to [0, cap]); rows past the
// count are not read or written. Uses x, w13, w2, a16, a_scale, yhat, H, I,
// E, b and max_workgroups of p.
hipError_t launch_grouped_gate_up_batched(const GroupedArgs& p, const int32_t* counts, int cap, hipStream_t stream);
hipError_t launch_grouped_down_batched(const GroupedArgs& p, const int32_t* counts, int cap, hipStream_t stream);

}  // namespace moe
