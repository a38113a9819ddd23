/*
 * moe_ffn.h — C ABI of the MI355X (gfx950) routed MoE expert-FFN layer.
 *
 * The layer computes, for M tokens each routed to k of E experts,
 *   (1) route alignment: group the M*k flattened routes by expert in route-ID
 *       order, pad each expert's count to a multiple of b, and emit the
 *       expert-block vector;
 *   (2) gate/up projection over packed 4-bit AWQ-style group-quantised expert
 *       weights with the SwiGLU activation silu(gate) * up;
 *   (3) the down projection;
 *   (4) the router-weighted top-k combine.
 * Steps (1) and the packed-weight format follow "Route-Block Membership Selects
 * Packed-AWQ Arithmetic" (arXiv 2607.26316: first paragraph, the A_e / B(e,j)
 * paragraph, the stable-construction paragraph, and the fixture paragraph for
 * 4-bit AWQ with group 128). Steps (2)-(4) follow "Hardware-Native Joint
 * Sparse-Quantization for Trillion-Scale MoE" (arXiv 2610.02241, Sections 2,
 * 3.3 with Eq. 4, 3.4) and the warp-decode write-up (cursor.com blog, "Cómo
 * funcionan los dos kernels").
 *
 * Conventions for every entry point:
 *   - Every array pointer is DEVICE memory owned by the caller. The library
 *     allocates nothing, keeps no pointer after returning, and never
 *     synchronises the host: work is enqueued on `stream` and the buffers must
 *     stay valid until it completes.
 *   - Host-checkable errors return a status synchronously and enqueue nothing.
 *     Launch failures return MOE_ERR_HIP. M == 0 is a no-op returning MOE_OK.
 *   - Data-dependent conditions are defined behaviour, not errors: an expert
 *     ID outside the experts held here ([expert_base, expert_base + E); [0, E)
 *     for moe_align) marks an invalid route, which alignment skips and which
 *     contributes nothing to the output.
 *   - Results are deterministic: the same inputs, shapes and path give the
 *     same output bytes on every run and for every workgroup cap (no
 *     floating-point atomics; every reduction has a fixed order).
 *   - Route IDs are the row-major flattening r = t*k + j of the [M][k]
 *     top-k arrays; token(r) = r / k.
 */
#ifndef MOE_FFN_H
#define MOE_FFN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef MOE_API
#define MOE_API __attribute__((visibility("default")))
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,  /* null pointer, negative or inconsistent sizes */
  MOE_ERR_UNSUPPORTED = 2,  /* shape/format/path combination not implemented */
  MOE_ERR_CAPACITY = 3,     /* alignment buffers smaller than moe_align_capacity */
  MOE_ERR_WORKSPACE = 4,    /* workspace smaller than moe_ffn_workspace_size */
  MOE_ERR_HIP = 5           /* a HIP launch failed */
} moe_status;

typedef enum {
  MOE_W_INT4_AWQ = 0,  /* q: uint32 [E][N][K/8]; word kk/8 holds elements 8*(kk/8)..+7
                          in AWQ's interleaved order: nibble slot i (bits 4i..4i+3)
                          holds element [0,2,4,6,1,3,5,7][i];
                          scale: fp16 [E][N][K/group]; zero: uint8 [E][N][K/group] in 0..15;
                          w = (q - zero) * scale */
  MOE_W_MXFP8 = 1      /* q: uint8 OCP E4M3FN [E][N][K]; scale: uint8 E8M0 [E][N][K/32];
                          zero: NULL; w = e4m3(q) * 2^(scale - 127); group must be 32 */
} moe_wfmt;

typedef enum {
  MOE_PATH_AUTO = 0,     /* decode for M <= moe_ffn_auto_decode_max_m(), else grouped; when the
                            chosen path's shape rules fail, the other path */
  MOE_PATH_DECODE = 1,   /* output-stationary: one wave64 per output neuron set, no alignment */
  MOE_PATH_GROUPED = 2   /* alignment + LDS-dequantised MFMA grouped GEMMs + combine; needs H and I
                            multiples of 32 (as every path), b <= 1024, at most 256 scale groups
                            per row (K/group; MXFP8: K/32) whose scales and zeros fit one CU's
                            LDS beside the tile's ring, and (int4) group dividing 128 or a
                            multiple of it */
} moe_path;

/* One projection's resident packed weights for all E experts. */
typedef struct {
  int32_t fmt;          /* moe_wfmt */
  int32_t group;        /* elements per scale group along K (int4: multiple of 32; mxfp8: 32) */
  const void* q;        /* packed values, layout per moe_wfmt */
  const void* scale;    /* per-group scales, layout per moe_wfmt */
  const uint8_t* zero;  /* int4 zero points, NULL for MXFP8 */
} moe_weights;

/* Layer description. W13 has N = 2*I rows (rows 0..I-1 gate, I..2I-1 up) and
 * K = H; W2 has N = H rows and K = I. Both projections must use the same fmt. */
typedef struct {
  int32_t M;               /* tokens (>= 0) */
  int32_t H;               /* hidden size, multiple of 32 and of w13.group */
  int32_t I;               /* per-expert intermediate size, multiple of 32 and of w2.group */
  int32_t E;               /* experts held here (1..2048): IDs expert_base .. expert_base + E - 1 */
  int32_t k;               /* routes per token (>= 1) */
  int32_t b;               /* alignment block size used by the grouped path (>= 1; the
                              grouped GEMMs take b <= 1024, in parts of up to 64 routes) */
  moe_weights w13;
  moe_weights w2;
  int32_t path;            /* moe_path */
  int32_t max_workgroups;  /* 0: library default grid. > 0: cap on workgroups per launch.
                              Output bytes do not depend on it. */
  int32_t expert_base;     /* first expert ID held here (>= 0; 0 for a whole layer). A route
                              whose ID lies outside [expert_base, expert_base + E) is skipped,
                              so the E experts of one expert-parallel shard compute that
                              shard's share of y; w13 / w2 hold those E experts, ID e at
                              index e - expert_base. */
} moe_ffn_desc;

/* Number of int32 entries sorted_route_ids needs: roundup(M*k + min(E, M*k)*(b-1), b).
 * The alignment ("Route-Block Membership Selects Packed-AWQ Arithmetic", first
 * paragraph) pads each expert's count to a multiple of b, so every expert that
 * holds a route adds at most b - 1 padding rows, and at most min(E, M*k) experts
 * hold one; the page gives no buffer size, and this bound is the plainest one.
 * expert_block_ids needs capacity / b entries. Host-only and pure; returns 0 when
 * M < 0, k < 1, E < 1 or b < 1. */
MOE_API size_t moe_align_capacity(int32_t M, int32_t k, int32_t E, int32_t b);

/* Step (1), route alignment ("Route-Block Membership Selects Packed-AWQ
 * Arithmetic": first paragraph; A_e / B(e,j) paragraph; stable-construction
 * paragraph). Same as moe_align_ex with expert_base 0 and no workspace.
 *   topk_ids          [M*k] int32, row-major [M][k]
 *   sorted_route_ids  [capacity] out: for each expert e ascending, its valid route
 *                     IDs in ascending order, then the sentinel M*k up to a multiple
 *                     of b; positions num_padded..capacity-1 hold the sentinel.
 *   expert_block_ids  [capacity/b] out: expert of each b-row block; -1 past the end.
 *   num_padded        [1] out: total aligned rows, sum_e ceil(c_e/b)*b.
 * Runs as one workgroup (M*k up to 2^24 routes, E <= 2048).
 * Errors: MOE_ERR_INVALID_ARG (null pointers, M < 0, k < 1, E < 1, b < 1),
 * MOE_ERR_UNSUPPORTED (E > 2048 or M*k > 2^24), MOE_ERR_CAPACITY (capacity too small). */
MOE_API moe_status moe_align(const int32_t* topk_ids, int32_t M, int32_t k, int32_t E, int32_t b,
                     int32_t* sorted_route_ids, int32_t* expert_block_ids, int32_t* num_padded,
                     size_t capacity, hipStream_t stream);

/* Step (1) for the experts held here and at any size: only routes whose ID
 * lies in [expert_base, expert_base + E) are valid, and expert_block_ids holds
 * local indices e - expert_base (an expert-parallel shard aligns its own
 * routes; the pages' stable order and padding apply unchanged to the valid
 * routes). Outputs, capacity (with E the number of experts held here) and
 * errors as moe_align, plus MOE_ERR_INVALID_ARG for expert_base < 0 or
 * expert_base + E > INT32_MAX, and MOE_ERR_WORKSPACE for a workspace smaller
 * than moe_align_ex_workspace_size.
 *   ws, ws_bytes  device scratch (256-byte aligned) of moe_align_ex_workspace_size
 *                 bytes, or NULL. With it, more than 8192 routes run as three
 *                 launches over workgroups of 4096 routes (per-workgroup histogram,
 *                 per-expert prefix over workgroups, stable scatter); without it,
 *                 or for fewer routes, as one workgroup. The output is the same. */
MOE_API moe_status moe_align_ex(const int32_t* topk_ids, int32_t M, int32_t k, int32_t E,
                                int32_t expert_base, int32_t b, int32_t* sorted_route_ids,
                                int32_t* expert_block_ids, int32_t* num_padded, size_t capacity,
                                void* ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes of moe_align_ex for M*k routes over E experts (0 when one
 * workgroup runs it). Errors: MOE_ERR_INVALID_ARG (null bytes, M < 0, k < 1,
 * E < 1), MOE_ERR_UNSUPPORTED (E > 2048 or M*k > 2^24). */
MOE_API moe_status moe_align_ex_workspace_size(int32_t M, int32_t k, int32_t E, size_t* bytes);

/* Bytes of device workspace moe_ffn_forward needs for this description (path
 * resolved as moe_ffn_forward resolves it). The workspace holds what the layer
 * keeps on the device between its steps: the alignment outputs (grouped path;
 * counts stay device-resident as in "Hardware-Native Joint Sparse-Quantization
 * for Trillion-Scale MoE", App. D.1, so no host synchronisation sizes anything),
 * the route-indexed activation silu(gate)*up and, on the grouped path, the
 * routed-W2 rows yhat: the intermediate surfaces that "Route-Block Membership
 * Selects Packed-AWQ Arithmetic" captures (the paragraph on the sparse native
 * differences). Errors as moe_ffn_forward's validation. */
MOE_API moe_status moe_ffn_workspace_size(const moe_ffn_desc* d, size_t* bytes);

/* Steps (1)-(4): y = sum_j w[t,j] * W2[e] (silu(W13g[e] x_t) * W13u[e] x_t).
 *   x         [M][H] bf16 bit patterns
 *   topk_ids  [M][k] int32 expert IDs (out-of-range IDs are skipped)
 *   topk_w    [M][k] fp32 combine weights, used as given
 *   y         [M][H] fp32, overwritten
 *   ws        workspace of at least moe_ffn_workspace_size bytes, 256-byte aligned
 * The decode path needs no alignment (the output-stationary design of the
 * warp-decode write-up, "Eliminación del relleno"); the grouped path runs
 * moe_align into the workspace first. The route-indexed intermediate
 * silu(gate)*up is left in the workspace (see moe_ffn_intermediate).
 * Errors: MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED (the path's shape rules, or
 * a layer whose kernels would have more than 2^30 tasks), MOE_ERR_WORKSPACE,
 * MOE_ERR_HIP. */
MOE_API moe_status moe_ffn_forward(const moe_ffn_desc* d, const uint16_t* x, const int32_t* topk_ids,
                           const float* topk_w, float* y, void* ws, size_t ws_bytes,
                           hipStream_t stream);

/* moe_ffn_forward without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). The library keeps one static device
 * scratch buffer of moe_ffn_noalloc_max_bytes() bytes (32 MiB) per GPU, held
 * from the first use on that GPU until the process ends; its address is looked
 * up once per device. This call allocates nothing, launches the same kernels
 * as moe_ffn_forward with that buffer as the workspace, and gives the same
 * output bytes. No part of the scratch needs clearing (every region the layer
 * reads is written earlier in the same call). Calls that overlap in time on
 * one GPU share the buffer and race: serialise them (one stream, or events).
 * The intermediate and yhat of the last call stay in the scratch but are not
 * exposed.
 * Errors as moe_ffn_forward, and MOE_ERR_WORKSPACE when the layer needs more
 * than moe_ffn_noalloc_max_bytes() of workspace (moe_ffn_workspace_size). */
MOE_API moe_status moe_ffn_forward_noalloc(const moe_ffn_desc* d, const uint16_t* x,
                                           const int32_t* topk_ids, const float* topk_w, float* y,
                                           hipStream_t stream);

/* Bytes of the static scratch moe_ffn_forward_noalloc uses per GPU. */
MOE_API size_t moe_ffn_noalloc_max_bytes(void);

/* Grouped path (whatever d->path says) on a caller-supplied alignment (same
 * layout and meaning as moe_align's outputs, with the given capacity). Lets a
 * caller reorder routes within an expert's rows: "Route-Block Membership
 * Selects Packed-AWQ Arithmetic" (the A_e / B(e,j) paragraph, and the paragraph
 * on reordering routes 22 and 28 inside block 40) states that swapping two
 * valid routes inside one B(e,j) leaves the computation's identity unchanged;
 * here the output bytes must not change for any order within an expert. Route entries
 * outside [0, M*k) are padding; blocks whose expert is outside [0, E) are skipped.
 * Each valid route must appear at most once. The workspace must be sized with
 * d->path = MOE_PATH_GROUPED. Errors as moe_ffn_forward. */
MOE_API moe_status moe_ffn_forward_aligned(const moe_ffn_desc* d, const uint16_t* x,
                                   const int32_t* topk_ids, const float* topk_w,
                                   const int32_t* sorted_route_ids,
                                   const int32_t* expert_block_ids,
                                   const int32_t* num_padded, size_t capacity, float* y,
                                   void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_ffn_forward that also writes the W13 outputs of every valid route,
 * the sums the gate/up kernels form before the activation: w13_out fp32
 * [M*k][2I], columns 0..I-1 gate = W13g[e] x_t and I..2I-1 up = W13u[e] x_t
 * (16-byte aligned, device, caller-owned; rows of invalid routes are left as
 * they were). With the intermediate (moe_ffn_intermediate), the grouped
 * path's routed-W2 rows (moe_ffn_route_outputs) and y, these are the four
 * surfaces "Route-Block Membership Selects Packed-AWQ Arithmetic" captures
 * (W13 output, activation, routed-W2 output, final output; the paragraph on
 * the sparse native differences). The same kernels run, with one extra store
 * per output; y and the other surfaces are bitwise those of moe_ffn_forward.
 * Errors as moe_ffn_forward, and MOE_ERR_INVALID_ARG for a null or
 * misaligned w13_out. */
MOE_API moe_status moe_ffn_forward_capture(const moe_ffn_desc* d, const uint16_t* x, const int32_t* topk_ids,
                                           const float* topk_w, float* y, void* ws, size_t ws_bytes,
                                           float* w13_out, hipStream_t stream);

/* Same as moe_ffn_forward, and records the start and end of kernel i (in
 * launch order, the kernels moe_ffn_kernel_name lists) into events[2i] and
 * events[2i + 1] (n_events must be 2 * moe_ffn_kernel_count): the kernel's own
 * dispatch timestamps (hipExtLaunchKernel), so that hipEventElapsedTime of the
 * pair is the kernel's duration with no launch gap around it. A kernel made of
 * several launches (alignment of more than 8192 routes) spans from the first
 * launch's start to the last one's end. Events are caller-created; not for use
 * under graph capture. */
MOE_API moe_status moe_ffn_forward_profiled(const moe_ffn_desc* d, const uint16_t* x,
                                    const int32_t* topk_ids, const float* topk_w, float* y,
                                    void* ws, size_t ws_bytes, hipStream_t stream,
                                    hipEvent_t* events, int32_t n_events);

/* Step (2) alone (preceded by step (1) on the grouped path): enqueues the
 * kernels of moe_ffn_forward up to the intermediate silu(gate)*up, which is
 * left in the workspace (see moe_ffn_intermediate). Lets a caller inspect or
 * time the stages separately. Arguments and errors as moe_ffn_forward. */
MOE_API moe_status moe_ffn_gate_up(const moe_ffn_desc* d, const uint16_t* x, const int32_t* topk_ids,
                                   void* ws, size_t ws_bytes, hipStream_t stream);

/* Steps (3)-(4) alone: the down projection and the top-k combine, reading the
 * intermediate (and, on the grouped path, the alignment) that a preceding
 * moe_ffn_gate_up call with the same description and topk_ids left in ws.
 * moe_ffn_gate_up followed by moe_ffn_down_combine gives the same bytes as
 * moe_ffn_forward. Arguments and errors as moe_ffn_forward. */
MOE_API moe_status moe_ffn_down_combine(const moe_ffn_desc* d, const int32_t* topk_ids,
                                        const float* topk_w, float* y, void* ws, size_t ws_bytes,
                                        hipStream_t stream);

/* The grouped path's two GEMMs on a fixed-capacity batched layout (the
 * layout of "Hardware-Native Joint Sparse-Quantization for Trillion-Scale
 * MoE", App. D.1: every expert's operands at a fixed stride, token counts
 * kept on the device, a partial last tile per expert). Expert e (weight index
 * e, 0 <= e < E) owns rows e*capacity .. e*capacity + counts[e] - 1 of every
 * batched operand; counts[e] is read on the device and clamped to
 * [0, capacity]; rows past it are neither read nor written.
 *   xb        bf16 [E][capacity][H]            (gate/up input)
 *   a16       fp16 [E][capacity][I] and
 *   a_scale   fp32 [E][capacity][ceil(I/128)][4]: silu(gate)*up in format 2 of
 *             moe_ffn_intermediate (gate/up output, down input)
 *   yb        fp32 [E][capacity][H]            (down output, before any combine)
 *   counts    int32 [E] device
 * Uses d->H, I, E, b (rows per tile, <= 64), w13 / w2 and max_workgroups; M, k,
 * path and expert_base are not used. Same arithmetic, per row, as the grouped
 * path of moe_ffn_forward.
 * Errors: MOE_ERR_INVALID_ARG (null or misaligned pointers: 16 bytes for the
 * row arrays and a_scale; capacity < 1; the layer checks of moe_ffn_forward),
 * MOE_ERR_UNSUPPORTED (grouped-path shape rules; E*capacity > INT32_MAX),
 * MOE_ERR_HIP. */
MOE_API moe_status moe_ffn_gate_up_batched(const moe_ffn_desc* d, const uint16_t* xb, const int32_t* counts,
                                           int32_t capacity, uint16_t* a16, float* a_scale,
                                           hipStream_t stream);
MOE_API moe_status moe_ffn_down_batched(const moe_ffn_desc* d, const uint16_t* a16, const float* a_scale,
                                        const int32_t* counts, int32_t capacity, float* yb,
                                        hipStream_t stream);

/* Number of kernels moe_ffn_forward launches for this description (0 on error). */
MOE_API int32_t moe_ffn_kernel_count(const moe_ffn_desc* d);

/* Name of kernel i of moe_ffn_forward for this description, or NULL. */
MOE_API const char* moe_ffn_kernel_name(const moe_ffn_desc* d, int32_t i);

/* Where a forward call leaves the route-indexed intermediate a = silu(gate)*up
 * inside the workspace (rows of invalid routes are unspecified), and in which
 * format (0 is reserved for an fp32 plane):
 *   1 (decode path): a bf16 hi plane [M*k][I] at *offset and a bf16 lo plane
 *     at *aux_offset; a = hi + lo within 2^-17 relative.
 *   2 (grouped path): an fp16 plane [M*k][I] at *offset and fp32 multipliers
 *     [M*k][ceil(I/128)][4] at *aux_offset; element i of route r is
 *     fp16[r][i] * mult[r][i/128][(i/64) % 2] (entries 2 and 3 unused). Each
 *     64-element chunk is scaled by a power of two that puts its largest
 *     magnitude in [2^14, 2^15) before rounding to fp16, so every element is
 *     within 2^-11 relative of the fp32 value (elements below 2^-28 of their
 *     chunk's largest aside). */
MOE_API moe_status moe_ffn_intermediate(const moe_ffn_desc* d, size_t* offset, size_t* aux_offset,
                                int32_t* format);

/* Where a grouped-path forward call leaves the routed-W2 rows
 * yhat_r = W2[e] a_r (before the router weight) inside the workspace: fp32
 * [M*k][H] at *offset, each valid route's row written once by the down GEMM
 * and read by the combine. Rows of invalid routes are unspecified. This is the
 * "routed-W2" surface of "Route-Block Membership Selects Packed-AWQ
 * Arithmetic" (the paragraph on the sparse native differences), which tells a
 * down-projection error apart from a combine error. The decode path folds the
 * combine into the down projection's accumulator and keeps no such rows:
 * MOE_ERR_UNSUPPORTED. Other errors as moe_ffn_forward's validation. */
MOE_API moe_status moe_ffn_route_outputs(const moe_ffn_desc* d, size_t* offset);

/* Largest M for which MOE_PATH_AUTO picks the decode path. */
MOE_API int32_t moe_ffn_auto_decode_max_m(void);

/* The path moe_ffn_forward takes for this description (MOE_PATH_AUTO
 * resolved), or -1 when the description is rejected. Host-only. */
MOE_API int32_t moe_ffn_resolved_path(const moe_ffn_desc* d);

/* Static string for a status code. Status codes report host-checkable
 * argument errors only: data-dependent conditions stay on the device (token
 * counts are device-resident in "Hardware-Native Joint Sparse-Quantization for
 * Trillion-Scale MoE", App. D.1), so an expert ID outside the experts held here
 * is a skipped route ("valid routes" in "Route-Block Membership Selects
 * Packed-AWQ Arithmetic", first paragraph), never an error. */
MOE_API const char* moe_status_str(moe_status s);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FFN_H */
