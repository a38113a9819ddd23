/*
 * moe_bench.h — measurement kernels for the MoE expert-FFN benchmark (not part
 * of the layer). They give the hardware floor the layer's kernels are set
 * against: the time a plain streaming read of the same bytes takes, the
 * copy-kernel bandwidth peak on the same GPU (the warp-decode write-up,
 * "Eficiencia de hardware", sets its bandwidth against a measured copy-kernel
 * peak), and the dense MFMA rate the same GPU sustains.
 *
 * Conventions: device pointers owned by the caller; work is enqueued on
 * `stream`; nothing is allocated and the host is not synchronised.
 */
#ifndef MOE_BENCH_H
#define MOE_BENCH_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef MOE_BENCH_API
#define MOE_BENCH_API __attribute__((visibility("default")))
#endif

/* Reads `bytes` bytes at `src` once with 16-byte nontemporal loads: every
 * workgroup of 256 lanes streams whole tiles of 256 * loads_per_lane * 16
 * bytes, all of a tile's loads in flight at once (loads_per_lane is 1, 2, 4,
 * 8 or 16), and writes the XOR of all 32-bit words it read to sink[workgroup].
 *   src         device, 16-byte aligned; bytes a multiple of 16
 *   sink        device, sink_words uint32 entries (the grid is capped there)
 *   grid_out    host, optional: the number of workgroups launched (sink
 *               entries written); the XOR of those entries is the XOR of all
 *               words of the buffer
 *   start/stop  optional caller-created events that take the kernel's own
 *               start and end timestamps (hipExtLaunchKernel); NULL for none
 * Returns 0 on success, 1 for bad arguments (null or misaligned pointers,
 * bytes not a multiple of 16, sink_words < 1, an unsupported loads_per_lane),
 * 2 when the launch fails. */
MOE_BENCH_API int32_t moe_bench_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t sink_words,
                                            int32_t loads_per_lane, int32_t* grid_out, hipEvent_t start,
                                            hipEvent_t stop, hipStream_t stream);

/* Copies `bytes` bytes from src to dst (16-byte loads and stores, the same
 * tiling as moe_bench_stream_read; start/stop as there). Returns 0, 1 for bad
 * arguments (null or misaligned pointers, bytes not a multiple of 16, an
 * unsupported loads_per_lane), or 2. */
MOE_BENCH_API int32_t moe_bench_copy(const void* src, void* dst, size_t bytes, int32_t loads_per_lane,
                                     hipEvent_t start, hipEvent_t stop, hipStream_t stream);

/* Measures the dense MFMA rate: grid workgroups of four waves, each wave
 * running 8 independent chains of `iters` 16x16x32 MFMAs (fp16 operands when
 * fp16 != 0, else bf16; fp32 accumulation) on register operands, with no
 * memory traffic. pattern 0 makes every operand 1.0 (each wave's lane 0 then
 * writes exactly 8 * 32 * iters), pattern 1 seeded values in [1, 2).
 *   sink        device, 4 * grid floats: one per wave
 *   flops_out   host, optional: the FLOPs of the launch,
 *               grid * 4 * iters * 8 * 16384
 *   start/stop  optional events, as for moe_bench_stream_read
 * The grouped GEMMs' MFMA fraction is set against this rate as well as
 * against the data-sheet peak. Returns 0, 1 for bad arguments (null sink,
 * iters or grid < 1, grid > 8192, pattern not 0 or 1), or 2. */
MOE_BENCH_API int32_t moe_bench_mfma(int32_t fp16, int32_t pattern, int32_t iters, int32_t grid, float* sink,
                                     double* flops_out, hipEvent_t start, hipEvent_t stop, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_BENCH_H */
