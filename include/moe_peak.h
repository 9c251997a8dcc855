/*
 * moe_peak.h - achievable-peak microbenchmarks of libmoe_peak.so (gfx950).
 *
 * Measurement infrastructure, separate from the layer's library: the kernels of libmoe.so
 * are measured against datasheet peaks (dense bf16 MFMA 2.5 PFLOP/s at 2.4 GHz, HBM3E
 * 8 TB/s); these calls measure what this GPU sustains under the same kind of load, so that
 * a kernel's fraction of the datasheet peak can be read next to its fraction of the
 * achievable one. Nothing here is an operation of the MoE layer, so no page passage
 * defines them.
 *
 * Every pointer is a device pointer owned by the caller; every call only enqueues one
 * kernel on `stream` and returns a hipError_t value (0 = hipSuccess; hipErrorInvalidValue,
 * with nothing enqueued, for a NULL or misaligned pointer or a non-positive size).
 */
#ifndef MOE_PEAK_H
#define MOE_PEAK_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Matrix-core loop: `grid` workgroups of 8 waves; every wave issues 4 * iters
 * v_mfma_f32_32x32x16_bf16 (32768 flop each) on register operands, no memory traffic.
 * seed: 256 x 16 bytes of bf16 operands (four 64-lane fragments). out: grid * 512 floats
 * (keeps the results live). clk: 2 * grid uint64, per workgroup the shader-cycle counter
 * (s_memtime) and the 100 MHz real-time counter (s_memrealtime) elapsed over its loop, so
 * clk[2i] / clk[2i+1] * 100 MHz is the clock the loop ran at. */
int moe_peak_mfma(const void *seed, float *out, uint64_t *clk, int grid, int iters,
                  hipStream_t stream);

/* LDS read loop: `grid` workgroups of 8 waves; every wave issues 8 * iters 16-byte-per-lane
 * LDS reads (1 KB each, spread over all banks) from a 64 KB buffer. out: grid * 512 floats. */
int moe_peak_lds(float *out, int grid, int iters, hipStream_t stream);

/* Stream copy dst[0, bytes) = src[0, bytes) with 16-byte loads and stores, `grid`
 * workgroups of 256 threads (bytes a multiple of 16, both pointers 16-byte aligned). */
int moe_peak_copy(const void *src, void *dst, size_t bytes, int grid, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_PEAK_H */
