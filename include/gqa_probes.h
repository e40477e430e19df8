/*
 * gqa_probes.h -- C ABI of libgqa_probes.so: achievable-peak probes for the roofline figures
 * of the attention library (not part of the attention path).
 *
 * Both calls enqueue one kernel on `stream` (a hipStream_t, NULL = default) and return 0, 1
 * for an invalid argument (nothing enqueued) or 2 if the HIP runtime refused the launch.
 * Every pointer is DEVICE memory owned by the caller; the library allocates nothing.
 */
#ifndef GQA_PROBES_H
#define GQA_PROBES_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Dense bf16 matrix-core rate: `blocks` workgroups of `waves_per_block` (4 or 8) wavefronts,
 * each wavefront running `iters` rounds of 8 independent v_mfma_f32_32x32x16_bf16 chains
 * (32768 flops each).  out: blocks * 64 * waves_per_block floats (a fold of the accumulators);
 * clocks: 2 words per wavefront, the s_memtime (shader clock) and s_memrealtime (100 MHz)
 * ticks its loop took, so the clock the matrix cores ran at is 100 MHz * clocks[0] / clocks[1]. */
int gqa_probe_mfma(float* out, uint64_t* clocks, int blocks, int waves_per_block, int iters, void* stream);

/* Streaming read of `bytes` bytes (a multiple of 16, src 16-byte aligned) by `blocks`
 * workgroups of 256 lanes, each workgroup one contiguous slice, 16-byte loads with eight in
 * flight per lane; out: blocks * 256 words (a fold of the data, so the loads stay). */
int gqa_probe_read(const void* src, size_t bytes, uint32_t* out, int blocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_PROBES_H */
