/*
 * gqa_probes.h -- C ABI of libgqa_probes.so: achievable-peak probes for the roofline figures
 * of the attention library (not part of the attention path).
 *
 * Each call enqueues one kernel on `stream` (a hipStream_t, NULL = default) and return 0, 1
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

/* The same instruction with VALU work beside it: `blocks` workgroups of 8 wavefronts, each
 * running `iters` rounds of 16 MFMAs on `chains` independent accumulators (1: each MFMA depends
 * on the one before; or 4), each MFMA followed by `n_valu` independent VALU operations on other
 * registers, v_exp_f32 if exp_op else FMAs.  Supported (chains, n_valu, exp_op): (1,0,0),
 * (1,2,0), (1,4,0), (1,1,1), (1,2,1), (4,0,0), (4,4,0); others return 1.  out: blocks * 512
 * floats. */
int gqa_probe_mfma_mix(float* out, int blocks, int iters, int chains, int n_valu, int exp_op, void* stream);

/* LDS read rate: `blocks` workgroups of 8 wavefronts read a 64 KiB LDS array, eight reads in
 * flight per wavefront, `iters` rounds; kind 0 = ds_read_b128 (1 KiB a read), kind 1 =
 * ds_read_b64_tr_b16 at the V-operand lane addresses of the attention main pass (512 B a
 * read).  Bytes read: blocks * 8 * 8 * iters * (1024 or 512).  out: blocks * 512 floats. */
int gqa_probe_lds(float* out, int blocks, int iters, int kind, void* stream);

/* Streaming read of `bytes` bytes (a multiple of 16, src 16-byte aligned) by `blocks`
 * workgroups of 256 lanes, each workgroup one contiguous slice, 16-byte loads with eight in
 * flight per lane; out: blocks * 256 words (a fold of the data, so the loads stay). */
int gqa_probe_read(const void* src, size_t bytes, uint32_t* out, int blocks, void* stream);

/* The decode main pass's key stream without its compute: `blocks` workgroups of four
 * wavefronts (one a CU: each holds a 128 KiB LDS ring) each stream a contiguous slice of `bytes`
 * (src 16-byte aligned) in 32 KiB tiles, every wavefront moving 8 KiB of each tile in 1 KiB
 * loads, three tiles in flight.  mode 0: buffer-to-LDS loads with a wait and a workgroup
 * barrier per tile (the main pass's cadence); 1: without the barrier; 2: the same loads into
 * registers.  out: blocks * 256 words.  Returns 1 on a bad argument (a slice must stay below
 * 2 GiB), 2 on a launch error. */
int gqa_probe_tile_stream(const void* src, size_t bytes, uint32_t* out, int blocks, int mode, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_PROBES_H */
