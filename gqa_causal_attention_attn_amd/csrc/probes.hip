// Achievable-peak probes for the roofline figures (libgqa_probes.so, include/gqa_probes.h).
//
// mfma_peak_kernel: every wavefront runs `iters` rounds of kChains independent accumulation
// chains of v_mfma_f32_32x32x16_bf16 (the instruction of the attention kernels), nothing else
// in the loop; 32 * 32 * 16 * 2 flops per instruction.  Lane 0 of each wavefront also reads the
// shader-clock counter (s_memtime) and the constant 100 MHz counter (s_memrealtime) around the
// loop, so the clock the matrix cores ran at follows from their ratio.
//
// read_stream_kernel: a streaming read of `bytes` bytes (16-byte loads, kUnroll of them in
// flight per lane, each workgroup one contiguous slice), folded into one word per lane that is
// written out so the loads cannot be dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gqa_probes.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChains = 8;

__global__ __launch_bounds__(512) void mfma_peak_kernel(float* out, uint64_t* clocks, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)(lane + i));
    b[i] = (__bf16)(0.002f * (float)(lane - i));
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = (f32x16){};
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) {
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (lane == 0) {
    const size_t w = (size_t)blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64;
    clocks[2 * w] = t1 - t0;
    clocks[2 * w + 1] = r1 - r0;
  }
}

constexpr int kUnroll = 8;

__global__ __launch_bounds__(256) void read_stream_kernel(const u32x4* src, size_t n16, uint32_t* out) {
  // workgroup slice [lo, hi) in 16-byte units; each step the 256 lanes read kUnroll * 256
  // consecutive units, lane-interleaved
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t lo = (size_t)blockIdx.x * per;
  const size_t hi = lo + per < n16 ? lo + per : n16;
  uint32_t x = 0;
  size_t base = lo;
  for (; base + kUnroll * 256 <= hi; base += kUnroll * 256) {  // whole steps: every load unconditional
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = src[base + (size_t)u * 256 + threadIdx.x];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (size_t i = base + threadIdx.x; i < hi; i += 256) {  // the slice's tail
    const u32x4 v = src[i];
    x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = x;
}

}  // namespace

extern "C" {

int gqa_probe_mfma(float* out, uint64_t* clocks, int blocks, int waves_per_block, int iters, void* stream) {
  if (!out || !clocks || blocks < 1 || iters < 1 || (waves_per_block != 4 && waves_per_block != 8)) return 1;
  hipLaunchKernelGGL(mfma_peak_kernel, dim3((unsigned)blocks), dim3((unsigned)(64 * waves_per_block)), 0,
                     static_cast<hipStream_t>(stream), out, clocks, iters);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

int gqa_probe_read(const void* src, size_t bytes, uint32_t* out, int blocks, void* stream) {
  if (!src || !out || blocks < 1 || bytes < 16 || (bytes % 16) != 0 || (reinterpret_cast<uintptr_t>(src) & 15u))
    return 1;
  hipLaunchKernelGGL(read_stream_kernel, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), bytes / 16, out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
