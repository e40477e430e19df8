// Achievable-peak probes for the roofline figures (libgqa_probes.so, include/gqa_probes.h).
//
// mfma_mix_kernel and lds_read_kernel (below) measure what the main pass's schedule can expect:
// the matrix-core rate of one dependent chain, how much VALU work runs beside it, and the LDS
// read rates of the two read forms it uses.
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

// The decode main pass's key stream without its compute: one workgroup of four wavefronts per
// CU (a 128 KiB LDS ring keeps it alone there) streams its contiguous slice in 32 KiB tiles,
// each wavefront moving 8 KiB of every tile, three tiles in flight.  MODE 0: buffer-to-LDS loads
// (the main pass's form) with a wait and a workgroup barrier per tile; MODE 1: the same without
// the barrier; MODE 2: the same loads into registers (16-byte global loads, folded).  Loads past
// the slice read zeros (the buffer's range ends there).
typedef __attribute__((address_space(3))) void lds_void_t;
// one 1 KiB buffer-to-LDS load of a wavefront (a device function: the LDS pointer cast has no
// host form)
__device__ __forceinline__ void dma_1k(__amdgpu_buffer_rsrc_t rs, uint8_t* dst, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)dst, 16, off, 0, 0, 0);
}
template <int MODE>
__global__ __launch_bounds__(256) void tile_stream_kernel(const uint8_t* src, size_t bytes, uint32_t* out) {
  constexpr int kTile = 32768, kWaveBytes = 8192, kLoads = kWaveBytes / 1024, kPF = 3, kRing = 4;
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kRing * kTile];
  const size_t per = ((bytes + gridDim.x - 1) / gridDim.x + kTile - 1) / kTile * kTile;
  const size_t lo = (size_t)blockIdx.x * per;
  const size_t len = lo >= bytes ? 0 : (bytes - lo < per ? bytes - lo : per);
  const int n_tiles = (int)((len + kTile - 1) / kTile);
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const uint32_t lane = threadIdx.x & 63;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(src) + (len ? lo : 0), (short)0, (int)len, 0x00020000);
  auto off_of = [&](int t, int i) { return (uint32_t)t * kTile + (uint32_t)wave * kWaveBytes + lane * 16 + i * 1024; };
  uint32_t x = 0;
  if constexpr (MODE == 2) {
    // three tiles of registers in flight, folded in turn (the loop runs in steps of three tiles)
    u32x4 r0[kLoads], r1[kLoads], r2[kLoads];
    auto load = [&](u32x4(&r)[kLoads], int t) {
#pragma unroll
      for (int i = 0; i < kLoads; ++i) r[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, off_of(t, i), 0, 0);
    };
    auto fold = [&](const u32x4(&r)[kLoads]) {
#pragma unroll
      for (int i = 0; i < kLoads; ++i) x ^= r[i][0] ^ r[i][1] ^ r[i][2] ^ r[i][3];
    };
    load(r0, 0), load(r1, 1), load(r2, 2);
    for (int t = 0; t < n_tiles; t += 3) {
      fold(r0), load(r0, t + 3);
      fold(r1), load(r1, t + 4);
      fold(r2), load(r2, t + 5);
    }
    fold(r0), fold(r1), fold(r2);
  } else {
    auto issue = [&](int t) {
      uint8_t* dst = ring + (t % kRing) * kTile + wave * kWaveBytes;
#pragma unroll
      for (int i = 0; i < kLoads; ++i) dma_1k(rs, dst + i * 1024, off_of(t, i));
    };
    for (int t = 0; t < kPF; ++t) issue(t);
    for (int t = 0; t < n_tiles; ++t) {
      asm volatile("s_waitcnt vmcnt(16)" ::: "memory");  // this wavefront's 8 loads of tile t are in
      if constexpr (MODE == 0) __builtin_amdgcn_s_barrier();
      issue(t + kPF);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    x = ring[wave * kWaveBytes + lane * 16];  // this wavefront's own bytes of stage 0
  }
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = x;
}

// MFMA with VALU beside it: every wavefront runs `iters` rounds of 16 v_mfma_f32_32x32x16_bf16
// on CHAINS independent accumulators (1: each MFMA depends on the one before), each MFMA
// followed by NV independent VALU operations (EXP: v_exp_f32, else FMAs) on other registers.
// Eight wavefronts a workgroup, two a SIMD, as in the attention main pass.
template <int CHAINS, int NV, bool EXP>
__global__ __launch_bounds__(512) void mfma_mix_kernel(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)(lane + i));
    b[i] = (__bf16)(0.002f * (float)(lane - i));
  }
  f32x16 acc[CHAINS];
#pragma unroll
  for (int c = 0; c < CHAINS; ++c) acc[c] = (f32x16){};
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = 0.01f * (float)(lane + i);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      acc[k % CHAINS] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k % CHAINS], 0, 0, 0);
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        if constexpr (EXP) x[v % 8] = __builtin_amdgcn_exp2f(x[v % 8]) * 0.5f;
        else x[v % 8] = __builtin_fmaf(x[v % 8], 0.999f, 0.001f);
      }
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < CHAINS; ++c) {
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) s += x[i];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// LDS read rate: eight wavefronts a workgroup read a 64 KiB array, eight reads in flight per
// wavefront.  KIND 0: ds_read_b128 at consecutive 16-byte cells (1 KiB a read); KIND 1:
// ds_read_b64_tr_b16 at the lane addresses the attention main pass uses for its V operand
// (groups of 1040 bytes; 512 B a read).
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
template <int KIND>
__global__ __launch_bounds__(512) void lds_read_kernel(float* out, int iters) {
  __shared__ __attribute__((aligned(16))) uint32_t buf[16384];
  for (int i = threadIdx.x; i < 16384; i += blockDim.x) buf[i] = (uint32_t)i;
  __syncthreads();
  const uint32_t l = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint32_t*)buf;
  // the main pass's V lane address within a tile: (4 tq + hf) groups of 1040 B, then 16-byte
  // and 8-byte steps (at most 13,584 + 448 + 8 bytes, inside the array)
  const uint32_t vlane = (4 * ((l >> 2) & 3) + (l >> 5)) * 1040 + 16 * (2 * ((l >> 4) & 1) + ((l & 3) >> 1)) + 8 * (l & 1);
  uint32_t accu = 0;
  for (int it = 0; it < iters; ++it) {
    const uint32_t off = ((uint32_t)(it + wave) & 3u) * 8192u;  // at most 24,576
    // the eight reads and their wait in one asm statement: the registers an outstanding read
    // will write are outputs of the statement that waits for it, so nothing else can use them
    if constexpr (KIND == 0) {
      u32x4 r0, r1, r2, r3, r4, r5, r6, r7;
      const uint32_t a = base + off + l * 16;
      asm volatile(
          "ds_read_b128 %0, %8\n\tds_read_b128 %1, %8 offset:1024\n\t"
          "ds_read_b128 %2, %8 offset:2048\n\tds_read_b128 %3, %8 offset:3072\n\t"
          "ds_read_b128 %4, %8 offset:4096\n\tds_read_b128 %5, %8 offset:5120\n\t"
          "ds_read_b128 %6, %8 offset:6144\n\tds_read_b128 %7, %8 offset:7168\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7)
          : "v"(a)
          : "memory");
      accu ^= r0[0] ^ r1[1] ^ r2[2] ^ r3[3] ^ r4[0] ^ r5[1] ^ r6[2] ^ r7[3];
    } else {
      u32x2 r0, r1, r2, r3, r4, r5, r6, r7;
      const uint32_t a = base + off + vlane;
      asm volatile(
          "ds_read_b64_tr_b16 %0, %8\n\tds_read_b64_tr_b16 %1, %8 offset:64\n\t"
          "ds_read_b64_tr_b16 %2, %8 offset:128\n\tds_read_b64_tr_b16 %3, %8 offset:192\n\t"
          "ds_read_b64_tr_b16 %4, %8 offset:256\n\tds_read_b64_tr_b16 %5, %8 offset:320\n\t"
          "ds_read_b64_tr_b16 %6, %8 offset:384\n\tds_read_b64_tr_b16 %7, %8 offset:448\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7)
          : "v"(a)
          : "memory");
      accu ^= r0[0] ^ r1[1] ^ r2[0] ^ r3[1] ^ r4[0] ^ r5[1] ^ r6[0] ^ r7[1];
    }
  }
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = (float)accu;
}

}  // namespace

extern "C" {

int gqa_probe_mfma(float* out, uint64_t* clocks, int blocks, int waves_per_block, int iters, void* stream) {
  if (!out || !clocks || blocks < 1 || iters < 1 || (waves_per_block != 4 && waves_per_block != 8)) return 1;
  hipLaunchKernelGGL(mfma_peak_kernel, dim3((unsigned)blocks), dim3((unsigned)(64 * waves_per_block)), 0,
                     static_cast<hipStream_t>(stream), out, clocks, iters);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

int gqa_probe_mfma_mix(float* out, int blocks, int iters, int chains, int n_valu, int exp_op, void* stream) {
  if (!out || blocks < 1 || iters < 1) return 1;
  const hipStream_t s = static_cast<hipStream_t>(stream);
#define GQA_MIX(C, N, E)                                                                            \
  if (chains == C && n_valu == N && (exp_op != 0) == E) {                                           \
    hipLaunchKernelGGL((mfma_mix_kernel<C, N, E>), dim3((unsigned)blocks), dim3(512), 0, s, out, iters); \
    return hipGetLastError() == hipSuccess ? 0 : 2;                                                 \
  }
  GQA_MIX(1, 0, false)
  GQA_MIX(1, 2, false)
  GQA_MIX(1, 4, false)
  GQA_MIX(1, 1, true)
  GQA_MIX(1, 2, true)
  GQA_MIX(4, 0, false)
  GQA_MIX(4, 4, false)
#undef GQA_MIX
  return 1;
}

int gqa_probe_lds(float* out, int blocks, int iters, int kind, void* stream) {
  if (!out || blocks < 1 || iters < 1 || (kind != 0 && kind != 1)) return 1;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (kind == 0) hipLaunchKernelGGL(lds_read_kernel<0>, dim3((unsigned)blocks), dim3(512), 0, s, out, iters);
  else hipLaunchKernelGGL(lds_read_kernel<1>, dim3((unsigned)blocks), dim3(512), 0, s, out, iters);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

int gqa_probe_read(const void* src, size_t bytes, uint32_t* out, int blocks, void* stream) {
  if (!src || !out || blocks < 1 || bytes < 16 || (bytes % 16) != 0 || (reinterpret_cast<uintptr_t>(src) & 15u))
    return 1;
  hipLaunchKernelGGL(read_stream_kernel, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), bytes / 16, out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

int gqa_probe_tile_stream(const void* src, size_t bytes, uint32_t* out, int blocks, int mode, void* stream) {
  if (!src || !out || blocks < 1 || bytes < 16 || bytes > ((size_t)1 << 31) * (size_t)blocks ||
      (reinterpret_cast<uintptr_t>(src) & 15u) || mode < 0 || mode > 2)
    return 1;
  const size_t per = (bytes + blocks - 1) / blocks;
  if (per + 32768 * 4 > ((size_t)1 << 31)) return 1;  // 32-bit buffer offsets
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const auto src8 = static_cast<const uint8_t*>(src);
  if (mode == 0) hipLaunchKernelGGL(tile_stream_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, s, src8, bytes, out);
  else if (mode == 1) hipLaunchKernelGGL(tile_stream_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, s, src8, bytes, out);
  else hipLaunchKernelGGL(tile_stream_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, s, src8, bytes, out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
