// Composed (materialised-score) arm of gated causal GQA attention, gfx950.
//
// "perf(qwen36): qualify M4 head-256 attention" (d-inference PR #640, Summary) weighs a
// composed attention route against the fused kernel for head_dim 256 at query blocks of 128
// and 512 rows.  This is that route on MI355X, for the comparison: the same operation as the
// fused main pass (TensorFold PR #1009, attention kernel-contract commit), in three passes
// through HBM instead of one:
//
//   1. scores:  S[b, h, r, j] = <Q[b,h,r,:], K[b,g,j,:]> in fp32 for every key of the block's
//      key range, written to the workspace (bf16/fp16 MFMA 32x32x16, fp32 accumulate);
//   2. softmax: per row, m = max over the admissible keys of S * scale (log2 units), the weights
//      exp2(S * scale - m) rounded once to the 16-bit type and written to the workspace (0 for
//      keys the row cannot see), and 1 / l with l the sum of the rounded weights;
//   3. P.V:     O[b, h, r, :] = sum_j P[b,h,r,j] V[b,g,j,:] on MFMA (V staged in LDS), times
//      1 / l and sigmoid(gate), rounded once to the 16-bit output.
//
// Head dims 64, 128 and 256 (a template parameter; the fused kernel is written for 256 only).
// No mask: the arm serves the prompt comparison (causal or not).  The transient workspace is
// B Hq rows kvp (4 + 2) bytes + B Hq rows 4 bytes, kvp = the block's key range rounded up to
// 32 keys: 2.4 GB for a 512-row block of 24 heads at the end of a 32k prompt, against the fused
// kernel's 63 MB of split partials.  Inputs are taken to be finite.
#include <hip/hip_runtime.h>
#include <math.h>

#include "attn_internal.h"

namespace gqa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

template <int DT>
__device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (DT == 0) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                  0);
  }
}

template <int DT>
__device__ __forceinline__ float to_f32(uint16_t w) {
  if constexpr (DT == 0) return __builtin_bit_cast(float, (uint32_t)w << 16);
  else return (float)__builtin_bit_cast(_Float16, w);
}

template <int DT>
__device__ __forceinline__ uint16_t to_16(float x) {
  if constexpr (DT == 0) return __builtin_bit_cast(uint16_t, (__bf16)x);
  else return __builtin_bit_cast(uint16_t, (_Float16)x);
}

template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (DT == 0) return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
  else return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, f16x2));
}

// the key bound of row r (exclusive): its causal bound within the cache
__device__ __forceinline__ int row_lim(const ComposedParams& p, int r) {
  return p.causal ? min(p.kv_len, p.kv_offset + r + 1) : p.kv_len;
}

// Pass 1.  Workgroup = four wavefronts on one (b, h) and 32 rows; wavefront w takes the 32-key
// tile 4 blockIdx.x + w.  S^T[key, row] = K[key, :] . Q[row, :] with A = K (lane: key l % 32,
// dims 16 kk + 8 (l / 32) .. + 7) and B = Q (lane: row l % 32, the same dims), both loaded
// straight from memory; accumulator element i of lane l is key 8 (i / 4) + 4 (l / 32) + i % 4
// of row l % 32, four consecutive keys per group of four, stored as one 16-byte write.
template <int DT, int D>
__global__ __launch_bounds__(256) void composed_scores_kernel(const ComposedParams p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 31, hf = lane >> 5;
  const int kt = blockIdx.x * 4 + wave;
  if (kt * 32 >= p.kv_hi) return;  // wavefront-uniform; no barrier in this kernel
  const int r0 = blockIdx.y * 32;
  const int bh = blockIdx.z;
  const int b = bh / p.Hq, h = bh - b * p.Hq, g = h / p.G;
  const int key = kt * 32 + li, row = r0 + li;
  const uint16_t* krow = p.k + (int64_t)b * p.k_sb + (int64_t)g * p.k_sh + (int64_t)min(key, p.kv_len - 1) * p.k_st;
  const uint16_t* qrow = p.q + (int64_t)b * p.q_sb + (int64_t)h * p.q_sh + (int64_t)min(row, p.rows - 1) * p.q_sr;
  f32x16 acc = {};
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(krow + 16 * kk + 8 * hf);
    const u32x4 bq = *reinterpret_cast<const u32x4*>(qrow + 16 * kk + 8 * hf);
    acc = mfma<DT>(a, bq, acc);
  }
  if (row >= p.rows) return;
  float* srow = p.s + ((int64_t)bh * p.rows + row) * p.kvp + kt * 32 + 4 * hf;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    *reinterpret_cast<f32x4*>(srow + 8 * a) = (f32x4){acc[4 * a], acc[4 * a + 1], acc[4 * a + 2], acc[4 * a + 3]};
  }
}

// Pass 2.  One workgroup of 256 threads per row (b, h, r): the row's maximum over its
// admissible keys, then its weights rounded to 16 bits (0 past the row's bound, up to kvp) and
// the reciprocal of their sum.
template <int DT>
__global__ __launch_bounds__(256) void composed_softmax_kernel(const ComposedParams p) {
  __shared__ float red[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row_id = blockIdx.x;  // (b h) rows + r
  const int r = (int)(row_id % p.rows);
  const int lim = row_lim(p, r);
  const float* srow = p.s + row_id * p.kvp;
  uint16_t* prow = p.pw + row_id * p.kvp;
  float m = -INFINITY;
  for (int j = tid; j < lim; j += 256) m = fmaxf(m, srow[j]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if (lane == 0) red[wave] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();  // red is reused below
  const float mx = m * p.scale_log2;  // lim >= 1 for every row, so m is finite for finite inputs
  float l = 0.0f;
  for (int j = tid; j < p.kvp; j += 256) {
    uint16_t w = 0;
    if (j < lim) {
      w = to_16<DT>(exp2f(srow[j] * p.scale_log2 - mx));
      l += to_f32<DT>(w);
    }
    prow[j] = w;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) l += __shfl_xor(l, off);
  if (lane == 0) red[wave] = l;
  __syncthreads();
  if (tid == 0) p.inv_l[row_id] = 1.0f / ((red[0] + red[1]) + (red[2] + red[3]));
}

// Pass 3.  Workgroup = four wavefronts on one (b, h) and 32 rows; wavefront w owns the 32-dim
// MFMA blocks NBW w .. NBW w + NBW - 1 (two at head_dim 256, one at 128; at 64 wavefronts 2 and
// 3 only stage V).  O^T[dim, row] += V^T[dim, key] . P^T[key, row] over 32-key steps: the V
// rows of the step are staged in LDS by the whole workgroup (64 D bytes),
// A = V^T (lane: dim l % 32, keys 8 (l / 32) .. + 7, eight 16-bit LDS reads) and B = P (lane:
// row l % 32, the same keys, one 16-byte load).  The epilogue applies 1 / l and the gate.
template <int DT, int D>
__global__ __launch_bounds__(256) void composed_pv_kernel(const ComposedParams p) {
  constexpr int NBW = D >= 256 ? D / 128 : 1;         // 32-dim blocks per wavefront
  constexpr int kChunkShift = D == 256 ? 5 : D == 128 ? 4 : 3;  // log2 of the 16-byte chunks per row
  static_assert(D == 64 || D == 128 || D == 256, "head dims 64, 128, 256");
  __shared__ __attribute__((aligned(16))) uint16_t vt[32][D];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 31, hf = lane >> 5;
  const int r0 = blockIdx.x * 32;
  const int bh = blockIdx.y;
  const int b = bh / p.Hq, h = bh - b * p.Hq, g = h / p.G;
  const int row = r0 + li;
  const bool mfma_wave = wave * NBW < D / 32;  // wavefront-uniform
  // keys up to the last row's bound; the weights past each row's own bound are 0
  const int kend = row_lim(p, min(r0 + 31, p.rows - 1));
  const uint16_t* vbase = p.v + (int64_t)b * p.v_sb + (int64_t)g * p.v_sh;
  const uint16_t* prow = p.pw + ((int64_t)bh * p.rows + min(row, p.rows - 1)) * p.kvp;
  f32x16 acc0 = {}, acc1 = {};
  for (int j0 = 0; j0 < kend; j0 += 32) {
    __syncthreads();  // the previous step's V reads are done
    // 32 keys x D dims: thread t copies 16-byte chunks t, t + 256, ... (D / 64 of them)
#pragma unroll
    for (int e = 0; e < D / 64; ++e) {
      const int c = tid + 256 * e, kr = c >> kChunkShift, cc = c & ((1 << kChunkShift) - 1);
      const int key = min(j0 + kr, p.kv_len - 1);  // keys past kv_len carry weight 0
      *reinterpret_cast<u32x4*>(&vt[kr][8 * cc]) =
          *reinterpret_cast<const u32x4*>(vbase + (int64_t)key * p.v_st + 8 * cc);
    }
    __syncthreads();
    if (!mfma_wave) continue;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int kb = 16 * ks + 8 * hf;  // this lane's 8 keys of the 16-key MFMA step
      const u32x4 pb = *reinterpret_cast<const u32x4*>(prow + j0 + kb);
#pragma unroll
      for (int blk = 0; blk < NBW; ++blk) {
        const int d = 32 * (NBW * wave + blk) + li;
        u32x4 va;
#pragma unroll
        for (int t = 0; t < 4; ++t) va[t] = (uint32_t)vt[kb + 2 * t][d] | ((uint32_t)vt[kb + 2 * t + 1][d] << 16);
        if (blk == 0) acc0 = mfma<DT>(va, pb, acc0);
        else acc1 = mfma<DT>(va, pb, acc1);
      }
    }
  }
  if (row >= p.rows || !mfma_wave) return;
  const int64_t row_id = (int64_t)bh * p.rows + row;
  const float inv = p.inv_l[row_id];
  const uint16_t* grow = p.gate + (int64_t)b * p.g_sb + (int64_t)h * p.g_sh + (int64_t)row * p.g_sr;
  uint16_t* orow = p.out + (int64_t)b * p.o_sb + (int64_t)h * p.o_sh + (int64_t)row * p.o_sr;
  // accumulator element i of lane l: dim 8 (i / 4) + 4 (l / 32) + i % 4 of the block, row l % 32
#pragma unroll
  for (int blk = 0; blk < NBW; ++blk) {
    const f32x16& acc = blk == 0 ? acc0 : acc1;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int d0 = 32 * (NBW * wave + blk) + 8 * a + 4 * hf;
      const u32x2 gw = *reinterpret_cast<const u32x2*>(grow + d0);
      float res[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint16_t gv = (uint16_t)(t < 2 ? (gw[0] >> (16 * t)) : (gw[1] >> (16 * (t - 2))));
        res[t] = acc[4 * a + t] * inv * __builtin_amdgcn_rcpf(1.0f + __expf(-to_f32<DT>(gv)));
      }
      u32x2 ow;
      ow[0] = pack2<DT>(res[0], res[1]);
      ow[1] = pack2<DT>(res[2], res[3]);
      *reinterpret_cast<u32x2*>(orow + d0) = ow;
    }
  }
}

}  // namespace

namespace {

template <int DT, int D>
void launch_composed_t(const ComposedParams& p, hipStream_t stream) {
  const dim3 g1((unsigned)((p.kvp / 32 + 3) / 4), (unsigned)((p.rows + 31) / 32), (unsigned)(p.B * p.Hq));
  const dim3 g2((unsigned)((int64_t)p.B * p.Hq * p.rows));
  const dim3 g3((unsigned)((p.rows + 31) / 32), (unsigned)(p.B * p.Hq));
  hipLaunchKernelGGL((composed_scores_kernel<DT, D>), g1, dim3(256), 0, stream, p);
  hipLaunchKernelGGL(composed_softmax_kernel<DT>, g2, dim3(256), 0, stream, p);
  hipLaunchKernelGGL((composed_pv_kernel<DT, D>), g3, dim3(256), 0, stream, p);
}

template <int DT>
void launch_composed_d(const ComposedParams& p, hipStream_t stream) {
  if (p.D == 64) launch_composed_t<DT, 64>(p, stream);
  else if (p.D == 128) launch_composed_t<DT, 128>(p, stream);
  else launch_composed_t<DT, 256>(p, stream);
}

}  // namespace

hipError_t launch_composed(const ComposedParams& p, int dtype, hipStream_t stream) {
  if (dtype == 0) launch_composed_d<0>(p, stream);
  else launch_composed_d<1>(p, stream);
  return hipGetLastError();
}

}  // namespace gqa
