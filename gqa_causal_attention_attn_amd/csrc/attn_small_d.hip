// Fused gated causal GQA attention for head dims 64 and 128, gfx950.
//
// The same operation as the head_dim-256 main pass (TensorFold PR #1009, attention
// kernel-contract commit), for the smaller head dims of the family ("perf(qwen36): qualify M4
// head-256 attention", Summary: other head dims exist and take their own route rather than the
// head-256 one).  A plainer kernel than the head-256 one: HW (2, or 1 for an odd group)
// wavefronts per workgroup, each 32 query rows of one head, HW heads of one KV group, and one
// KV split of the row tile's key range, in 32-key tiles staged in LDS by all the wavefronts
// together and read by each (rows padded by 16 bytes).  With several splits the epilogue
// writes the normalised partial o and its natural-log lse (the head-256 partial format, rows
// of D) for the merge.
//
//   S^T[key, row]  = K[key, :] . Q[row, :]           A = K (LDS), B = Q (VGPRs), D/16 MFMAs
//   O^T[dim, row] += V^T[dim, key] . P^T[key, row]   A = V^T (LDS, transposing read), B = P
//
// v_mfma_f32_32x32x16 (bf16/fp16 in, fp32 accumulate).  Accumulator element i of lane l holds
// key 8 (i / 4) + 4 (l / 32) + i % 4 of row l % 32, so the S accumulator packed to 16 bits is
// the B operand of P.V with its k-slots in that key order.  Those k-slots are two runs of four
// consecutive keys per lane half.  At D = 64 the A operand (V^T) is two ds_read_b64_tr_b16 per
// MFMA: in each 16-lane group, lane i points at key row i / 4 and dims 4 (i % 4) .. + 3 of a
// 4-key x 16-dim block and receives dim i of the four keys.  At D = 128 it is gathered with
// eight 16-bit reads, which measured faster there (351 against 283 TFLOP/s on a 32k prompt at
// 24/4 heads; 206 against 221 the other way round at D = 64).  Online softmax in the exp2 domain per row (the two lanes of a row exchange
// their halves), weights rounded once to 16 bits and used both in l and in P.V, then
// O / l * sigmoid(gate) rounded once.  Causal bound and cache bound only (no mask); inputs are
// taken to be finite.
#include <hip/hip_runtime.h>
#include <math.h>

#include "attn_internal.h"

namespace gqa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Four 16-bit values of a 4 x 16 block of LDS rows, transposed across each 16-lane group.
__device__ __forceinline__ u32x2 read_tr16(const uint16_t* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p)));
}

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
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (DT == 0) return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
  else return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, f16x2));
}

// Key (within the tile) of accumulator element i for lane half hf.
__device__ __forceinline__ constexpr int key_of(int i, int hf) { return 8 * (i >> 2) + 4 * hf + (i & 3); }

template <int DT, int D, int HW>
__global__ __launch_bounds__(64 * HW) void attn_small_d_kernel(const SmallDParams p) {
  static_assert(D == 64 || D == 128, "head dims 64 and 128");
  constexpr int kRow = D + 8;    // K rows in LDS, 16-bit elements (16 bytes of padding)
  // V rows: for the transposing read 64 bytes of padding (a row pitch of 64 mod 256 bytes) put
  // the 4 rows x 32 dims that 32 lanes read on 64 distinct banks; for the gather, 16 bytes
  constexpr bool kTr = D == 64;
  constexpr int kVRow = kTr ? D + 32 : D + 8;
  constexpr int kBlocks = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t ks[32 * kRow];
  __shared__ __attribute__((aligned(16))) uint16_t vs[32 * kVRow];
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 31, hf = lane >> 5;
  const int r0 = blockIdx.x * 32;
  const int h0 = blockIdx.y * HW, h = h0 + (tid >> 6);  // HW divides G: one KV group
  const int b = blockIdx.z / p.n_splits, split = blockIdx.z - b * p.n_splits, g = h0 / p.G;
  const int row = r0 + li;
  const bool valid = row < p.rows;
  const int lim = valid ? (p.causal ? min(p.kv_len, p.kv_offset + row + 1) : p.kv_len) : 0;
  const int last = min(r0 + 31, p.rows - 1);
  const int kv_lo = split * p.keys_per_split;
  const int kv_end = min(kv_lo + p.keys_per_split, p.causal ? min(p.kv_len, p.kv_offset + last + 1) : p.kv_len);

  // Q of this lane's row in the B-operand order: element t of q[kk] is dim 16 kk + 8 hf + t
  u32x4 q[D / 16];
  const uint16_t* qrow = p.q + (int64_t)b * p.q_sb + (int64_t)h * p.q_sh + (int64_t)min(row, p.rows - 1) * p.q_sr;
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) q[kk] = *reinterpret_cast<const u32x4*>(qrow + 16 * kk + 8 * hf);
  const uint16_t* kbase = p.k + (int64_t)b * p.k_sb + (int64_t)g * p.k_sh;
  const uint16_t* vbase = p.v + (int64_t)b * p.v_sb + (int64_t)g * p.v_sh;

  // this lane's V read: key row 4 hf + (lane % 16) / 4 of a run, dims 16 ((lane / 16) % 2) +
  // 4 (lane % 4) of a 32-dim block
  const uint16_t* vlane = &vs[(4 * hf + ((lane & 15) >> 2)) * kVRow + 16 * ((lane >> 4) & 1) + 4 * (lane & 3)];
  f32x16 o[kBlocks];
#pragma unroll
  for (int db = 0; db < kBlocks; ++db) o[db] = (f32x16){};
  float m = -INFINITY, l = 0.0f;

  for (int j0 = kv_lo; j0 < kv_end; j0 += 32) {
    // stage the tile: 32 rows of K and of V, D / 8 16-byte chunks each; thread t copies chunks
    // t, t + 64 HW, ... (keys past kv_len re-read the last key; every row masks them)
    constexpr int kChunks = 32 * (D / 8);
#pragma unroll
    for (int e = 0; e < (kChunks + 64 * HW - 1) / (64 * HW); ++e) {
      const int c = tid + 64 * HW * e;
      if (kChunks % (64 * HW) != 0 && c >= kChunks) break;
      const int kr = c / (D / 8), cc = c % (D / 8);
      const int key = min(j0 + kr, p.kv_len - 1);
      *reinterpret_cast<u32x4*>(&ks[kr * kRow + 8 * cc]) =
          *reinterpret_cast<const u32x4*>(kbase + (int64_t)key * p.k_st + 8 * cc);
      *reinterpret_cast<u32x4*>(&vs[kr * kVRow + 8 * cc]) =
          *reinterpret_cast<const u32x4*>(vbase + (int64_t)key * p.v_st + 8 * cc);
    }
    __syncthreads();  // the tile is in LDS before any wavefront reads it

    // scores (raw dot products) of this lane's row against keys key_of(i, hf)
    f32x16 s = {};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(&ks[li * kRow + 16 * kk + 8 * hf]);
      s = mfma<DT>(a, q[kk], s);
    }
    // log2 units, keys the row cannot see at -inf
    float mt = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int j = j0 + key_of(i, hf);
      s[i] = j < lim && j < kv_end ? s[i] * p.scale_log2 : -INFINITY;
      mt = fmaxf(mt, s[i]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m, mt);
    const float alpha = m_new == -INFINITY ? 1.0f : exp2f(m - m_new);
    const float neg = m_new == -INFINITY ? 0.0f : -m_new;
    m = m_new;
    // weights rounded once; the packed pairs are the B operand (k-slot 4 a + t of half hf is
    // key_of(4 a + t, hf) for a = 0, 1 in step 0 and a = 2, 3 in step 1)
    uint32_t pw[8];
    float ls = 0.0f;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      pw[t] = pack2<DT>(exp2f(s[2 * t] + neg), exp2f(s[2 * t + 1] + neg));
      ls += to_f32<DT>((uint16_t)(pw[t] & 0xffffu)) + to_f32<DT>((uint16_t)(pw[t] >> 16));
    }
    ls += __shfl_xor(ls, 32);
    l = l * alpha + ls;
    const u32x4 pb0 = {pw[0], pw[1], pw[2], pw[3]};
    const u32x4 pb1 = {pw[4], pw[5], pw[6], pw[7]};
#pragma unroll
    for (int db = 0; db < kBlocks; ++db) {
      o[db] *= alpha;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        // A = V^T[dim 32 db + li][keys key_of(8 st + 0..7, hf)]: keys 16 st + 4 hf + 0..3, then
        // the same + 8
        u32x4 va;
        if constexpr (kTr) {
          const u32x2 w0 = read_tr16(vlane + 16 * st * kVRow + 32 * db);
          const u32x2 w1 = read_tr16(vlane + (16 * st + 8) * kVRow + 32 * db);
          va = (u32x4){w0[0], w0[1], w1[0], w1[1]};
        } else {
          const int d = 32 * db + li;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int k0 = key_of(8 * st + 2 * t, hf), k1 = key_of(8 * st + 2 * t + 1, hf);
            va[t] = (uint32_t)vs[k0 * kVRow + d] | ((uint32_t)vs[k1 * kVRow + d] << 16);
          }
        }
        o[db] = mfma<DT>(va, st == 0 ? pb0 : pb1, o[db]);
      }
    }
    __syncthreads();  // the tile's reads are done before it is overwritten
  }

  if (!valid) return;
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;  // a row with no admissible key gives 0
  if (p.n_splits > 1) {
    // this split's partial: o / l (dims 32 db + 8 a + 4 hf + t) and lse = ln 2 (m + log2 l)
    const int64_t row_id = (((int64_t)split * p.B + b) * p.Hq + h) * p.rows + row;
    float* prow = p.part_o + row_id * D;
#pragma unroll
    for (int db = 0; db < kBlocks; ++db) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        *reinterpret_cast<f32x4*>(prow + 32 * db + 8 * a + 4 * hf) =
            (f32x4){o[db][4 * a] * inv, o[db][4 * a + 1] * inv, o[db][4 * a + 2] * inv, o[db][4 * a + 3] * inv};
      }
    }
    if (hf == 0) p.part_lse[row_id] = l > 0.0f ? (m + __log2f(l)) * 0.6931471805599453f : -INFINITY;
    return;
  }
  const uint16_t* grow = p.gate + (int64_t)b * p.g_sb + (int64_t)h * p.g_sh + (int64_t)row * p.g_sr;
  uint16_t* orow = p.out + (int64_t)b * p.o_sb + (int64_t)h * p.o_sh + (int64_t)row * p.o_sr;
  // accumulator element i of lane l: dim 32 db + 8 (i / 4) + 4 hf + i % 4 of row l % 32
#pragma unroll
  for (int db = 0; db < kBlocks; ++db) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int d0 = 32 * db + 8 * a + 4 * hf;
      const u32x2 gw = *reinterpret_cast<const u32x2*>(grow + d0);
      float res[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint16_t gv = (uint16_t)(t < 2 ? (gw[0] >> (16 * t)) : (gw[1] >> (16 * (t - 2))));
        res[t] = o[db][4 * a + t] * inv * __builtin_amdgcn_rcpf(1.0f + __expf(-to_f32<DT>(gv)));
      }
      u32x2 ow;
      ow[0] = pack2<DT>(res[0], res[1]);
      ow[1] = pack2<DT>(res[2], res[3]);
      *reinterpret_cast<u32x2*>(orow + d0) = ow;
    }
  }
}

template <int DT, int D>
void launch_small_d_h(const SmallDParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)((p.rows + 31) / 32), (unsigned)(p.Hq / p.hw), (unsigned)(p.B * p.n_splits));
  if (p.hw == 2) hipLaunchKernelGGL((attn_small_d_kernel<DT, D, 2>), grid, dim3(128), 0, stream, p);
  else hipLaunchKernelGGL((attn_small_d_kernel<DT, D, 1>), grid, dim3(64), 0, stream, p);
}

template <int DT>
void launch_small_d_t(const SmallDParams& p, hipStream_t stream) {
  if (p.D == 64) launch_small_d_h<DT, 64>(p, stream);
  else launch_small_d_h<DT, 128>(p, stream);
}

}  // namespace

hipError_t launch_small_d(const SmallDParams& p, int dtype, hipStream_t stream) {
  if (dtype == 0) launch_small_d_t<0>(p, stream);
  else launch_small_d_t<1>(p, stream);
  return hipGetLastError();
}

}  // namespace gqa
