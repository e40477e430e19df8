// The split merge's arithmetic for one row and the append's 16-byte copy, in one place for the
// merge and append kernels (attn_aux.hip) and for the workgroups of a prompt main pass that carry
// an earlier query block's merge and a kv_append (attn_fwd.h): every route that merges a row
// runs this code, so they give the same bits.
//
// Merge of a row (TensorFold PR #1009, attention kernel-contract commit: decode rows over key
// chunks and a merge of the chunks): with the chunks' natural-log lse_c and normalised o_c,
// out = sum_c exp(lse_c - max lse) o_c / sum_c exp(lse_c - max lse) * sigmoid(gate); an empty
// chunk (lse_c = -Inf) is selected out, a row with every chunk empty gives 0, and a chunk whose
// lse is NaN makes the row NaN.  One wavefront per row, four dims per lane.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>

#include "attn_internal.h"

namespace gqa {
namespace mcore {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

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

// x, max'd with the value DPP control CTRL brings from another lane (lanes of rows outside
// ROW_MASK keep x)
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float max_dpp(float x) {
  const int xi = __builtin_bit_cast(int, x);
  return fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(xi, xi, CTRL, ROW_MASK, 0xf, false)));
}
// largest value over the wavefront's 64 lanes (fmaxf: a NaN lane is passed over), the same in
// every lane: within quads, then rows of 16 (rotations by 4 and 8), then lane 15 of each row
// into the next and lane 31 into the upper half, so that lane 63 holds the wavefront's max.
// DPP moves (no LDS round trips); max is exact, so the order of the steps cannot change it.
__device__ __forceinline__ float wave_max(float x) {
  x = max_dpp<0xb1>(x);        // quad_perm [1, 0, 3, 2]
  x = max_dpp<0x4e>(x);        // quad_perm [2, 3, 0, 1]
  x = max_dpp<0x124>(x);       // row_ror:4
  x = max_dpp<0x128>(x);       // row_ror:8
  x = max_dpp<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
  x = max_dpp<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

// Four values of a split partial row: KIND 0 fp32 rows of D values; KIND 1 the main pass's
// fp16 rows, value times 2^e (partial_row_bytes; e from its own array, loaded by the caller).
// Loads (issued together) and decode apart.
template <int KIND>
struct PartialLoad {
  f32x4 f;    // KIND 0
  u32x2 h;    // KIND 1: four fp16 values
  int32_t e;  // KIND 1: the row's exponent
};
template <int KIND>
__device__ __forceinline__ PartialLoad<KIND> load_values(const MergeParams& p, int64_t row, int dl) {
  PartialLoad<KIND> x;
  if constexpr (KIND == 0) {
    x.f = *reinterpret_cast<const f32x4*>(static_cast<const float*>(p.part_o) + row * p.D + dl);
  } else {
    x.h = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(p.part_o) + row * p.D + dl);
  }
  return x;
}
template <int KIND>
__device__ __forceinline__ f32x4 decode_partial(const PartialLoad<KIND>& x) {
  if constexpr (KIND == 0) {
    return x.f;
  } else {
    auto h2f = [](uint32_t bits) { return (float)__builtin_bit_cast(_Float16, (uint16_t)bits); };
    return (f32x4){__builtin_amdgcn_ldexpf(h2f(x.h[0] & 0xffffu), x.e), __builtin_amdgcn_ldexpf(h2f(x.h[0] >> 16), x.e),
                   __builtin_amdgcn_ldexpf(h2f(x.h[1] & 0xffffu), x.e), __builtin_amdgcn_ldexpf(h2f(x.h[1] >> 16), x.e)};
  }
}

// The weighted sums of one row over its nch chunks, NC >= nch slots (slot c < nch holds chunk c;
// the others re-read a chunk and are selected out).  Lane c holds chunk c's lse (and exponent);
// the row's largest lse is a wavefront max and each lane works out its chunk's weight; the sum
// reads weights and exponents out of the lanes in chunk order and decodes each partial as it
// goes.  nan_l: some chunk's lse is NaN.
struct RowSums {
  f32x4 acc;
  float wsum;
  bool nan_l;
};
template <int KIND, int NC>
__device__ __forceinline__ RowSums row_sums(int nch, int lane, float lse_lane, int32_t e_lane,
                                            const PartialLoad<KIND> (&raw)[NC]) {
  const bool mine = lane < nch;
  const float top = wave_max(mine ? lse_lane : -INFINITY);
  RowSums s;
  s.nan_l = __builtin_amdgcn_ballot_w64(mine && __builtin_isnan(lse_lane)) != 0;
  const float w_lane = top > -INFINITY ? exp2f((lse_lane - top) * kLog2e) : 0.0f;
  s.acc = (f32x4){0.f, 0.f, 0.f, 0.f};
  s.wsum = 0.0f;
  if (top > -INFINITY) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const float lc = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lse_lane), c));
      // an empty chunk is selected out, never multiplied in
      if (c < nch && lc != -INFINITY) {
        const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w_lane), c));
        PartialLoad<KIND> x = raw[c];
        if constexpr (KIND == 1) x.e = __builtin_amdgcn_readlane(e_lane, c);
        s.acc += w * decode_partial<KIND>(x);
        s.wsum += w;
      }
    }
  }
  return s;
}

// the lane's four output values: acc / wsum * sigmoid(gate), rounded once (NaN with a NaN lse,
// 0 for a row with every chunk empty)
template <int DT>
__device__ __forceinline__ u32x2 gated_row(const RowSums& s, u32x2 gw) {
  const float inv = s.nan_l ? NAN : s.wsum > 0.0f ? __builtin_amdgcn_rcpf(s.wsum) : 0.0f;
  float gv[4] = {to_f32<DT>((uint16_t)(gw[0] & 0xffffu)), to_f32<DT>((uint16_t)(gw[0] >> 16)),
                 to_f32<DT>((uint16_t)(gw[1] & 0xffffu)), to_f32<DT>((uint16_t)(gw[1] >> 16))};
  float res[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) res[i] = s.acc[i] * inv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv[i]));
  u32x2 ow;
  ow[0] = pack2<DT>(res[0], res[1]);
  ow[1] = pack2<DT>(res[2], res[3]);
  return ow;
}

// One workgroup (bx, by) of a gx x gy append grid of `nt` threads: one 16-byte chunk per thread
// and step.  Grid row by = (tensor, b, g); x runs over (row r, chunk c of 8 elements) =
// (r << chunk_shift) + c, so the index arithmetic is shifts (one division per grid row).  U
// steps at a time: their U loads go out before the U stores (a step past the end re-reads the
// last chunk and stores nothing), so a workgroup with many steps waits for memory U times less.
template <int U>
__device__ __forceinline__ void append_part(const AppendParams& p, uint32_t bx, uint32_t by, uint32_t gx,
                                            uint32_t gy, uint32_t nt) {
  const int64_t bg = (int64_t)p.B * p.Hkv;
  const int64_t n = (int64_t)p.rows << p.chunk_shift;
  const int cmask = (1 << p.chunk_shift) - 1;
  const int64_t step = (int64_t)gx * nt;
  for (int64_t y = by; y < 2 * bg; y += gy) {
    const int t = y >= bg;
    const int64_t yb = y - (t ? bg : 0);
    const int b = (int)(yb / p.Hkv), g = (int)(yb - (int64_t)b * p.Hkv);
    const uint16_t* src = p.src[t] + b * p.s_sb[t] + g * p.s_sh[t];
    uint16_t* dst = p.dst[t] + b * p.d_sb[t] + g * p.d_sh[t] +
                    (int64_t)(p.kv_offset + (GQA_CONTROL == 3 ? 1 : 0)) * p.d_st[t];
    const int64_t s_sr = p.s_sr[t], d_st = p.d_st[t];
    for (int64_t u0 = (int64_t)bx * nt + threadIdx.x; u0 < n; u0 += U * step) {
      u32x4 val[U];
#pragma unroll
      for (int k = 0; k < U; ++k) {
        const int64_t u = U == 1 ? u0 : min(u0 + k * step, n - 1);
        val[k] = *reinterpret_cast<const u32x4*>(src + (u >> p.chunk_shift) * s_sr + 8 * (int)(u & cmask));
      }
#pragma unroll
      for (int k = 0; k < U; ++k) {
        const int64_t u = u0 + k * step;
        if (k == 0 || u < n) *reinterpret_cast<u32x4*>(dst + (u >> p.chunk_shift) * d_st + 8 * (int)(u & cmask)) = val[k];
      }
    }
  }
}

}  // namespace mcore
}  // namespace gqa
