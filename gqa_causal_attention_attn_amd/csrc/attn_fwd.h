// Main pass of gated causal GQA attention for gfx950 (CDNA4), head dims 256, 128 and 64 (a
// template parameter; attn_fwd_d256.hip, attn_fwd_d128.hip and attn_fwd_d64.hip instantiate it).
#pragma once
//
// One workgroup = one (batch b, KV head g, KV split s, tile of (head, row) pairs of that
// group), one workgroup per CU.  Shapes: eight wavefronts of one 32-pair column block each (two
// wavefronts per SIMD), with the P.V product one tile behind (prompts) or without that lag and
// one more tile in flight (verify blocks, which stream their keys from HBM), and four
// wavefronts of one block (short decode / verify, whose KV group fits in four blocks).  The
// group's K and V are streamed through LDS in tiles of 16 KiB each (8192 / D keys) and every
// wavefront reuses every tile, so K/V is read once per group per split.  Tiles move from HBM to
// LDS with direct buffer->LDS loads (no registers, no VALU) into a ring of four stages.
//
// Per column block, 32 (head, row) pairs are the N dimension of v_mfma_f32_32x32x16 (bf16 or
// fp16 in, fp32 accumulate), the keys of a tile the M dimension of the scores in S blocks of 32:
//
//   S^T[key, pair]  = K[key, :] . Q[pair, :]          A = K tile (LDS), B = Q (VGPRs)
//   O^T[dim, pair] += V^T[dim, key] . P^T[key, pair]  A = V tile (LDS, transposing read), B = P
//
// With keys (and dims) on the MFMA rows and pairs on its columns, every lane owns one pair
// (lane % 32) of a block in both products: the online softmax needs no cross-lane traffic
// except an exchange with the lane 32 away, and the S accumulator, packed to 16 bits, is
// already the B operand of the second product.  The k-slots of that product follow the rows
// of the S accumulator: slot 4a + t of lane half h is row 8a + 4h + t (+16 for the second
// MFMA of the S block); the A operand is gathered in that order by ds_read_b64_tr_b16, which
// hands each lane of a 16-lane group one column of a 4 x 16 block of 16-bit values (4 rows x 16
// dims) that the group reads as rows.  O lives in the accumulation registers (AGPRs) for the
// whole pass; Q, S and everything the VALU touches stay in VGPRs.  Whatever the head dim, a tile
// costs each wavefront 16 MFMAs of scores and 16 of P.V and 16 KiB of K and of V reads from LDS.
//
// LDS layout of a tile: sixteen groups of R = 512 / D whole key rows (1 KiB, the unit one
// direct load of a wavefront fills from R consecutive rows), group i at i * 1040 bytes: the
// 16-byte skew per group puts the same dims of different groups on different banks.  MFMA row r
// of S block sb holds key R gamma(r % 16) + 2 sb + r / 16 with gamma(x) = 4 (x % 4) + x / 4, so
// the 16 lanes of a quarter of a K read (16 rows, one 16-byte cell) hit 16 groups and the
// transposing V reads (4 rows x 2 cells per 16 lanes, the 4 rows in groups 4 apart) hit
// distinct banks.  Every LDS address is a per-lane base plus a compile-time offset.
//
// Schedule.  On the prompt shape the P.V product of tile t - 1 runs on the matrix cores while
// the VALU turns tile t's scores into weights (the previous tile stays in its stage: two tiles
// in flight), and each wavefront's direct loads of tile t + 2 are issued one by one between the
// MFMAs of S(t), after the barrier that freed their stage.  The shapes that stream keys from
// HBM (decode and verify blocks, whose keys each workgroup reads alone) are bound by the
// latency of those loads rather than by the matrix cores: there P.V follows its softmax
// directly, which frees the previous tile's stage for a third tile in flight.
//
// Masks.  A mask that is the same for every head may be staged in LDS beside each K/V tile
// (chosen by the host), in one of two layouts.  Words: each key's mask word in a dword of its
// own (1-, 2- and 4-byte direct loads each write one zero-extended dword per lane), the window's
// rows at a 264- or 520-byte pitch so that lanes of different rows read different banks; any row
// stride and any kv_len, at most 1024 / T rows per workgroup (T keys a tile: 32, 16 and 8 rows at
// head dims 256, 128 and 64); every wavefront issues 16 / W of the 16 loads of a tile.  Rows: 16-byte chunks of rows whose pitch is a multiple of 16 bytes, up to 4 KiB of
// rows, loaded by wavefronts 0-3 (kept for prompt workgroups whose pairs span more than 32
// rows).  Otherwise each lane loads its words from memory.  All three give the same bits.
//
// The softmax is the online (flash) form of the plain definition: per pair a running max m
// (log2 units of the scaled score), a running sum l and the accumulator O, rescaled by
// exp2(m_old - m_new) just before the P.V product that follows a move of m.  m moves only
// when the new maximum exceeds it by more than 8 (a factor 256), so weights stay below 2^8 and
// most rescales are skipped; each lane first compares its half of the pair's keys and the two
// halves are exchanged only when some lane of the wavefront sees such a maximum.  Every
// decision is per pair, so a pair's arithmetic does not depend on which other pairs share its
// wavefront (head-chunked and unchunked launches agree bit for bit).  Weights are rounded to
// the 16-bit type once and both l and P.V use the rounded values.  With one split the epilogue
// applies 1/l and the gate sigmoid and rounds once to 16 bits; with several it writes the
// normalised partial o and its natural log-sum-exp for the merge.
//
// Operation: TensorFold PR #1009, attention kernel-contract commit (float64 gated GQA
// attention as the reference, decode chunks and their merge); "Qwen head-chunked SDPA
// (#113)", introduction (head chunks within a KV group).
#include <hip/hip_runtime.h>
#include <math.h>

#include <type_traits>

#include "attn_internal.h"
#include "attn_merge_core.h"

namespace gqa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;

template <int DT>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (DT == 0) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  }
}


// acc (+)= A B with the accumulator in VGPRs (FIRST: acc = A B), as inline assembly for the
// same reason and with the same leading wait states.
template <int DT, bool FIRST>
__device__ __forceinline__ void mfma32_v(f32x16& acc, const u32x4& a, const u32x4& b) {
  if constexpr (FIRST) {
    if constexpr (DT == 0) {
      asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(acc) : "v"(a), "v"(b));
    } else {
      asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=v"(acc) : "v"(a), "v"(b));
    }
  } else {
    if constexpr (DT == 0) {
      asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
    } else {
      asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
    }
  }
}

// Wait states between the last MFMA into sc and the first instruction that reads sc.
__device__ __forceinline__ void acc_settle_v(f32x16& sc) { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(sc)); }

// Wait states between the last MFMA into o and any other instruction that reads o
// (more than an 8-pass MFMA needs); tied to o so nothing that reads it moves above.
template <int N>
__device__ __forceinline__ void acc_settle(f32x16 (&o)[N]) {
  static_assert(N == 8 || N == 4 || N == 2, "8, 4 or 2 dim blocks");
  if constexpr (N == 8) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]), "+a"(o[6]), "+a"(o[7]));
  } else if constexpr (N == 4) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]));
  } else {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(o[0]), "+a"(o[1]));
  }
}

// Pins o[db] and o[db + 1] in place: whatever reads o[db + 1] after this stays after it, so
// the accumulators are taken out one 16-register tuple at a time.
__device__ __forceinline__ void acc_step(f32x16& cur, f32x16& next) { asm volatile("" : "+a"(cur), "+a"(next)); }

// Two floats -> two 16-bit values (round to nearest even), low half = a.
template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (DT == 0) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, f16x2));
  }
}

template <int DT>
__device__ __forceinline__ float lo16(uint32_t w) {
  if constexpr (DT == 0) return __builtin_bit_cast(float, w << 16);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}

template <int DT>
__device__ __forceinline__ float hi16(uint32_t w) {
  if constexpr (DT == 0) return __builtin_bit_cast(float, w & 0xffff0000u);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// acc + (low 16-bit value of w) + (high 16-bit value of w), both values taken exactly (one
// v_dot2 against (1, 1)).
template <int DT>
__device__ __forceinline__ float sum2(uint32_t w, float acc) {
  if constexpr (DT == 0) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, 0x3f803f80u), acc,
                                           false);
  } else {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), __builtin_bit_cast(f16x2, 0x3c003c00u), acc, false);
  }
}

// One ds_read_b64_tr_b16 at a per-lane LDS byte address plus an immediate offset.  Written as
// inline assembly so the offset stays in the instruction; the caller waits with lgkm_wait
// before using the result (the compiler does not track this load).
template <int OFF>
__device__ __forceinline__ u32x2 ds_read_tr16(uint32_t addr) {
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}

// Wait until at most N LDS operations of this wave are outstanding; the operands tie the
// wait to the registers that the following instructions read.
template <int N>
__device__ __forceinline__ void lgkm_wait(u32x4& a, u32x4& b) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "i"(N));
}

// sigmoid with the hardware reciprocal (1 ulp): 1 / (1 + e^-x); +-Inf and NaN map as the
// plain formula does
__device__ __forceinline__ float sigmoidf_(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// Workgroup i is dispatched to XCD i % 8.  Map it to a logical index so that each XCD
// receives one contiguous range of logical workgroups (which share K/V in that XCD's L2).
__device__ __forceinline__ int xcd_remap(int x, int n) {
  const int q = n >> 3, r = n & 7;
  const int xcd = x & 7, slot = x >> 3;
  return xcd < r ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

// Additive term of a mask word (the u8 flag, the 16-bit value or the fp32 bits), in log2
// units (-inf hides the key).
template <int DT, int MK>
__device__ __forceinline__ float mask_term_of(uint32_t w) {
  if constexpr (MK == 1) {
    return w ? 0.0f : -INFINITY;
  } else if constexpr (MK == 2) {
    return lo16<DT>(w) * kLog2e;
  } else if constexpr (MK == 3) {
    return __builtin_bit_cast(float, w) * kLog2e;
  } else {
    return 0.0f;
  }
}

// The term of key j for this lane's (b, h, r), read from memory.
template <int DT, int MK>
__device__ __forceinline__ float mask_term(const void* base, int64_t row_off, int j) {
  if constexpr (MK == 1) {
    return mask_term_of<DT, MK>(static_cast<const uint8_t*>(base)[row_off + j]);
  } else if constexpr (MK == 2) {
    return mask_term_of<DT, MK>(static_cast<const uint16_t*>(base)[row_off + j]);
  } else if constexpr (MK == 3) {
    return mask_term_of<DT, MK>(__builtin_bit_cast(uint32_t, static_cast<const float*>(base)[row_off + j]));
  } else {
    return 0.0f;
  }
}

// Buffer resource over `bytes` bytes from `base` (gfx9 word 3: raw, untyped).  Reads at
// offsets past `bytes` return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// Issue the direct loads of the tile of keys j0 .. j0 + 8192 / D - 1 into the K and V halves of
// one LDS stage.  Group i = the R = 512 / D consecutive keys R i .. R i + R - 1, R whole rows of
// 2 D bytes (lane l: key R i + l / (D / 8), dims 8 (l % (D / 8)) .. + 7), lands at
// i * kGroupStride; with W wavefronts, wavefront w loads the G = 16 / W groups G w .. G w + G - 1
// (keys j0 + R G w ..).  The per-lane byte offsets koff / voff (row and 16-byte cell) stay fixed;
// each wavefront's rows get a resource that ends at key kv_end, so keys past the end read as
// zeros (every pair masks them) and nothing past it is touched.
template <int W, int D>
__device__ __forceinline__ void issue_tile(const uint16_t* kbase, const uint16_t* vbase, int64_t k_st, int64_t v_st,
                                           int j0, int kv_end, uint8_t* stage, int wave, uint32_t koff,
                                           uint32_t voff) {
  constexpr int kGroups = 16 / W;
  constexpr int kRpg = 512 / D;
  const int j = j0 + kRpg * kGroups * wave;
  const int rows = min(max(kv_end - j, 0), kRpg * kGroups);
  const int kbytes = rows ? (rows - 1) * (int)k_st * 2 + 2 * D : 0;
  const int vbytes = rows ? (rows - 1) * (int)v_st * 2 + 2 * D : 0;
  const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(kbase + (int64_t)j * k_st, kbytes);
  const __amdgpu_buffer_rsrc_t vr = buffer_rsrc(vbase + (int64_t)j * v_st, vbytes);
  uint8_t* g0 = stage + (kGroups * wave) * kGroupStride;
#pragma unroll
  for (int e = 0; e < kGroups; ++e) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)(g0 + e * kGroupStride), 16,
                                             koff + 2 * kRpg * e * (uint32_t)k_st, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)(g0 + kTileLds + e * kGroupStride), 16,
                                             voff + 2 * kRpg * e * (uint32_t)v_st, 0, 0, 0);
  }
}

// The same loads, prepared once per tile (resources and stage address in scalar registers)
// and issued one at a time: load i < G is K group i of this wavefront, load G + i its V group.
// The main pass spreads them between the MFMAs of a tile's scores, in the shadow of the
// matrix cores, instead of issuing them in one burst.
template <int W, int D>
struct TileDma {
  static constexpr int kGroups = 16 / W;
  static constexpr int kLoads = 2 * kGroups;
  static constexpr int kRpg = 512 / D;
  __amdgpu_buffer_rsrc_t kr, vr;
  uint8_t* g0;
  uint32_t koff, voff, kst, vst;

  __device__ __forceinline__ void prep(const uint16_t* kbase, const uint16_t* vbase, int64_t k_st, int64_t v_st,
                                       int j0, int kv_end, uint8_t* stage, int wave) {
    const int j = j0 + kRpg * kGroups * wave;
    const int rows = min(max(kv_end - j, 0), kRpg * kGroups);
    const int kbytes = rows ? (rows - 1) * (int)k_st * 2 + 2 * D : 0;
    const int vbytes = rows ? (rows - 1) * (int)v_st * 2 + 2 * D : 0;
    kr = buffer_rsrc(kbase + (int64_t)j * k_st, kbytes);
    vr = buffer_rsrc(vbase + (int64_t)j * v_st, vbytes);
    g0 = stage + (kGroups * wave) * kGroupStride;
  }

  template <int I>
  __device__ __forceinline__ void issue() const {
    if constexpr (I < kGroups) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)(g0 + I * kGroupStride), 16, koff + 2 * kRpg * I * kst,
                                               0, 0, 0);
    } else {
      constexpr int e = I - kGroups;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)(g0 + kTileLds + e * kGroupStride), 16,
                                               voff + 2 * kRpg * e * vst, 0, 0, 0);
    }
  }
};

// One ds_read_b128 at a per-lane LDS byte address plus an immediate offset (inline assembly:
// the compiler neither tracks it nor waits for it; see lgkm_wait1).
template <int OFF>
__device__ __forceinline__ u32x4 ds_read_b128(uint32_t addr) {
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}

template <int N>
__device__ __forceinline__ void lgkm_wait1(u32x4& a) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(a) : "i"(N));
}

// Wait until at most n_tiles (<= 2) tiles' direct loads of this wavefront are in flight; a
// tile is 32 / W direct loads of each of the W wavefronts.
template <int W, int PLUS>
__device__ __forceinline__ void wait_tiles_in_flight_n(int n_tiles) {
  constexpr int kPerTile = 32 / W + PLUS;
  if (n_tiles == 0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else if (n_tiles == 1) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"i"(kPerTile) : "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(%0)" ::"i"(2 * kPerTile) : "memory");
  }
}

// The mask loads a wavefront adds to each tile's: none (ML = 0), one 16-byte row load on
// wavefronts 0-3 (ML = 1, mask_wave), or 16 / W word loads on every wavefront (ML = 2).
template <int W, int ML>
__device__ __forceinline__ void wait_tiles_in_flight(int n_tiles, bool mask_wave) {
  if constexpr (ML == 2) {
    wait_tiles_in_flight_n<W, 16 / W>(n_tiles);
  } else if (ML == 1 && mask_wave) {
    wait_tiles_in_flight_n<W, 1>(n_tiles);
  } else {
    wait_tiles_in_flight_n<W, 0>(n_tiles);
  }
}

// This lane's index, read afresh each time (volatile): a per-lane address derived from it is
// recomputed where it is used instead of occupying a register across the whole tile loop.
__device__ __forceinline__ uint32_t lane_fresh() {
  uint32_t l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// LDS byte offset (from a stage) of lane l's transposing V reads: lane 16 g16 + 4 t + u reads
// MFMA row 4 hf + t (+8 a, +16 m) and dims 32 db + 16 (g16 % 2) + 4 u .. + 3, where a, m and
// db are immediates
__device__ __forceinline__ uint32_t v_lane_of(uint32_t l) {
  // group 4 tq + hf = (l & 12) + (l >> 5); bytes 32 (g16 % 2) + 16 (uq >> 1) + 8 (uq % 2)
  const uint32_t grp = (l & 12u) + (l >> 5);
  const uint32_t lo = ((l & 16u) << 1) | ((l & 2u) << 3) | ((l & 1u) << 3);
  return kTileLds + __umul24(grp, (uint32_t)kGroupStride) + lo;
}

// Key (within the tile, less R hf, R = 512 / D rows per group) of element q of S block sb: row
// 8 (q / 4) + 4 hf + q % 4 of the block's MFMA holds key R gamma(row % 16) + 2 sb + row / 16,
// gamma(x) = 4 (x % 4) + x / 4.
template <int D>
__device__ __forceinline__ constexpr int key_of(int q, int sb = 0) {
  return (512 / D) * (4 * (q & 3) + 2 * ((q >> 2) & 1)) + 2 * sb + (q >> 3);
}

// LDS byte offset (from a lane's K base) of the K operand of S MFMA f of a tile (S block
// f / (D / 16), k-step f % (D / 16): rows 2 sb + r / 16 of the groups, dims 16 kk + 8 hf ..)
template <int D>
__device__ __forceinline__ constexpr int k_operand_offset(int f) {
  return 2 * (f / (D / 16)) * (2 * D) + 32 * (f % (D / 16));
}

// max(x, x of the lane 32 away), the same value on both lanes
__device__ __forceinline__ float max_halves(float x) { return fmaxf(x, __shfl_xor(x, 32)); }

// x + (x of the lane 32 away), the same sum on both lanes
__device__ __forceinline__ float sum_halves(float x) { return x + __shfl_xor(x, 32); }

// Nonfinite repair of one (head, row) pair of a launch that keeps the keys in one split: the
// pair's gated output computed again over the admissible keys of [kv_lo, j_end) only, one key
// at a time, in fp32 on the VALU.  This lane writes the dims 32 db + 8 q4 + 4 hf + (0..3) of
// the pair, as the epilogue does.
// It runs only for inputs that hold nonfinite values; one dim block per pass over the keys keeps
// its registers few.
template <int D, int DT, int MK>
__device__ __forceinline__ void exact_pair(const FwdParams& p, int b, int h, int r, int hf, int kv_lo,
                                        int j_end, int64_t mrow, const uint16_t* kbase, const uint16_t* vbase) {
  const uint16_t* qrow = p.q + (int64_t)b * p.q_sb + (int64_t)h * p.q_sh + (int64_t)r * p.q_sr;
  // admissible: not hidden by the mask (the range is the caller's); x = the score in log2 units
  auto score = [&](int j, bool& adm) {
    float mt = 0.0f;
    if constexpr (MK != 0) mt = mask_term<DT, MK>(p.mask, mrow, j);
    adm = mt > -INFINITY;
    const uint16_t* krow = kbase + (int64_t)j * p.k_st;
    float acc = 0.0f;
#pragma nounroll
    for (int d = 0; d < D; d += 8) {
      const u32x4 qa = *reinterpret_cast<const u32x4*>(qrow + d);
      const u32x4 ka = *reinterpret_cast<const u32x4*>(krow + d);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = __builtin_fmaf(lo16<DT>(qa[e]), lo16<DT>(ka[e]), acc);
        acc = __builtin_fmaf(hi16<DT>(qa[e]), hi16<DT>(ka[e]), acc);
      }
    }
    return acc * p.scale_log2 + mt;
  };
  bool any = false, nan_s = false;
  float m = -INFINITY;
#pragma nounroll
  for (int j = kv_lo; j < j_end; ++j) {
    bool adm;
    const float x = score(j, adm);
    if (!adm) continue;
    any = true;
    nan_s = nan_s || __builtin_isnan(x);
    m = fmaxf(m, x);
  }
  if (nan_s) m = NAN;  // the max of a set holding NaN
  float l = 0.0f, inv = 0.0f;
  const uint16_t* grow = p.gate + (int64_t)b * p.g_sb + (int64_t)h * p.g_sh + (int64_t)r * p.g_sr;
  uint16_t* orow = p.out + (int64_t)b * p.o_sb + (int64_t)h * p.o_sh + (int64_t)r * p.o_sr;
  // one dim block (32 db ..) per pass over the keys
#pragma nounroll
  for (int c = 0; c < D / 32; ++c) {
    float acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
    if (any) {
#pragma nounroll
      for (int j = kv_lo; j < j_end; ++j) {
        bool adm;
        const float x = score(j, adm);
        if (!adm) continue;
        const float w = exp2f(x - m);
        if (c == 0) l += w;
        const uint16_t* vrow = vbase + (int64_t)j * p.v_st;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d0 = 32 * c + 8 * i + 4 * hf;
          const u32x2 vv = *reinterpret_cast<const u32x2*>(vrow + d0);
          acc[4 * i + 0] = __builtin_fmaf(w, lo16<DT>(vv[0]), acc[4 * i + 0]);
          acc[4 * i + 1] = __builtin_fmaf(w, hi16<DT>(vv[0]), acc[4 * i + 1]);
          acc[4 * i + 2] = __builtin_fmaf(w, lo16<DT>(vv[1]), acc[4 * i + 2]);
          acc[4 * i + 3] = __builtin_fmaf(w, hi16<DT>(vv[1]), acc[4 * i + 3]);
        }
      }
    }
    if (c == 0) inv = any ? 1.0f / l : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = 32 * c + 8 * i + 4 * hf;
      const u32x2 gw = *reinterpret_cast<const u32x2*>(grow + d0);
      u32x2 ow;
      ow[0] = pack2<DT>(acc[4 * i] * inv * sigmoidf_(lo16<DT>(gw[0])),
                        acc[4 * i + 1] * inv * sigmoidf_(hi16<DT>(gw[0])));
      ow[1] = pack2<DT>(acc[4 * i + 2] * inv * sigmoidf_(lo16<DT>(gw[1])),
                        acc[4 * i + 3] * inv * sigmoidf_(hi16<DT>(gw[1])));
      *reinterpret_cast<u32x2*>(orow + d0) = ow;
    }
  }
}

// ---- work carried by a prompt main pass's launch, in its workgroups past the main pass's own
// (FwdParams extra_blocks, on CUs the main pass leaves idle): workgroup e of n_extra runs its
// share of a kv_append (8 steps of its grid at a time) and then of the merge of an earlier query
// block's fp16 partials.  The merge takes one wavefront per row with the arithmetic of the merge
// kernel of as many chunk slots as chunks (mcore::row_sums<1, NC>, gated_row), so each row comes
// out as attn_merge gives it; a wavefront has the loads of R rows in flight at once (R from the
// registers NC slots leave).  No repair inputs travel with it: a NaN stays NaN, as with
// attn_merge on its own.
template <int DT, int NC>
__device__ void carried_merge(const MergeParams& p, int e, int n_extra) {
  constexpr int R = NC <= 3 ? 8 : NC <= 5 ? 6 : 4;  // rows in flight per wavefront
  const int lane = threadIdx.x & 63;
  const int wv = e * (int)(blockDim.x >> 6) + (int)(threadIdx.x >> 6);
  const int n_wv = n_extra * (int)(blockDim.x >> 6);
  const int64_t n_rows = (int64_t)p.B * p.Hq * p.rows;
  const int nch = GQA_CONTROL == 2 ? (NC > 1 ? NC - 1 : 1) : NC;
  const int d0 = 4 * lane;
  const int dl = min(d0, p.D - 4);  // lanes past the head dim re-read its last 4 dims and store nothing
  for (int64_t base = (int64_t)wv * R; base < n_rows; base += (int64_t)n_wv * R) {
    float lse_l[R];
    int32_t e_l[R];
    u32x2 gw[R];
    uint32_t rw[R];
    mcore::PartialLoad<1> raw[R][NC];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      // rows past the last re-read it and store nothing; (b, h, r) in 32-bit arithmetic (the
      // host keeps B Hq rows below 2^31)
      const uint32_t row32 = (uint32_t)min(base + i, n_rows - 1);
      const uint32_t bh = row32 / (uint32_t)p.rows;
      const int r = (int)(row32 - bh * (uint32_t)p.rows);
      const int b = (int)(bh / (uint32_t)p.Hq);
      const int h = (int)(bh - (uint32_t)b * (uint32_t)p.Hq);
      rw[i] = row32;
      gw[i] = *reinterpret_cast<const u32x2*>(p.gate + (int64_t)b * p.g_sb + (int64_t)h * p.g_sh +
                                              (int64_t)r * p.g_sr + dl);
      const int64_t lrow = (int64_t)min(lane, nch - 1) * n_rows + row32;
      lse_l[i] = p.part_lse[lrow];
      e_l[i] = p.part_e[lrow];
#pragma unroll
      for (int c = 0; c < NC; ++c) raw[i][c] = mcore::load_values<1>(p, (int64_t)min(c, nch - 1) * n_rows + row32, dl);
    }
    // every load of the R rows goes out before the first row's sums (one round trip)
#pragma unroll
    for (int i = 0; i < R; ++i) {
#pragma unroll
      for (int c = 0; c < NC; ++c) asm volatile("" : "+v"(lse_l[0]) : "v"(raw[i][c].h));
      asm volatile("" : "+v"(lse_l[0]) : "v"(lse_l[i]), "v"(e_l[i]), "v"(gw[i]));
    }
    // the R rows' sums are independent (no branch between them, so their cross-lane steps
    // interleave); a row past the last is computed and not stored
    u32x2 ow[R];
#pragma unroll
    for (int i = 0; i < R; ++i) ow[i] = mcore::gated_row<DT>(mcore::row_sums<1, NC>(nch, lane, lse_l[i], e_l[i], raw[i]), gw[i]);
#pragma unroll
    for (int i = 0; i < R; ++i) {
      if (base + i < n_rows && d0 < p.D) {
        const uint32_t bh = rw[i] / (uint32_t)p.rows;
        const int r = (int)(rw[i] - bh * (uint32_t)p.rows);
        const int b = (int)(bh / (uint32_t)p.Hq);
        const int h = (int)(bh - (uint32_t)b * (uint32_t)p.Hq);
        *reinterpret_cast<u32x2*>(p.out + (int64_t)b * p.o_sb + (int64_t)h * p.o_sh + (int64_t)r * p.o_sr + d0) = ow[i];
      }
    }
  }
}

template <int DT>
__device__ void carried_work(const MergeParams& p, int e, int n_extra) {
  if (p.carry && e < p.app_bx * p.app_by) {
    const int by = e / p.app_bx;
    mcore::append_part<8>(p.app, (uint32_t)(e - by * p.app_bx), (uint32_t)by, (uint32_t)p.app_bx,
                          (uint32_t)p.app_by, blockDim.x);
  }
  switch (p.n_chunks) {  // 0: no merge carried; the host carries merges of at most kFewChunks chunks
    case 1: carried_merge<DT, 1>(p, e, n_extra); break;
    case 2: carried_merge<DT, 2>(p, e, n_extra); break;
    case 3: carried_merge<DT, 3>(p, e, n_extra); break;
    case 4: carried_merge<DT, 4>(p, e, n_extra); break;
    case 5: carried_merge<DT, 5>(p, e, n_extra); break;
    case 6: carried_merge<DT, 6>(p, e, n_extra); break;
    case 7: carried_merge<DT, 7>(p, e, n_extra); break;
    case 8: carried_merge<DT, 8>(p, e, n_extra); break;
    default: break;
  }
}

template <int D, int DT, int MK, int W, bool LAG, int ML, int SPLIT>
__global__ __launch_bounds__(W * 64, 1) void attn_fwd_kernel(const FwdParams p) {
  static_assert(D == 256 || D == 128 || D == 64, "head dims 256, 128 and 64");
  // A K (or V) tile is 16 KiB whatever the head dim: 8192 / D keys in 16 groups of R = 512 / D
  // rows; the scores of a tile are T / 32 S blocks of 32 keys, each D / 16 MFMA k-steps, so a
  // tile costs every wavefront 16 MFMAs for S and 16 for P.V at any head dim.
  constexpr int kRowBytes = 2 * D;
  constexpr int kRpg = 512 / D;            // rows per 1 KiB group
  constexpr int kTileKeys = 8192 / D;      // keys per tile
  constexpr int kSB = kTileKeys / 32;      // S blocks per tile
  constexpr int kKSteps = D / 16;          // MFMA k-steps per S block
  constexpr int kDB = D / 32;              // 32-dim blocks of O
  constexpr int kCells = D / 8;            // 16-byte cells per row
  static_assert(kSB * kKSteps == 16 && kDB * kSB == 8, "16 S MFMAs and 8 P.V steps per tile");
  static_assert(W == 4 || W == 8, "four or eight wavefronts of one column block each");
  static_assert(!LAG || W == 8, "the lagged P.V is an eight-wavefront schedule");
  static_assert(ML >= 0 && ML <= 2 && (ML == 0 || MK != 0), "mask in LDS: masked kernels");
  static_assert(ML != 1 || D == 256, "16-byte mask rows: head dim 256 only");
  // LAG: P.V one tile behind its softmax (prompts).  Without it (decode / verify, which stream
  // their keys from HBM) P.V runs right after its softmax, which frees the previous tile's stage
  // for a third tile in flight.
  constexpr int PF = LAG ? kPrefetch : kPrefetch + 1;  // tiles in flight
  static_assert(PF < kStages || !LAG, "the lagged P.V keeps tile t - 1 in its stage");
  static_assert(PF <= kStages - 1 && PF <= 3, "a stage for the tile consumed");
  constexpr int kGroupBlocks = W;  // column blocks of this workgroup
  // kStages stages of (K tile, V tile): kPrefetch tiles in flight while one is consumed and
  // the one before it finishes its P.V product.  Stage of tile t: t % kStages.
  // with the mask in LDS, kStages stages of its window follow the K/V stages
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kFwdLdsBytes + (ML ? kStages * kMaskStageLds : 0)];

  // workgroups past the main pass's own run the work the launch carries (unmasked prompts: in
  // the masked kernels the extra code cost the main loop registers)
  if constexpr (LAG && SPLIT == 2 && MK == 0) {
    if ((int)blockIdx.x >= p.grid) {
      carried_work<DT>(p.carried, (int)blockIdx.x - p.grid, p.extra_blocks);
      return;
    }
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps branches on it scalar
  const int li = lane & 31;  // pair slot of this lane in each column block
  const int hf = lane >> 5;  // which half of the MFMA k-slots this lane feeds

  // ---- which (b, g, split, tile) this workgroup serves
  int bid = xcd_remap((int)blockIdx.x, p.grid);
  const int tile_rev = bid % p.n_tiles;
  bid /= p.n_tiles;
  const int split = bid % p.n_splits;
  bid /= p.n_splits;
  const int g = bid % p.Hkv;
  const int b = bid / p.Hkv;
  const int tile = p.n_tiles - 1 - tile_rev;  // later rows (more keys) first

  auto lim_of = [&](int row) {
    return p.causal ? min(p.kv_len, p.kv_offset + row + 1 + (GQA_CONTROL == 1 ? 1 : 0)) : p.kv_len;
  };

  // ---- the (head, row) pairs of this lane: wavefront w holds column block w of the
  // workgroup; a chunk of heads takes blocks_per_chunk blocks
  auto pair_of = [&](int& h_out, int& r_out) {
    const int bi = tile * kGroupBlocks + wave;
    const int chunk_idx = bi / p.blocks_per_chunk;
    const int f = (bi - chunk_idx * p.blocks_per_chunk) * kPairsPerBlock + li;
    const int hstart = chunk_idx * p.chunk;
    const int cs = min(p.chunk, p.G - hstart);
    const bool valid = hstart < p.G && f < cs * p.rows;
    r_out = valid ? f / cs : 0;
    h_out = g * p.G + hstart + (valid ? f - (f / cs) * cs : 0);
    return valid;
  };
  int h0, r0;
  const bool valid0 = pair_of(h0, r0);
  const int lim0 = valid0 ? lim_of(r0) : 0;
  const bool act0 = __builtin_amdgcn_ballot_w64(valid0) != 0;

  // ---- key range of the workgroup [kv_lo, kv_end) and the smallest bound of its pairs, from
  // the pair layout of its column blocks (uniform arithmetic)
  int kv_hi = 0, lim_min = 0x7fffffff, r_lo = 0x7fffffff, r_hi = 0;
  // the (last) column block with pairs: first pair, first head and heads of its chunk, pairs
  int pb_f0 = 0, pb_hs = 0, pb_cs = 1, pb_np = 0;
  for (int bj = tile * kGroupBlocks; bj < (tile + 1) * kGroupBlocks; ++bj) {
    const int cj = bj / p.blocks_per_chunk;
    const int f0 = (bj - cj * p.blocks_per_chunk) * kPairsPerBlock;
    const int hs = cj * p.chunk;
    if (hs >= p.G) continue;
    const int csj = min(p.chunk, p.G - hs);
    const int npairs = csj * p.rows;
    if (f0 >= npairs) continue;
    kv_hi = max(kv_hi, lim_of((min(f0 + kPairsPerBlock, npairs) - 1) / csj));
    lim_min = min(lim_min, lim_of(f0 / csj));
    r_lo = min(r_lo, f0 / csj);
    r_hi = max(r_hi, (min(f0 + kPairsPerBlock, npairs) - 1) / csj);
    pb_f0 = f0, pb_hs = hs, pb_cs = csj, pb_np = min(kPairsPerBlock, npairs - f0);
  }
  const int kv_lo = split * p.keys_per_split;
  const int kv_end = __builtin_amdgcn_readfirstlane(min(kv_lo + p.keys_per_split, kv_hi));
  const int n_kt = kv_end > kv_lo ? (kv_end - kv_lo + kTileKeys - 1) / kTileKeys : 0;
  lim_min = __builtin_amdgcn_readfirstlane(lim_min);

  const uint16_t* kbase = p.k + (int64_t)b * p.k_sb + (int64_t)g * p.k_sh;
  const uint16_t* vbase = p.v + (int64_t)b * p.v_sb + (int64_t)g * p.v_sh;

  // ---- the mask in LDS (ML > 0: the mask is the same for every head and the workgroup's rows
  // r_lo .. r_hi fit a mask stage, or, with p.mask_pairs, the mask has a row per head and the
  // workgroup's pairs form one column block of at most 1024 / T pairs; the host checked).  ML = 1 (head dim 256): the 32-key
  // window of those rows for each tile in 16-byte chunks (wavefronts 0-3 load 1 KiB each: stage
  // byte 1024 w + 16 l is byte (1024 w + 16 l) % kMaskRowBytes of window row (1024 w + 16 l) /
  // kMaskRowBytes).  ML = 2: one dword per key of the tile's window of 1024 / T rows of T keys;
  // load n = 0 .. 15 covers words 64 n .. 64 n + 63 of the window in row order (lane l: row
  // (64 n + l) / T, key (64 n + l) % T); window row rho starts at word_row(rho) (rows 8 bytes
  // apart in their banks).  Keys past the mask's end read as zeros; every pair masks them.
  // ML = 0: each lane loads its words from memory.
  constexpr int kMaskEsz = MK == 1 ? 1 : MK == 2 ? 2 : 4;
  constexpr int kMaskRowBytes = kTileKeys * kMaskEsz;
  constexpr int kMaskRows = ML == 2 ? 1024 / kTileKeys : 4096 / kMaskRowBytes;
  constexpr int kWordLoads = 16 / W;  // ML = 2: loads per tile of each wavefront
  // byte of window row rho in the stage: T = 32 two rows per 264-byte load, T = 64 one row per
  // load (264 bytes), T = 128 one row per two loads (520 bytes)
  auto word_row = [](int rho) {
    if constexpr (kTileKeys == 32) return (rho >> 1) * 264 + (rho & 1) * 128;
    else if constexpr (kTileKeys == 64) return rho * 264;
    else return rho * 520;
  };
  auto word_load = [](int n) {  // stage byte of load n
    if constexpr (kTileKeys == 128) return (n >> 1) * 520 + (n & 1) * 256;
    else return n * 264;
  };
  static_assert(ML != 2 || kMaskRows * kTileKeys == 1024, "16 loads of 64 words a tile");
  const bool mwave = ML == 1 && wave < 4;  // ML = 1: this wavefront issues a mask load per tile
  const int mbytes =
      ML ? (int)(((p.mask_pairs ? (int64_t)(p.Hq - 1) * p.m_sh : 0) + (int64_t)(p.rows - 1) * p.m_sr + p.kv_len) *
                 kMaskEsz)
         : 0;
  const __amdgpu_buffer_rsrc_t mrs =
      buffer_rsrc(static_cast<const uint8_t*>(p.mask) + (ML ? (int64_t)b * p.m_sb * kMaskEsz : 0), mbytes);
  const uint32_t mpos = (uint32_t)(wave * 1024 + lane * 16);
  const uint32_t mvoff =
      ML == 1 ? (uint32_t)(r_lo + mpos / kMaskRowBytes) * (uint32_t)p.m_sr * kMaskEsz + mpos % kMaskRowBytes : 0u;
  uint32_t mwoff[ML == 2 ? kWordLoads : 1];  // ML = 2: byte offset of this lane's word of each load
#pragma unroll
  for (int i = 0; i < (ML == 2 ? kWordLoads : 1); ++i) {
    const int f = 64 * (wave * kWordLoads + i) + lane;
    uint32_t row_off = (uint32_t)(r_lo + f / kTileKeys) * (uint32_t)p.m_sr;
    if (p.mask_pairs) {
      // window row w: pair w of the column block (rows past its pairs repeat pair 0's row)
      const int w = f / kTileKeys;
      const int fp = pb_f0 + (w < pb_np ? w : 0);
      row_off = (uint32_t)(g * p.G + pb_hs + fp % pb_cs) * (uint32_t)p.m_sh + (uint32_t)(fp / pb_cs) * (uint32_t)p.m_sr;
    }
    mwoff[i] = ML == 2 ? (row_off + (uint32_t)(f % kTileKeys)) * (uint32_t)kMaskEsz : 0u;
  }
  auto issue_mask = [&](int j0, int st) {
    if constexpr (ML == 1) {
      if (mwave) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            mrs, (lds_void*)(lds + kFwdLdsBytes + st * kMaskStageLds + wave * 1024), 16,
            mvoff + (uint32_t)j0 * kMaskEsz, 0, 0, 0);
      }
    } else if constexpr (ML == 2) {
#pragma unroll
      for (int i = 0; i < kWordLoads; ++i) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            mrs, (lds_void*)(lds + kFwdLdsBytes + st * kMaskStageLds + word_load(wave * kWordLoads + i)),
            kMaskEsz, mwoff[i], j0 * kMaskEsz, 0, 0);
      }
    }
  };

  // ---- Q of this lane's pairs, in the B-operand order: element t of q*[kk] is dim
  // 16 kk + 8 hf + t.  A lane without a pair loads row 0 of the group's first head instead
  // (in range, finite): its S column only feeds a P.V column that is never stored.  All 16
  // loads go out unconditionally, back to back (a per-load branch on the lane's validity
  // would split them and wait on some before issuing the rest).
  u32x4 q0[kKSteps];
  if (act0) {
    const int hq = valid0 ? h0 : g * p.G, rq = valid0 ? r0 : 0;
    const uint16_t* qa = p.q + (int64_t)b * p.q_sb + (int64_t)hq * p.q_sh + (int64_t)rq * p.q_sr + 8 * hf;
#pragma unroll
    for (int kk = 0; kk < kKSteps; ++kk) q0[kk] = *reinterpret_cast<const u32x4*>(qa + 16 * kk);
  } else {
#pragma unroll
    for (int kk = 0; kk < kKSteps; ++kk) q0[kk] = (u32x4){0u, 0u, 0u, 0u};
  }
  const int64_t mrow0 = MK ? (int64_t)b * p.m_sb + (int64_t)h0 * p.m_sh + (int64_t)r0 * p.m_sr : 0;
  // the first tiles are issued right behind Q, so that the two round trips overlap; Q is
  // older than every tile load, so each wait for a tile covers it as well
  const uint32_t koff = (uint32_t)(lane / kCells) * (uint32_t)p.k_st * 2 + 16 * (lane % kCells);
  const uint32_t voff = (uint32_t)(lane / kCells) * (uint32_t)p.v_st * 2 + 16 * (lane % kCells);
  // Every shape issues PF tiles up front and every step's loads, past the last tile too (those
  // read nothing), so the number of loads in flight is the same at every wait and the waits
  // need no tail cases.
  static_for<PF>([&](auto tc) {
    constexpr int t = decltype(tc)::value;
    issue_mask(kv_lo + t * kTileKeys, t);
    issue_tile<W, D>(kbase, vbase, p.k_st, p.v_st, kv_lo + t * kTileKeys, kv_end, lds + t * kStageLds, wave, koff,
                     voff);
  });
  // a use of Q right behind those loads: the compiler's wait for Q then counts them as still
  // in flight (left to the tile loop, it would wait for every load before entering it)
#pragma unroll
  for (int kk = 0; kk < kKSteps; ++kk) asm volatile("" ::"v"(q0[kk]));

  // per-lane LDS byte addresses (see the layout above); every read adds a compile-time offset.
  // MFMA row r of S block sb holds key R gamma(r % 16) + 2 sb + r / 16 with gamma(x) =
  // 4 (x % 4) + x / 4: the 16 lanes of a quarter of a K read then touch 16 different groups, one
  // per bank quad, and the 4 keys of a transposing V read sit 64 bytes apart in their banks.
  const uint32_t lds0 = (uint32_t)(uintptr_t)(const lds_u8*)lds;
  const int li16 = li & 15;
  const uint32_t k_lane = (4 * (li16 & 3) + (li16 >> 2)) * kGroupStride + (li >> 4) * kRowBytes + hf * 16;

  // the accumulators live in the accumulation registers (AGPRs), everything the VALU touches
  // every tile in VGPRs
  f32x16 o0[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db) {
    o0[db] = (f32x16){};
    asm volatile("" : "+a"(o0[db]));
  }

  float m0 = -INFINITY, l0 = 0.0f;

  // One step of the 4-wavefront tile stream: wait for tile t (issued PF steps ago), sync, and
  // start tile t + PF in one burst.  Returns the LDS address of tile t's stage.
  int stage = 0;
  auto stream_step = [&](int t) {
    // tile t landed for this wavefront once only the tiles issued after it remain in flight
    wait_tiles_in_flight<W, ML>(PF - 1, mwave);
    // ... and for everyone; everyone is done with tile t - 1, whose stage is refilled next
    __builtin_amdgcn_s_barrier();
    int st2 = stage + PF;
    if (st2 >= kStages) st2 -= kStages;
    issue_mask(kv_lo + (t + PF) * kTileKeys, st2);
    issue_tile<W, D>(kbase, vbase, p.k_st, p.v_st, kv_lo + (t + PF) * kTileKeys, kv_end, lds + st2 * kStageLds, wave,
                     koff, voff);
    const uint32_t sb = lds0 + stage * kStageLds;
    stage = stage + 1 == kStages ? 0 : stage + 1;
    return sb;
  };

  // The 8-wavefront stream: after the barrier of tile t the loads of tile t + PF are prepared,
  // and the S product of tile t issues them one by one between its MFMAs (a burst of them at
  // the barrier would hold up the wavefront that issues it).  PF - 1 tiles are in flight beyond
  // the one consumed at every wait.
  TileDma<W, D> dma;
  dma.koff = koff, dma.voff = voff, dma.kst = (uint32_t)p.k_st, dma.vst = (uint32_t)p.v_st;
  auto sync_step = [&](int t) {
    wait_tiles_in_flight<W, ML>(PF - 1, mwave);
    __builtin_amdgcn_s_barrier();
    int st2 = stage + PF;
    if (st2 >= kStages) st2 -= kStages;
    issue_mask(kv_lo + (t + PF) * kTileKeys, st2);
    dma.prep(kbase, vbase, p.k_st, p.v_st, kv_lo + (t + PF) * kTileKeys, kv_end, lds + st2 * kStageLds, wave);
    const uint32_t sb = lds0 + stage * kStageLds;
    stage = stage + 1 == kStages ? 0 : stage + 1;
    return sb;
  };
  auto dma_hook = [&](auto kkc) {
    constexpr int kk = decltype(kkc)::value;
    constexpr int every = 16 / TileDma<W, D>::kLoads;
    if constexpr (kk % every == 1 % every) dma.template issue<kk / every>();
  };
  auto no_hook = [](auto) {};

  if (!act0) {
    // a wavefront without pairs only helps stream the tiles
    if constexpr (W == 8) {
      for (int t = 0; t < n_kt; ++t) {
        sync_step(t);
        static_for<TileDma<W, D>::kLoads>([&](auto ic) { dma.template issue<decltype(ic)::value>(); });
      }
    } else {
      for (int t = 0; t < n_kt; ++t) stream_step(t);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    return;
  }

  // ---- the S^T blocks of the tile at sb (stage address): block i = 32 keys (rows) x the 32
  // pairs of this wavefront's column block; the 16 MFMAs of a tile (kSB blocks of kKSteps
  // k-steps) with the K operands read two steps ahead
  auto scores = [&](uint32_t sb, const u32x4(&q)[kKSteps], auto&& hook, f32x16(&sc)[kSB]) {
    const uint32_t kaddr = sb + k_lane;
    constexpr int kAhead = 2;  // K operands in flight beyond the one consumed
    u32x4 kop[kAhead + 1];
    static_for<kAhead>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      kop[i] = ds_read_b128<k_operand_offset<D>(i)>(kaddr);
    });
    static_for<16>([&](auto fc) {
      constexpr int f = decltype(fc)::value;
      if constexpr (f + kAhead < 16)
        kop[(f + kAhead) % (kAhead + 1)] = ds_read_b128<k_operand_offset<D>(f + kAhead)>(kaddr);
      constexpr int issued = f + kAhead + 1 < 16 ? f + kAhead + 1 : 16;
      lgkm_wait1<issued - f - 1>(kop[f % (kAhead + 1)]);
      mfma32_v<DT, f % kKSteps == 0>(sc[f / kKSteps], kop[f % (kAhead + 1)], q[f % kKSteps]);
      hook(fc);
    });
    static_for<kSB>([&](auto ic) { acc_settle_v(sc[decltype(ic)::value]); });
  };

  // ---- element q of S block i is MFMA row 8 (q / 4) + 4 hf + q % 4, i.e. key jb +
  // key_of<D>(q, i) + R hf of this lane's pair.  Keys the pair cannot see go to -inf; only tiles
  // that reach some pair's bound compare keys (wave-uniform test).  The scale is applied later,
  // in the exponent (the max commutes with it, scale > 0), except that an additive mask adds its
  // value to the scaled score: there the score becomes scale s + mask (natural-log units) and
  // the exponent applies log2(e).  A bool mask only hides keys.
  auto add_mask = [&](float s, uint32_t w) {
    if constexpr (MK == 1) return w ? s : -INFINITY;
    else if constexpr (MK == 2) return __builtin_fmaf(s, p.scale, lo16<DT>(w));
    else return __builtin_fmaf(s, p.scale, __builtin_bit_cast(float, w));
  };
  // Per-lane mask words (no window in LDS): the word of each of the lane's keys, every load
  // unconditional (a key past the pair's bound reads the pair's key 0 instead, in range, and is
  // hidden by mask_words_apply), so the 16 loads go out together and are waited for once.
  auto mask_fetch = [&](uint32_t(&w)[kSB][16], int jb, int lim, int64_t mrow) {
    const int jl = jb + kRpg * hf;
    static_for<kSB>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int j = jl + key_of<D>(q, i);
        const int64_t at = mrow + (j < lim ? j : 0);
        if constexpr (MK == 1) w[i][q] = static_cast<const uint8_t*>(p.mask)[at];
        else if constexpr (MK == 2) w[i][q] = static_cast<const uint16_t*>(p.mask)[at];
        else w[i][q] = __builtin_bit_cast(uint32_t, static_cast<const float*>(p.mask)[at]);
      }
    });
  };
  auto mask_words_apply = [&](f32x16(&sc)[kSB], const uint32_t(&w)[kSB][16], int jb, int lim) {
    const int jl = jb + kRpg * hf;
    static_for<kSB>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int j = jl + key_of<D>(q, i);
        sc[i][q] = j < lim ? add_mask(sc[i][q], w[i][q]) : -INFINITY;
      }
    });
  };
  auto mask_scores = [&](f32x16(&sc)[kSB], int jb, int lim, int64_t mrow) {
    if constexpr (MK == 0) {
      if (jb + kTileKeys > lim_min) {
        const int jl = jb + kRpg * (int)(lane_fresh() >> 5);  // recomputed: not held across the loop
        static_for<kSB>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            if (jl + key_of<D>(q, i) >= lim) sc[i][q] = -INFINITY;
          }
        });
      }
    } else {
      uint32_t w[kSB][16];
      mask_fetch(w, jb, lim, mrow);
      mask_words_apply(sc, w, jb, lim);
    }
  };

  // The same with the tile's mask window in LDS (the stage of K/V stage address sb): the words
  // of keys q and q + 8 are adjacent, one read each.
  auto mask_lds_apply = [&](f32x16(&sc)[kSB], int jb, int lim, uint32_t sb) {
    if constexpr (ML != 0) {
      // window row of this lane's pair: its query row, or (per-pair windows) its pair slot
      const int rho = p.mask_pairs ? min(li, kMaskRows - 1) : min(max(r0 - r_lo, 0), kMaskRows - 1);
      const uint32_t mst = lds0 + kFwdLdsBytes + ((sb - lds0) / kStageLds) * kMaskStageLds;
      static_for<kSB>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        auto apply = [&](int q, uint32_t w) { sc[i][q] = add_mask(sc[i][q], w); };
        if constexpr (ML == 2) {
          const uint32_t row = mst + word_row(rho) + kRpg * hf * 4;
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const u32x2 x = *reinterpret_cast<const __attribute__((address_space(3))) u32x2*>(
                (uintptr_t)(row + key_of<D>(q, i) * 4));
            apply(q, x[0]);
            apply(q + 8, x[1]);
          }
        } else {
          const lds_u8* row =
              reinterpret_cast<const lds_u8*>((uintptr_t)(mst + rho * kMaskRowBytes + kRpg * hf * kMaskEsz));
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const lds_u8* at = row + key_of<D>(q, i) * kMaskEsz;
            if constexpr (MK == 1) {
              const uint16_t x = *reinterpret_cast<const __attribute__((address_space(3))) uint16_t*>(at);
              apply(q, x & 0xffu);
              apply(q + 8, x >> 8);
            } else if constexpr (MK == 2) {
              const uint32_t x = *reinterpret_cast<const __attribute__((address_space(3))) uint32_t*>(at);
              apply(q, x & 0xffffu);
              apply(q + 8, x >> 16);
            } else {
              const u32x2 x = *reinterpret_cast<const __attribute__((address_space(3))) u32x2*>(at);
              apply(q, x[0]);
              apply(q + 8, x[1]);
            }
          }
        }
      });
      // keys past some pair's bound (wave-uniform test: only tiles that reach a bound)
      if (jb + kTileKeys > lim_min) {
        const int jl = jb + kRpg * hf;
        static_for<kSB>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            if (jl + key_of<D>(q, i) >= lim) sc[i][q] = -INFINITY;
          }
        });
      }
    }
  };
  auto mask_any = [&](f32x16(&sc)[kSB], int jb, int lim, int64_t mrow, uint32_t sb) {
    if constexpr (ML != 0) mask_lds_apply(sc, jb, lim, sb);
    else mask_scores(sc, jb, lim, mrow);
  };

  // ---- online softmax of one block, in two parts.  stats: the new running max of each
  // pair.  m moves only when the tile's max exceeds it by more than kRescaleSlack; a lane
  // compares its own half of the pair's keys first, and only when some lane of the wavefront
  // sees such a max are the two halves exchanged, so the common case stays off the LDS pipe.
  // The decision per pair is the same as with the exchange every time.  Returns the factor
  // alpha for l and o (1 when m stays) and whether any pair of the wavefront moved.
  auto stats = [&](const f32x16(&sc)[kSB], float& m_run, float& alpha) {
    float mr = fmaxf(fmaxf(sc[0][0], sc[0][1]), sc[0][2]);
#pragma unroll
    for (int q = 3; q < 15; q += 2) mr = fmaxf(fmaxf(mr, sc[0][q]), sc[0][q + 1]);
    mr = fmaxf(mr, sc[0][15]);
#pragma unroll
    for (int i = 1; i < kSB; ++i) {
#pragma unroll
      for (int q = 0; q < 16; q += 2) mr = fmaxf(fmaxf(mr, sc[i][q]), sc[i][q + 1]);
    }
    const float scale = MK >= 2 ? kLog2e : p.scale_log2;
    alpha = 1.0f;
    if (__builtin_amdgcn_ballot_w64(mr * scale > m_run + kRescaleSlack)) {
      const float mx = max_halves(mr) * scale;
      const bool upd = mx > m_run + kRescaleSlack;
      const float m_next = upd ? mx : m_run;
      alpha = upd ? __builtin_amdgcn_exp2f(m_run - m_next) : 1.0f;
      m_run = m_next;
      return __builtin_amdgcn_ballot_w64(upd) != 0;
    }
    return false;
  };

  // exp part: the tile's weights exp2(s - m), rounded once to 16 bits and packed as the B
  // operands of P.V (S block i: pb0[i] for its first 16 keys, pb1[i] for the other 16);
  // l_run = alpha l_run + the sum of the rounded weights
  auto weights = [&](const f32x16(&sc)[kSB], float m_run, float alpha, float& l_run, u32x4(&pb0)[kSB],
                     u32x4(&pb1)[kSB]) {
    const float scale = MK >= 2 ? kLog2e : p.scale_log2;
    const float neg_m = (m_run == -INFINITY) ? 0.0f : -m_run;
    float lsum = 0.0f;
#pragma unroll
    for (int i = 0; i < kSB; ++i) {
      uint32_t pw[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        pw[q] = pack2<DT>(__builtin_amdgcn_exp2f(__builtin_fmaf(sc[i][2 * q], scale, neg_m)),
                          __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i][2 * q + 1], scale, neg_m)));
        lsum = sum2<DT>(pw[q], lsum);
      }
      pb0[i] = (u32x4){pw[0], pw[1], pw[2], pw[3]};
      pb1[i] = (u32x4){pw[4], pw[5], pw[6], pw[7]};
    }
    l_run = l_run * alpha + lsum;
    // keep this work in the phase it is written in (beside the P.V issued just before),
    // instead of letting it sink next to its use
    if constexpr (kSB == 1) {
      asm volatile("" : "+v"(pb0[0]), "+v"(pb1[0]), "+v"(l_run));
    } else {
#pragma unroll
      for (int i = 0; i < kSB; ++i) asm volatile("" : "+v"(pb0[i]), "+v"(pb1[i]));
      asm volatile("" : "+v"(l_run));
    }
  };

  // o *= alpha when some pair's max moved (issued before the P.V product that follows it)
  auto rescale = [&](f32x16(&o)[kDB], float alpha, bool moved) {
    if (moved) {
      acc_settle(o);
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        o[db] *= alpha;
        if (db < kDB - 1) acc_step(o[db], o[db + 1]);
      }
      acc_settle(o);
    }
  };

  // ---- O^T += V^T P^T over the tile at sb in 8 steps (dim block s / kSB, S block s % kSB);
  // the V operands of step s + 1 are read while the two MFMAs of step s run
  auto pv = [&](uint32_t sb, uint32_t vl, const u32x4(&pb0)[kSB], const u32x4(&pb1)[kSB], f32x16(&o)[kDB]) {
    const uint32_t va = sb + vl;
    u32x4 va4[2][2];
    auto read_v = [&](auto sc_, u32x4(&dst)[2]) {
      constexpr int st = decltype(sc_)::value;
      constexpr int db = st / kSB, sbk = st % kSB;
      // MFMA m of S block sbk covers its rows 16 m .. 16 m + 15 (row 2 sbk + m of each group);
      // its k-slots 4 a + t take rows 8 a + 4 h + t (+2 kGroupStride for a = 1)
      constexpr int o00 = 64 * db + 2 * sbk * kRowBytes, o10 = o00 + 2 * kGroupStride;
      constexpr int o01 = o00 + kRowBytes, o11 = o10 + kRowBytes;
      const u32x2 w00 = ds_read_tr16<o00>(va), w10 = ds_read_tr16<o10>(va);
      const u32x2 w01 = ds_read_tr16<o01>(va), w11 = ds_read_tr16<o11>(va);
      dst[0] = (u32x4){w00[0], w00[1], w10[0], w10[1]};
      dst[1] = (u32x4){w01[0], w01[1], w11[0], w11[1]};
    };
    read_v(std::integral_constant<int, 0>{}, va4[0]);
    static_for<8>([&](auto sc_) {
      constexpr int st = decltype(sc_)::value;
      constexpr int db = st / kSB, sbk = st % kSB;
      if constexpr (st < 7) {
        read_v(std::integral_constant<int, st + 1>{}, va4[(st + 1) & 1]);
        lgkm_wait<4>(va4[st & 1][0], va4[st & 1][1]);
      } else {
        lgkm_wait<0>(va4[st & 1][0], va4[st & 1][1]);
      }
      o[db] = mfma32<DT>(va4[st & 1][0], pb0[sbk], o[db]);
      o[db] = mfma32<DT>(va4[st & 1][1], pb1[sbk], o[db]);
      asm volatile("" : "+a"(o[db]));
    });
  };

  // ---- the tile loop.  On the eight-wavefront shape the matrix-core work of one tile and the
  // VALU work of the next are paired so that each runs beside the other:
  //   [S(t)] [PV(t-1) | weights(t)]
  // The rescale of o by tile t's alpha is issued just before P_t V_t, so per pair the
  // operations on o keep the plain order (scale by alpha_t, then add P_t V_t).
  if constexpr (!LAG) {
    for (int t = 0; t < n_kt; ++t) {
      const uint32_t sb = W == 8 ? sync_step(t) : stream_step(t);
      const int jb = kv_lo + t * kTileKeys;
      u32x4 pa0[kSB], pa1[kSB];
      float a0;
      f32x16 s0[kSB];
      if constexpr (MK != 0 && ML == 0) {
        // the tile's mask words are requested ahead of S (and of the tile loads it issues), so
        // that waiting for them leaves those loads in flight
        uint32_t mw[kSB][16];
        mask_fetch(mw, jb, lim0, mrow0);
        if constexpr (W == 8) scores(sb, q0, dma_hook, s0);
        else scores(sb, q0, no_hook, s0);
        mask_words_apply(s0, mw, jb, lim0);
      } else {
        if constexpr (W == 8) scores(sb, q0, dma_hook, s0);
        else scores(sb, q0, no_hook, s0);
        mask_any(s0, jb, lim0, mrow0, sb);
      }
      const bool f0 = stats(s0, m0, a0);
      rescale(o0, a0, f0);
      weights(s0, m0, a0, l0, pa0, pa1);
      pv(sb, v_lane_of(lane_fresh()), pa0, pa1, o0);
    }
  } else if (n_kt > 0) {
    u32x4 pa0[kSB], pa1[kSB];
    float a0;
    bool f0;
    uint32_t sb = sync_step(0);
    f32x16 s0[kSB];
    scores(sb, q0, dma_hook, s0);
    mask_any(s0, kv_lo, lim0, mrow0, sb);
    f0 = stats(s0, m0, a0);
    weights(s0, m0, a0, l0, pa0, pa1);
    uint32_t sprev = sb;
    for (int t = 1; t < n_kt; ++t) {
      sb = sync_step(t);
      const int jb = kv_lo + t * kTileKeys;
      __builtin_amdgcn_sched_barrier(0);
      scores(sb, q0, dma_hook, s0);
      mask_any(s0, jb, lim0, mrow0, sb);
      // o still owes tile t - 1's alpha: keep it until its P.V is issued
      const float a_prev = a0;
      const bool f_prev = f0;
      // the lane's V read address is worked out while the S product drains (pinned here, ahead
      // of the max's branch, instead of sinking to the head of P.V)
      uint32_t vl = v_lane_of(lane_fresh());
      asm volatile("" : "+v"(vl));
      f0 = stats(s0, m0, a0);
      rescale(o0, a_prev, f_prev);
      __builtin_amdgcn_sched_barrier(0);
      pv(sprev, vl, pa0, pa1, o0);
      weights(s0, m0, a0, l0, pa0, pa1);
      sprev = sb;
    }
    rescale(o0, a0, f0);
    pv(sprev, v_lane_of(lane_fresh()), pa0, pa1, o0);
  }
  // the loads past the last tile have landed before the workgroup's LDS is given up
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- epilogue: element q of o*[db] is dim 32 db + 8 (q / 4) + 4 hf + (q % 4)
  const float lt0 = sum_halves(l0);
  // returns whether a NaN came out of o / l (one split only: the nonfinite repair below then
  // redoes the pair; split partials are checked and redone by the merge)
  auto finish = [&](bool valid, int h, int r, float l_tot, float m_run, f32x16(&o)[kDB]) {
    bool nan_seen = false;
    if (!valid) return nan_seen;
    const float inv = l_tot > 0.0f ? __builtin_amdgcn_rcpf(l_tot) : 0.0f;
    if constexpr (!SPLIT) {
      const uint16_t* grow = p.gate + (int64_t)b * p.g_sb + (int64_t)h * p.g_sh + (int64_t)r * p.g_sr;
      uint16_t* orow = p.out + (int64_t)b * p.o_sb + (int64_t)h * p.o_sh + (int64_t)r * p.o_sr;
      // every gate word of the lane is requested before the first store: one round trip (a load
      // after each store would wait for that store and its own load in turn)
      u32x2 gws[kDB][4];
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) gws[db][q4] = *reinterpret_cast<const u32x2*>(grow + 32 * db + 8 * q4 + 4 * hf);
      }
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        if (db > 0) acc_step(o[db - 1], o[db]);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d0 = 32 * db + 8 * q4 + 4 * hf;
          const u32x2 gw = gws[db][q4];
          const float g0 = sigmoidf_(lo16<DT>(gw[0])), g1 = sigmoidf_(hi16<DT>(gw[0]));
          const float g2 = sigmoidf_(lo16<DT>(gw[1])), g3 = sigmoidf_(hi16<DT>(gw[1]));
          const float x0 = o[db][4 * q4 + 0] * inv, x1 = o[db][4 * q4 + 1] * inv;
          const float x2 = o[db][4 * q4 + 2] * inv, x3 = o[db][4 * q4 + 3] * inv;
          nan_seen = nan_seen || __builtin_isnan(x0 + x1 + x2 + x3);  // see the repair below
          u32x2 ow;
          ow[0] = pack2<DT>(x0 * g0, x1 * g1);
          ow[1] = pack2<DT>(x2 * g2, x3 * g3);
          *reinterpret_cast<u32x2*>(orow + d0) = ow;
        }
      }
    } else {
      const int64_t row_id = (((int64_t)split * p.B + b) * p.Hq + h) * p.rows + r;
      int e = 0;
      if constexpr (SPLIT == 1) {
        float* prow = static_cast<float*>(p.part_o) + row_id * D;
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
          if (db > 0) acc_step(o[db - 1], o[db]);
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int d0 = 32 * db + 8 * q4 + 4 * hf;
            f32x4 v4 = {o[db][4 * q4] * inv, o[db][4 * q4 + 1] * inv, o[db][4 * q4 + 2] * inv,
                        o[db][4 * q4 + 3] * inv};
            *reinterpret_cast<f32x4*>(prow + d0) = v4;
          }
        }
      } else {
        uint16_t* prow = static_cast<uint16_t*>(p.part_o) + row_id * D;
        // the row's largest magnitude (this lane's half of the dims, then the other half's
        // lane): o / l is stored as fp16 times 2^-e with that magnitude in [0.5, 1)
        float mx = 0.0f;
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
          if (db > 0) acc_step(o[db - 1], o[db]);
#pragma unroll
          for (int q = 0; q < 16; ++q) mx = fmaxf(mx, fabsf(o[db][q]));
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32)) * inv;
        // (e at least -127: inv 2^-e stays finite, inv being at most 1 as l >= 1; a row below
        // 2^-127 keeps its largest magnitude at or above 2^-14, an fp16 normal, down to 2^-141)
        e = (mx > 0.0f && mx <= 3.4028234e38f) ? max(__builtin_amdgcn_frexp_expf(mx), -127) : 0;
        // one multiply by inv 2^-e (a power-of-two scaling of inv: exact unless it falls below
        // the normal range, for rows of magnitude near the fp32 maximum)
        const float sc = __builtin_amdgcn_ldexpf(inv, -e);
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
          if (db > 0) acc_step(o[db - 1], o[db]);
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            u32x2 w;
            w[0] = pack2<1>(o[db][4 * q4] * sc, o[db][4 * q4 + 1] * sc);
            w[1] = pack2<1>(o[db][4 * q4 + 2] * sc, o[db][4 * q4 + 3] * sc);
            *reinterpret_cast<u32x2*>(prow + 32 * db + 8 * q4 + 4 * hf) = w;
          }
        }
      }
      // an empty chunk has l = 0 and lse = -inf; a NaN sum keeps its NaN (the merge redoes the row)
      if (hf == 0) {
        p.part_lse[row_id] = l_tot > 0.0f ? (m_run + __log2f(l_tot)) * kLn2 : l_tot == 0.0f ? -INFINITY : NAN;
        if constexpr (SPLIT == 2) p.part_e[row_id] = e;
      }
    }
    return nan_seen;
  };

  // ---- nonfinite repair.  A key that a pair cannot see still sits in the tile that P.V
  // multiplies, with weight 0, and a V value of +-Inf or NaN there makes 0 * Inf = NaN, a
  // product the definition never forms (it sums over the admissible keys only).  With one
  // split, a pair whose output holds a NaN is therefore computed again, key by key over this
  // workgroup's key range, touching admissible keys only: plain fp32 on the VALU, slow,
  // reached only by inputs that hold nonfinite values (a NaN that the definition itself
  // produces comes out NaN again).  With several splits the merge does the same per chunk
  // (kept out of this kernel: the repair's code alone changes how the compiler schedules the
  // tile loop).
  // a pair (its own lane or the lane 32 away) whose normalised O came out NaN is computed again
  auto repair = [&](bool nan_seen, bool valid, int h, int r, int lim, int64_t mrow) {
    if constexpr (!SPLIT) {
      const uint64_t bm = __builtin_amdgcn_ballot_w64(nan_seen);
      if (bm != 0 && valid && (((bm >> li) | (bm >> (li + 32))) & 1u) != 0) {
        exact_pair<D, DT, MK>(p, b, h, r, hf, kv_lo, min(kv_end, lim), mrow, kbase, vbase);
      }
    }
  };
  acc_settle(o0);
  repair(finish(valid0, h0, r0, lt0, m0, o0), valid0, h0, r0, lim0, mrow0);
}

// shape 0: four wavefronts; 2: eight with the lagged P.V; 3: eight without it.  ml: the mask
// layout in LDS (0: none, per-lane loads; 1: 16-byte rows, shape 2 at head dim 256 only; 2: words).
template <int D, int DT, int MK, int SPLIT>
hipError_t launch_fwd_s(const FwdParams& p, int shape, hipStream_t stream) {
  // the carried work rides on the unmasked lagged shape with fp16 partials only (the host's plan)
  if (p.extra_blocks != 0 && (SPLIT != 2 || shape != 2 || MK != 0)) return hipErrorInvalidValue;
  const dim3 grid(p.grid + p.extra_blocks), b4(256), b8(512);
  const int ml = MK != 0 ? p.mask_lds : 0;
  if constexpr (MK != 0) {
    if (ml == 2) {
      if (shape == 0) hipLaunchKernelGGL((attn_fwd_kernel<D, DT, MK, 4, false, 2, SPLIT>), grid, b4, 0, stream, p);
      else if (shape == 2) hipLaunchKernelGGL((attn_fwd_kernel<D, DT, MK, 8, true, 2, SPLIT>), grid, b8, 0, stream, p);
      else hipLaunchKernelGGL((attn_fwd_kernel<D, DT, MK, 8, false, 2, SPLIT>), grid, b8, 0, stream, p);
      return hipGetLastError();
    }
    if (ml == 1) {
      if constexpr (D != 256) {
        return hipErrorInvalidValue;
      } else {
        if (shape != 2) return hipErrorInvalidValue;
        hipLaunchKernelGGL((attn_fwd_kernel<D, DT, MK, 8, true, 1, SPLIT>), grid, b8, 0, stream, p);
        return hipGetLastError();
      }
    }
  }
  if (shape == 0) hipLaunchKernelGGL((attn_fwd_kernel<D, DT, MK, 4, false, 0, SPLIT>), grid, b4, 0, stream, p);
  else if (shape == 2) hipLaunchKernelGGL((attn_fwd_kernel<D, DT, MK, 8, true, 0, SPLIT>), grid, b8, 0, stream, p);
  else hipLaunchKernelGGL((attn_fwd_kernel<D, DT, MK, 8, false, 0, SPLIT>), grid, b8, 0, stream, p);
  return hipGetLastError();
}

// the split form is a compile-time choice (0: no split, 1: fp32 partials, 2: fp16 partials
// and their exponents): the epilogue writes either the gated output or the split partials, and
// only the former carries the in-kernel nonfinite repair; the partials' kind is a template
// argument as well, since a runtime choice between the two partial epilogues costs the kernel
// a second copy of its accumulators
template <int D, int DT, int MK>
hipError_t launch_fwd_t(const FwdParams& p, int shape, hipStream_t stream) {
  if (p.n_splits <= 1) return launch_fwd_s<D, DT, MK, 0>(p, shape, stream);
  return p.part_kind == 1 ? launch_fwd_s<D, DT, MK, 2>(p, shape, stream) : launch_fwd_s<D, DT, MK, 1>(p, shape, stream);
}

// every variant of head dim D (the planted-mistake builds: head dim 256 in bf16 without a mask)
template <int D>
hipError_t launch_fwd_d(const FwdParams& p, int dtype, int mask_kind, int shape, hipStream_t stream) {
#if GQA_CONTROL
  if (D != 256 || dtype != 0 || mask_kind != 0) return hipErrorInvalidValue;
  return launch_fwd_t<256, 0, 0>(p, shape, stream);
#else
  if (dtype == 0) {
    switch (mask_kind) {
      case 0: return launch_fwd_t<D, 0, 0>(p, shape, stream);
      case 1: return launch_fwd_t<D, 0, 1>(p, shape, stream);
      case 2: return launch_fwd_t<D, 0, 2>(p, shape, stream);
      default: return launch_fwd_t<D, 0, 3>(p, shape, stream);
    }
  }
  switch (mask_kind) {
    case 0: return launch_fwd_t<D, 1, 0>(p, shape, stream);
    case 1: return launch_fwd_t<D, 1, 1>(p, shape, stream);
    case 2: return launch_fwd_t<D, 1, 2>(p, shape, stream);
    default: return launch_fwd_t<D, 1, 3>(p, shape, stream);
  }
#endif
}

}  // namespace
}  // namespace gqa
