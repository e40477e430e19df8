// Merge pass and KV append for gfx950.
//
// Merge (TensorFold PR #1009, attention kernel-contract commit: decode rows over key chunks
// and a merge of the chunks): per (b, h, r), lse = log sum_c exp(lse_c),
// out = sum_c exp(lse_c - lse) o_c * sigmoid(gate), an empty chunk (lse_c = -Inf) adds
// nothing (its slot is selected out, never multiplied in) and a row with every chunk empty
// gives 0; a chunk whose lse is NaN makes the row NaN.  Few chunks: one wavefront per row
// with every partial loaded at once; many chunks (decode): one workgroup of 4, 8 or 16
// wavefronts per row (the fewest that hold the chunks), each loading its share of the chunks
// at once.  HBM-bound (n_chunks x (4 D + 4) bytes per row).
//
// Append and keep (the same commit compares both bit for bit, keep also when it is repeated
// on the caches its first call produced): 16-byte copies of K/V rows into the cache, no arithmetic on the bits.
// Keep compacts the accepted rows of a verify block in place, one workgroup per (b, g) reading
// every kept row before writing any.
#include <hip/hip_runtime.h>
#include <math.h>

#include "attn_internal.h"
#include "attn_merge_core.h"

namespace gqa {
namespace {

using mcore::u32x4;
using mcore::u32x2;
using mcore::f32x4;
using mcore::kLog2e;
using mcore::to_f32;
using mcore::pack2;
using mcore::wave_max;
using mcore::PartialLoad;
using mcore::load_values;
using mcore::decode_partial;

// Nonfinite repair of a row (b, h, r) whose chunk partials hold a NaN (a key hidden from the
// row met a nonfinite V value in a tile the row shared with others, and 0 * Inf became NaN):
// the row's output computed again from the main pass's inputs over its admissible keys only,
// by the plain definition in fp32, one key at a time, the whole wavefront on the row (lanes
// below D / 4 hold 4 dims each, dims 4 lane .. + 3, the others none; every score is summed
// across the wavefront and taken from lane 0, so all lanes use the same one), gated and rounded
// once.  A NaN that the definition itself produces comes out NaN again.  Only rows with such a
// chunk get here.
template <int DT>
__device__ __forceinline__ void exact_row(const RepairParams& f, int D, int b, int h, int r, int lane, u32x2 gw,
                                          uint16_t* orow) {
  const int g = h / f.G;
  const int hi = f.causal ? min(f.kv_len, f.kv_offset + r + 1) : f.kv_len;
  const int lo = 0;
  const bool on = 4 * lane < D;  // this lane holds dims of the row
  const int dl = on ? 4 * lane : 0;
  const u32x2 qw0 = *reinterpret_cast<const u32x2*>(f.q + (int64_t)b * f.q_sb + (int64_t)h * f.q_sh +
                                                    (int64_t)r * f.q_sr + dl);
  const u32x2 qw = on ? qw0 : (u32x2){0u, 0u};
  const float q0 = to_f32<DT>((uint16_t)(qw[0] & 0xffffu)), q1 = to_f32<DT>((uint16_t)(qw[0] >> 16));
  const float q2 = to_f32<DT>((uint16_t)(qw[1] & 0xffffu)), q3 = to_f32<DT>((uint16_t)(qw[1] >> 16));
  const uint16_t* kb = f.k + (int64_t)b * f.k_sb + (int64_t)g * f.k_sh + dl;
  const uint16_t* vb = f.v + (int64_t)b * f.v_sb + (int64_t)g * f.v_sh + dl;
  const int64_t mrow = (int64_t)b * f.m_sb + (int64_t)h * f.m_sh + (int64_t)r * f.m_sr;
  // the score of key j in log2 units; adm: the mask does not hide it
  auto score = [&](int j, bool& adm) {
    float mt = 0.0f;
    if (f.mask_kind == 1) mt = static_cast<const uint8_t*>(f.mask)[mrow + j] ? 0.0f : -INFINITY;
    else if (f.mask_kind == 2) mt = to_f32<DT>(static_cast<const uint16_t*>(f.mask)[mrow + j]);
    else if (f.mask_kind == 3) mt = static_cast<const float*>(f.mask)[mrow + j];
    adm = mt > -INFINITY;
    const u32x2 kw = *reinterpret_cast<const u32x2*>(kb + (int64_t)j * f.k_st);
    float part = q0 * to_f32<DT>((uint16_t)(kw[0] & 0xffffu));
    part = __builtin_fmaf(q1, to_f32<DT>((uint16_t)(kw[0] >> 16)), part);
    part = __builtin_fmaf(q2, to_f32<DT>((uint16_t)(kw[1] & 0xffffu)), part);
    part = __builtin_fmaf(q3, to_f32<DT>((uint16_t)(kw[1] >> 16)), part);
    part = on ? part : 0.0f;  // lanes past the head dim add nothing (not even 0 * Inf)
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
    part = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, part)));
    return (part * f.scale_log2) + mt * kLog2e;
  };
  bool any = false, nan_s = false;
  float m = -INFINITY;
#pragma nounroll
  for (int j = lo; j < hi; ++j) {
    bool adm;
    const float x = score(j, adm);
    if (!adm) continue;
    any = true;
    nan_s = nan_s || __builtin_isnan(x);
    m = fmaxf(m, x);
  }
  if (nan_s) m = NAN;  // the max of a set holding NaN
  float l = 0.0f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma nounroll
  for (int j = lo; j < hi; ++j) {
    bool adm;
    const float x = score(j, adm);
    if (!adm) continue;
    const float w = exp2f(x - m);
    l += w;
    const u32x2 vw = *reinterpret_cast<const u32x2*>(vb + (int64_t)j * f.v_st);
    acc[0] = __builtin_fmaf(w, to_f32<DT>((uint16_t)(vw[0] & 0xffffu)), acc[0]);
    acc[1] = __builtin_fmaf(w, to_f32<DT>((uint16_t)(vw[0] >> 16)), acc[1]);
    acc[2] = __builtin_fmaf(w, to_f32<DT>((uint16_t)(vw[1] & 0xffffu)), acc[2]);
    acc[3] = __builtin_fmaf(w, to_f32<DT>((uint16_t)(vw[1] >> 16)), acc[3]);
  }
  const float inv = any ? 1.0f / l : 0.0f;  // a row with no admissible key gives 0
  const float gv[4] = {to_f32<DT>((uint16_t)(gw[0] & 0xffffu)), to_f32<DT>((uint16_t)(gw[0] >> 16)),
                       to_f32<DT>((uint16_t)(gw[1] & 0xffffu)), to_f32<DT>((uint16_t)(gw[1] >> 16))};
  float res[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) res[i] = acc[i] * inv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv[i]));
  u32x2 ow;
  ow[0] = pack2<DT>(res[0], res[1]);
  ow[1] = pack2<DT>(res[2], res[3]);
  if (on) *reinterpret_cast<u32x2*>(orow + dl) = ow;
}

// Workgroups of a merge launch past the merge's own run the kv_append it carries; returns
// whether this workgroup was one of them (the whole workgroup, so it leaves before any barrier).
__device__ __forceinline__ bool merge_carried_append(const MergeParams& p) {
  if (blockIdx.x < (uint32_t)p.merge_blocks) return false;
  const uint32_t a = blockIdx.x - (uint32_t)p.merge_blocks;
  const uint32_t by = a / (uint32_t)p.app_bx;
  mcore::append_part<1>(p.app, a - by * (uint32_t)p.app_bx, by, (uint32_t)p.app_bx, (uint32_t)p.app_by, blockDim.x);
  return true;
}

// whether any of the four values is NaN
__device__ __forceinline__ bool has_nan4(const f32x4& x) { return __builtin_isnan(x[0] + x[1] + x[2] + x[3]); }

// Many chunks: one workgroup of MW wavefronts per row (MW = 4, 8 or 16, the fewest whose
// MW x kMergeBatch slots hold the chunks, up to 16); wavefront w takes the chunks w, w + MW, ...
// (kMergeBatch per pass).  A pass issues all of its lse and partial loads (and the gate) at
// once; only the row's largest lse crosses the wavefronts (through LDS) before the weights are
// applied, so a row up to MW x kMergeBatch chunks costs one round trip to memory.  The partial
// sums meet in LDS.
template <int DT, int MW, int KIND>
__global__ __launch_bounds__(MW * 64) void merge_kernel(const MergeParams p) {
  if (merge_carried_append(p)) return;
  constexpr int kMergeWaves = MW;
  __shared__ f32x4 part_acc[kMergeWaves][64];
  __shared__ float part_w[kMergeWaves];
  __shared__ float part_top[kMergeWaves];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t n_rows = (int64_t)p.B * p.Hq * p.rows;
  const int64_t row_id = blockIdx.x;
  const uint32_t bh = blockIdx.x / (uint32_t)p.rows;
  const int r = (int)(blockIdx.x - bh * (uint32_t)p.rows);
  const int b = (int)(bh / (uint32_t)p.Hq);
  const int h = (int)(bh - (uint32_t)b * (uint32_t)p.Hq);
  const int d0 = 4 * lane;
  const int dl = min(d0, p.D - 4);  // lanes past the head dim re-read its last 4 dims and store nothing
  const uint16_t* grow = p.gate + (int64_t)b * p.g_sb + (int64_t)h * p.g_sh + (int64_t)r * p.g_sr;
  const u32x2 gw = *reinterpret_cast<const u32x2*>(grow + dl);

  // acc and wsum are kept relative to ref, the largest lse seen so far (the same in every
  // wavefront: each pass's largest lse is shared through LDS)
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.0f;
  float ref = -INFINITY;
  bool nan_l = false;  // a chunk whose lse is NaN makes the row NaN, as the unsplit definition does
  const int nch = GQA_CONTROL == 2 ? max(p.n_chunks - 1, 1) : p.n_chunks;
  for (int c0 = 0; c0 < nch; c0 += kMergeWaves * kMergeBatch) {
    // this pass's chunks of the wavefront, all loads in flight together (indices past the
    // last chunk re-read it and are selected out)
    // lane j (j < kMergeBatch) loads the lse and exponent of the wavefront's j-th chunk; they are
    // read out of those lanes as scalars
    const int64_t lrow = (int64_t)min(c0 + wave + min(lane, kMergeBatch - 1) * kMergeWaves, nch - 1) * n_rows + row_id;
    const float lse_lane = p.part_lse[lrow];
    int32_t e_lane = 0;
    if constexpr (KIND == 1) e_lane = p.part_e[lrow];
    PartialLoad<KIND> raw[kMergeBatch];
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const int cc = min(c0 + wave + j * kMergeWaves, nch - 1);
      raw[j] = load_values<KIND>(p, (int64_t)cc * n_rows + row_id, dl);
    }
    float lc[kMergeBatch];
    f32x4 oc[kMergeBatch];
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      lc[j] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lse_lane), j));
      if constexpr (KIND == 1) raw[j].e = __builtin_amdgcn_readlane(e_lane, j);
      oc[j] = decode_partial<KIND>(raw[j]);
    }
    float top = -INFINITY;
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const bool in = c0 + wave + j * kMergeWaves < nch;
      top = in ? fmaxf(top, lc[j]) : top;
      nan_l = nan_l || (in && __builtin_isnan(lc[j]));
    }
    if (lane == 0) part_top[wave] = top;
    __syncthreads();
    float pass_top = part_top[0];
#pragma unroll
    for (int w = 1; w < kMergeWaves; ++w) pass_top = fmaxf(pass_top, part_top[w]);
    const float new_ref = fmaxf(ref, pass_top);
    if (ref > -INFINITY && new_ref > ref) {
      const float f = exp2f((ref - new_ref) * kLog2e);
      acc *= f;
      wsum *= f;
    }
    ref = new_ref;
    if (ref > -INFINITY) {
#pragma unroll
      for (int j = 0; j < kMergeBatch; ++j) {
        // an empty chunk is selected out, never multiplied in
        if (c0 + wave + j * kMergeWaves < nch && lc[j] != -INFINITY) {
          const float w = exp2f((lc[j] - ref) * kLog2e);
          acc += w * oc[j];
          wsum += w;
        }
      }
    }
    __syncthreads();  // part_top is rewritten by the next pass
  }
  part_acc[wave][lane] = acc;
  if (lane == 0) part_w[wave] = nan_l ? NAN : wsum;
  __syncthreads();
  if (wave != 0) return;
  acc = part_acc[0][lane];
  wsum = part_w[0];
#pragma unroll
  for (int w = 1; w < kMergeWaves; ++w) {
    acc += part_acc[w][lane];
    wsum += part_w[w];
  }
  uint16_t* orow = p.out + (int64_t)b * p.o_sb + (int64_t)h * p.o_sh + (int64_t)r * p.o_sr;
  // a NaN in the sums (a chunk's partial or lse held one) with the main pass's inputs at hand:
  // the row is computed again (a wavefront-uniform branch)
  if (p.fix.q && __builtin_amdgcn_ballot_w64(__builtin_isnan(wsum) || (d0 < p.D && has_nan4(acc))) != 0) {
    exact_row<DT>(p.fix, p.D, b, h, r, lane, gw, orow);
    return;
  }
  // a NaN weight sum carries a NaN chunk of some wavefront
  const float inv = __builtin_isnan(wsum) ? NAN : wsum > 0.0f ? __builtin_amdgcn_rcpf(wsum) : 0.0f;
  float gv[4] = {to_f32<DT>((uint16_t)(gw[0] & 0xffffu)), to_f32<DT>((uint16_t)(gw[0] >> 16)),
                 to_f32<DT>((uint16_t)(gw[1] & 0xffffu)), to_f32<DT>((uint16_t)(gw[1] >> 16))};
  float res[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) res[i] = acc[i] * inv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv[i]));
  u32x2 ow;
  ow[0] = pack2<DT>(res[0], res[1]);
  ow[1] = pack2<DT>(res[2], res[3]);
  if (d0 < p.D) *reinterpret_cast<u32x2*>(orow + d0) = ow;
}

// Chunks up to 64 (merge_slots): one wavefront per row, four rows per workgroup, four dims per
// lane, and a partial load of every chunk slot issued at once (independent loads), so the pass
// costs one round trip instead of a load after another.  NC slots: NC = the chunk count for up
// to 8 chunks, else the chunk count rounded up to a multiple of 4 up to 32, of 8 up to 64 (fp32
// partials: up to 32), the slots past the row's chunks re-reading its last chunk and selected
// out (each slot costs its load: 17 chunks in 32 slots took 1.3x the time of 16 in 16).  Lane c holds chunk c's lse (and
// exponent) and works out its weight; the sum reads them out of the lanes in chunk order and
// decodes each partial as it goes.
template <int DT, int KIND, int NC>
__global__ __launch_bounds__(256) void merge_few_kernel(const MergeParams p) {
  if (merge_carried_append(p)) return;
  const int lane = threadIdx.x & 63;
  const int64_t n_rows = (int64_t)p.B * p.Hq * p.rows;
  const uint32_t row32 = blockIdx.x * 4u + (threadIdx.x >> 6);
  if (row32 >= (uint64_t)n_rows) return;
  const int64_t row_id = row32;
  // (b, h, r) of the row in 32-bit arithmetic (the host keeps B Hq rows below 2^31)
  const uint32_t bh = row32 / (uint32_t)p.rows;
  const int r = (int)(row32 - bh * (uint32_t)p.rows);
  const int b = (int)(bh / (uint32_t)p.Hq);
  const int h = (int)(bh - (uint32_t)b * (uint32_t)p.Hq);
  const int d0 = 4 * lane;
  const int dl = min(d0, p.D - 4);  // lanes past the head dim re-read its last 4 dims and store nothing
  constexpr bool kExact = NC <= kFewChunks;
  int nch;
  if constexpr (kExact) nch = GQA_CONTROL == 2 ? (NC > 1 ? NC - 1 : 1) : NC;
  else nch = GQA_CONTROL == 2 ? max(p.n_chunks - 1, 1) : p.n_chunks;
  const uint16_t* grow = p.gate + (int64_t)b * p.g_sb + (int64_t)h * p.g_sh + (int64_t)r * p.g_sr;
  const u32x2 gw = *reinterpret_cast<const u32x2*>(grow + dl);
  // lane c (c < nch; the others re-read chunk nch - 1) loads chunk c's lse and exponent
  const int64_t lrow = (int64_t)min(lane, nch - 1) * n_rows + row_id;
  float lse_lane = p.part_lse[lrow];
  int32_t e_lane = 0;
  if constexpr (KIND == 1) e_lane = p.part_e[lrow];
  PartialLoad<KIND> raw[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) raw[c] = load_values<KIND>(p, (int64_t)min(c, nch - 1) * n_rows + row_id, dl);
  // one use of every partial here, each passing the lse through, keeps all the loads together,
  // in one round trip: left alone, the compiler sinks each partial's load into its chunk's
  // branch, after the lse loads have come back, or works out the row's largest lse first
  // (loads made conditional on the slot holding a chunk were each followed by a wait)
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if constexpr (KIND == 0) {
      asm volatile("" : "+v"(lse_lane) : "v"(raw[c].f));
    } else {
      asm volatile("" : "+v"(lse_lane) : "v"(raw[c].h));
    }
  }
  const mcore::RowSums sums = mcore::row_sums<KIND, NC>(nch, lane, lse_lane, e_lane, raw);
  uint16_t* orow = p.out + (int64_t)b * p.o_sb + (int64_t)h * p.o_sh + (int64_t)r * p.o_sr;
  // a NaN in a chunk's partial or lse with the main pass's inputs at hand: the row is computed
  // again (one wavefront per row)
  if (p.fix.q &&
      __builtin_amdgcn_ballot_w64(sums.nan_l || __builtin_isnan(sums.wsum) || (d0 < p.D && has_nan4(sums.acc))) != 0) {
    exact_row<DT>(p.fix, p.D, b, h, r, lane, gw, orow);
    return;
  }
  const u32x2 ow = mcore::gated_row<DT>(sums, gw);
  if (d0 < p.D) *reinterpret_cast<u32x2*>(orow + d0) = ow;
}

// kv_append: one workgroup of the append grid (append_part).  Head dims 64, 128 and 256.
__global__ __launch_bounds__(256) void append_kernel(const AppendParams p) {
  mcore::append_part<1>(p, blockIdx.x, blockIdx.y, gridDim.x, gridDim.y, 256);
}

// kv_keep: one workgroup per (b, g).  Every kept row of the block is read into registers
// (1024 16-byte chunks of K and 1024 of V at most: 8 per thread), the workgroup waits until all
// reads have landed, and only then are the rows written to their new places (row r goes to
// kv_offset + the number of kept rows below r <= r), so moving rows in place is safe.
__global__ __launch_bounds__(256) void keep_kernel(const KeepParams p) {
  constexpr int kChunks = kHeadDim / 8;                        // 16-byte chunks per row
  constexpr int kPerThread = 2 * 32 * kChunks / 256;           // both tensors, 32 rows at most
  const int b = blockIdx.x / p.Hkv, g = blockIdx.x % p.Hkv;
  const uint32_t m = p.keep[b];
  u32x4 val[kPerThread];
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    const int u = threadIdx.x + 256 * k;
    const int t = u / (32 * kChunks), r = (u / kChunks) % 32, c = u % kChunks;
    if (r < p.rows && ((m >> r) & 1u)) {
      val[k] = *reinterpret_cast<const u32x4*>(p.cache[t] + b * p.c_sb[t] + g * p.c_sh[t] +
                                               (int64_t)(p.kv_offset + r) * p.c_st[t] + 8 * c);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // every read of this (b, g) has landed ...
  __syncthreads();                                   // ... in every thread, before any write
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    const int u = threadIdx.x + 256 * k;
    const int t = u / (32 * kChunks), r = (u / kChunks) % 32, c = u % kChunks;
    if (r < p.rows && ((m >> r) & 1u)) {
      const int d = __builtin_popcount(m & ((1u << r) - 1u));
      *reinterpret_cast<u32x4*>(p.cache[t] + b * p.c_sb[t] + g * p.c_sh[t] + (int64_t)(p.kv_offset + d) * p.c_st[t] +
                                8 * c) = val[k];
    }
  }
}

}  // namespace

hipError_t launch_keep(const KeepParams& p, int B, hipStream_t stream) {
  hipLaunchKernelGGL(keep_kernel, dim3((unsigned)(B * p.Hkv)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int KIND, int NC>
void launch_few_nc(const MergeParams& p, int dtype, dim3 grid, hipStream_t stream) {
  if (dtype == 0) hipLaunchKernelGGL((merge_few_kernel<0, KIND, NC>), grid, dim3(256), 0, stream, p);
  else hipLaunchKernelGGL((merge_few_kernel<1, KIND, NC>), grid, dim3(256), 0, stream, p);
}
template <int KIND>
void launch_few(const MergeParams& p, int dtype, dim3 grid, hipStream_t stream) {
  switch (merge_slots(p.n_chunks, KIND, (int64_t)p.B * p.Hq * p.rows)) {
    case 1: launch_few_nc<KIND, 1>(p, dtype, grid, stream); break;
    case 2: launch_few_nc<KIND, 2>(p, dtype, grid, stream); break;
    case 3: launch_few_nc<KIND, 3>(p, dtype, grid, stream); break;
    case 4: launch_few_nc<KIND, 4>(p, dtype, grid, stream); break;
    case 5: launch_few_nc<KIND, 5>(p, dtype, grid, stream); break;
    case 6: launch_few_nc<KIND, 6>(p, dtype, grid, stream); break;
    case 7: launch_few_nc<KIND, 7>(p, dtype, grid, stream); break;
    case 8: launch_few_nc<KIND, 8>(p, dtype, grid, stream); break;
    case 12: launch_few_nc<KIND, 12>(p, dtype, grid, stream); break;
    case 16: launch_few_nc<KIND, 16>(p, dtype, grid, stream); break;
    case 20: launch_few_nc<KIND, 20>(p, dtype, grid, stream); break;
    case 24: launch_few_nc<KIND, 24>(p, dtype, grid, stream); break;
    case 28: launch_few_nc<KIND, 28>(p, dtype, grid, stream); break;
    case 32: launch_few_nc<KIND, 32>(p, dtype, grid, stream); break;
    default:
      if constexpr (KIND == 1) {
        switch (merge_slots(p.n_chunks, KIND, (int64_t)p.B * p.Hq * p.rows)) {
          case 40: launch_few_nc<KIND, 40>(p, dtype, grid, stream); break;
          case 48: launch_few_nc<KIND, 48>(p, dtype, grid, stream); break;
          case 56: launch_few_nc<KIND, 56>(p, dtype, grid, stream); break;
          default: launch_few_nc<KIND, 64>(p, dtype, grid, stream); break;
        }
      }
      break;
  }
}

template <int KIND>
void launch_merge_k(const MergeParams& p0, int dtype, hipStream_t stream) {
  const int64_t n_rows = (int64_t)p0.B * p0.Hq * p0.rows;
  MergeParams p = p0;
  int64_t blocks;
  int threads;
  merge_shape(p.n_chunks, KIND, n_rows, &blocks, &threads);
  p.merge_blocks = (int)blocks;
  int64_t extra = 0;
  if (p.carry) {
    int64_t bx, by;
    append_grid(p.app, threads, &bx, &by);
    p.app_bx = (int)bx, p.app_by = (int)by;
    extra = bx * by;
  }
  const dim3 grid((unsigned)(blocks + extra));
  if (merge_slots(p.n_chunks, KIND, n_rows) > 0) {
    launch_few<KIND>(p, dtype, grid, stream);
  } else {
    const int mw = threads / 64;
    if (mw == 4) {
      if (dtype == 0) hipLaunchKernelGGL((merge_kernel<0, 4, KIND>), grid, dim3(4 * 64), 0, stream, p);
      else hipLaunchKernelGGL((merge_kernel<1, 4, KIND>), grid, dim3(4 * 64), 0, stream, p);
    } else if (mw == 8) {
      if (dtype == 0) hipLaunchKernelGGL((merge_kernel<0, 8, KIND>), grid, dim3(8 * 64), 0, stream, p);
      else hipLaunchKernelGGL((merge_kernel<1, 8, KIND>), grid, dim3(8 * 64), 0, stream, p);
    } else {
      if (dtype == 0) hipLaunchKernelGGL((merge_kernel<0, 16, KIND>), grid, dim3(16 * 64), 0, stream, p);
      else hipLaunchKernelGGL((merge_kernel<1, 16, KIND>), grid, dim3(16 * 64), 0, stream, p);
    }
  }
}

hipError_t launch_merge(const MergeParams& p, int dtype, hipStream_t stream) {
  if (p.part_kind == 0) launch_merge_k<0>(p, dtype, stream);
  else launch_merge_k<1>(p, dtype, stream);
  return hipGetLastError();
}

hipError_t launch_append(const AppendParams& p, hipStream_t stream) {
  int64_t bx, by;
  append_grid(p, 256, &bx, &by);
  hipLaunchKernelGGL(append_kernel, dim3((unsigned)bx, (unsigned)by), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gqa
