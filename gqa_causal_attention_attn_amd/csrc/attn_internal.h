// Internal declarations shared by the host side and the kernel launchers of libgqa_attn.
// Not part of the public ABI (include/gqa_attn.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Planted-mistake builds, for the tests that must see a wrong kernel miss the oracle (TensorFold
// PR #1009, Receipt, "Attention": controls that must go red): 1 = a query row sees one key past
// its own; 2 = the merge drops the last chunk of a row; 3 = the append lands one row late.  Such
// a build goes to a library of its own with the head-256 main pass in bf16 without a mask only;
// the product library is built with 0.
#ifndef GQA_CONTROL
#define GQA_CONTROL 0
#endif

namespace gqa {

constexpr int kHeadDim = 256;
constexpr int kKeysPerTile = 32;     // keys staged in LDS per step at head dim 256
// keys per tile of the main pass at head dim D: a K (or V) tile is 16 KiB whatever D
constexpr int tile_keys(int D) { return 8192 / D; }
constexpr int kBlocksPerGroup = 8;   // 32-pair column blocks of the largest workgroup
constexpr int kPairsPerBlock = 32;   // (head, row) pairs per column block (the MFMA N dimension)
constexpr int kTileBytes = kKeysPerTile * kHeadDim * 2;      // one K (or V) tile: 16 KiB of data
constexpr int kGroupStride = 1040;   // LDS bytes per two-key group: 1 KiB + a 16-byte bank skew
constexpr int kTileLds = (kKeysPerTile / 2) * kGroupStride;  // one K (or V) tile in LDS: 16,640 B
constexpr int kStageLds = 2 * kTileLds;                      // one stage = K tile + V tile
constexpr int kStages = 4;                                   // LDS stages of (K tile, V tile)
constexpr int kPrefetch = 2;                                 // tiles in flight ahead of the one consumed
constexpr int kFwdLdsBytes = kStages * kStageLds;            // 133,120 B
constexpr int kTargetBlocks = 256;   // main-pass workgroups aimed for (one per CU)
// A prompt main pass carries work on its idle CUs (FwdParams extra_blocks) when that work is
// covered by the main pass: a merge the size of the call's own (n_rows rows, five fp16 chunks)
// takes about 1.25 us per row on one wavefront there, eight wavefronts a CU, and a main-pass tile
// 1.7 us or more at every head dim, so the launch carries it when n_rows <= kCarryRowsPerTile x
// idle CUs x tiles per split (10 leaves a margin of about 1.1).
constexpr int64_t kCarryRowsPerTile = 10;
constexpr int kMaskStageLds = 4352;  // LDS bytes per stage for the mask window of a tile (masked kernels)
constexpr size_t kScratchBytes = (size_t)64 << 20;  // the device scratch of attn_decode_noalloc, per GPU

// The main pass's inputs, handed to the merge so that it can compute a chunk partial again
// when the main pass left a NaN in it (a key hidden from a row met a nonfinite V value in a
// tile the row shares with others).  q == nullptr: no repair (a merge called on its own).
struct RepairParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const void* mask;
  int64_t q_sb, q_sh, q_sr;
  int64_t k_sb, k_sh, k_st;
  int64_t v_sb, v_sh, v_st;
  int64_t m_sb, m_sh, m_sr;
  int mask_kind, G, kv_offset, kv_len, causal, keys_per_split;
  float scale_log2;
};

struct AppendParams {
  const uint16_t* src[2];
  uint16_t* dst[2];
  int64_t s_sb[2], s_sh[2], s_sr[2];
  int64_t d_sb[2], d_sh[2], d_st[2];
  int B, Hkv, rows;
  int kv_offset;
  int chunk_shift;  // log2 of the 16-byte chunks per row: 3, 4 or 5 (head dim 64, 128 or 256)
};

// The append's workgroups: x over (row, 16-byte chunk) pairs of `threads` threads, y over
// (tensor, b, g), each capped (the kernel strides over what a cap leaves).
inline void append_grid(const AppendParams& p, int threads, int64_t* bx, int64_t* by) {
  *bx = (((int64_t)p.rows << p.chunk_shift) + threads - 1) / threads;
  if (*bx > 1024) *bx = 1024;
  *by = 2LL * p.B * p.Hkv;
  if (*by > 65535) *by = 65535;
}

struct MergeParams {
  const void* part_o;  // part_kind 0: fp32 rows of D; 1: the main pass's fp16 rows (partial_row_bytes)
  const float* part_lse;
  const int32_t* part_e;  // part_kind 1: each row's power of two
  int part_kind;
  const uint16_t* gate;
  uint16_t* out;
  int64_t g_sb, g_sh, g_sr;
  int64_t o_sb, o_sh, o_sr;
  int n_chunks, B, Hq, rows;
  int D;  // head dim: 256, 128 or 64 (the partials' row length)
  RepairParams fix;
  // carry = 1: a kv_append (app) carried by the same launch: workgroups from merge_blocks on run
  // it, app_bx x app_by of them, as the append kernel's grid would (all three set by the launcher)
  int carry;
  AppendParams app;
  int app_bx, app_by;
  int merge_blocks;
};

// Parameters of the main (flash / split-KV) pass.  Strides are in elements.
struct FwdParams {
  const uint16_t* q;
  const uint16_t* gate;
  uint16_t* out;
  const uint16_t* k;
  const uint16_t* v;
  const void* mask;
  void* part_o;      // [n_splits, B, Hq, rows, D]: fp32 (part_kind 0) or fp16 (1, partial_row_bytes)
  float* part_lse;   // [n_splits, B, Hq, rows]
  int32_t* part_e;   // [n_splits, B, Hq, rows]: the power of two of each fp16 partial row
  int part_kind;     // 0 or 1, as the merge's
  int64_t q_sb, q_sh, q_sr;
  int64_t g_sb, g_sh, g_sr;
  int64_t o_sb, o_sh, o_sr;
  int64_t k_sb, k_sh, k_st;
  int64_t v_sb, v_sh, v_st;
  int64_t m_sb, m_sh, m_sr;
  int kv_offset;
  int kv_len;
  int B, Hq, Hkv, G, rows;
  int causal;
  float scale_log2;      // scale * log2(e)
  float scale;           // the score scale itself (additive masks add in natural-log units)
  int chunk;             // heads per chunk
  int blocks_per_chunk;  // column blocks serving one chunk
  int n_tiles;           // workgroups per (batch, kv head, split)
  int n_splits;
  int keys_per_split;    // multiple of kKeysPerTile
  int grid;              // workgroups in the launch
  int mask_lds;          // mask window of each tile staged in LDS: 0 no (per-lane loads), 1 in
                         // 16-byte row chunks, 2 one dword per key (see attn_fwd.h)
  int mask_pairs;        // with mask_lds 2: the window's rows are the mask rows of the workgroup's
                         // (head, row) pairs (a full-head mask, one column block of pairs)
                         // instead of its query rows (a mask the same for every head)
  // Work carried by the launch (prompt main passes writing fp16 partials, on CUs the main pass
  // leaves idle): workgroups grid .. grid + extra_blocks - 1 run it instead of the main pass.
  // carried.n_chunks > 0: the merge of an earlier call's fp16 partials (at most kFewChunks
  // chunks, no repair inputs); carried.carry = 1: the kv_append carried.app over an
  // app_bx x app_by grid of those workgroups.
  int extra_blocks;
  MergeParams carried;
};

constexpr int kKeepMaxBatch = 64;  // keep masks travel in the kernel arguments

struct KeepParams {
  uint16_t* cache[2];       // K, V
  int64_t c_sb[2], c_sh[2], c_st[2];
  int Hkv, rows, kv_offset;
  uint32_t keep[kKeepMaxBatch];
};

// Parameters of the composed (materialised-score) arm: the fused pass's inputs plus the
// workspace of scores s, 16-bit weights pw (both [B, Hq, rows, kvp]) and 1 / l per row.
struct ComposedParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* gate;
  uint16_t* out;
  int64_t q_sb, q_sh, q_sr;
  int64_t k_sb, k_sh, k_st;
  int64_t v_sb, v_sh, v_st;
  int64_t g_sb, g_sh, g_sr;
  int64_t o_sb, o_sh, o_sr;
  float* s;
  uint16_t* pw;
  float* inv_l;
  int64_t kvp;  // keys per row of s and pw: the key range rounded up to 32
  int D;        // head dim: 64, 128 or 256
  int B, Hq, G, rows, kv_offset, kv_len, causal, kv_hi;
  float scale_log2;
};

// Split partial rows.  Kind 0: the D values of o / l in fp32.  Kind 1: the D values of o / l
// times 2^-e in fp16 (round to nearest even), e chosen so that the row's largest magnitude lands
// in [0.5, 1) (0 when it is 0 or not finite); e goes to an int32 array of its own beside the lse,
// so a row is whole 128-byte lines (D = 64, 128, 256) and no write covers part of a line.  The
// merge multiplies each kind-1 value by 2^e exactly.
constexpr int64_t partial_row_bytes(int D, int kind) { return (kind == 1 ? 2 : 4) * (int64_t)D; }
// Kind 1 halves the partials' write and read-back at the price of an exponent pass in the main
// pass's epilogue, which only pays where the partials are large: the planner takes it from
// 8 MiB of fp32 partials up (prompt blocks, verify rows), kind 0 below (short decodes).
constexpr int64_t kHalfPartialsFromBytes = (int64_t)8 << 20;

// Merge launch shape, shared by the launcher and the host's checks.  Up to kFewChunks chunks,
// and up to 64 (32 of fp32 partials) where the rows fill the chip (kWideMergeRows: a workgroup
// of four rows per CU), take one wavefront per row, four rows a workgroup, with
// merge_slots(n, kind, rows) chunk slots: the chunk count itself up to kFewChunks, else the
// count rounded up to a multiple of 4 (up to 32) or of 8 (up to 64).  The rest take a workgroup
// of merge_waves(n) wavefronts per row.
constexpr int kFewChunks = 8;
constexpr int kMergeBatch = 4;  // chunks a wavefront of the many-chunk merge loads at once
constexpr int64_t kWideMergeRows = 1024;
inline int merge_slots(int n_chunks, int kind, int64_t n_rows) {
  if (n_chunks <= kFewChunks) return n_chunks;
  if (n_rows < kWideMergeRows) return 0;
  if (n_chunks <= 32) return (n_chunks + 3) / 4 * 4;
  return n_chunks <= 64 && kind == 1 ? (n_chunks + 7) / 8 * 8 : 0;
}
inline int merge_waves(int n_chunks) {
  return n_chunks <= 4 * kMergeBatch ? 4 : n_chunks <= 8 * kMergeBatch ? 8 : 16;
}
// A launch dimension holds at most 2^32 - 1 work-items.
inline bool grid_fits(int64_t blocks, int64_t threads) { return blocks >= 1 && blocks * threads <= 0xffffffffLL; }
// The merge's own launch: workgroups and threads per workgroup.
inline void merge_shape(int n_chunks, int kind, int64_t n_rows, int64_t* blocks, int* threads) {
  if (merge_slots(n_chunks, kind, n_rows) > 0) {
    *blocks = (n_rows + 3) / 4;
    *threads = 256;
  } else {
    *blocks = n_rows;
    *threads = 64 * merge_waves(n_chunks);
  }
}
inline bool merge_fits(int n_chunks, int kind, int64_t n_rows) {
  int64_t blocks;
  int threads;
  merge_shape(n_chunks, kind, n_rows, &blocks, &threads);
  return grid_fits(blocks, threads);
}
// The merge's launch with a carried append: the merge's workgroups plus the append's.
inline bool merge_with_append_fits(int n_chunks, int kind, int64_t n_rows, const AppendParams& app) {
  int64_t blocks, bx, by;
  int threads;
  merge_shape(n_chunks, kind, n_rows, &blocks, &threads);
  append_grid(app, threads, &bx, &by);
  return grid_fits(blocks + bx * by, threads);
}

// Launchers (return hipGetLastError()).  dtype 0 = bf16, 1 = fp16; mask_kind as attn_mask_kind.
// shape: 0 = 4 wavefronts, 2 = 8 wavefronts with the P.V product one tile behind (prompts),
// 3 = 8 wavefronts without that lag (decode / verify); each wavefront one 32-pair column block.
// The main pass per head dim (attn_fwd_d256.hip, attn_fwd_d128.hip, attn_fwd_d64.hip).
hipError_t launch_fwd_256(const FwdParams& p, int dtype, int mask_kind, int shape, hipStream_t stream);
hipError_t launch_fwd_128(const FwdParams& p, int dtype, int mask_kind, int shape, hipStream_t stream);
hipError_t launch_fwd_64(const FwdParams& p, int dtype, int mask_kind, int shape, hipStream_t stream);
inline hipError_t launch_fwd(const FwdParams& p, int D, int dtype, int mask_kind, int shape, hipStream_t stream) {
  return D == 256 ? launch_fwd_256(p, dtype, mask_kind, shape, stream)
                  : D == 128 ? launch_fwd_128(p, dtype, mask_kind, shape, stream)
                             : launch_fwd_64(p, dtype, mask_kind, shape, stream);
}
hipError_t launch_merge(const MergeParams& p, int dtype, hipStream_t stream);
hipError_t launch_append(const AppendParams& p, hipStream_t stream);
hipError_t launch_keep(const KeepParams& p, int B, hipStream_t stream);
hipError_t launch_composed(const ComposedParams& p, int dtype, hipStream_t stream);
// Device address of the library's scratch array on the current device (looked up on the first
// call per device and kept; attn_noalloc.hip).
hipError_t scratch_of_current_device(void** ptr);

}  // namespace gqa
