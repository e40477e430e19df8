// Host side of libgqa_attn: argument validation, the head-chunk and KV-split plans, workspace
// sizing, the launches, and the prompt policy (block size and route per head dim and device).  Every check runs before anything is enqueued, so an invalid call
// writes nothing.  Head counts are validated before any division (TensorFold PR #1009, the
// config-reader commit: zero heads and uneven head groups are refused with ordinary errors).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>

#include <string>
#include <vector>

#include "attn_internal.h"
#include "gqa_attn.h"

namespace {

using gqa::kHeadDim;
using gqa::kKeysPerTile;
using gqa::kBlocksPerGroup;
using gqa::kPairsPerBlock;

constexpr int kRowPairLimit = 32;  // the head-chunk rule's 32 (head, row) pairs per call

struct Plan {
  int G;
  int chunk;
  int n_chunks;
  int chunk_sizes[ATTN_MAX_CHUNKS];
  int blocks_per_chunk;
  int shape;     // 0: 4 wavefronts of one column block each; 2: 8 wavefronts, P.V one tile behind
                 // (prompts); 3: 8 wavefronts without the lag (decode / verify); 1 is not used
  int mask_lds;  // the main pass stages each tile's mask window in LDS: 0 no, 1 rows, 2 words,
                 // 3 words of the (head, row) pairs' rows (a full-head mask)
  int waves;     // wavefronts per workgroup
  int n_tiles;
  int n_splits;
  int keys_per_split;
  int64_t grid;
  int part_kind;       // partial rows in fp32 (0) or fp16 with a power of two per row (1)
  size_t ws_o_bytes;  // partial rows at offset 0, then the lse ...
  size_t ws_e_offset;  // ... and (kind 1) each row's power of two at this offset
  size_t ws_bytes;
};

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline bool strides_ok(const attn_tensor& t) {
  return t.stride_b % 8 == 0 && t.stride_h % 8 == 0 && t.stride_row % 8 == 0;
}

// The rule itself, for one group of `gqa` heads (callers validated the head counts).
int chunk_rule(int rows, int gqa, int enabled, int* sizes, int cap) {
  int n = 0;
  if (!enabled || rows > kRowPairLimit || (int64_t)rows * gqa <= kRowPairLimit) {
    if (cap < 1) return -1;
    sizes[n++] = gqa;
    return n;
  }
  const int size = gqa < kRowPairLimit / rows ? gqa : kRowPairLimit / rows;
  for (int left = gqa; left > 0; left -= size) {
    if (n >= cap) return -1;
    sizes[n++] = left < size ? left : size;
  }
  return n;
}

int validate(const attn_args* a, int op) {
  if (!a) return ATTN_E_NULL;
  if (op != ATTN_OP_PREFILL && op != ATTN_OP_DECODE && op != ATTN_OP_COMPOSED) return ATTN_E_ARG;
  if (a->dtype != ATTN_BF16 && a->dtype != ATTN_F16) return ATTN_E_DTYPE;
  if (a->B <= 0 || a->Hq <= 0 || a->Hkv <= 0) return ATTN_E_HEADS;
  if (a->Hq % a->Hkv != 0) return ATTN_E_HEADS;
  const int G = a->Hq / a->Hkv;
  if (G > ATTN_MAX_CHUNKS) return ATTN_E_HEADS;
  // head dims 256, 128 and 64 (the last two by their own kernels); any other fails closed
  if (a->D != ATTN_HEAD_DIM && a->D != 64 && a->D != 128) return ATTN_E_HEAD_DIM;
  if (a->rows < 1) return ATTN_E_ROWS;
  if (op == ATTN_OP_DECODE && a->rows > ATTN_MAX_DECODE_ROWS) return ATTN_E_ROWS;
  if (a->kv_offset < 0 || a->kv_len < 1 || a->capacity < a->kv_len) return ATTN_E_KV;
  // (kernels index keys in 32 bits, up to a tile of 128 keys past kv_len)
  if (a->kv_len > INT32_MAX - 128 || a->kv_offset + a->rows > INT32_MAX - 128) return ATTN_E_KV;
  if (a->causal && a->kv_len < a->kv_offset + a->rows) return ATTN_E_KV;
  if (!(a->scale >= 0.0f) || !isfinite(a->scale)) return ATTN_E_ARG;
  if (a->causal != 0 && a->causal != 1) return ATTN_E_ARG;
  if (a->n_splits < 0) return ATTN_E_ARG;
  if (a->head_chunk < 0 || a->head_chunk > G) return ATTN_E_HEAD_CHUNK;
  if (!a->q.ptr || !a->gate.ptr || !a->out.ptr || !a->k_cache.ptr || !a->v_cache.ptr) return ATTN_E_NULL;
  const attn_tensor* ts[5] = {&a->q, &a->gate, &a->out, &a->k_cache, &a->v_cache};
  for (const attn_tensor* t : ts) {
    if (!aligned16(t->ptr) || !strides_ok(*t)) return ATTN_E_LAYOUT;
  }
  const attn_mask& m = a->mask;
  if (m.kind < ATTN_MASK_NONE || m.kind > ATTN_MASK_ADD_F32) return ATTN_E_MASK;
  if (m.kind != ATTN_MASK_NONE) {
    if (!m.ptr) return ATTN_E_MASK;
    if (m.Bm != 1 && m.Bm != a->B) return ATTN_E_MASK;
    if (m.Hm != 1 && m.Hm != a->Hq) return ATTN_E_MASK;
    if (m.stride_b < 0 || m.stride_h < 0 || m.stride_row < 0) return ATTN_E_MASK;
  }
  if (op == ATTN_OP_COMPOSED) {
    if (m.kind != ATTN_MASK_NONE) return ATTN_E_MASK;
    // the softmax pass runs one workgroup of 256 per row
    if ((int64_t)a->B * a->Hq > 65535 || !gqa::grid_fits((int64_t)a->B * a->Hq * a->rows, 256)) return ATTN_E_ARG;
  }
  return ATTN_OK;
}

// Workspace of the composed arm: scores (fp32), weights (16-bit), 1 / l; each part 256-aligned.
struct ComposedLayout {
  int64_t kv_hi, kvp;
  size_t s_bytes, p_bytes, l_bytes;
};

inline size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

ComposedLayout composed_layout(const attn_args* a) {
  ComposedLayout L;
  L.kv_hi = a->causal ? (a->kv_len < a->kv_offset + a->rows ? a->kv_len : a->kv_offset + a->rows) : a->kv_len;
  L.kvp = cdiv(L.kv_hi, kKeysPerTile) * kKeysPerTile;
  const int64_t n = (int64_t)a->B * a->Hq * a->rows;
  L.s_bytes = round256((size_t)n * L.kvp * 4);
  L.p_bytes = round256((size_t)n * L.kvp * 2);
  L.l_bytes = round256((size_t)n * 4);
  return L;
}

int make_plan(const attn_args* a, int op, Plan* P) {
  memset(P, 0, sizeof(*P));
  const int G = a->Hq / a->Hkv;
  P->G = G;
  if (a->head_chunk == 0) {
    P->n_chunks = chunk_rule(a->rows, G, 1, P->chunk_sizes, ATTN_MAX_CHUNKS);
  } else {
    const int c = a->head_chunk;
    P->n_chunks = 0;
    for (int left = G; left > 0; left -= c) P->chunk_sizes[P->n_chunks++] = left < c ? left : c;
  }
  if (P->n_chunks <= 0) return ATTN_E_ARG;
  P->chunk = P->chunk_sizes[0];
  P->blocks_per_chunk = (int)cdiv((int64_t)P->chunk * a->rows, kPairsPerBlock);
  // four wavefronts of one 32-pair column block when they cover the whole KV group (short
  // decode / verify), else eight wavefronts of one block (two per SIMD): with the P.V product one
  // tile behind for prompts, without it (one more tile in flight) for decode / verify rows, whose
  // keys stream from HBM
  const int64_t n_blocks = (int64_t)P->n_chunks * P->blocks_per_chunk;
  P->shape = n_blocks <= 4 ? 0 : op == ATTN_OP_DECODE ? 3 : 2;
  P->waves = P->shape == 0 ? 4 : 8;
  P->n_tiles = (int)cdiv(n_blocks, (int64_t)P->waves);

  // KV splits depend only on the unchunked shape, so every head-chunk choice splits the keys
  // the same way and gives the same bits.
  const int64_t base_tiles = cdiv(cdiv((int64_t)G * a->rows, kPairsPerBlock), kBlocksPerGroup);
  const int64_t kv_hi = a->causal ? (a->kv_len < a->kv_offset + a->rows ? a->kv_len : a->kv_offset + a->rows)
                                  : a->kv_len;
  const int T = gqa::tile_keys(a->D);  // keys per tile of the main pass
  const int64_t n_kt = cdiv(kv_hi, T);
  int64_t S;
  if (a->n_splits == 0) {
    const int64_t base = (int64_t)a->B * a->Hkv * base_tiles;
    // fill the CUs in one round of workgroups: never more than kTargetBlocks, so no second,
    // mostly idle round follows
    const int64_t want = gqa::kTargetBlocks / base;
    const int64_t min_tiles = op == ATTN_OP_DECODE ? 2 : 4;
    int64_t most = n_kt / min_tiles;
    if (most < 1) most = 1;
    S = want < most ? want : most;
    if (S < 1) S = 1;
  } else {
    S = a->n_splits < n_kt ? a->n_splits : n_kt;
  }
  const int64_t tps = cdiv(n_kt, S);
  S = cdiv(n_kt, tps);
  P->n_splits = (int)S;
  P->keys_per_split = (int)(tps * T);
  // Mask window in LDS.  The mask is the same for every head (Hm = 1), spans < 2 GiB, and every
  // workgroup's (head, row) pairs cover few enough mask rows: at most 1024 / T for one dword per
  // key (32 at head dim 256; any row stride and kv_len; the word offsets of the window's rows
  // stay below 2^32), else, on the prompt shape at head dim 256 only, 16-byte row chunks of at
  // most 4 KiB of rows, when rows are 16-byte aligned and end on a whole chunk at kv_len (a chunk
  // that reached past the mask's last word would read as zeros).
  if (a->mask.kind != ATTN_MASK_NONE) {
    const attn_mask& m = a->mask;
    const int64_t esz = m.kind == ATTN_MASK_BOOL_U8 ? 1 : m.kind == ATTN_MASK_ADD ? 2 : 4;
    const int64_t msb = m.Bm == 1 ? 0 : m.stride_b;
    const int64_t span = ((int64_t)(m.Bm - 1) * msb + (int64_t)(a->rows - 1) * m.stride_row + a->kv_len) * esz;
    int64_t window = 0;  // most mask rows any workgroup's pairs cover
    int64_t pair_window = 0;  // most pairs of any workgroup; INT64_MAX when one has two blocks
    const int wg_blocks = P->waves;
    for (int t = 0; t < P->n_tiles; ++t) {
      int64_t lo = INT64_MAX, hi = -1;
      int blocks_with_pairs = 0;
      for (int bj = t * wg_blocks; bj < (t + 1) * wg_blocks; ++bj) {
        const int cj = bj / P->blocks_per_chunk;
        const int64_t f0 = (int64_t)(bj - cj * P->blocks_per_chunk) * kPairsPerBlock;
        const int hs = cj * P->chunk;
        if (hs >= G) continue;
        const int csj = P->chunk < G - hs ? P->chunk : G - hs;
        const int64_t npairs = (int64_t)csj * a->rows;
        if (f0 >= npairs) continue;
        const int64_t last = (f0 + kPairsPerBlock < npairs ? f0 + kPairsPerBlock : npairs) - 1;
        lo = f0 / csj < lo ? f0 / csj : lo;
        hi = last / csj > hi ? last / csj : hi;
        ++blocks_with_pairs;
        if (last - f0 + 1 > pair_window) pair_window = last - f0 + 1;
      }
      if (hi >= 0 && hi - lo + 1 > window) window = hi - lo + 1;
      if (blocks_with_pairs > 1) pair_window = INT64_MAX;
    }
    const bool base = m.Hm == 1 && span < ((int64_t)1 << 31);
    const int64_t word_rows = 1024 / T;
    const bool words = base && window <= word_rows &&
                       ((int64_t)(a->rows + word_rows) * m.stride_row + a->kv_len + T) * esz < ((int64_t)1 << 32);
    const bool rows16 = base && a->D == kHeadDim && P->shape == 2 && ((uintptr_t)m.ptr % 16) == 0 &&
                        (m.stride_row * esz) % 16 == 0 &&
                        (msb * esz) % 16 == 0 && ((int64_t)a->kv_len * esz) % 16 == 0 &&
                        window <= 4096 / (kKeysPerTile * esz);
    // a full-head mask: one dword per key of each pair's own mask row, when every workgroup's
    // pairs form one column block of at most 1024 / T pairs
    const int64_t msh = m.Hm == 1 ? 0 : m.stride_h;
    const int64_t head_span = ((int64_t)(a->Hq - 1) * msh + (int64_t)(a->rows - 1) * m.stride_row + a->kv_len) * esz;
    const bool pair_words = m.Hm == a->Hq && m.Hm > 1 && pair_window <= word_rows &&
                            (int64_t)(m.Bm - 1) * msb * esz + head_span < ((int64_t)1 << 31) &&
                            head_span + T * esz < ((int64_t)1 << 31);
    P->mask_lds = words ? 2 : pair_words ? 3 : rows16 ? 1 : 0;
  }
  P->grid = (int64_t)a->B * a->Hkv * S * P->n_tiles;
  if (P->grid > INT32_MAX || !gqa::grid_fits(P->grid, 64 * P->waves)) return ATTN_E_ARG;
  const int64_t n_rows = (int64_t)a->B * a->Hq * a->rows;
  if (n_rows > (int64_t)INT32_MAX) return ATTN_E_ARG;  // the merge indexes rows in 32 bits
  if (S > 1) {
    const int64_t nrow = S * a->B * a->Hq * (int64_t)a->rows;
    // the kind depends on the unchunked shape only, like the splits
    P->part_kind = nrow * gqa::partial_row_bytes(a->D, 0) >= gqa::kHalfPartialsFromBytes ? 1 : 0;
    if (!gqa::merge_fits((int)S, P->part_kind, n_rows)) return ATTN_E_ARG;
    P->ws_o_bytes = (size_t)cdiv(nrow * gqa::partial_row_bytes(a->D, P->part_kind), 256) * 256;
    P->ws_e_offset = P->ws_o_bytes + (size_t)cdiv(nrow * 4, 256) * 256;
    P->ws_bytes = P->ws_e_offset + (P->part_kind == 1 ? (size_t)cdiv(nrow * 4, 256) * 256 : 0);
  }
  return ATTN_OK;
}

// id = head-dim slot * 128 + mask layout * 32 + shape * 8 + dtype * 4 + mask kind
inline int variant_of(const attn_args* a, const Plan& P) {
  const int dslot = a->D == 256 ? 0 : a->D == 128 ? 1 : 2;
  return dslot * 128 + P.mask_lds * 32 + P.shape * 8 + a->dtype * 4 + a->mask.kind;
}

// Workgroups a call of plan P adds to its main pass's launch for the work it carries (unmasked
// prompt blocks writing fp16 partials that leave CUs idle and run long enough to cover a merge
// the size of their own on those CUs).
inline int carry_blocks_of(const attn_args* a, const Plan& P) {
  if (P.shape != 2 || P.n_splits < 2 || P.part_kind != 1 || a->mask.kind != ATTN_MASK_NONE ||
      P.grid >= gqa::kTargetBlocks)
    return 0;
  const int64_t idle = gqa::kTargetBlocks - P.grid;
  const int64_t tiles = P.keys_per_split / gqa::tile_keys(a->D);
  const int64_t n_rows = (int64_t)a->B * a->Hq * a->rows;
  return n_rows <= gqa::kCarryRowsPerTile * idle * tiles ? (int)idle : 0;
}

// Checks a kv_append call and fills its kernel parameters (kv_append, and an append carried by
// attn_merge).
int append_params(const kv_append_args* a, gqa::AppendParams* pp) {
  if (!a) return ATTN_E_NULL;
  if (a->dtype != ATTN_BF16 && a->dtype != ATTN_F16) return ATTN_E_DTYPE;
  if (a->B <= 0 || a->Hkv <= 0) return ATTN_E_HEADS;
  if (a->D != 64 && a->D != 128 && a->D != ATTN_HEAD_DIM) return ATTN_E_HEAD_DIM;
  if (a->rows < 1) return ATTN_E_ROWS;
  // (the planted late-append build writes one row further: its bound moves with it)
  if (a->kv_offset < 0 || a->capacity < 1 || a->kv_offset + a->rows + (GQA_CONTROL == 3 ? 1 : 0) > a->capacity ||
      a->capacity > INT32_MAX)
    return ATTN_E_KV;
  const attn_tensor* ts[4] = {&a->k_new, &a->v_new, &a->k_cache, &a->v_cache};
  for (const attn_tensor* t : ts)
    if (!t->ptr) return ATTN_E_NULL;
  for (const attn_tensor* t : ts)
    if (!aligned16(t->ptr) || !strides_ok(*t)) return ATTN_E_LAYOUT;
  gqa::AppendParams& p = *pp;
  for (int t = 0; t < 2; ++t) {
    const attn_tensor& s = t ? a->v_new : a->k_new;
    const attn_tensor& d = t ? a->v_cache : a->k_cache;
    p.src[t] = static_cast<const uint16_t*>(s.ptr);
    p.dst[t] = static_cast<uint16_t*>(d.ptr);
    p.s_sb[t] = s.stride_b, p.s_sh[t] = s.stride_h, p.s_sr[t] = s.stride_row;
    p.d_sb[t] = d.stride_b, p.d_sh[t] = d.stride_h, p.d_st[t] = d.stride_row;
  }
  p.B = a->B, p.Hkv = a->Hkv, p.rows = a->rows, p.kv_offset = (int)a->kv_offset;
  p.chunk_shift = a->D == 64 ? 3 : a->D == 128 ? 4 : 5;
  return ATTN_OK;
}

// Checks an attn_merge call and fills its kernel parameters (attn_merge, and a merge carried by
// attn_args carry); no repair inputs.
int merge_params(const merge_args* a, gqa::MergeParams* pp) {
  if (!a) return ATTN_E_NULL;
  if (a->dtype != ATTN_BF16 && a->dtype != ATTN_F16) return ATTN_E_DTYPE;
  if (a->B <= 0 || a->Hq <= 0) return ATTN_E_HEADS;
  if (a->D != ATTN_HEAD_DIM && a->D != 64 && a->D != 128) return ATTN_E_HEAD_DIM;
  if (a->rows < 1) return ATTN_E_ROWS;
  if (a->n_chunks < 1) return ATTN_E_ARG;
  const int64_t n_rows = (int64_t)a->B * a->Hq * a->rows;
  if (a->partial_kind != 0 && a->partial_kind != 1) return ATTN_E_ARG;
  if (n_rows > (int64_t)INT32_MAX || !gqa::merge_fits(a->n_chunks, a->partial_kind, n_rows))
    return ATTN_E_ARG;  // 32-bit rows, launch size
  if (!a->partial_o || !a->partial_lse || !a->gate.ptr || !a->out.ptr) return ATTN_E_NULL;
  if (a->partial_kind == 1 && !a->partial_exp) return ATTN_E_NULL;
  if (!aligned16(a->partial_o) || !aligned16(a->gate.ptr) || !aligned16(a->out.ptr) || !strides_ok(a->gate) ||
      !strides_ok(a->out) || (reinterpret_cast<uintptr_t>(a->partial_lse) & 3u) ||
      (a->partial_kind == 1 && (reinterpret_cast<uintptr_t>(a->partial_exp) & 3u)))
    return ATTN_E_LAYOUT;
  gqa::MergeParams& p = *pp;
  memset(&p, 0, sizeof(p));  // no main-pass inputs: no repair
  p.part_o = a->partial_o;
  p.part_lse = a->partial_lse;
  p.part_e = a->partial_kind == 1 ? a->partial_exp : nullptr;
  p.part_kind = a->partial_kind;
  if (a->append) {  // checked as kv_append checks its arguments; nothing is enqueued on an error
    const int st = append_params(a->append, &p.app);
    if (st) return st;
    if (!gqa::merge_with_append_fits(a->n_chunks, a->partial_kind, n_rows, p.app)) return ATTN_E_ARG;
    p.carry = 1;
  }
  p.gate = static_cast<const uint16_t*>(a->gate.ptr);
  p.out = static_cast<uint16_t*>(a->out.ptr);
  p.g_sb = a->gate.stride_b, p.g_sh = a->gate.stride_h, p.g_sr = a->gate.stride_row;
  p.o_sb = a->out.stride_b, p.o_sh = a->out.stride_h, p.o_sr = a->out.stride_row;
  p.n_chunks = a->n_chunks, p.B = a->B, p.Hq = a->Hq, p.rows = a->rows, p.D = a->D;
  return ATTN_OK;
}

// whether [p, p + n) and [q, q + m) share a byte
inline bool overlaps(const void* p, size_t n, const void* q, size_t m) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
  return n && m && a < b + m && b < a + n;
}

// Checks the merge a call carries (attn_args carry): attn_merge's checks, no append of its own,
// and partials clear of the `used` bytes of the call's workspace, which the call overwrites.
int carry_params(const merge_args* c, const void* ws, size_t used, gqa::MergeParams* cm) {
  const int st = merge_params(c, cm);
  if (st) return st;
  if (c->append) return ATTN_E_ARG;
  const size_t nrow = (size_t)c->n_chunks * c->B * c->Hq * c->rows;
  const size_t obytes = nrow * (size_t)gqa::partial_row_bytes(c->D, c->partial_kind);
  if (overlaps(c->partial_o, obytes, ws, used) || overlaps(c->partial_lse, nrow * 4, ws, used) ||
      (c->partial_kind == 1 && overlaps(c->partial_exp, nrow * 4, ws, used)))
    return ATTN_E_ARG;
  return ATTN_OK;
}

int run_fwd(const attn_args* a, int op, void* ws, size_t ws_bytes, void* stream, bool merge = true,
            int32_t* n_chunks = nullptr, int32_t* part_kind = nullptr, size_t* lse_offset = nullptr,
            size_t* exp_offset = nullptr) {
  int st = validate(a, op);
  if (st) return st;
  Plan P;
  st = make_plan(a, op, &P);
  if (st) return st;
  if (ws_bytes < P.ws_bytes || (P.ws_bytes && !ws)) return ATTN_E_WORKSPACE;
  if (P.ws_bytes && !aligned16(ws)) return ATTN_E_LAYOUT;
  gqa::AppendParams app;  // the append the call carries, if any
  if (a->append) {
    st = append_params(a->append, &app);
    if (st) return st;
    const bool carried = P.n_splits > 1 && merge;
    const int64_t n_rows = (int64_t)a->B * a->Hq * a->rows;
    if (carried && !gqa::merge_with_append_fits(P.n_splits, P.part_kind, n_rows, app)) return ATTN_E_ARG;
  }
  gqa::MergeParams cm;  // the earlier call's merge this call carries, if any
  if (a->carry && (st = carry_params(a->carry, ws, P.ws_bytes, &cm)) != ATTN_OK) return st;
  // Work the main pass's launch carries, on the CUs it leaves idle (prompt blocks writing fp16
  // partials, long enough to cover it): the carried merge when it is an fp16 merge of at most
  // kFewChunks chunks in this call's dtype, and the append of a call that does not merge.
  int extra = 0;
  bool merge_in_launch = false, append_in_launch = false;
  if (const int cb = carry_blocks_of(a, P)) {
    merge_in_launch = a->carry && a->carry->partial_kind == 1 && a->carry->n_chunks <= gqa::kFewChunks &&
                      a->carry->dtype == a->dtype;
    append_in_launch = a->append && !merge;
    if (merge_in_launch || append_in_launch) extra = cb;
  }

  gqa::FwdParams p;
  memset(&p, 0, sizeof(p));
  p.q = static_cast<const uint16_t*>(a->q.ptr);
  p.gate = static_cast<const uint16_t*>(a->gate.ptr);
  p.out = static_cast<uint16_t*>(a->out.ptr);
  p.k = static_cast<const uint16_t*>(a->k_cache.ptr);
  p.v = static_cast<const uint16_t*>(a->v_cache.ptr);
  p.q_sb = a->q.stride_b, p.q_sh = a->q.stride_h, p.q_sr = a->q.stride_row;
  p.g_sb = a->gate.stride_b, p.g_sh = a->gate.stride_h, p.g_sr = a->gate.stride_row;
  p.o_sb = a->out.stride_b, p.o_sh = a->out.stride_h, p.o_sr = a->out.stride_row;
  p.k_sb = a->k_cache.stride_b, p.k_sh = a->k_cache.stride_h, p.k_st = a->k_cache.stride_row;
  p.v_sb = a->v_cache.stride_b, p.v_sh = a->v_cache.stride_h, p.v_st = a->v_cache.stride_row;
  if (a->mask.kind != ATTN_MASK_NONE) {
    p.mask = a->mask.ptr;
    p.m_sb = a->mask.Bm == 1 ? 0 : a->mask.stride_b;  // an extent of 1 broadcasts
    p.m_sh = a->mask.Hm == 1 ? 0 : a->mask.stride_h;
    p.m_sr = a->mask.stride_row;
    p.mask_lds = P.mask_lds == 3 ? 2 : P.mask_lds;  // the word kernels, with per-pair window rows
    p.mask_pairs = P.mask_lds == 3;
  }
  p.kv_offset = (int)a->kv_offset;
  p.kv_len = (int)a->kv_len;
  p.B = a->B, p.Hq = a->Hq, p.Hkv = a->Hkv, p.G = P.G, p.rows = a->rows;
  p.causal = a->causal;
  const float scale = a->scale > 0.0f ? a->scale : 1.0f / sqrtf((float)a->D);
  p.scale_log2 = scale * 1.4426950408889634f;
  p.scale = scale;
  p.chunk = P.chunk;
  p.blocks_per_chunk = P.blocks_per_chunk;
  p.n_tiles = P.n_tiles;
  p.n_splits = P.n_splits;
  p.keys_per_split = P.keys_per_split;
  p.grid = (int)P.grid;
  if (P.n_splits > 1) {
    p.part_o = ws;
    p.part_lse = reinterpret_cast<float*>(static_cast<char*>(ws) + P.ws_o_bytes);
    p.part_e = P.part_kind == 1 ? reinterpret_cast<int32_t*>(static_cast<char*>(ws) + P.ws_e_offset) : nullptr;
    p.part_kind = P.part_kind;
  }
  p.extra_blocks = extra;
  if (merge_in_launch) p.carried = cm;
  if (append_in_launch) {
    p.carried.carry = 1;
    p.carried.app = app;
    p.carried.app_by = 2 * a->B * a->Hkv < extra ? 2 * a->B * a->Hkv : extra;
    p.carried.app_bx = extra / p.carried.app_by;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (a->carry && !merge_in_launch && gqa::launch_merge(cm, a->carry->dtype, s) != hipSuccess) return ATTN_E_HIP;
  if (n_chunks) *n_chunks = P.n_splits;
  if (part_kind) *part_kind = P.n_splits > 1 ? P.part_kind : 0;
  if (lse_offset) *lse_offset = P.n_splits > 1 ? P.ws_o_bytes : 0;
  if (exp_offset) *exp_offset = P.n_splits > 1 && P.part_kind == 1 ? P.ws_e_offset : 0;
  if (gqa::launch_fwd(p, a->D, a->dtype, a->mask.kind, P.shape, s) != hipSuccess) return ATTN_E_HIP;
  if (P.n_splits > 1 && merge) {
    gqa::MergeParams mp;
    memset(&mp, 0, sizeof(mp));
    mp.part_o = p.part_o;
    mp.part_lse = p.part_lse;
    mp.part_e = p.part_e;
    mp.part_kind = p.part_kind;
    mp.gate = p.gate;
    mp.out = p.out;
    mp.g_sb = p.g_sb, mp.g_sh = p.g_sh, mp.g_sr = p.g_sr;
    mp.o_sb = p.o_sb, mp.o_sh = p.o_sh, mp.o_sr = p.o_sr;
    mp.n_chunks = P.n_splits, mp.B = a->B, mp.Hq = a->Hq, mp.rows = a->rows, mp.D = a->D;
    gqa::RepairParams& f = mp.fix;  // the inputs of this main pass, for the merge's repair
    f.q = p.q, f.k = p.k, f.v = p.v, f.mask = p.mask;
    f.q_sb = p.q_sb, f.q_sh = p.q_sh, f.q_sr = p.q_sr;
    f.k_sb = p.k_sb, f.k_sh = p.k_sh, f.k_st = p.k_st;
    f.v_sb = p.v_sb, f.v_sh = p.v_sh, f.v_st = p.v_st;
    f.m_sb = p.m_sb, f.m_sh = p.m_sh, f.m_sr = p.m_sr;
    f.mask_kind = a->mask.kind, f.G = P.G, f.kv_offset = p.kv_offset, f.kv_len = p.kv_len;
    f.causal = p.causal, f.keys_per_split = P.keys_per_split, f.scale_log2 = p.scale_log2;
    if (a->append) {
      mp.carry = 1;
      mp.app = app;
    }
    if (gqa::launch_merge(mp, a->dtype, s) != hipSuccess) return ATTN_E_HIP;
  } else if (a->append && !append_in_launch) {
    if (gqa::launch_append(app, s) != hipSuccess) return ATTN_E_HIP;
  }
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_abi_version(void) { return GQA_ATTN_ABI_VERSION; }

size_t attn_struct_size(int which) {
  switch (which) {
    case 0: return sizeof(attn_args);
    case 1: return sizeof(kv_append_args);
    case 4: return sizeof(kv_keep_args);
    case 2: return sizeof(merge_args);
    case 3: return sizeof(attn_plan_info);
    case 5: return sizeof(attn_prompt_query);
    case 6: return sizeof(attn_prompt_choice);
    default: return 0;
  }
}

const char* attn_strerror(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_E_NULL: return "a required pointer is NULL";
    case ATTN_E_DTYPE: return "unknown dtype";
    case ATTN_E_HEADS: return "invalid head counts (batch, query or KV heads not positive, or not a whole group)";
    case ATTN_E_HEAD_DIM: return "unsupported head_dim (256, 128 or 64; kv_keep takes 256 only)";
    case ATTN_E_ROWS: return "invalid number of query rows";
    case ATTN_E_KV: return "invalid KV offset, length or capacity";
    case ATTN_E_MASK: return "invalid mask (kind, extents, strides or pointer)";
    case ATTN_E_LAYOUT: return "misaligned pointer or stride (16-byte pointers, strides in multiples of 8)";
    case ATTN_E_HEAD_CHUNK: return "head_chunk must be 0 (policy) or 1..group size";
    case ATTN_E_WORKSPACE: return "workspace too small";
    case ATTN_E_HIP: return "HIP runtime error while enqueuing";
    case ATTN_E_ARG: return "invalid argument";
    default: return "unknown status";
  }
}

const char* attn_variant_name(int variant) {
  // id = head-dim slot (256, 128, 64) * 128 + mask layout in LDS * 32 + shape * 8 + dtype * 4 +
  // mask kind (see variant_of); ids of variants that do not exist name "unknown"
  static const std::vector<std::string> names = [] {
    std::vector<std::string> v(3 * 128);
    static const char* const kinds[4] = {"", "_maskbool", "_maskadd", "_maskf32"};
    static const char* const shapes[4] = {"_4x1", "", "_8x1", "_8x1_stream"};
    static const char* const layouts[4] = {"", "_ldsrows", "_ldswords", "_ldspairwords"};
    static const char* const dims[3] = {"", "_d128", "_d64"};
    for (int id = 0; id < 3 * 128; ++id) {
      const int dslot = id / 128, r = id % 128, ml = r / 32, shape = (r / 8) % 4, dtype = (r / 4) % 2, kind = r % 4;
      if (shape == 1 || (ml != 0 && kind == 0) || (ml == 1 && (shape != 2 || dslot != 0))) continue;
      v[id] = std::string("fwd_mfma32x32x16_") + (dtype ? "f16" : "bf16") + kinds[kind] + shapes[shape] + layouts[ml] +
              dims[dslot];
    }
    return v;
  }();
  if (variant < 0 || variant >= (int)names.size() || names[variant].empty()) return "unknown";
  return names[variant].c_str();
}

int attn_head_chunk_plan(int rows, int n_q_heads, int n_kv_heads, int enabled, int* sizes, int cap, int* n_chunks) {
  if (!sizes || !n_chunks) return ATTN_E_NULL;
  if (rows < 1) return ATTN_E_ROWS;
  if (n_q_heads <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads != 0) return ATTN_E_HEADS;
  const int n = chunk_rule(rows, n_q_heads / n_kv_heads, enabled, sizes, cap);
  if (n < 0) return ATTN_E_ARG;
  *n_chunks = n;
  return ATTN_OK;
}

int attn_prompt_policy(const attn_prompt_query* q, attn_prompt_choice* out) {
  if (!q || !out) return ATTN_E_NULL;
  if (q->D != 256 && q->D != 128 && q->D != 64) return ATTN_E_HEAD_DIM;
  if (q->B < 1 || q->Hq < 1 || q->Hkv < 1 || q->Hq % q->Hkv != 0) return ATTN_E_HEADS;
  if (q->n_tokens < 1) return ATTN_E_ROWS;
  if (q->dtype != ATTN_BF16 && q->dtype != ATTN_F16) return ATTN_E_DTYPE;
  // Fastest fused block size on gfx950 with 256 compute units, per head dim and group size
  // (measured at G = 6 and G = 8 for prompts up to and beyond 8192 rows; the composed route
  // never won).  Rows of {head dim, largest G, block rows}.
  struct Row {
    int D, g_max, q_block;
  };
  static const Row kTable[] = {
      {256, 6, 8192}, {256, 1 << 30, 4096}, {128, 6, 8192}, {128, 1 << 30, 4096},
      {64, 6, 8192},  {64, 1 << 30, 4096},
  };
  constexpr int64_t kWhole = 2048;  // up to this many rows the whole prompt is one call
  const int G = q->Hq / q->Hkv;
  out->route = ATTN_OP_PREFILL;
  out->qualified = (q->gfx == 950 && q->n_cus == 256) ? 1 : 0;
  int64_t qb;
  if (!out->qualified) {
    qb = 512;
    out->reason = ATTN_POLICY_DEFAULT;
  } else if (q->n_tokens <= kWhole) {
    qb = q->n_tokens;
    out->reason = ATTN_POLICY_WHOLE;
  } else {
    qb = 512;
    for (const Row& r : kTable) {
      if (r.D == q->D && G <= r.g_max) {
        qb = r.q_block;
        break;
      }
    }
    // the table holds at batch 1: keep the rows of a block times the batch
    qb = std::max<int64_t>(512, qb / q->B);
    out->reason = ATTN_POLICY_TABLE;
  }
  qb = std::min<int64_t>(qb, q->n_tokens);
  out->q_block = (int32_t)qb;
  out->n_calls = (q->n_tokens + qb - 1) / qb;
  return ATTN_OK;
}

int attn_workspace_bytes(const attn_args* a, int op, size_t* bytes) {
  if (!bytes) return ATTN_E_NULL;
  int st = validate(a, op);
  if (st) return st;
  if (op == ATTN_OP_COMPOSED) {
    const ComposedLayout L = composed_layout(a);
    *bytes = L.s_bytes + L.p_bytes + L.l_bytes;
    return ATTN_OK;
  }
  Plan P;
  st = make_plan(a, op, &P);
  if (st) return st;
  *bytes = P.ws_bytes;
  return ATTN_OK;
}

int attn_describe_plan(const attn_args* a, int op, attn_plan_info* info) {
  if (!info) return ATTN_E_NULL;
  if (op == ATTN_OP_COMPOSED) return ATTN_E_ARG;
  int st = validate(a, op);
  if (st) return st;
  Plan P;
  st = make_plan(a, op, &P);
  if (st) return st;
  memset(info, 0, sizeof(*info));
  info->op = op;
  info->variant = variant_of(a, P);
  info->group_size = P.G;
  info->n_head_chunks = P.n_chunks;
  info->head_chunk = P.chunk;
  info->rows_per_wave = kPairsPerBlock;
  info->waves_per_block = P.waves;
  info->n_row_tiles = P.n_tiles;
  info->n_splits = P.n_splits;
  info->keys_per_split = P.keys_per_split;
  info->keys_per_tile = gqa::tile_keys(a->D);
  info->lds_bytes = gqa::kFwdLdsBytes + (P.mask_lds ? gqa::kStages * gqa::kMaskStageLds : 0);
  info->grid_blocks = P.grid;
  info->partial_kind = P.n_splits > 1 ? P.part_kind : 0;
  info->carry_blocks = carry_blocks_of(a, P);
  info->workspace_bytes = (int64_t)P.ws_bytes;
  for (int i = 0; i < P.n_chunks; ++i) info->chunk_sizes[i] = P.chunk_sizes[i];
  return ATTN_OK;
}

int attn_prefill(const attn_args* a, void* workspace, size_t ws_bytes, void* stream) {
  return run_fwd(a, ATTN_OP_PREFILL, workspace, ws_bytes, stream);
}

int attn_prefill_partials(const attn_args* a, void* workspace, size_t ws_bytes, void* stream, int32_t* n_chunks,
                          int32_t* partial_kind, size_t* lse_offset, size_t* exp_offset) {
  if (!n_chunks || !partial_kind || !lse_offset || !exp_offset) return ATTN_E_NULL;
  return run_fwd(a, ATTN_OP_PREFILL, workspace, ws_bytes, stream, false, n_chunks, partial_kind, lse_offset,
                 exp_offset);
}

int attn_decode(const attn_args* a, void* workspace, size_t ws_bytes, void* stream) {
  return run_fwd(a, ATTN_OP_DECODE, workspace, ws_bytes, stream);
}

int attn_decode_noalloc(const attn_args* a, void* stream) {
  int st = validate(a, ATTN_OP_DECODE);
  if (st) return st;
  size_t need = 0;
  st = attn_workspace_bytes(a, ATTN_OP_DECODE, &need);
  if (st) return st;
  if (need > gqa::kScratchBytes) return ATTN_E_WORKSPACE;  // the partials do not fit the scratch
  void* ws = nullptr;
  if (need > 0 && gqa::scratch_of_current_device(&ws) != hipSuccess) return ATTN_E_HIP;
  return run_fwd(a, ATTN_OP_DECODE, ws, need > 0 ? gqa::kScratchBytes : 0, stream);
}

int attn_prefill_composed(const attn_args* a, void* workspace, size_t ws_bytes, void* stream) {
  int st = validate(a, ATTN_OP_COMPOSED);
  if (st) return st;
  const ComposedLayout L = composed_layout(a);
  if (!workspace || ws_bytes < L.s_bytes + L.p_bytes + L.l_bytes) return ATTN_E_WORKSPACE;
  if (!aligned16(workspace)) return ATTN_E_LAYOUT;
  gqa::AppendParams app;  // the append the call carries: a launch of its own after the route's
  if (a->append && (st = append_params(a->append, &app)) != ATTN_OK) return st;
  gqa::MergeParams cm;  // the merge the call carries: a launch of its own ahead of the route's
  if (a->carry && (st = carry_params(a->carry, workspace, L.s_bytes + L.p_bytes + L.l_bytes, &cm)) != ATTN_OK)
    return st;
  gqa::ComposedParams p;
  memset(&p, 0, sizeof(p));
  p.q = static_cast<const uint16_t*>(a->q.ptr);
  p.k = static_cast<const uint16_t*>(a->k_cache.ptr);
  p.v = static_cast<const uint16_t*>(a->v_cache.ptr);
  p.gate = static_cast<const uint16_t*>(a->gate.ptr);
  p.out = static_cast<uint16_t*>(a->out.ptr);
  p.q_sb = a->q.stride_b, p.q_sh = a->q.stride_h, p.q_sr = a->q.stride_row;
  p.k_sb = a->k_cache.stride_b, p.k_sh = a->k_cache.stride_h, p.k_st = a->k_cache.stride_row;
  p.v_sb = a->v_cache.stride_b, p.v_sh = a->v_cache.stride_h, p.v_st = a->v_cache.stride_row;
  p.g_sb = a->gate.stride_b, p.g_sh = a->gate.stride_h, p.g_sr = a->gate.stride_row;
  p.o_sb = a->out.stride_b, p.o_sh = a->out.stride_h, p.o_sr = a->out.stride_row;
  char* ws = static_cast<char*>(workspace);
  p.s = reinterpret_cast<float*>(ws);
  p.pw = reinterpret_cast<uint16_t*>(ws + L.s_bytes);
  p.inv_l = reinterpret_cast<float*>(ws + L.s_bytes + L.p_bytes);
  p.kvp = L.kvp;
  p.D = a->D;
  p.B = a->B, p.Hq = a->Hq, p.G = a->Hq / a->Hkv, p.rows = a->rows;
  p.kv_offset = (int)a->kv_offset, p.kv_len = (int)a->kv_len, p.causal = a->causal, p.kv_hi = (int)L.kv_hi;
  const float scale = a->scale > 0.0f ? a->scale : 1.0f / sqrtf((float)a->D);
  p.scale_log2 = scale * 1.4426950408889634f;
  if (a->carry && gqa::launch_merge(cm, a->carry->dtype, static_cast<hipStream_t>(stream)) != hipSuccess)
    return ATTN_E_HIP;
  if (gqa::launch_composed(p, a->dtype, static_cast<hipStream_t>(stream)) != hipSuccess) return ATTN_E_HIP;
  if (a->append && gqa::launch_append(app, static_cast<hipStream_t>(stream)) != hipSuccess) return ATTN_E_HIP;
  return ATTN_OK;
}

int kv_append(const kv_append_args* a, void* stream) {
  gqa::AppendParams p;
  const int st = append_params(a, &p);
  if (st) return st;
  if (gqa::launch_append(p, static_cast<hipStream_t>(stream)) != hipSuccess) return ATTN_E_HIP;
  return ATTN_OK;
}

int kv_keep(const kv_keep_args* a, void* stream) {
  if (!a || !a->keep) return ATTN_E_NULL;
  if (a->dtype != ATTN_BF16 && a->dtype != ATTN_F16) return ATTN_E_DTYPE;
  if (a->B <= 0 || a->B > gqa::kKeepMaxBatch || a->Hkv <= 0) return ATTN_E_HEADS;
  if (!gqa::grid_fits((int64_t)a->B * a->Hkv, 256)) return ATTN_E_HEADS;  // one workgroup of 256 per (b, g)
  if (a->D != ATTN_HEAD_DIM) return ATTN_E_HEAD_DIM;
  if (a->rows < 1 || a->rows > ATTN_MAX_DECODE_ROWS) return ATTN_E_ROWS;
  if (a->kv_offset < 0 || a->capacity < 1 || a->kv_offset + a->rows > a->capacity || a->capacity > INT32_MAX)
    return ATTN_E_KV;
  for (int b = 0; b < a->B; ++b)
    if (a->rows < 32 && (a->keep[b] >> a->rows) != 0u) return ATTN_E_ARG;
  if (!a->k_cache.ptr || !a->v_cache.ptr) return ATTN_E_NULL;
  if (!aligned16(a->k_cache.ptr) || !aligned16(a->v_cache.ptr) || !strides_ok(a->k_cache) || !strides_ok(a->v_cache))
    return ATTN_E_LAYOUT;
  gqa::KeepParams p;
  memset(&p, 0, sizeof(p));
  for (int t = 0; t < 2; ++t) {
    const attn_tensor& c = t ? a->v_cache : a->k_cache;
    p.cache[t] = static_cast<uint16_t*>(c.ptr);
    p.c_sb[t] = c.stride_b, p.c_sh[t] = c.stride_h, p.c_st[t] = c.stride_row;
  }
  p.Hkv = a->Hkv, p.rows = a->rows, p.kv_offset = (int)a->kv_offset;
  for (int b = 0; b < a->B; ++b) p.keep[b] = a->keep[b];
  if (gqa::launch_keep(p, a->B, static_cast<hipStream_t>(stream)) != hipSuccess) return ATTN_E_HIP;
  return ATTN_OK;
}

int attn_merge(const merge_args* a, void* stream) {
  gqa::MergeParams p;
  const int st = merge_params(a, &p);
  if (st) return st;
  if (gqa::launch_merge(p, a->dtype, static_cast<hipStream_t>(stream)) != hipSuccess) return ATTN_E_HIP;
  return ATTN_OK;
}

}  // extern "C"
