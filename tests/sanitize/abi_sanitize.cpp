// Host-side check of libgqa_attn's C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// Built with g++ from attn_api.cpp (the whole host library: validation, plans, workspace
// sizing, launch parameters) and this file, whose stub launchers stand in for the HIP kernels:
// they launch nothing and touch no memory, they count the launches and check the parameters
// each call hands to them against the plan that attn_describe_plan reports.  The driver runs
//   - the rejection matrix: every invalid call returns its status and reaches no launcher;
//   - launch-size limits: shapes whose main pass or merge would not fit a launch are rejected
//     by the planning calls and by the run alike, before anything is enqueued;
//   - a sweep of valid plans (head shapes, rows, offsets, head dims, head chunks, splits, masks)
//     through attn_workspace_bytes, attn_describe_plan, attn_prefill / attn_decode /
//     attn_prefill_partials and the composed route;
//   - kv_append, kv_keep and attn_merge, valid and invalid.
// Device pointers are placeholders (aligned, never dereferenced).  Exit status 0: every check held.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "attn_internal.h"
#include "gqa_attn.h"

namespace {

int g_fail = 0;
long g_checks = 0;
long g_launch_fwd = 0, g_launch_merge = 0, g_launch_other = 0;
gqa::FwdParams g_fwd;
gqa::MergeParams g_merge;
int g_fwd_shape = -1;

#define CHECK(cond, ...)                                       \
  do {                                                         \
    ++g_checks;                                                \
    if (!(cond)) {                                             \
      ++g_fail;                                                \
      fprintf(stderr, "FAIL %s:%d: %s: ", __FILE__, __LINE__, #cond); \
      fprintf(stderr, __VA_ARGS__);                            \
      fprintf(stderr, "\n");                                   \
    }                                                          \
  } while (0)

long launches() { return g_launch_fwd + g_launch_merge + g_launch_other; }

char* const kDev = reinterpret_cast<char*>(uintptr_t(1) << 32);  // aligned placeholder, never read

attn_tensor t4(int64_t H, int64_t rows, int64_t D, size_t slot) {
  attn_tensor t;
  t.ptr = kDev + (slot << 36);
  t.stride_row = D;
  t.stride_h = rows * D;
  t.stride_b = H * rows * D;
  return t;
}

attn_args args(int B, int Hq, int Hkv, int rows, int64_t off, int D = 256) {
  attn_args a;
  memset(&a, 0, sizeof(a));
  a.dtype = ATTN_BF16;
  a.B = B, a.Hq = Hq, a.Hkv = Hkv, a.D = D, a.rows = rows;
  a.kv_offset = off, a.kv_len = off + rows, a.capacity = off + rows;
  a.causal = 1;
  a.q = t4(Hq, rows, D, 1);
  a.gate = t4(Hq, rows, D, 2);
  a.out = t4(Hq, rows, D, 3);
  a.k_cache = t4(Hkv, a.capacity, D, 4);
  a.v_cache = t4(Hkv, a.capacity, D, 5);
  a.mask.kind = ATTN_MASK_NONE;
  a.mask.Bm = a.mask.Hm = 1;
  return a;
}

void* const kStream = nullptr;
char* const kWs = kDev + (uintptr_t(6) << 36);

}  // namespace

// ---- stub launchers: record and check, never touch memory
namespace gqa {

hipError_t launch_fwd_any(const FwdParams& p, int dtype, int mask_kind, int shape) {
  ++g_launch_fwd;
  g_fwd = p;
  g_fwd_shape = shape;
  CHECK(dtype == 0 || dtype == 1, "dtype %d", dtype);
  CHECK(mask_kind >= 0 && mask_kind <= 3, "mask kind %d", mask_kind);
  CHECK(shape == 0 || shape == 2 || shape == 3, "shape %d", shape);
  CHECK(p.mask_lds >= 0 && p.mask_lds <= 2 && (p.mask_lds != 1 || shape == 2) && (mask_kind != 0 || p.mask_lds == 0),
        "mask layout %d on shape %d", p.mask_lds, shape);
  CHECK(p.grid == (int64_t)p.B * p.Hkv * p.n_splits * p.n_tiles, "grid %d", p.grid);
  CHECK(p.keys_per_split % 32 == 0, "keys_per_split %d", p.keys_per_split);
  CHECK((p.n_splits > 1) == (p.part_o != nullptr), "partials %d", p.n_splits);
  CHECK(p.G * p.Hkv == p.Hq && p.chunk >= 1 && p.chunk <= p.G, "chunk %d", p.chunk);
  // carried work: only on the lagged shape writing fp16 partials, and only on CUs left idle
  CHECK(p.extra_blocks == 0 || (shape == 2 && p.n_splits > 1 && p.part_kind == 1 &&
                                p.grid + p.extra_blocks == kTargetBlocks),
        "extra blocks %d on shape %d, grid %d", p.extra_blocks, shape, p.grid);
  CHECK(p.extra_blocks > 0 || (p.carried.n_chunks == 0 && p.carried.carry == 0), "carried work without blocks");
  CHECK(p.carried.n_chunks == 0 || (p.carried.part_kind == 1 && p.carried.n_chunks <= kFewChunks &&
                                    p.carried.part_e && !p.carried.fix.q),
        "carried merge %d chunks kind %d", p.carried.n_chunks, p.carried.part_kind);
  CHECK(!p.carried.carry || (p.carried.app_bx >= 1 && p.carried.app_by >= 1 &&
                             p.carried.app_bx * p.carried.app_by <= p.extra_blocks),
        "carried append grid %d x %d", p.carried.app_bx, p.carried.app_by);
  return hipSuccess;
}

hipError_t launch_fwd_256(const FwdParams& p, int dtype, int mask_kind, int shape, hipStream_t) {
  return launch_fwd_any(p, dtype, mask_kind, shape);
}
hipError_t launch_fwd_128(const FwdParams& p, int dtype, int mask_kind, int shape, hipStream_t) {
  return launch_fwd_any(p, dtype, mask_kind, shape);
}
hipError_t launch_fwd_64(const FwdParams& p, int dtype, int mask_kind, int shape, hipStream_t) {
  return launch_fwd_any(p, dtype, mask_kind, shape);
}

hipError_t launch_merge(const MergeParams& p, int dtype, hipStream_t) {
  ++g_launch_merge;
  g_merge = p;
  CHECK(dtype == 0 || dtype == 1, "dtype %d", dtype);
  CHECK(p.n_chunks >= 1, "n_chunks %d", p.n_chunks);
  CHECK(merge_fits(p.n_chunks, p.part_kind, (int64_t)p.B * p.Hq * p.rows), "merge shape");
  CHECK(!p.carry || merge_with_append_fits(p.n_chunks, p.part_kind, (int64_t)p.B * p.Hq * p.rows, p.app),
        "merge + append shape");
  CHECK(p.D == 256 || p.D == 128 || p.D == 64, "D %d", p.D);
  return hipSuccess;
}

hipError_t launch_append(const AppendParams& p, hipStream_t) {
  ++g_launch_other;
  CHECK(p.chunk_shift >= 3 && p.chunk_shift <= 5, "chunk_shift %d", p.chunk_shift);
  return hipSuccess;
}

hipError_t launch_keep(const KeepParams& p, int B, hipStream_t) {
  ++g_launch_other;
  CHECK(B >= 1 && B <= kKeepMaxBatch && p.rows >= 1 && p.rows <= 32, "keep B %d rows %d", B, p.rows);
  return hipSuccess;
}

hipError_t launch_composed(const ComposedParams& p, int, hipStream_t) {
  ++g_launch_other;
  CHECK(p.kvp % 32 == 0 && p.kvp >= p.kv_hi, "kvp %lld", (long long)p.kvp);
  return hipSuccess;
}

hipError_t scratch_of_current_device(void** ptr) {
  *ptr = kWs;
  return hipSuccess;
}


}  // namespace gqa

namespace {

// A call that must be rejected with `want` and must launch nothing.
void expect_reject(const char* what, attn_args a, int want) {
  for (int op = ATTN_OP_PREFILL; op <= ATTN_OP_COMPOSED; ++op) {
    const long before = launches();
    size_t bytes = 0;
    const int w = attn_workspace_bytes(&a, op, &bytes);
    const int r = op == ATTN_OP_PREFILL ? attn_prefill(&a, kWs, SIZE_MAX / 2, kStream)
                  : op == ATTN_OP_DECODE ? attn_decode(&a, kWs, SIZE_MAX / 2, kStream)
                                         : attn_prefill_composed(&a, kWs, SIZE_MAX / 2, kStream);
    CHECK(w == want && r == want, "%s (op %d): workspace %d, call %d, want %d", what, op, w, r, want);
    CHECK(launches() == before, "%s (op %d) launched", what, op);
    if (op != ATTN_OP_COMPOSED) {
      attn_plan_info info;
      CHECK(attn_describe_plan(&a, op, &info) == want, "%s (op %d) describe", what, op);
    }
  }
}

void rejection_matrix() {
  expect_reject("dtype", [] { auto a = args(1, 24, 4, 4, 100); a.dtype = 7; return a; }(), ATTN_E_DTYPE);
  expect_reject("zero kv heads", args(1, 24, 0, 4, 100), ATTN_E_HEADS);
  expect_reject("zero q heads", args(1, 0, 4, 4, 100), ATTN_E_HEADS);
  expect_reject("uneven groups", args(1, 10, 4, 4, 100), ATTN_E_HEADS);
  expect_reject("batch 0", args(0, 24, 4, 4, 100), ATTN_E_HEADS);
  expect_reject("group over 64", args(1, 130, 2, 4, 100), ATTN_E_HEADS);
  expect_reject("head dim 96", args(1, 24, 4, 4, 100, 96), ATTN_E_HEAD_DIM);
  expect_reject("rows 0", args(1, 24, 4, 0, 100), ATTN_E_ROWS);
  expect_reject("negative offset", [] { auto a = args(1, 24, 4, 4, 100); a.kv_offset = -1; return a; }(), ATTN_E_KV);
  expect_reject("kv_len short", [] { auto a = args(1, 24, 4, 4, 100); a.kv_len = 102; return a; }(), ATTN_E_KV);
  expect_reject("kv_len > capacity", [] { auto a = args(1, 24, 4, 4, 100); a.kv_len = 105; return a; }(), ATTN_E_KV);
  expect_reject("kv_len 0", [] { auto a = args(1, 24, 4, 4, 100); a.kv_len = 0; return a; }(), ATTN_E_KV);
  expect_reject("kv past int32", [] { auto a = args(1, 24, 4, 4, 100); a.kv_len = a.capacity = 1LL << 33; return a; }(),
                ATTN_E_KV);
  expect_reject("head_chunk > G", [] { auto a = args(1, 24, 4, 4, 100); a.head_chunk = 7; return a; }(),
                ATTN_E_HEAD_CHUNK);
  expect_reject("head_chunk < 0", [] { auto a = args(1, 24, 4, 4, 100); a.head_chunk = -1; return a; }(),
                ATTN_E_HEAD_CHUNK);
  expect_reject("negative splits", [] { auto a = args(1, 24, 4, 4, 100); a.n_splits = -2; return a; }(), ATTN_E_ARG);
  expect_reject("nan scale", [] { auto a = args(1, 24, 4, 4, 100); a.scale = NAN; return a; }(), ATTN_E_ARG);
  expect_reject("inf scale", [] { auto a = args(1, 24, 4, 4, 100); a.scale = INFINITY; return a; }(), ATTN_E_ARG);
  expect_reject("causal 2", [] { auto a = args(1, 24, 4, 4, 100); a.causal = 2; return a; }(), ATTN_E_ARG);
  expect_reject("null q", [] { auto a = args(1, 24, 4, 4, 100); a.q.ptr = nullptr; return a; }(), ATTN_E_NULL);
  expect_reject("null v", [] { auto a = args(1, 24, 4, 4, 100); a.v_cache.ptr = nullptr; return a; }(), ATTN_E_NULL);
  expect_reject("misaligned q", [] { auto a = args(1, 24, 4, 4, 100); a.q.ptr = kDev + 8; return a; }(),
                ATTN_E_LAYOUT);
  expect_reject("odd row stride", [] { auto a = args(1, 24, 4, 4, 100); a.k_cache.stride_row = 260; return a; }(),
                ATTN_E_LAYOUT);
  expect_reject("mask kind", [] { auto a = args(1, 24, 4, 4, 100); a.mask.kind = 9; return a; }(), ATTN_E_MASK);
  expect_reject("mask null", [] { auto a = args(1, 24, 4, 4, 100); a.mask.kind = 1; return a; }(), ATTN_E_MASK);
  expect_reject("mask batch extent", [] {
    auto a = args(1, 24, 4, 4, 100);
    a.mask.kind = 1, a.mask.ptr = kDev, a.mask.Bm = 2;
    return a;
  }(), ATTN_E_MASK);
  expect_reject("mask head extent", [] {
    auto a = args(1, 24, 4, 4, 100);
    a.mask.kind = 2, a.mask.ptr = kDev, a.mask.Hm = 6;
    return a;
  }(), ATTN_E_MASK);
  expect_reject("negative mask stride", [] {
    auto a = args(1, 24, 4, 4, 100);
    a.mask.kind = 2, a.mask.ptr = kDev, a.mask.stride_row = -8;
    return a;
  }(), ATTN_E_MASK);
  // null argument structs
  size_t bytes;
  attn_plan_info info;
  CHECK(attn_workspace_bytes(nullptr, 0, &bytes) == ATTN_E_NULL, "null args");
  CHECK(attn_describe_plan(nullptr, 0, &info) == ATTN_E_NULL, "null args");
  CHECK(attn_prefill(nullptr, nullptr, 0, kStream) == ATTN_E_NULL, "null args");
  CHECK(attn_decode(nullptr, nullptr, 0, kStream) == ATTN_E_NULL, "null args");
  auto a = args(1, 24, 4, 4, 100);
  CHECK(attn_workspace_bytes(&a, 7, &bytes) == ATTN_E_ARG, "bad op");
  CHECK(attn_workspace_bytes(&a, 0, nullptr) == ATTN_E_NULL, "null bytes");
  // decode takes 1..32 rows, prefill any
  auto d = args(1, 16, 2, 33, 4096);
  CHECK(attn_decode(&d, kWs, SIZE_MAX / 2, kStream) == ATTN_E_ROWS, "decode rows 33");
  // a too-small workspace is rejected before anything is enqueued
  auto w = args(2, 16, 2, 1, 32768);
  CHECK(attn_workspace_bytes(&w, ATTN_OP_DECODE, &bytes) == ATTN_OK && bytes > 0, "decode ws");
  const long before = launches();
  CHECK(attn_decode(&w, kWs, bytes - 1, kStream) == ATTN_E_WORKSPACE, "small ws");
  CHECK(attn_decode(&w, nullptr, bytes, kStream) == ATTN_E_WORKSPACE, "null ws");
  CHECK(launches() == before, "rejected calls launched");
}

// Shapes whose launches would not fit are rejected by planning and run alike, before any launch.
void launch_limits() {
  // decode rows 32 at B 4096, 32/1 heads over a 4128-key cache, 100 splits asked (65 planned, more
  // than the one-wavefront merge's 64 slots): the merge would run 4.19M rows x 1024 threads
  auto a = args(4096, 32, 1, 32, 4096);
  a.n_splits = 100;
  size_t bytes = 0;
  attn_plan_info info;
  const long before = launches();
  CHECK(attn_workspace_bytes(&a, ATTN_OP_DECODE, &bytes) == ATTN_E_ARG, "merge too large: workspace");
  CHECK(attn_describe_plan(&a, ATTN_OP_DECODE, &info) == ATTN_E_ARG, "merge too large: describe");
  CHECK(attn_decode(&a, kWs, SIZE_MAX / 2, kStream) == ATTN_E_ARG, "merge too large: run");
  // fewer splits fit (one wavefront per row for <= 64 chunks of fp16 partials)
  a.n_splits = 8;
  CHECK(attn_workspace_bytes(&a, ATTN_OP_DECODE, &bytes) == ATTN_OK, "8 splits fit");
  a.n_splits = 40;
  CHECK(attn_workspace_bytes(&a, ATTN_OP_DECODE, &bytes) == ATTN_OK, "33 splits fit");
  // head dim 64 (128-key tiles): the same merge limit (100 splits asked, 65 planned)
  auto s64 = args(4096, 32, 1, 32, 8192, 64);
  s64.n_splits = 100;
  CHECK(attn_workspace_bytes(&s64, ATTN_OP_DECODE, &bytes) == ATTN_E_ARG, "head dim 64 merge too large: workspace");
  CHECK(attn_decode(&s64, kWs, SIZE_MAX / 2, kStream) == ATTN_E_ARG, "head dim 64 merge too large: run");
  s64.n_splits = 8;
  CHECK(attn_workspace_bytes(&s64, ATTN_OP_DECODE, &bytes) == ATTN_OK, "head dim 64, 8 splits fit");
  // the merge called on its own
  merge_args m;
  memset(&m, 0, sizeof(m));
  m.dtype = 0, m.n_chunks = 40, m.B = 4096, m.Hq = 32, m.rows = 32, m.D = 256;
  m.partial_o = reinterpret_cast<const float*>(kWs), m.partial_lse = reinterpret_cast<const float*>(kWs);
  m.gate = t4(32, 32, 256, 2), m.out = t4(32, 32, 256, 3);
  CHECK(attn_merge(&m, kStream) == ATTN_E_ARG, "merge alone too large");
  // the composed route's softmax pass (one workgroup of 256 per row)
  auto c = args(1, 64, 8, 300000, 0);
  CHECK(attn_prefill_composed(&c, kWs, SIZE_MAX / 2, kStream) == ATTN_E_ARG, "composed too large");
  CHECK(launches() == before, "a rejected launch-size case launched");
}

// Valid calls: planning and run agree, and the launched parameters match the described plan.
void sweep() {
  const int heads[][2] = {{24, 4}, {16, 2}, {8, 8}, {6, 1}, {12, 2}, {64, 1}, {2, 2}};
  const int rows_list[] = {1, 2, 4, 5, 6, 9, 17, 32, 33, 48, 128, 300, 512};
  const int64_t offs[] = {0, 1, 63, 4096, 4097, 32768};
  for (const auto& hh : heads) {
    for (int rows : rows_list) {
      for (int64_t off : offs) {
        for (int D : {256, 128, 64}) {
          for (int B : {1, 2}) {
            for (int n_splits : {0, 1, 3, 70}) {
              for (int op : {ATTN_OP_PREFILL, ATTN_OP_DECODE}) {
                if (op == ATTN_OP_DECODE && rows > 32) continue;
                auto a = args(B, hh[0], hh[1], rows, off, D);
                a.n_splits = n_splits;
                size_t bytes = 0;
                attn_plan_info info;
                const int w = attn_workspace_bytes(&a, op, &bytes);
                const int d = attn_describe_plan(&a, op, &info);
                CHECK(w == ATTN_OK && d == ATTN_OK, "valid shape rejected: %d %d (B %d Hq %d rows %d off %lld D %d)", w,
                      d, B, hh[0], rows, (long long)off, D);
                if (w || d) continue;
                CHECK((int64_t)bytes == info.workspace_bytes, "workspace mismatch");
                CHECK(info.n_splits >= 1 && (int64_t)info.n_splits * info.keys_per_split >= off + rows,
                      "splits do not cover the keys");
                CHECK((int64_t)(info.n_splits - 1) * info.keys_per_split < off + rows, "an empty split");
                const long f0 = g_launch_fwd, m0 = g_launch_merge, o0 = g_launch_other;
                const int r = op == ATTN_OP_PREFILL ? attn_prefill(&a, kWs, bytes, kStream)
                                                    : attn_decode(&a, kWs, bytes, kStream);
                CHECK(r == ATTN_OK, "run %d", r);
                const bool split = info.n_splits > 1;
                CHECK(g_launch_fwd == f0 + 1 && g_launch_merge == m0 + (split ? 1 : 0) && g_launch_other == o0,
                      "launch count");
                CHECK(g_fwd.grid == info.grid_blocks && g_fwd.n_splits == info.n_splits &&
                          g_fwd.keys_per_split == info.keys_per_split && g_fwd.n_tiles == info.n_row_tiles,
                      "launched plan differs from the described one");
                CHECK(g_fwd.keys_per_split % info.keys_per_tile == 0 && info.keys_per_tile == 8192 / D,
                      "tile keys %d at head dim %d", info.keys_per_tile, D);
                CHECK((g_fwd_shape == 0 ? 4 : 8) == info.waves_per_block, "shape");
                CHECK(g_fwd_shape != 3 || op == ATTN_OP_DECODE, "the streaming shape is for decode rows");
                if (split) {
                  const size_t nrow = (size_t)info.n_splits * B * hh[0] * rows;
                  const char* o = reinterpret_cast<const char*>(g_fwd.part_o);
                  const char* lse = reinterpret_cast<const char*>(g_fwd.part_lse);
                  const char* ex = reinterpret_cast<const char*>(g_fwd.part_e);
                  const int kind = g_fwd.part_kind;
                  CHECK(kind == (nrow * 4 * D >= (8u << 20) ? 1 : 0), "partial kind");
                  CHECK(o == kWs && lse >= o + (kind ? 2 : 4) * D * nrow &&
                            (kind ? ex >= lse + 4 * nrow && ex + 4 * nrow <= kWs + bytes
                                  : !ex && lse + 4 * nrow <= kWs + bytes),
                        "partials outside the workspace or overlapping");
                  CHECK(g_merge.n_chunks == info.n_splits && g_merge.D == D && g_merge.part_kind == kind &&
                            g_merge.part_o == g_fwd.part_o && g_merge.part_lse == g_fwd.part_lse &&
                            g_merge.part_e == g_fwd.part_e,
                        "merge chunks / head dim / partials");
                }
                if (op == ATTN_OP_PREFILL) {
                  int32_t n = 0, kind = -1;
                  size_t lse_off = 0, exp_off = 0;
                  const long m1 = g_launch_merge;
                  CHECK(attn_prefill_partials(&a, kWs, bytes, kStream, &n, &kind, &lse_off, &exp_off) == ATTN_OK,
                        "partials");
                  CHECK(n == info.n_splits && g_launch_merge == m1, "partials: chunks or a merge");
                  CHECK(!split || (kind == g_fwd.part_kind && lse_off > 0 && (kind ? exp_off > lse_off : !exp_off)),
                        "partial kind / lse / exponent offsets");
                }
              }
            }
          }
        }
      }
    }
  }
  // head chunks and masks at head dim 256 (decode)
  for (int rows : {1, 4, 5, 6, 9, 12, 17, 32}) {
    for (int hc = 0; hc <= 8; ++hc) {
      for (int kind : {0, 1, 2, 3}) {
        auto a = args(2, 16, 2, rows, 4097);
        a.head_chunk = hc;
        if (kind) {
          a.mask.kind = kind, a.mask.ptr = kDev;
          a.mask.stride_row = a.kv_len + (kind == 1 ? 16 : 8);
        }
        size_t bytes = 0;
        attn_plan_info info;
        CHECK(attn_workspace_bytes(&a, ATTN_OP_DECODE, &bytes) == ATTN_OK, "chunk/mask ws");
        CHECK(attn_describe_plan(&a, ATTN_OP_DECODE, &info) == ATTN_OK, "chunk/mask plan");
        int sum = 0;
        for (int i = 0; i < info.n_head_chunks; ++i) sum += info.chunk_sizes[i];
        CHECK(sum == 8, "chunks cover the group");
        CHECK(attn_decode(&a, kWs, bytes, kStream) == ATTN_OK, "chunk/mask run");
        CHECK(strcmp(attn_variant_name(info.variant), "unknown") != 0, "variant name");
      }
    }
  }
  // the composed route
  for (int rows : {1, 128, 512}) {
    auto a = args(1, 24, 4, rows, 32768 - rows);
    size_t bytes = 0;
    CHECK(attn_workspace_bytes(&a, ATTN_OP_COMPOSED, &bytes) == ATTN_OK && bytes > 0, "composed ws");
    CHECK(attn_prefill_composed(&a, kWs, bytes, kStream) == ATTN_OK, "composed run");
    CHECK(attn_prefill_composed(&a, kWs, bytes - 1, kStream) == ATTN_E_WORKSPACE, "composed small ws");
  }
}

void aux_calls() {
  kv_append_args p;
  memset(&p, 0, sizeof(p));
  p.dtype = 0, p.B = 2, p.Hkv = 2, p.D = 256, p.rows = 5, p.kv_offset = 11, p.capacity = 20;
  p.k_new = t4(2, 5, 256, 1), p.v_new = t4(2, 5, 256, 2);
  p.k_cache = t4(2, 20, 256, 3), p.v_cache = t4(2, 20, 256, 4);
  CHECK(kv_append(&p, kStream) == ATTN_OK, "append");
  kv_append_args q = p;
  q.kv_offset = 16;
  CHECK(kv_append(&q, kStream) == ATTN_E_KV, "append past capacity");
  q = p, q.D = 96;
  CHECK(kv_append(&q, kStream) == ATTN_E_HEAD_DIM, "append head dim");
  q = p, q.k_new.ptr = nullptr;
  CHECK(kv_append(&q, kStream) == ATTN_E_NULL, "append null");
  CHECK(kv_append(nullptr, kStream) == ATTN_E_NULL, "append null args");

  uint32_t keep[4] = {0x9u, 0x7fu, 0u, 0xffffffffu};
  kv_keep_args k;
  memset(&k, 0, sizeof(k));
  k.dtype = 0, k.B = 4, k.Hkv = 2, k.D = 256, k.rows = 32, k.kv_offset = 100, k.capacity = 160;
  k.keep = keep;
  k.k_cache = t4(2, 160, 256, 3), k.v_cache = t4(2, 160, 256, 4);
  CHECK(kv_keep(&k, kStream) == ATTN_OK, "keep");
  kv_keep_args k2 = k;
  k2.rows = 3;
  CHECK(kv_keep(&k2, kStream) == ATTN_E_ARG, "keep bit past rows");
  k2 = k, k2.B = 65;
  CHECK(kv_keep(&k2, kStream) == ATTN_E_HEADS, "keep batch");
  k2 = k, k2.keep = nullptr;
  CHECK(kv_keep(&k2, kStream) == ATTN_E_NULL, "keep null");

  merge_args m;
  memset(&m, 0, sizeof(m));
  m.dtype = 1, m.n_chunks = 21, m.B = 1, m.Hq = 8, m.rows = 5, m.D = 128;
  m.partial_o = reinterpret_cast<const float*>(kWs), m.partial_lse = reinterpret_cast<const float*>(kWs + 4096);
  m.gate = t4(8, 5, 128, 2), m.out = t4(8, 5, 128, 3);
  CHECK(attn_merge(&m, kStream) == ATTN_OK, "merge");
  merge_args m2 = m;
  m2.n_chunks = 0;
  CHECK(attn_merge(&m2, kStream) == ATTN_E_ARG, "merge 0 chunks");
  m2 = m, m2.partial_lse = reinterpret_cast<const float*>(kWs + 2);
  CHECK(attn_merge(&m2, kStream) == ATTN_E_LAYOUT, "merge lse alignment");
  m2 = m, m2.D = 32;
  CHECK(attn_merge(&m2, kStream) == ATTN_E_HEAD_DIM, "merge head dim");
  {  // a carried append: checked like kv_append, then one launch with the merge
    kv_append_args ap;
    memset(&ap, 0, sizeof(ap));
    ap.dtype = 1, ap.B = 1, ap.Hkv = 2, ap.D = 128, ap.rows = 5, ap.kv_offset = 30, ap.capacity = 40;
    ap.k_new = t4(2, 5, 128, 4), ap.v_new = t4(2, 5, 128, 5), ap.k_cache = t4(2, 40, 128, 6),
    ap.v_cache = t4(2, 40, 128, 7);
    m2 = m, m2.append = &ap;
    const long merges = g_launch_merge, others = g_launch_other;
    CHECK(attn_merge(&m2, kStream) == ATTN_OK && g_merge.carry == 1 && g_merge.app.rows == 5 &&
              g_merge.app.kv_offset == 30 && g_merge.app.chunk_shift == 4 && g_launch_merge == merges + 1 &&
              g_launch_other == others,
          "merge carrying an append");
    ap.kv_offset = 36;  // rows 36..40 past capacity 40
    CHECK(attn_merge(&m2, kStream) == ATTN_E_KV && g_launch_merge == merges + 1, "carried append out of range");
  }
  {  // attn_prefill carrying the next query block's append: in its merge when it splits the keys,
     // else a launch of its own after the main pass; a bad append is refused before any launch
    kv_append_args ap;
    memset(&ap, 0, sizeof(ap));
    ap.dtype = 0, ap.B = 1, ap.Hkv = 4, ap.D = 256, ap.rows = 512, ap.kv_offset = 4608, ap.capacity = 8192;
    ap.k_new = t4(4, 512, 256, 8), ap.v_new = t4(4, 512, 256, 9), ap.k_cache = t4(4, 8192, 256, 10),
    ap.v_cache = t4(4, 8192, 256, 11);
    auto pa = args(1, 24, 4, 512, 4096);
    pa.capacity = 8192, pa.k_cache = t4(4, 8192, 256, 4), pa.v_cache = t4(4, 8192, 256, 5);
    pa.append = &ap;
    size_t need = 0;
    CHECK(attn_workspace_bytes(&pa, ATTN_OP_PREFILL, &need) == ATTN_OK && need > 0, "split prompt block");
    long f0 = g_launch_fwd, m0 = g_launch_merge, o0 = g_launch_other;
    CHECK(attn_prefill(&pa, kWs, need, kStream) == ATTN_OK && g_launch_fwd == f0 + 1 && g_launch_merge == m0 + 1 &&
              g_launch_other == o0 && g_merge.carry == 1 && g_merge.app.kv_offset == 4608 && g_merge.app.rows == 512,
          "prefill carrying the next append in its merge");
    pa.n_splits = 1;
    f0 = g_launch_fwd, m0 = g_launch_merge, o0 = g_launch_other;
    CHECK(attn_prefill(&pa, kWs, need, kStream) == ATTN_OK && g_launch_fwd == f0 + 1 && g_launch_merge == m0 &&
              g_launch_other == o0 + 1,
          "prefill without a split: the append after it");
    ap.kv_offset = 8000;  // 8000 + 512 past capacity 8192
    f0 = g_launch_fwd, m0 = g_launch_merge, o0 = g_launch_other;
    CHECK(attn_prefill(&pa, kWs, need, kStream) == ATTN_E_KV && g_launch_fwd == f0 && g_launch_other == o0,
          "bad carried append refused before any launch");
  }
  m2 = m, m2.partial_kind = 2;
  CHECK(attn_merge(&m2, kStream) == ATTN_E_ARG, "merge partial kind");
  m2 = m, m2.partial_kind = 1;
  CHECK(attn_merge(&m2, kStream) == ATTN_E_NULL, "merge fp16 partials without exponents");
  m2.partial_exp = reinterpret_cast<const int32_t*>(kWs + 8192 + 2);
  CHECK(attn_merge(&m2, kStream) == ATTN_E_LAYOUT, "merge exponent alignment");
  m2.partial_exp = reinterpret_cast<const int32_t*>(kWs + 8192);
  CHECK(attn_merge(&m2, kStream) == ATTN_OK, "merge fp16 partials");

  int sizes[64], n = 0;
  for (int rows = 0; rows <= 40; ++rows)
    for (int hq = 0; hq <= 33; ++hq)
      for (int hkv = 0; hkv <= 17; ++hkv) {
        const int r = attn_head_chunk_plan(rows, hq, hkv, 1, sizes, 64, &n);
        const bool ok = rows >= 1 && hq > 0 && hkv > 0 && hq % hkv == 0;
        CHECK((r == ATTN_OK) == ok, "chunk plan %d %d %d", rows, hq, hkv);
      }
  CHECK(attn_head_chunk_plan(4, 24, 2, 1, sizes, 1, &n) == ATTN_E_ARG, "chunk plan cap");
  for (int s = -1; s <= 13; ++s) CHECK(attn_strerror(s) != nullptr, "strerror");
}

}  // namespace

// attn_args carry: an earlier block's merge inside the main pass's launch where the plan allows
// it (attn_plan_info carry_blocks), a launch of its own ahead of the main pass otherwise, and the
// checks that refuse it before anything is enqueued.
void carried_merge() {
  kv_append_args ap;
  memset(&ap, 0, sizeof(ap));
  ap.dtype = 0, ap.B = 1, ap.Hkv = 4, ap.D = 256, ap.rows = 512, ap.capacity = 32768;
  ap.k_new = t4(4, 512, 256, 8), ap.v_new = t4(4, 512, 256, 9), ap.k_cache = t4(4, 32768, 256, 10),
  ap.v_cache = t4(4, 32768, 256, 11);
  // the last 512-row block of a 32k prompt at 24/4 heads: 5 splits over 240 workgroups
  auto pa = args(1, 24, 4, 512, 32256);
  pa.capacity = 32768, pa.k_cache = t4(4, 32768, 256, 4), pa.v_cache = t4(4, 32768, 256, 5);
  attn_plan_info info;
  CHECK(attn_describe_plan(&pa, ATTN_OP_PREFILL, &info) == ATTN_OK && info.n_splits == 5 &&
            info.partial_kind == 1 && info.grid_blocks == 240 && info.carry_blocks == 16,
        "last prompt block: %d splits, kind %d, grid %ld, carry %d", info.n_splits, info.partial_kind,
        (long)info.grid_blocks, info.carry_blocks);
  const size_t need = (size_t)info.workspace_bytes;
  // the previous block's partials, in a second workspace
  const int64_t nrow = 5LL * 24 * 512;
  char* const ws2 = kDev + (uintptr_t(12) << 36);
  merge_args m;
  memset(&m, 0, sizeof(m));
  m.dtype = 0, m.n_chunks = 5, m.B = 1, m.Hq = 24, m.rows = 512, m.D = 256, m.partial_kind = 1;
  m.partial_o = ws2;
  m.partial_lse = reinterpret_cast<const float*>(ws2 + nrow * 512);
  m.partial_exp = reinterpret_cast<const int32_t*>(ws2 + nrow * 512 + nrow * 4);
  m.gate = t4(24, 512, 256, 13), m.out = t4(24, 512, 256, 14);
  pa.carry = &m;
  pa.append = &ap;
  ap.kv_offset = 32768 - 512;  // (any rows the call does not read; here the block's own, as a placeholder)
  int32_t nc = 0, kind = 0;
  size_t lo = 0, eo = 0;
  long f0 = g_launch_fwd, m0 = g_launch_merge, o0 = g_launch_other;
  CHECK(attn_prefill_partials(&pa, kWs, need, kStream, &nc, &kind, &lo, &eo) == ATTN_OK && g_launch_fwd == f0 + 1 &&
            g_launch_merge == m0 && g_launch_other == o0,
        "merge and append carried in the main pass's launch");
  CHECK(g_fwd.extra_blocks == 16 && g_fwd.carried.n_chunks == 5 && g_fwd.carried.part_o == ws2 &&
            g_fwd.carried.carry == 1 && g_fwd.carried.app.rows == 512 && g_fwd.carried.app_by == 8 &&
            g_fwd.carried.app_bx == 2,
        "carried work: %d blocks, %d chunks, append %d x %d", g_fwd.extra_blocks, g_fwd.carried.n_chunks,
        g_fwd.carried.app_bx, g_fwd.carried.app_by);
  // attn_prefill merges itself: the append rides on that merge, the carried merge in the launch
  f0 = g_launch_fwd, m0 = g_launch_merge, o0 = g_launch_other;
  CHECK(attn_prefill(&pa, kWs, need, kStream) == ATTN_OK && g_launch_fwd == f0 + 1 && g_launch_merge == m0 + 1 &&
            g_launch_other == o0 && g_fwd.extra_blocks == 16 && g_fwd.carried.n_chunks == 5 &&
            g_fwd.carried.carry == 0 && g_merge.carry == 1,
        "attn_prefill carrying a merge");
  // fp32 partials or more than 8 chunks: a merge launch of its own ahead of the main pass (the
  // append still rides in the launch)
  merge_args m32 = m;
  m32.partial_kind = 0, m32.partial_exp = nullptr;
  pa.carry = &m32;
  f0 = g_launch_fwd, m0 = g_launch_merge, o0 = g_launch_other;
  CHECK(attn_prefill_partials(&pa, kWs, need, kStream, &nc, &kind, &lo, &eo) == ATTN_OK && g_launch_fwd == f0 + 1 &&
            g_launch_merge == m0 + 1 && g_launch_other == o0 && g_fwd.extra_blocks == 16 &&
            g_fwd.carried.n_chunks == 0 && g_fwd.carried.carry == 1,
        "fp32 carried merge launched on its own");
  merge_args m12 = m;
  m12.n_chunks = 12;
  pa.carry = &m12;
  pa.append = nullptr;
  f0 = g_launch_fwd, m0 = g_launch_merge, o0 = g_launch_other;
  CHECK(attn_prefill_partials(&pa, kWs, need, kStream, &nc, &kind, &lo, &eo) == ATTN_OK && g_launch_fwd == f0 + 1 &&
            g_launch_merge == m0 + 1 && g_launch_other == o0 && g_fwd.extra_blocks == 0,
        "12-chunk carried merge launched on its own, nothing carried");
  // refused before any launch: partials in this call's workspace, an append of its own, null
  // partials, a bad kind
  merge_args bad = m;
  bad.partial_lse = reinterpret_cast<const float*>(kWs + 4096);
  pa.carry = &bad;
  const long before = launches();
  CHECK(attn_prefill_partials(&pa, kWs, need, kStream, &nc, &kind, &lo, &eo) == ATTN_E_ARG, "carry in the workspace");
  bad = m, bad.append = &ap;
  CHECK(attn_prefill(&pa, kWs, need, kStream) == ATTN_E_ARG, "carry with an append of its own");
  bad = m, bad.partial_o = nullptr;
  CHECK(attn_prefill(&pa, kWs, need, kStream) == ATTN_E_NULL, "carry without partials");
  bad = m, bad.partial_kind = 3;
  CHECK(attn_prefill(&pa, kWs, need, kStream) == ATTN_E_ARG, "carry of an unknown kind");
  CHECK(launches() == before, "refused carries launch nothing");
  // a short block (16 tiles over 4 splits): nothing carried in the launch
  auto pb = args(1, 24, 4, 512, 0);
  pb.capacity = 32768, pb.k_cache = t4(4, 32768, 256, 4), pb.v_cache = t4(4, 32768, 256, 5);
  CHECK(attn_describe_plan(&pb, ATTN_OP_PREFILL, &info) == ATTN_OK && info.n_splits > 1 && info.carry_blocks == 0,
        "first prompt block carries nothing (%d splits)", info.n_splits);
  pb.carry = &m;
  pb.append = &ap;
  ap.kv_offset = 512;
  f0 = g_launch_fwd, m0 = g_launch_merge, o0 = g_launch_other;
  CHECK(attn_prefill_partials(&pb, kWs, (size_t)info.workspace_bytes, kStream, &nc, &kind, &lo, &eo) == ATTN_OK &&
            g_launch_fwd == f0 + 1 && g_launch_merge == m0 + 1 && g_launch_other == o0 + 1 && g_fwd.extra_blocks == 0,
        "short block: merge before, append after");
  // the composed route: the carried merge ahead of it
  pb.append = nullptr;
  m0 = g_launch_merge, o0 = g_launch_other;
  CHECK(attn_prefill_composed(&pb, kWs, (size_t)1 << 34, kStream) == ATTN_OK && g_launch_merge == m0 + 1 &&
            g_launch_other == o0 + 1,
        "composed route carrying a merge");
}

int main() {
  rejection_matrix();
  carried_merge();
  launch_limits();
  sweep();
  aux_calls();
  printf("sanitize: %ld checks, %d failed, %ld launches\n", g_checks, g_fail, launches());
  return g_fail == 0 ? 0 : 1;
}
