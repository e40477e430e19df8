/*
 * gqa_attn.h -- C ABI of the gated causal GQA attention library (head_dim 256, also 128 and
 * 64; gfx950).
 *
 * The operation (TensorFold PR #1009, attention kernel-contract commit and
 * Receipt "Attention"; "Qwen head-chunked SDPA (#113)", introduction):
 *
 *   for batch b, query head h, query row r (absolute position kv_offset + r):
 *     g   = h / (Hq / Hkv)                       consecutive heads share a KV head
 *     A   = { j < kv_len : j <= kv_offset + r (if causal), mask admits j }
 *     s_j = scale * <Q[b,h,r,:], K[b,g,j,:]> + mask_add[b,h,r,j]
 *     o   = sum_{j in A} softmax_A(s)_j * V[b,g,j,:]          (0 if A is empty)
 *     out[b,h,r,:] = o * sigmoid(gate[b,h,r,:])
 *
 * with fp32 accumulation and one final rounding to the 16-bit output type.
 * Prompts are processed in query blocks of `rows` rows that attend to the
 * cache plus themselves ("perf(qwen36): qualify M4 head-256 attention",
 * Summary); decode and verify rows (1..32) read the same contiguous cache.
 *
 * Conventions for every entry point:
 *   - Every pointer argument named as a tensor is DEVICE memory owned by the
 *     caller; the library never allocates or frees device memory and keeps no
 *     pointer after the call returns.  Argument structs are HOST memory, read
 *     during the call only.
 *   - Tensors are described by a base pointer and strides in ELEMENTS; the
 *     last (head_dim) dimension is contiguous.  Base pointers must be 16-byte
 *     aligned and row/head/batch strides multiples of 8 elements.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     asynchronously; buffers must stay alive until the stream reaches it.
 *   - Functions return ATTN_OK (0) or an attn_status code.  All validation
 *     happens before anything is enqueued; on an error nothing is written.
 *     The library never aborts.
 *   - The library holds no mutable global state and is reentrant; calls on
 *     different streams may overlap if their output/workspace buffers differ.
 *     The one exception is attn_decode_noalloc's device scratch (see there).
 */
#ifndef GQA_ATTN_H
#define GQA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GQA_ATTN_ABI_VERSION 7
#define ATTN_HEAD_DIM 256
#define ATTN_MAX_DECODE_ROWS 32
#define ATTN_MAX_CHUNKS 64

typedef enum {
  ATTN_OK = 0,
  ATTN_E_NULL = 1,       /* a required pointer is NULL */
  ATTN_E_DTYPE = 2,      /* unknown dtype */
  ATTN_E_HEADS = 3,      /* Hq <= 0, Hkv <= 0, Hq % Hkv != 0, B <= 0, or Hq/Hkv > 64 (checked before dividing) */
  ATTN_E_HEAD_DIM = 4,   /* D not 256, 128 or 64: fail closed */
  ATTN_E_ROWS = 5,       /* rows < 1, or rows > 32 for attn_decode */
  ATTN_E_KV = 6,         /* kv_offset < 0, kv_len < 1, kv_len > capacity, kv_len < kv_offset + rows when causal,
                            or an append beyond capacity */
  ATTN_E_MASK = 7,       /* unknown mask kind, Bm not in {1, B}, Hm not in {1, Hq}, or a NULL mask pointer */
  ATTN_E_LAYOUT = 8,     /* misaligned pointer or stride */
  ATTN_E_HEAD_CHUNK = 9, /* head_chunk < 0 or > Hq/Hkv */
  ATTN_E_WORKSPACE = 10, /* workspace smaller than attn_workspace_bytes() reports */
  ATTN_E_HIP = 11,       /* the HIP runtime reported an error when enqueuing */
  ATTN_E_ARG = 12        /* any other invalid argument (bad op, n_splits < 0, scale not finite, ...) */
} attn_status;

typedef enum { ATTN_BF16 = 0, ATTN_F16 = 1 } attn_dtype;

/* Mask kinds ("Qwen head-chunked SDPA (#113)", "Exact scope found during review": no mask,
 * boolean and additive masks, broadcast over batch and heads).  kv is the contiguous last
 * dimension; entries for keys >= kv_len are never read. */
typedef enum {
  ATTN_MASK_NONE = 0,
  ATTN_MASK_BOOL_U8 = 1,  /* uint8: nonzero = may attend */
  ATTN_MASK_ADD = 2,      /* same 16-bit type as Q: added to the score, -Inf hides the key */
  ATTN_MASK_ADD_F32 = 3   /* float32 additive */
} attn_mask_kind;

typedef enum { ATTN_OP_PREFILL = 0, ATTN_OP_DECODE = 1, ATTN_OP_COMPOSED = 2 } attn_op;

/* A strided 4-d tensor [B, H, rows_or_tokens, 256]; strides in elements. */
typedef struct {
  void* ptr;
  int64_t stride_b;
  int64_t stride_h;
  int64_t stride_row;
} attn_tensor;

/* Optional mask [Bm, Hm, rows, >= kv_len]; a stride may be 0 to broadcast. */
typedef struct {
  int32_t kind;   /* attn_mask_kind */
  int32_t Bm;     /* 1 or B */
  int32_t Hm;     /* 1 or Hq (indexed by the global query head) */
  int32_t reserved;
  const void* ptr;
  int64_t stride_b;
  int64_t stride_h;
  int64_t stride_row;
} attn_mask;

typedef struct kv_append_args kv_append_args;
typedef struct merge_args merge_args;

/* Arguments of attn_prefill / attn_decode. */
typedef struct {
  int32_t dtype;       /* attn_dtype of q, k/v cache, gate, out and an ATTN_MASK_ADD mask */
  int32_t B;           /* batch */
  int32_t Hq;          /* query heads */
  int32_t Hkv;         /* KV heads; Hq / Hkv = GQA group size G */
  int32_t D;           /* head_dim: 256, 128 or 64 (else ATTN_E_HEAD_DIM) */
  int32_t rows;        /* query rows in this call (a query block, or 1..32 decode/verify rows) */
  int64_t kv_offset;   /* cached keys before row 0 = absolute position of row 0 */
  int64_t kv_len;      /* valid keys in the cache (normally kv_offset + rows, after kv_append) */
  int64_t capacity;    /* allocated tokens per (b, kv head) in the cache */
  float scale;         /* score scale; 0 means 1/sqrt(head_dim) (1/16 at 256) */
  int32_t causal;      /* 1: row r sees keys <= kv_offset + r; 0: all keys < kv_len */
  int32_t head_chunk;  /* 0: the head-chunk policy; k in 1..G: chunks of k heads (k = G: off) */
  int32_t n_splits;    /* KV splits; 0 = automatic */
  attn_tensor q;       /* [B, Hq, rows, 256] */
  attn_tensor gate;    /* [B, Hq, rows, 256] */
  attn_tensor out;     /* [B, Hq, rows, 256], written */
  attn_tensor k_cache; /* [B, Hkv, capacity, 256] */
  attn_tensor v_cache; /* [B, Hkv, capacity, 256] */
  attn_mask mask;
  const kv_append_args* append; /* NULL, or a kv_append enqueued with the call: in the merge's
                                   launch when the call splits the keys and merges them (workgroups
                                   of its own, one launch fewer); for attn_prefill_partials, in the
                                   main pass's launch where that carries work (see carry), else a
                                   launch of its own after the call.  Checked as kv_append checks
                                   it, with the call's other arguments, before anything is
                                   enqueued.  Unordered with the call's own work, so it must not
                                   touch what the call reads or writes; a prompt's loop passes the
                                   next query block's rows */
  const merge_args* carry;      /* NULL, or an attn_merge of an EARLIER call's split partials (say
                                   the previous query block's, from attn_prefill_partials), done by
                                   this call and unordered with the rest of it: its partials, gate
                                   and out must not be touched by this call (partials overlapping
                                   this call's workspace: ATTN_E_ARG), and its own append must be
                                   NULL (else ATTN_E_ARG).  Checked as attn_merge checks it, before
                                   anything is enqueued.  Where the call's plan has carry_blocks
                                   (attn_plan_info: an unmasked prompt block writing fp16 partials
                                   that leaves CUs idle) and the merge is of at most 8 chunks of
                                   fp16 partials in the call's dtype, it runs on those CUs inside
                                   the main pass's launch (the same bits as attn_merge); otherwise
                                   it is a launch of its own ahead of the main pass.  A prompt's
                                   loop carries block i - 1's merge with block i's main pass: one
                                   launch per block */
} attn_args;

/* Arguments of kv_append: k_cache[b, g, kv_offset + r, :] = k_new[b, g, r, :] (and V), bit for bit. */
struct kv_append_args {
  int32_t dtype;
  int32_t B;
  int32_t Hkv;
  int32_t D;
  int32_t rows;
  int32_t reserved;
  int64_t kv_offset;
  int64_t capacity;
  attn_tensor k_new;   /* [B, Hkv, rows, 256] */
  attn_tensor v_new;   /* [B, Hkv, rows, 256] */
  attn_tensor k_cache; /* [B, Hkv, capacity, 256], written */
  attn_tensor v_cache; /* [B, Hkv, capacity, 256], written */
};

/* Arguments of kv_keep.  After a verify block of `rows` rows was appended at kv_offset and some
 * of its rows were accepted: for each batch entry b, the rows r with bit r of keep[b] set move,
 * in increasing r, to cache rows kv_offset, kv_offset + 1, ... of every KV head, bit for bit;
 * the block's rows after the kept ones are left as they were.  An accepted path of a draft tree
 * whose rows are numbered parents first (a chain being the special case 0, 1, 2, ...) keeps
 * its order.  TensorFold PR #1009 (attention kernel-contract commit) compares keep bit for bit,
 * also when it is repeated on the caches its first call produced. */
typedef struct {
  int32_t dtype;
  int32_t B;              /* 1..64 */
  int32_t Hkv;
  int32_t D;
  int32_t rows;           /* rows of the verify block: 1..32 */
  int32_t reserved;
  int64_t kv_offset;      /* cache index of the block's first row */
  int64_t capacity;
  const uint32_t* keep;   /* host array [B]: bit r set = keep row r (bits at or past rows must be 0);
                             read during the call only */
  attn_tensor k_cache;    /* [B, Hkv, capacity, 256]: rows kv_offset .. kv_offset + rows - 1 rewritten */
  attn_tensor v_cache;    /* [B, Hkv, capacity, 256], the same */
} kv_keep_args;

/* Arguments of attn_merge. */
struct merge_args {
  int32_t dtype;
  int32_t n_chunks;         /* >= 1 */
  int32_t B;
  int32_t Hq;
  int32_t rows;
  int32_t D;                /* head dim: 256, 128 or 64 (else ATTN_E_HEAD_DIM) */
  const void* partial_o;    /* [n_chunks, B, Hq, rows] rows, contiguous, normalised per chunk; see partial_kind */
  const float* partial_lse; /* [n_chunks, B, Hq, rows] fp32, contiguous, natural log; -Inf = empty chunk */
  attn_tensor gate;         /* [B, Hq, rows, D] */
  attn_tensor out;          /* [B, Hq, rows, D], written */
  int32_t partial_kind;     /* 0: rows of D fp32 values; 1: the rows attn_prefill_partials leaves, D fp16
                               values v_d each (round to nearest even), the partial being v_d 2^e with e
                               the row's entry of partial_exp (it puts the row's largest magnitude in
                               [0.5, 1)); anything else: ATTN_E_ARG */
  const int32_t* partial_exp; /* partial_kind 1: [n_chunks, B, Hq, rows] int32, contiguous (NULL:
                                 ATTN_E_NULL); ignored for partial_kind 0 */
  const kv_append_args* append; /* NULL, or a kv_append carried by the merge's launch (workgroups of
                                   their own, checked as kv_append checks it: its errors, and
                                   ATTN_E_ARG if the two exceed a launch); the two are unordered, so
                                   the append must not touch what the merge reads or writes.  A
                                   prompt's loop enqueues block i's merge with block i + 1's append,
                                   one launch fewer per block */
};

/* The resolved plan of one call (what would run, for logging and validation). */
typedef struct {
  int32_t op;              /* attn_op */
  int32_t variant;         /* kernel variant id (see attn_variant_name) */
  int32_t group_size;      /* G = Hq / Hkv */
  int32_t n_head_chunks;   /* chunks per KV group */
  int32_t head_chunk;      /* heads per chunk (last chunk may be smaller) */
  int32_t rows_per_wave;   /* (head, row) pairs per wavefront: 32 (one 32-wide MFMA column block) */
  int32_t waves_per_block; /* wavefronts per workgroup of the main pass */
  int32_t n_row_tiles;     /* workgroups per (batch, KV head, split) */
  int32_t n_splits;        /* KV splits (1: the gate is applied in the same kernel) */
  int32_t keys_per_split;
  int32_t keys_per_tile;   /* keys staged in LDS per step */
  int32_t lds_bytes;
  int64_t grid_blocks;     /* workgroups of the main pass */
  int64_t workspace_bytes; /* bytes of workspace the call needs */
  int32_t chunk_sizes[ATTN_MAX_CHUNKS]; /* heads per chunk within a KV group, first n_head_chunks valid */
  int32_t partial_kind;    /* with n_splits > 1: the split partials' form (merge_args partial_kind;
                              1 from 8 MiB of fp32 partials up), else 0 */
  int32_t carry_blocks;    /* workgroups the main pass's launch adds for work a call carries on the
                              CUs it leaves idle (attn_args carry, and the append of
                              attn_prefill_partials): unmasked prompt blocks with fp16 partials
                              whose main pass is long enough to cover, on those CUs, a merge of
                              its own size (B Hq rows <= 10 x idle CUs x tiles per split); 0 where
                              such work gets launches of its own */
} attn_plan_info;

/* A prompt to be run as query blocks (kv_append + attn_prefill per block), for
 * attn_prompt_policy. */
typedef struct {
  int32_t D;          /* head_dim: 256, 128 or 64 */
  int32_t B;          /* batch */
  int32_t Hq;         /* query heads */
  int32_t Hkv;        /* KV heads */
  int64_t n_tokens;   /* prompt rows */
  int32_t dtype;      /* attn_dtype */
  int32_t gfx;        /* the device's gfx number (950 for gfx950); 0 if unknown */
  int32_t n_cus;      /* compute units of the device; 0 if unknown */
} attn_prompt_query;

typedef enum {
  ATTN_POLICY_WHOLE = 0,   /* short prompt: one call for all of it */
  ATTN_POLICY_TABLE = 1,   /* the block size measured fastest on this device */
  ATTN_POLICY_DEFAULT = 2  /* device not the one the table was measured on: blocks of 512 */
} attn_policy_reason;

/* The route and query-block size attn_prompt_policy picks. */
typedef struct {
  int32_t route;      /* ATTN_OP_PREFILL (fused) or ATTN_OP_COMPOSED */
  int32_t q_block;    /* rows per call (the last call may be shorter) */
  int32_t qualified;  /* 1: the device is the one the table was measured on */
  int32_t reason;     /* attn_policy_reason */
  int64_t n_calls;    /* calls for the whole prompt: ceil(n_tokens / q_block) */
} attn_prompt_choice;

/* ABI version (GQA_ATTN_ABI_VERSION). */
int attn_abi_version(void);

/* sizeof of the argument structs as compiled into the library: which = 0 attn_args,
 * 1 kv_append_args, 2 merge_args, 3 attn_plan_info, 4 kv_keep_args, 5 attn_prompt_query,
 * 6 attn_prompt_choice.  Returns 0 for an unknown value. */
size_t attn_struct_size(int which);

/* Static description of a status code.  Never NULL. */
const char* attn_strerror(int status);

/* Name of a kernel variant id from attn_plan_info.variant ("unknown" for an id no variant has).
 * Never NULL.  The name lists the dtype, the mask kind, the shape (4x1, 8x1, 8x1_stream), how
 * the mask reaches the main pass (nothing: per-lane loads; _ldsrows / _ldswords: staged in LDS
 * with each K/V tile from a mask the same for every head; _ldspairwords: the same from a
 * full-head mask, when each workgroup's pairs form one column block) and the head dim. */
const char* attn_variant_name(int variant);

/* The head-chunk rule of "Qwen head-chunked SDPA (#113)" (introduction; "Exact scope found
 * during review"): if enabled and rows * G > 32 with rows <= 32, a KV group's G query heads
 * are cut into chunks of min(G, 32 / rows) heads (integer division), the remainder forming a
 * last, smaller chunk; otherwise one chunk of G.  Writes the chunk sizes of one group to
 * sizes[0 .. *n_chunks) (host memory, capacity `cap`).  Pure host function; no device use.
 * Errors: ATTN_E_ROWS (rows < 1), ATTN_E_HEADS (bad head counts), ATTN_E_NULL, ATTN_E_ARG
 * (cap too small). */
int attn_head_chunk_plan(int rows, int n_q_heads, int n_kv_heads, int enabled, int* sizes, int cap,
                         int* n_chunks);

/* The prompt policy ("perf(qwen36): qualify M4 head-256 attention", Summary and the review
 * comment on eligibility: the query-block size and composed vs fused chosen per machine and per
 * head dimension).  Keyed on the device (gfx number and compute units) and the head dim, from
 * the fused prompt times measured per block size on gfx950 with 256 compute units (head dims
 * 256, 128, 64; 24/4 and 16/2 heads; 2048, 8192 and 32768 tokens):
 *   - the route is always the fused pass (the composed route is 9-13x slower at every head dim);
 *   - prompts of at most 2048 rows run as one call;
 *   - longer prompts run in blocks of 8192 rows when G = Hq / Hkv <= 6 and of 4096 rows when
 *     G > 6 (the same at every head dim), divided by the batch (down to 512), at most the
 *     prompt;
 *   - any other device gets blocks of 512 rows, flagged unqualified.
 * Pure host function; no device use.  Errors: ATTN_E_NULL, ATTN_E_HEAD_DIM, ATTN_E_HEADS
 * (B < 1 or heads not a whole group), ATTN_E_ROWS (n_tokens < 1), ATTN_E_DTYPE. */
int attn_prompt_policy(const attn_prompt_query* q, attn_prompt_choice* out);

/* Workspace bytes a call with these arguments needs (0 when it needs none).  op is attn_op
 * (ATTN_OP_COMPOSED: attn_prefill_composed).  Validates `a` like the call itself would.  No
 * device use. */
int attn_workspace_bytes(const attn_args* a, int op, size_t* bytes);

/* The resolved plan of a call with these arguments (op ATTN_OP_PREFILL or ATTN_OP_DECODE;
 * ATTN_E_ARG otherwise).  No device use. */
int attn_describe_plan(const attn_args* a, int op, attn_plan_info* info);

/* Gated causal GQA attention for a block of query rows (any rows >= 1): the flash-style
 * pass over the cache in 16 KiB K/V tiles (8192 / head_dim keys: 32 at 256, 64 at 128, 128 at
 * 64), split over KV when the grid would be too small, the
 * log-sum-exp merge of the splits and the gate.  `workspace` (device, >= the bytes
 * attn_workspace_bytes(a, ATTN_OP_PREFILL) reports; may be NULL if that is 0) holds the
 * split partials.  Writes a->out.  Keys a row cannot see never reach it, also when their
 * V (or K) rows hold +-Inf or NaN (TensorFold PR #1009: -Inf times a zero probability must
 * not become NaN): a pair whose result came out NaN is computed again over its admissible
 * keys, in the epilogue (one split) or in the merge (several). */
int attn_prefill(const attn_args* a, void* workspace, size_t ws_bytes, void* stream);
/* Head dims 128 and 64 (attn_prefill, attn_decode, attn_prefill_partials and
 * attn_decode_noalloc) take the same main pass, plans, head chunks, masks and nonfinite repair
 * as 256; the partials hold rows of head_dim values, and scale = 0 means 1 / sqrt(head_dim). */

/* The main pass of attn_prefill alone, for callers that put one query block's merge beside the
 * next block's main pass (two workspaces, in turn): the next call's attn_args carry (inside its
 * main pass's launch where its plan has carry_blocks), or attn_merge on a second stream.  *n_chunks
 * receives the number of KV chunks of the plan.  With *n_chunks = 1 the call is complete and out
 * is written.  With *n_chunks > 1 out is not written: the normalised partials stay in the
 * workspace in the form *partial_kind gives (that of merge_args): o at offset 0
 * ([n_chunks, B, Hq, rows, head_dim], fp32 for kind 0, fp16 for kind 1), the natural-log lse at
 * byte offset *lse_offset ([n_chunks, B, Hq, rows] fp32) and, for kind 1, each row's power of
 * two at byte offset *exp_offset ([n_chunks, B, Hq, rows] int32; 0 for kind 0).  The plan takes
 * kind 1 from 8 MiB of fp32 partials up (n_chunks B Hq rows head_dim 4 bytes), kind 0 below.
 * The caller completes the call with attn_merge (that partial_kind, gate and out as here) on a
 * stream ordered after this one, before the workspace is reused.  Errors as attn_prefill, plus
 * ATTN_E_NULL for a null n_chunks, partial_kind, lse_offset or exp_offset.  The
 * merge called on its own has no inputs to redo a row from: with nonfinite inputs a hidden key
 * may leave NaN in the result of this pair of calls (attn_prefill repairs it). */
int attn_prefill_partials(const attn_args* a, void* workspace, size_t ws_bytes, void* stream, int32_t* n_chunks,
                          int32_t* partial_kind, size_t* lse_offset, size_t* exp_offset);

/* The same operation for 1..32 decode / verify rows: a split-KV pass in which each
 * workgroup reads its KV chunk once for all heads of the group, each wavefront serving one
 * head chunk (a->head_chunk), then the merge pass.  TensorFold PR #1009 (attention
 * kernel-contract commit) splits decode rows over key chunks and merges them. */
int attn_decode(const attn_args* a, void* workspace, size_t ws_bytes, void* stream);

/* attn_decode for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same plan, kernels and result as
 * attn_decode (bit for bit), with the split partials in the library's own device scratch
 * instead of a caller workspace.  The caller still passes its inputs and outputs; the call
 * allocates nothing.
 *   - The scratch is a 64 MiB device array (GQA_ATTN_SCRATCH_BYTES) that every GPU the library
 *     runs on holds until the process ends.  Its address on a device is looked up on the first
 *     call made with that device current (make that first call outside graph capture); the
 *     stream must belong to the current device.
 *   - A plan whose partials (attn_workspace_bytes(a, ATTN_OP_DECODE)) exceed the scratch is
 *     rejected with ATTN_E_WORKSPACE before anything is enqueued (set n_splits lower to fit).
 *     At head_dim 256 the partials of n_splits chunks take n_splits B Hq rows 1028 bytes (fp32)
 *     below 8 MiB of values and 520 bytes (fp16 and a power of two) from there: 32 rows of 16
 *     heads at batch 2 fit up to 126 chunks.
 *   - Every call on one GPU shares that GPU's scratch: calls that overlap on one GPU (on
 *     different streams) race and must be ordered by the caller.  Nothing in the scratch needs
 *     to start at zero: the main pass writes every partial the merge reads.
 * Errors: those of attn_decode, ATTN_E_WORKSPACE as above, ATTN_E_HIP if the scratch's address
 * cannot be found on the current device. */
#define GQA_ATTN_SCRATCH_BYTES (64u << 20)
int attn_decode_noalloc(const attn_args* a, void* stream);

/* The composed (materialised-score) route for the same block, for comparison with the fused
 * kernel ("perf(qwen36): qualify M4 head-256 attention", Summary: composed against fused
 * attention for head_dim 256 at query blocks of 128 and 512 rows).  Three passes through the
 * workspace: the fp32 scores Q K^T of every key of the block's key range, the row softmax
 * writing weights rounded to the 16-bit type (and 1 / their sum), then P V with the gate.
 * Same arguments and result as attn_prefill (within the same tolerance) except: no mask
 * (ATTN_E_MASK otherwise), head_chunk and n_splits are ignored, inputs are taken to be finite.
 * scale = 0 means 1 / sqrt(head_dim).
 * `workspace` (device) must hold attn_workspace_bytes(a, ATTN_OP_COMPOSED) bytes:
 * B Hq rows kvp (4 + 2) + B Hq rows 4 bytes (each part rounded up to 256), kvp = the key range
 * (kv_len, or kv_offset + rows when causal) rounded up to 32.  ATTN_E_ARG when B Hq > 65535 or
 * B Hq rows > 2^31 - 1. */
int attn_prefill_composed(const attn_args* a, void* workspace, size_t ws_bytes, void* stream);

/* Append `rows` new K and V rows to the cache at kv_offset: a pure bit copy (signed zeros
 * and NaN payloads survive).  head_dim 64, 128 or 256.  TensorFold PR #1009 compares append
 * bit for bit. */
int kv_append(const kv_append_args* a, void* stream);

/* Compact the kept rows of a verify block in the caches, in place (see kv_keep_args): a pure bit
 * copy.  Errors (nothing is written): ATTN_E_NULL (a, keep or a cache pointer), ATTN_E_DTYPE,
 * ATTN_E_HEADS (B not in 1..64 or Hkv < 1), ATTN_E_HEAD_DIM, ATTN_E_ROWS (rows not in 1..32),
 * ATTN_E_KV (kv_offset < 0 or the block past capacity), ATTN_E_ARG (a keep bit at or past
 * rows), ATTN_E_LAYOUT.  TensorFold PR #1009 compares keep bit for bit. */
int kv_keep(const kv_keep_args* a, void* stream);

/* Combine per-chunk partials (o_c normalised within chunk c, lse_c = its log-sum-exp):
 * out = sum_c exp(lse_c - lse) o_c / sum_c exp(lse_c - lse) * sigmoid(gate), chunks with
 * lse_c = -Inf contribute nothing and an all-empty row gives 0.  The decode merge of
 * TensorFold PR #1009 (attention kernel-contract commit), usable by callers that split KV
 * across calls (a prefix and a tail, for instance).  A chunk whose lse_c is NaN makes the row
 * NaN. */
int attn_merge(const merge_args* a, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_ATTN_H */
