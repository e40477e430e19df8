"""ctypes mirror of include/gqa_attn.h (structs, enums, prototypes).

Argument marshalling only: every step of the computation runs in libgqa_attn.so.
The struct sizes are checked against the library's own (attn_struct_size) when it loads.
"""

import ctypes as C
import os

ABI_VERSION = 7
HEAD_DIM = 256
MAX_DECODE_ROWS = 32
MAX_CHUNKS = 64

OK = 0
STATUS = {
    0: "ATTN_OK", 1: "ATTN_E_NULL", 2: "ATTN_E_DTYPE", 3: "ATTN_E_HEADS", 4: "ATTN_E_HEAD_DIM", 5: "ATTN_E_ROWS",
    6: "ATTN_E_KV", 7: "ATTN_E_MASK", 8: "ATTN_E_LAYOUT", 9: "ATTN_E_HEAD_CHUNK", 10: "ATTN_E_WORKSPACE",
    11: "ATTN_E_HIP", 12: "ATTN_E_ARG",
}
STATUS_CODE = {v: k for k, v in STATUS.items()}

BF16, F16 = 0, 1
MASK_NONE, MASK_BOOL_U8, MASK_ADD, MASK_ADD_F32 = 0, 1, 2, 3
OP_PREFILL, OP_DECODE, OP_COMPOSED = 0, 1, 2

EXPORTS = (
    "attn_abi_version", "attn_struct_size", "attn_strerror", "attn_variant_name", "attn_head_chunk_plan",
    "attn_workspace_bytes", "attn_describe_plan", "attn_prefill", "attn_decode", "kv_append", "attn_merge",
    "kv_keep", "attn_prefill_partials", "attn_prefill_composed", "attn_decode_noalloc", "attn_prompt_policy",
)
SCRATCH_BYTES = 64 << 20  # the device scratch of attn_decode_noalloc, per GPU
KEEP_MAX_BATCH = 64


class Tensor(C.Structure):
    _fields_ = [("ptr", C.c_void_p), ("stride_b", C.c_int64), ("stride_h", C.c_int64), ("stride_row", C.c_int64)]


class Mask(C.Structure):
    _fields_ = [("kind", C.c_int32), ("Bm", C.c_int32), ("Hm", C.c_int32), ("reserved", C.c_int32),
                ("ptr", C.c_void_p), ("stride_b", C.c_int64), ("stride_h", C.c_int64), ("stride_row", C.c_int64)]


class KvAppendArgs(C.Structure):
    _fields_ = [("dtype", C.c_int32), ("B", C.c_int32), ("Hkv", C.c_int32), ("D", C.c_int32), ("rows", C.c_int32),
                ("reserved", C.c_int32), ("kv_offset", C.c_int64), ("capacity", C.c_int64), ("k_new", Tensor),
                ("v_new", Tensor), ("k_cache", Tensor), ("v_cache", Tensor)]


class MergeArgs(C.Structure):
    _fields_ = [("dtype", C.c_int32), ("n_chunks", C.c_int32), ("B", C.c_int32), ("Hq", C.c_int32),
                ("rows", C.c_int32), ("D", C.c_int32), ("partial_o", C.c_void_p), ("partial_lse", C.c_void_p),
                ("gate", Tensor), ("out", Tensor), ("partial_kind", C.c_int32),
                ("partial_exp", C.c_void_p), ("append", C.POINTER(KvAppendArgs))]


class AttnArgs(C.Structure):
    _fields_ = [("dtype", C.c_int32), ("B", C.c_int32), ("Hq", C.c_int32), ("Hkv", C.c_int32), ("D", C.c_int32),
                ("rows", C.c_int32), ("kv_offset", C.c_int64), ("kv_len", C.c_int64), ("capacity", C.c_int64),
                ("scale", C.c_float), ("causal", C.c_int32), ("head_chunk", C.c_int32), ("n_splits", C.c_int32),
                ("q", Tensor), ("gate", Tensor), ("out", Tensor), ("k_cache", Tensor), ("v_cache", Tensor),
                ("mask", Mask), ("append", C.POINTER(KvAppendArgs)), ("carry", C.POINTER(MergeArgs))]


class KvKeepArgs(C.Structure):
    _fields_ = [("dtype", C.c_int32), ("B", C.c_int32), ("Hkv", C.c_int32), ("D", C.c_int32), ("rows", C.c_int32),
                ("reserved", C.c_int32), ("kv_offset", C.c_int64), ("capacity", C.c_int64),
                ("keep", C.POINTER(C.c_uint32)), ("k_cache", Tensor), ("v_cache", Tensor)]


class PlanInfo(C.Structure):
    _fields_ = [("op", C.c_int32), ("variant", C.c_int32), ("group_size", C.c_int32), ("n_head_chunks", C.c_int32),
                ("head_chunk", C.c_int32), ("rows_per_wave", C.c_int32), ("waves_per_block", C.c_int32),
                ("n_row_tiles", C.c_int32), ("n_splits", C.c_int32), ("keys_per_split", C.c_int32),
                ("keys_per_tile", C.c_int32), ("lds_bytes", C.c_int32), ("grid_blocks", C.c_int64),
                ("workspace_bytes", C.c_int64), ("chunk_sizes", C.c_int32 * MAX_CHUNKS), ("partial_kind", C.c_int32),
                ("carry_blocks", C.c_int32)]


class PromptQuery(C.Structure):
    _fields_ = [("D", C.c_int32), ("B", C.c_int32), ("Hq", C.c_int32), ("Hkv", C.c_int32),
                ("n_tokens", C.c_int64), ("dtype", C.c_int32), ("gfx", C.c_int32), ("n_cus", C.c_int32)]


class PromptChoice(C.Structure):
    _fields_ = [("route", C.c_int32), ("q_block", C.c_int32), ("qualified", C.c_int32), ("reason", C.c_int32),
                ("n_calls", C.c_int64)]


POLICY_REASON = {0: "whole_prompt", 1: "table", 2: "unqualified_default"}

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgqa_attn.so")


def load(path: str = LIB_PATH) -> C.CDLL:
    """Load the shared library and declare its prototypes; raises if it is missing."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -m gqa_causal_attention_attn_amd.build` "
                           "(or __graft_entry__.build()) first")
    lib = C.CDLL(path)
    P = C.POINTER
    lib.attn_abi_version.restype = C.c_int
    lib.attn_abi_version.argtypes = []
    lib.attn_struct_size.restype = C.c_size_t
    lib.attn_struct_size.argtypes = [C.c_int]
    lib.attn_strerror.restype = C.c_char_p
    lib.attn_strerror.argtypes = [C.c_int]
    lib.attn_variant_name.restype = C.c_char_p
    lib.attn_variant_name.argtypes = [C.c_int]
    lib.attn_head_chunk_plan.restype = C.c_int
    lib.attn_head_chunk_plan.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, P(C.c_int), C.c_int, P(C.c_int)]
    lib.attn_workspace_bytes.restype = C.c_int
    lib.attn_workspace_bytes.argtypes = [P(AttnArgs), C.c_int, P(C.c_size_t)]
    lib.attn_describe_plan.restype = C.c_int
    lib.attn_describe_plan.argtypes = [P(AttnArgs), C.c_int, P(PlanInfo)]
    for name in ("attn_prefill", "attn_decode", "attn_prefill_composed"):
        fn = getattr(lib, name)
        fn.restype = C.c_int
        fn.argtypes = [P(AttnArgs), C.c_void_p, C.c_size_t, C.c_void_p]
    lib.kv_append.restype = C.c_int
    lib.kv_append.argtypes = [P(KvAppendArgs), C.c_void_p]
    lib.attn_merge.restype = C.c_int
    lib.attn_merge.argtypes = [P(MergeArgs), C.c_void_p]
    lib.attn_prefill_partials.restype = C.c_int
    lib.attn_prefill_partials.argtypes = [P(AttnArgs), C.c_void_p, C.c_size_t, C.c_void_p, P(C.c_int32),
                                          P(C.c_int32), P(C.c_size_t), P(C.c_size_t)]
    lib.attn_decode_noalloc.restype = C.c_int
    lib.attn_decode_noalloc.argtypes = [P(AttnArgs), C.c_void_p]
    lib.kv_keep.restype = C.c_int
    lib.kv_keep.argtypes = [P(KvKeepArgs), C.c_void_p]
    lib.attn_prompt_policy.restype = C.c_int
    lib.attn_prompt_policy.argtypes = [P(PromptQuery), P(PromptChoice)]
    if lib.attn_abi_version() != ABI_VERSION:
        raise RuntimeError("libgqa_attn ABI version mismatch")
    for i, st in enumerate((AttnArgs, KvAppendArgs, MergeArgs, PlanInfo, KvKeepArgs, PromptQuery, PromptChoice)):
        if lib.attn_struct_size(i) != C.sizeof(st):
            raise RuntimeError(f"struct {st.__name__} size mismatch: lib {lib.attn_struct_size(i)} vs {C.sizeof(st)}")
    return lib
