"""Gated causal GQA attention at head_dim 256 for MI355X (gfx950): Python binding.

A thin layer over the C ABI of libgqa_attn.so (include/gqa_attn.h) with the same
names.  It turns torch tensors into pointers and strides, takes the stream from
torch, allocates the workspace through torch when the caller gives none, and
raises AttnError for a nonzero status.  Every step of the computation runs in
the library's HIP kernels; there is no fallback: if the library is not built,
every call raises.
"""

from __future__ import annotations

import ctypes as C

import torch

from . import _abi

__all__ = [
    "AttnError", "lib", "prefill", "prefill_partials", "prefill_composed", "decode", "decode_noalloc", "kv_append",
    "kv_keep", "merge", "head_chunk_plan",
    "workspace_bytes",
    "describe_plan", "plan_args", "variant_name", "prompt_prefill",
]

_LIB = None


class AttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_abi.STATUS.get(status, status)}: {message}")
        self.status = status
        self.name = _abi.STATUS.get(status, str(status))


def lib() -> C.CDLL:
    """The loaded library (loaded once)."""
    global _LIB
    if _LIB is None:
        _LIB = _abi.load()
    return _LIB


def _check(status: int) -> None:
    if status != _abi.OK:
        raise AttnError(status, lib().attn_strerror(status).decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return _abi.BF16
    if t.dtype == torch.float16:
        return _abi.F16
    raise TypeError(f"q/k/v/gate must be bfloat16 or float16, got {t.dtype}")


def _t4(t: torch.Tensor | None) -> _abi.Tensor:
    if t is None:
        return _abi.Tensor(None, 0, 0, 0)
    if t.dim() != 4:
        raise ValueError("tensors are 4-d [B, H, rows, head_dim]")
    if t.stride(3) != 1:
        raise ValueError("the last (head_dim) dimension must be contiguous")
    return _abi.Tensor(t.data_ptr(), t.stride(0), t.stride(1), t.stride(2))


def _stream_handle(t: torch.Tensor):
    if t.is_cuda:
        return C.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)
    return C.c_void_p(0)


def _mask_struct(mask, dtype_code: int) -> _abi.Mask:
    if mask is None:
        return _abi.Mask(_abi.MASK_NONE, 1, 1, 0, None, 0, 0, 0)
    if mask.dim() != 4:
        raise ValueError("mask must be 4-d [Bm, Hm, rows, >= kv_len]")
    if mask.stride(3) != 1:
        raise ValueError("the mask's key dimension must be contiguous")
    if mask.dtype in (torch.bool, torch.uint8):
        kind = _abi.MASK_BOOL_U8
    elif mask.dtype == torch.float32:
        kind = _abi.MASK_ADD_F32
    elif (mask.dtype == torch.bfloat16 and dtype_code == _abi.BF16) or (
            mask.dtype == torch.float16 and dtype_code == _abi.F16):
        kind = _abi.MASK_ADD
    else:
        raise TypeError(f"unsupported mask dtype {mask.dtype}")
    return _abi.Mask(kind, mask.shape[0], mask.shape[1], 0, mask.data_ptr(),
                     mask.stride(0) if mask.shape[0] > 1 else 0, mask.stride(1) if mask.shape[1] > 1 else 0,
                     mask.stride(2))


def _args(q, k_cache, v_cache, gate, out, *, kv_offset, kv_len, causal, scale, head_chunk, n_splits, mask):
    dt = _dtype_code(q)
    a = _abi.AttnArgs()
    a.dtype = dt
    a.B, a.Hq, a.rows, a.D = q.shape[0], q.shape[1], q.shape[2], q.shape[3]
    a.Hkv = k_cache.shape[1]
    a.kv_offset = int(kv_offset)
    a.kv_len = int(kv_len)
    a.capacity = k_cache.shape[2]
    a.scale = float(scale)
    a.causal = 1 if causal else 0
    a.head_chunk = int(head_chunk)
    a.n_splits = int(n_splits)
    a.q, a.gate, a.out = _t4(q), _t4(gate), _t4(out)
    a.k_cache, a.v_cache = _t4(k_cache), _t4(v_cache)
    a.mask = _mask_struct(mask, dt)
    for t in (k_cache, v_cache, gate, out):
        if t is not None and t.dtype != q.dtype:
            raise TypeError("q, k/v cache, gate and out must share one dtype")
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    return a


def _carry_args(a, carry):
    """Points attn_args `a` at the merge it carries: carry = (partial_o, partial_lse, partial_exp,
    gate, out) of an earlier prefill_partials call.  Returns what must stay alive with `a`."""
    if carry is None:
        return None
    po, pl, pe, cg, co = carry
    m, app = _merge_args(po, pl, cg, co, pe)
    a.carry = C.pointer(m)
    return (m, app)


def _run(op: int, q, k_cache, v_cache, gate, *, kv_offset: int, kv_len=None, causal=True, scale=0.0, head_chunk=0,
         n_splits=0, mask=None, out=None, workspace=None, append=None, carry=None):
    if kv_len is None:
        kv_len = kv_offset + q.shape[2]
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    a = _args(q, k_cache, v_cache, gate, out, kv_offset=kv_offset, kv_len=kv_len, causal=causal, scale=scale,
              head_chunk=head_chunk, n_splits=n_splits, mask=mask)
    app = None
    if append is not None:  # (k_new, v_new, k_cache, v_cache, kv_offset) of a kv_append the call carries
        app = _append_args(*append)
        a.append = C.pointer(app)
    _keep = _carry_args(a, carry)
    L = lib()
    need = C.c_size_t(0)
    _check(L.attn_workspace_bytes(C.byref(a), op, C.byref(need)))
    if workspace is None and need.value:
        workspace = torch.empty(need.value, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    fn = {_abi.OP_PREFILL: L.attn_prefill, _abi.OP_DECODE: L.attn_decode,
          _abi.OP_COMPOSED: L.attn_prefill_composed}[op]
    _check(fn(C.byref(a), ws_ptr, ws_len, _stream_handle(q)))
    return out


def prefill_partials(q, k_cache, v_cache, gate, *, kv_offset: int, workspace, kv_len=None, causal=True, scale=0.0,
                     head_chunk=0, n_splits=0, mask=None, out=None, append=None, carry=None):
    """attn_prefill_partials: the main pass only.  Returns (out, partials).  partials is None when
    the plan kept the keys in one chunk (out is then final); otherwise it is (partial_o,
    partial_lse, partial_exp), views into `workspace` (a uint8 tensor) to finish with
    merge(partial_o, partial_lse, gate, out, partial_exp=partial_exp) on a stream ordered after
    this one, or by a later call's carry.  partial_o [C, B, Hq, rows, D] is fp32 with
    partial_exp None (small plans), or fp16 with partial_exp [C, B, Hq, rows] int32, the partial
    being partial_o times 2^partial_exp (merge_args partial_kind 0 and 1).
    append = (k_new, v_new, k_cache, v_cache, kv_offset): a kv_append the call carries;
    carry = (partial_o, partial_lse, partial_exp, gate, out) of an EARLIER call: its merge, done
    by this call (attn_args carry: inside the main pass's launch where that has idle CUs); its
    partials must not lie in `workspace`."""
    if kv_len is None:
        kv_len = kv_offset + q.shape[2]
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    a = _args(q, k_cache, v_cache, gate, out, kv_offset=kv_offset, kv_len=kv_len, causal=causal, scale=scale,
              head_chunk=head_chunk, n_splits=n_splits, mask=mask)
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor")
    app = None
    if append is not None:
        app = _append_args(*append)
        a.append = C.pointer(app)
    _keep = _carry_args(a, carry)
    n, kind, off, eoff = C.c_int32(0), C.c_int32(0), C.c_size_t(0), C.c_size_t(0)
    _check(lib().attn_prefill_partials(C.byref(a), workspace.data_ptr(), workspace.numel(), _stream_handle(q),
                                       C.byref(n), C.byref(kind), C.byref(off), C.byref(eoff)))
    if n.value == 1:
        return out, None
    B, Hq, rows, D = q.shape
    cnt = n.value * B * Hq * rows
    pl = workspace[off.value:off.value + cnt * 4].view(torch.float32).view(n.value, B, Hq, rows)
    if kind.value == 0:
        po = workspace[:cnt * D * 4].view(torch.float32).view(n.value, B, Hq, rows, D)
        return out, (po, pl, None)
    po = workspace[:cnt * D * 2].view(torch.float16).view(n.value, B, Hq, rows, D)
    pe = workspace[eoff.value:eoff.value + cnt * 4].view(torch.int32).view(n.value, B, Hq, rows)
    return out, (po, pl, pe)


def prefill(q, k_cache, v_cache, gate, *, kv_offset: int, kv_len=None, causal=True, scale=0.0, head_chunk=0,
            n_splits=0, mask=None, out=None, workspace=None, append=None, carry=None):
    """attn_prefill: q/gate [B, Hq, rows, D], caches [B, Hkv, capacity, D] (D = 256, 128 or 64); returns out.
    append = (k_new, v_new, k_cache, v_cache, kv_offset): a kv_append the call carries (attn_args
    append: in the merge's launch when the keys are split), e.g. the next query block's rows.
    carry: an earlier call's merge, as for prefill_partials."""
    return _run(_abi.OP_PREFILL, q, k_cache, v_cache, gate, kv_offset=kv_offset, kv_len=kv_len, causal=causal,
                scale=scale, head_chunk=head_chunk, n_splits=n_splits, mask=mask, out=out, workspace=workspace,
                append=append, carry=carry)


def decode(q, k_cache, v_cache, gate, *, kv_offset: int, kv_len=None, causal=True, scale=0.0, head_chunk=0,
           n_splits=0, mask=None, out=None, workspace=None):
    """attn_decode: 1..32 rows; head_chunk 0 = the policy, k = chunks of k heads."""
    return _run(_abi.OP_DECODE, q, k_cache, v_cache, gate, kv_offset=kv_offset, kv_len=kv_len, causal=causal,
                scale=scale, head_chunk=head_chunk, n_splits=n_splits, mask=mask, out=out, workspace=workspace)


def decode_noalloc(q, k_cache, v_cache, gate, *, out, kv_offset: int, kv_len=None, causal=True, scale=0.0,
                   head_chunk=0, n_splits=0, mask=None):
    """attn_decode_noalloc: attn_decode with the split partials in the library's own device
    scratch (64 MiB per GPU); the call allocates nothing, so `out` is the caller's."""
    if kv_len is None:
        kv_len = kv_offset + q.shape[2]
    a = _args(q, k_cache, v_cache, gate, out, kv_offset=kv_offset, kv_len=kv_len, causal=causal, scale=scale,
              head_chunk=head_chunk, n_splits=n_splits, mask=mask)
    _check(lib().attn_decode_noalloc(C.byref(a), _stream_handle(q)))
    return out


def prefill_composed(q, k_cache, v_cache, gate, *, kv_offset: int, kv_len=None, causal=True, scale=0.0, out=None,
                     workspace=None):
    """attn_prefill_composed: the composed (materialised-score) route for the same block, for
    comparison with attn_prefill; no mask.  workspace: a uint8 device tensor of at least
    workspace_bytes(args, OP_COMPOSED) bytes (allocated here when None)."""
    return _run(_abi.OP_COMPOSED, q, k_cache, v_cache, gate, kv_offset=kv_offset, kv_len=kv_len, causal=causal,
                scale=scale, out=out, workspace=workspace)


def kv_append(k_new, v_new, k_cache, v_cache, *, kv_offset: int) -> None:
    """kv_append: copy [B, Hkv, rows, D] rows into the caches at kv_offset, bit for bit."""
    a = _append_args(k_new, v_new, k_cache, v_cache, kv_offset)
    _check(lib().kv_append(C.byref(a), _stream_handle(k_new)))


def _append_args(k_new, v_new, k_cache, v_cache, kv_offset):
    a = _abi.KvAppendArgs()
    a.dtype = _dtype_code(k_new)
    a.B, a.Hkv, a.rows, a.D = k_new.shape[0], k_new.shape[1], k_new.shape[2], k_new.shape[3]
    a.kv_offset = int(kv_offset)
    a.capacity = k_cache.shape[2]
    a.k_new, a.v_new, a.k_cache, a.v_cache = _t4(k_new), _t4(v_new), _t4(k_cache), _t4(v_cache)
    for t in (v_new, k_cache, v_cache):
        if t.dtype != k_new.dtype:
            raise TypeError("k/v rows and caches must share one dtype")
    if v_new.shape != k_new.shape or v_cache.shape != k_cache.shape:
        raise ValueError("k and v shapes differ")
    if k_cache.shape[0] != k_new.shape[0] or k_cache.shape[1] != k_new.shape[1]:
        raise ValueError("cache and new rows disagree on batch or KV heads")
    return a



def kv_keep(k_cache, v_cache, *, kv_offset: int, rows: int, keep) -> None:
    """kv_keep: in each batch entry, move the kept rows of the verify block at kv_offset (rows
    rows) to kv_offset, kv_offset + 1, ... in row order, bit for bit.  keep[b] is a bitmask
    (bit r = keep row r) or a sequence of row indices."""
    masks = []
    for k in keep:
        if isinstance(k, int):
            masks.append(k)
        else:
            m = 0
            for r in k:
                m |= 1 << int(r)
            masks.append(m)
    if len(masks) != k_cache.shape[0]:
        raise ValueError("keep needs one entry per batch entry")
    arr = (C.c_uint32 * max(1, len(masks)))(*[m & 0xFFFFFFFF for m in masks])
    if any(m >> 32 for m in masks):
        raise ValueError("keep bits past row 31")
    a = _abi.KvKeepArgs()
    a.dtype = _dtype_code(k_cache)
    a.B, a.Hkv, a.D, a.rows = k_cache.shape[0], k_cache.shape[1], k_cache.shape[3], int(rows)
    a.kv_offset, a.capacity = int(kv_offset), k_cache.shape[2]
    a.keep = C.cast(arr, C.POINTER(C.c_uint32))
    a.k_cache, a.v_cache = _t4(k_cache), _t4(v_cache)
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("k_cache and v_cache differ")
    _check(lib().kv_keep(C.byref(a), _stream_handle(k_cache)))

def _merge_args(partial_o, partial_lse, gate, out, partial_exp=None, append=None):
    """MergeArgs for these partials (and the ctypes objects it points to, kept alive with it)."""
    if partial_o.dtype not in (torch.float32, torch.float16) or partial_lse.dtype != torch.float32:
        raise TypeError("partial_o is float32 or float16, partial_lse float32")
    fp16 = partial_o.dtype == torch.float16
    if fp16 != (partial_exp is not None):
        raise ValueError("partial_exp goes with float16 partials, and only with them")
    if fp16 and (partial_exp.dtype != torch.int32 or tuple(partial_exp.shape) != tuple(partial_o.shape[:4])
                 or not partial_exp.is_contiguous()):
        raise ValueError("partial_exp is a contiguous int32 [C, B, Hq, rows]")
    if not partial_o.is_contiguous() or not partial_lse.is_contiguous():
        raise ValueError("partials must be contiguous")
    a = _abi.MergeArgs()
    a.dtype = _dtype_code(gate)
    a.n_chunks, a.B, a.Hq, a.rows, a.D = partial_o.shape
    a.partial_kind = 1 if fp16 else 0
    if tuple(partial_lse.shape) != tuple(partial_o.shape[:4]) or tuple(gate.shape) != tuple(partial_o.shape[1:]):
        raise ValueError("partials and gate disagree in shape")
    a.partial_o, a.partial_lse = partial_o.data_ptr(), partial_lse.data_ptr()
    a.partial_exp = partial_exp.data_ptr() if fp16 else None
    a.gate, a.out = _t4(gate), _t4(out)
    app = None
    if append is not None:
        k_new, v_new, k_cache, v_cache, kv_offset = append
        app = _append_args(k_new, v_new, k_cache, v_cache, kv_offset)
        a.append = C.pointer(app)
    return a, app


def merge(partial_o, partial_lse, gate, out=None, partial_exp=None, append=None):
    """attn_merge: partial_o [C, B, Hq, rows, D] (D 256, 128 or 64) fp32, or fp16 with
    partial_exp [C, B, Hq, rows] int32 (the form prefill_partials returns: the partial is
    partial_o times 2^partial_exp); partial_lse [C, B, Hq, rows] fp32 (natural log).
    append = (k_new, v_new, k_cache, v_cache, kv_offset): a kv_append of those rows carried by
    the same launch (it must not touch what the merge reads or writes)."""
    if out is None:
        out = torch.empty_like(gate, memory_format=torch.contiguous_format)
    a, _app = _merge_args(partial_o, partial_lse, gate, out, partial_exp, append)
    _check(lib().attn_merge(C.byref(a), _stream_handle(gate)))
    return out


def head_chunk_plan(rows: int, n_q_heads: int, n_kv_heads: int, enabled: bool = True) -> list:
    """Chunk sizes (heads) of one KV group under the head-chunk rule."""
    sizes = (C.c_int * _abi.MAX_CHUNKS)()
    n = C.c_int(0)
    _check(lib().attn_head_chunk_plan(rows, n_q_heads, n_kv_heads, 1 if enabled else 0, sizes, _abi.MAX_CHUNKS,
                                      C.byref(n)))
    return list(sizes[:n.value])


_FAKE = 1 << 20  # an aligned, never dereferenced address for shape-only planning


def plan_args(*, B: int, Hq: int, Hkv: int, rows: int, kv_offset: int, kv_len=None, capacity=None, causal=True,
              head_chunk=0, n_splits=0, dtype="bf16", mask_kind=_abi.MASK_NONE, Bm=1, Hm=1, D=256):
    """An AttnArgs for planning only (workspace_bytes / describe_plan): pointers are placeholders."""
    if kv_len is None:
        kv_len = kv_offset + rows
    a = _abi.AttnArgs()
    a.dtype = _abi.BF16 if dtype == "bf16" else _abi.F16
    a.B, a.Hq, a.Hkv, a.D, a.rows = B, Hq, Hkv, D, rows
    a.kv_offset, a.kv_len = kv_offset, kv_len
    a.capacity = capacity if capacity is not None else kv_len
    a.scale, a.causal, a.head_chunk, a.n_splits = 0.0, 1 if causal else 0, head_chunk, n_splits
    t = _abi.Tensor(_FAKE, Hq * rows * D, rows * D, D)
    a.q = a.gate = a.out = t
    a.k_cache = a.v_cache = _abi.Tensor(_FAKE, Hkv * a.capacity * D, a.capacity * D, D)
    a.mask = _abi.Mask(mask_kind, Bm, Hm, 0, _FAKE if mask_kind else None, 0, 0, kv_len)
    return a


def workspace_bytes(args: _abi.AttnArgs, op: int = _abi.OP_PREFILL) -> int:
    n = C.c_size_t(0)
    _check(lib().attn_workspace_bytes(C.byref(args), op, C.byref(n)))
    return n.value


def describe_plan(args: _abi.AttnArgs, op: int = _abi.OP_PREFILL) -> dict:
    info = _abi.PlanInfo()
    _check(lib().attn_describe_plan(C.byref(args), op, C.byref(info)))
    d = {name: getattr(info, name) for name, _ in _abi.PlanInfo._fields_ if name != "chunk_sizes"}
    d["chunk_sizes"] = list(info.chunk_sizes[:info.n_head_chunks])
    d["variant_name"] = variant_name(info.variant)
    return d


def variant_name(variant: int) -> str:
    return lib().attn_variant_name(variant).decode()


def device_key(device=None):
    """(gfx number, compute units) of a CUDA device for attn_prompt_policy; (0, 0) without one."""
    if not torch.cuda.is_available():
        return 0, 0
    props = torch.cuda.get_device_properties(device if device is not None else torch.cuda.current_device())
    arch = getattr(props, "gcnArchName", "") or ""
    digits = arch[3:].split(":")[0] if arch.startswith("gfx") else ""
    gfx = int(digits) if digits.isdigit() else 0
    return gfx, int(props.multi_processor_count)


def prompt_policy(*, D: int, B: int, Hq: int, Hkv: int, n_tokens: int, dtype: str = "bf16", gfx=None,
                  n_cus=None) -> dict:
    """attn_prompt_policy: route and query-block size for a prompt of n_tokens rows.  gfx and
    n_cus default to those of the current device."""
    if gfx is None or n_cus is None:
        dg, dc = device_key()
        gfx = dg if gfx is None else gfx
        n_cus = dc if n_cus is None else n_cus
    qy = _abi.PromptQuery(D, B, Hq, Hkv, n_tokens, _abi.BF16 if dtype == "bf16" else _abi.F16, gfx, n_cus)
    ch = _abi.PromptChoice()
    _check(lib().attn_prompt_policy(C.byref(qy), C.byref(ch)))
    return {"route": {_abi.OP_PREFILL: "fused", _abi.OP_COMPOSED: "composed"}[ch.route], "q_block": ch.q_block,
            "qualified": bool(ch.qualified), "reason": _abi.POLICY_REASON[ch.reason], "n_calls": ch.n_calls}


def prompt_prefill(q, k, v, gate, k_cache, v_cache, *, q_block: int = 0, kv_offset: int = 0, out=None,
                   workspace=None, head_chunk=0, n_splits=0, overlap_merge=False, composed=False, carry_merge=True):
    """A prompt in query blocks: each block's K/V rows are appended to the caches (kv_append),
    then the block runs attn_prefill (attn_prefill_composed with composed=True).  On the fused
    route without overlap_merge the first block's rows go by kv_append and every block's call
    carries the next block's rows (attn_args append).  With carry_merge (the default) each block
    runs attn_prefill_partials into one of two workspaces, in turn, and carries the previous
    block's merge (attn_args carry; inside its main pass's launch where that has idle CUs), the
    last block's merge following on its own: one launch per block.  Without it each block runs
    attn_prefill, its append in the merge's launch when the keys are split.

    q/gate [B, Hq, N, D] and k/v [B, Hkv, N, D] hold the prompt (positions kv_offset ..
    kv_offset + N - 1); k_cache/v_cache have room for them.  Block i attends to the cache plus
    itself ("perf(qwen36): qualify M4 head-256 attention", Summary: query blocks of 128 or 512).
    q_block = 0 takes the block size (and route) of attn_prompt_policy for this device.
    With overlap_merge, each block's merge runs on a second stream beside the next block's main
    pass (two workspaces, alternating); the caller's stream waits for the last merge.
    """
    N = q.shape[2]
    if q_block == 0:
        pol = prompt_policy(D=q.shape[3], B=q.shape[0], Hq=q.shape[1], Hkv=k.shape[1], n_tokens=N,
                            dtype="bf16" if q.dtype == torch.bfloat16 else "f16", gfx=None, n_cus=None)
        q_block = pol["q_block"]
        composed = composed or pol["route"] == "composed"
    if q_block < 1:
        raise ValueError("q_block must be positive (or 0 for the prompt policy)")
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if composed:
        if overlap_merge:
            raise ValueError("the composed route has no merge to overlap")
        for s in range(0, N, q_block):
            e = min(s + q_block, N)
            kv_append(k[:, :, s:e], v[:, :, s:e], k_cache, v_cache, kv_offset=kv_offset + s)
            prefill_composed(q[:, :, s:e], k_cache, v_cache, gate[:, :, s:e], kv_offset=kv_offset + s,
                             kv_len=kv_offset + e, out=out[:, :, s:e], workspace=workspace)
        return out
    if workspace is None:
        need = 0
        for s in range(0, N, q_block):
            rows = min(q_block, N - s)
            a = plan_args(B=q.shape[0], Hq=q.shape[1], Hkv=k.shape[1], rows=rows, kv_offset=kv_offset + s,
                          capacity=k_cache.shape[2], head_chunk=head_chunk, n_splits=n_splits, D=q.shape[3])
            need = max(need, workspace_bytes(a, _abi.OP_PREFILL))
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if not overlap_merge:
        # each block's call carries the next block's append
        kv_append(k[:, :, :min(q_block, N)], v[:, :, :min(q_block, N)], k_cache, v_cache, kv_offset=kv_offset)

        def nxt(e):
            return (k[:, :, e:min(e + q_block, N)], v[:, :, e:min(e + q_block, N)], k_cache, v_cache,
                    kv_offset + e) if e < N else None

        if not carry_merge:
            for s in range(0, N, q_block):
                e = min(s + q_block, N)
                prefill(q[:, :, s:e], k_cache, v_cache, gate[:, :, s:e], kv_offset=kv_offset + s,
                        kv_len=kv_offset + e, out=out[:, :, s:e], workspace=workspace, head_chunk=head_chunk,
                        n_splits=n_splits, append=nxt(e))
            return out
        # blocks whose plan carries work in the main pass's launch (attn_plan_info carry_blocks)
        # take the previous block's merge there; the others run attn_prefill, their append in the
        # merge's launch
        spaces = [workspace, torch.empty_like(workspace)]
        pending = None  # a block's partials, gate and out, merged by the next call
        for i, s in enumerate(range(0, N, q_block)):
            e = min(s + q_block, N)
            a = plan_args(B=q.shape[0], Hq=q.shape[1], Hkv=k.shape[1], rows=e - s, kv_offset=kv_offset + s,
                          capacity=k_cache.shape[2], head_chunk=head_chunk, n_splits=n_splits, D=q.shape[3],
                          dtype="bf16" if q.dtype == torch.bfloat16 else "f16")
            if describe_plan(a)["carry_blocks"] > 0:
                _, parts = prefill_partials(q[:, :, s:e], k_cache, v_cache, gate[:, :, s:e], kv_offset=kv_offset + s,
                                            kv_len=kv_offset + e, out=out[:, :, s:e], workspace=spaces[i % 2],
                                            head_chunk=head_chunk, n_splits=n_splits, append=nxt(e), carry=pending)
                pending = (*parts, gate[:, :, s:e], out[:, :, s:e])
                continue
            if pending is not None:
                merge(pending[0], pending[1], pending[3], out=pending[4], partial_exp=pending[2])
                pending = None
            prefill(q[:, :, s:e], k_cache, v_cache, gate[:, :, s:e], kv_offset=kv_offset + s, kv_len=kv_offset + e,
                    out=out[:, :, s:e], workspace=spaces[i % 2], head_chunk=head_chunk, n_splits=n_splits,
                    append=nxt(e))
        if pending is not None:
            merge(pending[0], pending[1], pending[3], out=pending[4], partial_exp=pending[2])
        return out
    main = torch.cuda.current_stream(q.device)
    side = merge_stream(q.device)
    spaces = [workspace, torch.empty_like(workspace)]
    merged = [None, None]  # per workspace: the event after the merge that last read it
    for i, s in enumerate(range(0, N, q_block)):
        e = min(s + q_block, N)
        slot = i % 2
        if merged[slot] is not None:
            main.wait_event(merged[slot])
        kv_append(k[:, :, s:e], v[:, :, s:e], k_cache, v_cache, kv_offset=kv_offset + s)
        _, parts = prefill_partials(q[:, :, s:e], k_cache, v_cache, gate[:, :, s:e], kv_offset=kv_offset + s,
                                    kv_len=kv_offset + e, out=out[:, :, s:e], workspace=spaces[slot],
                                    head_chunk=head_chunk, n_splits=n_splits)
        if parts is not None:
            ready = torch.cuda.Event()
            ready.record(main)
            side.wait_event(ready)
            with torch.cuda.stream(side):
                merge(parts[0], parts[1], gate[:, :, s:e], out=out[:, :, s:e], partial_exp=parts[2])
            merged[slot] = torch.cuda.Event()
            merged[slot].record(side)
    main.wait_stream(side)
    return out


_MERGE_STREAMS = {}


def merge_stream(device):
    """The second stream prompt_prefill's overlapped merges run on: one per device, made once,
    so that it keeps the hardware queue it was given (a stream made per call can land on the
    queue of the caller's stream, which runs the two in turn)."""
    dev = torch.device(device)
    idx = dev.index if dev.index is not None else torch.cuda.current_device()
    if idx not in _MERGE_STREAMS:
        _MERGE_STREAMS[idx] = torch.cuda.Stream(device=idx)
    return _MERGE_STREAMS[idx]
