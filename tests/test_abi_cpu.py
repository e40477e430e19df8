"""The C-ABI library on the CPU: it loads, exports what include/gqa_attn.h declares, plans
like the oracle's head-chunk rule, and rejects every invalid argument with its status code
before touching a device (no kernel is launched by any test here)."""

import ctypes as C
import os
import re

import pytest

import gqa_causal_attention_attn_amd as ga
from gqa_causal_attention_attn_amd import _abi
from oracle import plan as oplan

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    with open(os.path.join(ROOT, "include", "gqa_attn.h")) as f:
        text = f.read()
    body = text.split('extern "C" {', 1)[1]
    return set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(\w+)\(", body, flags=re.M))


def test_library_exports_every_declared_symbol():
    lib = ga.lib()
    declared = _declared_functions()
    assert declared == set(_abi.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_struct_sizes_and_version():
    lib = ga.lib()
    assert lib.attn_abi_version() == _abi.ABI_VERSION
    for i, st in enumerate((_abi.AttnArgs, _abi.KvAppendArgs, _abi.MergeArgs, _abi.PlanInfo, _abi.KvKeepArgs,
                            _abi.PromptQuery, _abi.PromptChoice)):
        assert lib.attn_struct_size(i) == C.sizeof(st)
    assert lib.attn_struct_size(99) == 0
    for code in list(_abi.STATUS) + [12345]:
        assert lib.attn_strerror(code)


def test_chunk_plan_matches_oracle_rule():
    for rows in range(0, 41):
        for hq in range(0, 34):
            for hkv in range(0, 18):
                valid = rows >= 1 and hq > 0 and hkv > 0 and hq % hkv == 0
                if not valid:
                    with pytest.raises(ga.AttnError):
                        ga.head_chunk_plan(rows, hq, hkv)
                    continue
                assert ga.head_chunk_plan(rows, hq, hkv) == oplan.head_chunk_sizes(rows, hq, hkv)
                assert ga.head_chunk_plan(rows, hq, hkv, enabled=False) == [hq // hkv]


def test_plan_splits_do_not_depend_on_head_chunk():
    for rows, G in ((1, 6), (4, 6), (6, 6), (9, 8), (17, 8), (32, 8), (5, 8)):
        base = None
        for hc in range(0, G + 1):
            a = ga.plan_args(B=2, Hq=2 * G, Hkv=2, rows=rows, kv_offset=4097, head_chunk=hc)
            d = ga.describe_plan(a, _abi.OP_DECODE)
            key = (d["n_splits"], d["keys_per_split"])
            base = base or key
            assert key == base
            if hc == 0:
                assert d["chunk_sizes"] == oplan.head_chunk_sizes(rows, 2 * G, 2)
            elif hc:
                assert d["chunk_sizes"][0] == hc and sum(d["chunk_sizes"]) == G


def test_plan_covers_every_key():
    # the split plan reaches every key below the causal bound of the block
    for rows, off in ((128, 0), (128, 32640), (512, 16384), (1, 4096), (32, 32768), (7, 63)):
        a = ga.plan_args(B=1, Hq=24, Hkv=4, rows=rows, kv_offset=off)
        d = ga.describe_plan(a, _abi.OP_PREFILL)
        assert d["n_splits"] * d["keys_per_split"] >= off + rows
        assert (d["n_splits"] - 1) * d["keys_per_split"] < off + rows
        assert d["keys_per_split"] % d["keys_per_tile"] == 0


def _good(**kw):
    return ga.plan_args(**{**dict(B=1, Hq=24, Hkv=4, rows=4, kv_offset=100), **kw})


REJECT = [
    ("null args", None, "ATTN_E_NULL"),
    ("dtype", dict(_set={"dtype": 7}), "ATTN_E_DTYPE"),
    ("zero kv heads", dict(Hkv=0), "ATTN_E_HEADS"),
    ("zero q heads", dict(Hq=0), "ATTN_E_HEADS"),
    ("uneven groups", dict(Hq=10, Hkv=4), "ATTN_E_HEADS"),
    ("batch 0", dict(B=0), "ATTN_E_HEADS"),
    ("group over 64", dict(Hq=130, Hkv=2), "ATTN_E_HEADS"),
    ("head dim 96", dict(D=96), "ATTN_E_HEAD_DIM"),
    ("rows 0", dict(rows=0), "ATTN_E_ROWS"),
    ("negative offset", dict(kv_offset=-1, kv_len=3), "ATTN_E_KV"),
    ("kv_len short of causal rows", dict(kv_len=102), "ATTN_E_KV"),
    ("kv_len beyond capacity", dict(kv_len=104, capacity=103), "ATTN_E_KV"),
    ("kv_len 0", dict(_set={"kv_len": 0}), "ATTN_E_KV"),
    ("head_chunk > G", dict(head_chunk=7), "ATTN_E_HEAD_CHUNK"),
    ("head_chunk < 0", dict(head_chunk=-1), "ATTN_E_HEAD_CHUNK"),
    ("negative splits", dict(n_splits=-2), "ATTN_E_ARG"),
    ("nan scale", dict(_set={"scale": float("nan")}), "ATTN_E_ARG"),
    ("null q", dict(_tensor=("q", 0, None)), "ATTN_E_NULL"),
    ("null v cache", dict(_tensor=("v_cache", 0, None)), "ATTN_E_NULL"),
    ("misaligned q", dict(_tensor=("q", 0, (1 << 20) + 8)), "ATTN_E_LAYOUT"),
    ("odd row stride", dict(_tensor=("k_cache", 3, 260)), "ATTN_E_LAYOUT"),
    ("mask kind", dict(mask_kind=9), "ATTN_E_MASK"),
    ("mask batch extent", dict(mask_kind=1, Bm=2), "ATTN_E_MASK"),
    ("mask head extent", dict(mask_kind=2, Hm=6), "ATTN_E_MASK"),
    ("mask null", dict(_mask_null=True), "ATTN_E_MASK"),
]


def _build(spec):
    if spec is None:
        return None
    spec = dict(spec)
    setv = spec.pop("_set", {})
    tensor = spec.pop("_tensor", None)
    mask_null = spec.pop("_mask_null", False)
    a = _good(**spec)
    for k, v in setv.items():
        setattr(a, k, v)
    if tensor:
        name, field, val = tensor
        t = getattr(a, name)
        if field == 0:
            t.ptr = val
        else:
            t.stride_row = val
        setattr(a, name, t)
    if mask_null:
        a.mask.kind = 1
        a.mask.ptr = None
    return a


@pytest.mark.parametrize("name,spec,status", REJECT, ids=[r[0] for r in REJECT])
@pytest.mark.parametrize("op", [_abi.OP_PREFILL, _abi.OP_DECODE, _abi.OP_COMPOSED])
def test_rejections(name, spec, status, op):
    lib = ga.lib()
    a = _build(spec)
    ptr = C.byref(a) if a is not None else None
    n = C.c_size_t(0)
    want = _abi.STATUS_CODE[status]
    assert lib.attn_workspace_bytes(ptr, op, C.byref(n)) == want
    fn = {_abi.OP_PREFILL: lib.attn_prefill, _abi.OP_DECODE: lib.attn_decode,
          _abi.OP_COMPOSED: lib.attn_prefill_composed}[op]
    assert fn(ptr, None, 0, None) == want


@pytest.mark.parametrize("D", [64, 128])
def test_other_head_dims(D):
    # head dims 64 and 128 run on the same main pass as 256 (16 KiB tiles of 8192 / D keys),
    # masks included, and on the composed route; the append takes them; any other head dim fails
    # closed everywhere
    lib = ga.lib()
    a = _good(D=D)
    n = C.c_size_t(1)
    for op in (_abi.OP_PREFILL, _abi.OP_DECODE):
        assert lib.attn_workspace_bytes(C.byref(a), op, C.byref(n)) == 0 and n.value == 0  # no split here
        info = ga.describe_plan(a, op)
        assert info["variant_name"] == f"fwd_mfma32x32x16_bf16_4x1_d{D}" and info["n_splits"] == 1
        assert info["keys_per_tile"] == 8192 // D
    assert lib.attn_workspace_bytes(C.byref(a), _abi.OP_COMPOSED, C.byref(n)) == 0 and n.value > 0
    m = _good(D=D, mask_kind=2)
    m.mask.ptr = 1 << 20
    for op in (_abi.OP_PREFILL, _abi.OP_DECODE):
        assert lib.attn_workspace_bytes(C.byref(m), op, C.byref(n)) == 0
        assert ga.describe_plan(m, op)["variant_name"] == f"fwd_mfma32x32x16_bf16_maskadd_4x1_ldswords_d{D}"
    assert lib.attn_workspace_bytes(C.byref(m), _abi.OP_COMPOSED, C.byref(n)) == _abi.STATUS_CODE["ATTN_E_MASK"]
    odd = _good(D=96)
    for op in (_abi.OP_PREFILL, _abi.OP_DECODE, _abi.OP_COMPOSED):
        assert lib.attn_workspace_bytes(C.byref(odd), op, C.byref(n)) == _abi.STATUS_CODE["ATTN_E_HEAD_DIM"]
    t = _abi.Tensor(1 << 20, 4 * 16 * 96, 16 * 96, 96)
    ap = _abi.KvAppendArgs()
    ap.dtype, ap.B, ap.Hkv, ap.rows, ap.D, ap.kv_offset, ap.capacity = 0, 1, 4, 2, 96, 0, 16
    ap.k_new, ap.v_new, ap.k_cache, ap.v_cache = t, t, t, t
    assert lib.kv_append(C.byref(ap), None) == _abi.STATUS_CODE["ATTN_E_HEAD_DIM"]


@pytest.mark.parametrize("D", [64, 128, 256])
def test_tile_keys_per_head_dim(D):
    # the main pass moves 16 KiB K and V tiles at every head dim: 8192 / D keys a tile; splits
    # are whole tiles, the workspace holds a partial row of D values per (split, b, h, row), fp32
    # below 8 MiB of them and fp16 from there, then an fp32 lse per row and (fp16 only) an int32
    # exponent per row, each part rounded up to 256 bytes
    lib = ga.lib()
    T = 8192 // D
    r256 = lambda x: (x + 255) // 256 * 256
    for B, Hq, Hkv, rows, off, asked in ((2, 16, 2, 1, 32767, 0), (1, 24, 4, 512, 32256, 0), (1, 24, 4, 4, 100, 0),
                                         (1, 8, 2, 33, 1000, 3), (1, 16, 2, 32, 32768, 0)):
        for op in (_abi.OP_PREFILL, _abi.OP_DECODE):
            if op == _abi.OP_DECODE and rows > 32:
                continue
            a = _good(D=D, B=B, Hq=Hq, Hkv=Hkv, rows=rows, kv_offset=off, n_splits=asked)
            info = ga.describe_plan(a, op)
            S, kps = info["n_splits"], info["keys_per_split"]
            assert info["keys_per_tile"] == T and kps % T == 0
            assert S * kps >= off + rows and (S - 1) * kps < off + rows
            if asked:
                assert S <= asked
            nrow = S * B * Hq * rows
            half = nrow * D * 4 >= 8 << 20
            want = 0 if S == 1 else r256(nrow * D * (2 if half else 4)) + (2 if half else 1) * r256(nrow * 4)
            assert ga.workspace_bytes(a, op) == want and info["workspace_bytes"] == want
            assert info["partial_kind"] == (1 if S > 1 and half else 0)
            if S > 1:
                fn = lib.attn_prefill if op == _abi.OP_PREFILL else lib.attn_decode
                assert fn(C.byref(a), C.c_void_p(1 << 20), want - 1, None) == _abi.STATUS_CODE["ATTN_E_WORKSPACE"]
                assert fn(C.byref(a), None, want, None) == _abi.STATUS_CODE["ATTN_E_WORKSPACE"]
                assert fn(C.byref(a), C.c_void_p((1 << 20) + 8), want, None) == _abi.STATUS_CODE["ATTN_E_LAYOUT"]


def test_composed_workspace_and_rejections():
    # the composed route: scores fp32 + weights 16-bit per (b, h, row, key of the range rounded
    # up to 32) + 1 / l per row, each part rounded up to 256 bytes; no mask; no plan to describe
    lib = ga.lib()
    r256 = lambda x: (x + 255) // 256 * 256
    for rows, off in ((5, 3), (512, 32256), (1, 0)):
        a = _good(rows=rows, kv_offset=off)
        kvp = (off + rows + 31) // 32 * 32
        n = a.B * a.Hq * rows
        assert ga.workspace_bytes(a, _abi.OP_COMPOSED) == r256(n * kvp * 4) + r256(n * kvp * 2) + r256(n * 4)
    a = _good(rows=5, kv_offset=3)
    need = ga.workspace_bytes(a, _abi.OP_COMPOSED)
    assert lib.attn_prefill_composed(C.byref(a), C.c_void_p(1 << 20), need - 1, None) == \
        _abi.STATUS_CODE["ATTN_E_WORKSPACE"]
    assert lib.attn_prefill_composed(C.byref(a), None, need, None) == _abi.STATUS_CODE["ATTN_E_WORKSPACE"]
    assert lib.attn_prefill_composed(C.byref(a), C.c_void_p((1 << 20) + 8), need, None) == \
        _abi.STATUS_CODE["ATTN_E_LAYOUT"]
    m = _good(rows=5, kv_offset=3, mask_kind=2)
    m.mask.ptr = 1 << 20
    n = C.c_size_t(0)
    assert lib.attn_workspace_bytes(C.byref(m), _abi.OP_COMPOSED, C.byref(n)) == _abi.STATUS_CODE["ATTN_E_MASK"]
    assert lib.attn_workspace_bytes(C.byref(m), _abi.OP_PREFILL, C.byref(n)) == 0
    info = _abi.PlanInfo()
    assert lib.attn_describe_plan(C.byref(a), _abi.OP_COMPOSED, C.byref(info)) == _abi.STATUS_CODE["ATTN_E_ARG"]


def test_decode_rejects_more_than_32_rows_but_prefill_accepts():
    lib = ga.lib()
    a = _good(rows=33)
    n = C.c_size_t(0)
    assert lib.attn_workspace_bytes(C.byref(a), _abi.OP_DECODE, C.byref(n)) == _abi.STATUS_CODE["ATTN_E_ROWS"]
    assert lib.attn_workspace_bytes(C.byref(a), _abi.OP_PREFILL, C.byref(n)) == 0


def test_small_workspace_is_rejected_before_launch():
    lib = ga.lib()
    a = _good(rows=1, kv_offset=32768)
    need = ga.workspace_bytes(a, _abi.OP_DECODE)
    assert need > 0
    assert lib.attn_decode(C.byref(a), C.c_void_p(1 << 20), need - 1, None) == _abi.STATUS_CODE["ATTN_E_WORKSPACE"]
    assert lib.attn_decode(C.byref(a), None, need, None) == _abi.STATUS_CODE["ATTN_E_WORKSPACE"]


def test_append_and_merge_rejections():
    lib = ga.lib()
    t = _abi.Tensor(1 << 20, 4 * 16 * 256, 16 * 256, 256)
    a = _abi.KvAppendArgs(0, 1, 4, 256, 2, 0, 15, 16, t, t, t, t)
    assert lib.kv_append(C.byref(a), None) == _abi.STATUS_CODE["ATTN_E_KV"]
    a.kv_offset = 14
    a.D = 96
    assert lib.kv_append(C.byref(a), None) == _abi.STATUS_CODE["ATTN_E_HEAD_DIM"]
    a.D = 256
    a.dtype = 3
    assert lib.kv_append(C.byref(a), None) == _abi.STATUS_CODE["ATTN_E_DTYPE"]
    a.dtype = 0
    a.k_new = _abi.Tensor(None, 0, 0, 0)
    assert lib.kv_append(C.byref(a), None) == _abi.STATUS_CODE["ATTN_E_NULL"]
    assert lib.kv_append(None, None) == _abi.STATUS_CODE["ATTN_E_NULL"]
    m = _abi.MergeArgs(0, 0, 1, 2, 3, 256, 1 << 20, 1 << 20, t, t)
    assert lib.attn_merge(C.byref(m), None) == _abi.STATUS_CODE["ATTN_E_ARG"]
    m.n_chunks = 2
    m.partial_lse = (1 << 20) + 2
    assert lib.attn_merge(C.byref(m), None) == _abi.STATUS_CODE["ATTN_E_LAYOUT"]
    m.partial_lse = 1 << 20
    m.partial_kind = 2  # fp32 (0) and fp16 with exponents (1) only
    assert lib.attn_merge(C.byref(m), None) == _abi.STATUS_CODE["ATTN_E_ARG"]
    m.partial_kind = 1  # fp16 partials need their exponents, 4-byte aligned
    assert lib.attn_merge(C.byref(m), None) == _abi.STATUS_CODE["ATTN_E_NULL"]
    m.partial_exp = (1 << 20) + 2
    assert lib.attn_merge(C.byref(m), None) == _abi.STATUS_CODE["ATTN_E_LAYOUT"]
    m.partial_kind = 0
    # a carried append is checked as kv_append checks it, before anything is enqueued
    app = _abi.KvAppendArgs(0, 1, 4, 256, 2, 0, 15, 16, t, t, t, t)  # rows 15..16 past capacity 16
    m.append = C.pointer(app)
    assert lib.attn_merge(C.byref(m), None) == _abi.STATUS_CODE["ATTN_E_KV"]
    app.kv_offset, app.D = 14, 96
    assert lib.attn_merge(C.byref(m), None) == _abi.STATUS_CODE["ATTN_E_HEAD_DIM"]
    app.D, app.k_new = 256, _abi.Tensor(None, 0, 0, 0)
    assert lib.attn_merge(C.byref(m), None) == _abi.STATUS_CODE["ATTN_E_NULL"]
    m.append = None
    m.partial_o = None
    assert lib.attn_merge(C.byref(m), None) == _abi.STATUS_CODE["ATTN_E_NULL"]
    for D in (96, 32, 512):  # head dims 256, 128 and 64 only
        m2 = _abi.MergeArgs(0, 2, 1, 2, 3, D, 1 << 20, 1 << 20, t, t)
        assert lib.attn_merge(C.byref(m2), None) == _abi.STATUS_CODE["ATTN_E_HEAD_DIM"]


def test_keep_rejections():
    lib = ga.lib()
    t = _abi.Tensor(1 << 20, 2 * 40 * 256, 40 * 256, 256)
    masks = (C.c_uint32 * 2)(0b101, 0b1)
    keep = C.cast(masks, C.POINTER(C.c_uint32))
    a = _abi.KvKeepArgs(0, 2, 2, 256, 3, 0, 36, 40, keep, t, t)
    a.kv_offset = 38
    assert lib.kv_keep(C.byref(a), None) == _abi.STATUS_CODE["ATTN_E_KV"]
    a.kv_offset = 36
    a.rows = 33
    assert lib.kv_keep(C.byref(a), None) == _abi.STATUS_CODE["ATTN_E_ROWS"]
    a.rows = 0
    assert lib.kv_keep(C.byref(a), None) == _abi.STATUS_CODE["ATTN_E_ROWS"]
    a.rows = 2                                   # bit 2 of 0b101 is past the block
    assert lib.kv_keep(C.byref(a), None) == _abi.STATUS_CODE["ATTN_E_ARG"]
    a.rows = 3
    a.B = 65
    assert lib.kv_keep(C.byref(a), None) == _abi.STATUS_CODE["ATTN_E_HEADS"]
    a.B = 2
    a.D = 128
    assert lib.kv_keep(C.byref(a), None) == _abi.STATUS_CODE["ATTN_E_HEAD_DIM"]
    a.D = 256
    a.k_cache = _abi.Tensor((1 << 20) + 8, 2 * 40 * 256, 40 * 256, 256)
    assert lib.kv_keep(C.byref(a), None) == _abi.STATUS_CODE["ATTN_E_LAYOUT"]
    a.keep = None
    assert lib.kv_keep(C.byref(a), None) == _abi.STATUS_CODE["ATTN_E_NULL"]
    assert lib.kv_keep(None, None) == _abi.STATUS_CODE["ATTN_E_NULL"]


def test_carried_append_is_checked_before_the_call():
    # attn_prefill / attn_decode with an append to carry: the append's own errors come back and
    # nothing runs (no device here: a launch would fail with ATTN_E_HIP instead)
    lib = ga.lib()
    t = _abi.Tensor(1 << 20, 4 * 16 * 256, 16 * 256, 256)
    app = _abi.KvAppendArgs(0, 1, 4, 256, 2, 0, 15, 16, t, t, t, t)  # rows 15..16 past capacity 16
    for op, fn in ((_abi.OP_PREFILL, lib.attn_prefill), (_abi.OP_DECODE, lib.attn_decode)):
        a = _good()
        a.append = C.pointer(app)
        need = ga.workspace_bytes(a, op)
        assert fn(C.byref(a), C.c_void_p(1 << 20) if need else None, need, None) == _abi.STATUS_CODE["ATTN_E_KV"]
        app.dtype = 9
        assert fn(C.byref(a), C.c_void_p(1 << 20) if need else None, need, None) == _abi.STATUS_CODE["ATTN_E_DTYPE"]
        app.dtype = 0


@pytest.mark.parametrize("D", [256, 128])
def test_carry_blocks_of_prompt_plans(D):
    # a 512-row block of the 24/4-head prompt (12,288 rows, 240 workgroups over 5 splits) carries
    # work in its main pass's launch (attn_args carry, the append of attn_prefill_partials) on the
    # 16 CUs left idle once 10 x 16 x its tiles per split reach its rows: from 77 tiles per split
    # (381 tiles of keys) on; earlier blocks carry nothing.  A 1024-row block (192 workgroups over
    # 2 splits, 24,576 rows) carries from 39 tiles per split on, on 64 idle CUs.
    T = 8192 // D
    cases = [(512, 0, 0), (512, 380 * T - 512, 0), (512, 385 * T - 512, 16), (512, 32768 - 512, 16),
             (1024, 76 * T - 1024, 0), (1024, 78 * T - 1024, 64)]
    for rows, off, want in cases:
        d = ga.describe_plan(_good(rows=rows, kv_offset=off, capacity=32768, D=D))
        assert d["carry_blocks"] == want, (rows, off, d)
        if want:
            assert d["partial_kind"] == 1 and d["grid_blocks"] + want == 256
    # decode rows never carry
    assert ga.describe_plan(_good(rows=32, kv_offset=32768, capacity=40000, D=D), _abi.OP_DECODE)["carry_blocks"] == 0


def test_carried_merge_is_checked_before_the_call():
    # attn_args carry: attn_merge's checks, no append of its own, partials clear of the call's
    # workspace; each error comes back before anything runs (no device here: a launch would
    # fail with ATTN_E_HIP instead)
    lib = ga.lib()
    t = _abi.Tensor(1 << 40, 24 * 512 * 256, 512 * 256, 256)
    a = _good(rows=512, kv_offset=32256, capacity=32768)
    need = ga.workspace_bytes(a, _abi.OP_PREFILL)
    ws = 1 << 36
    m = _abi.MergeArgs(0, 5, 1, 24, 512, 256, 1 << 38, (1 << 38) + (1 << 30), t, t)
    m.partial_kind, m.partial_exp = 1, (1 << 38) + (1 << 31)
    a.carry = C.pointer(m)
    n, kind, off, eoff = C.c_int32(0), C.c_int32(0), C.c_size_t(0), C.c_size_t(0)
    outs = [C.byref(n), C.byref(kind), C.byref(off), C.byref(eoff)]
    S = _abi.STATUS_CODE

    def run():
        return lib.attn_prefill_partials(C.byref(a), ws, need, None, *outs)
    m.partial_lse = ws + 4096  # inside this call's workspace
    assert run() == S["ATTN_E_ARG"]
    m.partial_lse = (1 << 38) + 2
    assert run() == S["ATTN_E_LAYOUT"]
    m.partial_lse = (1 << 38) + (1 << 30)
    m.partial_kind = 2
    assert run() == S["ATTN_E_ARG"]
    m.partial_kind, m.partial_exp = 1, None
    assert run() == S["ATTN_E_NULL"]
    m.partial_exp = (1 << 38) + (1 << 31)
    m.D = 96
    assert run() == S["ATTN_E_HEAD_DIM"]
    m.D = 256
    app = _abi.KvAppendArgs(0, 1, 4, 256, 512, 0, 32256, 32768, t, t, t, t)
    m.append = C.pointer(app)  # a carried merge carries no append of its own
    assert run() == S["ATTN_E_ARG"]
    assert lib.attn_prefill(C.byref(a), ws, need, None) == S["ATTN_E_ARG"]
    m.append = None
    comp = _good(rows=64, kv_offset=0)
    comp.carry = C.pointer(m)
    m.partial_o = None
    assert lib.attn_prefill_composed(C.byref(comp), ws, 1 << 30, None) == S["ATTN_E_NULL"]


def test_prefill_partials_needs_its_outputs():
    lib = ga.lib()
    a = _good(rows=512, kv_offset=4096)
    n, kind, off, eoff = C.c_int32(7), C.c_int32(7), C.c_size_t(7), C.c_size_t(7)
    E = _abi.STATUS_CODE["ATTN_E_NULL"]
    outs = [C.byref(n), C.byref(kind), C.byref(off), C.byref(eoff)]
    for i in range(4):
        assert lib.attn_prefill_partials(C.byref(a), None, 0, None, *[None if j == i else x for j, x in
                                                                       enumerate(outs)]) == E
    need = ga.workspace_bytes(a, _abi.OP_PREFILL)
    assert need > 0
    st = lib.attn_prefill_partials(C.byref(a), None, 0, None, *outs)
    assert st == _abi.STATUS_CODE["ATTN_E_WORKSPACE"]


def test_launch_size_limits_are_rejected_by_planning_and_run_alike():
    # a decode whose merge would exceed a launch (4.19M rows x 16 wavefronts: more than 64 chunks),
    # at head dims 256 and 64: the planning calls reject it as the run would, before anything is
    # enqueued (100 splits asked for: 65 chunks of 2 tiles)
    a = ga.plan_args(B=4096, Hq=32, Hkv=1, rows=32, kv_offset=4096, n_splits=100)
    for fn in (lambda: ga.workspace_bytes(a, _abi.OP_DECODE), lambda: ga.describe_plan(a, _abi.OP_DECODE)):
        with pytest.raises(ga.AttnError) as e:
            fn()
        assert e.value.name == "ATTN_E_ARG"
    assert ga.lib().attn_decode(C.byref(a), None, 0, None) == _abi.STATUS_CODE["ATTN_E_ARG"]
    a.n_splits = 8  # one wavefront a row: fits
    assert ga.workspace_bytes(a, _abi.OP_DECODE) > 0
    a.n_splits = 40  # one wavefront a row with 64 slots (fp16 partials): fits
    assert ga.workspace_bytes(a, _abi.OP_DECODE) > 0
    s = ga.plan_args(B=4096, Hq=32, Hkv=1, rows=32, kv_offset=8192, n_splits=100, D=64)
    with pytest.raises(ga.AttnError):
        ga.workspace_bytes(s, _abi.OP_DECODE)
    assert ga.lib().attn_decode(C.byref(s), None, 0, None) == _abi.STATUS_CODE["ATTN_E_ARG"]
    s.n_splits = 8
    assert ga.workspace_bytes(s, _abi.OP_DECODE) > 0


def test_strerror_names_the_head_dims():
    msg = ga.lib().attn_strerror(_abi.STATUS_CODE["ATTN_E_HEAD_DIM"]).decode()
    assert "256" in msg and "128" in msg and "64" in msg


# The prompt policy ("perf(qwen36): qualify M4 head-256 attention", Summary and the review comment
# on eligibility): measured on gfx950 with 256 compute units, keyed on the device and head dim.
MI355X = {"gfx": 950, "n_cus": 256}


@pytest.mark.parametrize("D", [256, 128, 64])
def test_prompt_policy_table_on_the_measured_device(D):
    pol = lambda **kw: ga.prompt_policy(D=D, **{**MI355X, **kw})
    # 24 query heads over 4 (G 6): blocks of 8192 rows past 2048 tokens; 16 over 2 (G 8): 4096
    assert pol(B=1, Hq=24, Hkv=4, n_tokens=32768) == {"route": "fused", "q_block": 8192, "qualified": True,
                                                      "reason": "table", "n_calls": 4}
    assert pol(B=1, Hq=16, Hkv=2, n_tokens=32768) == {"route": "fused", "q_block": 4096, "qualified": True,
                                                      "reason": "table", "n_calls": 8}
    assert pol(B=1, Hq=16, Hkv=2, n_tokens=8192)["q_block"] == 4096
    assert pol(B=1, Hq=24, Hkv=4, n_tokens=8192)["q_block"] == 8192
    # at most the prompt, and short prompts in one call
    assert pol(B=1, Hq=24, Hkv=4, n_tokens=5000)["q_block"] == 5000
    for n in (1, 100, 2048):
        c = pol(B=1, Hq=24, Hkv=4, n_tokens=n)
        assert (c["q_block"], c["reason"], c["n_calls"]) == (n, "whole_prompt", 1)
    # the group size decides the row (G 1 and 6 take 8192, G 7 and 16 take 4096)
    assert pol(B=1, Hq=4, Hkv=4, n_tokens=32768)["q_block"] == 8192
    assert pol(B=1, Hq=7, Hkv=1, n_tokens=32768)["q_block"] == 4096
    assert pol(B=1, Hq=32, Hkv=2, n_tokens=32768)["q_block"] == 4096
    # the batch divides the block (down to 512 rows)
    assert pol(B=2, Hq=24, Hkv=4, n_tokens=32768)["q_block"] == 4096
    assert pol(B=64, Hq=24, Hkv=4, n_tokens=32768)["q_block"] == 512
    c = pol(B=1, Hq=24, Hkv=4, n_tokens=32769)
    assert (c["q_block"], c["n_calls"]) == (8192, 5)


@pytest.mark.parametrize("gfx,n_cus", [(942, 304), (950, 32), (950, 0), (0, 0), (1100, 256)])
def test_prompt_policy_other_devices_get_the_default(gfx, n_cus):
    # an MI300X, one 32-CU partition of an MI355X, or an unknown device: blocks of 512, unqualified
    for n in (100, 32768):
        c = ga.prompt_policy(D=256, B=1, Hq=24, Hkv=4, n_tokens=n, gfx=gfx, n_cus=n_cus)
        assert c == {"route": "fused", "q_block": min(512, n), "qualified": False, "reason": "unqualified_default",
                     "n_calls": -(-n // min(512, n))}


def test_prompt_policy_rejections():
    lib = ga.lib()
    ok = dict(D=256, B=1, Hq=24, Hkv=4, n_tokens=32768, dtype=_abi.BF16, gfx=950, n_cus=256)
    ch = _abi.PromptChoice()
    assert lib.attn_prompt_policy(C.byref(_abi.PromptQuery(**ok)), C.byref(ch)) == _abi.OK
    assert lib.attn_prompt_policy(None, C.byref(ch)) == _abi.STATUS_CODE["ATTN_E_NULL"]
    assert lib.attn_prompt_policy(C.byref(_abi.PromptQuery(**ok)), None) == _abi.STATUS_CODE["ATTN_E_NULL"]
    for bad, code in [(dict(D=96), "ATTN_E_HEAD_DIM"), (dict(B=0), "ATTN_E_HEADS"), (dict(Hq=5, Hkv=2), "ATTN_E_HEADS"),
                      (dict(Hkv=0), "ATTN_E_HEADS"), (dict(n_tokens=0), "ATTN_E_ROWS"), (dict(dtype=7), "ATTN_E_DTYPE")]:
        q = _abi.PromptQuery(**{**ok, **bad})
        assert lib.attn_prompt_policy(C.byref(q), C.byref(ch)) == _abi.STATUS_CODE[code], bad


def test_probe_library_exports_every_declared_symbol():
    # include/gqa_probes.h: the benchmark's achievable-peak probes; loaded, never called here
    from gqa_causal_attention_attn_amd import build as gbuild

    with open(os.path.join(ROOT, "include", "gqa_probes.h")) as f:
        body = f.read().split('extern "C" {', 1)[1]
    declared = set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(\w+)\(", body, flags=re.M))
    assert declared == {"gqa_probe_mfma", "gqa_probe_mfma_mix", "gqa_probe_lds", "gqa_probe_read",
                        "gqa_probe_tile_stream"}
    lib = C.CDLL(gbuild.PROBES_LIB)
    for name in declared:
        assert hasattr(lib, name), name


def test_full_head_mask_window_choice():
    # A full-head mask (a row per query head) is staged in LDS one dword per key of each pair's
    # own row only when every workgroup holds one column block of at most 1024 / T pairs (T keys
    # per tile: 32 pairs at head dim 256, 16 at 128, 8 at 64); otherwise each lane loads its words.
    # A mask the same for every head keeps the word window of its query rows.
    cases = [  # rows, Hq, Hkv, Hm, D, head_chunk, expected layout marker
        (1, 16, 2, 16, 256, 0, "_ldspairwords"),
        (4, 16, 2, 16, 256, 0, "_ldspairwords"),   # 8 heads x 4 rows = 32 pairs
        (5, 24, 4, 24, 256, 0, "_ldspairwords"),   # 6 x 5 = 30
        (6, 16, 2, 16, 256, 0, None),              # chunks [5, 3]: two blocks
        (4, 16, 2, 16, 256, 4, None),              # forced chunks of 4 heads: two blocks
        (32, 16, 2, 16, 256, 0, None),             # eight blocks
        (2, 16, 2, 16, 128, 0, "_ldspairwords"),   # 16 pairs at head dim 128
        (4, 16, 2, 16, 128, 0, None),              # 32 pairs > 16
        (1, 16, 2, 16, 64, 0, "_ldspairwords"),    # 8 pairs at head dim 64
        (2, 16, 2, 16, 64, 0, None),               # 16 pairs > 8
        (4, 16, 2, 1, 256, 0, "_ldswords"),        # broadcast over heads
    ]
    for rows, Hq, Hkv, Hm, D, hc, marker in cases:
        for mk in (_abi.MASK_BOOL_U8, _abi.MASK_ADD, _abi.MASK_ADD_F32):
            a = ga.plan_args(B=2, Hq=Hq, Hkv=Hkv, rows=rows, kv_offset=32768, mask_kind=mk, Hm=Hm, D=D,
                             head_chunk=hc)
            name = ga.describe_plan(a, _abi.OP_DECODE)["variant_name"]
            if marker:
                assert marker in name, (rows, Hq, Hkv, Hm, D, hc, name)
            else:
                assert "lds" not in name, (rows, Hq, Hkv, Hm, D, hc, name)
    # every variant id the library names decodes to its own name, and the per-pair layout exists
    # for every shape at every head dim
    lib = ga.lib()
    names = [lib.attn_variant_name(i).decode() for i in range(3 * 128)]
    known = [n for n in names if n != "unknown"]
    assert len(known) == len(set(known))
    for shape in ("_4x1", "_8x1", "_8x1_stream"):
        for dim in ("", "_d128", "_d64"):
            assert f"fwd_mfma32x32x16_bf16_maskadd{shape}_ldspairwords{dim}" in known
