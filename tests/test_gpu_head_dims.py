"""Head dims 128 and 64 on the main pass: masks, the nonfinite repair and head chunks, in bf16
and fp16, through the C ABI against the float64 oracle.

The main pass runs every head dim with the same tiling; a K/V tile holds 16 KiB (8192 / D keys),
so a head-broadcast mask is staged in LDS one dword per key for workgroups covering up to
1024 / tile keys mask rows (16 at D 128, 8 at D 64) and read per lane beyond that.  The mask kinds
and head chunks follow "Qwen head-chunked SDPA (#113)" ("Exact scope found during review"): the
caller's mask goes to every chunk, and every chunking gives the same bits.  Keys a row cannot see
never reach its output, whatever they hold (TensorFold PR #1009, attention kernel-contract
commit).  Scale 1 / sqrt(D).
"""

import numpy as np
import pytest
import torch

import gqa_causal_attention_attn_amd as ga
from oracle import reference
from synth import inputs as syn
from tests.gpu_util import lds_and_lane_strides, strided_mask, to_bits, to_dev
from tests.parity import assert_close, compare

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")

BITS = {"bf16": {"+inf": 0x7F80, "-inf": 0xFF80, "nan": 0x7FC0},
        "f16": {"+inf": 0x7C00, "-inf": 0xFC00, "nan": 0x7E00}}


def _say(*a):
    print(*a, flush=True)


def _case(seed, *, B, Hq, Hkv, rows, off, D, dtype):
    rng = syn.streams(seed)
    kv = off + rows
    qb = syn.normal_bits(rng["q"], (B, Hq, rows, D), dtype)
    gb = syn.normal_bits(rng["gate"], (B, Hq, rows, D), dtype)
    kb = syn.normal_bits(rng["k"], (B, Hkv, kv, D), dtype)
    vb = syn.normal_bits(rng["v"], (B, Hkv, kv, D), dtype)
    return qb, kb, vb, gb, rng


def _ref(qb, kb, vb, gb, dtype, Hkv, off, kv, **kw):
    return reference.attention(*(syn.widen(x, dtype) for x in (qb, kb, vb, gb)), n_kv_heads=Hkv, kv_offset=off,
                               kv_len=kv, **kw)


def _variant(q, k, v, g, off, kv, m, op=ga._abi.OP_DECODE, head_chunk=0, n_splits=0):
    a = ga._args(q, k, v, g, torch.empty_like(q), kv_offset=off, kv_len=kv, causal=True, scale=0.0,
                 head_chunk=head_chunk, n_splits=n_splits, mask=m)
    return ga.describe_plan(a, op)["variant_name"]


@needs_gpu
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("rows", [1, 4, 9, 17, 32])
def test_verify_with_mask_values(D, dtype, rows):
    # batch 2, 16 query heads over 2 KV heads, rows appended at offset 4097, a broadcast additive
    # mask with N(0, 1) values at the admitted keys; every head chunk gives the policy's bits
    _say("verify", D, dtype, rows)
    B, Hq, Hkv, off = 2, 16, 2, 4097
    kv = off + rows
    qb, kb, vb, gb, rng = _case(6000 + D + rows, B=B, Hq=Hq, Hkv=Hkv, rows=rows, off=off, D=D, dtype=dtype)
    mb = syn.verify_mask(rng["mask"], rows=rows, kv_offset=off, heads=1, kind="add", dtype=dtype, values="normal")
    q, k, v, g, m = (to_dev(x, dtype) for x in (qb, kb, vb, gb, mb))
    vn = _variant(q, k, v, g, off, kv, m)
    assert vn.endswith(f"_d{D}"), vn
    if rows <= 1024 // (8192 // D):  # mask rows a workgroup may cover for the word layout
        assert "ldswords" in vn, vn
    outs = {hc: to_bits(ga.decode(q, k, v, g, kv_offset=off, mask=m, head_chunk=hc)) for hc in (0, 1, 2, 3, 5, 8)}
    for hc, o in outs.items():
        assert np.array_equal(o, outs[0]), f"head_chunk {hc} differs from the policy"
    ref = _ref(qb, kb, vb, gb, dtype, Hkv, off, kv, mask=syn.widen(mb, dtype), mask_kind="add")
    _say(assert_close(syn.widen(outs[0], dtype), ref, f"verify D={D}"))
    # the values matter: zeroing the mask's finite entries moves the oracle away from the result
    zeroed = np.where(np.isfinite(syn.widen(mb, dtype)), 0.0, -np.inf)
    ref0 = _ref(qb, kb, vb, gb, dtype, Hkv, off, kv, mask=zeroed, mask_kind="add")
    assert not compare(syn.widen(outs[0], dtype), ref0)["ok"]


@needs_gpu
@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("kind", ["bool", "add", "f32"])
def test_mask_paths_agree(D, kind):
    # a head-broadcast mask at a 64-byte aligned row stride and at an odd one (both staged in LDS
    # as words), and a copy per query head (per-lane loads): the same bits, and the oracle's
    _say("mask paths", D, kind)
    B, Hq, Hkv, rows = 2, 16, 2, 6
    off = 4112 - rows
    kv = off + rows
    qb, kb, vb, gb, rng = _case(6100 + D, B=B, Hq=Hq, Hkv=Hkv, rows=rows, off=off, D=D, dtype="bf16")
    mb = syn.verify_mask(rng["mask"], rows=rows, kv_offset=off, heads=1,
                         kind={"bool": "bool", "add": "add", "f32": "add_f32"}[kind],
                         values="zero" if kind == "bool" else "normal")
    if kind == "add":
        mdev, mref, mk = to_dev(mb), syn.widen(mb), "add"
    elif kind == "bool":
        mdev, mref, mk = torch.from_numpy(mb).cuda(), mb.astype(bool), "bool"
    else:
        mdev, mref, mk = torch.from_numpy(mb).cuda(), mb.astype(np.float64), "add"
    lds_stride, lane_stride = lds_and_lane_strides(kv, mdev.element_size())
    storages = [strided_mask(mdev, lds_stride), strided_mask(mdev, lane_stride),
                mdev.expand(1, Hq, rows, kv).contiguous()]
    q, k, v, g = (to_dev(x) for x in (qb, kb, vb, gb))
    names = [_variant(q, k, v, g, off, kv, m) for m in storages]
    assert "ldswords" in names[0] and "ldswords" in names[1] and "lds" not in names[2], names
    outs = [ga.decode(q, k, v, g, kv_offset=off, mask=m) for m in storages]
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))
    ref = _ref(qb, kb, vb, gb, "bf16", Hkv, off, kv, mask=mref, mask_kind=mk)
    _say(assert_close(syn.widen(to_bits(outs[0])), ref, f"mask paths D={D} {kind}"))


@needs_gpu
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("n_splits", [1, 0])
def test_prompt_block_with_mask(D, dtype, n_splits):
    # 96 causal rows at offset 416 (24 query heads over 4 KV heads) under a broadcast fp32 additive
    # mask: workgroups of 32 rows, past the word window, so the mask is read per lane
    _say("prompt mask", D, dtype, n_splits)
    B, Hq, Hkv, rows, off = 1, 24, 4, 96, 416
    kv = off + rows
    qb, kb, vb, gb, rng = _case(6200 + D, B=B, Hq=Hq, Hkv=Hkv, rows=rows, off=off, D=D, dtype=dtype)
    mb = syn.verify_mask(rng["mask"], rows=rows, kv_offset=off, heads=1, kind="add_f32", values="normal")
    q, k, v, g = (to_dev(x, dtype) for x in (qb, kb, vb, gb))
    m = torch.from_numpy(mb).cuda()
    assert "lds" not in _variant(q, k, v, g, off, kv, m, op=ga._abi.OP_PREFILL, n_splits=n_splits)
    out = ga.prefill(q, k, v, g, kv_offset=off, kv_len=kv, mask=m, n_splits=n_splits)
    torch.cuda.synchronize()
    ref = _ref(qb, kb, vb, gb, dtype, Hkv, off, kv, mask=mb.astype(np.float64), mask_kind="add")
    _say(assert_close(syn.widen(to_bits(out), dtype), ref, f"prompt mask D={D}"))


@needs_gpu
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("rows,n_splits", [(1, 0), (9, 0), (9, 1), (17, 0)])
def test_nonfinite_hidden_keys(D, dtype, rows, n_splits):
    # keys the mask hides from some rows hold +-Inf / NaN in V and +Inf in K: one split recomputes
    # such pairs in the main pass, several recompute the rows in the merge; rows that see none of
    # them stay finite, the others follow float64 (head chunks compared with the oracle each)
    _say("nonfinite verify", D, dtype, rows, n_splits)
    B, Hq, Hkv, off = 2, 16, 2, 4097
    kv = off + rows
    qb, kb, vb, gb, rng = _case(6300 + D + rows, B=B, Hq=Hq, Hkv=Hkv, rows=rows, off=off, D=D, dtype=dtype)
    mb = syn.verify_mask(rng["mask"], rows=rows, kv_offset=off, heads=1, kind="add", dtype=dtype, values="normal")
    mref = syn.widen(mb, dtype)
    hidden = np.nonzero(mref[0, 0].min(axis=0) == -np.inf)[0]
    assert hidden.size > 20
    t = BITS[dtype]
    pick = np.random.default_rng(rows + D).choice(hidden, size=12, replace=False)
    for i, j in enumerate(pick):
        vb[i % B, (i // B) % Hkv, j, (37 * i) % D] = (t["+inf"], t["-inf"], t["nan"])[i % 3]
        kb[i % B, (i // B) % Hkv, j, (11 * i) % D] = t["+inf"]
    q, k, v, g, m = (to_dev(x, dtype) for x in (qb, kb, vb, gb, mb))
    ref = _ref(qb, kb, vb, gb, dtype, Hkv, off, kv, mask=mref, mask_kind="add")
    blind = ~(mref[0, 0][:, pick] > -np.inf).any(axis=1)
    assert np.isfinite(ref[:, :, blind]).all()
    for hc in (0, 1, 3):
        res = compare(syn.widen(to_bits(ga.decode(q, k, v, g, kv_offset=off, mask=m, n_splits=n_splits,
                                                  head_chunk=hc)), dtype), ref)
        _say("head_chunk", hc, res)
        assert res["ok"], res


@needs_gpu
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("n_splits", [1, 3])
def test_nonfinite_future_keys_in_a_prompt(D, dtype, n_splits):
    # 128 causal rows in one block, 24 query heads over 4 KV heads; values planted in diagonal
    # tiles, where earlier rows share the key's tile but must not see it
    _say("nonfinite prompt", D, dtype, n_splits)
    B, Hq, Hkv, N = 1, 24, 4, 128
    qb, kb, vb, gb, _ = _case(6400 + D, B=B, Hq=Hq, Hkv=Hkv, rows=N, off=0, D=D, dtype=dtype)
    t = BITS[dtype]
    vb[0, 1, 50, 7] = t["+inf"]
    vb[0, 2, 70, D - 5] = t["-inf"]
    vb[0, 3, 90, D // 2] = t["nan"]
    kb[0, 0, 60, 3] = t["+inf"]
    vb[0, 0, 127, :] = t["nan"]
    q, k, v, g = (to_dev(x, dtype) for x in (qb, kb, vb, gb))
    ref = _ref(qb, kb, vb, gb, dtype, Hkv, 0, N)
    assert np.isfinite(ref[0, 6:12, :50]).all() and np.isposinf(ref[0, 6:12, 50:, 7]).all()
    for hc in (0, 1, 4):
        out = ga.prefill(q, k, v, g, kv_offset=0, kv_len=N, n_splits=n_splits, head_chunk=hc)
        torch.cuda.synchronize()
        res = compare(syn.widen(to_bits(out), dtype), ref)
        _say("head_chunk", hc, res)
        assert res["ok"], res
