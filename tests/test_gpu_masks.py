"""Additive masks with finite nonzero values on the HIP path (through the C ABI).

An additive mask adds its value to the score of every key it admits and hides the keys where it
holds -Inf ("Qwen head-chunked SDPA (#113)", "Exact scope found during review": the caller's mask
is passed to every chunk and broadcast).  A mask holding only 0 and -Inf cannot tell a correct
scaling of the value from a wrong one (0 times anything is 0), so every mask here holds N(0, 1)
values at the admitted keys.  Each case runs the mask through both of the main pass's paths (its
rows staged in LDS beside each K/V tile, and per-lane loads), which must give the same bits, on
the four-wavefront decode shape and the eight-wavefront verify and prompt shapes, with one KV
split (the gated output written by the main pass) and with the planned splits (partials and the
merge), in bf16 and fp16, against the float64 oracle.
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


# (name, B, Hq, Hkv, rows, kv_offset, op, mask batch extent, expected shape in the variant name)
CASES = [
    ("decode_4x1", 2, 16, 2, 6, 4106, ga._abi.OP_DECODE, 2, "4x1"),
    ("verify_8x1", 2, 16, 2, 32, 4080, ga._abi.OP_DECODE, 1, "8x1"),
    ("prompt_8x1", 1, 24, 4, 160, 352, ga._abi.OP_PREFILL, 1, "8x1"),
]


def _inputs(seed, B, Hq, Hkv, rows, off, dtype, Bm, kind):
    rng = syn.streams(seed)
    kv = off + rows
    qb = syn.normal_bits(rng["q"], (B, Hq, rows, 256), dtype)
    gb = syn.normal_bits(rng["gate"], (B, Hq, rows, 256), dtype)
    kb = syn.normal_bits(rng["k"], (B, Hkv, kv, 256), dtype)
    vb = syn.normal_bits(rng["v"], (B, Hkv, kv, 256), dtype)
    mb = syn.verify_mask(rng["mask"], rows=rows, kv_offset=off, heads=1, kind=kind, dtype=dtype, values="normal",
                         batch=Bm)
    return qb, kb, vb, gb, mb


def _mask_dev(mb, kind, dtype):
    if kind == "add":
        return to_dev(mb, dtype), syn.widen(mb, dtype)
    return torch.from_numpy(mb).cuda(), mb.astype(np.float64)


def _run(op, q, k, v, g, off, kv, m, n_splits):
    fn = ga.decode if op == ga._abi.OP_DECODE else ga.prefill
    out = torch.full_like(q, float("nan"))
    fn(q, k, v, g, kv_offset=off, kv_len=kv, mask=m, out=out, n_splits=n_splits)
    torch.cuda.synchronize()
    return out


@needs_gpu
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("n_splits", [0, 1])
@pytest.mark.parametrize("case", range(len(CASES)), ids=[c[0] for c in CASES])
@pytest.mark.parametrize("kind", ["add", "add_f32"])
def test_additive_mask_values_both_paths(case, n_splits, dtype, kind):
    name, B, Hq, Hkv, rows, off, op, Bm, shape = CASES[case]
    _say("mask values", name, dtype, kind, "n_splits", n_splits)
    kv = off + rows
    assert (kv * 2) % 16 == 0  # every mask row ends on a 16-byte chunk: the LDS path is possible
    qb, kb, vb, gb, mb = _inputs(5000 + case, B, Hq, Hkv, rows, off, dtype, Bm, kind)
    mdev, mref = _mask_dev(mb, kind, dtype)
    q, k, v, g = (to_dev(x, dtype) for x in (qb, kb, vb, gb))
    lds_stride, lane_stride = lds_and_lane_strides(kv, mdev.element_size())
    m_lds, m_lane = strided_mask(mdev, lds_stride), strided_mask(mdev, lane_stride)
    names = []
    for m in (m_lds, m_lane):
        a = ga._args(q, k, v, g, torch.empty_like(q), kv_offset=off, kv_len=kv, causal=True, scale=0.0,
                     head_chunk=0, n_splits=n_splits, mask=m)
        d = ga.describe_plan(a, op)
        names.append(d["variant_name"])
        assert (d["n_splits"] == 1) == (n_splits == 1), d
    # a workgroup of the prompt shape covers 43 mask rows: more than an LDS stage holds in fp32
    # words (32), so that case takes the per-lane loads on both storages
    staged = not (kind == "add_f32" and name == "prompt_8x1")
    assert ("ldsmask" in names[0]) == staged and "ldsmask" not in names[1], names
    assert all(shape in n for n in names), names
    out_lds = _run(op, q, k, v, g, off, kv, m_lds, n_splits)
    out_lane = _run(op, q, k, v, g, off, kv, m_lane, n_splits)
    assert torch.equal(out_lds.view(torch.int16), out_lane.view(torch.int16)), "mask paths differ"
    ref = reference.attention(*(syn.widen(x, dtype) for x in (qb, kb, vb, gb)), n_kv_heads=Hkv, kv_offset=off,
                              kv_len=kv, mask=mref, mask_kind="add")
    _say(assert_close(syn.widen(to_bits(out_lds), dtype), ref, f"mask values {name}"))
    # the values matter: the same call with the mask's finite entries zeroed lands elsewhere
    zeroed = np.where(np.isfinite(mref), 0.0, -np.inf)
    ref0 = reference.attention(*(syn.widen(x, dtype) for x in (qb, kb, vb, gb)), n_kv_heads=Hkv, kv_offset=off,
                               kv_len=kv, mask=zeroed, mask_kind="add")
    assert not compare(syn.widen(to_bits(out_lds), dtype), ref0)["ok"]


@needs_gpu
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("n_splits", [1, 0])
@pytest.mark.parametrize("kind", ["add", "add_f32"])
def test_nonfinite_repair_under_mask_values(dtype, n_splits, kind):
    # keys the mask hides from some rows hold +-Inf / NaN in V and +Inf in K: with one split the
    # main pass recomputes such pairs itself, with several the merge recomputes their rows, in
    # both cases reading the mask's values
    _say("repair under mask values", dtype, kind, n_splits)
    B, Hq, Hkv, rows, off = 2, 16, 2, 9, 4103
    kv = off + rows
    qb, kb, vb, gb, mb = _inputs(5100 + n_splits, B, Hq, Hkv, rows, off, dtype, 1, kind)
    mdev, mref = _mask_dev(mb, kind, dtype)
    # keys hidden from row 2 (so that row sees none of them; other rows see some)
    hidden = np.nonzero(mref[0, 0, 2] == -np.inf)[0]
    t = BITS[dtype]
    pick = np.random.default_rng(7).choice(hidden, size=12, replace=False)
    for i, j in enumerate(pick):
        vb[i % B, (i // B) % Hkv, j, (37 * i) % 256] = (t["+inf"], t["-inf"], t["nan"])[i % 3]
        kb[i % B, (i // B) % Hkv, j, (11 * i) % 256] = t["+inf"]
    q, k, v, g = (to_dev(x, dtype) for x in (qb, kb, vb, gb))
    ref = reference.attention(*(syn.widen(x, dtype) for x in (qb, kb, vb, gb)), n_kv_heads=Hkv, kv_offset=off,
                              kv_len=kv, mask=mref, mask_kind="add")
    blind = ~(mref[0, 0][:, pick] > -np.inf).any(axis=1)
    assert blind[2] and np.isfinite(ref[:, :, blind]).all()
    assert not np.isfinite(ref).all()  # rows that see a planted key carry it
    for hc in (0, 1, 8):
        out = ga.decode(q, k, v, g, kv_offset=off, mask=mdev, n_splits=n_splits, head_chunk=hc)
        res = compare(syn.widen(to_bits(out), dtype), ref)
        _say("head_chunk", hc, res)
        assert res["ok"], res
