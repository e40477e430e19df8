"""Additive masks with finite nonzero values on the HIP path (through the C ABI).

An additive mask adds its value to the score of every key it admits and hides the keys where it
holds -Inf ("Qwen head-chunked SDPA (#113)", "Exact scope found during review": the caller's mask
is passed to every chunk and broadcast).  A mask holding only 0 and -Inf cannot tell a correct
scaling of the value from a wrong one (0 times anything is 0), so every mask here holds N(0, 1)
values at the admitted keys.  Each case runs the mask through the main pass's paths (its window
staged in LDS beside each K/V tile as one dword per key or as 16-byte row chunks, and per-lane
loads), which must give the same bits, on the four-wavefront decode shape and the eight-wavefront
verify and prompt shapes, with one KV split (the gated output written by the main pass) and with
the planned splits (partials and the merge), in bf16 and fp16, against the float64 oracle.

A full-head mask (a row per query head) whose workgroups hold a single column block of pairs
stages each pair's own mask row in the same word window; it must match the oracle, the per-lane
loads of the same mask and, for a mask the same for every head, that mask's own word window.
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


# (name, B, Hq, Hkv, rows, kv_offset, op, mask batch extent, shape in the variant name, mask rows a
# workgroup covers)
CASES = [
    ("decode_4x1", 2, 16, 2, 6, 4106, ga._abi.OP_DECODE, 2, "4x1", 6),
    ("verify_8x1", 2, 16, 2, 32, 4080, ga._abi.OP_DECODE, 1, "8x1_stream", 32),
    ("prompt_8x1_32rows", 1, 16, 2, 96, 416, ga._abi.OP_PREFILL, 1, "8x1", 32),
    ("prompt_8x1_43rows", 1, 24, 4, 160, 352, ga._abi.OP_PREFILL, 1, "8x1", 43),
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


def _expected_layouts(window, kind, name):
    """Variant-name markers of the three storages: 64-byte aligned rows, rows at an odd stride
    (both the same for every head), and a copy per query head (per-lane loads)."""
    if window <= 32:
        return "ldswords", "ldswords", None
    esz = {"add": 2, "add_f32": 4}[kind]
    rows16 = "_8x1" in name and window <= 4096 // (32 * esz)
    return ("ldsrows" if rows16 else None), None, None


@needs_gpu
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("n_splits", [0, 1])
@pytest.mark.parametrize("case", range(len(CASES)), ids=[c[0] for c in CASES])
@pytest.mark.parametrize("kind", ["add", "add_f32"])
def test_additive_mask_values_every_path(case, n_splits, dtype, kind):
    name, B, Hq, Hkv, rows, off, op, Bm, shape, window = CASES[case]
    _say("mask values", name, dtype, kind, "n_splits", n_splits)
    kv = off + rows
    qb, kb, vb, gb, mb = _inputs(5000 + case, B, Hq, Hkv, rows, off, dtype, Bm, kind)
    mdev, mref = _mask_dev(mb, kind, dtype)
    q, k, v, g = (to_dev(x, dtype) for x in (qb, kb, vb, gb))
    lds_stride, lane_stride = lds_and_lane_strides(kv, mdev.element_size())
    storages = [strided_mask(mdev, lds_stride), strided_mask(mdev, lane_stride),
                mdev.expand(Bm, Hq, rows, kv).contiguous()]
    want = _expected_layouts(window, kind, name)
    outs = []
    for m, marker in zip(storages, want):
        a = ga._args(q, k, v, g, torch.empty_like(q), kv_offset=off, kv_len=kv, causal=True, scale=0.0,
                     head_chunk=0, n_splits=n_splits, mask=m)
        d = ga.describe_plan(a, op)
        vn = d["variant_name"]
        assert (d["n_splits"] == 1) == (n_splits == 1), d
        assert f"_{shape}" in vn and (marker in vn if marker else "lds" not in vn), (vn, marker)
        outs.append(_run(op, q, k, v, g, off, kv, m, n_splits))
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16)), "mask paths differ"
    ref = reference.attention(*(syn.widen(x, dtype) for x in (qb, kb, vb, gb)), n_kv_heads=Hkv, kv_offset=off,
                              kv_len=kv, mask=mref, mask_kind="add")
    _say(assert_close(syn.widen(to_bits(outs[0]), dtype), ref, f"mask values {name}"))
    # the values matter: the same call with the mask's finite entries zeroed lands elsewhere
    zeroed = np.where(np.isfinite(mref), 0.0, -np.inf)
    ref0 = reference.attention(*(syn.widen(x, dtype) for x in (qb, kb, vb, gb)), n_kv_heads=Hkv, kv_offset=off,
                               kv_len=kv, mask=zeroed, mask_kind="add")
    assert not compare(syn.widen(to_bits(outs[0]), dtype), ref0)["ok"]


@needs_gpu
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("rows", [1, 4, 9, 32])
def test_decode_mask_rows_at_any_length(dtype, rows):
    # the decode workload's masks end mid-chunk (kv_len 32769, 32772, ...): the word layout stages
    # them in LDS anyway, and agrees with the per-lane loads of a full-head copy and the oracle
    _say("mask at any length", dtype, rows)
    B, Hq, Hkv, off = 2, 16, 2, 32768
    kv = off + rows
    qb, kb, vb, gb, mb = _inputs(5200 + rows, B, Hq, Hkv, rows, off, dtype, 1, "add")
    q, k, v, g, m = (to_dev(x, dtype) for x in (qb, kb, vb, gb, mb))
    a = ga._args(q, k, v, g, torch.empty_like(q), kv_offset=off, kv_len=kv, causal=True, scale=0.0, head_chunk=0,
                 n_splits=0, mask=m)
    assert "ldswords" in ga.describe_plan(a, ga._abi.OP_DECODE)["variant_name"]
    out = ga.decode(q, k, v, g, kv_offset=off, mask=m)
    full = ga.decode(q, k, v, g, kv_offset=off, mask=m.expand(1, Hq, rows, kv).contiguous())
    assert torch.equal(out.view(torch.int16), full.view(torch.int16))
    ref = reference.attention(*(syn.widen(x, dtype) for x in (qb, kb, vb, gb)), n_kv_heads=Hkv, kv_offset=off,
                              kv_len=kv, mask=syn.widen(mb, dtype), mask_kind="add")
    _say(assert_close(syn.widen(to_bits(out), dtype), ref, "mask at any length"))


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


# Full-head masks (a row per query head) whose workgroups hold one column block of at most
# 1024 / T pairs (T keys per tile: 32 pairs at head dim 256, 16 at 128, 8 at 64) stage each pair's
# own mask row beside the K/V tiles, one dword per key.  (B, Hq, Hkv, rows, kv_offset, D, Bm)
PAIR_CASES = [
    (2, 16, 2, 1, 4096, 256, 1),    # 8 pairs
    (2, 16, 2, 4, 32768, 256, 2),   # 32 pairs, 61 KV splits, a mask per batch entry
    (1, 24, 4, 5, 4091, 256, 1),    # 30 pairs (6 heads x 5 rows)
    (2, 16, 2, 2, 4094, 128, 1),    # 16 pairs at head dim 128
    (1, 16, 2, 1, 2047, 64, 1),     # 8 pairs at head dim 64
]


@needs_gpu
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("kind", ["bool", "add", "add_f32"])
@pytest.mark.parametrize("case", range(len(PAIR_CASES)),
                         ids=[f"B{c[0]}_{c[1]}x{c[2]}_r{c[3]}_D{c[5]}" for c in PAIR_CASES])
def test_full_head_mask_pair_windows(case, kind, dtype):
    B, Hq, Hkv, rows, off, D, Bm = PAIR_CASES[case]
    _say("pair windows", PAIR_CASES[case], kind, dtype)
    kv = off + rows
    rng = syn.streams(5400 + 10 * case)
    qb, gb = (syn.normal_bits(rng[n], (B, Hq, rows, D), dtype) for n in ("q", "gate"))
    kb, vb = (syn.normal_bits(rng[n], (B, Hkv, kv, D), dtype) for n in ("k", "v"))
    values = "zero" if kind == "bool" else "normal"
    mb = syn.verify_mask(rng["mask"], rows=rows, kv_offset=off, heads=Hq, kind=kind, dtype=dtype, values=values,
                         batch=Bm)
    q, k, v, g = (to_dev(x, dtype) for x in (qb, kb, vb, gb))

    def dev_mask(x):
        return to_dev(x, dtype) if kind == "add" else torch.from_numpy(x).cuda()

    def plan_name(m, head_chunk=0):
        a = ga._args(q, k, v, g, torch.empty_like(q), kv_offset=off, kv_len=kv, causal=True, scale=0.0,
                     head_chunk=head_chunk, n_splits=0, mask=m)
        return ga.describe_plan(a, ga._abi.OP_DECODE)["variant_name"]

    m = dev_mask(mb)
    assert "_ldspairwords" in plan_name(m), plan_name(m)
    out = ga.decode(q, k, v, g, kv_offset=off, mask=m)
    # two head chunks put the pairs in two column blocks: the per-lane mask loads, the same bits
    hc = (Hq // Hkv) // 2
    assert "lds" not in plan_name(m, hc), plan_name(m, hc)
    lane = ga.decode(q, k, v, g, kv_offset=off, mask=m, head_chunk=hc)
    assert torch.equal(lane.view(torch.int16), out.view(torch.int16)), "pair window and per-lane loads differ"
    if kind == "add":
        mref, mk = syn.widen(mb, dtype), "add"
    elif kind == "bool":
        mref, mk = mb.astype(bool), "bool"
    else:
        mref, mk = mb.astype(np.float64), "add"
    ref = reference.attention(*(syn.widen(x, dtype) for x in (qb, kb, vb, gb)), n_kv_heads=Hkv, kv_offset=off,
                              kv_len=kv, mask=mref, mask_kind=mk)
    _say(assert_close(syn.widen(to_bits(out), dtype), ref, f"pair windows {case} {kind}"))
    # a mask the same for every head: its own word window and its full-head copy give the same bits
    mb1 = syn.verify_mask(rng["mask"], rows=rows, kv_offset=off, heads=1, kind=kind, dtype=dtype, values=values,
                          batch=Bm)
    m1 = dev_mask(mb1)
    full = m1.expand(Bm, Hq, rows, kv).contiguous()
    assert "_ldswords" in plan_name(m1) and "_ldspairwords" in plan_name(full)
    one = ga.decode(q, k, v, g, kv_offset=off, mask=m1)
    per_head = ga.decode(q, k, v, g, kv_offset=off, mask=full)
    assert torch.equal(one.view(torch.int16), per_head.view(torch.int16)), "broadcast and full-head copy differ"
