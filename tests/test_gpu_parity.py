"""Parity of the HIP path (through the C ABI) with the float64 oracle on an MI355X.

Tolerance: max abs error <= 1.5e-2 and median relative error <= 4e-3 on 16-bit outputs
with fp32 accumulation; kv_append is compared bit for bit; head-chunk variants are
compared bit for bit with each other.
"""

import numpy as np
import pytest
import torch

import gqa_causal_attention_attn_amd as ga
from oracle import reference
from synth import inputs as syn
from tests.gpu_util import lds_and_lane_strides, prompt, strided_mask, to_bits, to_dev, to_f64
from tests.parity import assert_close, compare

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def _say(*a):
    print(*a, flush=True)


def _prompt_run(qb, kb, vb, gb, *, Hkv, q_block, dtype="bf16", head_chunk=0, n_splits=0):
    q, k, v, g = (to_dev(x, dtype) for x in (qb, kb, vb, gb))
    N = q.shape[2]
    kc = torch.full((k.shape[0], Hkv, N, 256), float("nan"), dtype=q.dtype, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    out = torch.full_like(q, float("nan"))
    ga.prompt_prefill(q, k, v, g, kc, vc, q_block=q_block, out=out, head_chunk=head_chunk, n_splits=n_splits)
    torch.cuda.synchronize()
    return out, kc, vc


@needs_gpu
@pytest.mark.parametrize("q_block", [128, 48])
def test_tiny_prefill_24_over_4(q_block):
    # batch 1, 24 query heads over 4 KV heads, 128 tokens, causal, gated
    _say("tiny prefill qL", q_block)
    qb, kb, vb, gb, _ = prompt(1000, B=1, Hq=24, Hkv=4, N=128)
    out, kc, vc = _prompt_run(qb, kb, vb, gb, Hkv=4, q_block=q_block)
    assert np.array_equal(to_bits(kc), kb) and np.array_equal(to_bits(vc), vb)
    ref = reference.attention(syn.widen(qb), syn.widen(kb), syn.widen(vb), syn.widen(gb), n_kv_heads=4, kv_offset=0,
                              kv_len=128)
    _say(assert_close(to_f64(out), ref, "tiny prefill"))


@needs_gpu
@pytest.mark.parametrize("Hq,Hkv,N,q_block,n_splits", [
    (24, 4, 200, 96, 0),     # ragged last block
    (16, 2, 333, 128, 0),    # ragged, GQA 8
    (16, 2, 300, 300, 3),    # forced KV splits + merge
    (8, 8, 70, 70, 1),       # no grouping
    (6, 1, 90, 32, 0),       # one KV head
])
def test_prefill_ragged_shapes(Hq, Hkv, N, q_block, n_splits):
    _say("prefill", Hq, Hkv, N, q_block, n_splits)
    qb, kb, vb, gb, _ = prompt(2000 + N, B=1, Hq=Hq, Hkv=Hkv, N=N)
    out, _, _ = _prompt_run(qb, kb, vb, gb, Hkv=Hkv, q_block=q_block, n_splits=n_splits)
    ref = reference.attention(syn.widen(qb), syn.widen(kb), syn.widen(vb), syn.widen(gb), n_kv_heads=Hkv,
                              kv_offset=0, kv_len=N)
    _say(assert_close(to_f64(out), ref, "prefill"))


@needs_gpu
@pytest.mark.parametrize("n_splits", [0, 3])
def test_prompt_with_merges_on_a_second_stream(n_splits):
    # attn_prefill_partials + attn_merge on a second stream, two workspaces alternating: the
    # same bits as attn_prefill block by block
    _say("overlapped merges", n_splits)
    qb, kb, vb, gb, _ = prompt(2100 + n_splits, B=1, Hq=24, Hkv=4, N=700)
    q, k, v, g = (to_dev(x) for x in (qb, kb, vb, gb))
    outs = []
    for overlap in (False, True):
        kc = torch.full((1, 4, 700, 256), float("nan"), dtype=q.dtype, device="cuda")
        vc = torch.full_like(kc, float("nan"))
        out = torch.full_like(q, float("nan"))
        ga.prompt_prefill(q, k, v, g, kc, vc, q_block=128, out=out, n_splits=n_splits, overlap_merge=overlap)
        torch.cuda.synchronize()
        outs.append(out)
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    ref = reference.attention(syn.widen(qb), syn.widen(kb), syn.widen(vb), syn.widen(gb), n_kv_heads=4,
                              kv_offset=0, kv_len=700)
    _say(assert_close(to_f64(outs[1]), ref, "overlapped merges"))


@needs_gpu
def test_prefill_batch2_fp16_noncausal():
    rng = syn.streams(31)
    B, Hq, Hkv, rows, kv = 2, 16, 2, 40, 150
    qb = syn.normal_bits(rng["q"], (B, Hq, rows, 256), "f16")
    kb = syn.normal_bits(rng["k"], (B, Hkv, kv, 256), "f16")
    vb = syn.normal_bits(rng["v"], (B, Hkv, kv, 256), "f16")
    gb = syn.normal_bits(rng["gate"], (B, Hq, rows, 256), "f16")
    q, k, v, g = (to_dev(x, "f16") for x in (qb, kb, vb, gb))
    out = ga.prefill(q, k, v, g, kv_offset=0, kv_len=kv, causal=False)
    ref = reference.attention(*(syn.widen(x, "f16") for x in (qb, kb, vb, gb)), n_kv_heads=Hkv, kv_offset=0,
                              kv_len=kv, causal=False)
    _say(assert_close(to_f64(out), ref, "fp16 noncausal"))


def _decode_case(seed, *, B, Hq, Hkv, offset, rows, dtype="bf16"):
    rng = syn.streams(seed)
    kv_len = offset + rows
    kb = syn.normal_bits(rng["k"], (B, Hkv, kv_len, 256), dtype)
    vb = syn.normal_bits(rng["v"], (B, Hkv, kv_len, 256), dtype)
    qb = syn.normal_bits(rng["q"], (B, Hq, rows, 256), dtype)
    gb = syn.normal_bits(rng["gate"], (B, Hq, rows, 256), dtype)
    return qb, kb, vb, gb, rng


@needs_gpu
@pytest.mark.parametrize("rows", [1, 4])
def test_decode_27b_shape(rows):
    # 24 query heads over 4 KV heads, cache of 4096 keys, rows appended at offset 4096
    _say("decode 27B rows", rows)
    qb, kb, vb, gb, _ = _decode_case(1001, B=1, Hq=24, Hkv=4, offset=4096, rows=rows)
    q, g = to_dev(qb), to_dev(gb)
    cap = 4096 + 32
    kc = torch.zeros((1, 4, cap, 256), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    kc[:, :, :4096] = to_dev(kb[:, :, :4096])
    vc[:, :, :4096] = to_dev(vb[:, :, :4096])
    ga.kv_append(to_dev(kb[:, :, 4096:]), to_dev(vb[:, :, 4096:]), kc, vc, kv_offset=4096)
    out = ga.decode(q, kc, vc, g, kv_offset=4096)
    ref = reference.attention(syn.widen(qb), syn.widen(kb), syn.widen(vb), syn.widen(gb), n_kv_heads=4,
                              kv_offset=4096, kv_len=4096 + rows)
    _say(assert_close(to_f64(out), ref, "decode"))


@needs_gpu
@pytest.mark.parametrize("kv_len,n_splits", [
    (1, 0), (31, 1), (33, 1), (97, 1),   # one to four tiles
    (4000, 1), (4064, 1),                # one split: a ragged and a whole last tile
    (4000, 0), (4000, 7),                # several splits + merge
])
def test_decode_short_and_split_caches(kv_len, n_splits):
    # one 32-pair block per KV group (8 heads x 1 row) against caches shorter than a tile, one
    # split of many tiles and several splits with the merge
    _say("decode caches", kv_len, n_splits)
    B, Hq, Hkv, rows = 1, 16, 2, 1
    qb, kb, vb, gb, _ = _decode_case(3000 + kv_len, B=B, Hq=Hq, Hkv=Hkv, offset=kv_len - rows, rows=rows)
    q, k, v, g = (to_dev(x) for x in (qb, kb, vb, gb))
    out = ga.decode(q, k, v, g, kv_offset=kv_len - rows, n_splits=n_splits)
    ref = reference.attention(*(syn.widen(x) for x in (qb, kb, vb, gb)), n_kv_heads=Hkv, kv_offset=kv_len - rows,
                              kv_len=kv_len)
    _say(assert_close(to_f64(out), ref, "decode"))
    # head chunks of 3 heads: the same bits
    chunked = ga.decode(q, k, v, g, kv_offset=kv_len - rows, n_splits=n_splits, head_chunk=3)
    assert torch.equal(chunked.view(torch.int16), out.view(torch.int16))


@needs_gpu
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("offset", [4097, 32768])
# rows 6, 8 and 12 give the policy plans [5, 3], [4, 4] and [2, 2, 2, 2] for groups of 8
@pytest.mark.parametrize("rows", [1, 4, 5, 6, 8, 9, 12, 17, 32])
def test_head_chunked_verify(dtype, offset, rows):
    # batch 2, 16 query heads over 2 KV heads, rows appended at the offset, broadcast additive mask
    _say("verify", dtype, offset, rows)
    B, Hq, Hkv = 2, 16, 2
    qb, kb, vb, gb, rng = _decode_case(1004 + rows, B=B, Hq=Hq, Hkv=Hkv, offset=offset, rows=rows, dtype=dtype)
    mb = syn.verify_mask(rng["mask"], rows=rows, kv_offset=offset, heads=1, kind="add", dtype=dtype,
                         values="normal")
    q, k, v, g, m = (to_dev(x, dtype) for x in (qb, kb, vb, gb, mb))
    outs = {}
    for hc in [0] + list(range(1, 9)):
        outs[hc] = to_bits(ga.decode(q, k, v, g, kv_offset=offset, mask=m, head_chunk=hc))
    for hc in range(1, 9):
        assert np.array_equal(outs[hc], outs[0]), f"head_chunk {hc} differs from the policy"
    ref = reference.attention(*(syn.widen(x, dtype) for x in (qb, kb, vb, gb)), n_kv_heads=Hkv, kv_offset=offset,
                              kv_len=offset + rows, mask=syn.widen(mb, dtype), mask_kind="add")
    _say(assert_close(syn.widen(outs[0], dtype), ref, "verify"))


@needs_gpu
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("kind", ["full_head_add", "bool", "f32"])
def test_verify_mask_kinds(kind, dtype):
    # full-head masks (one pattern per query head, N(0, 1) values at admitted keys), a bool
    # mask and an fp32 additive mask; every head-chunk variant agrees bit for bit
    B, Hq, Hkv, offset, rows = 2, 16, 2, 4097, 6
    _say("mask kind", kind, dtype)
    qb, kb, vb, gb, rng = _decode_case(77, B=B, Hq=Hq, Hkv=Hkv, offset=offset, rows=rows, dtype=dtype)
    if kind == "full_head_add":
        mb = syn.verify_mask(rng["mask"], rows=rows, kv_offset=offset, heads=Hq, kind="add", dtype=dtype,
                             values="normal")
        m = to_dev(mb, dtype)
        mref, mk = syn.widen(mb, dtype), "add"
    elif kind == "bool":
        mb = syn.verify_mask(rng["mask"], rows=rows, kv_offset=offset, heads=1, kind="bool")
        m = torch.from_numpy(mb).cuda()
        mref, mk = mb.astype(bool), "bool"
    else:
        mb = syn.verify_mask(rng["mask"], rows=rows, kv_offset=offset, heads=Hq, kind="add_f32", values="normal")
        m = torch.from_numpy(mb).cuda()
        mref, mk = mb.astype(np.float64), "add"
    q, k, v, g = (to_dev(x, dtype) for x in (qb, kb, vb, gb))
    out = ga.decode(q, k, v, g, kv_offset=offset, mask=m)
    ref = reference.attention(*(syn.widen(x, dtype) for x in (qb, kb, vb, gb)), n_kv_heads=Hkv, kv_offset=offset,
                              kv_len=offset + rows, mask=mref, mask_kind=mk)
    _say(assert_close(syn.widen(to_bits(out), dtype), ref, kind))
    for hc in (1, 3, 8):
        again = ga.decode(q, k, v, g, kv_offset=offset, mask=m, head_chunk=hc)
        assert torch.equal(again.view(torch.int16), out.view(torch.int16)), f"head_chunk {hc}"


@needs_gpu
@pytest.mark.parametrize("kind", ["bool", "add", "f32"])
@pytest.mark.parametrize("rows,Bm", [(6, 1), (32, 1), (32, 2)])
def test_mask_paths_agree(kind, rows, Bm):
    # A head-broadcast mask is staged in LDS with each K/V tile, one dword per key, whatever its
    # row stride (rows 6: the four-wavefront shape; rows 32: eight wavefronts); a copy with one
    # pattern per query head takes the per-lane loads.  All give the same bits and match the oracle.
    _say("mask paths", kind, rows, Bm)
    B, Hq, Hkv = 2, 16, 2
    offset = 4112 - rows
    kv = offset + rows
    qb, kb, vb, gb, rng = _decode_case(600 + rows, B=B, Hq=Hq, Hkv=Hkv, offset=offset, rows=rows)
    masks = [syn.verify_mask(rng["mask"], rows=rows, kv_offset=offset, heads=1,
                             kind={"bool": "bool", "add": "add", "f32": "add_f32"}[kind]) for _ in range(Bm)]
    mb = np.concatenate(masks, axis=0)
    if kind == "f32":
        mb = np.where(np.isfinite(mb), np.random.default_rng(9).standard_normal(mb.shape).astype(np.float32), mb)
    if kind == "add":
        mdev = to_dev(mb)
        mref, mk = syn.widen(mb), "add"
    else:
        mdev = torch.from_numpy(mb).cuda()
        mref, mk = (mb.astype(bool), "bool") if kind == "bool" else (mb.astype(np.float64), "add")
    lds_stride, lane_stride = lds_and_lane_strides(kv, mdev.element_size())
    storages = [strided_mask(mdev, lds_stride), strided_mask(mdev, lane_stride),
                mdev.expand(Bm, Hq, rows, kv).contiguous()]
    q, k, v, g = (to_dev(x) for x in (qb, kb, vb, gb))
    names = []
    for m in storages:
        a = ga._args(q, k, v, g, torch.empty_like(q), kv_offset=offset, kv_len=kv, causal=True, scale=0.0,
                     head_chunk=0, n_splits=0, mask=m)
        names.append(ga.describe_plan(a, 1)["variant_name"])
    assert "ldswords" in names[0] and "ldswords" in names[1] and "lds" not in names[2], names
    outs = [ga.decode(q, k, v, g, kv_offset=offset, mask=m) for m in storages]
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))
    ref = reference.attention(*(syn.widen(x) for x in (qb, kb, vb, gb)), n_kv_heads=Hkv, kv_offset=offset,
                              kv_len=kv, mask=mref, mask_kind=mk)
    _say(assert_close(to_f64(outs[0]), ref, f"mask paths {kind}"))


@needs_gpu
def test_kv_append_is_bit_exact():
    nf = syn.nonfinite_bits("bf16")
    rng = syn.streams(5)
    new_k = syn.normal_bits(rng["k"], (2, 2, 5, 256))
    new_v = syn.normal_bits(rng["v"], (2, 2, 5, 256))
    new_k[0, 0, 0, :4] = [nf["-0"], nf["nan"], nf["+inf"], nf["-inf"]]
    new_v[1, 1, 4, 250:] = nf["nan"]
    cache = syn.normal_bits(rng["plant"], (2, 2, 20, 256))
    kc, vc = to_dev(cache), to_dev(cache)
    ga.kv_append(to_dev(new_k), to_dev(new_v), kc, vc, kv_offset=11)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(kc), reference.kv_append(cache, new_k, 11))
    assert np.array_equal(to_bits(vc), reference.kv_append(cache, new_v, 11))
    with pytest.raises(ga.AttnError):
        ga.kv_append(to_dev(new_k), to_dev(new_v), kc, vc, kv_offset=16)

@needs_gpu
@pytest.mark.parametrize("B,Hkv,rows,offset", [(3, 5, 300, 40), (1, 4, 512, 0), (2, 2, 1, 777)])
def test_kv_append_of_prompt_views(B, Hkv, rows, offset):
    # the new rows are a view of a longer prompt tensor (row stride 256, head stride 256 x its
    # length), as when a prompt is appended block by block; several row blocks and (b, g) pairs
    rng = syn.streams(6 + rows)
    big = syn.normal_bits(rng["k"], (B, Hkv, rows + 70, 256))
    bigv = syn.normal_bits(rng["v"], (B, Hkv, rows + 70, 256))
    cache = syn.normal_bits(rng["plant"], (B, Hkv, offset + rows + 9, 256))
    kc, vc = to_dev(cache), to_dev(cache)
    k, v = to_dev(big), to_dev(bigv)
    ga.kv_append(k[:, :, 33:33 + rows], v[:, :, 33:33 + rows], kc, vc, kv_offset=offset)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(kc), reference.kv_append(cache, big[:, :, 33:33 + rows], offset))
    assert np.array_equal(to_bits(vc), reference.kv_append(cache, bigv[:, :, 33:33 + rows], offset))


@needs_gpu
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_kv_keep_is_bit_exact(dtype):
    # a verify block of 32 rows at offset 100: batch entry 0 keeps a tree path, entry 1 a chain,
    # entry 2 nothing, entry 3 everything; then a second keep on the caches the first left
    nf = syn.nonfinite_bits(dtype)
    rng = syn.streams(17)
    B, Hkv, cap, off, rows = 4, 2, 160, 100, 32
    cache = syn.normal_bits(rng["k"], (B, Hkv, cap, 256), dtype)
    cache[0, 1, off + 9, :3] = [nf["nan"], nf["-0"], nf["-inf"]]
    vcache = syn.normal_bits(rng["v"], (B, Hkv, cap, 256), dtype)
    keep = [(1 << 0) | (1 << 3) | (1 << 9) | (1 << 30), (1 << 7) - 1, 0, 0xFFFFFFFF]
    kc, vc = to_dev(cache, dtype), to_dev(vcache, dtype)
    ga.kv_keep(kc, vc, kv_offset=off, rows=rows, keep=keep)
    torch.cuda.synchronize()
    want_k = reference.kv_keep(cache, off, rows, keep)
    want_v = reference.kv_keep(vcache, off, rows, keep)
    assert np.array_equal(to_bits(kc), want_k) and np.array_equal(to_bits(vc), want_v)
    keep2 = [0b0110, 0b1010101, 0, 1 << 31]
    ga.kv_keep(kc, vc, kv_offset=off, rows=rows, keep=keep2)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(kc), reference.kv_keep(want_k, off, rows, keep2))
    assert np.array_equal(to_bits(vc), reference.kv_keep(want_v, off, rows, keep2))
    with pytest.raises(ga.AttnError):
        ga.kv_keep(kc, vc, kv_offset=off, rows=3, keep=[0b1000, 0, 0, 0])


@needs_gpu
# few-chunk pass; many-chunk pass with 4, 8 and 16 wavefronts per row, in one round and in two;
# rows of 256, 128 and 64 (lanes past the head dim store nothing)
@pytest.mark.parametrize("D", [256, 128, 64])
@pytest.mark.parametrize("n_chunks", [4, 12, 21, 40, 100])
def test_merge_matches_oracle(n_chunks, D):
    rng = syn.streams(8)
    B, Hq, Hkv, rows, kv = 1, 8, 2, 5, 90
    q = syn.widen(syn.normal_bits(rng["q"], (B, Hq, rows, D)))
    k = syn.widen(syn.normal_bits(rng["k"], (B, Hkv, kv, D)))
    v = syn.widen(syn.normal_bits(rng["v"], (B, Hkv, kv, D)))
    gb = syn.normal_bits(rng["gate"], (B, Hq, rows, D))
    step = max(1, 120 // n_chunks)
    chunks = [(c * step, (c + 1) * step) for c in range(n_chunks)]  # the chunks past key 90 are empty
    o, l_ = reference.partials(q, k, v, n_kv_heads=Hkv, kv_offset=kv - rows, kv_len=kv, chunks=chunks)
    o32, l32 = o.astype(np.float32), l_.astype(np.float32)
    # one row empty in every chunk, with NaN partials: never multiplied in, the row is 0
    l32[:, 0, 3, 2] = -np.inf
    o32[:, 0, 3, 2, :] = np.nan
    # out starts as NaN: every element of the head dim is written, and nothing past it exists
    out = torch.full((B, Hq, rows, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    ga.merge(torch.from_numpy(o32).cuda(), torch.from_numpy(l32).cuda(), to_dev(gb), out=out)
    ref = reference.merge(o, l_, syn.widen(gb))
    ref[0, 3, 2, :] = 0.0
    got = to_f64(out)
    assert np.all(got[0, 3, 2, :] == 0.0)
    _say(assert_close(got, ref, f"merge {n_chunks} chunks, D={D}"))


@needs_gpu
@pytest.mark.parametrize("n_chunks", [2, 5, 8, 24, 40])
def test_merge_with_lse_far_apart(n_chunks):
    # chunk lse values drawn over [-600, 0] (natural log) with each row's largest in a random
    # chunk, so in any lane of the wavefront that holds the chunks: weights below the largest
    # underflow, and a row max taken short of the true one would overflow exp (Inf or NaN rows).
    # 1024 rows: the one-wavefront merge with the chunk count (up to 8) or 24 / 40 slots.
    rng = np.random.default_rng(600 + n_chunks)
    B, Hq, rows, D = 1, 8, 128, 256
    o = rng.standard_normal((n_chunks, B, Hq, rows, D))
    lse = rng.uniform(-600.0, 0.0, (n_chunks, B, Hq, rows))
    top = rng.integers(0, n_chunks, (B, Hq, rows))
    np.put_along_axis(lse, top[None], rng.uniform(-1.0, 1.0, (1, B, Hq, rows)), axis=0)
    gb = syn.normal_bits(np.random.default_rng(7), (B, Hq, rows, D))
    out = torch.full((B, Hq, rows, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    ga.merge(torch.from_numpy(o.astype(np.float32)).cuda(), torch.from_numpy(lse.astype(np.float32)).cuda(),
             to_dev(gb), out=out)
    torch.cuda.synchronize()
    got = to_f64(out)
    assert np.isfinite(got).all()
    ref = reference.merge(o.astype(np.float32).astype(np.float64), lse.astype(np.float32).astype(np.float64),
                          syn.widen(gb))
    _say(assert_close(got, ref, f"merge of {n_chunks} chunks with lse far apart"))


def _fp16_rows(o):
    """The main pass's partial form (merge_args partial_kind 1) of float64 partials o [..., D]:
    per row the exponent e that puts the largest magnitude in [0.5, 1) (0 for a zero or nonfinite
    row) and the values times 2^-e rounded to fp16 (nearest even).  Returns the float16 values,
    the int32 exponents [...] and the exact values they stand for (float64)."""
    with np.errstate(invalid="ignore"):
        mx = np.nanmax(np.abs(o), axis=-1)
    e = np.where((mx > 0) & np.isfinite(mx), np.frexp(np.where(np.isfinite(mx), mx, 1.0))[1], 0).astype(np.int32)
    vals = np.ldexp(o, -e[..., None]).astype(np.float16)
    return vals, e, np.ldexp(vals.astype(np.float64), e[..., None])


@needs_gpu
@pytest.mark.parametrize("D", [256, 128, 64])
@pytest.mark.parametrize("n_chunks", [5, 21, 100])
@pytest.mark.parametrize("mag", [1.0, 1e-30, 1e30])
def test_merge_fp16_rows(n_chunks, D, mag):
    # the partial form the main pass leaves (fp16 values and a power-of-two exponent per row)
    # through attn_merge: against the oracle at V magnitudes 1, 1e-30 and 1e30 (the exponent keeps
    # fp16 in range), and bit for bit against the fp32 form of the same values (the decode is exact)
    rng = syn.streams(9)
    B, Hq, Hkv, rows, kv = 1, 8, 2, 5, 90
    q = syn.widen(syn.normal_bits(rng["q"], (B, Hq, rows, D)))
    k = syn.widen(syn.normal_bits(rng["k"], (B, Hkv, kv, D)))
    v = syn.widen(syn.normal_bits(rng["v"], (B, Hkv, kv, D))) * mag
    gb = syn.normal_bits(rng["gate"], (B, Hq, rows, D))
    step = max(1, 120 // n_chunks)
    chunks = [(c * step, (c + 1) * step) for c in range(n_chunks)]
    o, l_ = reference.partials(q, k, v, n_kv_heads=Hkv, kv_offset=kv - rows, kv_len=kv, chunks=chunks)
    l32 = l_.astype(np.float32)
    l32[:, 0, 3, 2] = -np.inf  # a row empty in every chunk: 0 whatever its partials hold
    o = o.copy()
    o[:, 0, 3, 2, :] = np.nan
    vals16, exps, exact = _fp16_rows(o)
    out16 = torch.full((B, Hq, rows, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    ga.merge(torch.from_numpy(vals16).cuda(), torch.from_numpy(l32).cuda(), to_dev(gb), out=out16,
             partial_exp=torch.from_numpy(exps).cuda())
    out32 = torch.full_like(out16, float("nan"))
    ga.merge(torch.from_numpy(exact.astype(np.float32)).cuda(), torch.from_numpy(l32).cuda(), to_dev(gb), out=out32)
    assert torch.equal(out16.view(torch.int16), out32.view(torch.int16)), "fp16 rows and their fp32 values differ"
    ref = reference.merge(np.nan_to_num(o, nan=0.0), l_, syn.widen(gb))
    ref[0, 3, 2, :] = 0.0
    got = to_f64(out16)
    assert np.all(got[0, 3, 2, :] == 0.0)
    _say(assert_close(got / mag, ref / mag, f"merge fp16 rows {n_chunks} chunks, D={D}, |v|~{mag:g}"))


@needs_gpu
def test_closed_forms_on_gpu():
    # constant V: every row returns c * sigmoid(gate); row 0 of a prompt sees one key: V_0 * sigmoid(gate)
    qb, kb, vb, gb, _ = prompt(42, B=1, Hq=8, Hkv=2, N=100)
    vb[:] = syn.f32_to_bits(np.full(vb.shape, 0.375, dtype=np.float32))
    out, _, _ = _prompt_run(qb, kb, vb, gb, Hkv=2, q_block=100)
    ref = 0.375 * reference.sigmoid(syn.widen(gb))
    _say(assert_close(to_f64(out), ref, "constant V"))
    qb, kb, vb, gb, _ = prompt(43, B=1, Hq=8, Hkv=2, N=64)
    out, _, _ = _prompt_run(qb, kb, vb, gb, Hkv=2, q_block=64)
    first = to_f64(out)[0, :, 0]
    want = syn.widen(vb)[0, np.arange(8) // 4, 0] * reference.sigmoid(syn.widen(gb)[0, :, 0])
    _say(assert_close(first, want, "single key"))


@needs_gpu
def test_empty_row_gives_zero():
    B, Hq, Hkv, offset, rows = 1, 8, 2, 200, 3
    qb, kb, vb, gb, rng = _decode_case(9, B=B, Hq=Hq, Hkv=Hkv, offset=offset, rows=rows)
    mb = np.ones((1, 1, rows, offset + rows), dtype=np.uint8)
    mb[0, 0, 1] = 0
    q, k, v, g = (to_dev(x) for x in (qb, kb, vb, gb))
    out = to_f64(ga.decode(q, k, v, g, kv_offset=offset, mask=torch.from_numpy(mb).cuda()))
    assert np.all(out[0, :, 1] == 0.0)
    ref = reference.attention(*(syn.widen(x) for x in (qb, kb, vb, gb)), n_kv_heads=Hkv, kv_offset=offset,
                              kv_len=offset + rows, mask=mb.astype(bool), mask_kind="bool")
    _say(assert_close(out, ref, "empty row"))


@needs_gpu
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_stress_cancellation_passes_with_fp32_accumulation(dtype):
    rng = syn.streams(1234)
    B, Hq, Hkv, rows, off = 1, 4, 2, 8, 24
    qb, kb, vb, gb = syn.stress_cancellation(rng["plant"], B=B, Hq=Hq, Hkv=Hkv, rows=rows, kv_len=off + rows,
                                             dtype=dtype)
    q, k, v, g = (to_dev(x, dtype) for x in (qb, kb, vb, gb))
    out = ga.decode(q, k, v, g, kv_offset=off)
    ref = reference.attention(*(syn.widen(x, dtype) for x in (qb, kb, vb, gb)), n_kv_heads=Hkv, kv_offset=off,
                              kv_len=off + rows)
    _say(assert_close(syn.widen(to_bits(out), dtype), ref, "stress"))


@needs_gpu
def test_repeat_runs_are_bitwise_identical():
    qb, kb, vb, gb, _ = prompt(7, B=1, Hq=16, Hkv=2, N=256)
    a, _, _ = _prompt_run(qb, kb, vb, gb, Hkv=2, q_block=128)
    b, _, _ = _prompt_run(qb, kb, vb, gb, Hkv=2, q_block=128)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@needs_gpu
def test_planted_row_past_its_own_key_is_not_seen():
    # each row's query points at the key just after its own position: a kernel that lets a
    # row see one key too many lands far from the oracle
    B, Hq, Hkv, off, rows = 1, 8, 2, 40, 6
    qb, kb, vb, gb, _ = _decode_case(21, B=B, Hq=Hq, Hkv=Hkv, offset=off, rows=rows + 1)
    k = syn.widen(kb)
    q = syn.widen(qb)[:, :, :rows]
    for h in range(Hq):
        for r in range(rows):
            q[0, h, r] = 0.5 * k[0, h // 4, off + r + 1]
    qb2 = syn.f32_to_bits(q.astype(np.float32))
    gb = gb[:, :, :rows]
    dev = [to_dev(x) for x in (qb2, kb, vb, gb)]
    out = to_f64(ga.decode(dev[0], dev[1], dev[2], dev[3], kv_offset=off, kv_len=off + rows))
    good = reference.attention(syn.widen(qb2), k, syn.widen(vb), syn.widen(gb), n_kv_heads=Hkv, kv_offset=off,
                               kv_len=off + rows)
    assert compare(out, good)["ok"]
    past = reference.attention(syn.widen(qb2), k, syn.widen(vb), syn.widen(gb), n_kv_heads=Hkv, kv_offset=off + 1,
                               kv_len=off + rows + 1)
    assert not compare(out, past)["ok"]


@needs_gpu
@pytest.mark.parametrize("n_splits,kind", [(3, 0), (5, 1)])
@pytest.mark.parametrize("mag", [1.0, 1e-30])
def test_split_partials_either_side_of_the_fp16_line(n_splits, kind, mag):
    # 512 rows of 8 heads at head dim 128: 2 MiB of fp32 partials per split, so 3 splits keep
    # fp32 partials (6 MiB) and 5 take fp16 ones with a power of two per row (10 MiB); both against
    # the oracle, through attn_prefill and through attn_prefill_partials + attn_merge (bit for
    # bit with it), with V of magnitude 1 and 1e-30 (the exponent keeps fp16 in range)
    D, B, Hq, Hkv, rows, off = 128, 1, 8, 2, 512, 1536
    rng = syn.streams(77)
    qb = syn.normal_bits(rng["q"], (B, Hq, rows, D))
    kb = syn.normal_bits(rng["k"], (B, Hkv, off + rows, D))
    vb = syn.normal_bits(rng["v"], (B, Hkv, off + rows, D), scale=mag)
    gb = syn.normal_bits(rng["gate"], (B, Hq, rows, D))
    q, k, v, g = (to_dev(x) for x in (qb, kb, vb, gb))
    a = ga.plan_args(B=B, Hq=Hq, Hkv=Hkv, rows=rows, kv_offset=off, D=D, n_splits=n_splits)
    d = ga.describe_plan(a, 0)
    _say("partials", n_splits, d["n_splits"], d["partial_kind"], mag)
    assert d["n_splits"] == n_splits and d["partial_kind"] == kind
    out = ga.prefill(q, k, v, g, kv_offset=off, n_splits=n_splits)
    ws = torch.empty(d["workspace_bytes"], dtype=torch.uint8, device="cuda")
    out2, parts = ga.prefill_partials(q, k, v, g, kv_offset=off, n_splits=n_splits, workspace=ws)
    assert parts is not None and parts[0].shape == (n_splits, B, Hq, rows, D)
    assert parts[0].dtype == (torch.float16 if kind else torch.float32) and (parts[2] is None) == (kind == 0)
    ga.merge(parts[0], parts[1], g, out=out2, partial_exp=parts[2])
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    ref = reference.attention(*(syn.widen(x) for x in (qb, kb, vb, gb)), n_kv_heads=Hkv, kv_offset=off,
                              kv_len=off + rows)
    _say(assert_close(to_f64(out) / mag, ref / mag, f"split partials kind {kind}, |v|~{mag:g}"))



@needs_gpu
@pytest.mark.parametrize("n_chunks", [5, 21])
@pytest.mark.parametrize("D", [256, 64])
def test_merge_carrying_an_append(n_chunks, D):
    # attn_merge with a kv_append in the same launch (the prompt loop's merge of one block with
    # the next block's append): the merge's output bits and the cache bytes are those of the two
    # calls made one after the other; the rest of the cache is untouched
    rng = syn.streams(95)
    B, Hq, Hkv, rows, kv = 2, 8, 2, 7, 60
    q = syn.widen(syn.normal_bits(rng["q"], (B, Hq, rows, D)))
    k = syn.widen(syn.normal_bits(rng["k"], (B, Hkv, kv, D)))
    v = syn.widen(syn.normal_bits(rng["v"], (B, Hkv, kv, D)))
    gb = syn.normal_bits(rng["gate"], (B, Hq, rows, D))
    step = max(1, kv // n_chunks)
    chunks = [(c * step, kv if c == n_chunks - 1 else (c + 1) * step) for c in range(n_chunks)]
    o, l_ = reference.partials(q, k, v, n_kv_heads=Hkv, kv_offset=kv - rows, kv_len=kv, chunks=chunks)
    po = torch.from_numpy(o.astype(np.float32)).cuda()
    pl = torch.from_numpy(l_.astype(np.float32)).cuda()
    g = to_dev(gb)
    kn = to_dev(syn.normal_bits(rng["k"], (B, Hkv, 300, D)))
    vn = to_dev(syn.normal_bits(rng["v"], (B, Hkv, 300, D)))
    caches = []
    for carried in (False, True):
        kc = torch.full((B, Hkv, 1000, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        vc = torch.full_like(kc, float("nan"))
        out = torch.full((B, Hq, rows, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        if carried:
            ga.merge(po, pl, g, out=out, append=(kn, vn, kc, vc, 517))
        else:
            ga.merge(po, pl, g, out=out)
            ga.kv_append(kn, vn, kc, vc, kv_offset=517)
        torch.cuda.synchronize()
        caches.append((out, kc, vc))
    (o0, k0, v0), (o1, k1, v1) = caches
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))
    assert torch.equal(k0.view(torch.int16), k1.view(torch.int16)) and torch.equal(v0.view(torch.int16), v1.view(torch.int16))
    assert torch.equal(k1[:, :, 517:817].view(torch.int16), kn.view(torch.int16))
    assert torch.isnan(k1[:, :, :517].float()).all() and torch.isnan(v1[:, :, 817:].float()).all()
    _say(assert_close(to_f64(o1), reference.merge(o, l_, syn.widen(gb)), f"merge carrying an append, {n_chunks} chunks"))


@needs_gpu
@pytest.mark.parametrize("n_chunks", [12, 21, 40])
@pytest.mark.parametrize("fp16", [False, True])
def test_merge_of_many_chunks_over_many_rows(n_chunks, fp16):
    # 1024 rows (32 heads x 32 rows) fill the chip with one wavefront a row, so 9 to 64 chunks
    # (32 of fp32 partials) take the one-wavefront merge with 16, 32 or 64 slots; 40 fp32 chunks
    # take the many-wavefront one.  Against the oracle, with a row empty in every chunk.
    rng = syn.streams(97)
    D, B, Hq, Hkv, rows, kv = 64, 1, 32, 4, 32, 130
    q = syn.widen(syn.normal_bits(rng["q"], (B, Hq, rows, D)))
    k = syn.widen(syn.normal_bits(rng["k"], (B, Hkv, kv, D)))
    v = syn.widen(syn.normal_bits(rng["v"], (B, Hkv, kv, D)))
    gb = syn.normal_bits(rng["gate"], (B, Hq, rows, D))
    step = kv // n_chunks
    chunks = [(c * step, kv if c == n_chunks - 1 else (c + 1) * step) for c in range(n_chunks)]
    o, l_ = reference.partials(q, k, v, n_kv_heads=Hkv, kv_offset=kv - rows, kv_len=kv, chunks=chunks)
    l32 = l_.astype(np.float32)
    l32[:, 0, 5, 3] = -np.inf  # a row empty in every chunk: 0 whatever its partials hold
    o = o.copy()
    o[:, 0, 5, 3, :] = np.nan
    if fp16:
        vals16, exps, exact = _fp16_rows(o)
        po, pe = torch.from_numpy(vals16).cuda(), torch.from_numpy(exps).cuda()
    else:
        po, pe, exact = torch.from_numpy(o.astype(np.float32)).cuda(), None, o
    out = torch.full((B, Hq, rows, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    ga.merge(po, torch.from_numpy(l32).cuda(), to_dev(gb), out=out, partial_exp=pe)
    torch.cuda.synchronize()
    got = to_f64(out)
    assert np.all(got[0, 5, 3, :] == 0.0)
    ref = reference.merge(np.nan_to_num(o, nan=0.0), l_, syn.widen(gb))
    ref[0, 5, 3, :] = 0.0
    _say(assert_close(got, ref, f"merge of {n_chunks} chunks over 1024 rows, {'fp16' if fp16 else 'fp32'}"))


@needs_gpu
@pytest.mark.parametrize("n_splits", [1, 3])
@pytest.mark.parametrize("D", [256, 128])
def test_prefill_carrying_the_next_blocks_append(n_splits, D):
    # attn_prefill with attn_args append (the next query block's rows): in the merge's launch with
    # the keys split, in a launch of its own after the main pass without; the block's output and
    # both caches are those of the prefill and the kv_append made apart, bit for bit
    rng = syn.streams(99)
    B, Hq, Hkv, rows, off = 1, 8, 2, 40, 200
    qb = syn.normal_bits(rng["q"], (B, Hq, rows, D))
    gb = syn.normal_bits(rng["gate"], (B, Hq, rows, D))
    kb = syn.normal_bits(rng["k"], (B, Hkv, off + 2 * rows, D))
    vb = syn.normal_bits(rng["v"], (B, Hkv, off + 2 * rows, D))
    q, g = to_dev(qb), to_dev(gb)
    res = []
    for carried in (False, True):
        kc = torch.full((B, Hkv, off + 2 * rows, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        vc = torch.full_like(kc, float("nan"))
        kc[:, :, :off + rows] = to_dev(kb[:, :, :off + rows])
        vc[:, :, :off + rows] = to_dev(vb[:, :, :off + rows])
        kn, vn = to_dev(kb[:, :, off + rows:]), to_dev(vb[:, :, off + rows:])
        nxt = (kn, vn, kc, vc, off + rows)
        if carried:
            out = ga.prefill(q, kc, vc, g, kv_offset=off, n_splits=n_splits, append=nxt)
        else:
            out = ga.prefill(q, kc, vc, g, kv_offset=off, n_splits=n_splits)
            ga.kv_append(kn, vn, kc, vc, kv_offset=off + rows)
        torch.cuda.synchronize()
        res.append((out, kc, vc))
    (o0, k0, v0), (o1, k1, v1) = res
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))
    assert torch.equal(k1.view(torch.int16), to_dev(kb).view(torch.int16))
    assert torch.equal(v1.view(torch.int16), to_dev(vb).view(torch.int16))
    assert torch.equal(k0.view(torch.int16), k1.view(torch.int16)) and torch.equal(v0.view(torch.int16), v1.view(torch.int16))
    ref = reference.attention(*(syn.widen(x) for x in (qb, kb[:, :, :off + rows], vb[:, :, :off + rows], gb)),
                              n_kv_heads=Hkv, kv_offset=off, kv_len=off + rows)
    _say(assert_close(to_f64(o1), ref, f"prefill carrying an append, n_splits={n_splits}, D={D}"))


def _sampled_rows(o, qx, gx, kb, vb, off, rows_sel, Hkv, what):
    """Oracle rows one by one: row r of a block at kv_offset off sees keys 0 .. off + r."""
    ref = np.stack([reference.attention(syn.widen(qx[:, :, r:r + 1]), syn.widen(kb[:, :, :off + r + 1]),
                                        syn.widen(vb[:, :, :off + r + 1]), syn.widen(gx[:, :, r:r + 1]),
                                        n_kv_heads=Hkv, kv_offset=off + int(r), kv_len=off + int(r) + 1)[:, :, 0]
                    for r in rows_sel], axis=2)
    got = to_f64(o[:, :, torch.as_tensor(rows_sel, device=o.device)])
    _say(assert_close(got, ref, what))


@needs_gpu
@pytest.mark.parametrize("D", [256, 128])
def test_prefill_carrying_the_previous_blocks_merge(D):
    # Two 512-row query blocks of a 24/4-head prompt whose plans carry work in the main pass's
    # launch (5 splits of 96 and 100 tiles, fp16 partials, 16 idle CUs): block B's
    # attn_prefill_partials carries block A's merge (attn_args carry) and the next block's
    # append.  Block A's output is attn_merge's, block B's partials and output are those of the
    # calls made apart, and the caches those of a kv_append, all bit for bit; sampled rows of
    # both outputs match the oracle.
    rng = syn.streams(131)
    B, Hq, Hkv, rows = 1, 24, 4, 512
    off_a = 480 * (8192 // D) - rows
    off_b = off_a + rows
    kv = off_b + 2 * rows
    qb = syn.normal_bits(rng["q"], (B, Hq, 2 * rows, D))
    gb = syn.normal_bits(rng["gate"], (B, Hq, 2 * rows, D))
    kb = syn.normal_bits(rng["k"], (B, Hkv, kv, D))
    vb = syn.normal_bits(rng["v"], (B, Hkv, kv, D))
    q, g = to_dev(qb), to_dev(gb)
    qa, qb_, ga_, gb_ = q[:, :, :rows], q[:, :, rows:], g[:, :, :rows], g[:, :, rows:]
    for off in (off_a, off_b):
        d = ga.describe_plan(ga.plan_args(B=B, Hq=Hq, Hkv=Hkv, rows=rows, kv_offset=off, capacity=kv, D=D))
        _say("plan at", off, {k_: d[k_] for k_ in ("n_splits", "partial_kind", "grid_blocks", "carry_blocks")})
        assert d["carry_blocks"] > 0 and d["partial_kind"] == 1
    need = ga.workspace_bytes(ga.plan_args(B=B, Hq=Hq, Hkv=Hkv, rows=rows, kv_offset=off_b, capacity=kv, D=D))

    def caches():
        kc = torch.full((B, Hkv, kv, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        vc = torch.full_like(kc, float("nan"))
        kc[:, :, :off_b + rows] = to_dev(kb[:, :, :off_b + rows])
        vc[:, :, :off_b + rows] = to_dev(vb[:, :, :off_b + rows])
        return kc, vc

    kn, vn = to_dev(kb[:, :, off_b + rows:]), to_dev(vb[:, :, off_b + rows:])
    res = []
    for carried in (False, True):
        kc, vc = caches()
        ws = [torch.empty(need, dtype=torch.uint8, device="cuda") for _ in range(2)]
        oa = torch.full((B, Hq, rows, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        ob = torch.full_like(oa, float("nan"))
        _, pa = ga.prefill_partials(qa, kc, vc, ga_, kv_offset=off_a, out=oa, workspace=ws[0])
        if carried:
            _, pb = ga.prefill_partials(qb_, kc, vc, gb_, kv_offset=off_b, out=ob, workspace=ws[1],
                                        carry=(*pa, ga_, oa), append=(kn, vn, kc, vc, off_b + rows))
        else:
            ga.merge(pa[0], pa[1], ga_, out=oa, partial_exp=pa[2])
            _, pb = ga.prefill_partials(qb_, kc, vc, gb_, kv_offset=off_b, out=ob, workspace=ws[1])
            ga.kv_append(kn, vn, kc, vc, kv_offset=off_b + rows)
        parts = [t.clone() for t in pb]
        ga.merge(pb[0], pb[1], gb_, out=ob, partial_exp=pb[2])
        torch.cuda.synchronize()
        res.append((oa, ob, parts, kc, vc))
    (oa0, ob0, p0, k0, v0), (oa1, ob1, p1, k1, v1) = res
    assert torch.equal(oa0.view(torch.int16), oa1.view(torch.int16)), "carried merge differs from attn_merge"
    assert torch.equal(ob0.view(torch.int16), ob1.view(torch.int16))
    for x, y in zip(p0, p1):
        assert torch.equal(x.view(torch.int32) if x.element_size() == 4 else x.view(torch.int16),
                           y.view(torch.int32) if y.element_size() == 4 else y.view(torch.int16))
    assert torch.equal(k1.view(torch.int16), to_dev(kb).view(torch.int16))
    assert torch.equal(v1.view(torch.int16), to_dev(vb).view(torch.int16))
    sel = np.unique(np.concatenate([[0, 1, 255, 511], np.random.default_rng(D).choice(rows, 12, replace=False)]))
    _sampled_rows(oa1, qb[:, :, :rows], gb[:, :, :rows], kb, vb, off_a, sel, Hkv, f"block A (D={D}), merge carried")
    _sampled_rows(ob1, qb[:, :, rows:], gb[:, :, rows:], kb, vb, off_b, sel, Hkv, f"block B (D={D})")


@needs_gpu
def test_prompt_with_carried_merges_matches_the_plain_loop():
    # prompt_prefill over 4 blocks of 1024 rows (24/4 heads, 2 splits, 64 idle CUs): with
    # carry_merge the blocks whose plans carry work (blocks 2 and 3: 48 tiles per split and more)
    # take the previous block's merge and the next block's append in their main pass's launch; the
    # output and the caches are those of the loop of attn_prefill calls, bit for bit, and sampled
    # rows match the oracle
    _say("prompt with carried merges")
    N = 4096
    carrying = [ga.describe_plan(ga.plan_args(B=1, Hq=24, Hkv=4, rows=1024, kv_offset=s, capacity=N))["carry_blocks"]
                for s in range(0, N, 1024)]
    assert carrying[0] == 0 and carrying[2] > 0 and carrying[3] > 0, carrying
    qb, kb, vb, gb, _ = prompt(2200, B=1, Hq=24, Hkv=4, N=N)
    q, k, v, g = (to_dev(x) for x in (qb, kb, vb, gb))
    outs = []
    for carry in (False, True):
        kc = torch.full((1, 4, N, 256), float("nan"), dtype=q.dtype, device="cuda")
        vc = torch.full_like(kc, float("nan"))
        out = torch.full_like(q, float("nan"))
        ga.prompt_prefill(q, k, v, g, kc, vc, q_block=1024, out=out, carry_merge=carry)
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(kc), kb) and np.array_equal(to_bits(vc), vb)
        outs.append(out)
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    rows = np.unique(np.concatenate([[0, 1023, 1024, 2047, 2048, 3071, 3072, 4095],
                                     np.random.default_rng(5).choice(N, 10, replace=False)]))
    k64, v64 = syn.widen(kb), syn.widen(vb)
    ref = np.stack([reference.attention(syn.widen(qb[:, :, r:r + 1]), k64, v64, syn.widen(gb[:, :, r:r + 1]),
                                        n_kv_heads=4, kv_offset=int(r), kv_len=int(r) + 1)[:, :, 0] for r in rows],
                   axis=2)
    got = to_f64(outs[1][:, :, torch.as_tensor(rows, device="cuda")])
    _say(assert_close(got, ref, "prompt with carried merges, sampled rows"))
