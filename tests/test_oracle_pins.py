"""Pins of the float64 oracle against things other than itself (CPU only).

* brute force: Python loops with math.fsum / math.exp on tiny inputs;
* a library special case: torch's CPU float64 scaled_dot_product_attention
  with an explicit boolean mask and K/V repeated over each head group;
* closed forms: one admissible key, constant V, Q = 0, gate = 0;
* invariants: rows of p sum to 1, future keys get 0, head-chunked equals
  unchunked, query blocks equal the whole prompt, a KV split plus the merge
  equals the unsplit result, a masked -Inf value times probability 0 is not NaN.
"""

import math

import numpy as np
import pytest
import torch

from oracle import brute, plan, reference
from synth import inputs as syn

D = 256


def _tiny(seed, B=1, Hq=4, Hkv=2, rows=5, kv_offset=3, dim=D, cap_extra=0, scale_v=1.0):
    rng = syn.streams(seed)
    kv_len = kv_offset + rows
    q = syn.widen(syn.normal_bits(rng["q"], (B, Hq, rows, dim)))
    k = syn.widen(syn.normal_bits(rng["k"], (B, Hkv, kv_len + cap_extra, dim)))
    v = syn.widen(syn.normal_bits(rng["v"], (B, Hkv, kv_len + cap_extra, dim), scale=scale_v))
    g = syn.widen(syn.normal_bits(rng["gate"], (B, Hq, rows, dim)))
    return q, k, v, g, kv_len


def _rel(a, b):
    a, b = np.asarray(a), np.asarray(b)
    return float(np.max(np.abs(a - b)) / max(1e-300, float(np.max(np.abs(b)))))


TINY_CASES = [
    # (B, Hq, Hkv, rows, kv_offset, causal, dim, mask)
    (1, 4, 2, 5, 0, True, D, None),
    (2, 6, 2, 4, 7, True, D, None),
    (1, 3, 3, 3, 2, False, D, None),
    (1, 8, 1, 6, 9, True, 4, None),
    (2, 4, 2, 3, 5, True, D, "bool_bcast"),
    (1, 4, 2, 4, 6, True, D, "add_full"),
    (2, 2, 1, 4, 3, True, 4, "add_bcast"),
]


def _mask_for(kind, rng, B, Hq, rows, kv_len):
    if kind is None:
        return None, None
    if kind == "bool_bcast":
        m = rng.random((1, 1, rows, kv_len)) > 0.3
        return m, "bool"
    if kind == "add_full":
        m = np.where(rng.random((1, Hq, rows, kv_len)) > 0.3, rng.standard_normal((1, Hq, rows, kv_len)), -np.inf)
        return m, "add"
    if kind == "add_bcast":
        m = np.where(rng.random((B, 1, rows, kv_len)) > 0.25, 0.5 * rng.standard_normal((B, 1, rows, kv_len)), -np.inf)
        return m, "add"
    raise ValueError(kind)


@pytest.mark.parametrize("case", range(len(TINY_CASES)))
def test_brute_force_agrees(case):
    B, Hq, Hkv, rows, off, causal, dim, mkind = TINY_CASES[case]
    q, k, v, g, kv_len = _tiny(10 + case, B, Hq, Hkv, rows, off, dim)
    mask, kind = _mask_for(mkind, np.random.default_rng(case), B, Hq, rows, kv_len)
    ref = reference.attention(q, k, v, g, n_kv_heads=Hkv, kv_offset=off, kv_len=kv_len, causal=causal,
                              mask=mask, mask_kind=kind)
    bf = np.array(brute.attention(q.tolist(), k.tolist(), v.tolist(), g.tolist(), n_kv_heads=Hkv, kv_offset=off,
                                  kv_len=kv_len, causal=causal, mask=None if mask is None else mask.tolist(),
                                  mask_kind=kind))
    assert _rel(ref, bf) <= 1e-12


def _torch_sdpa(q, k, v, g, Hkv, off, kv_len, causal, mask=None, kind=None):
    B, Hq, R, Dd = q.shape
    G = Hq // Hkv
    qt = torch.from_numpy(q)
    kt = torch.from_numpy(k[:, :, :kv_len]).repeat_interleave(G, dim=1)
    vt = torch.from_numpy(v[:, :, :kv_len]).repeat_interleave(G, dim=1)
    allow = torch.ones(B, Hq, R, kv_len, dtype=torch.bool)
    if causal:
        j = torch.arange(kv_len)[None, :]
        r = torch.arange(R)[:, None]
        allow &= (j <= off + r)[None, None]
    add = None
    if mask is not None:
        mt = torch.from_numpy(np.asarray(mask))
        if kind == "bool":
            allow &= mt.expand(B, Hq, R, kv_len)
        else:
            allow &= torch.isfinite(mt).expand(B, Hq, R, kv_len)
            add = torch.where(torch.isfinite(mt), mt, torch.zeros_like(mt)).expand(B, Hq, R, kv_len)
    if add is None:
        attn_mask = allow
    else:
        attn_mask = torch.where(allow, add, torch.full_like(add, -math.inf))
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=attn_mask, scale=1.0 / math.sqrt(Dd))
    return (o * torch.sigmoid(torch.from_numpy(g))).numpy()


@pytest.mark.parametrize("B,Hq,Hkv,rows,off,causal,mkind", [
    (1, 24, 4, 40, 0, True, None),
    (2, 16, 2, 9, 70, True, None),
    (1, 16, 2, 32, 100, True, "add_full"),
    (1, 6, 2, 17, 33, False, "bool_bcast"),
])
def test_torch_sdpa_agrees(B, Hq, Hkv, rows, off, causal, mkind):
    q, k, v, g, kv_len = _tiny(77 + rows, B, Hq, Hkv, rows, off)
    mask, kind = _mask_for(mkind, np.random.default_rng(rows), B, Hq, rows, kv_len)
    if mask is not None:  # every row keeps its own key so no row is empty
        for r in range(rows):
            if kind == "bool":
                mask[..., r, off + r] = True
            else:
                mask[..., r, off + r] = 0.0
    ref = reference.attention(q, k, v, g, n_kv_heads=Hkv, kv_offset=off, kv_len=kv_len, causal=causal,
                              mask=mask, mask_kind=kind)
    ts = _torch_sdpa(q, k, v, g, Hkv, off, kv_len, causal, mask, kind)
    assert _rel(ref, ts) <= 1e-12


def test_closed_form_single_key():
    # row 0 of a causal prefill at offset 0 sees key 0 only: out = V_0 * sigmoid(gate)
    q, k, v, g, kv_len = _tiny(3, 1, 6, 2, 8, 0)
    out = reference.attention(q, k, v, g, n_kv_heads=2, kv_offset=0, kv_len=kv_len)
    for h in range(6):
        np.testing.assert_array_equal(out[0, h, 0], v[0, h // 3, 0] * reference.sigmoid(g[0, h, 0]))


def test_closed_form_constant_v():
    q, k, v, g, kv_len = _tiny(4, 1, 4, 2, 6, 11)
    v[:] = 0.75
    out = reference.attention(q, k, v, g, n_kv_heads=2, kv_offset=11, kv_len=kv_len)
    np.testing.assert_allclose(out, 0.75 * reference.sigmoid(g), rtol=1e-14, atol=0)


def test_closed_form_zero_q_is_prefix_mean():
    q, k, v, g, kv_len = _tiny(5, 1, 4, 2, 5, 4)
    q[:] = 0.0
    out = reference.attention(q, k, v, None, n_kv_heads=2, kv_offset=4, kv_len=kv_len)
    for h in range(4):
        for r in range(5):
            np.testing.assert_allclose(out[0, h, r], v[0, h // 2, :4 + r + 1].mean(axis=0), rtol=1e-13, atol=1e-15)


def test_closed_form_zero_gate_halves():
    q, k, v, g, kv_len = _tiny(6, 1, 4, 2, 5, 4)
    ungated = reference.attention(q, k, v, None, n_kv_heads=2, kv_offset=4, kv_len=kv_len)
    gated = reference.attention(q, k, v, np.zeros_like(g), n_kv_heads=2, kv_offset=4, kv_len=kv_len)
    np.testing.assert_array_equal(gated, ungated / 2)


def test_probabilities_sum_to_one_and_future_is_zero():
    q, k, v, g, kv_len = _tiny(7, 1, 4, 2, 9, 13)
    for h in range(4):
        p = reference.probabilities(q, k, n_kv_heads=2, kv_offset=13, kv_len=kv_len, h=h)
        np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)
        for r in range(9):
            assert np.all(p[r, 13 + r + 1:] == 0.0)
            assert np.all(p[r, :13 + r + 1] > 0.0)


@pytest.mark.parametrize("case", range(len(TINY_CASES)))
def test_probabilities_agree_with_brute_force(case):
    # every head of every group, against math.fsum / math.exp loops (the mask cases carry finite
    # nonzero additive values, and GQA groups of 2, 3, 4 and 8 heads)
    B, Hq, Hkv, rows, off, causal, dim, mkind = TINY_CASES[case]
    q, k, v, g, kv_len = _tiny(40 + case, B, Hq, Hkv, rows, off, dim)
    mask, kind = _mask_for(mkind, np.random.default_rng(50 + case), B, Hq, rows, kv_len)
    for b in range(B):
        for h in range(Hq):
            ref = reference.probabilities(q, k, n_kv_heads=Hkv, kv_offset=off, kv_len=kv_len, causal=causal,
                                          mask=mask, mask_kind=kind, b=b, h=h)
            bf = np.array(brute.probabilities(q.tolist(), k.tolist(), n_kv_heads=Hkv, kv_offset=off, kv_len=kv_len,
                                              causal=causal, mask=None if mask is None else mask.tolist(),
                                              mask_kind=kind, b=b, h=h))
            assert np.max(np.abs(ref - bf)) <= 1e-13


def test_probabilities_controls_are_caught():
    # planted mistakes in the weights (a wrong scale; the wrong KV head for a query head) must
    # miss the brute-force weights by far more than rounding
    B, Hq, Hkv, rows, off = 1, 8, 2, 5, 6
    q, k, v, g, kv_len = _tiny(60, B, Hq, Hkv, rows, off)
    bf = [np.array(brute.probabilities(q.tolist(), k.tolist(), n_kv_heads=Hkv, kv_offset=off, kv_len=kv_len, h=h))
          for h in range(Hq)]
    for h in range(Hq):
        wrong_scale = reference.probabilities(q, k, n_kv_heads=Hkv, kv_offset=off, kv_len=kv_len, h=h, scale=1 / 8)
        assert np.max(np.abs(wrong_scale - bf[h])) > 1e-3
        # h % Hkv instead of h // G: the other group's keys (for heads whose group changes)
        k_swapped = k[:, ::-1].copy()
        if (h % Hkv) != (h // (Hq // Hkv)):
            wrong_group = reference.probabilities(q, k_swapped, n_kv_heads=Hkv, kv_offset=off, kv_len=kv_len, h=h)
            assert np.max(np.abs(wrong_group - bf[h])) > 1e-3


@pytest.mark.parametrize("rows,G", [(4, 12), (6, 6), (9, 8), (32, 8), (5, 8)])
def test_head_chunked_equals_unchunked_bitwise(rows, G):
    Hkv = 2
    q, k, v, g, kv_len = _tiny(8 + rows, 1, G * Hkv, Hkv, rows, 20)
    mask = np.where(np.random.default_rng(rows).random((1, G * Hkv, rows, kv_len)) > 0.2, 0.0, -np.inf)
    for r in range(rows):
        mask[..., r, 20 + r] = 0.0
    kw = dict(kv_offset=20, kv_len=kv_len, mask=mask, mask_kind="add")
    full = reference.attention(q, k, v, g, n_kv_heads=Hkv, **kw)
    sizes = plan.head_chunk_sizes(rows, G * Hkv, Hkv)
    chunked = reference.head_chunked(q, k, v, g, n_kv_heads=Hkv, chunk_sizes=sizes, **kw)
    np.testing.assert_array_equal(chunked, full)
    # every forced chunk size too
    for c in range(1, G + 1):
        forced = [c] * (G // c) + ([G % c] if G % c else [])
        np.testing.assert_array_equal(reference.head_chunked(q, k, v, g, n_kv_heads=Hkv, chunk_sizes=forced, **kw), full)


def test_query_blocks_equal_whole_prompt_bitwise():
    q, k, v, g, N = _tiny(9, 1, 4, 2, 48, 0)
    whole = reference.attention(q, k, v, g, n_kv_heads=2, kv_offset=0, kv_len=N)
    for qL in (8, 16, 48):
        parts = [reference.attention(q[:, :, s:s + qL], k, v, g[:, :, s:s + qL], n_kv_heads=2, kv_offset=s,
                                     kv_len=s + qL) for s in range(0, N, qL)]
        np.testing.assert_array_equal(np.concatenate(parts, axis=2), whole)


@pytest.mark.parametrize("chunks", [[(0, 7), (7, 19), (19, 30)], [(0, 1), (1, 30)], [(0, 16), (16, 40)]])
def test_split_and_merge_equals_unsplit(chunks):
    q, k, v, g, kv_len = _tiny(10, 2, 4, 2, 6, 24)
    full = reference.attention(q, k, v, g, n_kv_heads=2, kv_offset=24, kv_len=kv_len)
    o, l_ = reference.partials(q, k, v, n_kv_heads=2, kv_offset=24, kv_len=kv_len, chunks=chunks)
    merged = reference.merge(o, l_, g)
    assert _rel(merged, full) <= 1e-13


def test_split_and_merge_keeps_nonfinite_classes():
    # a +Inf key score in one chunk (NaN rows in the unsplit definition: exp(Inf - Inf)) and a
    # +Inf in V at a visible key (+Inf in that dim): the merge of the chunk partials gives the
    # classes of the unsplit result, and its finite values
    q, k, v, g, kv_len = _tiny(12, 1, 4, 2, 6, 24)
    k = k.copy()
    v = v.copy()
    k[0, 0, 10, 0] = np.inf
    q[0, 0:2, :, 0] = np.abs(q[0, 0:2, :, 0]) + 0.5   # heads 0 and 1 see s = +Inf at key 10
    v[0, 1, 5, 3] = np.inf
    full = reference.attention(q, k, v, g, n_kv_heads=2, kv_offset=24, kv_len=kv_len)
    assert np.isnan(full[0, 0:2]).all() and np.isposinf(full[0, 2:4, :, 3]).all()
    for chunks in ([(0, 7), (7, 19), (19, 30)], [(0, 11), (11, 30)]):
        o, l_ = reference.partials(q, k, v, n_kv_heads=2, kv_offset=24, kv_len=kv_len, chunks=chunks)
        merged = reference.merge(o, l_, g)
        fin = np.isfinite(full)
        assert np.array_equal(np.isnan(merged), np.isnan(full))
        assert np.array_equal(merged[~fin & ~np.isnan(full)], full[~fin & ~np.isnan(full)])
        assert np.max(np.abs(merged[fin] - full[fin])) <= 1e-12


def test_merge_of_empty_chunks_is_zero():
    o = np.zeros((3, 1, 1, 2, 4))
    l_ = np.full((3, 1, 1, 2), -np.inf)
    np.testing.assert_array_equal(reference.merge(o, l_, np.zeros((1, 1, 2, 4))), 0.0)


def test_empty_row_is_zero():
    q, k, v, g, kv_len = _tiny(11, 1, 2, 1, 3, 2)
    mask = np.ones((1, 1, 3, kv_len), dtype=bool)
    mask[0, 0, 1, :] = False
    out = reference.attention(q, k, v, g, n_kv_heads=1, kv_offset=2, kv_len=kv_len, mask=mask, mask_kind="bool")
    assert np.all(out[0, :, 1] == 0.0)
    assert np.all(out[0, :, 0] != 0.0)


def test_masked_nonfinite_value_does_not_leak():
    # -Inf in V at a masked (future) key, +Inf at a visible key: expect +Inf, not NaN
    q, k, v, g, kv_len = _tiny(12, 1, 2, 1, 2, 3)
    v[0, 0, 3 + 1, 0] = -np.inf     # key 4 is in row 0's future
    v[0, 0, 1, 1] = np.inf          # key 1 is visible to both rows
    out = reference.attention(q, k, v, None, n_kv_heads=1, kv_offset=3, kv_len=kv_len)
    assert np.all(np.isfinite(out[0, :, 0, 0]))
    assert np.all(out[0, :, :, 1] == np.inf)
    assert not np.isnan(out).any()


def test_scale_default_is_one_over_sixteen():
    q, k, v, g, kv_len = _tiny(13, 1, 2, 1, 3, 2)
    a = reference.attention(q, k, v, g, n_kv_heads=1, kv_offset=2, kv_len=kv_len)
    b = reference.attention(q, k, v, g, n_kv_heads=1, kv_offset=2, kv_len=kv_len, scale=0.0625)
    np.testing.assert_array_equal(a, b)


def test_kv_keep_moves_kept_rows_in_order():
    # pins from the definition, written out by hand: a chain (rows 0..n-1 kept) leaves the cache
    # unchanged; a tree path {1, 3, 4} lands at offsets 0, 1, 2 in that order; the rows after
    # the kept ones and everything outside the block stay; NaN payloads and -0 survive
    nf = syn.nonfinite_bits("bf16")
    cache = np.arange(2 * 1 * 12 * 4, dtype=np.uint16).reshape(2, 1, 12, 4)
    cache[0, 0, 7, 0] = nf["nan"]
    cache[1, 0, 5, 3] = nf["-0"]
    off, rows = 3, 6                        # block rows are cache rows 3..8
    chain = reference.kv_keep(cache, off, rows, [0b111, 0b111111])
    np.testing.assert_array_equal(chain, cache)
    out = reference.kv_keep(cache, off, rows, [0b011010, 0b000001])
    want = cache.copy()
    want[0, 0, 3] = cache[0, 0, 4]          # row 1 -> slot 0
    want[0, 0, 4] = cache[0, 0, 6]          # row 3 -> slot 1
    want[0, 0, 5] = cache[0, 0, 7]          # row 4 -> slot 2 (carries the NaN payload)
    np.testing.assert_array_equal(out, want)
    assert out[0, 0, 5, 0] == nf["nan"] and out[1, 0, 5, 3] == nf["-0"]
    # a second keep on the cache the first left: keep slots {0, 2} of the 3 kept rows
    twice = reference.kv_keep(out, off, 3, [0b101, 0b1])
    want2 = out.copy()
    want2[0, 0, 4] = out[0, 0, 5]
    np.testing.assert_array_equal(twice, want2)
    with pytest.raises(ValueError):
        reference.kv_keep(cache, off, rows, [1 << rows, 0])
    with pytest.raises(ValueError):
        reference.kv_keep(cache, 8, rows, [1, 1])


def test_kv_append_is_a_bit_copy():
    nf = syn.nonfinite_bits("bf16")
    cache = np.zeros((1, 2, 8, 4), dtype=np.uint16)
    new = np.array([[[[nf["-0"], nf["nan"], nf["+inf"], 0x1234]]], [[[nf["-inf"], 1, 2, 3]]]], dtype=np.uint16)
    new = new.reshape(1, 2, 1, 4)
    out = reference.kv_append(cache, new, 5)
    assert out[0, 0, 5, 0] == 0x8000 and out[0, 0, 5, 1] == nf["nan"] and out[0, 1, 5, 0] == nf["-inf"]
    assert np.all(out[:, :, :5] == 0) and np.all(out[:, :, 6:] == 0)
    with pytest.raises(ValueError):
        reference.kv_append(cache, new, 8)
