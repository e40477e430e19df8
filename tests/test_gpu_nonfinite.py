"""Nonfinite values on the HIP path: keys a row cannot see never reach its output.

The definition sums over the admissible keys only, so a +-Inf or NaN planted in V (or K) at a
key that a row cannot see (its future, or hidden by the mask) must leave that row finite,
while the same value at a key the row sees spreads as it does in float64 (TensorFold PR #1009,
attention kernel-contract commit: masked -Inf times a zero probability must not become NaN).
Results are compared with the float64 oracle: nonfinite elements by class, the rest within
the tolerance.  Every head-chunk variant is compared with the oracle on its own: a pair whose
workgroup runs on past the pair's own keys (for other pairs) may meet a hidden nonfinite value
there and be recomputed exactly, so with nonfinite inputs the variants agree within the
tolerance, not bit for bit (with finite inputs they agree bit for bit).
"""

import numpy as np
import pytest
import torch

import gqa_causal_attention_attn_amd as ga
from oracle import reference
from synth import inputs as syn
from tests.gpu_util import prompt, to_bits, to_dev
from tests.parity import compare

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")

# 16-bit patterns of +Inf, -Inf and a quiet NaN
BITS = {"bf16": {"+inf": 0x7F80, "-inf": 0xFF80, "nan": 0x7FC0},
        "f16": {"+inf": 0x7C00, "-inf": 0xFC00, "nan": 0x7E00}}


def _say(*a):
    print(*a, flush=True)


def _check(got_bits, ref, dtype, what):
    res = compare(syn.widen(got_bits, dtype), ref)
    _say(what, res)
    assert res["ok"], f"{what}: {res}"
    return res


@needs_gpu
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("n_splits", [1, 3])
def test_prefill_future_keys_with_nonfinite_values(dtype, n_splits):
    # 24 query heads over 4 KV heads, 128 causal rows in one block.  Planted values sit in
    # diagonal tiles, where the rows before the key share its tile but must not see it.
    _say("nonfinite prefill", dtype, n_splits)
    B, Hq, Hkv, N = 1, 24, 4, 128
    qb, kb, vb, gb, _ = prompt(4100, B=B, Hq=Hq, Hkv=Hkv, N=N, dtype=dtype)
    t = BITS[dtype]
    vb[0, 1, 50, 7] = t["+inf"]
    vb[0, 2, 70, 100] = t["-inf"]
    vb[0, 3, 90, 200] = t["nan"]
    kb[0, 0, 60, 3] = t["+inf"]     # score +-Inf for the rows that see key 60
    vb[0, 0, 127, :] = t["nan"]     # only the last row sees key 127
    q, k, v, g = (to_dev(x, dtype) for x in (qb, kb, vb, gb))
    out = torch.full_like(q, float("nan"))
    ga.prefill(q, k, v, g, kv_offset=0, kv_len=N, out=out, n_splits=n_splits)
    torch.cuda.synchronize()
    ref = reference.attention(*(syn.widen(x, dtype) for x in (qb, kb, vb, gb)), n_kv_heads=Hkv, kv_offset=0,
                              kv_len=N)
    # the planted rows' future stays finite in the oracle, and spreads where it is seen
    assert np.isfinite(ref[0, 6:12, :50]).all() and np.isposinf(ref[0, 6:12, 50:, 7]).all()
    assert np.isnan(ref[0, 18:24, 90:, 200]).all() and np.isfinite(ref[0, 18:24, :90]).all()
    _check(to_bits(out), ref, dtype, "nonfinite prefill")
    for hc in (1, 4):
        o2 = torch.full_like(q, float("nan"))
        ga.prefill(q, k, v, g, kv_offset=0, kv_len=N, out=o2, n_splits=n_splits, head_chunk=hc)
        torch.cuda.synchronize()
        _check(to_bits(o2), ref, dtype, f"nonfinite prefill, head_chunk {hc}")


@needs_gpu
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("rows", [1, 4, 17])
def test_verify_hidden_keys_with_nonfinite_values(dtype, rows):
    # batch 2, 16 query heads over 2 KV heads at offset 4097, broadcast additive mask; keys the
    # mask hides from some rows hold +-Inf / NaN in V and +Inf in K: the rows that cannot see
    # them stay finite, the rows that see them follow float64
    _say("nonfinite verify", dtype, rows)
    B, Hq, Hkv, off = 2, 16, 2, 4097
    kv_len = off + rows
    rng = syn.streams(4200 + rows)
    qb = syn.normal_bits(rng["q"], (B, Hq, rows, 256), dtype)
    gb = syn.normal_bits(rng["gate"], (B, Hq, rows, 256), dtype)
    kb = syn.normal_bits(rng["k"], (B, Hkv, kv_len, 256), dtype)
    vb = syn.normal_bits(rng["v"], (B, Hkv, kv_len, 256), dtype)
    mb = syn.verify_mask(rng["mask"], rows=rows, kv_offset=off, heads=1, kind="add", dtype=dtype)
    hidden = np.nonzero(syn.widen(mb, dtype)[0, 0].min(axis=0) == -np.inf)[0]  # hidden from some row
    assert hidden.size > 20
    t = BITS[dtype]
    pick = np.random.default_rng(rows).choice(hidden, size=12, replace=False)
    for i, j in enumerate(pick):
        vb[i % B, (i // B) % Hkv, j, (37 * i) % 256] = (t["+inf"], t["-inf"], t["nan"])[i % 3]
        kb[i % B, (i // B) % Hkv, j, (11 * i) % 256] = t["+inf"]
    q, k, v, g, m = (to_dev(x, dtype) for x in (qb, kb, vb, gb, mb))
    ref = reference.attention(*(syn.widen(x, dtype) for x in (qb, kb, vb, gb)), n_kv_heads=Hkv, kv_offset=off,
                              kv_len=kv_len, mask=syn.widen(mb, dtype), mask_kind="add")
    # rows that see none of the planted keys are finite in the oracle
    blind = ~(syn.widen(mb, dtype)[0, 0][:, pick] > -np.inf).any(axis=1)
    assert np.isfinite(ref[:, :, blind]).all()
    for hc in (0, 1, 3, 8):
        _check(to_bits(ga.decode(q, k, v, g, kv_offset=off, mask=m, head_chunk=hc)), ref, dtype,
               f"nonfinite verify, head_chunk {hc}")


@needs_gpu
def test_decode_visible_infinity_spreads_and_hidden_one_does_not():
    # one decode row over a 4000-key cache split many ways: +Inf in V at a key the row sees
    # gives +Inf in that dim (every head of the group); the same at a key past kv_len (inside
    # the last tile) changes nothing
    _say("nonfinite decode")
    B, Hq, Hkv, kv_len, cap = 1, 16, 2, 4000, 4032
    rng = syn.streams(4300)
    qb = syn.normal_bits(rng["q"], (B, Hq, 1, 256))
    gb = syn.normal_bits(rng["gate"], (B, Hq, 1, 256))
    kb = syn.normal_bits(rng["k"], (B, Hkv, cap, 256))
    vb = syn.normal_bits(rng["v"], (B, Hkv, cap, 256))
    vb[0, 0, 1234, 9] = BITS["bf16"]["+inf"]
    vb[0, 1, 4010, :] = BITS["bf16"]["nan"]   # beyond kv_len
    kb[0, 1, 4011, :] = BITS["bf16"]["+inf"]
    q, k, v, g = (to_dev(x) for x in (qb, kb, vb, gb))
    out = ga.decode(q, k, v, g, kv_offset=kv_len - 1, kv_len=kv_len)
    ref = reference.attention(*(syn.widen(x) for x in (qb, kb, vb, gb)), n_kv_heads=Hkv, kv_offset=kv_len - 1,
                              kv_len=kv_len)
    assert np.isposinf(ref[0, :8, 0, 9]).all() and np.isfinite(ref[0, 8:]).all()
    _check(to_bits(out), ref, "bf16", "nonfinite decode")
