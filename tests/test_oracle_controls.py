"""Planted mistakes in the oracle must be caught by the parity comparison (CPU only).

TensorFold PR #1009 (attention kernel-contract commit; Receipt, "Attention")
runs three controls that must go red: a row that sees one key beyond its causal bound, a
merge dropping later tail chunks, and an append one row late.  Each is planted
here in a copy of the oracle's behaviour, with inputs built so the mistake is
large, and the comparison used by the GPU parity tests must flag it.
"""

import numpy as np

from oracle import reference
from synth import inputs as syn
from tests.parity import MAX_ABS, compare

B, HQ, HKV, ROWS, OFF = 1, 8, 2, 6, 40
G = HQ // HKV


def _inputs(seed):
    rng = syn.streams(seed)
    kv_len = OFF + ROWS
    q = syn.widen(syn.normal_bits(rng["q"], (B, HQ, ROWS, 256)))
    k = syn.widen(syn.normal_bits(rng["k"], (B, HKV, kv_len + 1, 256)))
    v = syn.widen(syn.normal_bits(rng["v"], (B, HKV, kv_len + 1, 256)))
    g = syn.widen(syn.normal_bits(rng["gate"], (B, HQ, ROWS, 256)))
    return q, k, v, g, kv_len


def test_control_row_sees_one_key_past_its_own(monkeypatch):
    q, k, v, g, kv_len = _inputs(21)
    # plant: every row's query points at the key right after its own position
    for h in range(HQ):
        for r in range(ROWS - 1):
            q[0, h, r] = 0.5 * k[0, h // G, OFF + r + 1]
    good = reference.attention(q, k, v, g, n_kv_heads=HKV, kv_offset=OFF, kv_len=kv_len)
    orig = reference.causal_keep

    def one_past(row_index, kv_offset, kv_len_, causal):
        return orig(np.asarray(row_index) + 1, kv_offset, kv_len_, causal)

    monkeypatch.setattr(reference, "causal_keep", one_past)
    bad = reference.attention(q, k, v, g, n_kv_heads=HKV, kv_offset=OFF, kv_len=kv_len)
    res = compare(bad, good)
    assert not res["ok"] and res["max_abs"] > 10 * MAX_ABS


def test_control_merge_drops_last_chunk():
    q, k, v, g, kv_len = _inputs(22)
    # plant: a dominant key in the last chunk for every row
    for h in range(HQ):
        for r in range(ROWS):
            q[0, h, r] = 0.5 * k[0, h // G, OFF - 2]
    chunks = [(0, 16), (16, 32), (32, kv_len)]
    o, l_ = reference.partials(q, k, v, n_kv_heads=HKV, kv_offset=OFF, kv_len=kv_len, chunks=chunks)
    good = reference.merge(o, l_, g)
    bad = reference.merge(o[:-1], l_[:-1], g)
    res = compare(bad, good)
    assert not res["ok"] and res["max_abs"] > 10 * MAX_ABS
    assert compare(good, reference.attention(q, k, v, g, n_kv_heads=HKV, kv_offset=OFF, kv_len=kv_len))["ok"]


def test_control_append_one_row_late():
    q, k, v, g, kv_len = _inputs(23)
    rng = syn.streams(99)
    cache_k = np.zeros((B, HKV, kv_len + 1, 256), dtype=np.uint16)
    cache_v = np.zeros_like(cache_k)
    cache_k[:, :, :OFF] = syn.normal_bits(rng["k"], (B, HKV, OFF, 256))
    cache_v[:, :, :OFF] = syn.normal_bits(rng["v"], (B, HKV, OFF, 256))
    new_k = syn.normal_bits(rng["k"], (B, HKV, ROWS, 256))
    new_v = syn.normal_bits(rng["v"], (B, HKV, ROWS, 256))
    kk = syn.widen(reference.kv_append(cache_k, new_k, OFF))
    # plant: each row's query points at its own (new) key
    for h in range(HQ):
        for r in range(ROWS):
            q[0, h, r] = 0.5 * kk[0, h // G, OFF + r]
    good = reference.attention(q, kk, syn.widen(reference.kv_append(cache_v, new_v, OFF)), g, n_kv_heads=HKV,
                               kv_offset=OFF, kv_len=kv_len)
    bad = reference.attention(q, syn.widen(reference.kv_append(cache_k, new_k, OFF + 1)),
                              syn.widen(reference.kv_append(cache_v, new_v, OFF + 1)), g, n_kv_heads=HKV,
                              kv_offset=OFF, kv_len=kv_len)
    res = compare(bad, good)
    assert not res["ok"] and res["max_abs"] > 10 * MAX_ABS
