"""Precision separation: the tolerance must catch low-precision score sums (CPU only).

TensorFold PR #1009 (Receipt, "Attention") wants attention stress inputs on
which fp16 score sums fail outright and bf16 sums fail by a large factor while
fp32 passes.  Here the oracle's score step is re-evaluated with the
dot products accumulated sequentially in bf16, fp16 and fp32 on the stress
inputs from ``synth.stress_cancellation``; the rest of the definition is the
oracle's own.  bf16 must miss the max-abs tolerance by at least 100x, fp16 must
give nonfinite results, fp32 must pass.
"""

import numpy as np
import pytest

from oracle import reference
from synth import inputs as syn
from tests.parity import MAX_ABS, compare

B, HQ, HKV, ROWS, OFF = 1, 4, 2, 8, 24


def _round(x, kind):
    x = np.asarray(x, dtype=np.float32)
    if kind == "bf16":
        return syn.bits_to_f32(syn.f32_to_bits(x, "bf16"), "bf16")
    if kind == "f16":
        with np.errstate(over="ignore"):
            return x.astype(np.float16).astype(np.float32)
    return x


def _scores_accumulated(q, k, kind):
    """s[r, j] = sum_d q[r, d] k[j, d] accumulated in order d = 0..255, rounding every partial sum."""
    acc = np.zeros((q.shape[0], k.shape[0]), dtype=np.float32)
    for d in range(q.shape[1]):
        with np.errstate(over="ignore", invalid="ignore"):
            acc = _round(acc + np.outer(q[:, d], k[:, d]).astype(np.float32), kind)
    return acc.astype(np.float64)


def _attention_with_scores(q, k, v, g, kind):
    kv_len = OFF + ROWS
    G = HQ // HKV
    out = np.zeros(q.shape)
    for h in range(HQ):
        s = _scores_accumulated(q[0, h], k[0, h // G, :kv_len], kind) / 16.0
        keep = reference.causal_keep(np.arange(ROWS), OFF, kv_len, True)
        with np.errstate(invalid="ignore", over="ignore"):
            m = np.where(keep, s, -np.inf).max(axis=1)
            w = np.where(keep, np.exp(s - m[:, None]), 0.0)
            o = (w @ v[0, h // G, :kv_len]) / w.sum(axis=1)[:, None]
        out[0, h] = o * reference.sigmoid(g[0, h])
    return out


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_separation(dtype):
    rng = syn.streams(1234)
    qb, kb, vb, gb = syn.stress_cancellation(rng["plant"], B=B, Hq=HQ, Hkv=HKV, rows=ROWS, kv_len=OFF + ROWS,
                                             dtype=dtype)
    q, k, v, g = (syn.widen(x, dtype) for x in (qb, kb, vb, gb))
    ref = reference.attention(q, k, v, g, n_kv_heads=HKV, kv_offset=OFF, kv_len=OFF + ROWS)
    assert compare(_attention_with_scores(q, k, v, g, "f32"), ref)["ok"]
    bf = compare(_attention_with_scores(q, k, v, g, "bf16"), ref)
    assert bf["max_abs"] >= 100 * MAX_ABS, bf
    f16 = _attention_with_scores(q, k, v, g, "f16")
    assert not np.isfinite(f16).all()
