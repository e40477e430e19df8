"""Seeded random shapes through attn_prefill and attn_decode (C ABI) against the float64 oracle.

Batches, group sizes, head dims 64/128/256, bf16 and fp16, planned and forced KV splits (so
both partial forms and both merge kernels run), KV offsets, and additive masks with finite
N(0, 1) entries and -Inf holes.  A few fixed cases have 1024 or more merge rows with 10 to 34
chunks, which the one-wavefront merge takes with 16, 32 and 64 slots.  Tolerance as the other
parity tests: max abs error <= 1.5e-2, median relative error <= 4e-3.
"""

import numpy as np
import pytest
import torch

import gqa_causal_attention_attn_amd as ga
from oracle import reference
from synth import inputs as syn
from tests.gpu_util import to_dev, to_f64
from tests.parity import assert_close

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def _random_cases():
    r = np.random.default_rng(2026)
    out = []
    for i in range(18):
        op = "decode" if i % 3 == 0 else "prefill"
        D = int(r.choice([64, 128, 256]))
        Hkv = int(r.choice([1, 2, 4]))
        G = int(r.choice([1, 2, 4, 6, 8]))
        B = int(r.choice([1, 2]))
        rows = int(r.integers(1, 33)) if op == "decode" else int(r.choice([17, 64, 128, 200]))
        off = int(r.integers(0, 1500))
        n_splits = int(r.choice([0, 0, 3, 12, 24]))
        dtype = "bf16" if r.random() < 0.7 else "f16"
        masked = bool(r.random() < 0.35)
        out.append((f"r{i}", op, B, G * Hkv, Hkv, rows, off, D, n_splits, dtype, masked))
    # merges of 1024+ rows with 9..64 chunks: 32 fp16 slots, 32 fp16 slots through decode,
    # 16 fp32 slots, 64 fp16 slots
    out.append(("wide32", "prefill", 1, 32, 4, 32, 1500, 256, 24, "bf16", False))
    out.append(("wide32_decode", "decode", 2, 16, 2, 32, 2000, 256, 40, "f16", True))
    out.append(("wide16_fp32", "prefill", 1, 32, 4, 32, 1200, 128, 12, "bf16", False))
    out.append(("wide64", "prefill", 2, 16, 2, 32, 2100, 256, 64, "bf16", True))
    return out


CASES = _random_cases()


@needs_gpu
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_random_shape_against_the_oracle(case):
    name, op, B, Hq, Hkv, rows, off, D, n_splits, dtype, masked = case
    print("case", case, flush=True)
    rng = syn.streams(4000 + CASES.index(case))
    kv = off + rows
    qb = syn.normal_bits(rng["q"], (B, Hq, rows, D), dtype)
    gb = syn.normal_bits(rng["gate"], (B, Hq, rows, D), dtype)
    kb = syn.normal_bits(rng["k"], (B, Hkv, kv, D), dtype)
    vb = syn.normal_bits(rng["v"], (B, Hkv, kv, D), dtype)
    mb = None
    if masked:
        mb = syn.verify_mask(rng["mask"], rows=rows, kv_offset=off, heads=1, kind="add", dtype=dtype,
                             values="normal")
    q, g, k, v = (to_dev(x, dtype) for x in (qb, gb, kb, vb))
    m = to_dev(mb, dtype) if masked else None
    a = ga.plan_args(B=B, Hq=Hq, Hkv=Hkv, rows=rows, kv_offset=off, D=D, dtype=dtype, n_splits=n_splits,
                     mask_kind=2 if masked else 0)
    plan = ga.describe_plan(a, 1 if op == "decode" else 0)
    print("plan", {k_: plan[k_] for k_ in ("variant_name", "n_splits", "partial_kind", "n_head_chunks")}, flush=True)
    if name.startswith("wide"):
        n_rows = B * Hq * rows
        assert n_rows >= 1024 and 8 < plan["n_splits"] <= 64
    fn = ga.decode if op == "decode" else ga.prefill
    out = fn(q, k, v, g, kv_offset=off, n_splits=n_splits, mask=m)
    torch.cuda.synchronize()
    ref = reference.attention(*(syn.widen(x, dtype) for x in (qb, kb, vb, gb)), n_kv_heads=Hkv, kv_offset=off,
                              kv_len=kv, mask=None if mb is None else syn.widen(mb, dtype),
                              mask_kind="add" if masked else None)
    print(assert_close(to_f64(out), ref, f"{name} {op}"), flush=True)
