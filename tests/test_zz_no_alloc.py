"""attn_decode_noalloc against attn_decode (through the C ABI, on the GPU).

The allocation-free entry point runs the same plan and kernels as attn_decode with the split
partials in the library's own device scratch, so its output must equal attn_decode's bit for
bit (and so meet the oracle's tolerance as attn_decode does).  Two calls in a row share the
scratch, the second with a smaller input; a plan whose partials exceed the scratch is refused
before anything is written.
"""

import ctypes as C

import numpy as np
import pytest
import torch

import gqa_causal_attention_attn_amd as ga
from gqa_causal_attention_attn_amd import _abi
from oracle import reference
from synth import inputs as syn
from tests.gpu_util import to_bits, to_dev
from tests.parity import assert_close

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def _say(*a):
    print(*a, flush=True)


def _case(seed, B, Hq, Hkv, rows, off, dtype, masked):
    rng = syn.streams(seed)
    kv = off + rows
    bits = [syn.normal_bits(rng[n], s, dtype) for n, s in
            (("q", (B, Hq, rows, 256)), ("k", (B, Hkv, kv, 256)), ("v", (B, Hkv, kv, 256)),
             ("gate", (B, Hq, rows, 256)))]
    mb = None
    if masked:
        mb = syn.verify_mask(rng["mask"], rows=rows, kv_offset=off, heads=1, kind="add", dtype=dtype, values="normal")
    return bits, mb


@needs_gpu
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_decode_noalloc_matches_decode_twice(dtype):
    # first the head-chunked verify (32 masked rows at offset 32768, batch 2, 16/2 heads: 61 chunks,
    # 62 MiB of partials), then a smaller one-row decode reusing the scratch
    for seed, B, Hq, Hkv, rows, off, masked in ((8800, 2, 16, 2, 32, 32768, True), (8801, 1, 24, 4, 1, 4096, False)):
        _say("noalloc", dtype, B, Hq, Hkv, rows, off)
        (qb, kb, vb, gb), mb = _case(seed, B, Hq, Hkv, rows, off, dtype, masked)
        q, k, v, g = (to_dev(x, dtype) for x in (qb, kb, vb, gb))
        m = to_dev(mb, dtype) if masked else None
        plan = ga.describe_plan(ga._args(q, k, v, g, torch.empty_like(q), kv_offset=off, kv_len=off + rows,
                                         causal=True, scale=0.0, head_chunk=0, n_splits=0, mask=m), _abi.OP_DECODE)
        assert plan["n_splits"] > 1 and plan["workspace_bytes"] <= _abi.SCRATCH_BYTES
        want = ga.decode(q, k, v, g, kv_offset=off, mask=m)
        out = torch.full_like(q, float("nan"))
        ga.decode_noalloc(q, k, v, g, kv_offset=off, mask=m, out=out)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), "noalloc differs from attn_decode"
        ref = reference.attention(*(syn.widen(x, dtype) for x in (qb, kb, vb, gb)), n_kv_heads=Hkv, kv_offset=off,
                                  kv_len=off + rows, mask=None if mb is None else syn.widen(mb, dtype),
                                  mask_kind="add" if masked else None)
        _say(assert_close(syn.widen(to_bits(out), dtype), ref, "noalloc"))


@needs_gpu
def test_decode_noalloc_refuses_partials_past_the_scratch():
    # 32 rows of 16 heads at batch 4 over 32768 keys, asked for 128 splits: 114 chunks of 532 bytes
    # per row need 118 MiB of partials
    B, Hq, Hkv, rows, off = 4, 16, 2, 32, 32768
    q = torch.zeros((B, Hq, rows, 256), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, Hkv, off + rows, 256), dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(q, float("nan"))
    a = ga._args(q, k, k, q, out, kv_offset=off, kv_len=off + rows, causal=True, scale=0.0, head_chunk=0,
                 n_splits=128, mask=None)
    assert ga.workspace_bytes(a, _abi.OP_DECODE) > _abi.SCRATCH_BYTES
    assert ga.lib().attn_decode_noalloc(C.byref(a), None) == _abi.STATUS_CODE["ATTN_E_WORKSPACE"]
    torch.cuda.synchronize()
    assert torch.isnan(out).all()  # nothing was written
    a.n_splits = 16  # fewer chunks fit
    assert ga.workspace_bytes(a, _abi.OP_DECODE) <= _abi.SCRATCH_BYTES
    ga.decode_noalloc(q, k, k, q, kv_offset=off, n_splits=16, out=out)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ga.decode(q, k, k, q, kv_offset=off, n_splits=16).view(torch.int16))
