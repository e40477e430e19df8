"""The composed (materialised-score) route, the main pass at head dims 128 and 64, and the
prompt policy, on the GPU against the float64 oracle.

attn_prefill_composed computes the same block as attn_prefill in three passes through HBM
("perf(qwen36): qualify M4 head-256 attention", Summary: composed against fused attention at
head_dim 256 for query blocks of 128 and 512; its review comment: eligibility by head
dimension).  Same tolerance: max abs error <= 1.5e-2 and median relative error <= 4e-3 on
16-bit outputs with fp32 accumulation.
"""

import numpy as np
import pytest
import torch

import gqa_causal_attention_attn_amd as ga
from oracle import reference
from synth import inputs as syn
from tests.gpu_util import prompt, to_bits, to_dev, to_f64
from tests.parity import assert_close

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def _say(*a):
    print(*a, flush=True)


@needs_gpu
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("Hq,Hkv,N,q_block", [
    (24, 4, 128, 128),   # the tiny prefill in one block
    (24, 4, 200, 96),    # ragged last block, offsets not multiples of 32
    (16, 2, 333, 128),   # GQA 8, ragged
    (6, 1, 70, 32),      # one KV head, row tiles of 32
])
def test_composed_prompt_matches_oracle(dtype, Hq, Hkv, N, q_block):
    _say("composed", dtype, Hq, Hkv, N, q_block)
    qb, kb, vb, gb, _ = prompt(5000 + N, B=1, Hq=Hq, Hkv=Hkv, N=N, dtype=dtype)
    q, k, v, g = (to_dev(x, dtype) for x in (qb, kb, vb, gb))
    kc = torch.full((1, Hkv, N, 256), float("nan"), dtype=q.dtype, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    out = torch.full_like(q, float("nan"))
    ga.prompt_prefill(q, k, v, g, kc, vc, q_block=q_block, out=out, composed=True)
    torch.cuda.synchronize()
    ref = reference.attention(*(syn.widen(x, dtype) for x in (qb, kb, vb, gb)), n_kv_heads=Hkv, kv_offset=0,
                              kv_len=N)
    _say(assert_close(syn.widen(to_bits(out), dtype), ref, "composed prompt"))
    # the fused route on the same block sizes is within the same tolerance of the oracle
    kc2, vc2 = torch.zeros_like(kc), torch.zeros_like(vc)
    fused = ga.prompt_prefill(q, k, v, g, kc2, vc2, q_block=q_block)
    torch.cuda.synchronize()
    _say(assert_close(syn.widen(to_bits(fused), dtype), ref, "fused prompt"))


@needs_gpu
def test_composed_batch2_noncausal_and_offset():
    # batch 2, 8 query heads over 2 KV heads: 40 rows against a 150-key cache, not causal;
    # then causal rows at offset 110 (the block's own keys appended)
    _say("composed batch 2")
    rng = syn.streams(5100)
    B, Hq, Hkv, rows, kv = 2, 8, 2, 40, 150
    qb = syn.normal_bits(rng["q"], (B, Hq, rows, 256))
    gb = syn.normal_bits(rng["gate"], (B, Hq, rows, 256))
    kb = syn.normal_bits(rng["k"], (B, Hkv, kv, 256))
    vb = syn.normal_bits(rng["v"], (B, Hkv, kv, 256))
    q, g, k, v = (to_dev(x) for x in (qb, gb, kb, vb))
    for causal, off in ((False, 0), (True, kv - rows)):
        out = ga.prefill_composed(q, k, v, g, kv_offset=off, kv_len=kv, causal=causal)
        torch.cuda.synchronize()
        ref = reference.attention(*(syn.widen(x) for x in (qb, kb, vb, gb)), n_kv_heads=Hkv, kv_offset=off,
                                  kv_len=kv, causal=causal)
        _say(assert_close(to_f64(out), ref, f"composed causal={causal}"))


@needs_gpu
def test_composed_8k_prompt_in_512_row_blocks_sampled():
    # the 35B-A3B attention shape (16 query heads over 2 KV heads) over 8192 tokens in blocks of
    # 512, as the benchmark launches the route; rows sampled across the prompt against the oracle
    _say("composed 8k")
    N, Hq, Hkv = 8192, 16, 2
    qb, kb, vb, gb, _ = prompt(5200, B=1, Hq=Hq, Hkv=Hkv, N=N)
    q, k, v, g = (to_dev(x) for x in (qb, kb, vb, gb))
    kc = torch.zeros((1, Hkv, N, 256), dtype=q.dtype, device="cuda")
    vc = torch.zeros_like(kc)
    out = ga.prompt_prefill(q, k, v, g, kc, vc, q_block=512, composed=True)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 511, 512, 513, 2047, 4100, 6000, 8190, 8191])
    ref = reference.attention(*(syn.widen(x) for x in (qb, kb, vb, gb)), n_kv_heads=Hkv, kv_offset=0, kv_len=N,
                              rows=rows)
    _say(assert_close(to_f64(out)[:, :, rows], ref, "composed 8k sampled"))


@needs_gpu
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
def test_composed_other_head_dims(D, dtype):
    # head dims 64 and 128: 8 query heads over 2 KV heads, 150 causal rows in blocks of 64
    # (kv_append + attn_prefill_composed, then the fused pass), scale 1 / sqrt(D); the append
    # bit for bit
    _say("composed head dim", D, dtype)
    Hq, Hkv, N = 8, 2, 150
    rng = syn.streams(5300 + D)
    qb = syn.normal_bits(rng["q"], (1, Hq, N, D), dtype)
    kb = syn.normal_bits(rng["k"], (1, Hkv, N, D), dtype)
    vb = syn.normal_bits(rng["v"], (1, Hkv, N, D), dtype)
    gb = syn.normal_bits(rng["gate"], (1, Hq, N, D), dtype)
    q, k, v, g = (to_dev(x, dtype) for x in (qb, kb, vb, gb))
    kc = torch.full((1, Hkv, N, D), float("nan"), dtype=q.dtype, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    out = ga.prompt_prefill(q, k, v, g, kc, vc, q_block=64, composed=True)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(kc), kb) and np.array_equal(to_bits(vc), vb)
    ref = reference.attention(*(syn.widen(x, dtype) for x in (qb, kb, vb, gb)), n_kv_heads=Hkv, kv_offset=0,
                              kv_len=N)
    _say(assert_close(syn.widen(to_bits(out), dtype), ref, f"composed D={D}"))
    # the fused pass for this head dim, same blocks
    kc2, vc2 = torch.zeros_like(kc), torch.zeros_like(vc)
    fused = ga.prompt_prefill(q, k, v, g, kc2, vc2, q_block=64)
    torch.cuda.synchronize()
    _say(assert_close(syn.widen(to_bits(fused), dtype), ref, f"fused D={D}"))


@needs_gpu
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("rows,offset,causal,B", [(1, 1000, True, 1), (5, 777, True, 2), (32, 4096, True, 1),
                                                   (70, 0, False, 2)])
def test_fused_small_head_dims(D, rows, offset, causal, B, dtype):
    # the main pass at head dims 64 and 128: decode / verify rows over a cache (the heads of a KV
    # group stacked in one workgroup, or one head a workgroup when chunked by one: the same bits),
    # and a non-causal block
    _say("fused small D", D, rows, offset, causal, B, dtype)
    Hq, Hkv = 16, 2
    kv = offset + rows if causal else 150
    rng = syn.streams(5400 + D + rows)
    qb = syn.normal_bits(rng["q"], (B, Hq, rows, D), dtype)
    gb = syn.normal_bits(rng["gate"], (B, Hq, rows, D), dtype)
    kb = syn.normal_bits(rng["k"], (B, Hkv, kv + 7, D), dtype)
    vb = syn.normal_bits(rng["v"], (B, Hkv, kv + 7, D), dtype)
    q, g, k, v = (to_dev(x, dtype) for x in (qb, gb, kb, vb))
    call = ga.decode if rows <= 32 else ga.prefill
    out = call(q, k, v, g, kv_offset=offset, kv_len=kv, causal=causal)
    torch.cuda.synchronize()
    ref = reference.attention(*(syn.widen(x, dtype) for x in (qb, kb, vb, gb)), n_kv_heads=Hkv, kv_offset=offset,
                              kv_len=kv, causal=causal)
    _say(assert_close(syn.widen(to_bits(out), dtype), ref, f"fused D={D}"))
    if rows <= 32:
        if rows < 32:  # the policy stacks several heads of the group in a workgroup
            a0 = ga.plan_args(B=B, Hq=Hq, Hkv=Hkv, rows=rows, kv_offset=offset, kv_len=kv, causal=causal, D=D)
            assert ga.describe_plan(a0, 1)["n_head_chunks"] < Hq // Hkv
        again = ga.decode(q, k, v, g, kv_offset=offset, kv_len=kv, causal=causal, head_chunk=1)
        assert torch.equal(again.view(torch.int16), out.view(torch.int16))


@needs_gpu
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_fused_small_head_dims_split_keys(D, dtype):
    # the same pass with its keys split (the planned count, then 1, 3 and 7 asked) and merged:
    # 100 causal rows at offset 2900 (ragged last row tile, split bounds inside row tiles), and
    # the main pass alone plus attn_merge giving the same bits as the whole call
    _say("fused small D splits", D, dtype)
    B, Hq, Hkv, rows, off = 2, 8, 2, 100, 2900
    kv = off + rows
    rng = syn.streams(5500 + D)
    qb = syn.normal_bits(rng["q"], (B, Hq, rows, D), dtype)
    gb = syn.normal_bits(rng["gate"], (B, Hq, rows, D), dtype)
    kb = syn.normal_bits(rng["k"], (B, Hkv, kv, D), dtype)
    vb = syn.normal_bits(rng["v"], (B, Hkv, kv, D), dtype)
    q, g, k, v = (to_dev(x, dtype) for x in (qb, gb, kb, vb))
    ref = reference.attention(*(syn.widen(x, dtype) for x in (qb, kb, vb, gb)), n_kv_heads=Hkv, kv_offset=off,
                              kv_len=kv)
    a = ga.plan_args(B=B, Hq=Hq, Hkv=Hkv, rows=rows, kv_offset=off, D=D)
    assert ga.describe_plan(a, 0)["n_splits"] > 1
    outs = {}
    for ns in (0, 1, 3, 7):
        outs[ns] = ga.prefill(q, k, v, g, kv_offset=off, n_splits=ns)
        torch.cuda.synchronize()
        _say(assert_close(syn.widen(to_bits(outs[ns]), dtype), ref, f"fused D={D} n_splits={ns}"))
    ws = torch.empty(ga.workspace_bytes(ga.plan_args(B=B, Hq=Hq, Hkv=Hkv, rows=rows, kv_offset=off, D=D,
                                                     n_splits=3), 0), dtype=torch.uint8, device="cuda")
    out, parts = ga.prefill_partials(q, k, v, g, kv_offset=off, n_splits=3, workspace=ws)
    kind = ga.describe_plan(ga.plan_args(B=B, Hq=Hq, Hkv=Hkv, rows=rows, kv_offset=off, D=D, n_splits=3),
                            0)["partial_kind"]
    assert parts is not None and parts[0].shape == (3, B, Hq, rows, D)
    assert parts[0].dtype == (torch.float16 if kind else torch.float32) and (parts[2] is None) == (kind == 0)
    ga.merge(parts[0], parts[1], g, out=out, partial_exp=parts[2])
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), outs[3].view(torch.int16))


@needs_gpu
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(24, 4), (6, 3), (5, 5), (16, 2)])
def test_fused_small_head_dims_heads_per_workgroup(D, Hq, Hkv, dtype):
    # the heads of a KV group sharing K/V tiles in one workgroup (G 6, 2 and 8) and one head
    # alone (G 1); 70 causal rows at offset 1500 (ragged row tile), keys split as planned
    _say("fused small D heads per workgroup", D, Hq, Hkv, dtype)
    B, rows, off = 1, 70, 1500
    kv = off + rows
    rng = syn.streams(5600 + D + Hq)
    qb = syn.normal_bits(rng["q"], (B, Hq, rows, D), dtype)
    gb = syn.normal_bits(rng["gate"], (B, Hq, rows, D), dtype)
    kb = syn.normal_bits(rng["k"], (B, Hkv, kv, D), dtype)
    vb = syn.normal_bits(rng["v"], (B, Hkv, kv, D), dtype)
    q, g, k, v = (to_dev(x, dtype) for x in (qb, gb, kb, vb))
    out = ga.prefill(q, k, v, g, kv_offset=off)
    torch.cuda.synchronize()
    ref = reference.attention(*(syn.widen(x, dtype) for x in (qb, kb, vb, gb)), n_kv_heads=Hkv, kv_offset=off,
                              kv_len=kv)
    _say(assert_close(syn.widen(to_bits(out), dtype), ref, f"fused D={D} {Hq}/{Hkv}"))


@needs_gpu
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [128, 64])
def test_fused_small_head_dims_32k_prompt_sampled(D, dtype):
    # the benchmark's launch configuration for these head dims: a 32768-token prompt at 24 query
    # heads over 4 KV heads in blocks of 512 rows (kv_append + attn_prefill, keys split as
    # planned); rows sampled across the prompt and every head against the oracle
    _say("fused small D 32k", D, dtype)
    N, Hq, Hkv = 32768, 24, 4
    rng = syn.streams(5700 + D)
    qb = syn.normal_bits(rng["q"], (1, Hq, N, D), dtype)
    kb = syn.normal_bits(rng["k"], (1, Hkv, N, D), dtype)
    vb = syn.normal_bits(rng["v"], (1, Hkv, N, D), dtype)
    gb = syn.normal_bits(rng["gate"], (1, Hq, N, D), dtype)
    q, k, v, g = (to_dev(x, dtype) for x in (qb, kb, vb, gb))
    kc = torch.zeros((1, Hkv, N, D), dtype=q.dtype, device="cuda")
    vc = torch.zeros_like(kc)
    out = ga.prompt_prefill(q, k, v, g, kc, vc, q_block=512)
    torch.cuda.synchronize()
    assert torch.equal(kc, k) and torch.equal(vc, v)
    rows = np.array([0, 31, 32, 511, 512, 4097, 16383, 20000, 32255, 32256, 32767])
    ref = reference.attention(*(syn.widen(x, dtype) for x in (qb, kb, vb, gb)), n_kv_heads=Hkv, kv_offset=0,
                              kv_len=N, rows=rows)
    _say(assert_close(to_f64(out[:, :, rows]), ref, f"fused D={D} {dtype} 32k sampled"))


@needs_gpu
@pytest.mark.parametrize("D,Hq,Hkv,N", [(256, 16, 2, 8192), (128, 24, 4, 4608), (64, 24, 4, 1500)])
def test_prompt_policy_block_size_on_this_device(D, Hq, Hkv, N):
    # prompt_prefill(q_block=0) takes attn_prompt_policy's block size for this device (the table
    # on an MI355X: 4096 rows for G 8, 8192 for G 6 at most the prompt, one call up to 2048
    # rows); rows sampled across the prompt against the oracle
    gfx, n_cus = ga.device_key()
    pol = ga.prompt_policy(D=D, B=1, Hq=Hq, Hkv=Hkv, n_tokens=N)
    _say("policy", D, Hq, Hkv, N, gfx, n_cus, pol)
    if (gfx, n_cus) == (950, 256):
        assert pol["qualified"] and pol["route"] == "fused"
        assert pol["q_block"] == (N if N <= 2048 else min(N, 4096 if Hq // Hkv > 6 else 8192))
    rng = syn.streams(5800 + D)
    qb = syn.normal_bits(rng["q"], (1, Hq, N, D))
    kb = syn.normal_bits(rng["k"], (1, Hkv, N, D))
    vb = syn.normal_bits(rng["v"], (1, Hkv, N, D))
    gb = syn.normal_bits(rng["gate"], (1, Hq, N, D))
    q, k, v, g = (to_dev(x) for x in (qb, kb, vb, gb))
    kc = torch.zeros((1, Hkv, N, D), dtype=q.dtype, device="cuda")
    vc = torch.zeros_like(kc)
    out = ga.prompt_prefill(q, k, v, g, kc, vc, q_block=0)
    torch.cuda.synchronize()
    assert torch.equal(kc, k) and torch.equal(vc, v)
    rows = np.unique(np.array([0, 1, N // 3, pol["q_block"] - 1, min(pol["q_block"], N - 1), N - 2, N - 1]))
    ref = reference.attention(*(syn.widen(x) for x in (qb, kb, vb, gb)), n_kv_heads=Hkv, kv_offset=0, kv_len=N,
                              rows=rows)
    _say(assert_close(to_f64(out[:, :, rows]), ref, f"policy D={D}"))
