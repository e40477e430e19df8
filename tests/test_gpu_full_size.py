"""Parity at the full workload sizes, in the launch configuration the benchmark times,
checked on sampled output rows that the float64 oracle computes one by one."""

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


def _run_prompt(qb, kb, vb, gb, Hkv, q_block):
    q, k, v, g = (to_dev(x) for x in (qb, kb, vb, gb))
    N = q.shape[2]
    kc = torch.empty((1, Hkv, N, 256), dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)
    out = torch.full_like(q, float("nan"))
    ga.prompt_prefill(q, k, v, g, kc, vc, q_block=q_block, out=out)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any()
    return out


def _sampled_check(out, qb, kb, vb, gb, Hkv, rows, what):
    """Oracle rows one by one: row r of the prompt sits at position r and sees keys 0..r."""
    k64, v64 = syn.widen(kb), syn.widen(vb)
    ref = np.stack([
        reference.attention(syn.widen(qb[:, :, r:r + 1]), k64, v64, syn.widen(gb[:, :, r:r + 1]), n_kv_heads=Hkv,
                            kv_offset=int(r), kv_len=int(r) + 1)[:, :, 0]
        for r in rows], axis=2)
    got = to_f64(out[:, :, torch.as_tensor(rows, device=out.device)])
    _say(what, assert_close(got, ref, what))


@needs_gpu
@pytest.mark.slow
def test_35b_prefill_8192_near_ties_full_size():
    # 16 query heads over 2 KV heads, 8192-token causal prompt in blocks of 512, 10% near-tie rows
    _say("35B-A3B prefill 8192, near ties")
    qb, kb, vb, gb, rec = prompt(1002, B=1, Hq=16, Hkv=2, N=8192, near_ties=True)
    out = _run_prompt(qb, kb, vb, gb, 2, 512)
    tie_rows = np.unique(rec[:, 2])
    sel = np.random.default_rng(0)
    rows = np.unique(np.concatenate([sel.choice(tie_rows, 48, replace=False), sel.choice(8192, 32, replace=False),
                                     [0, 1, 511, 512, 8191]]))
    _sampled_check(out, qb, kb, vb, gb, 2, rows, "35B 8192")


@needs_gpu
@pytest.mark.slow
@pytest.mark.parametrize("q_block", [512, 128])
def test_27b_long_prefill_32768_full_size(q_block):
    # 24 query heads over 4 KV heads, 32768-token causal prompt, query blocks of 512 and 128
    _say("27B prefill 32768 qL", q_block)
    qb, kb, vb, gb, _ = prompt(1003, B=1, Hq=24, Hkv=4, N=32768)
    out = _run_prompt(qb, kb, vb, gb, 4, q_block)
    sel = np.random.default_rng(1)
    rows = np.unique(np.concatenate([sel.choice(32768, 40, replace=False), [0, 127, 128, 511, 512, 16383, 32767]]))
    _sampled_check(out, qb, kb, vb, gb, 4, rows, f"32k qL{q_block}")


@needs_gpu
@pytest.mark.parametrize("B,Hq,Hkv,kv_len,rows,dtype", [
    (1, 16, 2, 131072, 1, "bf16"),   # 128k context: 4096 tiles, the most splits a plan takes
    (1, 24, 4, 131072, 4, "f16"),
    (16, 16, 2, 4096, 1, "bf16"),    # a large batch: 32 (b, KV head) groups, fewer splits each
    (64, 8, 1, 1024, 32, "bf16"),    # the largest batch kv_keep takes, verify-sized rows
])
def test_decode_long_context_and_large_batch(B, Hq, Hkv, kv_len, rows, dtype):
    # decode / verify rows at the end of a long cache or over many batch entries, planned as the
    # library plans them (splits, head chunks); every output element against the oracle
    _say("decode size", B, Hq, Hkv, kv_len, rows, dtype)
    rng = syn.streams(9100 + kv_len // 1024 + B)
    off = kv_len - rows
    qb = syn.normal_bits(rng["q"], (B, Hq, rows, 256), dtype)
    gb = syn.normal_bits(rng["gate"], (B, Hq, rows, 256), dtype)
    kb = syn.normal_bits(rng["k"], (B, Hkv, kv_len, 256), dtype)
    vb = syn.normal_bits(rng["v"], (B, Hkv, kv_len, 256), dtype)
    q, g, k, v = (to_dev(x, dtype) for x in (qb, gb, kb, vb))
    a = ga.plan_args(B=B, Hq=Hq, Hkv=Hkv, rows=rows, kv_offset=off, kv_len=kv_len, dtype=dtype)
    plan = ga.describe_plan(a, 1)
    _say(plan["variant_name"], plan["n_splits"], plan["grid_blocks"])
    out = ga.decode(q, k, v, g, kv_offset=off, kv_len=kv_len)
    torch.cuda.synchronize()
    ref = reference.attention(*(syn.widen(x, dtype) for x in (qb, kb, vb, gb)), n_kv_heads=Hkv, kv_offset=off,
                              kv_len=kv_len)
    _say(assert_close(syn.widen(to_bits(out), dtype), ref, f"decode B={B} kv={kv_len} rows={rows}"))
