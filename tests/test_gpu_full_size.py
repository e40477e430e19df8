"""Parity at the full workload sizes, in the launch configuration the benchmark times,
checked on sampled output rows that the float64 oracle computes one by one."""

import numpy as np
import pytest
import torch

import gqa_causal_attention_attn_amd as ga
from oracle import reference
from synth import inputs as syn
from tests.gpu_util import prompt, to_dev, to_f64
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
