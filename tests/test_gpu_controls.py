"""Planted mistakes in the HIP path must miss the oracle (controls that must go red).

TensorFold PR #1009 (Receipt, "Attention") runs its attention checks against three planted
mistakes that must all fail: a query row that sees one key past its own, a merge that drops its
last chunk, and an append one row late.  Each is built into a library of its own from the same
sources (libgqa_attn_control{1,2,3}.so, compiled with GQA_CONTROL=n); the inputs are planted so
that the mistake moves the output far past the tolerance.  Each case also runs on the library
itself, which must pass, so a red control means the planted mistake was caught, not that the
inputs were hard.  The mistakes give wrong numbers only: every access stays inside the buffers
(the late append's capacity check moves with it).
"""

import contextlib

import numpy as np
import pytest
import torch

import gqa_causal_attention_attn_amd as ga
from gqa_causal_attention_attn_amd import _abi, build
from oracle import reference
from synth import inputs as syn
from tests.gpu_util import to_bits, to_dev, to_f64
from tests.parity import MAX_ABS, compare

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def _say(*a):
    print(*a, flush=True)


@contextlib.contextmanager
def _library(n):
    """Route the binding's calls through control library n (0: the library itself)."""
    saved = ga.lib()
    ga._LIB = saved if n == 0 else _abi.load(build.control_lib(n))
    try:
        yield
    finally:
        ga._LIB = saved


def _red(got, ref, what):
    res = compare(got, ref)
    _say(what, res)
    assert not res["ok"] and res["max_abs"] > 10 * MAX_ABS, f"{what}: the planted mistake was not caught: {res}"


def _green(got, ref, what):
    res = compare(got, ref)
    _say(what, res)
    assert res["ok"], f"{what}: {res}"


@needs_gpu
@pytest.mark.parametrize("rows,op", [(6, "decode"), (100, "prefill")])
def test_control_row_sees_one_key_past_its_own(rows, op):
    # every row's query points at the key just after its own position (decode: the four-wavefront
    # shape; prefill: eight wavefronts)
    _say("control: one key past", rows, op)
    B, Hq, Hkv, off = 1, 8, 2, 40
    rng = syn.streams(7100 + rows)
    kv = off + rows
    kb = syn.normal_bits(rng["k"], (B, Hkv, kv, 256))
    vb = syn.normal_bits(rng["v"], (B, Hkv, kv, 256))
    gb = syn.normal_bits(rng["gate"], (B, Hq, rows, 256))
    k = syn.widen(kb)
    q = syn.widen(syn.normal_bits(rng["q"], (B, Hq, rows, 256)))
    for h in range(Hq):
        for r in range(rows - 1):
            q[0, h, r] = 0.5 * k[0, h // (Hq // Hkv), off + r + 1]
    qb = syn.f32_to_bits(q.astype(np.float32))
    ref = reference.attention(syn.widen(qb), k, syn.widen(vb), syn.widen(gb), n_kv_heads=Hkv, kv_offset=off,
                              kv_len=kv)
    dq, dk, dv, dg = (to_dev(x) for x in (qb, kb, vb, gb))
    fn = ga.decode if op == "decode" else ga.prefill
    for n in (0, 1):
        with _library(n):
            out = to_f64(fn(dq, dk, dv, dg, kv_offset=off, kv_len=kv))
        (_green if n == 0 else _red)(out, ref, f"library {n}")


@needs_gpu
@pytest.mark.parametrize("n_splits", [5, 12, 40])
def test_control_merge_drops_last_chunk(n_splits):
    # one decode row over 4000 keys in n_splits chunks (the few-chunk merge, and the many-chunk
    # merge with 4 and 16 wavefronts a row); every query points at a key of the last chunk
    _say("control: merge drops last chunk", n_splits)
    B, Hq, Hkv, kv = 1, 16, 2, 4000
    rng = syn.streams(7200 + n_splits)
    kb = syn.normal_bits(rng["k"], (B, Hkv, kv, 256))
    vb = syn.normal_bits(rng["v"], (B, Hkv, kv, 256))
    gb = syn.normal_bits(rng["gate"], (B, Hq, 1, 256))
    plan = ga.describe_plan(ga.plan_args(B=B, Hq=Hq, Hkv=Hkv, rows=1, kv_offset=kv - 1, n_splits=n_splits),
                            _abi.OP_DECODE)
    assert plan["n_splits"] > 1
    last = (plan["n_splits"] - 1) * plan["keys_per_split"]
    assert last < kv - 10
    k = syn.widen(kb)
    q = np.stack([0.5 * k[0, h // 8, last + 3 + h] for h in range(Hq)])[None, :, None]
    qb = syn.f32_to_bits(q.astype(np.float32))
    ref = reference.attention(syn.widen(qb), k, syn.widen(vb), syn.widen(gb), n_kv_heads=Hkv, kv_offset=kv - 1,
                              kv_len=kv)
    dq, dk, dv, dg = (to_dev(x) for x in (qb, kb, vb, gb))
    for n in (0, 2):
        with _library(n):
            out = to_f64(ga.decode(dq, dk, dv, dg, kv_offset=kv - 1, n_splits=n_splits))
        (_green if n == 0 else _red)(out, ref, f"library {n}")


@needs_gpu
def test_control_append_one_row_late():
    # six verify rows appended at offset 40, each row's query pointing at its own new key
    _say("control: append one row late")
    B, Hq, Hkv, off, rows = 1, 8, 2, 40, 6
    rng = syn.streams(7300)
    cap = off + rows + 1
    cache_k = np.zeros((B, Hkv, cap, 256), dtype=np.uint16)
    cache_v = np.zeros_like(cache_k)
    cache_k[:, :, :off] = syn.normal_bits(rng["k"], (B, Hkv, off, 256))
    cache_v[:, :, :off] = syn.normal_bits(rng["v"], (B, Hkv, off, 256))
    new_k = syn.normal_bits(rng["k"], (B, Hkv, rows, 256))
    new_v = syn.normal_bits(rng["v"], (B, Hkv, rows, 256))
    want_k = reference.kv_append(cache_k, new_k, off)
    want_v = reference.kv_append(cache_v, new_v, off)
    kk = syn.widen(want_k)
    q = np.zeros((B, Hq, rows, 256))
    for h in range(Hq):
        for r in range(rows):
            q[0, h, r] = 0.5 * kk[0, h // 4, off + r]
    qb = syn.f32_to_bits(q.astype(np.float32))
    gb = syn.normal_bits(rng["gate"], (B, Hq, rows, 256))
    ref = reference.attention(syn.widen(qb), kk, syn.widen(want_v), syn.widen(gb), n_kv_heads=Hkv, kv_offset=off,
                              kv_len=off + rows)
    for n in (0, 3):
        kc, vc = to_dev(cache_k), to_dev(cache_v)
        with _library(n):
            ga.kv_append(to_dev(new_k), to_dev(new_v), kc, vc, kv_offset=off)
            out = to_f64(ga.decode(to_dev(qb), kc, vc, to_dev(gb), kv_offset=off))
        same = np.array_equal(to_bits(kc), want_k) and np.array_equal(to_bits(vc), want_v)
        assert same == (n == 0)
        (_green if n == 0 else _red)(out, ref, f"library {n}")
