"""Checks of the seeded input generators (CPU only)."""

import os

import numpy as np
import pytest
import torch

from oracle import reference
from synth import inputs as syn

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_streams_are_deterministic_and_independent():
    a, b = syn.streams(1000), syn.streams(1000)
    x = syn.normal_bits(a["q"], (4, 256))
    assert np.array_equal(x, syn.normal_bits(b["q"], (4, 256)))
    assert not np.array_equal(syn.normal_bits(a["k"], (4, 256)), syn.normal_bits(b["q"], (4, 256)))


@pytest.mark.parametrize("dtype,tdtype", [("bf16", torch.bfloat16), ("f16", torch.float16)])
def test_rounding_matches_torch(dtype, tdtype):
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 7
    x[:4] = [np.inf, -np.inf, -0.0, 3.0e38]
    bits = syn.f32_to_bits(x, dtype)
    tbits = torch.from_numpy(x).to(tdtype).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, tbits)
    np.testing.assert_array_equal(syn.bits_to_f32(bits, dtype), torch.from_numpy(x).to(tdtype).float().numpy())


def test_bf16_step_golden():
    with open(os.path.join(GOLDEN, "bf16_step.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                val, step = (float(p) for p in line.split("|"))
                assert syn.bf16_ulp(val) == step


def test_near_ties_are_top_two_within_two_steps():
    N, Hq, Hkv = 320, 4, 2
    rng = syn.streams(1002)
    q = syn.normal_bits(rng["q"], (1, Hq, N, 256))
    k = syn.normal_bits(rng["k"], (1, Hkv, N, 256))
    q2, rec = syn.plant_near_ties(q, k, n_kv_heads=Hkv, rng=rng["plant"], frac=0.1)
    assert len(rec) == 32 * Hq
    qw, kw = syn.widen(q2), syn.widen(k)
    split = 0
    for b, h, r, j1, j2 in rec:
        s = (qw[b, h, r] @ kw[b, h // 2, :r + 1].T) / 16.0
        order = np.argsort(s)[::-1]
        assert set(order[:2]) == {j1, j2}
        assert abs(s[j1] - s[j2]) <= 2 * syn.bf16_ulp(max(abs(s[j1]), abs(s[j2])))
        split += (j1 // 64) != (j2 // 64)
        p = reference.probabilities(qw[:, :, r:r + 1], kw, n_kv_heads=2, kv_offset=r, kv_len=r + 1, h=h)[0]
        assert p[j1] + p[j2] > 0.3
    assert split > 0


def test_verify_mask_structure():
    rng = syn.streams(1004)
    m = syn.verify_mask(rng["mask"], rows=12, kv_offset=100, heads=3, kind="bool")
    assert m.shape == (1, 3, 12, 112)
    for h in range(3):
        for r in range(12):
            assert m[0, h, r, 100 + r] == 1            # own key kept
            assert m[0, h, r, 100 + r + 1:].sum() == 0  # the tree never points forward
    frac = 1 - m[0, :, :, :100].mean()
    assert 0.05 < frac < 0.15
    add = syn.verify_mask(syn.streams(1004)["mask"], rows=12, kv_offset=100, heads=3, kind="add")
    assert np.array_equal(np.isfinite(syn.bits_to_f32(add)), m.astype(bool))


def test_verify_mask_normal_values():
    # finite N(0, 1) values at the admitted keys, -Inf exactly where the 0/-Inf mask of the same
    # seed has its holes; batch entries get patterns of their own
    for dtype in ("bf16", "f16"):
        zero = syn.verify_mask(syn.streams(5)["mask"], rows=9, kv_offset=300, heads=2, kind="add", dtype=dtype)
        vals = syn.verify_mask(syn.streams(5)["mask"], rows=9, kv_offset=300, heads=2, kind="add", dtype=dtype,
                               values="normal")
        z, v = syn.widen(zero, dtype), syn.widen(vals, dtype)
        assert np.array_equal(np.isfinite(z), np.isfinite(v))
        fin = v[np.isfinite(v)]
        assert np.count_nonzero(fin) > 0.99 * fin.size
        assert 0.8 < fin.std() < 1.2 and abs(fin.mean()) < 0.1
    f32 = syn.verify_mask(syn.streams(6)["mask"], rows=5, kv_offset=40, kind="add_f32", values="normal", batch=2)
    assert f32.shape == (2, 1, 5, 45) and f32.dtype == np.float32
    assert not np.array_equal(np.isfinite(f32[0]), np.isfinite(f32[1]))


def test_near_ties_every_row_including_tile_boundaries():
    # frac 1: every row 1..N-1, so rows sitting on a 64-key tile start (64, 128) are planted too
    N = 140
    rng = syn.streams(7)
    q = syn.normal_bits(rng["q"], (1, 2, N, 256))
    k = syn.normal_bits(rng["k"], (1, 1, N, 256))
    q2, rec = syn.plant_near_ties(q, k, n_kv_heads=1, rng=rng["plant"], frac=1.0)
    assert len(rec) == 2 * (N - 1)
    assert np.all(rec[:, 3] < rec[:, 4]) and np.all(rec[:, 4] <= rec[:, 2])
