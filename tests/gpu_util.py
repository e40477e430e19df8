"""Helpers for the GPU tests: seeded bits to device tensors and device tensors back to float64."""

import numpy as np
import torch

from synth import inputs as syn

TORCH_DTYPE = {"bf16": torch.bfloat16, "f16": torch.float16}


def to_dev(bits, dtype="bf16", device="cuda"):
    """16-bit patterns (uint16 numpy) -> a device tensor of that dtype holding the same bits."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device).view(TORCH_DTYPE[dtype])


def to_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def to_bits(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def prompt(seed, *, B, Hq, Hkv, N, dtype="bf16", near_ties=False):
    """Seeded prompt bits q/gate [B, Hq, N, 256], k/v [B, Hkv, N, 256] (+ near-tie records)."""
    rng = syn.streams(seed)
    q = syn.normal_bits(rng["q"], (B, Hq, N, 256), dtype)
    k = syn.normal_bits(rng["k"], (B, Hkv, N, 256), dtype)
    v = syn.normal_bits(rng["v"], (B, Hkv, N, 256), dtype)
    g = syn.normal_bits(rng["gate"], (B, Hq, N, 256), dtype)
    rec = None
    if near_ties:
        q, rec = syn.plant_near_ties(q, k, n_kv_heads=Hkv, rng=rng["plant"], dtype=dtype)
    return q, k, v, g, rec
