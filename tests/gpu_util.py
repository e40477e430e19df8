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


def strided_mask(m, row_stride):
    """m ([Bm, Hm, rows, kv] on the GPU) copied into storage with the given row stride (elements)."""
    Bm, Hm, rows, kv = m.shape
    store = torch.zeros((Bm, Hm, rows, row_stride), dtype=m.dtype, device=m.device)
    store[..., :kv] = m
    return store[..., :kv]


def lds_and_lane_strides(kv, esz):
    """Row strides (elements) for a mask of kv keys: one 64-byte aligned (the planner may stage
    its rows in LDS) and one that is not a multiple of 16 bytes (per-lane loads)."""
    aligned = (kv * esz + 63) // 64 * 64 // esz
    odd = kv
    while (odd * esz) % 16 == 0:
        odd += 1
    return aligned, odd
