"""Seeded synthetic inputs for gated causal GQA attention at head_dim 256.

Recipe (the same on every machine, so the oracle and the GPU see the same bits):

* one ``numpy.random.SeedSequence(seed)`` per problem, spawned into independent
  PCG64 streams in the fixed order ``q, k, v, gate, mask, plant``;
* every tensor is drawn as float32 N(0, 1) and rounded to bf16 (round to nearest
  even, done on the bit pattern here) or to fp16 (numpy's IEEE conversion);
* tensors are handed around as raw 16-bit patterns (``uint16``); ``widen`` turns
  them into exact float64 for the oracle, and the torch side views the same bits
  as ``torch.bfloat16`` / ``torch.float16``.

The workloads follow the head shapes the pages name: 24 query heads over 4 KV
heads (the 27B) and 16 over 2 (the 35B-A3B), head_dim 256 (TensorFold PR #1009,
attention kernel-contract commit; Receipt, "Attention").  The checkpoints and
prompts the pages measured on are not available; N(0, 1) inputs at the same
shapes stand in for them.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "HEAD_DIM",
    "STREAMS",
    "streams",
    "f32_to_bits",
    "bits_to_f32",
    "widen",
    "normal_bits",
    "bf16_ulp",
    "plant_near_ties",
    "verify_mask",
    "nonfinite_bits",
    "stress_cancellation",
]

HEAD_DIM = 256
STREAMS = ("q", "k", "v", "gate", "mask", "plant")
_DTYPES = ("bf16", "f16")


def streams(seed: int) -> dict:
    """Independent PCG64 generators, one per input tensor, from one seed."""
    children = np.random.SeedSequence(int(seed)).spawn(len(STREAMS))
    return {name: np.random.Generator(np.random.PCG64(c)) for name, c in zip(STREAMS, children)}


def _check_dtype(dtype: str) -> None:
    if dtype not in _DTYPES:
        raise ValueError(f"dtype must be one of {_DTYPES}, got {dtype!r}")


def f32_to_bits(x, dtype: str = "bf16") -> np.ndarray:
    """Round float32 values to bf16 or fp16 (nearest, ties to even); return the bits."""
    _check_dtype(dtype)
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        with np.errstate(over="ignore"):
            return x.astype(np.float16).view(np.uint16)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():  # keep NaN a NaN (quiet bit set) instead of rounding into Inf
        rounded[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return rounded


def bits_to_f32(bits, dtype: str = "bf16") -> np.ndarray:
    """Exact float32 value of bf16/fp16 bit patterns."""
    _check_dtype(dtype)
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float32)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def widen(bits, dtype: str = "bf16") -> np.ndarray:
    """Exact float64 value of bf16/fp16 bit patterns (what the oracle consumes)."""
    return bits_to_f32(bits, dtype).astype(np.float64)


def normal_bits(rng: np.random.Generator, shape, dtype: str = "bf16", scale: float = 1.0) -> np.ndarray:
    """N(0, scale^2) drawn in float32 and rounded to the 16-bit type."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return f32_to_bits(x, dtype)


def bf16_ulp(x) -> np.ndarray:
    """Spacing of bf16 numbers at |x|: 2**(floor(log2|x|) - 7).

    TensorFold PR #1009 (the comment on the staged float64 references) measures
    near-ties in "bf16 steps" and notes a step is 0.125 for logits between 16 and 32.
    """
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - 7), 2.0 ** -133)


def plant_near_ties(q_bits, k_bits, *, n_kv_heads: int, rng: np.random.Generator, frac: float = 0.1,
                    target: float = 8.5, max_gap: float = 0.12, tile: int = 64, scale: float = 1.0 / 16.0,
                    dtype: str = "bf16", max_tries: int = 8):
    """Give a seeded fraction of query rows two near-tied top scores in every head.

    Prompt layout: ``q_bits`` is [B, Hq, N, D] (positions 0..N-1), ``k_bits`` is
    [B, Hkv, N, D]; query row r may see keys 0..r.  For each chosen row r >= 1
    and head h two keys j1 < j2 <= r of the head's KV group are picked (in
    different 64-key tiles for half the rows when r allows, in one tile for the
    other half) and q is rebuilt as

        q = a (k1 + k2) + b (k1 - k2) + n,   n = 0.5 * (z projected off span{k1, k2})

    with (a, b) solved so that the scaled scores are s1 = target and
    s2 = target - delta, delta ~ U[0, max_gap].  At target 8.5 a bf16 step is
    0.0625, so the pair sits within two steps.  After rounding q to the 16-bit
    type the gap is re-measured on the rounded q and the row is redrawn (at most
    ``max_tries`` times) if it left two steps.

    Returns (new_q_bits, records) with records an int64 array of rows
    (b, h, r, j1, j2).  Modifies nothing in place.
    """
    q_bits = np.array(q_bits, dtype=np.uint16, copy=True)
    B, Hq, N, D = q_bits.shape
    G = Hq // n_kv_heads
    k64 = widen(k_bits, dtype)
    n_rows = int(round(frac * N))
    chosen = np.sort(rng.choice(np.arange(1, N), size=min(n_rows, N - 1), replace=False))
    records = []
    for b in range(B):
        for idx, r in enumerate(chosen):
            split_tiles = (idx % 2 == 0) and r >= tile
            for h in range(Hq):
                g = h // G
                for _ in range(max_tries):
                    if split_tiles:
                        t2 = int(rng.integers(1, r // tile + 1))
                        t1 = int(rng.integers(0, t2))
                        j1 = int(rng.integers(t1 * tile, t1 * tile + tile))
                        j2 = int(rng.integers(t2 * tile, min(t2 * tile + tile, r + 1)))
                    else:
                        t = int(rng.integers(0, (r - 1) // tile + 1))  # a tile holding >= 2 keys <= r
                        lo, hi = t * tile, min(t * tile + tile, r + 1)
                        j1, j2 = sorted(int(v) for v in rng.choice(np.arange(lo, hi), size=2, replace=False))
                    k1, k2 = k64[b, g, j1], k64[b, g, j2]
                    delta = float(rng.uniform(0.0, max_gap))
                    basis = np.stack([k1 + k2, k1 - k2])           # 2 x D
                    # row i: how a and b move the unscaled score of key i
                    lhs = np.array([[basis[0] @ k1, basis[1] @ k1],
                                    [basis[0] @ k2, basis[1] @ k2]])
                    rhs = np.array([target, target - delta]) / scale
                    try:
                        ab = np.linalg.solve(lhs, rhs)
                    except np.linalg.LinAlgError:
                        continue
                    z = rng.standard_normal(D)
                    qk, _ = np.linalg.qr(np.stack([k1, k2]).T)      # orthonormal basis of span{k1, k2}
                    z = z - qk @ (qk.T @ z)
                    q = ab[0] * basis[0] + ab[1] * basis[1] + 0.5 * z
                    qb = f32_to_bits(q.astype(np.float32), dtype)
                    qw = widen(qb, dtype)
                    s1, s2 = scale * (qw @ k1), scale * (qw @ k2)
                    if abs(s1 - s2) <= 2.0 * bf16_ulp(max(abs(s1), abs(s2))):
                        q_bits[b, h, r] = qb
                        records.append((b, h, int(r), j1, j2))
                        break
    return q_bits, np.array(records, dtype=np.int64).reshape(-1, 5)


def verify_mask(rng: np.random.Generator, *, rows: int, kv_offset: int, heads: int = 1,
                drop: float = 0.1, kind: str = "add", dtype: str = "bf16", values: str = "zero",
                batch: int = 1) -> np.ndarray:
    """Verify-block mask [1, heads, rows, kv_offset + rows] for speculative-decoding verify rows.

    Prefix keys (positions < kv_offset) are hidden independently with
    probability ``drop``; inside the block, row r sees block key r' only if r'
    is r itself or one of r's ancestors in a seeded random tree (parent of row r
    drawn uniformly from rows 0..r-1, row 0 hangs off the prefix).  Every row
    keeps its own key, so no row is left without an admissible key.

    kind "add": 16-bit bits of 0 (attend) / -Inf (hidden) in ``dtype``;
    kind "add_f32": float32 0 / -Inf; kind "bool": uint8 1 (attend) / 0.
    values "normal" (additive kinds): an admitted key holds a finite N(0, 1) value
    instead of 0 (drawn after the pattern, in float32, then rounded to ``dtype`` for
    kind "add"), the holes stay -Inf.  ``batch`` > 1 gives a [batch, heads, ...] mask with
    a pattern of its own per batch entry.
    """
    if values not in ("zero", "normal"):
        raise ValueError(f"values must be 'zero' or 'normal', got {values!r}")
    kv_len = kv_offset + rows
    keep = rng.random((batch, heads, rows, kv_len)) >= drop
    for bb in range(batch):
        for h in range(heads):
            parent = [-1] + [int(rng.integers(0, r)) for r in range(1, rows)]
            for r in range(rows):
                anc = set()
                a = r
                while a >= 0:
                    anc.add(a)
                    a = parent[a]
                for rp in range(rows):
                    keep[bb, h, r, kv_offset + rp] = rp in anc
    if kind == "bool":
        return keep.astype(np.uint8)
    fill = np.float32(0.0)
    if values == "normal":
        fill = rng.standard_normal(keep.shape, dtype=np.float32)
    vals = np.where(keep, fill, np.float32(-np.inf)).astype(np.float32)
    if kind == "add_f32":
        return vals
    if kind == "add":
        return f32_to_bits(vals, dtype)
    raise ValueError(f"unknown mask kind {kind!r}")


def nonfinite_bits(dtype: str = "bf16") -> dict:
    """Bit patterns of +Inf, -Inf, a quiet NaN with a payload, and -0.0."""
    _check_dtype(dtype)
    if dtype == "bf16":
        return {"+inf": 0x7F80, "-inf": 0xFF80, "nan": 0x7FC5, "-0": 0x8000}
    return {"+inf": 0x7C00, "-inf": 0xFC00, "nan": 0x7E05, "-0": 0x8000}


def stress_cancellation(rng: np.random.Generator, *, B: int, Hq: int, Hkv: int, rows: int, kv_len: int,
                        dtype: str = "bf16", amp: float = 32.0):
    """Inputs whose score sums have large cancelling halves (precision-separation stress).

    Every query element is ``amp``; every key has +amp in dims 0..127 and
    -amp + n * step in dims 128..255 (n in {0, 1, 2, 3}, step = 0.25, exact in
    bf16 and fp16 at this size).  A score sum climbs to 128 * amp^2 = 131072
    before the second half cancels it, leaving 8 * sum(n): exact in fp32, lost
    entirely by bf16 accumulation and past fp16's largest finite value.
    TensorFold PR #1009 (Receipt, "Attention") asks the same of its attention
    inputs: fp16 and bf16 score sums must miss the tolerance by a wide margin.
    Returns bit arrays (q, k, v, gate) with q/gate [B, Hq, rows, 256] and
    k/v [B, Hkv, kv_len, 256].
    """
    half = HEAD_DIM // 2
    q = np.full((B, Hq, rows, HEAD_DIM), amp, dtype=np.float32)
    n = rng.integers(0, 4, size=(B, Hkv, kv_len, half)).astype(np.float32)
    k = np.empty((B, Hkv, kv_len, HEAD_DIM), dtype=np.float32)
    k[..., :half] = amp
    k[..., half:] = -amp + 0.25 * n
    v = rng.standard_normal((B, Hkv, kv_len, HEAD_DIM), dtype=np.float32)
    gate = rng.standard_normal((B, Hq, rows, HEAD_DIM), dtype=np.float32)
    return f32_to_bits(q, dtype), f32_to_bits(k, dtype), f32_to_bits(v, dtype), f32_to_bits(gate, dtype)
