"""Float64 reference for gated causal GQA attention (test infrastructure only).

This is the plain definition, written out so that it can be checked against the
pages by eye; flash tiling, KV splits and head chunks are exact reorganisations
of it, so the same definition serves every entry point of the library.

Sources (the pages):
  * TensorFold PR #1009, attention kernel-contract commit: decode rows and
    prompt rows of gated attention at the 24/4 and 16/2 head shapes are checked against float64 gated attention; a merge combines decode
    chunks; pack/append/keep are bit copies.  Receipt, "Attention": the same,
    with the controls (a row that sees one key beyond its causal bound, a merge dropping
    later tail chunks, an append one row late).
  * "perf(qwen36): qualify M4 head-256 attention" (d-inference PR #640),
    Summary: prompts are processed in query blocks of qL rows (128 or 512).
  * "Qwen head-chunked SDPA (#113)", introduction and "Exact scope found during
    review": query heads inside a KV group may be split into chunks, each chunk
    attends with its group's K/V, and the results are concatenated in head
    order; the mask is passed to every chunk.

Definition, for batch b, query head h, query row r (absolute position
kv_offset + r) and head group size G = Hq / Hkv:
  1. g = floor(h / G): consecutive query heads share a KV head.
  2. A = { j : 0 <= j < kv_len, j <= kv_offset + r if causal, the mask admits j }.
     A bool mask admits where it is true; an additive mask admits where its
     value is above -Inf.
  3. If A is empty the output row is 0.
  4. s_j = scale * sum_d Q[b,h,r,d] K[b,g,j,d] + M_add[b,h,r,j].
  5. m = max_{j in A} s_j, w_j = exp(s_j - m), L = sum_{j in A} w_j.
  6. o = sum_{j in A} w_j V[b,g,j,:] / L  (only admissible keys are touched).
  7. out = o * sigmoid(gate[b,h,r,:]), sigmoid(x) = 1 / (1 + exp(-x)).

Readings where the pages are silent: the gate is elementwise over
[B, Hq, rows, D] and applied after normalisation; causal alignment is
bottom-right (row r sees keys up to kv_offset + r); a row with no admissible
key gives 0; the mask extents are 1 or B over batch and 1 or Hq over heads.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "sigmoid",
    "causal_keep",
    "mask_keep_and_add",
    "attention",
    "probabilities",
    "partials",
    "merge",
    "head_chunked",
    "kv_append",
    "kv_keep",
]

_ROW_BLOCK = 256  # rows evaluated together; each row is computed independently


def sigmoid(x):
    """1 / (1 + exp(-x)) in float64, elementwise."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def causal_keep(row_index, kv_offset: int, kv_len: int, causal: bool) -> np.ndarray:
    """[len(row_index), kv_len] bool: key j is inside the cache and not in row r's future."""
    row_index = np.asarray(row_index, dtype=np.int64)
    j = np.arange(kv_len, dtype=np.int64)
    keep = np.ones((row_index.size, kv_len), dtype=bool)
    if causal:
        keep &= j[None, :] <= (kv_offset + row_index)[:, None]
    return keep


def mask_keep_and_add(mask, mask_kind, b: int, h: int, row_index, kv_len: int):
    """Slice of the caller's mask for (b, h, rows): (keep bool, additive float64 or None).

    ``mask`` is [Bm, Hm, rows, kv_len] with Bm in {1, B} and Hm in {1, Hq};
    an extent of 1 broadcasts.  kind "bool": True attends.  kind "add": values
    are added to the scores and -Inf hides the key.
    """
    if mask is None or mask_kind in (None, "none"):
        return None, None
    mask = np.asarray(mask)
    mb = b if mask.shape[0] > 1 else 0
    mh = h if mask.shape[1] > 1 else 0
    sl = mask[mb, mh][np.asarray(row_index)][:, :kv_len]
    if mask_kind == "bool":
        return sl.astype(bool), None
    if mask_kind == "add":
        add = sl.astype(np.float64)
        return add > -np.inf, add
    raise ValueError(f"unknown mask kind {mask_kind!r}")


def _softmax_times_v(s, keep, V):
    """Steps 3, 5 and 6 for a block of rows: returns (o [R, D], lse [R])."""
    has = keep.any(axis=1)
    s_adm = np.where(keep, s, -np.inf)
    with np.errstate(invalid="ignore"):
        m = s_adm.max(axis=1) if s.shape[1] else np.full(s.shape[0], -np.inf)
    m_safe = np.where(has, m, 0.0)
    with np.errstate(invalid="ignore", over="ignore"):
        w = np.where(keep, np.exp(s - m_safe[:, None]), 0.0)
    L = w.sum(axis=1)
    if np.isfinite(V).all():
        # w is exactly 0 off A and 0 * x = 0 for finite x, so this equals the sum over A
        num = w @ V
    else:
        num = np.zeros((s.shape[0], V.shape[1]))
        for i in range(s.shape[0]):
            sel = np.nonzero(keep[i])[0]
            num[i] = w[i, sel] @ V[sel]
    with np.errstate(invalid="ignore", divide="ignore"):
        o = np.where(has[:, None], num / np.where(has, L, 1.0)[:, None], 0.0)
        lse = np.where(has, m_safe + np.log(np.where(has, L, 1.0)), -np.inf)
    return o, lse


def _check_shapes(q, k, v, gate, n_kv_heads):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be 4-d [B, H, rows|cap, D]")
    B, Hq, _, D = q.shape
    if n_kv_heads <= 0 or Hq <= 0 or Hq % n_kv_heads:
        raise ValueError("query heads must be a positive multiple of KV heads")
    if k.shape[0] != B or k.shape[1] != n_kv_heads or k.shape[3] != D or v.shape != k.shape:
        raise ValueError("k/v must be [B, Hkv, cap, D] matching q")
    if gate is not None and gate.shape != q.shape:
        raise ValueError("gate must have q's shape")
    return B, Hq, D, Hq // n_kv_heads


def attention(q, k, v, gate, *, n_kv_heads: int, kv_offset: int, kv_len: int, causal: bool = True,
              scale: float | None = None, mask=None, mask_kind=None, rows=None, heads=None,
              key_range=None, return_lse: bool = False):
    """Gated GQA attention in float64 (steps 1-7 of the module docstring).

    q, gate: [B, Hq, R, D]; k, v: [B, Hkv, cap, D] with cap >= kv_len.
    ``rows`` / ``heads`` restrict the evaluation to a subset (sampled checks at
    full size); ``key_range=(lo, hi)`` additionally restricts A to lo <= j < hi
    (used by ``partials``).  gate=None skips step 7 (the ungated o).
    Returns out [B, len(heads), len(rows), D] (and lse [B, heads, rows] if asked).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    gate = None if gate is None else np.asarray(gate, dtype=np.float64)
    B, Hq, D, G = _check_shapes(q, k, v, gate, n_kv_heads)
    if kv_len > k.shape[2]:
        raise ValueError("kv_len beyond the cache")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    rows = np.arange(q.shape[2]) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = np.arange(Hq) if heads is None else np.asarray(heads, dtype=np.int64)
    out = np.zeros((B, heads.size, rows.size, D))
    lse = np.full((B, heads.size, rows.size), -np.inf)
    for b in range(B):
        for hi, h in enumerate(heads):
            g = int(h) // G
            K = k[b, g, :kv_len]
            V = v[b, g, :kv_len]
            for r0 in range(0, rows.size, _ROW_BLOCK):
                ri = rows[r0:r0 + _ROW_BLOCK]
                keep = causal_keep(ri, kv_offset, kv_len, causal)
                if key_range is not None:
                    jj = np.arange(kv_len)
                    keep &= (jj >= key_range[0]) & (jj < key_range[1])
                mkeep, madd = mask_keep_and_add(mask, mask_kind, b, int(h), ri, kv_len)
                if mkeep is not None:
                    keep &= mkeep
                with np.errstate(invalid="ignore", over="ignore"):
                    s = scale * (q[b, h][ri] @ K.T)
                    if madd is not None:
                        s = s + np.where(keep, madd, 0.0)
                o, l_ = _softmax_times_v(s, keep, V)
                if gate is not None:
                    o = o * sigmoid(gate[b, h][ri])
                out[b, hi, r0:r0 + ri.size] = o
                lse[b, hi, r0:r0 + ri.size] = l_
    return (out, lse) if return_lse else out


def probabilities(q, k, *, n_kv_heads: int, kv_offset: int, kv_len: int, causal: bool = True,
                  scale: float | None = None, mask=None, mask_kind=None, b: int = 0, h: int = 0):
    """Softmax weights p[r, j] = w_j / L (0 off A) for one (b, h): the debug view of step 5."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    Hq, D = q.shape[1], q.shape[3]
    G = Hq // n_kv_heads
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    ri = np.arange(q.shape[2])
    keep = causal_keep(ri, kv_offset, kv_len, causal)
    mkeep, madd = mask_keep_and_add(mask, mask_kind, b, h, ri, kv_len)
    if mkeep is not None:
        keep &= mkeep
    s = scale * (q[b, h] @ k[b, h // G, :kv_len].T)
    if madd is not None:
        s = s + np.where(keep, madd, 0.0)
    has = keep.any(axis=1)
    m = np.where(has, np.where(keep, s, -np.inf).max(axis=1), 0.0)
    w = np.where(keep, np.exp(s - m[:, None]), 0.0)
    L = w.sum(axis=1)
    return np.where(has[:, None], w / np.where(has, L, 1.0)[:, None], 0.0)


def partials(q, k, v, *, n_kv_heads: int, kv_offset: int, kv_len: int, chunks, causal: bool = True,
             scale: float | None = None, mask=None, mask_kind=None):
    """Per-KV-chunk partial results: o_c normalised within chunk c and lse_c = m_c + log L_c.

    ``chunks`` is a list of key ranges (lo, hi).  An empty chunk for a row has
    o_c = 0 and lse_c = -Inf.  Returns (o [C, B, Hq, R, D], lse [C, B, Hq, R]).
    This is the decode-chunk state that the merge combines (TensorFold PR
    #1009, attention kernel-contract commit and Receipt, "Attention").
    """
    os_, ls_ = [], []
    for lo, hi in chunks:
        o, l_ = attention(q, k, v, None, n_kv_heads=n_kv_heads, kv_offset=kv_offset, kv_len=kv_len,
                          causal=causal, scale=scale, mask=mask, mask_kind=mask_kind,
                          key_range=(lo, hi), return_lse=True)
        os_.append(o)
        ls_.append(l_)
    return np.stack(os_), np.stack(ls_)


def merge(o_parts, lse_parts, gate):
    """Combine chunk partials: out = sum_c exp(lse_c - lse) o_c * sigmoid(gate).

    lse = log sum_c exp(lse_c); chunks with lse_c = -Inf contribute nothing and a
    row whose chunks are all empty gives 0.  A chunk whose lse_c is NaN (its keys
    held a NaN score, or +Inf) makes the row NaN, as the unsplit definition does.
    o_parts [C, ...] float, lse_parts [C, ...].
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    nan_row = np.isnan(lse_parts).any(axis=0)
    fin = np.isfinite(lse_parts)
    top = np.where(fin, lse_parts, -np.inf).max(axis=0)
    has = np.isfinite(top)
    top_safe = np.where(has, top, 0.0)
    w = np.where(fin, np.exp(np.where(fin, lse_parts, 0.0) - top_safe[None]), 0.0)
    total = w.sum(axis=0)
    with np.errstate(invalid="ignore"):
        o = (w[..., None] * o_parts).sum(axis=0) / np.where(has, total, 1.0)[..., None]
    o = np.where(has[..., None], o, 0.0)
    o = np.where(nan_row[..., None], np.nan, o)
    return o * sigmoid(gate) if gate is not None else o


def head_chunked(q, k, v, gate, *, n_kv_heads: int, chunk_sizes, **kw):
    """The head-chunked evaluation order of "Qwen head-chunked SDPA (#113)" (introduction).

    For every KV group, its query heads are cut into consecutive chunks of the
    given sizes; each chunk attends with that group's K/V alone and the chunk
    outputs are put back in the original head order.  A mask with one entry per
    query head is sliced to the chunk's heads; a broadcast mask is passed as is.
    """
    q = np.asarray(q, dtype=np.float64)
    Hq = q.shape[1]
    G = Hq // n_kv_heads
    if sum(chunk_sizes) != G:
        raise ValueError("chunk sizes must cover the group")
    mask = kw.pop("mask", None)
    mask_kind = kw.pop("mask_kind", None)
    out = np.zeros(q.shape)
    for g in range(n_kv_heads):
        h0 = g * G
        for cs in chunk_sizes:
            hs = slice(h0, h0 + cs)
            sub_mask = mask
            if mask is not None and np.asarray(mask).shape[1] == Hq and Hq > 1:
                sub_mask = np.asarray(mask)[:, hs]
            out[:, hs] = attention(q[:, hs], np.asarray(k)[:, g:g + 1], np.asarray(v)[:, g:g + 1],
                                   None if gate is None else np.asarray(gate)[:, hs], n_kv_heads=1,
                                   mask=sub_mask, mask_kind=mask_kind, **kw)
            h0 += cs
    return out


def kv_append(cache_bits, new_bits, kv_offset: int):
    """Copy new rows' bits into cache[:, :, kv_offset:kv_offset+rows] (no arithmetic).

    cache [B, Hkv, cap, D] and new [B, Hkv, rows, D] as raw 16-bit patterns;
    returns a new array.  Signed zeros and NaN payloads are kept because nothing
    is computed (Qwen head-chunked SDPA (#113), "Isolated oracle evidence": an
    extra copy that adds zero would change signed-zero bits).
    """
    cache = np.array(cache_bits, copy=True)
    new = np.asarray(new_bits)
    rows = new.shape[2]
    if kv_offset < 0 or kv_offset + rows > cache.shape[2]:
        raise ValueError("append beyond the cache capacity")
    cache[:, :, kv_offset:kv_offset + rows] = new
    return cache


def kv_keep(cache_bits, kv_offset: int, rows: int, keep):
    """After a verify block of `rows` rows at kv_offset: in each batch entry b, the rows r whose
    bit is set in keep[b] move, in increasing r, to kv_offset, kv_offset + 1, ...; the block's
    rows after them are unchanged.  A pure copy of raw bit patterns, as the TensorFold PR #1009
    kernel-contract commit compares keep (bit for bit, also a second time on the caches the
    first left).  cache [B, Hkv, cap, D]; keep: one bitmask per batch entry; returns a new array.
    """
    cache = np.array(cache_bits, copy=True)
    if kv_offset < 0 or kv_offset + rows > cache.shape[2] or not 1 <= rows <= 32:
        raise ValueError("verify block outside the cache")
    if len(keep) != cache.shape[0]:
        raise ValueError("one keep mask per batch entry")
    src = np.asarray(cache_bits)
    for b, m in enumerate(keep):
        if m >> rows:
            raise ValueError("keep bit past the block")
        kept = [r for r in range(rows) if (m >> r) & 1]
        for i, r in enumerate(kept):
            cache[b, :, kv_offset + i] = src[b, :, kv_offset + r]
    return cache
