"""The head-chunk rule as "Qwen head-chunked SDPA (#113)" states it (test infrastructure only).

Introduction of that page: with the policy enabled (its default), for at most 32
rows and more than 32 (row, head) pairs per group (rows * GQA > 32), the query heads inside each KV group are split
into chunks of min(GQA, 32 / rows) heads, the remainder heads are kept as a
last, smaller chunk, each chunk attends with its group's K/V, and the outputs
are concatenated in the original head order.  An explicit off switch keeps the
unchunked consumer.  "Exact scope found during review": rows above 32 pass
through unchanged.  32 / rows is read as integer division; the page's
"Completion review" example (4 rows, 12 query heads per KV group, two groups,
four calls of 8 + 4 heads) reproduces under that reading.
"""

from __future__ import annotations

__all__ = ["head_chunk_sizes", "n_calls"]

ROW_PAIR_LIMIT = 32


def head_chunk_sizes(rows: int, n_q_heads: int, n_kv_heads: int, enabled: bool = True) -> list:
    """Chunk sizes for one KV group, in head order.

    Raises ValueError for rows < 1, non-positive head counts, or query heads
    that are not a multiple of KV heads (checked before any division).
    """
    if rows < 1:
        raise ValueError("rows must be >= 1")
    if n_q_heads <= 0 or n_kv_heads <= 0:
        raise ValueError("head counts must be positive")
    if n_q_heads % n_kv_heads:
        raise ValueError("query heads must be a multiple of KV heads")
    gqa = n_q_heads // n_kv_heads
    if not enabled or rows > ROW_PAIR_LIMIT or rows * gqa <= ROW_PAIR_LIMIT:
        return [gqa]
    size = min(gqa, ROW_PAIR_LIMIT // rows)
    sizes = [size] * (gqa // size)
    if gqa % size:
        sizes.append(gqa % size)
    return sizes


def n_calls(rows: int, n_q_heads: int, n_kv_heads: int, enabled: bool = True) -> int:
    """Number of per-chunk attention calls over all KV groups."""
    return n_kv_heads * len(head_chunk_sizes(rows, n_q_heads, n_kv_heads, enabled))
