"""Pins of the head-chunk rule (oracle.plan) against the pages and an independent search."""

import os

import pytest

from oracle import plan

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows():
    rows = []
    with open(os.path.join(GOLDEN, "head_chunk_worked_example.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            lhs, sizes, calls = (p.strip() for p in line.split("|"))
            r, hq, hkv, en = (int(x) for x in lhs.split())
            rows.append((r, hq, hkv, bool(en), [int(x) for x in sizes.split()], int(calls)))
    return rows


@pytest.mark.parametrize("case", _golden_rows())
def test_pages_worked_example(case):
    r, hq, hkv, en, sizes, calls = case
    assert plan.head_chunk_sizes(r, hq, hkv, enabled=en) == sizes
    assert plan.n_calls(r, hq, hkv, enabled=en) == calls


def _search(rows, gqa):
    """Independent formulation: the largest chunk c <= GQA with c * rows <= 32, then
    consume the group's heads greedily in order; one chunk when no split is needed."""
    if rows > 32 or rows * gqa <= 32:
        return [gqa]
    best = max(c for c in range(1, gqa + 1) if c * rows <= 32)
    left, out = gqa, []
    while left:
        take = min(best, left)
        out.append(take)
        left -= take
    return out


def test_enumeration_matches_independent_search():
    n = 0
    for rows in range(0, 41):
        for hq in range(0, 34):
            for hkv in range(0, 18):
                valid = rows >= 1 and hq > 0 and hkv > 0 and hq % hkv == 0
                if not valid:
                    with pytest.raises(ValueError):
                        plan.head_chunk_sizes(rows, hq, hkv)
                    continue
                got = plan.head_chunk_sizes(rows, hq, hkv)
                assert got == _search(rows, hq // hkv), (rows, hq, hkv)
                assert sum(got) == hq // hkv
                assert all(c * rows <= 32 for c in got) or len(got) == 1
                n += 1
    assert n > 1000
