"""Brute-force gated GQA attention with Python loops (test infrastructure only).

The definition of ``oracle.reference`` (steps 1-7 there) evaluated one scalar at
a time: math.fsum for every sum (correctly rounded), math.exp for every
exponential, explicit key sets.  No NumPy arithmetic.  Meant for tiny inputs
(a few heads, rows and keys) to pin the vectorised float64 oracle.
"""

from __future__ import annotations

import math

__all__ = ["attention", "probabilities"]


def _sigmoid(x: float) -> float:
    if x >= 0:
        return 1.0 / (1.0 + math.exp(-x))
    e = math.exp(x)
    return e / (1.0 + e)


def attention(q, k, v, gate, *, n_kv_heads: int, kv_offset: int, kv_len: int, causal: bool = True,
              scale=None, mask=None, mask_kind=None):
    """q, gate: nested sequences [B][Hq][R][D]; k, v: [B][Hkv][cap][D]; mask [Bm][Hm][R][kv_len].

    Returns a nested list [B][Hq][R][D] of floats.
    """
    B, Hq, R, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    G = Hq // n_kv_heads
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = []
    for b in range(B):
        out_b = []
        for h in range(Hq):
            g = h // G
            out_h = []
            for r in range(R):
                admissible = []
                for j in range(kv_len):
                    if causal and j > kv_offset + r:
                        continue
                    add = 0.0
                    if mask is not None and mask_kind not in (None, "none"):
                        mv = mask[b if len(mask) > 1 else 0][h if len(mask[0]) > 1 else 0][r][j]
                        if mask_kind == "bool":
                            if not mv:
                                continue
                        else:
                            if mv == -math.inf:
                                continue
                            add = float(mv)
                    admissible.append((j, add))
                if not admissible:
                    out_h.append([0.0] * D)
                    continue
                scores = {}
                for j, add in admissible:
                    scores[j] = scale * math.fsum(float(q[b][h][r][d]) * float(k[b][g][j][d]) for d in range(D)) + add
                top = max(scores.values())
                weights = {j: math.exp(s - top) for j, s in scores.items()}
                total = math.fsum(weights.values())
                row = []
                for d in range(D):
                    o = math.fsum(weights[j] * float(v[b][g][j][d]) for j in weights) / total
                    row.append(o if gate is None else o * _sigmoid(float(gate[b][h][r][d])))
                out_h.append(row)
            out_b.append(out_h)
        out.append(out_b)
    return out


def probabilities(q, k, *, n_kv_heads: int, kv_offset: int, kv_len: int, causal: bool = True, scale=None,
                  mask=None, mask_kind=None, b: int = 0, h: int = 0):
    """Softmax weights of one (b, h): p[r][j] = exp(s_j - m) / sum over A of exp(s_i - m) for j in A,
    0 off A (steps 2, 4 and 5 of the definition), one scalar at a time.

    q: [B][Hq][R][D]; k: [B][Hkv][cap][D]; mask [Bm][Hm][R][kv_len].  Returns [R][kv_len] floats.
    """
    Hq, R, D = len(q[0]), len(q[0][0]), len(q[0][0][0])
    G = Hq // n_kv_heads
    g = h // G
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = []
    for r in range(R):
        scores = {}
        for j in range(kv_len):
            if causal and j > kv_offset + r:
                continue
            add = 0.0
            if mask is not None and mask_kind not in (None, "none"):
                mv = mask[b if len(mask) > 1 else 0][h if len(mask[0]) > 1 else 0][r][j]
                if mask_kind == "bool":
                    if not mv:
                        continue
                elif mv == -math.inf:
                    continue
                else:
                    add = float(mv)
            scores[j] = scale * math.fsum(float(q[b][h][r][d]) * float(k[b][g][j][d]) for d in range(D)) + add
        row = [0.0] * kv_len
        if scores:
            top = max(scores.values())
            weights = {j: math.exp(s - top) for j, s in scores.items()}
            total = math.fsum(weights.values())
            for j, w in weights.items():
                row[j] = w / total
        out.append(row)
    return out
