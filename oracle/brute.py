"""Pure-Python brute force for tiny inputs (TEST INFRASTRUCTURE ONLY).

An independent restatement of selection and attention with Python's
``sorted`` over tuples, ``math.fsum`` and exact rationals; used to pin the
numpy reference on inputs of a few thousand entries.
"""
from __future__ import annotations

import math
from fractions import Fraction


def retention_exact(beta: float, age: int) -> Fraction:
    """r = beta^(t-i) exactly: a float32 beta is a dyadic rational
    (DBTrimKV Method 2)."""
    return Fraction(beta) ** age


def select_sorted(entries, budget):
    """entries: list of (score, head, index).  Keep the first min(M, N) of a
    full sort by score descending, then head, then index ascending; a NaN
    score ranks below every other score (-inf included)."""
    ranked = sorted(entries, key=lambda e: (math.isnan(e[0]), 0.0 if math.isnan(e[0]) else -e[0], e[1], e[2]))
    return set((h, i) for _, h, i in ranked[:max(0, min(budget, len(ranked)))])


def attention_direct(K, V, q, scale, keep):
    """Direct sums over lists: returns (out list, dropped) for one query."""
    n = len(K)
    if n == 0:
        return [0.0] * len(q), 1.0
    z = [scale * math.fsum(a * b for a, b in zip(k, q)) for k in K]
    m = max(z)
    w = [math.exp(x - m) for x in z]
    la = math.fsum(w[j] for j in range(n) if keep[j])
    ld = math.fsum(w[j] for j in range(n) if not keep[j])
    if la > 0.0:
        out = [math.fsum(w[j] * V[j][d] for j in range(n) if keep[j]) / la for d in range(len(V[0]))]
    else:
        out = [0.0] * len(q)
    return out, ld / (la + ld)


def shift_in_place(pool, slots_of_head, keep):
    """Stable in-place compaction of one head, one entry at a time: the j-th
    kept entry (in slot order) is written to the head's j-th slot.  pool is a
    list of per-physical-slot values, modified in place; slots_of_head lists
    the head's physical slots in slot order."""
    j = 0
    for i, k in enumerate(keep):
        if k:
            pool[slots_of_head[j]] = pool[slots_of_head[i]]
            j += 1
    return j
