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
    full sort by score descending, then head ascending, then index
    descending (the more recent entry of a head first); a NaN score ranks
    below every other score (-inf included)."""
    ranked = sorted(entries, key=lambda e: (math.isnan(e[0]), 0.0 if math.isnan(e[0]) else -e[0], e[1], -e[2]))
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


def compact_by_appending(rows_by_head, keep, reserve):
    """Physical eviction built one entry at a time (DBTrimKV Method 4: paged
    per-head storage; ContourKV section 2: the kept entries are stored, not
    masked).  Heads in flat order; each kept row of a head, in slot order, is
    appended to the head's current page, a fresh 16-slot page being opened
    (numbered in opening order) whenever the head has no free slot; after its
    rows, pages are opened until the head has `reserve` free slots.

    Returns (page_off, page_ids, lengths, pages) with pages a list of
    16-slot lists of row tuples (None for a free slot)."""
    pages, page_off, lengths = [], [0], []
    for h, rows in enumerate(rows_by_head):
        mine, n = [], 0
        for i, r in enumerate(rows):
            if not keep[h][i]:
                continue
            if n == 16 * len(mine):
                pages.append([None] * 16)
                mine.append(len(pages) - 1)
            pages[mine[-1]][n % 16] = r
            n += 1
        while 16 * len(mine) - n < reserve:
            pages.append([None] * 16)
            mine.append(len(pages) - 1)
        lengths.append(n)
        page_off.append(page_off[-1] + len(mine))
    return page_off, list(range(len(pages))), lengths, pages


def largest_remainder_l2(x, total):
    """All integer vectors b >= 0 with sum(b) == total that minimise
    sum_h (b_h - x_h)^2, by exhaustive search over compositions of `total`
    (tiny inputs only).  A classical property of apportionment by largest
    remainders: its result is such a minimiser, and the only one when the
    fractional parts of x are distinct."""
    H = len(x)
    best, arg = None, []

    def rec(h, left, pre):
        nonlocal best, arg
        if h == H - 1:
            b = pre + [left]
            d = math.fsum((bi - xi) ** 2 for bi, xi in zip(b, x))
            if best is None or d < best - 1e-12:
                best, arg = d, [b]
            elif abs(d - best) <= 1e-12:
                arg.append(b)
            return
        for v in range(left + 1):
            rec(h + 1, left - v, pre + [v])

    rec(0, total, [])
    return arg


def tailfill_in_place(pool, slots_of_head, keep):
    """Tail-filled eviction of one head, one entry at a time: walking the
    slots from the front, each dropped slot below the new length takes the
    next kept entry found walking from the new length on.  pool is a list of
    per-physical-slot values, modified in place; returns the new length."""
    n_keep = sum(1 for k in keep if k)
    src = n_keep
    for i in range(n_keep):
        if keep[i]:
            continue
        while not keep[src]:
            src += 1
        pool[slots_of_head[i]] = pool[slots_of_head[src]]
        src += 1
    return n_keep
