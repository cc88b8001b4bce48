"""Plain float64 reference of the retention-scored eviction + decode path.

TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU baseline).  Slow on
purpose: every step is the definition written out, with numpy primitives
(log, matmul, lexsort, cumsum) as the only building blocks.

Data model.  A head's entries are reached through its page table: logical
page c of head h is CSR entry page_off[h] + c, stored in physical page
page_ids[page_off[h] + c]; entry i of the head is slot i % 16 of logical page
i // 16, and only i < len[h] is valid.  Per-slot "planes" that the method
produces (scores, keep flags, masses) are indexed by CSR slot
(page_off[h] + i // 16) * 16 + i % 16; pools (K, V, ln beta, pos) by
physical slot page_ids[...] * 16 + i % 16.
"""
from __future__ import annotations

import math
from decimal import Decimal, localcontext

import numpy as np

PAGE = 16


# --------------------------------------------------------------------------
# page-table views
# --------------------------------------------------------------------------
def head_phys_slots(page_off, page_ids, length, h) -> np.ndarray:
    """Physical flat slot index of each valid entry of head h, in slot order
    (the paged per-head layout of DBTrimKV, Method 4)."""
    n = int(length[h])
    i = np.arange(n, dtype=np.int64)
    c = int(page_off[h]) + i // PAGE
    return np.asarray(page_ids, np.int64)[c] * PAGE + i % PAGE


def head_csr_slots(page_off, length, h) -> np.ndarray:
    """CSR-order flat slot index of each valid entry of head h."""
    n = int(length[h])
    i = np.arange(n, dtype=np.int64)
    return (int(page_off[h]) + i // PAGE) * PAGE + i % PAGE


def gather_heads(plane, page_off, page_ids, length):
    """Split a physical per-slot plane ([n_pages, 16, ...]) into per-head
    arrays in slot order."""
    flat = plane.reshape((-1,) + plane.shape[2:])
    return [flat[head_phys_slots(page_off, page_ids, length, h)] for h in range(len(length))]


def csr_plane_to_heads(plane, page_off, length):
    flat = np.asarray(plane).reshape(-1)
    return [flat[head_csr_slots(page_off, length, h)] for h in range(len(length))]


# --------------------------------------------------------------------------
# a0: ln beta, stored once per entry
# --------------------------------------------------------------------------
def _ln_f32_exact(x: float) -> np.float32:
    """ln(x) rounded to nearest float32 (ties to even), decided at 60 digits."""
    with localcontext() as ctx:
        ctx.prec = 60
        L = Decimal(x).ln()
        f0 = np.float32(float(L))
        cands = [np.nextafter(f0, np.float32(-np.inf)), f0, np.nextafter(f0, np.float32(np.inf))]
        best, bestd = None, None
        for c in cands:
            d = abs(Decimal(float(c)) - L)
            if bestd is None or d < bestd or (d == bestd and (int(np.float32(c).view(np.uint32)) & 1) == 0):
                best, bestd = c, d
    return np.float32(best)


def ln_beta(beta) -> np.ndarray:
    """Retention in the log domain, ln(beta), correctly rounded to float32.

    TRIM-KV section 2 (retention gate): beta in [0, 1] is fixed when the
    token is created, so its logarithm is taken once per entry; DBTrimKV
    Method 2 gives r = beta^(t-i), i.e. ln r = (t-i) ln beta.  beta = 1 gives
    +0.0 and beta = 0 gives -inf.

    Method: float64 log, rounded to float32; any input whose float64 log lies
    within 64 float64 ulps of a float32 rounding midpoint is decided again
    with 60-digit decimal arithmetic.
    """
    b = np.ascontiguousarray(beta, dtype=np.float32)
    flat = b.reshape(-1)
    x = flat.astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        y = np.log(x)
    f = y.astype(np.float32)
    fin = np.isfinite(y) & (y != 0.0)
    fu = np.nextafter(f, np.float32(np.inf)).astype(np.float64)
    fd = np.nextafter(f, np.float32(-np.inf)).astype(np.float64)
    f64 = f.astype(np.float64)
    mu, md = (f64 + fu) * 0.5, (f64 + fd) * 0.5
    with np.errstate(invalid="ignore"):
        tol = 64.0 * np.abs(np.spacing(y, where=fin, out=np.ones_like(y)))
        near = fin & ((np.abs(y - mu) < tol) | (np.abs(y - md) < tol))
    for i in np.flatnonzero(near):
        f[i] = _ln_f32_exact(float(x[i]))
    return f.reshape(b.shape)


# --------------------------------------------------------------------------
# a1: retention score
# --------------------------------------------------------------------------
def score_f64(beta, t, pos) -> np.ndarray:
    """ln r_{t,i} = (t - i) ln beta_i in float64 (DBTrimKV Method 2; TRIM-KV
    section 2 decay beta^(t-i))."""
    age = (np.int64(t) - np.asarray(pos, np.int64)).astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        return age * np.log(np.asarray(beta, np.float64))


def score_f32(lnb, t, pos) -> np.ndarray:
    """The stored float32 score: float32(t - i) times the stored float32
    ln beta, one IEEE single-precision product (ages are below 2^24, so
    float32(t - i) is exact)."""
    age = (np.int64(t) - np.asarray(pos, np.int64)).astype(np.float32)
    with np.errstate(invalid="ignore"):
        return (age * np.asarray(lnb, np.float32)).astype(np.float32)


# --------------------------------------------------------------------------
# a2: one global top-M per segment, ties by (head, position)
# --------------------------------------------------------------------------
def select_global(scores, seg_head_begin, budgets, positions=None):
    """Keep flags per head (slot order) and kept count per head.

    DBTrimKV Method 3: rank every cached entry of all layers and heads by its
    predicted utility and keep the top M_global; TRIM-KV section 2: when the
    budget is exceeded, the lowest current scores are evicted.  Order: score
    descending (-0.0 equal to +0.0, -inf below every finite score, NaN
    lowest), then flat head (l, h) ascending, then slot (= position)
    descending: among equal scores of one head the more recent entry ranks
    first, so that with beta = 1 everywhere (no decay, every score 0) a head
    keeps its most recent entries.  A segment keeps min(M, N) entries.
    positions: per-head token positions in slot order, for caches whose slots
    are not in position order (tail-filled eviction); by default the slot
    index stands for the position.
    """
    keep = [np.zeros(len(s), dtype=bool) for s in scores]
    for s in range(len(seg_head_begin) - 1):
        hs = list(range(int(seg_head_begin[s]), int(seg_head_begin[s + 1])))
        if not hs:
            continue
        sc = np.concatenate([np.asarray(scores[h], np.float64) for h in hs])
        sc = np.where(sc == 0.0, 0.0, sc)            # -0.0 -> +0.0
        head = np.concatenate([np.full(len(scores[h]), h, np.int64) for h in hs])
        idx = np.concatenate([np.arange(len(scores[h]), dtype=np.int64) for h in hs])
        pos = idx if positions is None else np.concatenate([np.asarray(positions[h], np.int64) for h in hs])
        order = np.lexsort((-pos, head, -sc))
        m = max(0, min(int(budgets[s]), len(sc)))
        chosen = order[:m]
        for h in hs:
            sel = idx[chosen[head[chosen] == h]]
            keep[h][sel] = True
    kept = np.array([int(k.sum()) for k in keep], dtype=np.int32)
    return keep, kept


def select_flat(score, head, pos, budget):
    """The selection of select_global for one segment given as flat arrays
    (any entry order): keep mask of the top min(M, N) entries under the same
    total order (score descending with -0.0 equal to +0.0 and NaN lowest,
    then head ascending, then position descending).  The M-th key comes from
    a partial sort (numpy partition) instead of a full sort: every entry
    ranked above it is kept, and the entries equal to it are ranked by
    (head, position) for the places left.  For long runs of selections
    (one per decode step)."""
    key = -np.asarray(score, np.float32)    # exact; ascending = score descending; NaN last
    n = len(key)
    m = max(0, min(int(budget), n))
    keep = np.zeros(n, dtype=bool)
    if m == 0:
        return keep
    if m == n:
        keep[:] = True
        return keep
    kth = np.partition(key, m - 1)[m - 1]
    if np.isnan(kth):
        above, ties = ~np.isnan(key), np.isnan(key)
    else:
        above, ties = key < kth, key == kth
    keep[above] = True
    need = m - int(above.sum())
    idx = np.flatnonzero(ties)
    order = np.lexsort((-np.asarray(pos, np.int64)[idx], np.asarray(head, np.int64)[idx]))
    keep[idx[order[:need]]] = True
    return keep


# --------------------------------------------------------------------------
# a3: stable out-of-place compaction with prefix-sum page ids
# --------------------------------------------------------------------------
def compact_layout(kept, reserve):
    """Destination page table: head h gets ceil((kept_h + reserve)/16) pages,
    numbered by a prefix sum over heads in flat order; page_ids is the
    identity; len = kept (physical eviction, ContourKV section 2)."""
    kept = np.asarray(kept, np.int64)
    pages = -(-(kept + int(reserve)) // PAGE)
    page_off = np.zeros(len(kept) + 1, np.int64)
    np.cumsum(pages, out=page_off[1:])
    page_ids = np.arange(int(page_off[-1]), dtype=np.int64)
    return page_off, page_ids, kept.copy()


def compact(rows_by_head, keep, reserve):
    """Kept rows of every head, in slot order, with the destination layout.

    rows_by_head: dict name -> list over heads of per-entry arrays.
    Returns (page_off, page_ids, len, dict name -> list of kept arrays)."""
    kept = np.array([int(np.count_nonzero(k)) for k in keep], np.int64)
    page_off, page_ids, length = compact_layout(kept, reserve)
    out = {name: [np.asarray(r)[np.asarray(k, bool)] for r, k in zip(rows, keep)]
           for name, rows in rows_by_head.items()}
    return page_off, page_ids, length, out


# --------------------------------------------------------------------------
# incremental eviction: in place, within each head's own pages
# --------------------------------------------------------------------------
def compact_inplace_layout(kept, reserve, home_off, home_ids):
    """Page table after in-place eviction (DBTrimKV Method 4: per-head paged
    storage; ContourKV section 2: eviction shrinks storage, here without a
    second pool).  Every head keeps its kept entries, in slot order, in the
    first slots of its own pages, so its content equals the out-of-place
    compaction's; its page list becomes the first
    min(ceil((kept_h + reserve)/16), home pages of h) pages of its home list,
    with page_off a prefix sum over heads in flat order; len = kept.

    Returns (page_off, page_ids, len) as int64 arrays."""
    kept = np.asarray(kept, np.int64)
    home_off = np.asarray(home_off, np.int64)
    home_ids = np.asarray(home_ids, np.int64)
    want = -(-(kept + int(reserve)) // PAGE)
    pages = np.minimum(want, np.diff(home_off))
    page_off = np.zeros(len(kept) + 1, np.int64)
    np.cumsum(pages, out=page_off[1:])
    page_ids = np.concatenate([home_ids[home_off[h]:home_off[h] + pages[h]] for h in range(len(kept))] +
                              [np.zeros(0, np.int64)])
    return page_off, page_ids, kept.copy()


def evict_tailfill_order(keep, reserve=0, home_off=None, home_ids=None):
    """Eviction in place that moves only what it must (DBTrimKV Method 4:
    per-head paged storage; ContourKV section 2: storage shrinks), for the
    streaming loop.  Per head with kept count k: the dropped entries among
    its first k slots (holes) take, one each, the kept entries from slot k on
    (movers), both in slot order; every other kept entry stays in its slot.
    Slot order then no longer follows position order.

    Returns, per head, the old slot index held by each new slot 0..k-1; with
    home_off / home_ids also the new page table (as
    compact_inplace_layout)."""
    order = []
    for k in keep:
        k = np.asarray(k, bool)
        n_keep = int(k.sum())
        o = np.arange(n_keep, dtype=np.int64)
        holes = np.flatnonzero(~k[:n_keep])
        movers = n_keep + np.flatnonzero(k[n_keep:])
        o[holes] = movers
        order.append(o)
    if home_off is None:
        return order
    kept = [len(o) for o in order]
    return order, compact_inplace_layout(kept, reserve, home_off, home_ids)


# --------------------------------------------------------------------------
# a4: renormalised decode attention with dropped mass
# --------------------------------------------------------------------------
def decode_attn(k_heads, v_heads, q, group, scale, keep=None, lse_ref=None):
    """Per Q head qh (KV head h = qh // group):
    z_j = scale <q, k_j>, p_j = softmax over U (all valid entries of h);
    out = sum_{A} p_j v_j / sum_{A} p_j (forced weights renormalised over the
    retained set A, ContourKV problem definition); dropped = sum_{U\\A} p_j
    (ContourKV section 3).  keep=None means A = U.  With lse_ref, dropped is
    1 - exp(LSE_A - lse_ref) (dropped mass against a reference set that is
    no longer stored).  Empty A: out = 0, dropped = 1.

    Returns out [n_q, D], dropped [n_q], lse_A [n_q] (natural log of
    sum_{A} e^{z_j}); all float64.
    """
    q = np.asarray(q, np.float64)
    nq, d = q.shape
    out = np.zeros((nq, d))
    dropped = np.zeros(nq)
    lse = np.full(nq, -np.inf)
    for qh in range(nq):
        h = qh // group
        K = np.asarray(k_heads[h], np.float64)
        V = np.asarray(v_heads[h], np.float64)
        n = K.shape[0]
        A = np.ones(n, bool) if keep is None else np.asarray(keep[h], bool)
        if n == 0:
            dropped[qh] = 1.0
            continue
        z = scale * (K @ q[qh])
        m = z.max()
        w = np.exp(z - m)
        la, ld = w[A].sum(), w[~A].sum()
        if la > 0.0:
            out[qh] = (w[A] @ V[A]) / la
            lse[qh] = m + math.log(la)
        dropped[qh] = ld / (la + ld)
        if lse_ref is not None:
            dropped[qh] = -math.expm1(lse[qh] - float(lse_ref[qh])) if la > 0.0 else 1.0
    return out, dropped, lse


def decode_attn_gated(k_heads, v_heads, q, group, scale, gate_heads, keep=None):
    """Retention-gated decode attention (TRIM-KV section 2, attention
    modulation: the retention score multiplies each attention weight),
    applied at decode time and renormalised.  Per Q head qh (h = qh // group),
    with ln r_j = gate_heads[h][j] (the retention score of entry j):
    w_j = e^{z_j} r_j, z_j = scale <q, k_j>;
    out = sum_{A} w_j v_j / sum_{A} w_j; dropped = sum_{U\\A} w_j / sum_{U} w_j;
    lse = ln sum_{A} w_j.  keep=None means A = U.  Zero total weight over A
    (A empty, or r_j = 0 on all of A): out = 0, lse = -inf; dropped = 1 then.

    Returns out [n_q, D], dropped [n_q], lse [n_q]; all float64.
    """
    q = np.asarray(q, np.float64)
    nq, d = q.shape
    out = np.zeros((nq, d))
    dropped = np.ones(nq)
    lse = np.full(nq, -np.inf)
    for qh in range(nq):
        h = qh // group
        K = np.asarray(k_heads[h], np.float64)
        V = np.asarray(v_heads[h], np.float64)
        n = K.shape[0]
        if n == 0:
            continue
        A = np.ones(n, bool) if keep is None else np.asarray(keep[h], bool)
        y = scale * (K @ q[qh]) + np.asarray(gate_heads[h], np.float64)   # ln w_j
        m = y.max()
        if m == -np.inf:
            continue
        w = np.exp(y - m)
        la, ld = w[A].sum(), w[~A].sum()
        if la > 0.0:
            out[qh] = (w[A] @ V[A]) / la
            lse[qh] = m + math.log(la)
        dropped[qh] = ld / (la + ld)
    return out, dropped, lse


def subset_error(k_heads, v_heads, q, group, scale, keep):
    """e_s(A) = || mu - m_A ||_2 per Q head: mu the dense output over U,
    m_A the forced-weight output over A (ContourKV section 1)."""
    mu, _, _ = decode_attn(k_heads, v_heads, q, group, scale, keep=None)
    ma, _, _ = decode_attn(k_heads, v_heads, q, group, scale, keep=keep)
    return np.sqrt(((mu - ma) ** 2).sum(axis=1))


# --------------------------------------------------------------------------
# a5/a6: full-cache attention mass, dropped-mass statistic, allocation
# --------------------------------------------------------------------------
def attn_mass(k_heads, q, group, scale):
    """Per KV head: mass_j = (1/G) sum_g softmax_j(z_g) over the full cache
    (query-aware top-mass, ContourKV sections 1 and 3), and
    LSE_full[qh] = log sum_j e^{z_qh,j}.  Returns (list of mass arrays,
    lse_full [n_q]) in float64."""
    q = np.asarray(q, np.float64)
    nq = q.shape[0]
    lse = np.full(nq, -np.inf)
    mass = []
    for h in range(len(k_heads)):
        K = np.asarray(k_heads[h], np.float64)
        acc = np.zeros(K.shape[0])
        for g in range(group):
            qh = h * group + g
            if K.shape[0] == 0:
                continue
            z = scale * (K @ q[qh])
            m = z.max()
            l = np.exp(z - m).sum()
            lse[qh] = m + math.log(l)
            acc += np.exp(z - lse[qh])
        mass.append(acc / group)
    return mass, lse


def allocate(keptsum, length, total_budget):
    """ContourKV section 3: budget follows the dropped mass.

    mbar_h = 1 - keptsum_h (mass left outside head h's top-s set).
    S = sum_h mbar_h (float64, head order); x_h = (B * mbar_h) / S, or B / H
    when S == 0; b_h = floor(x_h); the B - sum b_h leftover units go one each
    to the largest x_h - b_h (ties to the lower head); then b_h is capped at
    len_h and the excess is offered again, one unit per head per pass, in the
    same order, to heads below their length.  Returns (b [H] int64, mbar).
    """
    keptsum = np.asarray(keptsum, np.float64)
    H = len(keptsum)
    mbar = 1.0 - keptsum
    B = int(total_budget)
    S = 0.0
    for h in range(H):
        S += float(mbar[h])
    if S > 0.0:
        x = np.array([(float(B) * float(mbar[h])) / S for h in range(H)])
    else:
        x = np.full(H, float(B) / H)
    b = np.floor(x).astype(np.int64)
    order = sorted(range(H), key=lambda h: (-(x[h] - b[h]), h))
    R = B - int(b.sum())
    for i in range(R):
        b[order[i % H]] += 1
    length = np.asarray(length, np.int64)
    excess = int(np.maximum(b - length, 0).sum())
    b = np.minimum(b, length)
    while excess > 0 and bool((b < length).any()):
        for h in order:
            if excess == 0:
                break
            if b[h] < length[h]:
                b[h] += 1
                excess -= 1
    return b, mbar


def allocate_floor(keptsum, length, total_budget, floor):
    """ContourKV section 3 with its recency floor: every head first keeps its
    most recent min(w, len_h) entries; the budget left, max(B - sum of the
    floors, 0), follows the dropped mass exactly as in allocate(), capped at
    the entries above each head's floor.  Returns (per-head totals b_h =
    floor_h + share_h, mbar)."""
    length = np.asarray(length, np.int64)
    fl = np.minimum(int(floor), length)
    share, mbar = allocate(keptsum, length - fl, max(int(total_budget) - int(fl.sum()), 0))
    return share + fl, mbar


def select_floor(per_head_scores, budgets, floor):
    """Per head: the most recent min(w, len_h) entries (the last slots, since
    positions ascend in slot order), plus the top b_h - floor_h of the other
    entries by score descending, then position descending (-0.0 == +0.0, NaN
    lowest, as in select_global).  Returns keep flags per head."""
    keep = []
    for h, sc in enumerate(per_head_scores):
        n = len(sc)
        fl = min(int(floor), n)
        k = np.zeros(n, dtype=bool)
        k[n - fl:] = True
        rest = np.asarray(sc[:n - fl], np.float64)
        rest = np.where(rest == 0.0, 0.0, rest)
        key = np.where(np.isnan(rest), -np.inf, -rest)        # ascending sort = score descending
        nan_last = np.isnan(rest).astype(np.int64)
        order = np.lexsort((-np.arange(n - fl), key, nan_last))
        m = max(0, min(int(budgets[h]) - fl, n - fl))
        k[order[:m]] = True
        keep.append(k)
    return keep


# --------------------------------------------------------------------------
# byte accounting (IndexMem section 1: a 70B model needs ~320 GB of KV at 1M tokens)
# --------------------------------------------------------------------------
def kv_cache_bytes(layers, kv_heads, head_dim, tokens, elt_bytes):
    return layers * kv_heads * head_dim * 2 * elt_bytes * tokens
