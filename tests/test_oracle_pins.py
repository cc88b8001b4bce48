"""Pins of the CPU oracle against what the pages and mathematics fix.

Each block names the passage it follows.  Expected values come from closed
forms, library routines (mpmath, torch.softmax in float64), exact rationals
or brute force, never from the oracle itself.
"""
import json
import math
import os
from fractions import Fraction

import mpmath
import numpy as np
import pytest
import torch

from oracle import brute
from oracle import reference as ref
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# helpers: an independent round-to-nearest float32 of an mpmath value
# --------------------------------------------------------------------------
def rn32(x: mpmath.mpf) -> np.float32:
    if mpmath.isinf(x):
        return np.float32(-np.inf if x < 0 else np.inf)
    f0 = np.float32(float(x))
    best = None
    for c in (np.nextafter(f0, np.float32(-np.inf)), f0, np.nextafter(f0, np.float32(np.inf))):
        d = abs(mpmath.mpf(float(c)) - x)
        if best is None or d < best[1] or (d == best[1] and (int(np.float32(c).view(np.uint32)) & 1) == 0):
            best = (c, d)
    return np.float32(best[0])


def mp_ln32(b: float) -> np.float32:
    with mpmath.workdps(50):
        if b == 0.0:
            return np.float32(-np.inf)
        return rn32(mpmath.log(mpmath.mpf(float(b))))


def bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


# --------------------------------------------------------------------------
# a0: ln beta (DBTrimKV Method 2; TRIM-KV section 2, beta in [0,1])
# --------------------------------------------------------------------------
def test_ln_beta_special_values():
    out = ref.ln_beta(np.array([1.0, 0.0], np.float32))
    assert bits(out)[0] == 0, "beta = 1 must give +0.0 (no decay)"
    assert out[1] == -np.inf, "beta = 0 must give -inf (forgotten at once)"


def test_ln_beta_powers_of_two_closed_form():
    # ln(2^-k) = -k ln 2, including subnormal beta
    ks = np.arange(1, 150)
    beta = np.ldexp(np.float32(1.0), -ks).astype(np.float32)
    got = ref.ln_beta(beta)
    with mpmath.workdps(50):
        want = np.array([rn32(-int(k) * mpmath.log(2)) for k in ks], np.float32)
    assert np.array_equal(bits(got), bits(want))


# Inputs whose ln lies within 4 float64 ulps of a float32 rounding midpoint
# (found by an exhaustive quad-precision scan of (0,1)); a plain
# "float64 log then round" gets some of these wrong.
HARD_LN_INPUTS = [0x064cb44b, 0x07c060fa, 0x0dc8bba4, 0x0f61ff63, 0x111c87f8, 0x145cb6d4,
                  0x16c5ee7a, 0x1a8446cb, 0x1f116ab8, 0x2423c085, 0x28e3fa26, 0x29e6126b,
                  0x29fd22f8, 0x2c4c24b7, 0x2e492984, 0x38dcbe38, 0x3bf86ef0, 0x3c413d3a]


def test_ln_beta_hard_rounding_cases():
    beta = np.array(HARD_LN_INPUTS, np.uint32).view(np.float32)
    got = ref.ln_beta(beta)
    want = np.array([mp_ln32(float(b)) for b in beta], np.float32)
    assert np.array_equal(bits(got), bits(want))


def test_ln_beta_random_correctly_rounded():
    rng = np.random.default_rng(7)
    beta = np.concatenate([
        rng.beta(2, 2, 1500), rng.beta(50, 1, 1500), rng.beta(1, 20, 500),
        1.0 - rng.random(300) * 1e-6,                                   # very close to 1
    ]).astype(np.float32)
    # plus raw float32 bit patterns over [0, 1]
    beta = np.concatenate([beta, rng.integers(0, 0x3F800000, 2000, dtype=np.uint32).view(np.float32)])
    got = ref.ln_beta(beta)
    want = np.array([mp_ln32(float(b)) for b in beta], np.float32)
    assert np.array_equal(bits(got), bits(want))


def test_ln_beta_monotone():
    rng = np.random.default_rng(8)
    beta = np.sort(rng.random(20000).astype(np.float32))
    assert np.all(np.diff(ref.ln_beta(beta).astype(np.float64)) >= 0)


# --------------------------------------------------------------------------
# a1: scores (DBTrimKV Method 2; TRIM-KV section 2, decay beta^(t-i))
# --------------------------------------------------------------------------
def test_score_relative_error_and_specials():
    rng = np.random.default_rng(9)
    beta = rng.beta(2, 2, 5000).astype(np.float32)
    pos = rng.integers(0, 139263, 5000)
    t = 139264
    s32 = ref.score_f32(ref.ln_beta(beta), t, pos)
    s64 = ref.score_f64(beta, t, pos)
    assert np.max(np.abs(s32 - s64) / np.abs(s64)) <= 1e-6
    # beta = 1 -> +0.0 at every age; beta = 0 -> -inf
    z = ref.score_f32(ref.ln_beta(np.ones(4, np.float32)), 100, np.array([0, 50, 98, 99]))
    assert np.all(bits(z) == 0)
    z = ref.score_f32(ref.ln_beta(np.zeros(3, np.float32)), 100, np.array([0, 50, 99]))
    assert np.all(z == -np.inf)


def test_score_powers_of_two():
    # beta = 2^-k, age a: s = -a k ln 2 within 1.5 float32 ulp
    for k in (1, 3, 17):
        for a in (1, 7, 4096, 139264):
            s = float(ref.score_f32(ref.ln_beta(np.float32(2.0 ** -k)), a, 0).reshape(-1)[0])
            with mpmath.workdps(40):
                want = float(-a * k * mpmath.log(2))
            assert abs(s - want) <= 1.5 * np.spacing(np.float32(abs(want)))


def test_score_order_preserved_under_decay():
    # Ranking by exact r = beta^(t-i) equals ranking by the float64 log-score
    # wherever two log-scores differ by more than 4 ulps.
    rng = np.random.default_rng(10)
    n, t = 120, 300
    beta = rng.beta(5, 1, n).astype(np.float32)
    pos = rng.integers(0, t, n)
    s64 = ref.score_f64(beta, t, pos)
    r = [brute.retention_exact(float(b), int(t - p)) for b, p in zip(beta, pos)]
    for i in range(n):
        for j in range(i + 1, n):
            if abs(s64[i] - s64[j]) > 4 * np.spacing(max(abs(s64[i]), abs(s64[j]))):
                assert (s64[i] > s64[j]) == (r[i] > r[j])


def test_score_ranking_monotone_in_t():
    # if beta_a >= beta_b and a outranks b at step t, a outranks b later too
    rng = np.random.default_rng(11)
    beta = rng.beta(2, 2, 400).astype(np.float32)
    pos = rng.integers(0, 1000, 400)
    for t0 in (1000, 1500):
        s0 = ref.score_f64(beta, t0, pos)
        s1 = ref.score_f64(beta, t0 + 333, pos)
        a, b = np.meshgrid(np.arange(400), np.arange(400), indexing="ij")
        m = (beta[a] >= beta[b]) & (s0[a] > s0[b])
        assert np.all(s1[a][m] > s1[b][m] - 1e-9)


# --------------------------------------------------------------------------
# a2: global top-M selection (DBTrimKV Method 3; TRIM-KV section 2)
# --------------------------------------------------------------------------
def _random_scores(rng, kind, lens):
    out = []
    for n in lens:
        if kind == "cont":
            s = -rng.random(n) * 10
        elif kind == "alpha3":
            s = rng.choice([-1.5, -0.25, 0.0], n)
        elif kind == "equal":
            s = np.full(n, -0.5)
        elif kind == "zeros":
            s = rng.choice([0.0, -0.0], n)
        elif kind == "nan":  # NaN, -inf, signed zeros and finite values
            s = np.where(rng.random(n) < 0.25, np.nan, rng.choice([-np.inf, -2.0, -0.0, 0.0, 1.5], n))
        else:  # with -inf
            s = np.where(rng.random(n) < 0.3, -np.inf, -rng.integers(0, 4, n).astype(np.float64))
        out.append(s.astype(np.float32))
    return out


SORT_KINDS = ["cont", "alpha3", "equal", "zeros", "inf", "nan"]


@pytest.mark.parametrize("kind", SORT_KINDS)
def test_select_equals_full_sort(kind):
    rng = np.random.default_rng(SORT_KINDS.index(kind) + 100)
    for trial in range(300):
        H = int(rng.integers(1, 7))
        lens = rng.integers(0, 40, H)
        scores = _random_scores(rng, kind, lens)
        n_seg = int(rng.integers(1, H + 1))
        cuts = np.sort(rng.choice(np.arange(1, H), size=n_seg - 1, replace=False)) if n_seg > 1 else []
        seg = np.concatenate([[0], cuts, [H]]).astype(np.int32)
        budgets = []
        for s in range(len(seg) - 1):
            N = int(sum(lens[seg[s]:seg[s + 1]]))
            budgets.append(int(rng.choice([0, 1, max(N - 1, 0), N, N + 5, int(rng.integers(0, N + 1))])))
        keep, kept = ref.select_global(scores, seg, budgets)
        for s in range(len(seg) - 1):
            ent = [(float(scores[h][i]), h, i) for h in range(seg[s], seg[s + 1]) for i in range(lens[h])]
            want = brute.select_sorted(ent, budgets[s])
            got = set((h, i) for h in range(seg[s], seg[s + 1]) for i in np.flatnonzero(keep[h]))
            assert got == want
            assert sum(kept[seg[s]:seg[s + 1]]) == min(max(budgets[s], 0), sum(lens[seg[s]:seg[s + 1]]))


@pytest.mark.parametrize("kind", SORT_KINDS)
def test_select_flat_equals_full_sort(kind):
    """The partial-sort selection over flat, shuffled entries keeps exactly
    the set of a brute-force full sort (pure Python)."""
    rng = np.random.default_rng(SORT_KINDS.index(kind) + 300)
    for trial in range(150):
        H = int(rng.integers(1, 7))
        lens = rng.integers(0, 40, H)
        scores = _random_scores(rng, kind, lens)
        head = np.concatenate([np.full(n, h) for h, n in enumerate(lens)] + [np.zeros(0, int)])
        pos = np.concatenate([np.sort(rng.choice(500, n, replace=False)) for n in lens] + [np.zeros(0, int)])
        sc = np.concatenate(scores + [np.zeros(0, np.float32)])
        perm = rng.permutation(len(sc))
        N = len(sc)
        for M in (0, 1, max(N - 1, 0), N, N + 4, int(rng.integers(0, N + 1))):
            keep = ref.select_flat(sc[perm], head[perm], pos[perm], M)
            got = set((int(head[perm][j]), int(pos[perm][j])) for j in np.flatnonzero(keep))
            want = brute.select_sorted([(float(sc[j]), int(head[j]), int(pos[j])) for j in range(N)], M)
            assert got == want, (trial, M)


def test_select_constant_beta_is_sliding_window():
    # beta = c in (0,1) everywhere: the score only depends on age, so the
    # kept set is the newest floor(M/H) of every head plus one more for the
    # first M mod H heads (ties broken by head index).
    H, n, t = 5, 64, 64
    lnb = ref.ln_beta(np.full(n, 0.9, np.float32))
    pos = np.arange(n)
    scores = [ref.score_f32(lnb, t, pos) for _ in range(H)]
    for M in (0, 1, 7, 63, 64, 100, 319, 320, 400):
        keep, kept = ref.select_global(scores, [0, H], [M])
        m = min(M, H * n)
        for h in range(H):
            w = m // H + (1 if h < m % H else 0)
            want = np.zeros(n, bool)
            want[n - w:] = True
            assert np.array_equal(keep[h], want), (M, h)


def test_select_beta_one_retains_all_or_most_recent():
    """beta = 1 for every entry: no decay, every score is 0.  A budget of at
    least N keeps every entry; a smaller one fills the heads in (l, h) order,
    and every head it reaches keeps its most recent entries (a suffix of the
    head in position order)."""
    rng = np.random.default_rng(23)
    for trial in range(60):
        H = int(rng.integers(1, 7))
        lens = rng.integers(0, 40, H)
        t = 64
        scores = [ref.score_f32(ref.ln_beta(np.ones(n, np.float32)), t, np.sort(rng.choice(t, n, replace=False)))
                  for n in lens]
        N = int(lens.sum())
        for M in (0, 1, int(rng.integers(0, N + 1)), max(N - 1, 0), N, N + 3):
            keep, kept = ref.select_global(scores, [0, H], [M])
            left = min(M, N)
            for h in range(H):
                k = min(left, int(lens[h]))
                want = np.zeros(int(lens[h]), bool)
                want[int(lens[h]) - k:] = True
                assert np.array_equal(keep[h], want), (trial, M, h)
                left -= k
            if M >= N:
                assert all(k.all() for k in keep)


def test_select_segments_independent():
    rng = np.random.default_rng(12)
    scores = _random_scores(rng, "alpha3", rng.integers(5, 30, 8))
    keep, _ = ref.select_global(scores, [0, 3, 8], [10, 17])
    k1, _ = ref.select_global(scores[:3], [0, 3], [10])
    k2, _ = ref.select_global(scores[3:], [0, 5], [17])
    for a, b in zip(keep, k1 + k2):
        assert np.array_equal(a, b)


# --------------------------------------------------------------------------
# a3: compaction (DBTrimKV Method 4; ContourKV section 2, physical budget)
# --------------------------------------------------------------------------
def test_compaction_round_trip_and_layout():
    cache = synth.random_ragged_cache(13, n_heads=6, d=8, dtype="f32", max_len=70)
    po, pi, ln = cache.page_off, cache.page_ids, cache.length
    rng = np.random.default_rng(13)
    keep = [rng.random(int(n)) < 0.4 for n in ln]
    rows = {"k": ref.gather_heads(cache.k, po, pi, ln), "pos": ref.gather_heads(cache.pos, po, pi, ln)}
    for reserve in (0, 1, 3):
        dpo, dpi, dlen, out = ref.compact(rows, keep, reserve)
        kept = np.array([k.sum() for k in keep])
        assert np.array_equal(dlen, kept)
        assert np.array_equal(np.diff(dpo), -(-(kept + reserve) // 16))
        assert np.array_equal(dpi, np.arange(dpo[-1]))
        for h in range(6):
            assert np.array_equal(out["k"][h], rows["k"][h][keep[h]])
            assert np.all(np.diff(out["pos"][h]) > 0)     # positions stay ascending


def test_compaction_equals_page_by_page_appending():
    """The compacted layout built constructively: every head's kept rows are
    appended one at a time into fresh 16-slot pages opened in order, with
    `reserve` free slots left per head (brute force, pure Python).  The
    oracle's page table, lengths and rows read back through its CSR must
    equal that construction."""
    rng = np.random.default_rng(29)
    for trial in range(60):
        H = int(rng.integers(1, 7))
        lens = rng.integers(0, 70, H)
        rows = [[(h, i, int(rng.integers(1 << 30))) for i in range(int(n))] for h, n in enumerate(lens)]
        keep = [rng.random(int(n)) < rng.uniform(0.0, 1.0) for n in lens]
        reserve = int(rng.choice([0, 1, 3, 16, 17]))
        bpo, bpi, bln, bpages = brute.compact_by_appending(rows, [k.tolist() for k in keep], reserve)
        po, pi, ln, out = ref.compact({"r": [np.array(r, dtype=object).reshape(-1, 3) for r in rows]}, keep,
                                      reserve)
        assert list(po) == bpo and list(pi) == bpi and list(ln) == bln, trial
        for h in range(H):
            got = [tuple(int(v) for v in out["r"][h][j]) for j in range(int(ln[h]))]
            back = [bpages[bpi[bpo[h] + j // 16]][j % 16] for j in range(bln[h])]
            assert got == back, (trial, h)
            # free slots: the head's pages hold exactly `reserve` or more spare slots, fewer than 16 + reserve
            spare = 16 * (bpo[h + 1] - bpo[h]) - bln[h]
            assert reserve <= spare < reserve + 16 or (spare == 0 and reserve == 0)


def test_tailfill_eviction_order():
    """Tail-filled eviction against a one-entry-at-a-time walk (brute force,
    pure Python): the kept rows of every head fill its first slots, entries
    kept below the new length stay where they were, and exactly the drops
    below the new length move."""
    rng = np.random.default_rng(37)
    for trial in range(40):
        H = int(rng.integers(1, 6))
        length = rng.integers(0, 70, H)
        home_pages = -(-length // 16) + rng.integers(0, 3, H)
        home_off = np.concatenate([[0], np.cumsum(home_pages)]).astype(np.int64)
        home_ids = rng.permutation(int(home_off[-1]) + 2)[:home_off[-1]].astype(np.int64)
        pool = list(rng.integers(0, 1 << 30, (int(home_off[-1]) + 2) * 16))
        keep = [rng.random(int(n)) < rng.uniform(0.0, 1.0) for n in length]
        slots = [[int(home_ids[home_off[h] + i // 16]) * 16 + i % 16 for i in range(int(length[h]))]
                 for h in range(H)]
        rows = [[pool[x] for x in slots[h]] for h in range(H)]
        reserve = int(rng.integers(0, 20))
        order, (po, pi, ln) = ref.evict_tailfill_order(keep, reserve, home_off, home_ids)
        for h in range(H):
            n = brute.tailfill_in_place(pool, slots[h], keep[h].tolist())
            assert n == int(ln[h]) == len(order[h])
            got = [pool[slots[h][j]] for j in range(n)]
            assert got == [rows[h][i] for i in order[h]], (trial, h)
            assert sorted(order[h].tolist()) == np.flatnonzero(keep[h]).tolist()
            stay = [j for j in range(n) if keep[h][j]]
            assert all(order[h][j] == j for j in stay)
            assert sum(1 for j in range(n) if order[h][j] != j) == int((~keep[h][:n]).sum())


def test_select_ties_rank_by_position_in_any_slot_order():
    """With positions given (slots out of position order), ties rank by
    position descending within a head: equal to a brute-force sort on
    (score, head, -position), and the same keep set as the slot-ordered
    cache that holds the same entries."""
    rng = np.random.default_rng(38)
    for trial in range(200):
        H = int(rng.integers(1, 6))
        lens = rng.integers(0, 30, H)
        kind = SORT_KINDS[trial % len(SORT_KINDS)]
        scores = _random_scores(rng, kind, lens)
        pos = [np.sort(rng.choice(200, int(n), replace=False)) for n in lens]
        perm = [rng.permutation(int(n)) for n in lens]
        sp = [s[p] for s, p in zip(scores, perm)]
        pp = [x[p] for x, p in zip(pos, perm)]
        M = int(rng.integers(0, int(lens.sum()) + 3))
        keep, kept = ref.select_global(sp, [0, H], [M], positions=pp)
        want = brute.select_sorted([(float(sp[h][i]), h, int(pp[h][i])) for h in range(H) for i in range(int(lens[h]))],
                                   M)
        got = set((h, int(pp[h][i])) for h in range(H) for i in np.flatnonzero(keep[h]))
        assert got == want, trial
        k2, kept2 = ref.select_global(scores, [0, H], [M])
        assert set((h, int(pos[h][i])) for h in range(H) for i in np.flatnonzero(k2[h])) == got
        assert np.array_equal(kept, kept2)


def test_inplace_compaction_layout_and_sequential_shift():
    """In-place eviction: a one-entry-at-a-time shift over a tiny pool (brute
    force, in pure Python) leaves every head's kept rows, in order, in the
    first slots of its own pages; read back through the oracle's new table
    they equal the out-of-place rows.  The table is the home prefix of
    ceil((kept + reserve)/16) pages, clamped to the home list; rows of other
    heads are untouched."""
    rng = np.random.default_rng(17)
    for trial in range(30):
        H = int(rng.integers(1, 6))
        length = rng.integers(0, 60, H)
        extra = rng.integers(0, 3, H)                            # spare home pages per head
        home_pages = -(-length // 16) + extra
        home_off = np.concatenate([[0], np.cumsum(home_pages)]).astype(np.int64)
        n_pages = int(home_off[-1]) + 2
        home_ids = rng.permutation(n_pages)[:home_off[-1]].astype(np.int64)
        pool = list(rng.integers(0, 1 << 30, n_pages * 16))
        keep = [rng.random(int(n)) < rng.uniform(0.2, 1.0) for n in length]
        slots = [[int(home_ids[home_off[h] + i // 16]) * 16 + i % 16 for i in range(int(length[h]))]
                 for h in range(H)]
        rows = [[pool[x] for x in slots[h]] for h in range(H)]
        reserve = int(rng.integers(0, 40))
        before = list(pool)
        kept = [brute.shift_in_place(pool, slots[h], keep[h].tolist()) for h in range(H)]
        po, pi, ln = ref.compact_inplace_layout(kept, reserve, home_off, home_ids)
        assert np.array_equal(ln, [int(k.sum()) for k in keep])
        for h in range(H):
            n = min(-(-(kept[h] + reserve) // 16), int(home_pages[h]))
            assert po[h + 1] - po[h] == n
            assert np.array_equal(pi[po[h]:po[h + 1]], home_ids[home_off[h]:home_off[h] + n])
            got = [pool[int(pi[po[h] + j // 16]) * 16 + j % 16] for j in range(kept[h])]
            assert got == [r for r, k in zip(rows[h], keep[h]) if k], (trial, h)
        # slots outside every head's pages are untouched
        owned = set(x for h in range(H) for x in slots[h])
        assert all(pool[x] == before[x] for x in range(len(pool)) if x not in owned)


# --------------------------------------------------------------------------
# a4: renormalised decode attention (ContourKV problem definition, sections 1, 3)
# --------------------------------------------------------------------------
def _heads(rng, H, n, d):
    K = [rng.standard_normal((int(x), d)) for x in n]
    V = [rng.standard_normal((int(x), d)) for x in n]
    return K, V


def test_attention_zero_query_is_uniform():
    rng = np.random.default_rng(14)
    K, V = _heads(rng, 3, [9, 16, 5], 8)
    keep = [rng.random(len(k)) < 0.5 for k in K]
    for k in keep:
        k[0] = True
    keep[2][:] = False
    keep[2][3] = True
    out, dropped, _ = ref.decode_attn(K, V, np.zeros((3, 8)), 1, 0.3, keep=keep)
    for h in range(3):
        A = keep[h]
        assert np.allclose(out[h], V[h][A].mean(0), atol=1e-14)
        assert abs(dropped[h] - (1 - A.sum() / len(A))) < 1e-15


def test_attention_full_set_matches_torch_softmax():
    rng = np.random.default_rng(15)
    K, V = _heads(rng, 2, [33, 17], 16)
    q = rng.standard_normal((8, 16))
    out, dropped, lse = ref.decode_attn(K, V, q, 4, 0.25)
    for qh in range(8):
        h = qh // 4
        z = torch.tensor(K[h] @ q[qh] * 0.25, dtype=torch.float64)
        p = torch.softmax(z, 0).numpy()
        assert np.allclose(out[qh], p @ V[h], atol=1e-13)
        assert dropped[qh] == 0.0
        assert abs(lse[qh] - torch.logsumexp(z, 0).item()) < 1e-12


def test_attention_single_and_empty_kept_set():
    rng = np.random.default_rng(16)
    K, V = _heads(rng, 2, [12, 0], 4)
    keep = [np.zeros(12, bool), np.zeros(0, bool)]
    keep[0][5] = True
    q = rng.standard_normal((2, 4))
    out, dropped, _ = ref.decode_attn(K, V, q, 1, 0.5, keep=keep)
    assert np.allclose(out[0], V[0][5], atol=1e-15)
    assert np.all(out[1] == 0) and dropped[1] == 1.0
    keep[0][:] = False
    out, dropped, lse = ref.decode_attn(K, V, q, 1, 0.5, keep=keep)
    assert np.all(out[0] == 0) and dropped[0] == 1.0 and lse[0] == -np.inf


def test_attention_renormalised_equals_softmax_over_kept_and_dilution():
    rng = np.random.default_rng(17)
    K, V = _heads(rng, 1, [50], 8)
    q = rng.standard_normal((1, 8)) * 2
    keep = [rng.random(50) < 0.3]
    out, dropped, _ = ref.decode_attn(K, V, q, 1, 0.35, keep=keep)
    A = keep[0]
    z = K[0][A] @ q[0] * 0.35
    p = torch.softmax(torch.tensor(z, dtype=torch.float64), 0).numpy()
    assert np.allclose(out[0], p @ V[0][A], atol=1e-13)
    zfull = torch.tensor(K[0] @ q[0] * 0.35, dtype=torch.float64)
    pfull = torch.softmax(zfull, 0).numpy()
    assert abs(dropped[0] - pfull[~A].sum()) < 1e-14
    assert abs((1 - dropped[0]) - pfull[A].sum()) < 1e-14      # kept + dropped = 1
    assert np.all(p >= pfull[A] - 1e-16)                        # dilution: p_j/kept >= p_j


def test_attention_matches_direct_sums():
    rng = np.random.default_rng(18)
    K, V = _heads(rng, 3, [7, 21, 1], 6)
    q = rng.standard_normal((6, 6))
    keep = [rng.random(len(k)) < 0.6 for k in K]
    out, dropped, _ = ref.decode_attn(K, V, q, 2, 0.4, keep=keep)
    for qh in range(6):
        h = qh // 2
        o, d = brute.attention_direct(K[h].tolist(), V[h].tolist(), q[qh].tolist(), 0.4, keep[h].tolist())
        assert np.allclose(out[qh], o, atol=1e-13) and abs(dropped[qh] - d) < 1e-14


def test_attention_reference_mode_matches_mask_mode():
    rng = np.random.default_rng(19)
    K, V = _heads(rng, 2, [40, 25], 8)
    q = rng.standard_normal((4, 8))
    keep = [rng.random(len(k)) < 0.5 for k in K]
    _, dmask, _ = ref.decode_attn(K, V, q, 2, 0.3, keep=keep)
    _, _, lse_full = ref.decode_attn(K, V, q, 2, 0.3)
    Kk = [k[m] for k, m in zip(K, keep)]
    Vk = [v[m] for v, m in zip(V, keep)]
    _, dref, _ = ref.decode_attn(Kk, Vk, q, 2, 0.3, lse_ref=lse_full)
    assert np.allclose(dref, dmask, atol=1e-13)


def test_subset_error():
    rng = np.random.default_rng(20)
    K, V = _heads(rng, 1, [10], 4)
    q = rng.standard_normal((1, 4))
    e = ref.subset_error(K, V, q, 1, 0.5, [np.ones(10, bool)])
    assert e[0] < 1e-15
    one = np.zeros(10, bool)
    one[4] = True
    mu, _, _ = ref.decode_attn(K, V, q, 1, 0.5)
    e = ref.subset_error(K, V, q, 1, 0.5, [one])
    assert abs(e[0] - np.linalg.norm(mu[0] - V[0][4])) < 1e-14


def test_subset_error_decomposition():
    """The dense output splits as mu = (1 - d) m_A + d m_D (d the dropped
    mass, m_D the output renormalised over the dropped keys), so
    e_s(A) = d ||m_A - m_D||.  m_A, m_D and d come from direct sums (brute
    force), not from the oracle.  Empty A: m_A = 0, so e = ||mu||."""
    rng = np.random.default_rng(31)
    for trial in range(40):
        n, d = int(rng.integers(2, 14)), int(rng.integers(1, 6))
        K = [rng.standard_normal((n, d)) * 2]
        V = [rng.standard_normal((n, d))]
        q = rng.standard_normal((1, d))
        keep = rng.random(n) < 0.5
        keep[int(rng.integers(0, n))] = True
        e = ref.subset_error(K, V, q, 1, 0.7, [keep])[0]
        oa, dm = brute.attention_direct(K[0].tolist(), V[0].tolist(), q[0].tolist(), 0.7, keep.tolist())
        if keep.all():
            assert e < 1e-14
            continue
        od, _ = brute.attention_direct(K[0].tolist(), V[0].tolist(), q[0].tolist(), 0.7, (~keep).tolist())
        want = dm * math.sqrt(math.fsum((x - y) ** 2 for x, y in zip(oa, od)))
        assert abs(e - want) <= 1e-13 * max(1.0, want), trial
    mu, _ = brute.attention_direct(K[0].tolist(), V[0].tolist(), q[0].tolist(), 0.7, [True] * len(K[0]))
    e0 = ref.subset_error(K, V, q, 1, 0.7, [np.zeros(len(K[0]), bool)])[0]
    assert abs(e0 - math.sqrt(math.fsum(x * x for x in mu))) < 1e-13


# --------------------------------------------------------------------------
# retention-gated attention (TRIM-KV section 2, attention modulation)
# --------------------------------------------------------------------------
def test_gated_attention_direct_weights():
    """Weights e^{z_j} * beta_j^(t - pos_j) formed as a product with pow (not
    in the log domain), sums by fsum; the oracle is given ln r = the float64
    score.  Includes beta = 0 (weight 0) and beta = 1 (weight e^z)."""
    rng = np.random.default_rng(41)
    for trial in range(40):
        n, d = int(rng.integers(1, 12)), int(rng.integers(1, 6))
        K = rng.standard_normal((n, d))
        V = rng.standard_normal((n, d))
        q = rng.standard_normal((1, d))
        beta = rng.uniform(0.2, 1.0, n)
        beta[rng.random(n) < 0.15] = 0.0
        beta[rng.random(n) < 0.15] = 1.0
        pos = rng.permutation(40)[:n]
        t = 40 + int(rng.integers(0, 5))
        keep = rng.random(n) < 0.6
        gate = ref.score_f64(beta, t, pos)
        out, dropped, lse = ref.decode_attn_gated([K], [V], q, 1, 0.8, [gate], keep=[keep])
        w = [math.exp(0.8 * math.fsum(a * b for a, b in zip(K[j], q[0]))) * float(beta[j]) ** (t - int(pos[j]))
             for j in range(n)]
        la = math.fsum(w[j] for j in range(n) if keep[j])
        lu = math.fsum(w)
        if la == 0.0:
            assert np.all(out[0] == 0) and lse[0] == -np.inf and dropped[0] == 1.0
            continue
        want = [math.fsum(w[j] * V[j][c] for j in range(n) if keep[j]) / la for c in range(d)]
        assert np.allclose(out[0], want, rtol=1e-12, atol=1e-13), trial
        assert abs(dropped[0] - (lu - la) / lu) < 1e-13
        assert abs(lse[0] - math.log(la)) < 1e-12 * max(1.0, abs(math.log(la)))


def test_gated_attention_reductions():
    """beta = 1 everywhere is ungated attention; a gate constant over a head
    changes only lse (by that constant); q = 0 with one beta makes the
    weights geometric, whose sums have closed forms; beta = 0 on every entry
    of a head (age > 0) leaves no weight: out 0, dropped 1."""
    rng = np.random.default_rng(42)
    K, V = [rng.standard_normal((n, 6)) for n in (9, 0, 20)], [rng.standard_normal((n, 6)) for n in (9, 0, 20)]
    q = rng.standard_normal((6, 6))
    keep = [rng.random(len(k)) < 0.5 for k in K]
    zero = [np.zeros(len(k)) for k in K]
    for kp in (None, keep):
        a = ref.decode_attn(K, V, q, 2, 0.6, keep=kp)
        b = ref.decode_attn_gated(K, V, q, 2, 0.6, zero, keep=kp)
        for x, y in zip(a, b):
            assert np.array_equal(x, y)
        c = ref.decode_attn_gated(K, V, q, 2, 0.6, [np.full(len(k), -3.25) for k in K], keep=kp)
        assert np.allclose(c[0], a[0], atol=1e-14) and np.allclose(c[1], a[1], atol=1e-14)
        fin = np.isfinite(a[2])
        assert np.allclose(c[2][fin], a[2][fin] - 3.25, atol=1e-13) and np.all(c[2][~fin] == -np.inf)
    # geometric: n entries at positions 0..n-1, t = n, v_i = i, weights x^(n-i)
    for n, x in ((1, 0.5), (7, 0.9), (30, 0.97), (12, 0.25)):
        Kg = [np.ones((n, 1))]
        Vg = [np.arange(n, dtype=np.float64).reshape(n, 1)]
        gate = [ref.score_f64(np.full(n, x), n, np.arange(n))]
        out, dropped, _ = ref.decode_attn_gated(Kg, Vg, np.zeros((1, 1)), 1, 1.0, gate)
        s1 = x * (1 - x ** n) / (1 - x)                                     # sum_{k=1..n} x^k
        sk = x * (1 - (n + 1) * x ** n + n * x ** (n + 1)) / (1 - x) ** 2   # sum_{k=1..n} k x^k
        assert abs(out[0, 0] - (n * s1 - sk) / s1) < 1e-12 * n and dropped[0] == 0.0
    gate = [np.full(9, -np.inf), np.zeros(0), ref.score_f64(np.linspace(0.5, 1.0, 20), 30, np.arange(20))]
    out, dropped, lse = ref.decode_attn_gated(K, V, q, 2, 0.6, gate)
    assert np.all(out[:4] == 0) and np.all(dropped[:4] == 1) and np.all(lse[:4] == -np.inf)
    assert np.all(np.isfinite(lse[4:]))


# --------------------------------------------------------------------------
# a5/a6: attention mass and allocation (ContourKV section 3)
# --------------------------------------------------------------------------
def test_mass_is_mean_softmax():
    rng = np.random.default_rng(21)
    K, _ = _heads(rng, 2, [30, 11], 8)
    q = rng.standard_normal((6, 8))
    mass, lse = ref.attn_mass(K, q, 3, 0.5)
    for h in range(2):
        assert abs(mass[h].sum() - 1) < 1e-14
        want = np.zeros(len(K[h]))
        for g in range(3):
            want += torch.softmax(torch.tensor(K[h] @ q[h * 3 + g] * 0.5, dtype=torch.float64), 0).numpy() / 3
        assert np.allclose(mass[h], want, atol=1e-15)
    m1, _ = ref.attn_mass(K, q[[0, 3]], 1, 0.5)
    p = torch.softmax(torch.tensor(K[0] @ q[0] * 0.5, dtype=torch.float64), 0).numpy()
    assert np.allclose(m1[0], p, atol=1e-16)


def test_recency_floor_selection_and_allocation():
    """ContourKV recency floor.  Selection equals a brute-force sort of the
    non-floor entries plus the floor; w = 0 reduces to the plain per-head
    selection and allocation; every total stays within [floor_h, len_h] and
    sums to the budget when the floors fit (else the floors alone are kept)."""
    rng = np.random.default_rng(41)
    for trial in range(200):
        H = int(rng.integers(1, 6))
        lens = rng.integers(0, 30, H)
        sc = [rng.choice([-1.0, 0.0, 0.5, 2.0, np.nan, np.inf], int(n)).astype(np.float32) for n in lens]
        w = int(rng.integers(0, 8))
        b = [int(rng.integers(0, n + 3)) for n in lens]
        got = ref.select_floor(sc, b, w)
        for h in range(H):
            n, fl = int(lens[h]), min(w, int(lens[h]))
            ent = [(float(sc[h][i]), h, i) for i in range(n - fl)]
            want = brute.select_sorted(ent, b[h] - fl) | {(h, i) for i in range(n - fl, n)}
            assert set((h, i) for i in np.flatnonzero(got[h])) == want, trial
        if w == 0:
            plain, _ = ref.select_global(sc, np.arange(H + 1), b)
            assert all(np.array_equal(x, y) for x, y in zip(got, plain))
        ks = rng.random(H)
        B = int(rng.integers(0, int(lens.sum()) + 5))
        bt, _ = ref.allocate_floor(ks, lens, B, w)
        fl = np.minimum(w, lens)
        assert np.all(bt >= fl) and np.all(bt <= lens)
        if B >= fl.sum():
            assert bt.sum() == min(B, int(lens.sum()))
        else:
            assert np.array_equal(bt, fl)
        if w == 0:
            assert np.array_equal(bt, ref.allocate(ks, lens, B)[0])


def test_allocation_is_the_least_squares_apportionment():
    """Uncapped allocation against a property of largest-remainder
    apportionment: among integer budgets with the right total it minimises
    sum (b_h - x_h)^2, x_h = B mbar_h / S (brute force over every
    composition of B); with distinct fractional parts it is the unique
    minimiser.  Lengths never bind here."""
    rng = np.random.default_rng(27)
    for trial in range(150):
        H = int(rng.integers(1, 5))
        ks = rng.random(H)
        B = int(rng.integers(0, 14))
        b, mbar = ref.allocate(ks, [10 ** 6] * H, B)
        S = math.fsum(1.0 - k for k in ks)
        x = [B * (1.0 - k) / S for k in ks]
        mins = brute.largest_remainder_l2(x, B)
        assert list(b) in mins, (trial, list(b), mins)
        fr = [xi - math.floor(xi) for xi in x]
        if len(set(round(f, 9) for f in fr)) == H:
            assert len(mins) == 1


def test_allocation_rules():
    # proportional, exact
    b, mbar = ref.allocate([0.5, 0.75, 0.75], [100, 100, 100], 8)
    assert list(b) == [4, 2, 2] and np.allclose(mbar, [0.5, 0.25, 0.25])
    # uniform dropped mass: B/H each, leftover to the lowest heads
    b, _ = ref.allocate([0.6] * 4, [100] * 4, 10)
    assert list(b) == [3, 3, 2, 2]
    # leftover goes to the largest fractional part
    b, _ = ref.allocate([0.0, 0.5, 0.8], [100] * 3, 10)   # mbar 1, .5, .2 -> x 5.88, 2.94, 1.18
    assert list(b) == [6, 3, 1]
    # capped at the head length; excess offered again in remainder order
    b, _ = ref.allocate([0.5, 0.75, 0.75], [1, 100, 100], 8)
    assert list(b) == [1, 4, 3]
    # budget above the cache: everything kept
    b, _ = ref.allocate([0.2, 0.9], [5, 7], 100)
    assert list(b) == [5, 7]
    # zero dropped mass everywhere -> uniform
    b, _ = ref.allocate([1.0, 1.0, 1.0], [50] * 3, 7)
    assert list(b) == [3, 2, 2]
    rng = np.random.default_rng(22)
    for _ in range(200):
        H = int(rng.integers(1, 30))
        ks = rng.random(H)
        ln = rng.integers(0, 500, H)
        B = int(rng.integers(0, ln.sum() + 1))
        b, _ = ref.allocate(ks, ln, B)
        assert b.sum() == B and np.all(b <= ln) and np.all(b >= 0)


# --------------------------------------------------------------------------
# byte accounting and budgets (IndexMem section 1; the workloads' budgets)
# --------------------------------------------------------------------------
def test_closed_forms():
    g = json.load(open(os.path.join(GOLDEN, "closed_forms.json")))
    s = g["kv_bytes_70b_1m_tokens_bf16"]["shape"]
    assert ref.kv_cache_bytes(s["layers"], s["kv_heads"], s["head_dim"], s["tokens"], s["elt_bytes"]) \
        == g["kv_bytes_70b_1m_tokens_bf16"]["value"] == 320 * 2 ** 30
    assert synth.WORKLOADS["llama8b_32k"].budget() == g["budget_8b_32k"]["value"]
    assert synth.WORKLOADS["batched16_16k"].budget() == g["budget_batched_16k"]["value"]
    w = synth.WORKLOADS["qwen8b_128k"]
    assert int(math.floor(Fraction(1, 20) * w.n_heads * w.ctx + Fraction(1, 2))) == g["budget_128k_5pct"]["value"]
    assert synth.WORKLOADS["tiny"].budget() == 256
