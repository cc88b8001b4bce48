"""GPU parity: every C-ABI call against the CPU oracle on the same seeded
inputs.  Integer and selection results must match bit for bit; attention
outputs within 2e-3 max-abs and dropped mass within 1e-5 of the float64
oracle on the bf16-rounded inputs."""
import dataclasses
import math
import os

import numpy as np
import pytest
import torch

import synth
from oracle import reference as ref
from retention_scored_decode_amd import trimkv as tk
from gpu_helpers import (DROP_TOL, OUT_TOL, OracleView, cuda, download_cache, dst_capacity, f32_bits,
                         heads_from_plane, kv_dev, plane_from_heads, scale_of, seg_t, upload)

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
SMALL = {
    "tiny": W["tiny"],
    "c2s": W["llama8b_32k"].scaled(layers=2, ctx=3001),
    "c3s": W["batched16_16k"].scaled(batch=3, layers=2, ctx=1500),
    "c5s": W["stream_gqa7"].scaled(layers=2, ctx=2000, budget_abs=1024, steps=8,
                                   beta_block=(600, 1200, ("mix", 0.5, (1.0, 20.0), (40.0, 1.0)))),
}


def announce(*a):
    print("[case]", *a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    tk.lib()


# --------------------------------------------------------------------------
# a0: ln beta
# --------------------------------------------------------------------------
def test_log_beta_specials_and_hard_cases():
    from test_oracle_pins import HARD_LN_INPUTS
    rng = np.random.default_rng(1)
    x = np.concatenate([
        np.array([0.0, 1.0, 2 ** -149, 2 ** -126, 0.5, 1 - 2 ** -24], np.float32),
        np.array(HARD_LN_INPUTS, np.uint32).view(np.float32),
        rng.integers(0, 0x3F800001, 1 << 20, dtype=np.uint32).view(np.float32),
        rng.beta(50, 1, 1 << 16).astype(np.float32),
    ])
    announce("log_beta", x.size)
    out = torch.empty(x.size, dtype=torch.float32, device="cuda")
    tk.log_beta(cuda(x), out)
    got = out.cpu().numpy()
    assert np.array_equal(f32_bits(got), f32_bits(ref.ln_beta(x)))
    # strided output (the ln beta half of metadata blocks); the other half untouched
    n = (x.size // 16) * 16
    meta = torch.full((n // 16, 2, 16), 7, dtype=torch.int32, device="cuda")
    tk.log_beta(cuda(x[:n]), meta, out_page_stride=32)
    mh = meta.cpu().numpy()
    assert np.array_equal(mh[:, 0, :].reshape(-1).view(np.uint32), f32_bits(ref.ln_beta(x[:n])))
    assert np.all(mh[:, 1, :] == 7)


EXH_CHUNK = 1 << 26


@pytest.mark.slow
@pytest.mark.skipif(os.environ.get("TRIMKV_EXHAUSTIVE") != "1", reason="opt-in: TRIMKV_EXHAUSTIVE=1 (every fp32 in [0, 1]: about 20 s on an MI355X with a 16-core host)")
@pytest.mark.parametrize("lo", list(range(0, 0x3F800001, EXH_CHUNK)))
def test_log_beta_exhaustive_unit_interval(lo):
    """Every float32 in [0, 1]: the GPU's ln beta is the correctly rounded one."""
    hi = min(lo + EXH_CHUNK, 0x3F800001)
    announce("log_beta exhaustive", hex(lo))
    x = torch.arange(lo, hi, dtype=torch.int64, device="cuda").to(torch.int32).view(torch.float32)
    out = torch.empty(hi - lo, dtype=torch.float32, device="cuda")
    tk.log_beta(x, out)
    got = out.cpu().numpy()
    want = ref.ln_beta(x.cpu().numpy())
    bad = np.flatnonzero(f32_bits(got) != f32_bits(want))
    assert bad.size == 0, [hex(lo + int(i)) for i in bad[:10]]


# --------------------------------------------------------------------------
# a1: scores
# --------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["tiny", "c2s", "c3s", "c5s"])
def test_score_parity(name):
    w = SMALL[name]
    announce("score", name)
    pc = synth.build_cache(w)
    c = upload(pc)
    ov = OracleView(pc)
    seg = w.seg_head_begin()
    t_seg = np.array([w.t + 1 + 7 * s for s in range(w.n_seg)], np.int32)
    out = torch.full((pc.n_pages * 16,), 123.0, dtype=torch.float32, device="cuda")
    tk.score(c, cuda(seg, np.int32), cuda(t_seg), out)
    plane = out.cpu().numpy()
    t_h = seg_t(seg, t_seg, pc.n_heads)
    got = heads_from_plane(plane, pc.page_off, pc.length)
    want = ov.scores(t_h)
    for h in range(pc.n_heads):
        assert np.array_equal(f32_bits(got[h]), f32_bits(want[h])), h
        s64 = ref.score_f64(ref.gather_heads(pc.beta, pc.page_off, pc.page_ids, pc.length)[h], t_h[h], ov.pos[h])
        fin = np.isfinite(s64) & (s64 != 0)
        assert np.all(np.abs(got[h][fin] - s64[fin]) <= 1e-6 * np.abs(s64[fin]))
    # padding slots of used pages hold NaN
    total = int(pc.page_off[-1]) * 16
    valid = np.zeros(total, bool)
    for h in range(pc.n_heads):
        valid[ref.head_csr_slots(pc.page_off, pc.length, h)] = True
    assert np.all(np.isnan(plane[:total][~valid]))


def pad_pool(c: tk.Cache, extra_pages: int) -> tk.Cache:
    """The same cache in a pool with extra_pages more (unused) pages."""
    P, N = c.n_pages, c.n_pages + extra_pages

    def grow(x):
        y = torch.zeros((N,) + tuple(x.shape[1:]), dtype=x.dtype, device=x.device)
        y[:P] = x
        return y
    return tk.Cache(grow(c.k), grow(c.v), grow(c.meta), c.page_off, grow(c.page_ids), c.length)


def _score_select_case(pc, seg, t_seg, budgets, extra_pages=0):
    """trimkv_score_select against trimkv_score then trimkv_select_global on
    the same cache (score plane, keep plane, kept counts and kept sums bit
    for bit), and both against the oracle."""
    c = upload(pc)
    if extra_pages:
        c = pad_pool(c, extra_pages)
    ov = OracleView(pc)
    n = c.n_pages * 16
    seg_d, t_d, b_d = cuda(seg, np.int32), cuda(np.asarray(t_seg, np.int32)), cuda(np.asarray(budgets), np.int64)
    s1 = torch.full((n,), 123.0, dtype=torch.float32, device="cuda")
    s2 = torch.full((n,), 321.0, dtype=torch.float32, device="cuda")
    k1 = torch.full((n,), 7, dtype=torch.uint8, device="cuda")
    k2 = torch.full((n,), 9, dtype=torch.uint8, device="cuda")
    kept1 = torch.full((pc.n_heads,), -1, dtype=torch.int32, device="cuda")
    kept2 = torch.full((pc.n_heads,), -2, dtype=torch.int32, device="cuda")
    ks1 = torch.empty(pc.n_heads, dtype=torch.float64, device="cuda")
    ks2 = torch.empty(pc.n_heads, dtype=torch.float64, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    tk.score(c, seg_d, t_d, s1)
    tk.select_global(c, s1, seg_d, b_d, k1, kept1, ks1, status=status)
    tk.score_select(c, seg_d, t_d, b_d, s2, k2, kept2, ks2, status=status)
    total = int(pc.page_off[-1]) * 16
    assert np.array_equal(f32_bits(s1.cpu().numpy()[:total]), f32_bits(s2.cpu().numpy()[:total]))
    assert np.array_equal(k1.cpu().numpy()[:total], k2.cpu().numpy()[:total])
    assert np.array_equal(kept1.cpu().numpy(), kept2.cpu().numpy())
    assert np.array_equal(ks1.cpu().numpy().view(np.uint64), ks2.cpu().numpy().view(np.uint64))
    assert int(status.item()) == 0
    want_keep, want_kept = ref.select_global(ov.scores(seg_t(seg, t_seg, pc.n_heads)), seg, budgets)
    got = heads_from_plane(k2.cpu().numpy(), pc.page_off, pc.length)
    for h in range(pc.n_heads):
        assert np.array_equal(got[h].astype(bool), want_keep[h]), h
    assert np.array_equal(kept2.cpu().numpy(), want_kept)


@pytest.mark.parametrize("name", ["tiny", "c2s", "c3s", "c5s"])
def test_score_select_parity(name):
    w = SMALL[name]
    announce("score_select", name)
    pc = synth.build_cache(w)
    seg = w.seg_head_begin()
    t_seg = [w.t + 1 + 5 * s for s in range(w.n_seg)]
    _score_select_case(pc, seg, t_seg, [w.budget()] * w.n_seg)


def test_score_select_ties_and_ragged():
    """beta = 1 (every score 0: a budget below N fills heads in order, each
    keeping its most recent entries), beta = 0 (-inf), and ragged heads with
    segments ending inside 32-chunk blocks."""
    for seed, dist in ((31, ("beta", 5.0, 1.0)), (32, ("const", 1.0)), (33, ("const", 0.0)),
                       (34, ("const", 0.5))):
        pc = synth.random_ragged_cache(seed, n_heads=23, d=64, dtype="bf16", max_len=5000, beta_dist=dist)
        seg = np.array([0, 5, 17, 23], np.int32)
        N = [int(pc.length[seg[s]:seg[s + 1]].sum()) for s in range(3)]
        t = int(pc.pos.max()) + 1
        for budgets in ([n // 3 for n in N], [0, 1, max(N[2] - 1, 0)], [n + 2 for n in N]):
            announce("score_select ragged", dist, budgets)
            _score_select_case(pc, seg, [t, t + 3, t + 9], budgets)


def empty_heads(pc, heads):
    """The same cache with the given heads emptied: no pages, length 0 (their
    physical pages stay in the pool, unused, at the end of the page list)."""
    po, ids = pc.page_off, pc.page_ids
    length = pc.length.copy()
    keep_ids, dropped, off = [], [], [0]
    for h in range(pc.n_heads):
        seg_ids = list(ids[po[h]:po[h + 1]])
        if h in heads:
            length[h] = 0
            dropped += seg_ids
        else:
            keep_ids += seg_ids
        off.append(len(keep_ids))
    rest = list(ids[po[-1]:])
    page_ids = np.array(keep_ids + dropped + rest, np.int32)
    return dataclasses.replace(pc, page_off=np.array(off, np.int32), page_ids=page_ids, length=length)


def test_score_select_ties_with_empty_heads():
    """A head without pages takes a tie ticket but has no chunk, so a segment
    can hold more heads than chunks: segments whose ties straddle the budget,
    with empty heads at their start, inside them and at their end."""
    for seed, dist in ((51, ("const", 1.0)), (52, ("const", 0.5)), (53, ("beta", 5.0, 1.0))):
        pc = synth.random_ragged_cache(seed, n_heads=23, d=64, dtype="bf16", max_len=3000, min_len=40,
                                       beta_dist=dist)
        pc = empty_heads(pc, {1, 2, 3, 6, 8, 10, 11, 12, 13, 14, 18, 22})
        seg = np.array([0, 8, 16, 23], np.int32)
        N = [int(pc.length[seg[s]:seg[s + 1]].sum()) for s in range(3)]
        t = int(pc.pos.max()) + 1
        for budgets in ([n // 3 for n in N], [n // 2 + 1 for n in N], [1, max(N[1] - 1, 0), N[2]]):
            announce("score_select empty heads", dist, budgets)
            _score_select_case(pc, seg, [t, t + 3, t + 9], budgets)


@pytest.mark.parametrize("chunks", [0, 1500, 3000, 4200])
def test_score_select_block_sizes(chunks):
    """The selection takes 4, 8, 16 or 32 chunks of 64 pages per block by the
    pool's capacity (about n_pages / 64 + heads chunks): the same ragged
    caches in pools of growing capacity (extra pages unused) give the same
    outputs, equal to the oracle's, with ties below and straddling the
    budget."""
    for seed, dist in ((41, ("beta", 5.0, 1.0)), (42, ("const", 1.0))):
        pc = synth.random_ragged_cache(seed, n_heads=23, d=64, dtype="bf16", max_len=5000, beta_dist=dist)
        seg = np.array([0, 5, 17, 23], np.int32)
        N = [int(pc.length[seg[s]:seg[s + 1]].sum()) for s in range(3)]
        t = int(pc.pos.max()) + 1
        extra = max(chunks * 64 - pc.n_pages, 0)
        announce("score_select block size", chunks, dist, extra)
        for budgets in ([n // 3 for n in N], [1, max(N[1] - 7, 0), N[2] + 1]):
            _score_select_case(pc, seg, [t, t + 3, t + 9], budgets, extra_pages=extra)


# --------------------------------------------------------------------------
# a2: selection on identical fp32 scores
# --------------------------------------------------------------------------
def run_select(c, plane, seg, budgets, keptsum=False):
    n_seg = len(seg) - 1
    keep = torch.full((c.n_pages * 16,), 7, dtype=torch.uint8, device="cuda")
    kept = torch.full((c.n_heads,), -1, dtype=torch.int32, device="cuda")
    ks = torch.full((c.n_heads,), np.nan, dtype=torch.float64, device="cuda") if keptsum else None
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    tk.select_global(c, cuda(plane, np.float32), cuda(seg, np.int32), cuda(np.asarray(budgets), np.int64),
                     keep, kept, ks, status=status)
    assert int(status.item()) == 0, "a tie-rank wait timed out"
    return keep.cpu().numpy(), kept.cpu().numpy(), (ks.cpu().numpy() if keptsum else None)


def check_select(pc, per_head_scores, seg, budgets, keptsum=True):
    c = upload(pc)
    plane = plane_from_heads(per_head_scores, pc.page_off, pc.length, pc.n_pages)
    keep, kept, ks = run_select(c, plane, seg, budgets, keptsum)
    want_keep, want_kept = ref.select_global(per_head_scores, seg, budgets)
    got = heads_from_plane(keep, pc.page_off, pc.length)
    for h in range(pc.n_heads):
        assert np.array_equal(got[h].astype(bool), want_keep[h]), ("head", h)
        assert np.all((got[h] == 0) | (got[h] == 1))
    assert np.array_equal(kept, want_kept)
    # padding slots of used pages are 0
    total = int(pc.page_off[-1]) * 16
    valid = np.zeros(total, bool)
    for h in range(pc.n_heads):
        valid[ref.head_csr_slots(pc.page_off, pc.length, h)] = True
    assert np.all(keep[:total][~valid] == 0)
    if keptsum:
        for h in range(pc.n_heads):
            want = float(np.sum(per_head_scores[h][want_keep[h]].astype(np.float64)))
            if np.isfinite(want):
                assert abs(ks[h] - want) <= 1e-12 * max(1.0, abs(want)), h
            else:   # inf or NaN sums (infinite or NaN scores kept)
                assert ks[h] == want or (np.isnan(want) and np.isnan(ks[h])), h
    return keep


@pytest.mark.parametrize("name", ["tiny", "c2s", "c3s", "c5s"])
def test_select_parity_workloads(name):
    w = SMALL[name]
    announce("select", name)
    pc = synth.build_cache(w)
    ov = OracleView(pc)
    seg = w.seg_head_begin()
    scores = ov.scores(seg_t(seg, [w.t] * w.n_seg, pc.n_heads))
    check_select(pc, scores, seg, [w.budget()] * w.n_seg)


KINDS = ["alpha3", "equal", "zeros", "inf", "cont", "nan", "ulps", "denorm"]


@pytest.mark.parametrize("kind", KINDS)
def test_select_parity_adversarial(kind):
    rng = np.random.default_rng(KINDS.index(kind))
    for trial in range(4):
        H = int(rng.integers(3, 12))
        pc = synth.random_ragged_cache(100 + trial, n_heads=H, d=64, dtype="bf16", max_len=2500)
        lens = pc.length
        if kind == "alpha3":
            sc = [rng.choice([-1.5, -0.25, 0.0], n).astype(np.float32) for n in lens]
        elif kind == "equal":
            sc = [np.full(n, -0.5, np.float32) for n in lens]
        elif kind == "zeros":
            sc = [rng.choice([0.0, -0.0], n).astype(np.float32) for n in lens]
        elif kind == "inf":
            sc = [np.where(rng.random(n) < 0.3, -np.inf, -rng.integers(0, 3, n)).astype(np.float32) for n in lens]
        elif kind == "nan":   # NaN ranks below every score, -inf included
            sc = [np.where(rng.random(n) < 0.2, np.nan,
                           rng.choice([-np.inf, -2.0, -0.0, 0.0, 1.5], n)).astype(np.float32) for n in lens]
        elif kind == "ulps":   # a few units in the last place apart: one bin until the last radix pass
            base = np.float32(-0.75).view(np.int32)
            sc = [(base + rng.integers(0, 24, n).astype(np.int32)).view(np.float32) for n in lens]
        elif kind == "denorm":   # subnormals of both signs beside zeros and the smallest normals
            pool = np.array([0.0, -0.0, 1e-45, -1e-45, 3e-39, -3e-39, 1.2e-38, -1.2e-38, 1e-40, -1e-40],
                            np.float32)
            sc = [rng.choice(pool, n) for n in lens]
        else:
            sc = [(-rng.random(n) * 50).astype(np.float32) for n in lens]
        n_seg = int(rng.integers(1, 4))
        cuts = sorted(rng.choice(np.arange(1, H), size=n_seg - 1, replace=False).tolist()) if n_seg > 1 else []
        seg = np.array([0] + cuts + [H], np.int32)
        N = [int(lens[seg[s]:seg[s + 1]].sum()) for s in range(n_seg)]
        for budgets in ([0] * n_seg, [1] * n_seg, [max(n - 1, 0) for n in N], N, [n + 5 for n in N],
                        [int(rng.integers(0, n + 1)) for n in N]):
            announce("select adversarial", kind, trial, budgets)
            check_select(pc, sc, seg, budgets)


@pytest.mark.parametrize("kind", ["alpha3", "equal"])
def test_select_ranked_many_lists(kind):
    """Ties straddling the budget in segments that span many 32-chunk blocks,
    so the ties are ranked across candidate lists by the in-order look-back;
    segment boundaries fall inside blocks."""
    rng = np.random.default_rng(7 + ["alpha3", "equal"].index(kind))
    H = 40
    pc = synth.random_ragged_cache(900, n_heads=H, d=64, dtype="bf16", max_len=20000, min_len=6000)
    lens = pc.length
    if kind == "alpha3":
        sc = [rng.choice([-1.5, -0.25, 0.0], n).astype(np.float32) for n in lens]
    else:
        sc = [np.full(n, -0.5, np.float32) for n in lens]
    seg = np.array([0, 7, 23, H], np.int32)
    N = [int(lens[seg[s]:seg[s + 1]].sum()) for s in range(3)]
    for budgets in ([n // 3 for n in N], [int(rng.integers(1, n)) for n in N]):
        announce("select ranked", kind, budgets)
        check_select(pc, sc, seg, budgets)


# --------------------------------------------------------------------------
# a3: compaction
# --------------------------------------------------------------------------
def check_compact(pc, keep_heads, reserve, given_counts=False):
    """given_counts: pass the per-head kept counts (as selection writes them)
    instead of letting compaction count the keep plane."""
    c = upload(pc)
    ov = OracleView(pc)
    kept_total = int(sum(int(k.sum()) for k in keep_heads))
    cap = dst_capacity(pc.n_heads, kept_total, reserve)
    kd = c.k.dtype
    dst = tk.Cache.empty(pc.n_heads, cap, pc.head_dim, kd)
    keep_plane = plane_from_heads([k.astype(np.uint8) for k in keep_heads], pc.page_off, pc.length, pc.n_pages,
                                  fill=0, dtype=np.uint8)
    used = torch.zeros(1, dtype=torch.int64, device="cuda")
    counts = cuda(np.array([int(k.sum()) for k in keep_heads], np.int32)) if given_counts else None
    tk.compact(c, cuda(keep_plane), reserve, kept_total, dst, used, kept=counts)
    po, pi, ln, k, v, lnb, pos = download_cache(dst)
    wpo, wpi, wlen, rows = ref.compact({"k": ov.k_raw, "v": ov.v_raw, "lnb": ov.lnb, "pos": ov.pos}, keep_heads,
                                       reserve)
    assert np.array_equal(po, wpo) and np.array_equal(ln, wlen)
    assert int(used.item()) == int(wpo[-1])
    assert np.array_equal(pi[:int(wpo[-1])], wpi)
    for h in range(pc.n_heads):
        gk = ref.gather_heads(k, po, pi, ln)[h]
        gv = ref.gather_heads(v, po, pi, ln)[h]
        gl = ref.gather_heads(lnb, po, pi, ln)[h]
        gp = ref.gather_heads(pos, po, pi, ln)[h]
        assert np.array_equal(gk, rows["k"][h]) and np.array_equal(gv, rows["v"][h]), h
        assert np.array_equal(f32_bits(gl), f32_bits(rows["lnb"][h])) and np.array_equal(gp, rows["pos"][h]), h
    return dst


@pytest.mark.parametrize("name", ["tiny", "c2s", "c3s", "c5s"])
def test_compact_parity_workloads(name):
    w = SMALL[name]
    announce("compact", name)
    pc = synth.build_cache(w)
    ov = OracleView(pc)
    seg = w.seg_head_begin()
    scores = ov.scores(seg_t(seg, [w.t] * w.n_seg, pc.n_heads))
    keep, _ = ref.select_global(scores, seg, [w.budget()] * w.n_seg)
    check_compact(pc, keep, reserve=w.reserve)
    check_compact(pc, keep, reserve=w.reserve, given_counts=True)


def test_compact_ragged_edges():
    rng = np.random.default_rng(5)
    for trial, (dtype, d) in enumerate([("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)]):
        pc = synth.random_ragged_cache(200 + trial, n_heads=9, d=d, dtype=dtype, max_len=1100)
        for p_keep in (0.0, 0.05, 0.5, 1.0):
            keep = [rng.random(int(n)) < p_keep for n in pc.length]
            for reserve in (0, 1, 17):
                announce("compact ragged", dtype, d, p_keep, reserve)
                check_compact(pc, keep, reserve, given_counts=reserve == 1)


def test_compact_counts_that_disagree_with_keep():
    """Per-head counts above or below the keep plane's nonzero bytes: the
    layout is unspecified, but every access stays inside the pools (pairs
    the counts reserve and the keep plane does not fill copy nothing), the
    page table is the prefix sum of the given counts, and the heads before
    the first wrong count are compacted exactly."""
    rng = np.random.default_rng(55)
    pc = synth.random_ragged_cache(321, n_heads=8, d=128, dtype="bf16", max_len=900, min_len=100)
    keep = [rng.random(int(n)) < 0.4 for n in pc.length]
    true = np.array([int(k.sum()) for k in keep], np.int64)
    for delta in ([0, 0, 0, 5, 0, 0, 0, 0], [0, 0, 0, 0, -7, 0, 9, 0], [0, 3, 0, 0, 0, 0, 0, 11]):
        counts = np.maximum(true + np.array(delta), 0)
        announce("compact mismatched counts", delta)
        c = upload(pc)
        total = int(max(counts.sum(), true.sum()))
        cap = dst_capacity(pc.n_heads, total, 1)
        dst = tk.Cache.empty(pc.n_heads, cap, pc.head_dim, c.k.dtype)
        keep_plane = plane_from_heads([k.astype(np.uint8) for k in keep], pc.page_off, pc.length, pc.n_pages,
                                      fill=0, dtype=np.uint8)
        used = torch.zeros(1, dtype=torch.int64, device="cuda")
        tk.compact(c, cuda(keep_plane), 1, total, dst, used, kept=cuda(counts.astype(np.int32)))
        torch.cuda.synchronize()
        po, pi, ln, k, v, lnb, pos = download_cache(dst)
        wpo, _, wln = ref.compact_layout(counts, 1)
        assert np.array_equal(po, wpo) and np.array_equal(ln, wln)
        ov = OracleView(pc)
        first_bad = int(np.flatnonzero(np.array(delta) != 0)[0])
        for h in range(first_bad):
            assert np.array_equal(ref.gather_heads(k, po, pi, ln)[h], ov.k_raw[h][keep[h]]), h
            assert np.array_equal(ref.gather_heads(pos, po, pi, ln)[h], ov.pos[h][keep[h]]), h


def test_append_reports_heads_without_a_free_slot():
    """trimkv_append into a cache whose heads are partly full: every full
    head is left unchanged and counted in the status word (which the call
    only increments); every other head receives the entry."""
    pc = synth.random_ragged_cache(77, n_heads=6, d=64, dtype="bf16", max_len=70, min_len=40)
    rng = np.random.default_rng(77)
    keep = [np.ones(int(n), bool) for n in pc.length]
    # compact without spare slots, so heads whose kept count is a multiple of 16 are full
    for h in (1, 4):
        keep[h][:] = False
        keep[h][:32] = True
    c = upload(pc)
    cap = dst_capacity(pc.n_heads, int(pc.length.sum()), 0)
    dst = tk.Cache.empty(pc.n_heads, cap, pc.head_dim, c.k.dtype)
    keep_plane = plane_from_heads([k.astype(np.uint8) for k in keep], pc.page_off, pc.length, pc.n_pages,
                                  fill=0, dtype=np.uint8)
    used = torch.zeros(1, dtype=torch.int64, device="cuda")
    tk.compact(c, cuda(keep_plane), 0, int(pc.length.sum()), dst, used)
    len0 = dst.length.cpu().numpy().copy()
    full = (len0 % 16 == 0)
    assert full[1] and full[4]
    status = torch.full((1,), 5, dtype=torch.int32, device="cuda")
    t = int(pc.pos.max()) + 2
    kn = synth.f64_to_bf16_bits(rng.standard_normal((pc.n_heads, 64)))
    for rep in range(2):
        tk.append(dst, kv_dev(kn, "bf16"), kv_dev(kn, "bf16"), cuda(np.full(pc.n_heads, 0.5, np.float32)),
                  cuda(np.array([t + rep], np.int32)), status=status)
    torch.cuda.synchronize()
    n_full = int(full.sum())
    # second call: heads that had one free slot are full after the first append
    one_free = (len0 % 16 == 15)
    assert int(status.item()) == 5 + 2 * n_full + int(one_free.sum())
    ln = dst.length.cpu().numpy()
    want = len0 + np.where(full, 0, np.where(one_free, 1, 2))
    assert np.array_equal(ln, want)


# --------------------------------------------------------------------------
# a4: decode attention
# --------------------------------------------------------------------------
def run_attn(c, q_dev, group, scale, keep_plane=None, lse_ref=None):
    nq = c.n_heads * group
    out = torch.full((nq, c.head_dim), np.nan, dtype=torch.float32, device="cuda")
    dropped = torch.full((nq,), np.nan, dtype=torch.float32, device="cuda")
    lse = torch.full((nq,), np.nan, dtype=torch.float32, device="cuda")
    tk.decode_attn(c, q_dev, group, scale, out, dropped,
                   keep=None if keep_plane is None else cuda(keep_plane),
                   lse_ref=None if lse_ref is None else cuda(lse_ref, np.float32), lse_out=lse)
    return out.cpu().numpy(), dropped.cpu().numpy(), lse.cpu().numpy()


def make_q(rng, nq, d, dtype, scale=1.0):
    x = rng.standard_normal((nq, d)) * scale
    bits = synth.f64_to_bf16_bits(x) if dtype == "bf16" else x.astype(np.float32)
    f64 = (synth.bf16_bits_to_f32(bits) if dtype == "bf16" else bits).astype(np.float64)
    return kv_dev(bits, dtype), f64


def check_attn(got, want):
    out, dropped, lse = got
    wout, wdrop, wlse = want
    assert np.max(np.abs(out - wout)) <= OUT_TOL, np.max(np.abs(out - wout))
    assert np.max(np.abs(dropped - wdrop)) <= DROP_TOL, np.max(np.abs(dropped - wdrop))
    fin = np.isfinite(wlse)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.all(np.abs(lse[fin] - wlse[fin]) <= 1e-4 * np.maximum(1, np.abs(wlse[fin])))


@pytest.mark.parametrize("dtype,d,group,long", [("bf16", 128, 4, False), ("bf16", 128, 7, False),
                                                ("bf16", 128, 1, False), ("bf16", 128, 2, False),
                                                ("bf16", 128, 8, False), ("bf16", 128, 16, False),
                                                ("bf16", 64, 4, False), ("bf16", 64, 3, False),
                                                ("f32", 64, 1, False), ("f32", 128, 2, False),
                                                ("bf16", 64, 4, True), ("bf16", 128, 16, True), ("bf16", 128, 1, True),
                                                ("bf16", 128, 7, True)])
def test_attention_modes(dtype, d, group, long):
    """Plain, mask and reference modes against the float64 oracle.  Long
    cases (7 heads of 12K-16K entries) give every wave several pages, so the
    load pipeline runs in its steady state."""
    rng = np.random.default_rng(d * 100 + group + long)
    if long:
        pc = synth.random_ragged_cache(330 + group, n_heads=7, d=d, dtype=dtype, max_len=16384, min_len=12000)
    else:
        pc = synth.random_ragged_cache(300 + group, n_heads=7, d=d, dtype=dtype, max_len=700)
    # force edge lengths: empty, one entry, one page, page + 1
    ov = OracleView(pc)
    q_dev, q64 = make_q(rng, pc.n_heads * group, d, dtype, scale=1.5)
    c = upload(pc)
    sc = scale_of(d)
    announce("attn plain", dtype, d, group)
    check_attn(run_attn(c, q_dev, group, sc), ref.decode_attn(ov.k, ov.v, q64, group, sc))
    keep = [rng.random(int(n)) < 0.3 for n in pc.length]
    keep[0][:] = False
    plane = plane_from_heads([k.astype(np.uint8) for k in keep], pc.page_off, pc.length, pc.n_pages, 0, np.uint8)
    announce("attn mask", dtype, d, group)
    check_attn(run_attn(c, q_dev, group, sc, keep_plane=plane),
               ref.decode_attn(ov.k, ov.v, q64, group, sc, keep=keep))
    _, _, lse_full = ref.decode_attn(ov.k, ov.v, q64, group, sc)
    kc = check_compact(pc, keep, 0)
    kk = [k[m] for k, m in zip(ov.k, keep)]
    vv = [v[m] for v, m in zip(ov.v, keep)]
    announce("attn ref", dtype, d, group)
    check_attn(run_attn(kc, q_dev, group, sc, lse_ref=lse_full.astype(np.float32)),
               ref.decode_attn(kk, vv, q64, group, sc, lse_ref=lse_full.astype(np.float32).astype(np.float64)))


@pytest.mark.parametrize("d,group,long", [(128, 4, False), (128, 7, False), (128, 1, False), (128, 16, False),
                                           (64, 4, False), (64, 3, False), (128, 4, True)])
def test_gated_attention(d, group, long):
    """Retention-gated decode attention (TRIM-KV section 2, attention
    modulation, at decode time): weights e^{z_j} r_j renormalised, plain and
    mask modes, against the float64 oracle given the float32 scores as ln r.
    Two segments with their own t; beta = 0 and 1 sprinkled in; head 0 has
    beta = 0 everywhere (no weight: out 0, dropped 1), head 1 beta = 0 on its
    first 40 entries (whole pages of -inf gates before any finite logit).
    The long case (9 heads of 12K-16K entries) gives every wave of the launch
    several pages, so the two-page load pipeline runs in its steady state."""
    rng = np.random.default_rng(900 + d + group + long)
    if long:
        pc = synth.random_ragged_cache(960, n_heads=9, d=d, dtype="bf16", max_len=16384, min_len=12000, t=17000,
                                       beta_dist=("beta", 200.0, 1.0))
    else:
        pc = synth.random_ragged_cache(950 + group, n_heads=9, d=d, dtype="bf16", max_len=900, min_len=60, t=1000,
                                       beta_dist=("beta", 20.0, 1.0))
    pc.length[5] = 0   # an empty head
    beta = pc.beta.reshape(-1)
    for h in range(pc.n_heads):
        sl = ref.head_phys_slots(pc.page_off, pc.page_ids, pc.length, h)
        beta[sl[rng.random(len(sl)) < 0.05]] = 0.0
        beta[sl[rng.random(len(sl)) < 0.05]] = 1.0
        if h == 0:
            beta[sl] = 0.0
        if h == 1:
            beta[sl[:40]] = 0.0
            beta[sl[40:]] = 1.0
    ov = OracleView(pc)
    seg = np.array([0, 4, pc.n_heads], np.int32)
    t_seg = np.array([17000, 17003] if long else [1000, 1003], np.int32)
    t_h = seg_t(seg, t_seg, pc.n_heads)
    gate = [g.astype(np.float64) for g in ov.scores(t_h)]
    q_dev, q64 = make_q(rng, pc.n_heads * group, d, "bf16", scale=1.5)
    c = upload(pc)
    sc = scale_of(d)
    nq = pc.n_heads * group
    keep = [rng.random(int(n)) < 0.3 for n in pc.length]
    plane = plane_from_heads([k.astype(np.uint8) for k in keep], pc.page_off, pc.length, pc.n_pages, 0, np.uint8)
    for kp in (None, keep):
        out = torch.full((nq, d), np.nan, dtype=torch.float32, device="cuda")
        dropped = torch.full((nq,), np.nan, dtype=torch.float32, device="cuda")
        lse = torch.full((nq,), np.nan, dtype=torch.float32, device="cuda")
        announce("attn gated", d, group, "mask" if kp is not None else "plain", "lengths", pc.length.tolist())
        tk.decode_attn_gated(c, cuda(seg), cuda(t_seg), q_dev, group, sc, out, dropped,
                             keep=None if kp is None else cuda(plane), lse_out=lse)
        got = tuple(x.cpu().numpy() for x in (out, dropped, lse))
        want = ref.decode_attn_gated(ov.k, ov.v, q64, group, sc, gate, keep=kp)
        check_attn(got, want)
        assert np.all(got[0][:group] == 0) and np.all(got[1][:group] == 1)


@pytest.mark.parametrize("d,group,long", [(128, 4, False), (128, 7, False), (128, 1, False), (128, 16, False),
                                           (64, 4, False), (128, 4, True)])
def test_attention_error_output(d, group, long):
    """e_s(A) = ||mu - m_A||_2 (ContourKV section 1) beside the mask-mode
    outputs.  mu and m_A are checked element-wise against the float64
    oracle (2e-3); the norm against the oracle's within the bound those
    imply, 2 * sqrt(D) * 2e-3, and against the norm of the GPU's own mu and
    m_A within fp32 rounding.  Heads with an empty kept set and a fully
    kept set are included, and (D = 128, G = 4) heads of 0, 1, 16 and 17
    entries.  The long case (9 heads of 12K-16K entries) runs the load
    pipeline in its steady state (several pages per wave)."""
    rng = np.random.default_rng(700 + d + group + long)
    if long:
        pc = synth.random_ragged_cache(870, n_heads=9, d=d, dtype="bf16", max_len=16384, min_len=12000)
    elif (d, group) == (128, 4):   # edge lengths: no entries, one, one page, a page and one
        w = W["llama8b_32k"].scaled(layers=1, ctx=900)
        pc = synth.build_cache(w, lengths=np.array([600, 300, 0, 1, 16, 17, 900, 5], np.int32))
    else:
        pc = synth.random_ragged_cache(800 + group, n_heads=9, d=d, dtype="bf16", max_len=900)
    ov = OracleView(pc)
    q_dev, q64 = make_q(rng, pc.n_heads * group, d, "bf16", scale=1.5)
    c = upload(pc)
    sc = scale_of(d)
    keep = [rng.random(int(n)) < 0.3 for n in pc.length]
    keep[0][:] = False
    keep[1][:] = True
    plane = plane_from_heads([k.astype(np.uint8) for k in keep], pc.page_off, pc.length, pc.n_pages, 0, np.uint8)
    nq = pc.n_heads * group
    out = torch.full((nq, d), np.nan, dtype=torch.float32, device="cuda")
    mu = torch.full((nq, d), np.nan, dtype=torch.float32, device="cuda")
    dropped = torch.full((nq,), np.nan, dtype=torch.float32, device="cuda")
    err = torch.full((nq,), np.nan, dtype=torch.float32, device="cuda")
    announce("attn err", d, group, "lengths", pc.length.tolist())
    tk.decode_attn_err(c, q_dev, group, sc, cuda(plane), out, dropped, err, mu=mu)
    o, m, dr, e = (x.cpu().numpy() for x in (out, mu, dropped, err))
    wout, wdrop, _ = ref.decode_attn(ov.k, ov.v, q64, group, sc, keep=keep)
    wmu, _, _ = ref.decode_attn(ov.k, ov.v, q64, group, sc)
    werr = ref.subset_error(ov.k, ov.v, q64, group, sc, keep)
    assert np.max(np.abs(o - wout)) <= OUT_TOL
    assert np.max(np.abs(m - wmu)) <= OUT_TOL
    assert np.max(np.abs(dr - wdrop)) <= DROP_TOL
    assert np.all(np.abs(e - werr) <= 2 * math.sqrt(d) * OUT_TOL)
    own = np.sqrt(((m.astype(np.float64) - o.astype(np.float64)) ** 2).sum(axis=1))
    assert np.all(np.abs(e - own) <= 1e-5 * np.maximum(1.0, own))
    fully = np.arange(group, 2 * group)   # head 1 keeps everything
    assert np.all(e[fully] <= 1e-5)
    # the errorless mask mode gives the same kept-set outputs
    o2, d2, _ = run_attn(c, q_dev, group, sc, keep_plane=plane)
    assert np.max(np.abs(o2 - o)) <= 1e-6 and np.max(np.abs(d2 - dr)) <= 1e-7


def test_attention_edge_lengths_and_determinism():
    rng = np.random.default_rng(11)
    w = SMALL["c2s"].scaled(layers=1, kv_heads=6)
    lengths = np.array([0, 1, 16, 17, 255, 4097], np.int32)
    pc = synth.build_cache(w.scaled(ctx=4097), lengths=lengths)
    ov = OracleView(pc)
    q_dev, q64 = make_q(rng, pc.n_heads * 4, 128, "bf16")
    c = upload(pc)
    announce("attn edges")
    a = run_attn(c, q_dev, 4, scale_of(128))
    check_attn(a, ref.decode_attn(ov.k, ov.v, q64, 4, scale_of(128)))
    assert np.all(a[0][:4] == 0) and np.all(a[1][:4] == 1.0)      # empty head: out 0, dropped 1
    b = run_attn(c, q_dev, 4, scale_of(128))
    for x, y in zip(a, b):
        assert np.array_equal(f32_bits(x), f32_bits(y))           # run-to-run identical


@pytest.mark.parametrize("group", [4, 8, 9])
def test_attention_ranges_across_many_heads(group):
    """Wave ranges that cross many heads: 1,200 KV heads of 0-266 entries
    (about 10K pages, some five per wave on a 256-CU GPU), so that most
    waves take several head segments.  Some heads have no pages at all,
    some keep their pages with no entries, some hold one entry.  At each
    crossing the next segment's first pages, and for G <= 8 its query rows,
    are requested during the segment's last page; G = 9 loads the query at
    the segment's start instead.  Plain, mask and retention-gated (plain and
    mask) modes against the float64 oracle, and run-to-run identical."""
    rng = np.random.default_rng(1300 + group)
    pc = synth.random_ragged_cache(1300 + group, n_heads=1200, d=128, dtype="bf16", max_len=266)
    assert (np.diff(pc.page_off) == 0).any()   # heads without pages
    pc.length[::53] = 0                         # pages without entries
    pc.length[7::61] = np.minimum(pc.length[7::61], 1)
    ov = OracleView(pc)
    q_dev, q64 = make_q(rng, pc.n_heads * group, 128, "bf16", scale=1.5)
    c = upload(pc)
    sc = scale_of(128)
    keep = [rng.random(int(n)) < 0.4 for n in pc.length]
    plane = plane_from_heads([k.astype(np.uint8) for k in keep], pc.page_off, pc.length, pc.n_pages, 0, np.uint8)
    announce("attn many heads plain", group)
    a = run_attn(c, q_dev, group, sc)
    check_attn(a, ref.decode_attn(ov.k, ov.v, q64, group, sc))
    empty = np.repeat(pc.length == 0, group)
    assert np.all(a[0][empty] == 0) and np.all(a[1][empty] == 1.0)
    b = run_attn(c, q_dev, group, sc)
    for x, y in zip(a, b):
        assert np.array_equal(f32_bits(x), f32_bits(y))
    announce("attn many heads mask", group)
    check_attn(run_attn(c, q_dev, group, sc, keep_plane=plane),
               ref.decode_attn(ov.k, ov.v, q64, group, sc, keep=keep))
    t = int(pc.pos.max()) + 5
    seg = np.array([0, pc.n_heads], np.int32)
    t_seg = np.array([t], np.int32)
    gate = [g.astype(np.float64) for g in ov.scores(seg_t(seg, t_seg, pc.n_heads))]
    nq = pc.n_heads * group
    for kp in (None, keep):
        announce("attn many heads gated", group, "mask" if kp is not None else "plain")
        out = torch.full((nq, 128), np.nan, dtype=torch.float32, device="cuda")
        dropped = torch.full((nq,), np.nan, dtype=torch.float32, device="cuda")
        lse = torch.full((nq,), np.nan, dtype=torch.float32, device="cuda")
        tk.decode_attn_gated(c, cuda(seg), cuda(t_seg), q_dev, group, sc, out, dropped,
                             keep=None if kp is None else cuda(plane), lse_out=lse)
        check_attn(tuple(x.cpu().numpy() for x in (out, dropped, lse)),
                   ref.decode_attn_gated(ov.k, ov.v, q64, group, sc, gate, keep=kp))


@pytest.mark.parametrize("dtype,d,group", [("bf16", 128, 4), ("bf16", 64, 3), ("f32", 64, 2)])
def test_attention_extreme_logits(dtype, d, group):
    """Queries scaled by 40, so that logits spread over hundreds of units, and
    keep masks that keep each KV head's keys with the lowest 30% of logits
    for its first query head (a random 30% on the odd heads): the kept set
    lies far below the dropped keys (about 150 units for those query heads)
    and must still be renormalised over itself, its weights taken against
    its own maximum instead of underflowing against the dropped keys'.
    Plain and mask modes against the float64 oracle; the error mode's dense
    output on the bf16 cases."""
    rng = np.random.default_rng(1500 + d + group)
    pc = synth.random_ragged_cache(1500 + group, n_heads=9, d=d, dtype=dtype, max_len=900, min_len=40)
    ov = OracleView(pc)
    q_dev, q64 = make_q(rng, pc.n_heads * group, d, dtype, scale=40.0)
    c = upload(pc)
    sc = scale_of(d)
    keep = []
    for h, n in enumerate(pc.length):
        z = ov.k[h] @ q64[h * group]
        keep.append(z < np.quantile(z, 0.3) if h % 2 == 0 else rng.random(int(n)) < 0.3)
    plane = plane_from_heads([k.astype(np.uint8) for k in keep], pc.page_off, pc.length, pc.n_pages, 0, np.uint8)
    announce("attn extreme plain", dtype, d, group)
    check_attn(run_attn(c, q_dev, group, sc), ref.decode_attn(ov.k, ov.v, q64, group, sc))
    announce("attn extreme mask", dtype, d, group)
    got = run_attn(c, q_dev, group, sc, keep_plane=plane)
    want = ref.decode_attn(ov.k, ov.v, q64, group, sc, keep=keep)
    check_attn(got, want)
    if dtype == "bf16":
        nq = pc.n_heads * group
        out = torch.full((nq, d), np.nan, dtype=torch.float32, device="cuda")
        mu = torch.full((nq, d), np.nan, dtype=torch.float32, device="cuda")
        dropped = torch.full((nq,), np.nan, dtype=torch.float32, device="cuda")
        err = torch.full((nq,), np.nan, dtype=torch.float32, device="cuda")
        announce("attn extreme err", d, group)
        tk.decode_attn_err(c, q_dev, group, sc, cuda(plane), out, dropped, err, mu=mu)
        wmu, _, _ = ref.decode_attn(ov.k, ov.v, q64, group, sc)
        assert np.max(np.abs(out.cpu().numpy() - want[0])) <= OUT_TOL
        assert np.max(np.abs(mu.cpu().numpy() - wmu)) <= OUT_TOL
        assert np.max(np.abs(dropped.cpu().numpy() - want[1])) <= DROP_TOL


# --------------------------------------------------------------------------
# the eviction step end to end (a0 -> a1 -> a2 -> a4 mask -> a3 -> a4 plain)
# --------------------------------------------------------------------------
def eviction_step(pc, w, rng):
    c = upload(pc)
    seg = w.seg_head_begin()
    t_seg = np.full(w.n_seg, w.t, np.int32)
    H, G, D = pc.n_heads, w.group, w.head_dim
    score = torch.empty(pc.n_pages * 16, dtype=torch.float32, device="cuda")
    tk.score(c, cuda(seg, np.int32), cuda(t_seg), score)
    keep = torch.empty(pc.n_pages * 16, dtype=torch.uint8, device="cuda")
    kept = torch.empty(H, dtype=torch.int32, device="cuda")
    tk.select_global(c, score, cuda(seg, np.int32), cuda(np.full(w.n_seg, w.budget()), np.int64), keep, kept)
    q_dev, q64 = make_q(rng, H * G, D, w.dtype, w.q_scale)
    sc = scale_of(D)
    nq = H * G
    out_m = torch.empty((nq, D), dtype=torch.float32, device="cuda")
    drop_m = torch.empty(nq, dtype=torch.float32, device="cuda")
    tk.decode_attn(c, q_dev, G, sc, out_m, drop_m, keep=keep)
    max_kept = w.budget() * w.n_seg
    dst = tk.Cache.empty(H, dst_capacity(H, max_kept, w.reserve), D, c.k.dtype)
    used = torch.zeros(1, dtype=torch.int64, device="cuda")
    tk.compact(c, keep, w.reserve, max_kept, dst, used)
    out_p = torch.empty((nq, D), dtype=torch.float32, device="cuda")
    drop_p = torch.empty(nq, dtype=torch.float32, device="cuda")
    tk.decode_attn(dst, q_dev, G, sc, out_p, drop_p)
    return dict(keep=keep.cpu().numpy(), kept=kept.cpu().numpy(), out_m=out_m.cpu().numpy(),
                drop_m=drop_m.cpu().numpy(), out_p=out_p.cpu().numpy(), drop_p=drop_p.cpu().numpy(),
                dst=download_cache(dst), q64=q64)


@pytest.mark.parametrize("name", ["c2s", "c3s", "tiny"])
def test_eviction_step_pipeline(name):
    w = SMALL[name]
    announce("pipeline", name)
    pc = synth.build_cache(w)
    r = eviction_step(pc, w, np.random.default_rng(3))
    ov = OracleView(pc)
    seg = w.seg_head_begin()
    scores = ov.scores(seg_t(seg, [w.t] * w.n_seg, pc.n_heads))
    keep, kept = ref.select_global(scores, seg, [w.budget()] * w.n_seg)
    got_keep = heads_from_plane(r["keep"], pc.page_off, pc.length)
    for h in range(pc.n_heads):
        assert np.array_equal(got_keep[h].astype(bool), keep[h]), h
    assert np.array_equal(r["kept"], kept)
    sc = scale_of(w.head_dim)
    check_attn((r["out_m"], r["drop_m"], np.zeros(len(r["drop_m"]))),
               (*ref.decode_attn(ov.k, ov.v, r["q64"], w.group, sc, keep=keep)[:2], np.zeros(len(r["drop_m"]))))
    po, pi, ln, k, v, lnb, pos = r["dst"]
    wpo, _, wlen, rows = ref.compact({"k": ov.k_raw, "pos": ov.pos}, keep, w.reserve)
    assert np.array_equal(po, wpo) and np.array_equal(ln, wlen)
    for h in range(pc.n_heads):
        assert np.array_equal(ref.gather_heads(k, po, pi, ln)[h], rows["k"][h])
        assert np.array_equal(ref.gather_heads(pos, po, pi, ln)[h], rows["pos"][h])
    kk = [x[m] for x, m in zip(ov.k, keep)]
    vv = [x[m] for x, m in zip(ov.v, keep)]
    wout, wdrop, _ = ref.decode_attn(kk, vv, r["q64"], w.group, sc)
    assert np.max(np.abs(r["out_p"] - wout)) <= OUT_TOL
    assert np.all(r["drop_p"][ln.repeat(w.group) > 0] == 0.0)
    # the renormalised output over the kept set is the same in both modes
    assert np.max(np.abs(r["out_p"] - r["out_m"])) <= OUT_TOL


# --------------------------------------------------------------------------
# a5/a6: attention mass, dropped-mass statistic, allocation
# --------------------------------------------------------------------------
def test_attention_mass_parity():
    w = W["qwen8b_128k"].scaled(layers=1, ctx=5000)
    pc = synth.build_cache(w)
    ov = OracleView(pc)
    q = synth.queries(w)
    q64 = synth.bf16_bits_to_f32(q).astype(np.float64)
    c = upload(pc)
    announce("mass")
    mass = torch.full((pc.n_pages * 16,), 5.0, dtype=torch.float32, device="cuda")
    lse = torch.empty(pc.n_heads * w.group, dtype=torch.float32, device="cuda")
    tk.attn_mass(c, kv_dev(q, "bf16"), w.group, scale_of(128), mass, lse)
    want_mass, want_lse = ref.attn_mass(ov.k, q64, w.group, scale_of(128))
    got = heads_from_plane(mass.cpu().numpy(), pc.page_off, pc.length)
    for h in range(pc.n_heads):
        assert np.all(np.abs(got[h] - want_mass[h]) <= 1e-5 * want_mass[h] + 1e-12), h
    assert np.max(np.abs(lse.cpu().numpy() - want_lse)) <= 1e-4


@pytest.mark.parametrize("d,group", [(128, 4), (128, 7), (64, 1), (128, 16)])
def test_attention_mass_long(d, group):
    """Attention mass and full LSE on long ragged heads (10 heads of 36K-48K
    entries, about 30K pages): every wave of the logits kernel streams
    several pages, two in flight, while storing each page's logits."""
    rng = np.random.default_rng(1200 + d + group)
    pc = synth.random_ragged_cache(1210 + group, n_heads=10, d=d, dtype="bf16", max_len=48000, min_len=36000)
    ov = OracleView(pc)
    q_dev, q64 = make_q(rng, pc.n_heads * group, d, "bf16", scale=2.0)
    c = upload(pc)
    announce("mass long", d, group)
    mass = torch.full((pc.n_pages * 16,), 5.0, dtype=torch.float32, device="cuda")
    lse = torch.empty(pc.n_heads * group, dtype=torch.float32, device="cuda")
    tk.attn_mass(c, q_dev, group, scale_of(d), mass, lse)
    want_mass, want_lse = ref.attn_mass(ov.k, q64, group, scale_of(d))
    got = heads_from_plane(mass.cpu().numpy(), pc.page_off, pc.length)
    for h in range(pc.n_heads):
        assert np.all(np.abs(got[h] - want_mass[h]) <= 1e-5 * want_mass[h] + 1e-12), h
    assert np.max(np.abs(lse.cpu().numpy() - want_lse)) <= 1e-4


def test_allocation_parity():
    rng = np.random.default_rng(12)
    for trial in range(30):
        H = int(rng.integers(1, 300))
        ks = rng.random(H) * (rng.random() < 0.9)
        if trial % 7 == 3:
            ks[:] = 1.0
        ln = rng.integers(0, 3000, H).astype(np.int32)
        B = int(rng.integers(0, int(ln.sum()) + 1)) if trial % 5 else int(ln.sum()) + 10
        announce("allocate", trial, H, B)
        b = torch.full((H,), -1, dtype=torch.int64, device="cuda")
        mb = torch.empty(H, dtype=torch.float64, device="cuda")
        tk.allocate(cuda(ks, np.float64), cuda(ln, np.int32), B, b, mb)
        wb, wm = ref.allocate(ks, ln, B)
        assert np.array_equal(b.cpu().numpy(), wb), trial
        assert np.array_equal(mb.cpu().numpy(), wm)


@pytest.mark.parametrize("kind", ["magnitudes", "small_alphabet", "many_heads"])
def test_allocation_adversarial(kind):
    """The allocation (ContourKV section 3) on inputs that stress its fp64
    arithmetic and its ranking: dropped masses spread over 600 decades, a
    three-value alphabet (exact ties in the fractional parts, broken by the
    lower head), and 4,096 heads (one block ranks them all)."""
    rng = np.random.default_rng({"magnitudes": 31, "small_alphabet": 32, "many_heads": 33}[kind])
    for trial in range(8):
        if kind == "magnitudes":
            H = int(rng.integers(2, 300))
            ks = 10.0 ** rng.uniform(-300, 300, H)
            ks[rng.random(H) < 0.1] = 0.0
        elif kind == "small_alphabet":
            H = int(rng.integers(2, 300))
            ks = rng.choice([1.0, 2.0, 3.0], H)
        else:
            H = 4096
            ks = rng.random(H)
        ln = rng.integers(0, 3000, H).astype(np.int32)
        B = int(rng.integers(0, int(ln.sum()) + 1)) if trial % 3 else int(ln.sum() // 2)
        announce("allocate adversarial", kind, trial, H, B)
        b = torch.full((H,), -1, dtype=torch.int64, device="cuda")
        mb = torch.empty(H, dtype=torch.float64, device="cuda")
        tk.allocate(cuda(ks, np.float64), cuda(ln, np.int32), B, b, mb)
        wb, wm = ref.allocate(ks, ln, B)
        assert np.array_equal(b.cpu().numpy(), wb), trial
        assert np.array_equal(mb.cpu().numpy(), wm)


def test_dropped_mass_budget_pipeline():
    """Top-s mass per head -> dropped mass -> budget -> per-head top-b ->
    compaction -> attention against the full-cache reference LSE."""
    w = W["qwen8b_128k"].scaled(layers=1, ctx=6000, mass_topk=256)
    pc = synth.build_cache(w)
    ov = OracleView(pc)
    H, G = pc.n_heads, w.group
    q = synth.queries(w)
    q64 = synth.bf16_bits_to_f32(q).astype(np.float64)
    c = upload(pc)
    sc = scale_of(128)
    announce("dropped-mass pipeline")
    mass = torch.empty(pc.n_pages * 16, dtype=torch.float32, device="cuda")
    lse = torch.empty(H * G, dtype=torch.float32, device="cuda")
    q_dev = kv_dev(q, "bf16")
    tk.attn_mass(c, q_dev, G, sc, mass, lse)
    seg = np.arange(H + 1, dtype=np.int32)
    keep = torch.empty(pc.n_pages * 16, dtype=torch.uint8, device="cuda")
    kept = torch.empty(H, dtype=torch.int32, device="cuda")
    ks = torch.empty(H, dtype=torch.float64, device="cuda")
    tk.select_global(c, mass, cuda(seg), cuda(np.full(H, w.mass_topk), np.int64), keep, kept, ks)
    B = w.budget()
    b = torch.empty(H, dtype=torch.int64, device="cuda")
    tk.allocate(ks, c.length, B, b)
    tk.select_global(c, mass, cuda(seg), b, keep, kept)
    bh = b.cpu().numpy()
    assert bh.sum() == B and np.all(bh <= pc.length)
    dst = tk.Cache.empty(H, dst_capacity(H, B, 0), 128, torch.bfloat16)
    used = torch.zeros(1, dtype=torch.int64, device="cuda")
    tk.compact(c, keep, 0, B, dst, used)
    out = torch.empty((H * G, 128), dtype=torch.float32, device="cuda")
    dropped = torch.empty(H * G, dtype=torch.float32, device="cuda")
    tk.decode_attn(dst, q_dev, G, sc, out, dropped, lse_ref=lse)
    # oracle pipeline in float64
    wm, wlse = ref.attn_mass(ov.k, q64, G, sc)
    k1, _ = ref.select_global(wm, seg, [w.mass_topk] * H)
    wks = np.array([wm[h][k1[h]].sum() for h in range(H)])
    wb, _ = ref.allocate(wks, pc.length, B)
    assert np.max(np.abs(bh - wb)) <= 1
    k2, _ = ref.select_global(wm, seg, bh)
    kk = [x[m] for x, m in zip(ov.k, k2)]
    vv = [x[m] for x, m in zip(ov.v, k2)]
    wout, wdrop, _ = ref.decode_attn(kk, vv, q64, G, sc, lse_ref=wlse)
    assert np.max(np.abs(out.cpu().numpy() - wout)) <= OUT_TOL
    assert np.max(np.abs(dropped.cpu().numpy() - wdrop)) <= DROP_TOL
    # the dropped mass equals 1 - kept mass of the full softmax (float64)
    full = [np.exp(scale_of(128) * (ov.k[h] @ q64[h * G + g]) - wlse[h * G + g]) for h in range(H) for g in range(G)]
    kept_mass = np.array([full[h * G + g][k2[h]].sum() for h in range(H) for g in range(G)])
    assert np.max(np.abs(dropped.cpu().numpy() - (1 - kept_mass))) <= DROP_TOL


@pytest.mark.parametrize("floor", [0, 64, 700])
def test_recency_floor_pipeline(floor):
    """ContourKV recency floor: top-mass per head -> kept sums -> floor-first
    allocation -> floor marked in the mass plane -> per-head selection.  The
    allocation and the selection are compared exactly with the oracle on the
    GPU's own masses and kept sums; floor 700 exceeds the budget (only the
    floors are kept), floor 0 is the plain rule."""
    w = W["qwen8b_128k"].scaled(layers=1, ctx=3000, mass_topk=256)
    lengths = np.array([3000, 500, 40, 0, 2999, 1000, 64, 65], np.int32)
    pc = synth.build_cache(w, lengths=lengths)
    H, G = pc.n_heads, w.group
    q = synth.queries(w)
    c = upload(pc)
    sc = scale_of(128)
    announce("recency floor", floor)
    mass = torch.empty(pc.n_pages * 16, dtype=torch.float32, device="cuda")
    lse = torch.empty(H * G, dtype=torch.float32, device="cuda")
    tk.attn_mass(c, kv_dev(q, "bf16"), G, sc, mass, lse)
    segs = np.arange(H + 1, dtype=np.int32)
    keep = torch.empty(pc.n_pages * 16, dtype=torch.uint8, device="cuda")
    kept = torch.empty(H, dtype=torch.int32, device="cuda")
    ks = torch.empty(H, dtype=torch.float64, device="cuda")
    tk.select_global(c, mass, cuda(segs), cuda(np.full(H, w.mass_topk), np.int64), keep, kept, ks)
    B = int(0.05 * lengths.sum())
    b = torch.empty(H, dtype=torch.int64, device="cuda")
    tk.allocate_floor(ks, c.length, B, floor, b)
    gm = heads_from_plane(mass.cpu().numpy(), pc.page_off, pc.length)
    tk.mark_recent(c, floor, mass)
    tk.select_global(c, mass, cuda(segs), b, keep, kept)
    bh = b.cpu().numpy()
    wb, _ = ref.allocate_floor(ks.cpu().numpy(), lengths, B, floor)
    assert np.array_equal(bh, wb)
    want = ref.select_floor(gm, bh, floor)
    got = heads_from_plane(keep.cpu().numpy(), pc.page_off, pc.length)
    for h in range(H):
        assert np.array_equal(got[h].astype(bool), want[h]), h
    assert np.array_equal(kept.cpu().numpy(), [int(k.sum()) for k in want])
    marked = heads_from_plane(mass.cpu().numpy(), pc.page_off, pc.length)
    for h in range(H):
        n, fl = int(lengths[h]), min(floor, int(lengths[h]))
        assert np.all(np.isposinf(marked[h][n - fl:])) and np.array_equal(marked[h][:n - fl], gm[h][:n - fl])


# --------------------------------------------------------------------------
# a7 + streaming: append -> score -> select -> attention (mask) -> compact
# --------------------------------------------------------------------------
def test_streaming_steps():
    w = SMALL["c5s"]
    pc = synth.build_cache(w)
    ov = OracleView(pc)
    H, G, D = pc.n_heads, w.group, w.head_dim
    M = w.budget()
    sc = scale_of(D)
    cur = upload(pc)
    pools = [tk.Cache.empty(H, dst_capacity(H, M, 1), D, torch.bfloat16) for _ in range(2)]
    st = {"lnb": ov.lnb, "pos": ov.pos, "k": ov.k_raw, "v": ov.v_raw}
    seg = cuda(np.array([0, H], np.int32))
    bud = cuda(np.array([M], np.int64))
    for s in range(1, w.steps + 1):
        t = w.ctx + s
        announce("stream step", s)
        beta, kn, vn, qn = synth.stream_step(w, s)
        t_dev = cuda(np.array([t], np.int32))
        tk.append(cur, kv_dev(kn, "bf16"), kv_dev(vn, "bf16"), cuda(beta, np.float32), t_dev)
        score = torch.empty(cur.n_pages * 16, dtype=torch.float32, device="cuda")
        tk.score(cur, seg, t_dev, score)
        keep = torch.empty(cur.n_pages * 16, dtype=torch.uint8, device="cuda")
        kept = torch.empty(H, dtype=torch.int32, device="cuda")
        tk.select_global(cur, score, seg, bud, keep, kept)
        out = torch.empty((H * G, D), dtype=torch.float32, device="cuda")
        dropped = torch.empty(H * G, dtype=torch.float32, device="cuda")
        tk.decode_attn(cur, kv_dev(qn, "bf16"), G, sc, out, dropped, keep=keep)
        dst = pools[s % 2]
        used = torch.zeros(1, dtype=torch.int64, device="cuda")
        tk.compact(cur, keep, 1, M, dst, used)
        # oracle step
        lnb_new = ref.ln_beta(beta)
        for h in range(H):
            st["lnb"][h] = np.append(st["lnb"][h], lnb_new[h])
            st["pos"][h] = np.append(st["pos"][h], np.int32(t - 1))
            st["k"][h] = np.concatenate([st["k"][h], kn[h:h + 1]])
            st["v"][h] = np.concatenate([st["v"][h], vn[h:h + 1]])
        scores = [ref.score_f32(st["lnb"][h], t, st["pos"][h]) for h in range(H)]
        wkeep, wkept = ref.select_global(scores, [0, H], [M])
        assert np.array_equal(kept.cpu().numpy(), wkept), s
        kf = [synth.bf16_bits_to_f32(x).astype(np.float64) for x in st["k"]]
        vf = [synth.bf16_bits_to_f32(x).astype(np.float64) for x in st["v"]]
        q64 = synth.bf16_bits_to_f32(qn).astype(np.float64)
        wout, wdrop, _ = ref.decode_attn(kf, vf, q64, G, sc, keep=wkeep)
        assert np.max(np.abs(out.cpu().numpy() - wout)) <= OUT_TOL, s
        assert np.max(np.abs(dropped.cpu().numpy() - wdrop)) <= DROP_TOL, s
        wpo, wpi, wlen, rows = ref.compact(st, wkeep, 1)
        st = rows
        po, pi, ln, k, v, lnb, pos = download_cache(dst)
        assert np.array_equal(po, wpo) and np.array_equal(ln, wlen), s
        for h in range(H):
            assert np.array_equal(ref.gather_heads(pos, po, pi, ln)[h], st["pos"][h])
            assert np.array_equal(f32_bits(ref.gather_heads(lnb, po, pi, ln)[h]), f32_bits(st["lnb"][h]))
            assert np.array_equal(ref.gather_heads(k, po, pi, ln)[h], st["k"][h])
        cur = dst
    assert tk.validate_cache(cur, cuda(np.array([w.ctx + w.steps + 1], np.int32))) == tk.OK


# --------------------------------------------------------------------------
# incremental eviction in place (each head inside its own pages)
# --------------------------------------------------------------------------
def check_inplace(pc, cur, keep, reserve, home_off, home_ids, kept_given):
    """Run trimkv_compact_inplace on the device view `cur` of host cache pc
    (whose current rows are those of pc) and compare with the oracle."""
    H = pc.n_heads
    ov = OracleView(pc)
    plane = plane_from_heads([k.astype(np.uint8) for k in keep], pc.page_off, pc.length, pc.n_pages, 0, np.uint8)
    wk = np.array([int(k.sum()) for k in keep], np.int32)
    new_off = torch.full((H + 1,), -1, dtype=torch.int32, device="cuda")
    new_ids = torch.full((max(int(home_off[-1]), 1),), -1, dtype=torch.int32, device="cuda")
    view = tk.compact_inplace(cur, cuda(plane), reserve, cuda(home_off, np.int32), cuda(home_ids, np.int32),
                              new_off, new_ids, kept=cuda(wk) if kept_given else None)
    wpo, wpi, wlen = ref.compact_inplace_layout(wk, reserve, home_off, home_ids)
    po, pi, ln, k, v, lnb, pos = download_cache(view)
    assert np.array_equal(po, wpo) and np.array_equal(ln, wlen)
    assert np.array_equal(pi[:wpo[-1]], wpi)
    for name, plane_now, want in (("k", k, ov.k_raw), ("v", v, ov.v_raw), ("pos", pos, ov.pos)):
        got = ref.gather_heads(plane_now, po, pi[:max(int(po[-1]), 1)], ln)
        for h in range(H):
            assert np.array_equal(got[h], want[h][keep[h]]), (name, h)
    got = ref.gather_heads(lnb, po, pi[:max(int(po[-1]), 1)], ln)
    for h in range(H):
        assert np.array_equal(f32_bits(got[h]), f32_bits(ov.lnb[h][keep[h]])), ("lnb", h)
    return view


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)])
def test_compact_inplace(dtype, d):
    """Keep patterns per head: everything, nothing, random 30%, one drop
    near the start, one near the end, every other entry; lengths of 0, 1,
    16, 17 and up to 2500 (several 1024-slot windows).  The home table is the
    cache's own (current view = home); reserve 0, 3 and 40 (clamped to the
    home pages); counts given and counted."""
    rng = np.random.default_rng(1100 + d)
    pc = synth.random_ragged_cache(1200 + d, n_heads=12, d=d, dtype=dtype, max_len=2500, reserve=20)
    pc.length[:4] = [0, 1, 16, 17]
    for reserve, kept_given in ((0, True), (3, False), (40, True)):
        keep = []
        for h, n in enumerate(pc.length):
            n = int(n)
            pat = h % 6
            if pat == 0:
                kp = np.ones(n, bool)
            elif pat == 1:
                kp = np.zeros(n, bool)
            elif pat == 2:
                kp = rng.random(n) < 0.3
            elif pat == 3:
                kp = np.ones(n, bool)
                kp[min(2, n - 1):min(3, n)] = False
            elif pat == 4:
                kp = np.ones(n, bool)
                kp[max(n - 3, 0):max(n - 2, 0)] = False
            else:
                kp = np.arange(n) % 2 == 0
            keep.append(kp)
        announce("compact in place", dtype, d, "reserve", reserve, "lengths", pc.length.tolist())
        cur = upload(pc)
        check_inplace(pc, cur, keep, reserve, pc.page_off.astype(np.int64), pc.page_ids.astype(np.int64),
                      kept_given)


def test_streaming_steps_inplace():
    """The streaming loop with in-place eviction: append -> score -> select ->
    compact in place, every step checked against the oracle's selection and
    kept rows (content equals the out-of-place rule); the home table is the
    prefill table and every later view a prefix of it."""
    w = SMALL["c5s"]
    pc = synth.build_cache(w)
    ov = OracleView(pc)
    H, D = pc.n_heads, w.head_dim
    M = w.budget()
    cur = upload(pc)
    home_off, home_ids = cur.page_off.clone(), cur.page_ids.clone()
    home_off_np = pc.page_off.astype(np.int64)
    home_ids_np = pc.page_ids.astype(np.int64)
    tables = [(torch.empty(H + 1, dtype=torch.int32, device="cuda"),
               torch.empty(int(home_off_np[-1]), dtype=torch.int32, device="cuda")) for _ in range(2)]
    st = {"lnb": ov.lnb, "pos": ov.pos, "k": ov.k_raw, "v": ov.v_raw}
    seg = cuda(np.array([0, H], np.int32))
    bud = cuda(np.array([M], np.int64))
    for s in range(1, w.steps + 1):
        t = w.ctx + s
        announce("stream step in place", s)
        beta, kn, vn, _ = synth.stream_step(w, s)
        t_dev = cuda(np.array([t], np.int32))
        tk.append(cur, kv_dev(kn, "bf16"), kv_dev(vn, "bf16"), cuda(beta, np.float32), t_dev)
        score = torch.empty(cur.n_pages * 16, dtype=torch.float32, device="cuda")
        tk.score(cur, seg, t_dev, score)
        keep = torch.empty(cur.n_pages * 16, dtype=torch.uint8, device="cuda")
        kept = torch.empty(H, dtype=torch.int32, device="cuda")
        tk.select_global(cur, score, seg, bud, keep, kept)
        no, ni = tables[s % 2]
        cur = tk.compact_inplace(cur, keep, 1, home_off, home_ids, no, ni, kept=kept)
        lnb_new = ref.ln_beta(beta)
        for h in range(H):
            st["lnb"][h] = np.append(st["lnb"][h], lnb_new[h])
            st["pos"][h] = np.append(st["pos"][h], np.int32(t - 1))
            st["k"][h] = np.concatenate([st["k"][h], kn[h:h + 1]])
            st["v"][h] = np.concatenate([st["v"][h], vn[h:h + 1]])
        scores = [ref.score_f32(st["lnb"][h], t, st["pos"][h]) for h in range(H)]
        wkeep, wkept = ref.select_global(scores, [0, H], [M])
        assert np.array_equal(kept.cpu().numpy(), wkept), s
        _, _, _, rows = ref.compact(st, wkeep, 1)
        st = rows
        wpo, wpi, wlen = ref.compact_inplace_layout(wkept, 1, home_off_np, home_ids_np)
        po, pi, ln, k, v, lnb, pos = download_cache(cur)
        assert np.array_equal(po, wpo) and np.array_equal(ln, wlen) and np.array_equal(pi[:wpo[-1]], wpi), s
        pi = pi[:wpo[-1]]
        for h in range(H):
            assert np.array_equal(ref.gather_heads(pos, po, pi, ln)[h], st["pos"][h])
            assert np.array_equal(f32_bits(ref.gather_heads(lnb, po, pi, ln)[h]), f32_bits(st["lnb"][h]))
            assert np.array_equal(ref.gather_heads(k, po, pi, ln)[h], st["k"][h])
            assert np.array_equal(ref.gather_heads(v, po, pi, ln)[h], st["v"][h])
    assert tk.validate_cache(cur, cuda(np.array([w.ctx + w.steps + 1], np.int32))) == tk.OK


# --------------------------------------------------------------------------
# tail-filled eviction (only the entries that fill holes move)
# --------------------------------------------------------------------------
def _keep_patterns(rng, lengths):
    keep = []
    for h, n in enumerate(lengths):
        n = int(n)
        pat = h % 6
        if pat == 0:
            kp = np.ones(n, bool)
        elif pat == 1:
            kp = np.zeros(n, bool)
        elif pat == 2:
            kp = rng.random(n) < 0.3
        elif pat == 3:
            kp = np.ones(n, bool)
            kp[min(2, n - 1):min(3, n)] = False
        elif pat == 4:
            kp = rng.random(n) < 0.97
        else:
            kp = np.arange(n) % 2 == 0
        keep.append(kp)
    return keep


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)])
def test_evict_tailfill(dtype, d):
    """trimkv_evict_tailfill against the oracle's tail-fill order: every
    head's rows, ln(beta) and positions in their new slot order, the page
    table (home prefix) and lengths; lengths 0, 1, 16, 17 and up to 2500;
    counts given and counted."""
    rng = np.random.default_rng(1300 + d)
    pc = synth.random_ragged_cache(1400 + d, n_heads=12, d=d, dtype=dtype, max_len=2500, reserve=20)
    pc.length[:4] = [0, 1, 16, 17]
    ov = OracleView(pc)
    H = pc.n_heads
    home_off, home_ids = pc.page_off.astype(np.int64), pc.page_ids.astype(np.int64)
    for reserve, kept_given in ((0, True), (3, False), (40, True)):
        keep = _keep_patterns(rng, pc.length)
        announce("evict tail-fill", dtype, d, "reserve", reserve)
        cur = upload(pc)
        plane = plane_from_heads([k.astype(np.uint8) for k in keep], pc.page_off, pc.length, pc.n_pages, 0,
                                 np.uint8)
        wk = np.array([int(k.sum()) for k in keep], np.int32)
        new_off = torch.full((H + 1,), -1, dtype=torch.int32, device="cuda")
        new_ids = torch.full((int(home_off[-1]),), -1, dtype=torch.int32, device="cuda")
        view = tk.evict_tailfill(cur, cuda(plane), reserve, cuda(home_off, np.int32), cuda(home_ids, np.int32),
                                 new_off, new_ids, kept=cuda(wk) if kept_given else None)
        order, (wpo, wpi, wlen) = ref.evict_tailfill_order(keep, reserve, home_off, home_ids)
        po, pi, ln, k, v, lnb, pos = download_cache(view)
        assert np.array_equal(po, wpo) and np.array_equal(ln, wlen) and np.array_equal(pi[:wpo[-1]], wpi)
        pi = pi[:max(int(wpo[-1]), 1)]
        for name, now, was in (("k", k, ov.k_raw), ("v", v, ov.v_raw), ("pos", pos, ov.pos)):
            got = ref.gather_heads(now, po, pi, ln)
            for h in range(H):
                assert np.array_equal(got[h], was[h][order[h]]), (name, h)
        got = ref.gather_heads(lnb, po, pi, ln)
        for h in range(H):
            assert np.array_equal(f32_bits(got[h]), f32_bits(ov.lnb[h][order[h]])), ("lnb", h)


def test_streaming_steps_tailfill():
    """The streaming loop with tail-filled eviction: append -> score ->
    select -> mask-mode attention -> evict in place, the oracle tracking each
    head's slot order (its selection ranks ties by position); kept counts,
    page tables, rows, ln(beta) and positions in slot order every step, and
    attention within tolerance."""
    w = SMALL["c5s"]
    pc = synth.build_cache(w)
    ov = OracleView(pc)
    H, G, D = pc.n_heads, w.group, w.head_dim
    M = w.budget()
    sc = scale_of(D)
    cur = upload(pc)
    home_off, home_ids = cur.page_off.clone(), cur.page_ids.clone()
    home_off_np, home_ids_np = pc.page_off.astype(np.int64), pc.page_ids.astype(np.int64)
    tables = [(torch.empty(H + 1, dtype=torch.int32, device="cuda"),
               torch.empty(int(home_off_np[-1]), dtype=torch.int32, device="cuda")) for _ in range(2)]
    st = {"lnb": ov.lnb, "pos": ov.pos, "k": ov.k_raw, "v": ov.v_raw}
    seg = cuda(np.array([0, H], np.int32))
    bud = cuda(np.array([M], np.int64))
    status = torch.zeros(2, dtype=torch.int32, device="cuda")
    for s in range(1, w.steps + 1):
        t = w.ctx + s
        announce("stream step tail-fill", s)
        beta, kn, vn, qn = synth.stream_step(w, s)
        t_dev = cuda(np.array([t], np.int32))
        tk.append(cur, kv_dev(kn, "bf16"), kv_dev(vn, "bf16"), cuda(beta, np.float32), t_dev, status=status[0:1])
        score = torch.empty(cur.n_pages * 16, dtype=torch.float32, device="cuda")
        keep = torch.empty(cur.n_pages * 16, dtype=torch.uint8, device="cuda")
        kept = torch.empty(H, dtype=torch.int32, device="cuda")
        tk.score_select(cur, seg, t_dev, bud, score, keep, kept, status=status[1:2])
        out = torch.empty((H * G, D), dtype=torch.float32, device="cuda")
        dropped = torch.empty(H * G, dtype=torch.float32, device="cuda")
        tk.decode_attn(cur, kv_dev(qn, "bf16"), G, sc, out, dropped, keep=keep)
        no, ni = tables[s % 2]
        cur = tk.evict_tailfill(cur, keep, 1, home_off, home_ids, no, ni, kept=kept)
        lnb_new = ref.ln_beta(beta)
        for h in range(H):
            st["lnb"][h] = np.append(st["lnb"][h], lnb_new[h])
            st["pos"][h] = np.append(st["pos"][h], np.int32(t - 1))
            st["k"][h] = np.concatenate([st["k"][h], kn[h:h + 1]])
            st["v"][h] = np.concatenate([st["v"][h], vn[h:h + 1]])
        scores = [ref.score_f32(st["lnb"][h], t, st["pos"][h]) for h in range(H)]
        wkeep, wkept = ref.select_global(scores, [0, H], [M], positions=st["pos"])
        assert np.array_equal(kept.cpu().numpy(), wkept), s
        q64 = synth.bf16_bits_to_f32(qn).astype(np.float64)
        kf = [synth.bf16_bits_to_f32(x).astype(np.float64) for x in st["k"]]
        vf = [synth.bf16_bits_to_f32(x).astype(np.float64) for x in st["v"]]
        wout, wdrop, _ = ref.decode_attn(kf, vf, q64, G, sc, keep=wkeep)
        assert np.max(np.abs(out.cpu().numpy() - wout)) <= OUT_TOL, s
        assert np.max(np.abs(dropped.cpu().numpy() - wdrop)) <= DROP_TOL, s
        order, (wpo, wpi, wlen) = ref.evict_tailfill_order(wkeep, 1, home_off_np, home_ids_np)
        st = {name: [x[h][order[h]] for h in range(H)] for name, x in st.items()}
        po, pi, ln, k, v, lnb, pos = download_cache(cur)
        assert np.array_equal(po, wpo) and np.array_equal(ln, wlen) and np.array_equal(pi[:wpo[-1]], wpi), s
        pi = pi[:wpo[-1]]
        for h in range(H):
            assert np.array_equal(ref.gather_heads(pos, po, pi, ln)[h], st["pos"][h]), (s, h)
            assert np.array_equal(f32_bits(ref.gather_heads(lnb, po, pi, ln)[h]), f32_bits(st["lnb"][h]))
            assert np.array_equal(ref.gather_heads(k, po, pi, ln)[h], st["k"][h])
            assert np.array_equal(ref.gather_heads(v, po, pi, ln)[h], st["v"][h])
    assert int(status.sum().item()) == 0


@pytest.mark.parametrize("kind", ["alpha3", "equal", "zeros", "nan"])
def test_select_ties_out_of_position_order(kind):
    """Caches whose slots hold positions in shuffled order within every head
    (as after tail-filled eviction), with tie-heavy scores: the selection
    ranks ties by position, as the oracle given the positions; segments end
    inside 32-chunk blocks; heads of many chunks."""
    rng = np.random.default_rng(1500 + ["alpha3", "equal", "zeros", "nan"].index(kind))
    pc = synth.random_ragged_cache(1600, n_heads=14, d=64, dtype="bf16", max_len=9000)
    # shuffle positions within every head's slots
    for h in range(pc.n_heads):
        sl = ref.head_phys_slots(pc.page_off, pc.page_ids, pc.length, h)
        flat = pc.pos.reshape(-1)
        flat[sl] = flat[sl][rng.permutation(len(sl))]
    ov = OracleView(pc)
    lens = pc.length
    if kind == "alpha3":
        sc = [rng.choice([-1.5, -0.25, 0.0], n).astype(np.float32) for n in lens]
    elif kind == "equal":
        sc = [np.full(n, -0.5, np.float32) for n in lens]
    elif kind == "zeros":
        sc = [rng.choice([0.0, -0.0], n).astype(np.float32) for n in lens]
    else:
        sc = [np.where(rng.random(n) < 0.2, np.nan, rng.choice([-np.inf, -2.0, 1.5], n)).astype(np.float32)
              for n in lens]
    seg = np.array([0, 3, 9, 14], np.int32)
    N = [int(lens[seg[s]:seg[s + 1]].sum()) for s in range(3)]
    c = upload(pc)
    plane = plane_from_heads(sc, pc.page_off, pc.length, pc.n_pages)
    for budgets in ([n // 3 for n in N], [int(rng.integers(1, n + 1)) for n in N], [1, 0, N[2] - 1]):
        announce("select out of position order", kind, budgets)
        keep, kept, _ = run_select(c, plane, seg, budgets)
        want_keep, want_kept = ref.select_global(sc, seg, budgets, positions=ov.pos)
        got = heads_from_plane(keep, pc.page_off, pc.length)
        for h in range(pc.n_heads):
            assert np.array_equal(got[h].astype(bool), want_keep[h]), (budgets, h)
        assert np.array_equal(kept, want_kept)


# --------------------------------------------------------------------------
# the streaming step captured in HIP graphs
# --------------------------------------------------------------------------
@pytest.mark.parametrize("evict", ["out_of_place", "tail_fill", "tail_fill_separate"])
def test_streaming_graph_capture(evict):
    """Steps 3..S of the scaled streaming workload replayed from captured
    graphs (one per step) against the same steps run eagerly, evicting out
    of place or in place by tail fill (as two fused calls per step, or as the
    four separate calls): kept counts, outputs, dropped mass, page tables and
    the final pools bit for bit after every replay, with eager work and
    synchronisations between replays; the final state against the oracle."""
    from retention_scored_decode_amd.stream import StreamLoop

    w = SMALL["c5s"].scaled(steps=24)
    S = w.steps
    pc = synth.build_cache(w)
    H, G, D = pc.n_heads, w.group, w.head_dim
    M = w.budget()
    sc = scale_of(D)
    steps_in = [synth.stream_step(w, s) for s in range(1, S + 1)]
    banks = {"k": kv_dev(np.stack([x[1] for x in steps_in]), "bf16"),
             "v": kv_dev(np.stack([x[2] for x in steps_in]), "bf16"),
             "beta": cuda(np.stack([x[0] for x in steps_in]), np.float32),
             "q": kv_dev(np.stack([x[3] for x in steps_in]), "bf16"),
             "t": cuda(np.arange(w.ctx + 1, w.ctx + S + 1, dtype=np.int32).reshape(S, 1))}
    prefill = upload(pc)
    len0 = prefill.length.clone()

    def start():
        """step 1 (the prefill eviction) into a fresh pair of pools, or into
        home pages with a spare slot per head for every later step"""
        if evict.startswith("tail_fill"):
            pools = [tk.Cache.empty(H, dst_capacity(H, M, S), D, torch.bfloat16)]
            reserve = S
        else:
            pools = [tk.Cache.empty(H, dst_capacity(H, M, 1), D, torch.bfloat16) for _ in range(2)]
            reserve = 1
        prefill.length.copy_(len0)
        t = cuda(np.array([w.ctx + 1], np.int32))
        tk.append(prefill, banks["k"][0], banks["v"][0], banks["beta"][0], t)
        score = torch.empty(prefill.n_pages * 16, dtype=torch.float32, device="cuda")
        keep = torch.empty(prefill.n_pages * 16, dtype=torch.uint8, device="cuda")
        kept = torch.empty(H, dtype=torch.int32, device="cuda")
        seg = cuda(np.array([0, H], np.int32))
        tk.score(prefill, seg, t, score)
        tk.select_global(prefill, score, seg, cuda(np.array([M], np.int64)), keep, kept)
        tk.compact(prefill, keep, reserve, M, pools[0], torch.zeros(1, dtype=torch.int64, device="cuda"), kept=kept)
        return StreamLoop(pools, M, G, sc, banks, first=1, evict="tail_fill" if evict.startswith("tail_fill") else evict,
                          fused=evict == "tail_fill")

    def state(loop):
        torch.cuda.synchronize()
        c = loop.cache
        return (loop.kept.cpu().numpy(), loop.out.cpu().numpy().view(np.uint32),
                loop.dropped.cpu().numpy().view(np.uint32), c.page_off.cpu().numpy(), c.length.cpu().numpy())

    eager = start()
    want = []
    for s in range(2, S + 1):
        eager.run(1)
        want.append(state(eager))
    graph = start()
    graph.run(1)                      # step 2 eagerly (the library's first-call set-up done), then capture
    assert all(np.array_equal(a, b) for a, b in zip(state(graph), want[0]))
    graph.capture(S - 2, chunk=1)     # one graph per step, so every step can be checked
    noise = torch.arange(1 << 16, dtype=torch.float32, device="cuda")
    for s in range(3, S + 1):
        announce("graph replay step", s)
        graph.replay(1)
        noise.mul_(1.0001).add_(1.0)          # eager work between replays
        got = state(graph)
        for a, b in zip(got, want[s - 2]):
            assert np.array_equal(a, b), s
    assert int(graph.status.sum().item()) == 0 and int(eager.status.sum().item()) == 0
    ge, gg = download_cache(eager.cache), download_cache(graph.cache)
    for i in (3, 4, 5, 6):   # K, V, ln(beta), positions of every head
        for x, y in zip(ref.gather_heads(ge[i], ge[0], ge[1], ge[2]), ref.gather_heads(gg[i], gg[0], gg[1], gg[2])):
            assert np.array_equal(x.view(np.uint8), y.view(np.uint8))
    # the final state against the oracle: positions and ln(beta) of every head
    ov = OracleView(pc)
    lnb, pos = ov.lnb, ov.pos
    for s in range(1, S + 1):
        t = w.ctx + s
        lnb = [np.append(lnb[h], ref.ln_beta(steps_in[s - 1][0])[h]) for h in range(H)]
        pos = [np.append(pos[h], np.int32(t - 1)) for h in range(H)]
        keep, _ = ref.select_global([ref.score_f32(lnb[h], t, pos[h]) for h in range(H)], [0, H], [M])
        lnb = [lnb[h][keep[h]] for h in range(H)]
        pos = [pos[h][keep[h]] for h in range(H)]
    gpos = ref.gather_heads(gg[6], gg[0], gg[1], gg[2])
    glnb = ref.gather_heads(gg[5], gg[0], gg[1], gg[2])
    for h in range(H):
        o = np.argsort(gpos[h], kind="stable")   # tail fill keeps the entries, not their slot order
        assert np.array_equal(gpos[h][o], pos[h]) and np.array_equal(f32_bits(glnb[h][o]), f32_bits(lnb[h])), h
