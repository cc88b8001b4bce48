"""The streaming step's fused calls against the separate calls they replace,
bit for bit, and against the oracle: trimkv_append_score_select (the step's
append written by the selection's first kernel) must leave the cache, the
score plane and the selection exactly as trimkv_append followed by
trimkv_score_select (TRIM-KV page, section 2: a new entry per head with its
retention, then the lowest current scores are evicted once the budget is
exceeded)."""
import numpy as np
import pytest
import torch

import synth
from oracle import reference as ref
from retention_scored_decode_amd import trimkv as tk
from gpu_helpers import OracleView, cuda, download_cache, f32_bits, heads_from_plane, kv_dev, upload

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def announce(*a):
    print("[case]", *a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    tk.lib()


def clone_cache(c: tk.Cache) -> tk.Cache:
    return tk.Cache(c.k.clone(), c.v.clone(), c.meta.clone(), c.page_off.clone(), c.page_ids.clone(),
                    c.length.clone())


def same_cache(a: tk.Cache, b: tk.Cache):
    for x, y in zip(download_cache(a), download_cache(b)):
        assert np.array_equal(np.asarray(x).view(np.uint8), np.asarray(y).view(np.uint8))


def step_pair(ca, cb, kn, vn, beta, seg, t_dev, bud, dtype, keptsum=False):
    """The separate calls on ca, the fused call on cb; returns both outputs."""
    H = ca.n_heads
    n = ca.n_pages * 16
    outs = []
    for fused, c in ((False, ca), (True, cb)):
        score = torch.full((n,), 7.0, dtype=torch.float32, device="cuda")
        keep = torch.full((n,), 9, dtype=torch.uint8, device="cuda")
        kept = torch.empty(H, dtype=torch.int32, device="cuda")
        ks = torch.empty(H, dtype=torch.float64, device="cuda") if keptsum else None
        status = torch.zeros(2, dtype=torch.int32, device="cuda")
        if fused:
            tk.append_score_select(c, kv_dev(kn, dtype), kv_dev(vn, dtype), cuda(beta, np.float32), seg, t_dev,
                                   bud, score, keep, kept, keptsum=ks, append_status=status[0:1],
                                   select_status=status[1:2])
        else:
            tk.append(c, kv_dev(kn, dtype), kv_dev(vn, dtype), cuda(beta, np.float32), t_dev[0:1], status=status[0:1])
            tk.score_select(c, seg, t_dev, bud, score, keep, kept, keptsum=ks, status=status[1:2])
        torch.cuda.synchronize()
        outs.append(dict(score=score.cpu().numpy(), keep=keep.cpu().numpy(), kept=kept.cpu().numpy(),
                         ks=None if ks is None else ks.cpu().numpy(), status=status.cpu().numpy()))
    a, b = outs
    assert np.array_equal(f32_bits(a["score"]), f32_bits(b["score"]))
    assert np.array_equal(a["keep"], b["keep"]) and np.array_equal(a["kept"], b["kept"])
    if keptsum:
        assert np.array_equal(a["ks"].view(np.uint64), b["ks"].view(np.uint64))
    assert np.array_equal(a["status"], b["status"])
    same_cache(ca, cb)
    return a


def test_append_score_select_matches_separate_calls():
    """Scaled streaming cache (one spare slot per head): four generated steps,
    each followed by tail-filled eviction of both caches; the fused call's
    cache, scores, keep plane, kept counts and kept sums equal the separate
    calls' bit for bit, and the selection equals the oracle's."""
    w = W["stream_gqa7"].scaled(layers=2, ctx=2000, budget_abs=1024, steps=4)
    pc = synth.build_cache(w)
    ov = OracleView(pc)
    H, D = pc.n_heads, w.head_dim
    M = w.budget()
    ca = upload(pc)
    cb = clone_cache(ca)
    home_off, home_ids = ca.page_off.clone(), ca.page_ids.clone()
    tables = {n: [(torch.zeros_like(home_off), torch.zeros_like(home_ids)) for _ in range(2)] for n in "ab"}
    seg = cuda(np.array([0, H], np.int32))
    bud = cuda(np.array([M], np.int64))
    lnb, pos = ov.lnb, ov.pos
    for s in range(1, w.steps + 1):
        t = w.ctx + s
        announce("append+score+select, stream step", s)
        beta, kn, vn, _ = synth.stream_step(w, s)
        out = step_pair(ca, cb, kn, vn, beta, seg, cuda(np.array([t], np.int32)), bud, "bf16", keptsum=True)
        assert out["status"].tolist() == [0, 0]
        # oracle: append, score, select over the slot-ordered state
        lnb_new = ref.ln_beta(beta)
        lnb = [np.append(lnb[h], lnb_new[h]) for h in range(H)]
        pos = [np.append(pos[h], np.int32(t - 1)) for h in range(H)]
        scores = [ref.score_f32(lnb[h], t, pos[h]) for h in range(H)]
        wkeep, wkept = ref.select_global(scores, [0, H], [M], positions=pos)
        assert np.array_equal(out["kept"], wkept), s
        po, ln = ca.page_off.cpu().numpy(), ca.length.cpu().numpy()
        got = heads_from_plane(out["keep"], po, ln)
        for h in range(H):
            assert np.array_equal(got[h].astype(bool), wkeep[h]), (s, h)
            assert np.array_equal(f32_bits(heads_from_plane(out["score"], po, ln)[h]), f32_bits(scores[h])), (s, h)
        kept_dev = cuda(out["kept"], np.int32)
        keep = cuda(out["keep"], np.uint8)
        ca = tk.evict_tailfill(ca, keep, 1, home_off, home_ids, *tables["a"][s % 2], kept=kept_dev)
        cb = tk.evict_tailfill(cb, keep, 1, home_off, home_ids, *tables["b"][s % 2], kept=kept_dev)
        order, _ = ref.evict_tailfill_order(wkeep, 1, home_off.cpu().numpy().astype(np.int64),
                                            home_ids.cpu().numpy().astype(np.int64))
        lnb = [lnb[h][order[h]] for h in range(H)]
        pos = [pos[h][order[h]] for h in range(H)]
        same_cache(ca, cb)


def test_append_score_select_full_heads_and_segments():
    """Heads without a free slot are left unchanged and counted, as
    trimkv_append does; with several segments every head's new entry takes
    its own segment's step (position t_s - 1) and is scored at it."""
    w = W["stream_gqa7"].scaled(batch=3, layers=2, ctx=300, per_seq_segments=True, reserve=0)
    H = w.n_heads
    rng = np.random.default_rng(11)
    lengths = rng.integers(250, 301, H).astype(np.int32)
    lengths[::3] = 288                               # 18 full pages, no free slot
    pc = synth.build_cache(w, lengths=lengths)
    full = (lengths % 16) == 0
    ov = OracleView(pc)
    ca = upload(pc)
    cb = clone_cache(ca)
    segs = w.seg_head_begin()
    t = np.array([400, 333, 512], np.int32)
    M = 500
    beta = rng.uniform(0.0, 1.0, H).astype(np.float32)
    beta[:4] = [0.0, 1.0, 2 ** -149, 0.5]
    kn = synth.f64_to_bf16_bits(rng.standard_normal((H, w.head_dim)))
    vn = synth.f64_to_bf16_bits(rng.standard_normal((H, w.head_dim)))
    n = ca.n_pages * 16
    score = torch.empty(n, dtype=torch.float32, device="cuda")
    keep = torch.empty(n, dtype=torch.uint8, device="cuda")
    kept = torch.empty(H, dtype=torch.int32, device="cuda")
    status = torch.zeros(2, dtype=torch.int32, device="cuda")
    announce("append+score+select, 3 segments, full heads", int(full.sum()))
    tk.append_score_select(cb, kv_dev(kn, "bf16"), kv_dev(vn, "bf16"), cuda(beta), cuda(segs), cuda(t),
                           cuda(np.full(3, M, np.int64)), score, keep, kept, append_status=status[0:1],
                           select_status=status[1:2])
    torch.cuda.synchronize()
    assert status.cpu().numpy().tolist() == [int(full.sum()), 0]
    seg_of = np.searchsorted(segs, np.arange(H), side="right") - 1
    lnb_new = ref.ln_beta(beta)
    lnb, pos, kr, vr = ov.lnb, ov.pos, ov.k_raw, ov.v_raw
    for h in range(H):
        if not full[h]:
            lnb[h] = np.append(lnb[h], lnb_new[h])
            pos[h] = np.append(pos[h], np.int32(t[seg_of[h]] - 1))
            kr[h] = np.concatenate([kr[h], kn[h:h + 1]])
            vr[h] = np.concatenate([vr[h], vn[h:h + 1]])
    po, pi, ln, k, v, glnb, gpos = download_cache(cb)
    assert np.array_equal(ln, lengths + (~full))
    for h in range(H):
        assert np.array_equal(ref.gather_heads(gpos, po, pi, ln)[h], pos[h]), h
        assert np.array_equal(f32_bits(ref.gather_heads(glnb, po, pi, ln)[h]), f32_bits(lnb[h])), h
        assert np.array_equal(ref.gather_heads(k, po, pi, ln)[h], kr[h]), h
        assert np.array_equal(ref.gather_heads(v, po, pi, ln)[h], vr[h]), h
    scores = [ref.score_f32(lnb[h], int(t[seg_of[h]]), pos[h]) for h in range(H)]
    got_s = heads_from_plane(score.cpu().numpy(), po, ln)
    for h in range(H):
        assert np.array_equal(f32_bits(got_s[h]), f32_bits(scores[h])), h
    wkeep, wkept = ref.select_global(scores, segs, [M] * 3, positions=pos)
    assert np.array_equal(kept.cpu().numpy(), wkept)
    got = heads_from_plane(keep.cpu().numpy(), po, ln)
    for h in range(H):
        assert np.array_equal(got[h].astype(bool), wkeep[h]), h
    # one segment per call with the same step everywhere: the separate calls agree
    w1 = w.scaled(per_seq_segments=False)
    cc = upload(pc)
    cd = clone_cache(cc)
    step_pair(cc, cd, kn, vn, beta, cuda(np.array([0, H], np.int32)), cuda(np.array([400], np.int32)),
              cuda(np.array([w1.budget() // 2], np.int64)), "bf16")


def test_append_score_select_many_heads():
    """More heads than the selection's LDS head list (4,096): the first
    kernel then runs as one block and raises the lengths itself; fp32 cache,
    D = 64."""
    w = W["tiny"].scaled(layers=2100, kv_heads=2, ctx=40, reserve=1, budget_abs=60000)
    H = w.n_heads
    assert H > 4096
    pc = synth.build_cache(w)
    ca = upload(pc)
    cb = clone_cache(ca)
    rng = np.random.default_rng(5)
    beta = rng.beta(5.0, 1.0, H).astype(np.float32)
    kn = rng.standard_normal((H, w.head_dim)).astype(np.float32)
    vn = rng.standard_normal((H, w.head_dim)).astype(np.float32)
    announce("append+score+select, heads", H)
    out = step_pair(ca, cb, kn, vn, beta, cuda(np.array([0, H], np.int32)), cuda(np.array([w.ctx + 1], np.int32)),
                    cuda(np.array([w.budget()], np.int64)), "f32")
    assert out["status"].tolist() == [0, 0]
    assert np.array_equal(ca.length.cpu().numpy(), pc.length + 1)


@pytest.mark.parametrize("shape", ["bf16_d128", "bf16_d64", "f32_d64"])
def test_decode_attn_evict_tailfill_matches_separate_calls(shape):
    """trimkv_decode_attn_evict_tailfill against mask-mode trimkv_decode_attn
    followed by trimkv_evict_tailfill: outputs, dropped mass, rows, lengths
    and the new tables bit for bit over four streaming steps, and the
    outputs within tolerance of the oracle."""
    base = W["stream_gqa7"].scaled(layers=2, ctx=1500, budget_abs=900, steps=4)
    if shape == "bf16_d64":
        base = base.scaled(head_dim=64)
    elif shape == "f32_d64":
        base = base.scaled(head_dim=64, dtype="f32", group=3)
    w = base
    dt = w.dtype
    pc = synth.build_cache(w)
    ov = OracleView(pc)
    H, G, D = pc.n_heads, w.group, w.head_dim
    M = w.budget()
    sc = D ** -0.5
    ca = upload(pc)
    cb = clone_cache(ca)
    home_off, home_ids = ca.page_off.clone(), ca.page_ids.clone()
    tables = {n: [(torch.zeros_like(home_off), torch.zeros_like(home_ids)) for _ in range(2)] for n in "ab"}
    seg = cuda(np.array([0, H], np.int32))
    bud = cuda(np.array([M], np.int64))
    st = {"lnb": ov.lnb, "pos": ov.pos, "k": ov.k_raw, "v": ov.v_raw}
    rng = np.random.default_rng(77)
    for s in range(1, w.steps + 1):
        t = w.ctx + s
        announce("attention + tail fill,", shape, "step", s)
        beta = rng.beta(5.0, 1.0, H).astype(np.float32)
        kn = rng.standard_normal((H, D))
        vn = rng.standard_normal((H, D))
        qn = rng.standard_normal((H * G, D))
        conv = synth.f64_to_bf16_bits if dt == "bf16" else (lambda x: x.astype(np.float32))
        kn, vn, qn = conv(kn), conv(vn), conv(qn)
        t_dev = cuda(np.array([t], np.int32))
        outs = []
        for name in "ab":
            c = ca if name == "a" else cb
            n = c.n_pages * 16
            score = torch.empty(n, dtype=torch.float32, device="cuda")
            keep = torch.empty(n, dtype=torch.uint8, device="cuda")
            kept = torch.empty(H, dtype=torch.int32, device="cuda")
            tk.append_score_select(c, kv_dev(kn, dt), kv_dev(vn, dt), cuda(beta), seg, t_dev, bud, score, keep, kept)
            used = int(c.page_off[H].item()) * 16   # the keep plane's slots under the current table
            out = torch.full((H * G, D), 5.0, dtype=torch.float32, device="cuda")
            dropped = torch.full((H * G,), 5.0, dtype=torch.float32, device="cuda")
            no, ni = tables[name][s % 2]
            if name == "a":
                tk.decode_attn(c, kv_dev(qn, dt), G, sc, out, dropped, keep=keep)
                v = tk.evict_tailfill(c, keep, 1, home_off, home_ids, no, ni, kept=kept)
            else:
                v = tk.decode_attn_evict_tailfill(c, keep, kept, kv_dev(qn, dt), G, sc, out, dropped, 1, home_off,
                                                  home_ids, no, ni)
            torch.cuda.synchronize()
            outs.append((out.cpu().numpy(), dropped.cpu().numpy(), keep[:used].cpu().numpy(), kept.cpu().numpy()))
            if name == "a":
                ca = v
            else:
                cb = v
        (oa, da, ka, na), (ob, db, kb, nb) = outs
        assert np.array_equal(ka, kb) and np.array_equal(na, nb)
        assert np.array_equal(f32_bits(oa), f32_bits(ob)) and np.array_equal(f32_bits(da), f32_bits(db)), s
        same_cache(ca, cb)
        # oracle: the step's selection and attention over the slot-ordered state
        lnb_new = ref.ln_beta(beta)
        for h in range(H):
            st["lnb"][h] = np.append(st["lnb"][h], lnb_new[h])
            st["pos"][h] = np.append(st["pos"][h], np.int32(t - 1))
            st["k"][h] = np.concatenate([st["k"][h], kn[h:h + 1]])
            st["v"][h] = np.concatenate([st["v"][h], vn[h:h + 1]])
        scores = [ref.score_f32(st["lnb"][h], t, st["pos"][h]) for h in range(H)]
        wkeep, wkept = ref.select_global(scores, [0, H], [M], positions=st["pos"])
        assert np.array_equal(na, wkept), s
        tof = synth.bf16_bits_to_f32 if dt == "bf16" else (lambda x: x)
        q64 = tof(qn).astype(np.float64)
        kf = [tof(x).astype(np.float64) for x in st["k"]]
        vf = [tof(x).astype(np.float64) for x in st["v"]]
        wout, wdrop, _ = ref.decode_attn(kf, vf, q64, G, sc, keep=wkeep)
        assert np.max(np.abs(oa - wout)) <= 2e-3, s
        assert np.max(np.abs(da - wdrop)) <= 1e-5, s
        order, _ = ref.evict_tailfill_order(wkeep, 1, home_off.cpu().numpy().astype(np.int64),
                                            home_ids.cpu().numpy().astype(np.int64))
        st = {nm: [x[h][order[h]] for h in range(H)] for nm, x in st.items()}
        po, pi, ln, k, v, glnb, gpos = download_cache(cb)
        for h in range(H):
            assert np.array_equal(ref.gather_heads(gpos, po, pi, ln)[h], st["pos"][h]), (s, h)
            assert np.array_equal(ref.gather_heads(k, po, pi, ln)[h], st["k"][h]), (s, h)


def test_fused_step_ragged_edge_cases():
    """Both fused calls on a ragged cache: heads without pages, heads of one
    entry, lengths on and off page boundaries (heads whose pages are full get
    no entry and are counted), budgets of a third, one entry, nothing and
    more than everything, beta = 0 for some new entries (score -inf), G = 8
    query heads per KV head; against the separate calls bit for bit."""
    w = W["stream_gqa7"].scaled(layers=5, kv_heads=8, group=8, ctx=300, reserve=0, beta_block=None)
    H, D, G = w.n_heads, w.head_dim, w.group
    rng = np.random.default_rng(3)
    lens = rng.integers(0, 301, H).astype(np.int32)
    lens[:6] = [0, 1, 16, 17, 288, 300]            # empty, one entry, full page, one over, full pages
    pc = synth.build_cache(w, lengths=lens)
    ca = upload(pc)
    cb = clone_cache(ca)
    home_off, home_ids = ca.page_off.clone(), ca.page_ids.clone()
    tables = {n: [(torch.zeros_like(home_off), torch.zeros_like(home_ids)) for _ in range(2)] for n in "ab"}
    seg = cuda(np.array([0, H], np.int32))
    total = int(lens.sum())
    for s, M in enumerate((total // 3, 1, 0, total + 100)):
        t = w.ctx + s + 1
        beta = rng.beta(5.0, 1.0, H).astype(np.float32)
        beta[::5] = 0.0   # the new entry scores -inf: ranked below every other entry
        kn = synth.f64_to_bf16_bits(rng.standard_normal((H, D)))
        vn = synth.f64_to_bf16_bits(rng.standard_normal((H, D)))
        qn = synth.f64_to_bf16_bits(rng.standard_normal((H * G, D)))
        len_before = ca.length.cpu().numpy().astype(np.int64)
        po_now = ca.page_off.cpu().numpy().astype(np.int64)
        cap = (po_now[1:] - po_now[:-1]) * 16           # slots under the current table
        valid_after = np.minimum(len_before + 1, cap)   # a head with a free slot gains its new entry
        announce("fused step, ragged cache, budget", M)
        outs = []
        for name in "ab":
            c = ca if name == "a" else cb
            n = c.n_pages * 16
            score = torch.empty(n, dtype=torch.float32, device="cuda")
            keep = torch.empty(n, dtype=torch.uint8, device="cuda")
            kept = torch.empty(H, dtype=torch.int32, device="cuda")
            status = torch.zeros(2, dtype=torch.int32, device="cuda")
            t_dev = cuda(np.array([t], np.int32))
            bud = cuda(np.array([M], np.int64))
            out = torch.full((H * G, D), 5.0, dtype=torch.float32, device="cuda")
            dropped = torch.full((H * G,), 5.0, dtype=torch.float32, device="cuda")
            no, ni = tables[name][s % 2]
            used = int(c.page_off[H].item()) * 16   # keep-plane slots under the current table
            if name == "a":
                tk.append(c, kv_dev(kn, "bf16"), kv_dev(vn, "bf16"), cuda(beta), t_dev, status=status[0:1])
                tk.score_select(c, seg, t_dev, bud, score, keep, kept, status=status[1:2])
                tk.decode_attn(c, kv_dev(qn, "bf16"), G, D ** -0.5, out, dropped, keep=keep)
                v = tk.evict_tailfill(c, keep, 1, home_off, home_ids, no, ni, kept=kept)
            else:
                tk.append_score_select(c, kv_dev(kn, "bf16"), kv_dev(vn, "bf16"), cuda(beta), seg, t_dev, bud, score,
                                       keep, kept, append_status=status[0:1], select_status=status[1:2])
                v = tk.decode_attn_evict_tailfill(c, keep, kept, kv_dev(qn, "bf16"), G, D ** -0.5, out, dropped, 1,
                                                  home_off, home_ids, no, ni)
            torch.cuda.synchronize()
            outs.append((f32_bits(score[:used].cpu().numpy()), keep[:used].cpu().numpy(), kept.cpu().numpy(),
                         f32_bits(out.cpu().numpy()), f32_bits(dropped.cpu().numpy()), status.cpu().numpy()))
            if name == "a":
                ca = v
            else:
                cb = v
        for x, y in zip(*outs):
            assert np.array_equal(x, y), M
        same_cache(ca, cb)
        kept_np, st = outs[0][2], outs[0][5]
        assert st.tolist() == [int((len_before >= cap).sum()), 0], M
        assert int(kept_np.sum()) == min(M, int(valid_after.sum())), M
        assert np.all(kept_np <= valid_after)
        d = np.asarray(outs[0][4]).view(np.float32)
        assert np.all(np.isfinite(d)) and np.all((d >= 0) & (d <= 1))
        # heads that keep nothing: output 0, dropped 1
        none = np.repeat(kept_np == 0, G)
        o = np.asarray(outs[0][3]).view(np.float32).reshape(H * G, D)
        assert np.all(o[none] == 0.0) and np.all(d[none] == 1.0)


def test_append_score_select_ln_beta_hard_cases():
    """The fused call stores ln beta as trimkv_log_beta does: the correctly
    rounded float32 logarithm, checked on the hard-rounding inputs (ln within
    a few float64 ulps of a float32 rounding midpoint), the special values
    and random betas, one new entry per head of a 2,048-head cache."""
    from test_oracle_pins import HARD_LN_INPUTS
    w = W["tiny"].scaled(layers=1024, kv_heads=2, ctx=20, reserve=1, budget_abs=30000)
    H = w.n_heads
    pc = synth.build_cache(w)
    c = upload(pc)
    rng = np.random.default_rng(9)
    hard = np.array(HARD_LN_INPUTS, np.uint32).view(np.float32)
    specials = np.array([0.0, 1.0, 2 ** -149, 2 ** -126, 0.5, 1 - 2 ** -24], np.float32)
    beta = rng.uniform(0.0, 1.0, H).astype(np.float32)
    beta[:hard.size] = hard
    beta[hard.size:hard.size + specials.size] = specials
    kn = rng.standard_normal((H, w.head_dim)).astype(np.float32)
    vn = rng.standard_normal((H, w.head_dim)).astype(np.float32)
    n = c.n_pages * 16
    score = torch.empty(n, dtype=torch.float32, device="cuda")
    keep = torch.empty(n, dtype=torch.uint8, device="cuda")
    kept = torch.empty(H, dtype=torch.int32, device="cuda")
    announce("append+score+select, ln beta of", hard.size, "hard inputs")
    tk.append_score_select(c, kv_dev(kn, "f32"), kv_dev(vn, "f32"), cuda(beta), cuda(np.array([0, H], np.int32)),
                           cuda(np.array([w.ctx + 1], np.int32)), cuda(np.array([w.budget()], np.int64)), score, keep,
                           kept)
    torch.cuda.synchronize()
    po, pi, ln, _, _, glnb, gpos = download_cache(c)
    glnb_h, gpos_h = ref.gather_heads(glnb, po, pi, ln), ref.gather_heads(gpos, po, pi, ln)
    new_lnb = np.array([glnb_h[h][-1] for h in range(H)], np.float32)
    assert np.array_equal(f32_bits(new_lnb), f32_bits(ref.ln_beta(beta)))
    assert all(gpos_h[h][-1] == w.ctx for h in range(H))
