"""The streaming workload at full size over its whole run: 28 layers x 4 KV
heads (GQA 7), a 65,536-token prefill, a fixed budget of 458,752 entries and
8,192 generated steps, each appending one entry per KV head, scoring,
selecting, attending in mask mode and evicting (TRIM-KV page, section 2:
once the budget is exceeded the lowest current scores are evicted).

The oracle tracks the state of every step (ln beta, position and head of
every entry; selection by the oracle's partial-sort selection on its own
float32 scores) and the GPU runs the same 8,192 steps in four ways:
evicting out of place into the other of two pools; in place within each
head's own pages by a stable shift; in place by tail fill; and by tail fill
as two fused calls per step (trimkv_append_score_select, then
trimkv_decode_attn_evict_tailfill).  Checked:
  - every step: kept entries per head, the new page offsets and lengths,
    bit for bit (every variant);
  - steps 1-16, every 256th step and the last: the whole keep plane, the
    positions and ln beta of every retained entry, the K/V rows of sampled
    heads, and mask-mode attention on sampled heads against the float64
    oracle;
  - the failure counters of append and selection stay 0."""
import math
import os
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import synth
from oracle import reference as ref
from retention_scored_decode_amd import trimkv as tk
from gpu_helpers import DROP_TOL, OUT_TOL, f32_bits, heads_from_plane, kv_f64, upload

pytestmark = pytest.mark.gpu

SAMPLE_HEADS = [0, 45, 111]


def say(*a):
    print("[stream-full]", *a, flush=True)


def sample_steps(S):
    return sorted(set(range(1, min(16, S) + 1)) | set(range(256, S + 1, 256)) | {S})


@pytest.fixture(scope="module")
def stream_run():
    w = synth.WORKLOADS["stream_gqa7"]
    S = w.steps
    t0 = time.time()
    workers = min(16, os.cpu_count() or 1)
    pc = synth.build_cache(w, workers=workers)
    with ThreadPoolExecutor(workers) as ex:
        steps_in = list(ex.map(lambda s: synth.stream_step(w, s), range(1, S + 1)))
    say("generated the prefill and", S, "steps in %.1f s" % (time.time() - t0))
    return w, pc, steps_in


class GpuRun:
    """Per-step histories of one GPU run and snapshots at the sampled steps."""

    def __init__(self, S, H):
        self.kept = torch.empty((S, H), dtype=torch.int32, device="cuda")
        self.length = torch.empty((S, H), dtype=torch.int32, device="cuda")
        self.off = torch.empty((S, H + 1), dtype=torch.int32, device="cuda")
        self.snap = {}


def run_gpu(w, pc, steps_in, mode):
    inplace = mode != "out_of_place"
    tailfill = mode.startswith("tail_fill")
    fused = mode == "tail_fill_fused"   # two calls per step: append + score + select, attention + eviction
    S, H, G, D = w.steps, pc.n_heads, w.group, w.head_dim
    M = w.budget()
    scale = 1.0 / math.sqrt(D)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda").view(torch.bfloat16)
    beta_all = torch.from_numpy(np.stack([x[0] for x in steps_in])).to("cuda")
    k_all = bf(np.stack([x[1] for x in steps_in]))
    v_all = bf(np.stack([x[2] for x in steps_in]))
    q_all = bf(np.stack([x[3] for x in steps_in]))
    t_all = torch.arange(w.ctx + 1, w.ctx + S + 1, dtype=torch.int32, device="cuda").view(S, 1)
    prefill = upload(pc)
    seg = torch.tensor([0, H], dtype=torch.int32, device="cuda")
    bud = torch.tensor([M], dtype=torch.int64, device="cuda")
    score = torch.empty(prefill.n_pages * 16, dtype=torch.float32, device="cuda")
    keep = torch.empty(prefill.n_pages * 16, dtype=torch.uint8, device="cuda")
    kept = torch.empty(H, dtype=torch.int32, device="cuda")
    used = torch.zeros(1, dtype=torch.int64, device="cuda")
    out = torch.empty((H * G, D), dtype=torch.float32, device="cuda")
    dropped = torch.empty(H * G, dtype=torch.float32, device="cuda")
    st_app = torch.zeros(1, dtype=torch.int32, device="cuda")
    st_sel = torch.zeros(1, dtype=torch.int32, device="cuda")
    # out of place: two pools with one spare slot per head; in place: one
    # home pool whose heads have room for every step's entry
    res1 = S if inplace else 1
    cap = -(-(M + H * res1) // 16) + H
    pools = [tk.Cache.empty(H, cap, D, torch.bfloat16) for _ in range(1 if inplace else 2)]
    tables = [(torch.empty(H + 1, dtype=torch.int32, device="cuda"),
               torch.empty(cap, dtype=torch.int32, device="cuda")) for _ in range(2)]
    ws_inp = tk.workspace(tk.OP_EVICT_TAILFILL if tailfill else tk.OP_COMPACT_INPLACE, pools[0])
    ws_of = lambda c: (tk.workspace(tk.OP_SELECT, c, 1), tk.workspace(tk.OP_DECODE_ATTN, c, 0, G),
                       tk.workspace(tk.OP_COMPACT, c))
    ws_pre, ws_pool = ws_of(prefill), ws_of(pools[0])
    ws_de = tk.workspace(tk.OP_DECODE_EVICT, pools[0], 0, G) if fused else None
    r = GpuRun(S, H)
    samples = set(sample_steps(S))
    cur, home = prefill, None
    for s in range(1, S + 1):
        i = s - 1
        wsel, watt, wcmp = ws_pre if s == 1 else ws_pool
        snap = None
        if fused and s > 1:
            tk.append_score_select(cur, k_all[i], v_all[i], beta_all[i], seg, t_all[i], bud, score, keep, kept,
                                   ws=wsel, append_status=st_app, select_status=st_sel)
        else:
            tk.append(cur, k_all[i], v_all[i], beta_all[i], t_all[i], status=st_app)
            if tailfill:   # the fused score + select, on slots out of position order
                tk.score_select(cur, seg, t_all[i], bud, score, keep, kept, ws=wsel, status=st_sel)
            else:
                tk.score(cur, seg, t_all[i], score)
                tk.select_global(cur, score, seg, bud, keep, kept, ws=wsel, status=st_sel)
        if s in samples:
            snap = {"cur_off": cur.page_off.cpu().numpy(), "cur_len": cur.length.cpu().numpy()}
            snap["keep"] = keep[:int(snap["cur_off"][-1]) * 16].cpu().numpy()
            if tailfill:   # positions of the slots the keep plane refers to
                snap["cur_pos"] = ref.gather_heads(cur.meta[:, 1, :].cpu().numpy(), snap["cur_off"],
                                                   cur.page_ids.cpu().numpy(), snap["cur_len"])
        if fused and s > 1:   # attention, then eviction in place, the merge beside the eviction
            nt = tables[s % 2]
            nxt = tk.decode_attn_evict_tailfill(cur, keep, kept, q_all[i], G, scale, out, dropped, 1, home[0],
                                                home[1], nt[0], nt[1], ws=ws_de)
        else:
            tk.decode_attn(cur, q_all[i], G, scale, out, dropped, keep=keep, ws=watt)
            if inplace and s > 1:
                nt = tables[s % 2]
                evict = tk.evict_tailfill if tailfill else tk.compact_inplace
                nxt = evict(cur, keep, 1, home[0], home[1], nt[0], nt[1], kept=kept, ws=ws_inp)
            else:
                nxt = pools[s % len(pools)]
                tk.compact(cur, keep, res1 if s == 1 else 1, M, nxt, used, ws=wcmp, kept=kept)
                if inplace:
                    home = (nxt.page_off.clone(), nxt.page_ids.clone())
        if s in samples:
            snap["out"], snap["dropped"] = out.cpu().numpy(), dropped.cpu().numpy()
        r.kept[i].copy_(kept)
        r.length[i].copy_(nxt.length)
        r.off[i].copy_(nxt.page_off)
        if s in samples:
            off, ids, ln = nxt.page_off.cpu().numpy(), nxt.page_ids.cpu().numpy(), nxt.length.cpu().numpy()
            meta = nxt.meta.cpu().numpy()
            snap["pos"] = ref.gather_heads(np.ascontiguousarray(meta[:, 1, :]), off, ids, ln)
            snap["lnb"] = ref.gather_heads(np.ascontiguousarray(meta[:, 0, :]).view(np.float32), off, ids, ln)
            rows = {}
            for h in SAMPLE_HEADS:
                idx = torch.from_numpy(ref.head_phys_slots(off, ids, ln, h)).to("cuda")
                rows[h] = (nxt.k.view(-1, D)[idx].view(torch.int16).cpu().numpy().view(np.uint16),
                           nxt.v.view(-1, D)[idx].view(torch.int16).cpu().numpy().view(np.uint16))
            snap["rows"] = rows
            r.snap[s] = snap
        cur = nxt
    torch.cuda.synchronize()
    r.status = (int(st_app.item()), int(st_sel.item()))
    r.kept, r.length, r.off = r.kept.cpu().numpy(), r.length.cpu().numpy(), r.off.cpu().numpy()
    r.home = None if home is None else (home[0].cpu().numpy(), home[1].cpu().numpy())
    del prefill, pools, q_all, k_all, v_all, cur, nxt
    torch.cuda.empty_cache()
    return r


def oracle_run(w, pc, steps_in):
    """The oracle's state at every step: kept entries per head, and at the
    sampled steps the per-head keep flags over the head's entries before
    eviction (position order), their positions, and the retained ln beta."""
    S, H = w.steps, pc.n_heads
    M = w.budget()
    po, pi, ln = pc.page_off, pc.page_ids, pc.length
    lnb = np.concatenate(ref.gather_heads(ref.ln_beta(pc.beta), po, pi, ln))
    pos = np.concatenate(ref.gather_heads(pc.pos, po, pi, ln)).astype(np.int32)
    head = np.repeat(np.arange(H, dtype=np.int32), ln)
    hs = np.arange(H, dtype=np.int32)
    samples = set(sample_steps(S))
    kept_hist = np.zeros((S, H), np.int64)
    snaps = {}
    for s in range(1, S + 1):
        t = w.ctx + s
        lnb_new = ref.ln_beta(steps_in[s - 1][0])
        if s == 1:
            lnb = np.concatenate([lnb, lnb_new])
            pos = np.concatenate([pos, np.full(H, t - 1, np.int32)])
            head = np.concatenate([head, hs])
        else:   # the H entries evicted last step make room for the H new ones
            lnb[free], pos[free], head[free] = lnb_new, t - 1, hs
        keep = ref.select_flat(ref.score_f32(lnb, t, pos), head, pos, M)
        if s in samples:
            order = np.lexsort((pos, head))              # heads, then position (slot) order
            cnt = np.bincount(head, minlength=H)
            cuts = np.concatenate([[0], np.cumsum(cnt)])
            ko, po_, lo = keep[order], pos[order], lnb[order]
            snaps[s] = {"keep": [ko[cuts[h]:cuts[h + 1]] for h in range(H)],
                        "pos": [po_[cuts[h]:cuts[h + 1]] for h in range(H)],
                        "lnb": [lo[cuts[h]:cuts[h + 1]] for h in range(H)]}
        if s == 1:
            kept_hist[0] = np.bincount(head[keep], minlength=H)
            lnb, pos, head = (np.concatenate([x[keep], np.zeros(H, x.dtype)]) for x in (lnb, pos, head))
            free = np.arange(M, M + H)
        else:   # every head gained one entry; the evicted ones leave
            free = np.flatnonzero(~keep)
            kept_hist[s - 1] = kept_hist[s - 2] + 1 - np.bincount(head[free], minlength=H)
        assert len(free) == H
    return kept_hist, snaps


def entry_rows(w, pc, steps_in, h, positions):
    """K/V bits of head h's entries at the given positions: prefill entries
    from the prefill pool, generated ones from their step's inputs."""
    D = w.head_dim
    out_k = np.empty((len(positions), D), np.uint16)
    out_v = np.empty((len(positions), D), np.uint16)
    pre = positions < w.ctx
    phys = ref.head_phys_slots(pc.page_off, pc.page_ids, pc.length, h)
    out_k[pre] = pc.k.reshape(-1, D)[phys[positions[pre]]]
    out_v[pre] = pc.v.reshape(-1, D)[phys[positions[pre]]]
    for j in np.flatnonzero(~pre):
        st = int(positions[j]) - w.ctx   # entry of step st + 1
        out_k[j], out_v[j] = steps_in[st][1][h], steps_in[st][2][h]
    return out_k, out_v


@pytest.fixture(scope="module")
def oracle_state(stream_run):
    w, pc, steps_in = stream_run
    t0 = time.time()
    res = oracle_run(w, pc, steps_in)
    say("oracle tracked", w.steps, "steps in %.1f s" % (time.time() - t0))
    return res


@pytest.mark.parametrize("mode", ["out_of_place", "in_place", "tail_fill", "tail_fill_fused"])
def test_full_streaming_run(stream_run, oracle_state, mode):
    w, pc, steps_in = stream_run
    kept_hist, osnap = oracle_state
    S, H, G, D = w.steps, pc.n_heads, w.group, w.head_dim
    M = w.budget()
    inplace, tailfill = mode != "out_of_place", mode.startswith("tail_fill")
    t0 = time.time()
    r = run_gpu(w, pc, steps_in, mode)
    say("GPU ran", S, "steps", mode, "in %.1f s" % (time.time() - t0))
    assert r.status == (0, 0), "failure counters (append, select)"
    # every step: kept per head, page offsets and lengths
    assert np.array_equal(r.kept, kept_hist), np.argwhere(r.kept != kept_hist)[:5]
    assert np.array_equal(r.length, kept_hist)
    assert np.all(kept_hist.sum(axis=1) == M)
    for s in range(1, S + 1):
        if inplace and s > 1:
            wpo = ref.compact_inplace_layout(kept_hist[s - 1], 1, *r.home)[0]
        else:
            wpo = ref.compact_layout(kept_hist[s - 1], S if inplace else 1)[0]
        assert np.array_equal(r.off[s - 1], wpo), ("page offsets", s)
    say("kept counts, page offsets and lengths exact at all", S, "steps")
    # sampled steps: keep plane, retained metadata, rows and attention
    scale = 1.0 / math.sqrt(D)
    for s, g in sorted(r.snap.items()):
        o = osnap[s]
        got = heads_from_plane(g["keep"], g["cur_off"], g["cur_len"])
        gpos, glnb = g["pos"], g["lnb"]
        # tail-filled slots are not in position order: compare in position order
        srt = [np.argsort(gpos[h], kind="stable") if tailfill else slice(None) for h in range(H)]
        for h in range(H):
            if tailfill:
                assert np.array_equal(np.sort(g["cur_pos"][h][got[h].astype(bool)]),
                                      o["pos"][h][o["keep"][h]]), (s, "keep", h)
            else:
                assert np.array_equal(got[h].astype(bool), o["keep"][h]), (s, "keep", h)
            assert np.array_equal(gpos[h][srt[h]], o["pos"][h][o["keep"][h]]), (s, "pos", h)
            assert np.array_equal(f32_bits(glnb[h][srt[h]]), f32_bits(o["lnb"][h][o["keep"][h]])), (s, "lnb", h)
        q64 = kv_f64(steps_in[s - 1][3], "bf16")
        K, V, kp = [], [], []
        for h in SAMPLE_HEADS:
            kk, vv = entry_rows(w, pc, steps_in, h, o["pos"][h])
            kr, vr = g["rows"][h]
            j = SAMPLE_HEADS.index(h)
            kr, vr = kr[srt[h]], vr[srt[h]]
            assert np.array_equal(kr, kk[o["keep"][h]]) and np.array_equal(vr, vv[o["keep"][h]]), (s, "rows", h, j)
            K.append(kv_f64(kk, "bf16"))
            V.append(kv_f64(vv, "bf16"))
            kp.append(o["keep"][h])
        rows = np.concatenate([np.arange(h * G, (h + 1) * G) for h in SAMPLE_HEADS])
        wout, wdrop, _ = ref.decode_attn(K, V, q64[rows], G, scale, keep=kp)
        assert np.max(np.abs(g["out"][rows] - wout)) <= OUT_TOL, s
        assert np.max(np.abs(g["dropped"][rows] - wdrop)) <= DROP_TOL, s
        assert np.all(np.isfinite(g["out"])) and np.all((g["dropped"] >= 0) & (g["dropped"] <= 1))
    say("keep planes, retained metadata, rows and attention checked at", len(r.snap), "sampled steps")
